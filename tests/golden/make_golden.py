"""Write the stored expected values of the full-size parity tests.

Calls only the CPU oracle (float64) and the seeded input generators.  For each
full-size workload it decodes sampled streams in full and stores the PCM and
pre-tanh values at a fixed set of sample indices (a regular stride plus whole
frames at the start and end), together with the norms of the full outputs.

    python tests/golden/make_golden.py [name ...]

Names: qwen3_whole (the 250-frame whole-sequence workload, stream 0, which the
streamed workload must also reproduce), qwen3_whole_f16 (the same with every
matrix product's operands rounded to fp16, the half-precision decoder),
qwen3_whole_int8 (the same with the matrix weights stored as int8 with one
fp16 scale per 32 values), qwen3_batched (streams 0-3 of the
64-stream workload: their timed 25-frame chunk after warm-up), qwen3_longform
(stream 0 of the 16 x 1500-frame Zipf workload).
"""
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import synthetic as S  # noqa: E402
from oracle import decoder as O  # noqa: E402


def sample_index(n_samples, hop, stride):
    idx = set(range(0, n_samples, stride))
    idx.update(range(0, min(hop, n_samples)))
    idx.update(range(max(0, n_samples - hop), n_samples))
    return np.array(sorted(idx), dtype=np.int64)


def decode_stream(cfg, W, codes, chunk, operands=None):
    """Whole-sequence decode of one stream, evaluated in pieces of `chunk`
    frames to bound memory (streamed == whole is pinned by the oracle tests)."""
    st = O.new_state(cfg)
    pcm, pre = [], []
    for t0 in range(0, codes.shape[0], chunk):
        taps = {}
        p, st = O.decode_chunk(cfg, W, codes[t0:t0 + chunk], st, np.float64, taps, operands)
        pcm.append(p)
        pre.append(taps["pre_tanh"])
        print(f"    frames {t0 + codes[t0:t0 + chunk].shape[0]}/{codes.shape[0]}", flush=True)
    return np.concatenate(pcm), np.concatenate(pre)


def main(names):
    cfg = S.QWEN3
    W = None
    for name in names:
        t0 = time.time()
        if W is None:
            W = O.cast_weights(S.make_weights(cfg, 1), np.float64)
        hop = cfg["hop"]
        out = {}
        if name == "qwen3_whole_f16":
            # the fp16-operand decoder (matrix-product operands rounded to fp16)
            codes = S.workload_codes("qwen3_b1_t250_whole")
            W16 = O.cast_operand_weights(W, np.float64, "f16")
            pcm, pre = decode_stream(cfg, W16, codes[0], 125, operands="f16")
            idx = sample_index(pcm.size, hop, 61)
            out.update(stream=np.array([0]), frame0=np.array([0]), frames=np.array([250]), idx=idx,
                       pcm=pcm[idx], pre=pre[idx], pcm_norm=np.array([np.linalg.norm(pcm)]),
                       pre_norm=np.array([np.linalg.norm(pre)]))
        elif name == "qwen3_whole_int8":
            # int8 weights (one fp16 scale per 32 values), arithmetic unrounded
            codes = S.workload_codes("qwen3_b1_t250_whole")
            W8 = O.quantize_weights_int8(W)
            pcm, pre = decode_stream(cfg, W8, codes[0], 125)
            idx = sample_index(pcm.size, hop, 61)
            out.update(stream=np.array([0]), frame0=np.array([0]), frames=np.array([250]), idx=idx,
                       pcm=pcm[idx], pre=pre[idx], pcm_norm=np.array([np.linalg.norm(pcm)]),
                       pre_norm=np.array([np.linalg.norm(pre)]))
        elif name == "qwen3_whole":
            codes = S.workload_codes("qwen3_b1_t250_whole")
            pcm, pre = decode_stream(cfg, W, codes[0], 125)
            idx = sample_index(pcm.size, hop, 61)
            out.update(stream=np.array([0]), frame0=np.array([0]), frames=np.array([250]), idx=idx,
                       pcm=pcm[idx], pre=pre[idx], pcm_norm=np.array([np.linalg.norm(pcm)]),
                       pre_norm=np.array([np.linalg.norm(pre)]))
        elif name == "qwen3_batched":
            codes = S.workload_codes("qwen3_b64_chunk25")
            streams = [0, 1, 2, 3]
            idxs, pcms, pres, pn, qn = [], [], [], [], []
            for b in streams:
                nw = S.batched_warmup_frames(b)
                pcm, pre = decode_stream(cfg, W, codes[b, : nw + 25], 101)
                pcm, pre = pcm[nw * hop:], pre[nw * hop:]
                idx = sample_index(pcm.size, hop, 61)
                idxs.append(idx); pcms.append(pcm[idx]); pres.append(pre[idx])
                pn.append(np.linalg.norm(pcm)); qn.append(np.linalg.norm(pre))
            out.update(stream=np.array(streams), idx=np.stack(idxs), pcm=np.stack(pcms), pre=np.stack(pres),
                       pcm_norm=np.array(pn), pre_norm=np.array(qn))
        elif name == "qwen3_longform":
            codes = S.workload_codes("qwen3_b16_t1500_zipf")
            pcm, pre = decode_stream(cfg, W, codes[0], 125)
            idx = sample_index(pcm.size, hop, 211)
            out.update(stream=np.array([0]), frame0=np.array([0]), frames=np.array([1500]), idx=idx,
                       pcm=pcm[idx], pre=pre[idx], pcm_norm=np.array([np.linalg.norm(pcm)]),
                       pre_norm=np.array([np.linalg.norm(pre)]))
        else:
            raise SystemExit(f"unknown golden {name}")
        path = os.path.join(HERE, f"{name}.npz")
        np.savez_compressed(path, **out)
        print(f"{name}: wrote {path} in {time.time() - t0:.0f} s", flush=True)


if __name__ == "__main__":
    main(sys.argv[1:] or ["qwen3_whole", "qwen3_batched", "qwen3_longform"])
