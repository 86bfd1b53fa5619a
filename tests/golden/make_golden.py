"""Write the stored expected values of the full-size parity tests.

Calls only the CPU oracle (float64) and the seeded input generators.  For each
full-size workload it decodes the chosen streams in full and stores, per
stream:
  - idx / pcm / pre: the PCM and pre-tanh values at a fixed set of sample
    indices (a regular stride plus whole frames at the start and end), in
    float64, and the norms of the full outputs (pcm_norm / pre_norm);
  - pcm32 / pre32 (whole-sequence workloads in all three arithmetic modes, and
    the batched workload): every sample of the decoded span, rounded once to
    float32 for storage (a relative change of at most 2^-24, far below the
    parity bars);
  - bound_frames / pcm_bound32 / pre_bound32 (long-form workload): every
    sample of the frame before and the frame after each boundary between its
    25-frame chunks, rounded to float32 likewise.

    python tests/golden/make_golden.py [name ...]

Names: qwen3_whole (the 250-frame whole-sequence workload, stream 0, which the
streamed workload must also reproduce), qwen3_whole_f16 (the same with every
matrix product's operands rounded to fp16, the half-precision decoder),
qwen3_whole_int8 (the same with the matrix weights stored as int8 with one
fp16 scale per 32 values), qwen3_batched (streams 0-3, 37 and 63 of the
64-stream workload: their timed 25-frame chunk after warm-up; streams 0-3 sit
at the four warm-up positions), qwen3_longform (streams 0 and 15 of the
16 x 1500-frame Zipf workload).
"""
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import synthetic as S  # noqa: E402
from oracle import decoder as O  # noqa: E402

BATCHED_STREAMS = [0, 1, 2, 3, 37, 63]
LONGFORM_STREAMS = [0, 15]
CHUNK = 25


def sample_index(n_samples, hop, stride):
    idx = set(range(0, n_samples, stride))
    idx.update(range(0, min(hop, n_samples)))
    idx.update(range(max(0, n_samples - hop), n_samples))
    return np.array(sorted(idx), dtype=np.int64)


def boundary_frames(n_frames, chunk):
    """The frame before and the frame after every boundary between chunks."""
    fr = []
    for t in range(chunk, n_frames, chunk):
        fr += [t - 1, t]
    return np.array(fr, dtype=np.int64)


def frame_samples(frames, hop):
    return (frames[:, None] * hop + np.arange(hop)[None, :]).reshape(-1)


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


def sampled(pcm, pre, hop, stride):
    idx = sample_index(pcm.size, hop, stride)
    return dict(idx=idx, pcm=pcm[idx], pre=pre[idx], pcm_norm=np.linalg.norm(pcm), pre_norm=np.linalg.norm(pre))


def main(names):
    cfg = S.QWEN3
    W = None
    for name in names:
        t0 = time.time()
        if W is None:
            W = O.cast_weights(S.make_weights(cfg, 1), np.float64)
        hop = cfg["hop"]
        out = {}
        if name in ("qwen3_whole", "qwen3_whole_f16", "qwen3_whole_int8"):
            codes = S.workload_codes("qwen3_b1_t250_whole")
            if name == "qwen3_whole_f16":
                # the fp16-operand decoder (matrix-product operands rounded to fp16)
                pcm, pre = decode_stream(cfg, O.cast_operand_weights(W, np.float64, "f16"), codes[0], 125,
                                         operands="f16")
            elif name == "qwen3_whole_int8":
                # int8 weights (one fp16 scale per 32 values), arithmetic unrounded
                pcm, pre = decode_stream(cfg, O.quantize_weights_int8(W), codes[0], 125)
            else:
                pcm, pre = decode_stream(cfg, W, codes[0], 125)
            s = sampled(pcm, pre, hop, 61)
            out.update(stream=np.array([0]), frame0=np.array([0]), frames=np.array([250]), idx=s["idx"],
                       pcm=s["pcm"], pre=s["pre"], pcm_norm=np.array([s["pcm_norm"]]),
                       pre_norm=np.array([s["pre_norm"]]))
            out.update(pcm32=pcm.astype(np.float32), pre32=pre.astype(np.float32))
        elif name == "qwen3_batched":
            codes = S.workload_codes("qwen3_b64_chunk25")
            rec = {k: [] for k in ("idx", "pcm", "pre", "pcm_norm", "pre_norm", "pcm32", "pre32")}
            for b in BATCHED_STREAMS:
                nw = S.batched_warmup_frames(b)
                pcm, pre = decode_stream(cfg, W, codes[b, : nw + CHUNK], 101)
                pcm, pre = pcm[nw * hop:], pre[nw * hop:]
                for k, v in sampled(pcm, pre, hop, 61).items():
                    rec[k].append(v)
                rec["pcm32"].append(pcm.astype(np.float32))
                rec["pre32"].append(pre.astype(np.float32))
            out.update(stream=np.array(BATCHED_STREAMS), **{k: np.stack(v) for k, v in rec.items()})
        elif name == "qwen3_longform":
            codes = S.workload_codes("qwen3_b16_t1500_zipf")
            T = codes.shape[1]
            bf = boundary_frames(T, CHUNK)
            bs = frame_samples(bf, hop)
            rec = {k: [] for k in ("idx", "pcm", "pre", "pcm_norm", "pre_norm", "pcm_bound32", "pre_bound32")}
            for b in LONGFORM_STREAMS:
                pcm, pre = decode_stream(cfg, W, codes[b], 125)
                for k, v in sampled(pcm, pre, hop, 211).items():
                    rec[k].append(v)
                rec["pcm_bound32"].append(pcm[bs].astype(np.float32))
                rec["pre_bound32"].append(pre[bs].astype(np.float32))
            out.update(stream=np.array(LONGFORM_STREAMS), frame0=np.array([0]), frames=np.array([T]),
                       bound_frames=bf, **{k: np.stack(v) for k, v in rec.items()})
        else:
            raise SystemExit(f"unknown golden {name}")
        path = os.path.join(HERE, f"{name}.npz")
        np.savez_compressed(path, **out)
        print(f"{name}: wrote {path} in {time.time() - t0:.0f} s", flush=True)


if __name__ == "__main__":
    main(sys.argv[1:] or ["qwen3_whole", "qwen3_batched", "qwen3_longform"])
