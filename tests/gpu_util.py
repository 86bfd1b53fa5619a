"""Helpers shared by the GPU tests: build a decoder from seeded weights, run
streams through it, and compare with the oracle."""
import numpy as np
import torch

import synthetic as S
from oracle import decoder as O
from vocoder_rvq_codebook_amd import Decoder

# Waveform bar: max-abs and relative L2 against the float64 oracle.
PCM_MAX_ABS = 2e-3
REL_L2 = 1e-4

_CACHE = {}
_WEIGHTS = {}


def weights(model, seed):
    key = (model["name"], seed)
    if key not in _WEIGHTS:
        W = S.make_weights(model, seed)
        _WEIGHTS[key] = (W, torch.from_numpy(S.flatten_weights(model, W)))
    return _WEIGHTS[key]


def decoder(model, seed, max_batch, max_frames):
    key = (model["name"], seed, max_batch, max_frames)
    if key not in _CACHE:
        # one large decoder at a time keeps device memory modest
        for k in [k for k in _CACHE if k[0] == model["name"] and model["name"] == "qwen3_12hz"]:
            del _CACHE[k]
        torch.cuda.empty_cache()
        W, flat = weights(model, seed)
        dec = Decoder(model, flat, max_batch, max_frames)
        torch.cuda.synchronize()
        _CACHE[key] = (dec, W)
    return _CACHE[key]


def rel_l2(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    n = np.linalg.norm(ref)
    return float(np.linalg.norm(got - ref) / (n if n > 0 else 1.0))


def check_close(got, ref, what, rel=REL_L2, max_abs=None):
    r = rel_l2(got, ref)
    msg = f"{what}: rel-L2 {r:.3g}"
    print("  " + msg, flush=True)
    assert r <= rel, msg
    if max_abs is not None:
        m = float(np.max(np.abs(np.asarray(got, np.float64) - np.asarray(ref, np.float64))))
        assert m <= max_abs, f"{what}: max-abs {m:.3g}"
    return r


def run_schedule(dec, codes, schedule, state=None):
    """Decode codes [B][T][Q] (numpy) chunk by chunk on the GPU; returns (pcm [B][T*hop] numpy, state)."""
    B = codes.shape[0]
    st_a = dec.new_state(B) if state is None else state
    st_b = torch.empty_like(st_a)
    out, t0 = [], 0
    for n in schedule:
        c = torch.from_numpy(np.ascontiguousarray(codes[:, t0:t0 + n])).to(torch.int32).cuda()
        out.append(dec.decode(c, st_a, st_b))
        st_a, st_b = st_b, st_a
        t0 += n
    pcm = torch.cat(out, dim=1)
    torch.cuda.synchronize()
    return pcm, st_a


def oracle_stream(model, W, codes_1, schedule=None, taps=None, operands=None):
    """float64 oracle of one stream; with `taps`, the taps of the last chunk.
    operands="f16" evaluates the fp16-operand decoder."""
    if schedule is None:
        schedule = [codes_1.shape[0]]
    st = O.new_state(model)
    Wd = O.cast_operand_weights(W, np.float64, operands)
    out, t0 = [], 0
    for i, n in enumerate(schedule):
        tp = taps if i == len(schedule) - 1 else None
        p, st = O.decode_chunk(model, Wd, codes_1[t0:t0 + n], st, np.float64, tp, operands)
        out.append(p)
        t0 += n
    return np.concatenate(out)
