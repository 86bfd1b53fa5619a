"""GPU tests of the graph-replayed decode (vocoder_decode_chunk_graph): every
replay gives the eager call's bits, also with eager work and host
synchronisation between replays, for chunk schedules of the small-chunk
streaming path (1, 2, 4, 8 frames; a 4, 4, 8, 16, 25 ramp)."""
import numpy as np
import pytest
import torch

import synthetic as S
from tests.gpu_util import decoder, run_schedule
from vocoder_rvq_codebook_amd import binding as vb

pytestmark = pytest.mark.gpu


def run_graph_schedule(dec, codes, schedule, bufs, state=None):
    """Decode codes [B][T][Q] chunk by chunk through the graph entry point, with
    one code and one PCM buffer per chunk length and two ping-pong states."""
    B = codes.shape[0]
    if "states" not in bufs:
        bufs["states"] = (dec.new_state(B), dec.new_state(B))
    st_a, st_b = bufs["states"]
    if state is None:
        dec.reset(st_a)
    else:
        st_a.copy_(state)
    out, t0 = [], 0
    for n in schedule:
        if n not in bufs:
            bufs[n] = (torch.empty((B, n, codes.shape[2]), dtype=torch.int32, device="cuda"),
                       torch.empty((B, n * dec.hop), device="cuda"))
        cb, pb = bufs[n]
        cb.copy_(torch.from_numpy(np.ascontiguousarray(codes[:, t0:t0 + n])))
        dec.decode(cb, st_a, st_b, pb, graph=True)
        out.append(pb.clone())
        st_a, st_b = st_b, st_a
        t0 += n
    bufs["states"] = (st_a, st_b)
    torch.cuda.synchronize()
    return torch.cat(out, dim=1), st_a.clone()


SCHEDULES = {
    "1-2-4-8": [1, 2, 4, 8, 1, 1, 2, 2, 4, 8],
    "ramp": [4, 4, 8, 16, 25, 25, 25, 18],
}


@pytest.mark.parametrize("name", list(SCHEDULES))
@pytest.mark.parametrize("model", [S.MINI, dict(S.MINI, name="mini_f16", precision="f16"),
                                   dict(S.MINI, name="mini_q8", weights="int8"),
                                   dict(S.MINI, name="mini_q8_f16", weights="int8", precision="f16"),
                                   dict(S.MINI, name="mini_split", precision="split")],
                         ids=["f32", "f16", "int8", "int8_f16", "split"])
def test_graph_replays_equal_eager(name, model):
    schedule = SCHEDULES[name]
    T = sum(schedule)
    B = 2
    dec, _ = decoder(model, 21, B, max(schedule))
    codes = S.make_codes(model, B, T, 61)
    eager, st_e = run_schedule(dec, codes, schedule)
    bufs = {}
    for rep in range(3):
        got, st_g = run_graph_schedule(dec, codes, schedule, bufs)
        assert dec.status() == vb.VOCODER_OK
        assert torch.equal(got, eager), f"replay {rep}"
        assert torch.equal(st_g, st_e), f"replay {rep} state"
        # eager work and a host synchronisation between replays
        other = S.make_codes(model, 1, 5, 100 + rep)
        run_schedule(dec, other, [5])
        torch.cuda.synchronize()
    # two ping-pong states: at most two graphs per chunk length
    n = vb.vocoder_graph_cache_size(dec.handle)
    assert 0 < n <= 2 * len(set(schedule))


def test_graph_matches_whole_sequence_decode():
    """A ramp of graph-replayed chunks reproduces the one-call decode bitwise."""
    model = S.MINI
    dec, _ = decoder(model, 22, 1, 40)
    codes = S.make_codes(model, 1, 40, 62)
    whole, _ = run_schedule(dec, codes, [40])
    got, _ = run_graph_schedule(dec, codes, [4, 4, 8, 16, 8], {})
    assert torch.equal(got, whole)


def test_graph_cache_evicts_and_stays_correct():
    """More distinct (buffers, length) keys than the cache holds: least recently
    used graphs are dropped and re-recorded, results unchanged."""
    model = S.TINY
    dec, _ = decoder(model, 0, 1, 48)
    codes = S.make_codes(model, 1, 48, 63)
    sched = [1] * 48
    eager, _ = run_schedule(dec, codes, sched)
    # a fresh PCM buffer per call: every call is a new key
    st_a, st_b = dec.new_state(1), dec.new_state(1)
    cb = torch.empty((1, 1, model["n_codebooks"]), dtype=torch.int32, device="cuda")
    pcms = []
    for t in range(48):
        cb.copy_(torch.from_numpy(np.ascontiguousarray(codes[:, t:t + 1])))
        pb = torch.empty((1, dec.hop), device="cuda")
        pcms.append(pb)
        dec.decode(cb, st_a, st_b, pb, graph=True)
        st_a, st_b = st_b, st_a
    torch.cuda.synchronize()
    assert vb.vocoder_graph_cache_size(dec.handle) == 32
    assert torch.equal(torch.cat(pcms, dim=1), eager)


def test_graph_reports_device_errors_and_rejects_bad_arguments():
    model = S.TINY
    dec, _ = decoder(model, 0, 2, 8)
    n0 = vb.vocoder_graph_cache_size(dec.handle)
    st_a, st_b = dec.new_state(2), dec.new_state(2)
    codes = torch.zeros((2, 4, model["n_codebooks"]), dtype=torch.int32, device="cuda")
    pcm = torch.empty((2, 4 * dec.hop), device="cuda")
    # host-side argument errors: nothing recorded
    rc = vb.vocoder_decode_chunk_graph(dec.handle, codes, 2, 9, st_a, st_b, pcm)
    assert rc == vb.VOCODER_EINVAL
    st3 = dec.new_state(3)
    rc = vb.vocoder_decode_chunk_graph(dec.handle, codes, 2, 4, st3[0:2], st3[1:3], pcm)  # partial overlap
    assert rc == vb.VOCODER_EINVAL
    assert vb.vocoder_graph_cache_size(dec.handle) == n0
    # a code out of range, detected on the device, through a replayed graph
    dec.reset(st_a)
    dec.decode(codes, st_a, st_b, pcm, graph=True)
    assert dec.status() == vb.VOCODER_OK
    codes[1, 2, 3] = model["codebook_size"]
    dec.decode(codes, st_a, st_b, pcm, graph=True)
    assert dec.status() == vb.VOCODER_ECODE
    codes[1, 2, 3] = 0
    dec.decode(codes, st_a, st_b, pcm, graph=True)
    assert dec.status() == vb.VOCODER_OK
