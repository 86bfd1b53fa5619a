"""GPU parity at the full Qwen3-TTS-12Hz decoder shape, in the launch
configurations the benchmark uses, against float64 oracle values stored by
tests/golden/make_golden.py (sampled PCM and pre-tanh values of whole streams,
plus the norms of the full outputs), and the properties that hold at any size:
streamed == whole and batch independence, bitwise."""
import os

import numpy as np
import pytest
import torch

import synthetic as S
from tests.gpu_util import PCM_MAX_ABS, REL_L2, check_close, decoder, run_schedule

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
MODEL = S.QWEN3
HOP = MODEL["hop"]


def golden(name):
    path = os.path.join(GOLDEN, f"{name}.npz")
    assert os.path.exists(path), f"missing {path}: run tests/golden/make_golden.py {name}"
    return dict(np.load(path))


def _compare(pcm, pre, g, what, k=None):
    sel = (lambda a: a) if k is None else (lambda a: a[k])
    idx = sel(g["idx"])
    check_close(pcm[idx], sel(g["pcm"]), f"{what} pcm", rel=REL_L2, max_abs=PCM_MAX_ABS)
    check_close(pre[idx], sel(g["pre"]), f"{what} pre-tanh", rel=REL_L2)
    # the whole output, not just the samples, has the oracle's norm
    assert abs(np.linalg.norm(pcm) / sel(g["pcm_norm"]) - 1) < 1e-5, what
    assert abs(np.linalg.norm(pre) / sel(g["pre_norm"]) - 1) < 1e-5, what
    assert np.all(np.abs(pcm) <= 1.0)


@pytest.fixture(scope="module")
def whole_250():
    print("\n[full] 250-frame whole-sequence decode", flush=True)
    dec, _ = decoder(MODEL, 1, 1, 250)
    codes = S.workload_codes("qwen3_b1_t250_whole")
    pre = torch.empty(250 * HOP, device="cuda")
    dec.set_tap("pre_tanh", pre)
    pcm, _ = run_schedule(dec, codes, [250])
    dec.set_tap("pre_tanh", None)
    assert dec.status() == 0
    return dec, codes, pcm[0].cpu().numpy().astype(np.float64), pre.cpu().numpy().astype(np.float64)


def test_whole_sequence_250_frames(whole_250):
    _, _, pcm, pre = whole_250
    _compare(pcm, pre, golden("qwen3_whole"), "250 frames whole")


def test_streamed_1_then_25s_equals_whole(whole_250):
    """1 frame, nine 25-frame chunks, a final 24: bitwise equal to the whole decode."""
    print("\n[full] streamed 1 + 25x9 + 24", flush=True)
    dec, codes, pcm_whole, _ = whole_250
    sched = S.workload("qwen3_b1_t250_stream")["schedule"]
    assert sum(sched) == 250
    pcm, st = run_schedule(dec, codes, sched)
    assert dec.status() == 0
    assert np.array_equal(pcm[0].cpu().numpy().astype(np.float64), pcm_whole)


def test_ramp_through_graphs_equals_whole(whole_250):
    """Chunks of 4, 4, 8, 16, then 25s, each replayed from a HIP graph: bitwise
    equal to the whole decode (small-chunk streaming at full size)."""
    from tests.test_gpu_graph import run_graph_schedule

    print("\n[full] graph ramp 4, 4, 8, 16, 25 x 8, 18", flush=True)
    dec, codes, pcm_whole, _ = whole_250
    sched = S.workload("qwen3_b1_t250_ramp")["schedule"]
    assert sum(sched) == 250
    pcm, _ = run_graph_schedule(dec, codes, sched, {})
    assert dec.status() == 0
    assert np.array_equal(pcm[0].cpu().numpy().astype(np.float64), pcm_whole)


def _warm(dec, codes, warm):
    B = len(warm)
    common = min(warm)
    sched = [1] + [25] * ((common - 1) // 25)
    _, st = run_schedule(dec, codes[:, :common], sched)
    tmp = dec.new_state(1)
    for b in range(B):
        tb = common
        while tb < warm[b]:
            c = torch.from_numpy(np.ascontiguousarray(codes[b:b + 1, tb:tb + 25])).cuda()
            dec.decode(c, st[b:b + 1], tmp)
            st[b:b + 1].copy_(tmp)
            tb += 25
    torch.cuda.synchronize()
    return st


def test_batched_64_streams_chunk_25():
    print("\n[full] 64 streams x 25 frames after warm-up", flush=True)
    w = S.workload("qwen3_b64_chunk25")
    dec, _ = decoder(MODEL, 1, 64, 25)
    codes = S.workload_codes("qwen3_b64_chunk25")
    warm = [S.batched_warmup_frames(b) for b in range(64)]
    st = _warm(dec, codes, warm)
    saved = st.clone()
    chunk = np.stack([codes[b, warm[b]:warm[b] + 25] for b in range(64)])
    pre = torch.empty(64 * 25 * HOP, device="cuda")
    dec.set_tap("pre_tanh", pre)
    pcm, _ = run_schedule(dec, chunk, [25], state=st)
    dec.set_tap("pre_tanh", None)
    assert dec.status() == 0
    pcm_np = pcm.cpu().numpy().astype(np.float64)
    pre_np = pre.view(64, -1).cpu().numpy().astype(np.float64)
    assert np.isfinite(pcm_np).all()
    g = golden("qwen3_batched")
    for k, b in enumerate(g["stream"]):
        _compare(pcm_np[b], pre_np[b], g, f"stream {b}", k)
    # batch independence at full size: stream 37 decoded alone, same state
    alone, _ = run_schedule(dec, chunk[37:38], [25], state=saved[37:38].clone())
    assert torch.equal(alone[0], pcm[37])
    assert w["batch"] == 64


def test_longform_16_streams_1500_frames_zipf():
    print("\n[full] 16 streams x 1500 frames in 25-frame chunks (Zipf codes)", flush=True)
    w = S.workload("qwen3_b16_t1500_zipf")
    dec, _ = decoder(MODEL, 1, 16, 25)
    codes = S.workload_codes("qwen3_b16_t1500_zipf")
    B = codes.shape[0]
    st_a, st_b = dec.new_state(B), dec.new_state(B)
    pre = torch.empty(B * 25 * HOP, device="cuda")
    dec.set_tap("pre_tanh", pre)
    pcm0, pre0, sq = [], [], torch.zeros(B, dtype=torch.float64, device="cuda")
    for i, n in enumerate(w["schedule"]):
        c = torch.from_numpy(np.ascontiguousarray(codes[:, i * 25:(i + 1) * 25])).cuda()
        pcm = dec.decode(c, st_a, st_b)
        st_a, st_b = st_b, st_a
        pcm0.append(pcm[0].cpu())
        pre0.append(pre.view(B, -1)[0].cpu())
        sq += (pcm.double() ** 2).sum(dim=1)
        assert torch.isfinite(pcm).all()
        if i % 20 == 0:
            print(f"  chunk {i}", flush=True)
    dec.set_tap("pre_tanh", None)
    assert dec.status() == 0
    g = golden("qwen3_longform")
    _compare(torch.cat(pcm0).numpy().astype(np.float64), torch.cat(pre0).numpy().astype(np.float64), g,
             "stream 0 of 16, 1500 frames")
    assert torch.all(sq > 0)
