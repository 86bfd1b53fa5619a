"""GPU parity at the full Qwen3-TTS-12Hz decoder shape, in the launch
configurations the benchmark uses, against float64 oracle values stored by
tests/golden/make_golden.py, and the properties that hold at any size:
streamed == whole, in place == ping-pong and batch independence, bitwise.

Coverage of the stored values: the 250-frame whole decode in full (every
sample; the streamed decode must equal it bit for bit); six of the 64 batched
streams in full (streams 0-3 sit at the four warm-up positions); streams 0 and
15 of the 16-stream long-form workload at every 211th sample plus both frames
around each of its 59 chunk boundaries.  The RVQ gather-sum is compared bit
for bit with the oracle's float32 ascending-codebook sum on every frame of
every stream of all three workloads."""
import os

import numpy as np
import pytest
import torch

import synthetic as S
from oracle import decoder as O
from tests.gpu_util import PCM_MAX_ABS, REL_L2, check_close, decoder, run_schedule

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
MODEL = S.QWEN3
HOP = MODEL["hop"]
D_EMB = MODEL["embed_dim"]


def golden(name):
    path = os.path.join(GOLDEN, f"{name}.npz")
    assert os.path.exists(path), f"missing {path}: run tests/golden/make_golden.py {name}"
    return dict(np.load(path))


def _compare(pcm, pre, g, what, k=None):
    """Sampled values (float64) and the norms of the whole outputs."""
    sel = (lambda a: a) if k is None else (lambda a: a[k])
    idx = sel(g["idx"])
    check_close(pcm[idx], sel(g["pcm"]), f"{what} pcm (sampled)", rel=REL_L2, max_abs=PCM_MAX_ABS)
    check_close(pre[idx], sel(g["pre"]), f"{what} pre-tanh (sampled)", rel=REL_L2)
    # the whole output, not just the samples, has the oracle's norm
    assert abs(np.linalg.norm(pcm) / sel(g["pcm_norm"]) - 1) < 1e-5, what
    assert abs(np.linalg.norm(pre) / sel(g["pre_norm"]) - 1) < 1e-5, what
    assert np.all(np.abs(pcm) <= 1.0)


def _compare_all(pcm, pre, ref_pcm, ref_pre, what):
    """Every sample: the waveform bar (rel-L2 and max-abs) and rel-L2 of the pre-tanh signal."""
    assert pcm.shape == ref_pcm.shape and pre.shape == ref_pre.shape, what
    check_close(pcm, ref_pcm, f"{what} pcm (every sample)", rel=REL_L2, max_abs=PCM_MAX_ABS)
    check_close(pre, ref_pre, f"{what} pre-tanh (every sample)", rel=REL_L2)


def _embed_ref(W, codes_rows):
    """The oracle's RVQ sum in float32 (the codebooks' dtype), ascending codebook order."""
    assert W["codebooks"].dtype == np.float32
    return O.rvq_embed_sum(W["codebooks"], codes_rows.reshape(-1, MODEL["n_codebooks"]))


@pytest.fixture(scope="module")
def whole_250():
    print("\n[full] 250-frame whole-sequence decode", flush=True)
    dec, W = decoder(MODEL, 1, 1, 250)
    codes = S.workload_codes("qwen3_b1_t250_whole")
    pre = torch.empty(250 * HOP, device="cuda")
    emb = torch.full((250 * D_EMB,), float("nan"), device="cuda")
    dec.set_tap("pre_tanh", pre)
    dec.set_tap("embed", emb)
    pcm, _ = run_schedule(dec, codes, [250])
    dec.set_tap("pre_tanh", None)
    dec.set_tap("embed", None)
    assert dec.status() == 0
    return (dec, W, codes, pcm[0].cpu().numpy().astype(np.float64), pre.cpu().numpy().astype(np.float64),
            emb.cpu().numpy())


def test_whole_sequence_250_frames(whole_250):
    _, W, codes, pcm, pre, emb = whole_250
    g = golden("qwen3_whole")
    _compare(pcm, pre, g, "250 frames whole")
    _compare_all(pcm, pre, g["pcm32"].astype(np.float64), g["pre32"].astype(np.float64), "250 frames whole")
    np.testing.assert_array_equal(emb.reshape(250, D_EMB), _embed_ref(W, codes[0]))


def test_streamed_1_then_25s_equals_whole(whole_250):
    """1 frame, nine 25-frame chunks, a final 24: bitwise equal to the whole decode."""
    print("\n[full] streamed 1 + 25x9 + 24", flush=True)
    dec, _, codes, pcm_whole, _, _ = whole_250
    sched = S.workload("qwen3_b1_t250_stream")["schedule"]
    assert sum(sched) == 250
    pcm, st = run_schedule(dec, codes, sched)
    assert dec.status() == 0
    assert np.array_equal(pcm[0].cpu().numpy().astype(np.float64), pcm_whole)


def test_in_place_1_25_25_equals_whole(whole_250):
    """One state buffer updated in place over chunks of 1, 25 and 25 frames:
    bitwise the first 51 frames of the whole decode."""
    print("\n[full] in place 1 + 25 + 25", flush=True)
    dec, _, codes, pcm_whole, _, _ = whole_250
    st = dec.new_state(1)
    out, t0 = [], 0
    for n in (1, 25, 25):
        c = torch.from_numpy(np.ascontiguousarray(codes[:, t0:t0 + n])).cuda()
        out.append(dec.decode(c, st, st))
        t0 += n
    pcm = torch.cat(out, dim=1)[0].cpu().numpy().astype(np.float64)
    assert dec.status() == 0
    assert np.array_equal(pcm, pcm_whole[: 51 * HOP])


def test_ramp_through_graphs_equals_whole(whole_250):
    """Chunks of 4, 4, 8, 16, then 25s, each replayed from a HIP graph: bitwise
    equal to the whole decode (small-chunk streaming at full size)."""
    from tests.test_gpu_graph import run_graph_schedule

    print("\n[full] graph ramp 4, 4, 8, 16, 25 x 8, 18", flush=True)
    dec, _, codes, pcm_whole, _, _ = whole_250
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
    dec, W = decoder(MODEL, 1, 64, 25)
    codes = S.workload_codes("qwen3_b64_chunk25")
    warm = [S.batched_warmup_frames(b) for b in range(64)]
    st = _warm(dec, codes, warm)
    saved = st.clone()
    chunk = np.stack([codes[b, warm[b]:warm[b] + 25] for b in range(64)])
    pre = torch.empty(64 * 25 * HOP, device="cuda")
    emb = torch.full((64 * 25 * D_EMB,), float("nan"), device="cuda")
    dec.set_tap("pre_tanh", pre)
    dec.set_tap("embed", emb)
    pcm, _ = run_schedule(dec, chunk, [25], state=st)
    dec.set_tap("pre_tanh", None)
    dec.set_tap("embed", None)
    assert dec.status() == 0
    # the gather of all 64 streams, bit for bit
    np.testing.assert_array_equal(emb.cpu().numpy().reshape(64 * 25, D_EMB), _embed_ref(W, chunk))
    pcm_np = pcm.cpu().numpy().astype(np.float64)
    pre_np = pre.view(64, -1).cpu().numpy().astype(np.float64)
    assert np.isfinite(pcm_np).all() and np.all(np.abs(pcm_np) <= 1.0)
    g = golden("qwen3_batched")
    for k, b in enumerate(g["stream"]):
        _compare(pcm_np[b], pre_np[b], g, f"stream {b}", k)
        _compare_all(pcm_np[b], pre_np[b], g["pcm32"][k].astype(np.float64), g["pre32"][k].astype(np.float64),
                     f"stream {b}")
    # batch independence at full size: stream 37 decoded alone, same state
    alone, _ = run_schedule(dec, chunk[37:38], [25], state=saved[37:38].clone())
    assert torch.equal(alone[0], pcm[37])
    assert w["batch"] == 64


def test_longform_16_streams_1500_frames_zipf():
    print("\n[full] 16 streams x 1500 frames in 25-frame chunks (Zipf codes)", flush=True)
    w = S.workload("qwen3_b16_t1500_zipf")
    dec, W = decoder(MODEL, 1, 16, 25)
    codes = S.workload_codes("qwen3_b16_t1500_zipf")
    B = codes.shape[0]
    g = golden("qwen3_longform")
    streams = [int(b) for b in g["stream"]]
    emb_ref = _embed_ref(W, codes).reshape(B, -1, D_EMB)
    st_a, st_b = dec.new_state(B), dec.new_state(B)
    pre = torch.empty(B * 25 * HOP, device="cuda")
    emb = torch.empty(B * 25 * D_EMB, device="cuda")
    dec.set_tap("pre_tanh", pre)
    dec.set_tap("embed", emb)
    kept_pcm = {b: [] for b in streams}
    kept_pre = {b: [] for b in streams}
    sq = torch.zeros(B, dtype=torch.float64, device="cuda")
    for i, n in enumerate(w["schedule"]):
        c = torch.from_numpy(np.ascontiguousarray(codes[:, i * 25:(i + 1) * 25])).cuda()
        pcm = dec.decode(c, st_a, st_b)
        st_a, st_b = st_b, st_a
        for b in streams:
            kept_pcm[b].append(pcm[b].cpu())
            kept_pre[b].append(pre.view(B, -1)[b].cpu())
        sq += (pcm.double() ** 2).sum(dim=1)
        assert torch.isfinite(pcm).all()
        # every stream's gather of this chunk, bit for bit (Zipf codes: repeated rows)
        np.testing.assert_array_equal(emb.view(B, 25, D_EMB).cpu().numpy(), emb_ref[:, i * 25:(i + 1) * 25])
        if i % 20 == 0:
            print(f"  chunk {i}", flush=True)
    dec.set_tap("pre_tanh", None)
    dec.set_tap("embed", None)
    assert dec.status() == 0
    bf = g["bound_frames"]
    bs = (bf[:, None] * HOP + np.arange(HOP)[None, :]).reshape(-1)
    assert bf.size == 2 * 59
    for k, b in enumerate(streams):
        p = torch.cat(kept_pcm[b]).numpy().astype(np.float64)
        q = torch.cat(kept_pre[b]).numpy().astype(np.float64)
        _compare(p, q, g, f"stream {b} of 16, 1500 frames", k)
        _compare_all(p[bs], q[bs], g["pcm_bound32"][k].astype(np.float64), g["pre_bound32"][k].astype(np.float64),
                     f"stream {b}, both frames of each chunk boundary")
    assert torch.all(sq > 0)
