"""GPU parity of the split-fp16 precision (fp32 values; every product of a
matrix product made of three fp16 MFMA products: lo*hi + hi*lo + hi*hi) against
the float64 oracle at the fp32 bar: small shapes stage by stage, the full
Qwen3-TTS-12Hz shape on the stored oracle values in the launch configuration
the benchmark times, and bitwise chunk and batch invariance."""
import numpy as np
import pytest
import torch

import synthetic as S
from oracle import decoder as O
from tests.gpu_util import PCM_MAX_ABS, REL_L2, check_close, decoder, oracle_stream, rel_l2, run_schedule
from tests.test_gpu_full import HOP, _compare, _warm, golden
from tests.test_gpu_parity import _stage_names, _tap_rows
from vocoder_rvq_codebook_amd import binding as vb

pytestmark = pytest.mark.gpu


def split(model):
    return dict(model, name=model["name"] + "_split", precision="split")


def _split_launches(prof):
    return sum(v["launches"] for k, v in prof.items() if k.startswith("conv_gemm_x3_"))


def _check_taps(model, W, taps, ref_taps, what, view=None):
    last = len(model["rates"]) - 1
    for name in _stage_names(model)[1:]:
        got = taps[name].cpu().numpy() if view is None else view(name)
        r = ref_taps[name]
        if name == f"stage{last}":  # tapped after the final Snake
            r = O.snake(r, W["act_post.alpha"].astype(np.float64))
        check_close(got, r.reshape(-1), f"{what} {name}")


def test_split_tiny_stage_by_stage():
    w = S.workload("tiny_b1_t32")
    model = split(w["model"])
    dec, W = decoder(model, w["weight_seed"], 1, 32)
    codes = S.workload_codes("tiny_b1_t32")
    T = codes.shape[1]
    taps = {}
    for name in _stage_names(model):
        rows, ch = _tap_rows(model, name, T)
        taps[name] = torch.full((rows * ch,), float("nan"), device="cuda")
        dec.set_tap(name, taps[name])
    vb.vocoder_profile_begin(dec.handle)
    pcm, _ = run_schedule(dec, codes, [T])
    prof = vb.vocoder_profile_end(dec.handle)
    assert dec.status() == vb.VOCODER_OK
    # every GEMM with 32-multiple input channels takes the split kernel
    assert _split_launches(prof) > 0, sorted(prof)
    ref_taps = {}
    ref = oracle_stream(model, W, codes[0], taps=ref_taps)
    np.testing.assert_array_equal(taps["embed"].cpu().numpy(), O.rvq_embed_sum(W["codebooks"], codes[0]).ravel())
    _check_taps(model, W, taps, ref_taps, "split tiny")
    check_close(pcm.cpu().numpy()[0], ref, "split tiny pcm", max_abs=PCM_MAX_ABS)
    for name in taps:
        dec.set_tap(name, None)


@pytest.mark.parametrize("T", [1, 13])
def test_split_mini_streams_at_different_positions(T):
    """Three streams warmed to positions 0, 7 and 20 (window 6), then one chunk
    of T; the narrow decoder's 128-, 64- and 32-channel layers run the split
    kernel with M below one tile, its 16-channel stage the fp32 kernel."""
    model = split(S.MINI)
    dec, W = decoder(model, 5, 3, 20)
    warm = [0, 7, 20]
    codes = S.make_codes(model, 3, max(warm) + T, 77)
    states = dec.new_state(3)
    for b, nw in enumerate(warm):
        if nw:
            _, st2 = run_schedule(dec, codes[b:b + 1, :nw], [nw], state=states[b:b + 1].clone())
            states[b:b + 1].copy_(st2)
    chunk = np.stack([codes[b, nw:nw + T] for b, nw in enumerate(warm)])
    taps = {}
    for name in _stage_names(model):
        rows, ch = _tap_rows(model, name, T)
        taps[name] = torch.full((3 * rows * ch,), float("nan"), device="cuda")
        dec.set_tap(name, taps[name])
    pcm, _ = run_schedule(dec, chunk, [T], state=states)
    assert dec.status() == vb.VOCODER_OK
    for b, nw in enumerate(warm):
        ref_taps = {}
        ref = oracle_stream(model, W, codes[b, : nw + T], [nw, T] if nw else [T], taps=ref_taps)

        def view(name, b=b):
            rows, ch = _tap_rows(model, name, T)
            return taps[name].view(3, rows * ch)[b].cpu().numpy()

        _check_taps(model, W, taps, ref_taps, f"split stream {b}", view)
        check_close(pcm[b].cpu().numpy(), ref[nw * model["hop"]:], f"split stream {b} pcm", max_abs=PCM_MAX_ABS)
    for name in taps:
        dec.set_tap(name, None)


@pytest.mark.parametrize("model_name,schedule", [
    ("mini", [1] * 6 + [5, 13, 1, 14]),
    ("mini", [20, 20]),
    ("tiny", [1, 25, 6]),
])
def test_split_streamed_equals_whole_bitwise(model_name, schedule):
    model = split(S.MINI if model_name == "mini" else S.TINY)
    T = sum(schedule)
    dec, _ = decoder(model, 9, 2, 40)
    codes = S.make_codes(model, 2, T, 31)
    whole, st_w = run_schedule(dec, codes, [T])
    parts, st_p = run_schedule(dec, codes, schedule)
    assert torch.equal(whole, parts)
    assert torch.equal(st_w, st_p)


def test_split_batch_independence_bitwise():
    model = split(S.MINI)
    dec, _ = decoder(model, 9, 4, 16)
    codes = S.make_codes(model, 4, 16, 41)
    both, _ = run_schedule(dec, codes, [16])
    for b in (0, 3):
        alone, _ = run_schedule(dec, codes[b:b + 1], [16])
        assert torch.equal(alone[0], both[b])


def test_split_refuses_weights_beyond_its_range():
    """A weight whose scaled hi half would be infinite (|w| * 2^8 >= 65520)
    makes vocoder_create fail with VOCODER_EINVAL instead of decoding NaNs."""
    model = split(S.TINY)
    W = S.make_weights(model, 3)
    name = "stages.0.blocks.0.0.conv1.weight"  # 32 input channels: a split layer
    W[name].flat[5] = 300.0
    flat = torch.from_numpy(S.flatten_weights(model, W))
    with pytest.raises(vb.VocoderError) as e:
        vb.Decoder(model, flat, 1, 4)
    assert e.value.code == vb.VOCODER_EINVAL
    W[name].flat[5] = 250.0  # within range: accepted
    dec = vb.Decoder(model, torch.from_numpy(S.flatten_weights(model, W)), 1, 4)
    pcm, _ = run_schedule(dec, S.make_codes(model, 1, 4, 5), [4])
    assert torch.isfinite(pcm).all()


def test_split_kernel_keeps_subnormal_input_halves():
    """The split GEMM splits its fp32 inputs unscaled, so small activations
    have fp16-subnormal lo halves: the tiny decoder's embedding sums (std 0.08)
    feed its pre-conv (64 input channels, a split layer) with more than 90 % of
    lo halves subnormal.  Through the library's own split kernel, the pre-conv
    output matches the float64 convolution of the same (bitwise) inputs to
    fp32 accuracy.  Dropping the subnormal lo halves would move it by 1.6e-4,
    far past the 2e-6 bar."""
    model = split(S.TINY)
    dec, W = decoder(model, 0, 1, 32)
    codes = S.workload_codes("tiny_b1_t32")
    T, d = codes.shape[1], model["model_dim"]
    emb = torch.empty(T * model["embed_dim"], device="cuda")
    h = torch.empty(T * d, device="cuda")
    dec.set_tap("embed", emb)
    dec.set_tap("pre_conv", h)
    vb.vocoder_profile_begin(dec.handle)
    run_schedule(dec, codes, [T])
    prof = vb.vocoder_profile_end(dec.handle)
    dec.set_tap("embed", None)
    dec.set_tap("pre_conv", None)
    assert dec.status() == 0
    assert _split_launches(prof) > 0
    e = emb.cpu().numpy().reshape(T, -1)
    np.testing.assert_array_equal(e, O.rvq_embed_sum(W["codebooks"], codes[0]))
    hi = e.astype(np.float16).astype(np.float32)
    lo = (e - hi).astype(np.float16)
    sub = (lo != 0) & (np.abs(lo.astype(np.float32)) < 2.0 ** -14)
    assert sub.mean() > 0.9
    w64, b64 = W["pre_conv.weight"].astype(np.float64), W["pre_conv.bias"].astype(np.float64)
    ref, _ = O.causal_conv1d(e.astype(np.float64), w64, b64, 1)
    r = rel_l2(h.cpu().numpy().reshape(T, d), ref)
    print(f"  split pre-conv rel-L2 {r:.3g}")
    assert r < 2e-6
    flushed, _ = O.causal_conv1d(hi.astype(np.float64) + np.where(sub, 0, lo).astype(np.float64), w64, b64, 1)
    assert rel_l2(flushed, ref) > 20 * 2e-6


# ---- the full decoder shape -------------------------------------------------

MODEL = split(S.QWEN3)


@pytest.fixture(scope="module")
def whole_250_split():
    print("\n[split full] 250-frame whole-sequence decode", flush=True)
    dec, _ = decoder(MODEL, 1, 1, 250)
    codes = S.workload_codes("qwen3_b1_t250_whole")
    pre = torch.empty(250 * HOP, device="cuda")
    dec.set_tap("pre_tanh", pre)
    vb.vocoder_profile_begin(dec.handle)
    pcm, _ = run_schedule(dec, codes, [250])
    prof = vb.vocoder_profile_end(dec.handle)
    dec.set_tap("pre_tanh", None)
    assert dec.status() == 0
    # every GEMM of this shape has 32-multiple input channels: all split
    assert _split_launches(prof) > 0 and not [k for k in prof if k.startswith("conv_gemm_") and "x3" not in k], \
        sorted(prof)
    return dec, codes, pcm[0].cpu().numpy().astype(np.float64), pre.cpu().numpy().astype(np.float64)


def test_split_whole_sequence_250_frames(whole_250_split):
    _, _, pcm, pre = whole_250_split
    _compare(pcm, pre, golden("qwen3_whole"), "split 250 frames whole")


def test_split_streamed_and_graph_ramp_equal_whole(whole_250_split):
    from tests.test_gpu_graph import run_graph_schedule

    dec, codes, pcm_whole, _ = whole_250_split
    print("\n[split full] streamed 1 + 25x9 + 24", flush=True)
    pcm, _ = run_schedule(dec, codes, S.workload("qwen3_b1_t250_stream")["schedule"])
    assert dec.status() == 0
    assert np.array_equal(pcm[0].cpu().numpy().astype(np.float64), pcm_whole)
    print("[split full] graph ramp 4, 4, 8, 16, 25 x 8, 18", flush=True)
    pcm, _ = run_graph_schedule(dec, codes, S.workload("qwen3_b1_t250_ramp")["schedule"], {})
    assert dec.status() == 0
    assert np.array_equal(pcm[0].cpu().numpy().astype(np.float64), pcm_whole)


def test_split_batched_64_streams_chunk_25():
    """The benchmark's launch configuration: 64 streams at staggered positions, one 25-frame chunk."""
    print("\n[split full] 64 streams x 25 frames after warm-up", flush=True)
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
    g = golden("qwen3_batched")
    for k, b in enumerate(g["stream"]):
        _compare(pcm_np[b], pre_np[b], g, f"split stream {b}", k)
    alone, _ = run_schedule(dec, chunk[37:38], [25], state=saved[37:38].clone())
    assert torch.equal(alone[0], pcm[37])


def test_split_longform_16_streams_1500_frames_zipf():
    """16 streams x 1500 frames in 25-frame chunks with Zipf-distributed codes:
    stream 0 against the stored oracle values."""
    print("\n[split full] 16 streams x 1500 frames in 25-frame chunks (Zipf codes)", flush=True)
    w = S.workload("qwen3_b16_t1500_zipf")
    dec, _ = decoder(MODEL, 1, 16, 25)
    codes = S.workload_codes("qwen3_b16_t1500_zipf")
    B = codes.shape[0]
    st_a, st_b = dec.new_state(B), dec.new_state(B)
    pre = torch.empty(B * 25 * HOP, device="cuda")
    dec.set_tap("pre_tanh", pre)
    pcm0, pre0 = [], []
    for i, n in enumerate(w["schedule"]):
        c = torch.from_numpy(np.ascontiguousarray(codes[:, i * 25:(i + 1) * 25])).cuda()
        pcm = dec.decode(c, st_a, st_b)
        st_a, st_b = st_b, st_a
        pcm0.append(pcm[0].cpu())
        pre0.append(pre.view(B, -1)[0].cpu())
        assert torch.isfinite(pcm).all()
        if i % 20 == 0:
            print(f"  chunk {i}", flush=True)
    dec.set_tap("pre_tanh", None)
    assert dec.status() == 0
    _compare(torch.cat(pcm0).numpy().astype(np.float64), torch.cat(pre0).numpy().astype(np.float64),
             golden("qwen3_longform"), "split stream 0 of 16, 1500 frames", 0)
