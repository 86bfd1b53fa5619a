"""Whole-decoder invariants of the oracle (CPU only).

blixt/phonon, Speed item 7: every chunk size shares one decoder state and must
give the same audio; the streamed workload must equal the whole-sequence one.
Edge TTS design 2.2/2.3: reset() clears the conv context and the window; the
state lives across calls.  Every layer is causal, streams are independent.
"""
import numpy as np
import pytest

import synthetic as S
from oracle import decoder as O


@pytest.fixture(scope="module")
def mini():
    cfg = S.MINI
    W = O.cast_weights(S.make_weights(cfg, 3), np.float64)
    codes = S.make_codes(cfg, 1, 40, 11)[0]
    whole = O.decode_whole(cfg, W, codes)
    return cfg, W, codes, whole


@pytest.fixture(scope="module")
def tiny():
    w = S.workload("tiny_b1_t32")
    cfg = w["model"]
    W = O.cast_weights(S.make_weights(cfg, w["weight_seed"]), np.float64)
    codes = S.workload_codes("tiny_b1_t32")[0]
    return cfg, W, codes, O.decode_whole(cfg, W, codes)


def test_output_length_and_range(mini, tiny):
    for cfg, _, codes, whole in (mini, tiny):
        assert whole.shape == (codes.shape[0] * cfg["hop"],)
        assert np.all(np.abs(whole) <= 1.0) and np.isfinite(whole).all()
    assert S.TINY["hop"] == 48 and S.QWEN3["hop"] == 1920


@pytest.mark.parametrize("schedule", [
    [1] * 40,
    [1, 25, 14],
    [4, 4, 8, 16, 8],
    [24, 1, 15],
    [39, 1],
    [2, 3, 5, 7, 11, 12],
])
def test_streamed_equals_whole_mini(mini, schedule):
    cfg, W, codes, whole = mini
    got, st = O.decode_schedule(cfg, W, codes, schedule)
    assert st.pos == 40
    np.testing.assert_allclose(got, whole, rtol=0, atol=1e-12)


@pytest.mark.parametrize("schedule", [[1] * 32, [1, 25, 6], [8, 8, 8, 8], [31, 1]])
def test_streamed_equals_whole_tiny(tiny, schedule):
    cfg, W, codes, whole = tiny
    got, _ = O.decode_schedule(cfg, W, codes, schedule)
    np.testing.assert_allclose(got, whole, rtol=0, atol=1e-12)


def test_causality(mini):
    cfg, W, codes, whole = mini
    hop = cfg["hop"]
    for t0 in (0, 7, 39):
        c2 = codes.copy()
        c2[t0:] = (c2[t0:] + 1) % cfg["codebook_size"]
        out = O.decode_whole(cfg, W, c2)
        np.testing.assert_array_equal(out[: t0 * hop], whole[: t0 * hop])
        assert np.abs(out[t0 * hop:] - whole[t0 * hop:]).max() > 1e-6


def test_state_save_restore_resumes_exactly(mini):
    cfg, W, codes, whole = mini
    _, st = O.decode_schedule(cfg, W, codes[:13], [5, 8])
    saved = st.copy()
    a, _ = O.decode_schedule(cfg, W, codes[13:], [27], state=st)
    b, _ = O.decode_schedule(cfg, W, codes[13:], [20, 7], state=saved)
    np.testing.assert_allclose(a, whole[13 * cfg["hop"]:], rtol=0, atol=1e-12)
    np.testing.assert_allclose(b, whole[13 * cfg["hop"]:], rtol=0, atol=1e-12)


def test_reset_forgets_previous_utterance(mini):
    cfg, W, codes, whole = mini
    other = S.make_codes(cfg, 1, 9, 99)[0]
    O.decode_schedule(cfg, W, other, [9])  # an utterance, then reset = fresh state
    got, _ = O.decode_schedule(cfg, W, codes, [40], state=O.new_state(cfg))
    np.testing.assert_array_equal(got, whole)


@pytest.mark.parametrize("window", [5, 6, 7])
def test_window_limits_attention_reach(window):
    """A frame at position t attends keys [t - W, t] (the W previous frames and
    itself).  With the pre-conv's kernel k spreading a frame over k frames and
    each of the L layers spreading it W further, a change of frame t0's codes
    reaches the transformer output (the final LayerNorm) on exactly frames
    t0 .. t0 + (k - 1) + L * W and on no other frame, bit for bit.  A window
    one frame shorter or longer moves the last changed frame by L."""
    cfg = dict(S.MINI, window=window)
    W = O.cast_weights(S.make_weights(cfg, 3), np.float64)
    codes = S.make_codes(cfg, 1, 40, 11)[0]
    t0 = 5
    c2 = codes.copy()
    c2[t0] = (c2[t0] + 5) % cfg["codebook_size"]
    a, b = {}, {}
    O.decode_whole(cfg, W, codes, taps=a)
    O.decode_whole(cfg, W, c2, taps=b)
    changed = np.flatnonzero(np.any(a["final_ln"] != b["final_ln"], axis=1))
    last = t0 + (cfg["pre_kernel"] - 1) + cfg["n_layers"] * window
    assert last < codes.shape[0] - 1
    np.testing.assert_array_equal(changed, np.arange(t0, last + 1))


def test_float32_mode_close_to_float64(tiny):
    cfg, W, codes, whole = tiny
    got = O.decode_whole(cfg, W, codes, dtype=np.float32)
    assert got.dtype == np.float32
    rel = np.linalg.norm(got - whole) / np.linalg.norm(whole)
    assert rel < 1e-5


@pytest.mark.parametrize("schedule", [[1] * 12 + [28], [13, 27]])
def test_f16_operand_mode_streamed_equals_whole(mini, schedule):
    cfg, W, codes, whole = mini
    whole16 = O.decode_whole(cfg, W, codes, operands="f16")
    got, _ = O.decode_schedule(cfg, W, codes, schedule, operands="f16")
    np.testing.assert_allclose(got, whole16, rtol=0, atol=1e-12)
    # the rounding is applied and moves the result, but only by fp16-operand error
    rel = np.linalg.norm(whole16 - whole) / np.linalg.norm(whole)
    assert 1e-6 < rel < 5e-2


def test_stored_full_size_values_are_consistent():
    """The stored full-size oracle values (tests/golden, written by
    make_golden.py from the oracle alone): the same sample grid in both modes,
    outputs within tanh's range, and the fp16-operand decode differs from the
    float64 one by fp16 rounding error only (rel-L2 between 1e-3 and 5e-2)."""
    import os

    here = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
    g64 = np.load(os.path.join(here, "qwen3_whole.npz"))
    g16 = np.load(os.path.join(here, "qwen3_whole_f16.npz"))
    assert np.array_equal(g64["idx"], g16["idx"]) and g64["idx"][-1] == 250 * S.QWEN3["hop"] - 1
    for g in (g64, g16):
        assert np.all(np.abs(g["pcm"]) <= 1.0)
        np.testing.assert_allclose(g["pcm"], np.tanh(g["pre"]), rtol=0, atol=1e-12)
    for key in ("pre", "pcm"):
        rel = np.linalg.norm(g16[key] - g64[key]) / np.linalg.norm(g64[key])
        assert 1e-3 < rel < 5e-2, (key, rel)
    # int8 weights move this random-init decoder much more than fp16 operands
    # (measured: pre-tanh 6.6e-2, PCM 0.14); the stored values are its own
    g8 = np.load(os.path.join(here, "qwen3_whole_int8.npz"))
    assert np.array_equal(g8["idx"], g64["idx"])
    np.testing.assert_allclose(g8["pcm"], np.tanh(g8["pre"]), rtol=0, atol=1e-12)
    for key in ("pre", "pcm"):
        rel = np.linalg.norm(g8[key] - g64[key]) / np.linalg.norm(g64[key])
        assert 1e-2 < rel < 0.3, (key, rel)


@pytest.mark.parametrize("schedule", [[1] * 12 + [28], [13, 27]])
def test_int8_weights_streamed_equals_whole(mini, schedule):
    cfg, W, codes, whole = mini
    W8 = O.quantize_weights_int8(W)
    whole8 = O.decode_whole(cfg, W8, codes)
    got, _ = O.decode_schedule(cfg, W8, codes, schedule)
    np.testing.assert_allclose(got, whole8, rtol=0, atol=1e-12)
    # quantization moves the output, by int8 step error only
    rel = np.linalg.norm(whole8 - whole) / np.linalg.norm(whole)
    assert 1e-5 < rel < 5e-2
