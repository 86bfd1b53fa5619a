"""Pins of the oracle's layer primitives against things other than itself.

Each test fixes a primitive by brute force on tiny shapes, by a closed form or
special value, by an identity the pages state, or by an independent library
routine (PyTorch on the CPU in float64).  All CPU-only.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import synthetic as S
from oracle import decoder as O

RNG = np.random.default_rng(1234)


# ---------------------------------------------------------------------------
# RVQ embedding sum (Edge TTS design, 1.3)
# ---------------------------------------------------------------------------


def test_rvq_sum_matches_scalar_loop_bitwise():
    Q, V, D, T = 16, 37, 9, 11
    cb = RNG.standard_normal((Q, V, D)).astype(np.float32)
    codes = RNG.integers(0, V, (T, Q))
    got = O.rvq_embed_sum(cb, codes)
    assert got.dtype == np.float32
    for t in range(T):
        for c in range(D):
            acc = np.float32(0.0)
            for q in range(Q):
                acc = np.float32(acc + cb[q, codes[t, q], c]) if q else cb[q, codes[t, q], c]
            assert got[t, c] == acc  # one fp32 rounding per add, ascending q


def test_rvq_sum_equals_one_hot_product():
    Q, V, D, T = 16, 23, 7, 5
    cb = RNG.standard_normal((Q, V, D))
    codes = RNG.integers(0, V, (T, Q))
    onehot = np.zeros((T, Q, V))
    for t in range(T):
        for q in range(Q):
            onehot[t, q, codes[t, q]] = 1.0
    ref = np.einsum("tqv,qvd->td", onehot, cb)
    np.testing.assert_allclose(O.rvq_embed_sum(cb, codes), ref, rtol=0, atol=1e-13)


def test_rvq_sum_rejects_out_of_range_codes():
    cb = np.zeros((16, 8, 4), np.float32)
    with pytest.raises(ValueError):
        O.rvq_embed_sum(cb, np.full((2, 16), 8))
    with pytest.raises(ValueError):
        O.rvq_embed_sum(cb, np.full((2, 16), -1))


# ---------------------------------------------------------------------------
# causal dilated Conv1d
# ---------------------------------------------------------------------------


def _conv_brute(x, w, b, d, hist):
    N, Cin = x.shape
    Cout, _, k = w.shape
    H = (k - 1) * d
    full = np.concatenate([hist, x]) if H else x
    y = np.zeros((N, Cout))
    for n in range(N):
        for o in range(Cout):
            s = b[o]
            for j in range(k):
                src = n - (k - 1 - j) * d  # input row, negative = history
                for c in range(Cin):
                    s += w[o, c, j] * full[src + H, c]
            y[n, o] = s
    return y


@pytest.mark.parametrize("k,d", [(1, 1), (3, 1), (3, 3), (7, 1), (7, 5), (11, 3)])
@pytest.mark.parametrize("with_hist", [False, True])
def test_causal_conv_brute_force(k, d, with_hist):
    N, Cin, Cout = 9, 3, 4
    x = RNG.standard_normal((N, Cin))
    w = RNG.standard_normal((Cout, Cin, k))
    b = RNG.standard_normal(Cout)
    H = (k - 1) * d
    hist = RNG.standard_normal((H, Cin)) if with_hist else np.zeros((H, Cin))
    y, nh = O.causal_conv1d(x, w, b, d, hist if with_hist else None)
    np.testing.assert_allclose(y, _conv_brute(x, w, b, d, hist), rtol=0, atol=1e-12)
    # the new history is the last H rows of (history, input)
    np.testing.assert_array_equal(nh, np.concatenate([hist, x])[N + H - H:] if H else nh)
    assert nh.shape == (H, Cin)


@pytest.mark.parametrize("k,d", [(3, 1), (7, 3), (11, 5)])
def test_causal_conv_matches_torch_left_padded(k, d):
    N, Cin, Cout = 40, 6, 5
    x = RNG.standard_normal((N, Cin))
    w = RNG.standard_normal((Cout, Cin, k))
    b = RNG.standard_normal(Cout)
    y, _ = O.causal_conv1d(x, w, b, d)
    xt = torch.from_numpy(x.T[None])
    ref = F.conv1d(F.pad(xt, ((k - 1) * d, 0)), torch.from_numpy(w), torch.from_numpy(b), dilation=d)
    np.testing.assert_allclose(y, ref[0].numpy().T, rtol=0, atol=1e-12)


def test_causal_conv_history_is_exact_continuation():
    k, d, Cin, Cout = 7, 3, 4, 3
    x = RNG.standard_normal((30, Cin))
    w = RNG.standard_normal((Cout, Cin, k))
    b = RNG.standard_normal(Cout)
    whole, _ = O.causal_conv1d(x, w, b, d)
    y1, h = O.causal_conv1d(x[:5], w, b, d)   # chunk shorter than the history
    y2, h = O.causal_conv1d(x[5:6], w, b, d, h)
    y3, _ = O.causal_conv1d(x[6:], w, b, d, h)
    np.testing.assert_allclose(np.concatenate([y1, y2, y3]), whole, rtol=0, atol=1e-12)


# ---------------------------------------------------------------------------
# causal ConvTranspose1d, kernel = 2 x stride (blixt/phonon, Weights;
# Kokoro on Core AI, ConvTranspose1d passage)
# ---------------------------------------------------------------------------


@pytest.mark.parametrize("s", [2, 3, 4, 5, 8])
def test_conv_transpose_matches_torch_trimmed(s):
    N, Cin, Cout = 13, 5, 4
    x = RNG.standard_normal((N, Cin))
    u = RNG.standard_normal((Cin, Cout, 2 * s))
    b = RNG.standard_normal(Cout)
    y, nh = O.conv_transpose1d_causal(x, u, b, s)
    ref = F.conv_transpose1d(torch.from_numpy(x.T[None]), torch.from_numpy(u), torch.from_numpy(b), stride=s)
    np.testing.assert_allclose(y, ref[0].numpy().T[: N * s], rtol=0, atol=1e-12)
    np.testing.assert_array_equal(nh, x[-1:])


@pytest.mark.parametrize("s", [2, 3, 5])
def test_conv_transpose_with_history_matches_torch(s):
    N, Cin, Cout = 7, 4, 3
    x = RNG.standard_normal((N, Cin))
    h = RNG.standard_normal((1, Cin))
    u = RNG.standard_normal((Cin, Cout, 2 * s))
    b = RNG.standard_normal(Cout)
    y, _ = O.conv_transpose1d_causal(x, u, b, s, h)
    xh = np.concatenate([h, x])
    ref = F.conv_transpose1d(torch.from_numpy(xh.T[None]), torch.from_numpy(u), torch.from_numpy(b), stride=s)
    np.testing.assert_allclose(y, ref[0].numpy().T[s: s + N * s], rtol=0, atol=1e-12)


@pytest.mark.parametrize("s", [2, 3, 4])
def test_conv_transpose_equals_zero_insertion_and_flipped_conv(s):
    """Core AI Kokoro page: insert stride-1 zeros, then a plain conv with the
    flipped kernel (in/out swapped), padded by k-1 on both sides."""
    N, Cin, Cout = 6, 3, 2
    K = 2 * s
    x = RNG.standard_normal((N, Cin))
    u = RNG.standard_normal((Cin, Cout, K))
    b = RNG.standard_normal(Cout)
    z = np.zeros(((N - 1) * s + 1, Cin))
    z[::s] = x
    zp = np.concatenate([np.zeros((K - 1, Cin)), z, np.zeros((K - 1, Cin))])
    wf = u[:, :, ::-1].transpose(1, 0, 2)  # [Cout][Cin][K], flipped taps
    L = zp.shape[0] - K + 1
    full = np.zeros((L, Cout))
    for n in range(L):
        for j in range(K):
            full[n] += wf[:, :, j] @ zp[n + j]
    full += b
    y, _ = O.conv_transpose1d_causal(x, u, b, s)
    np.testing.assert_allclose(y, full[: N * s], rtol=0, atol=1e-12)


@pytest.mark.parametrize("s", [2, 3, 8])
def test_conv_transpose_polyphase_brute_force(s):
    """y[t*s + p] = b + U[:,:,p]^T x[t] + U[:,:,p+s]^T x[t-1] (kernel 2s: two taps per phase)."""
    N, Cin, Cout = 5, 3, 2
    x = RNG.standard_normal((N, Cin))
    h = RNG.standard_normal((1, Cin))
    u = RNG.standard_normal((Cin, Cout, 2 * s))
    b = RNG.standard_normal(Cout)
    y, _ = O.conv_transpose1d_causal(x, u, b, s, h)
    for t in range(N):
        prev = h[0] if t == 0 else x[t - 1]
        for p in range(s):
            for o in range(Cout):
                ref = b[o] + sum(u[c, o, p] * x[t, c] + u[c, o, p + s] * prev[c] for c in range(Cin))
                assert abs(y[t * s + p, o] - ref) < 1e-12


# ---------------------------------------------------------------------------
# Snake, LayerNorm, GELU
# ---------------------------------------------------------------------------


def test_snake_special_values():
    alpha = np.array([0.5, 1.0, 1.5, 0.75])
    assert np.all(O.snake(np.zeros(4), alpha) == 0.0)
    m = np.array([1.0, -2.0, 3.0, 7.0])
    x = m * np.pi / alpha  # sin(alpha x) = 0
    np.testing.assert_allclose(O.snake(x, alpha), x, rtol=0, atol=1e-12)
    x = (m + 0.5) * np.pi / alpha  # sin^2(alpha x) = 1
    np.testing.assert_allclose(O.snake(x, alpha), x + 1.0 / alpha, rtol=0, atol=1e-12)


def test_snake_closed_form_scalar():
    for _ in range(50):
        x, a = RNG.standard_normal() * 30, RNG.uniform(0.5, 1.5)
        assert abs(O.snake(np.array([x]), np.array([a]))[0] - (x + math.sin(a * x) ** 2 / a)) < 1e-12
        # sin^2(ax)/a = (1 - cos 2ax) / (2a)
        assert abs(O.snake(np.array([x]), np.array([a]))[0] - (x + (1 - math.cos(2 * a * x)) / (2 * a))) < 1e-11


def test_layer_norm_matches_torch():
    x = RNG.standard_normal((7, 33)) * 3 + 1
    g, b = RNG.standard_normal(33), RNG.standard_normal(33)
    ref = F.layer_norm(torch.from_numpy(x), (33,), torch.from_numpy(g), torch.from_numpy(b), eps=1e-5)
    np.testing.assert_allclose(O.layer_norm(x, g, b, 1e-5), ref.numpy(), rtol=0, atol=1e-12)


def test_gelu_matches_torch_and_symmetry():
    x = np.linspace(-8, 8, 1001)
    ref = F.gelu(torch.from_numpy(x), approximate="none").numpy()
    np.testing.assert_allclose(O.gelu(x), ref, rtol=0, atol=1e-14)
    np.testing.assert_allclose(O.gelu(x) - O.gelu(-x), x, rtol=0, atol=1e-13)
    assert O.gelu(np.array([0.0]))[0] == 0.0


# ---------------------------------------------------------------------------
# RoPE (blixt/phonon, Weights: rotary pairs as halves j, j + hd/2)
# ---------------------------------------------------------------------------


def test_rope_is_complex_rotation_of_half_pairs():
    T, H, hd, theta = 5, 3, 8, 10000.0
    x = RNG.standard_normal((T, H, hd))
    pos = np.array([0, 1, 7, 100, 1499])
    y = O.rope_rotate(x, pos, theta)
    half = hd // 2
    for t in range(T):
        for h in range(H):
            for i in range(half):
                z = complex(x[t, h, i], x[t, h, i + half])
                w = z * complex(math.cos(pos[t] * theta ** (-2 * i / hd)), math.sin(pos[t] * theta ** (-2 * i / hd)))
                assert abs(y[t, h, i] - w.real) < 1e-12 and abs(y[t, h, i + half] - w.imag) < 1e-12
    np.testing.assert_array_equal(O.rope_rotate(x[:1], np.array([0]), theta), x[:1])


def test_rope_scores_depend_only_on_relative_position():
    hd = 16
    q = RNG.standard_normal((1, 1, hd))
    k = RNG.standard_normal((1, 1, hd))
    for p, s in [(5, 2), (80, 9), (1400, 1399)]:
        base = (O.rope_rotate(q, [p], 1e4) * O.rope_rotate(k, [s], 1e4)).sum()
        for shift in (1, 37, 1000):
            moved = (O.rope_rotate(q, [p + shift], 1e4) * O.rope_rotate(k, [s + shift], 1e4)).sum()
            assert abs(moved - base) < 1e-10


# ---------------------------------------------------------------------------
# sliding-window attention
# ---------------------------------------------------------------------------


def test_window_attention_wide_window_is_causal_sdpa():
    T, H, hd = 12, 3, 8
    q, k, v = (RNG.standard_normal((T, H, hd)) for _ in range(3))
    pos = np.arange(T)
    got = O.window_attention(q, k, v, pos, pos, window=T)
    tq, tk, tv = (torch.from_numpy(a.transpose(1, 0, 2)) for a in (q, k, v))
    ref = F.scaled_dot_product_attention(tq, tk, tv, is_causal=True).numpy().transpose(1, 0, 2)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("window", [0, 1, 3, 5])
def test_window_attention_brute_force(window):
    T, S0, H, hd = 6, 4, 2, 4  # 4 cached keys before the chunk
    q = RNG.standard_normal((T, H, hd))
    k = RNG.standard_normal((S0 + T, H, hd))
    v = RNG.standard_normal((S0 + T, H, hd))
    p0 = 10
    qpos = np.arange(p0, p0 + T)
    kpos = np.arange(p0 - S0, p0 + T)
    got = O.window_attention(q, k, v, qpos, kpos, window)
    for t in range(T):
        for h in range(H):
            keys = [j for j in range(S0 + T) if qpos[t] - window <= kpos[j] <= qpos[t]]
            sc = [sum(q[t, h, i] * k[j, h, i] for i in range(hd)) / math.sqrt(hd) for j in keys]
            m = max(sc)
            e = [math.exp(s - m) for s in sc]
            z = sum(e)
            for i in range(hd):
                ref = sum(e[a] / z * v[keys[a], h, i] for a in range(len(keys)))
                assert abs(got[t, h, i] - ref) < 1e-12


# ---------------------------------------------------------------------------
# one transformer layer against torch modules
# ---------------------------------------------------------------------------


def test_transformer_layer_matches_torch_composition():
    import synthetic as S
    cfg = dict(S.MINI)
    W = {k: v.astype(np.float64) for k, v in S.make_weights(cfg, 7).items()}
    T, d, H, hd = 9, cfg["model_dim"], cfg["n_heads"], cfg["head_dim"]
    h = RNG.standard_normal((T, d))
    pos = np.arange(T)
    empty = (np.zeros((0, H, hd)), np.zeros((0, H, hd)))
    got, (kc, vc) = O.transformer_layer(h, W, 0, empty, pos, cfg)

    tw = {k: torch.from_numpy(v) for k, v in W.items()}
    x = torch.from_numpy(h)
    p = "layers.0."
    u = F.layer_norm(x, (d,), tw[p + "ln1.weight"], tw[p + "ln1.bias"], eps=cfg["ln_eps"])
    q = F.linear(u, tw[p + "q_proj.weight"], tw[p + "q_proj.bias"]).view(T, H, hd)
    k = F.linear(u, tw[p + "k_proj.weight"], tw[p + "k_proj.bias"]).view(T, H, hd)
    v = F.linear(u, tw[p + "v_proj.weight"], tw[p + "v_proj.bias"]).view(T, H, hd)
    # rotate-half RoPE written with torch ops
    half = hd // 2
    inv = cfg["rope_theta"] ** (-torch.arange(half, dtype=torch.float64) * 2 / hd)
    ang = torch.arange(T, dtype=torch.float64)[:, None] * inv[None]
    cos, sin = ang.cos()[:, None], ang.sin()[:, None]

    def rot(a):
        a1, a2 = a[..., :half], a[..., half:]
        return torch.cat([a1 * cos - a2 * sin, a1 * sin + a2 * cos], -1)

    q, k = rot(q), rot(k)
    i = torch.arange(T)
    mask = (i[None, :] <= i[:, None]) & (i[None, :] >= i[:, None] - cfg["window"])
    o = F.scaled_dot_product_attention(q.transpose(0, 1), k.transpose(0, 1), v.transpose(0, 1), attn_mask=mask)
    o = o.transpose(0, 1).reshape(T, d)
    x = x + F.linear(o, tw[p + "o_proj.weight"], tw[p + "o_proj.bias"])
    u = F.layer_norm(x, (d,), tw[p + "ln2.weight"], tw[p + "ln2.bias"], eps=cfg["ln_eps"])
    x = x + F.linear(F.gelu(F.linear(u, tw[p + "fc1.weight"], tw[p + "fc1.bias"])),
                     tw[p + "fc2.weight"], tw[p + "fc2.bias"])
    np.testing.assert_allclose(got, x.numpy(), rtol=0, atol=1e-11)
    # the cache keeps the last `window` rotated keys and values
    assert kc.shape[0] == cfg["window"]
    np.testing.assert_allclose(kc, k.numpy()[-cfg["window"]:], rtol=0, atol=1e-12)
    np.testing.assert_allclose(vc, v.numpy()[-cfg["window"]:], rtol=0, atol=1e-12)


# ---------------------------------------------------------------------------
# fp16-operand mode: rounding of contraction operands
# ---------------------------------------------------------------------------


def test_round_operand_matches_ieee_half():
    x = np.concatenate([RNG.standard_normal(10000) * 50, RNG.standard_normal(1000) * 1e-5,
                        [0.0, -0.0, 1.0 + 2.0 ** -11, 1.0 + 3 * 2.0 ** -11, 65504.0, 6.1e-5, 2049.0, 2051.0]])
    # float32-representable inputs: torch converts float64 -> float16 through
    # float32, which is a single rounding only for such values
    x = x.astype(np.float32).astype(np.float64)
    ref = torch.from_numpy(x).to(torch.float16).to(torch.float64).numpy()
    np.testing.assert_array_equal(O.round_operand(x, "f16"), ref)
    # ties go to even: 1 + 2^-11 is halfway between 1 and 1 + 2^-10
    assert O.round_operand(np.array([1.0 + 2.0 ** -11]), "f16")[0] == 1.0
    assert O.round_operand(np.array([1.0 + 3 * 2.0 ** -11]), "f16")[0] == 1.0 + 2 * 2.0 ** -10
    assert O.round_operand(x, None) is x
    with pytest.raises(ValueError):
        O.round_operand(x, "bf16")


def test_operand_rounding_covers_exactly_the_contraction_weights():
    import synthetic as S
    W = S.make_weights(S.MINI, 2)
    Wr = O.cast_operand_weights(W, np.float64, "f16")
    for name, v in W.items():
        rounded = not np.array_equal(Wr[name], v.astype(np.float64))
        is_gemm = name.endswith(".weight") and ("conv" in name or "proj" in name or "fc" in name
                                                or name.startswith("ups.") or name.endswith("up.weight"))
        is_gemm = is_gemm and not name.startswith("conv_post")
        assert rounded == is_gemm, name


# ---------------------------------------------------------------------------
# int8 weights (blixt/phonon, section Weights)
# ---------------------------------------------------------------------------


def test_int8_hand_worked_group():
    """Largest magnitude 127/256: the scale is exactly 1/256, so every multiple
    of 1/256 quantizes to its integer; halves go to the even neighbour."""
    vals = np.array([127, -127, 0, 1, -1, 5, 63.5, 62.5, -2.5, 3.5, 0.5, -0.5, 1.5, 100, -64, 2]
                    + [0] * 16, dtype=np.float64) / 256
    q, s = O.quantize_rows_int8(vals[None, :])
    assert s.dtype == np.float16 and s.shape == (1, 1) and float(s[0, 0]) == 1 / 256
    expect = [127, -127, 0, 1, -1, 5, 64, 62, -2, 4, 0, 0, 2, 100, -64, 2] + [0] * 16
    assert q.dtype == np.int8 and q[0].tolist() == expect
    np.testing.assert_array_equal(O.dequantize_rows_int8(q, s)[0], np.array(expect) / 256)


def test_int8_values_round_to_fp16_first():
    """The scale comes from the fp16-rounded values: 1 + 2^-12 rounds to 1 in
    fp16, so a group whose largest value is 1 + 2^-12 gets scale fp16(1/127)."""
    g = np.zeros(32)
    g[0] = 1 + 2.0 ** -12
    q, s = O.quantize_rows_int8(g[None, :])
    assert float(s[0, 0]) == float(np.float16(np.float32(1) / np.float32(127)))
    assert q[0, 0] == 127


def test_int8_error_bound_and_range():
    rng = np.random.default_rng(5)
    w = rng.normal(0, 0.02, size=(40, 256)) * rng.uniform(0.01, 10, size=(40, 1))
    w[3, 32:64] = 0  # an all-zero group
    q, s = O.quantize_rows_int8(w)
    v16 = w.astype(np.float16).astype(np.float64)
    deq = O.dequantize_rows_int8(q, s)
    step = np.repeat(s.astype(np.float64), 32, axis=1)
    # every value within half a step of its fp16 value, the largest of each group at +-127
    assert np.all(np.abs(deq - v16) <= step / 2 * (1 + 1e-6))
    gmax = np.abs(q.astype(np.int64)).reshape(40, 8, 32).max(axis=2)
    assert np.all((gmax == 127) | (s == 0))
    assert s[3, 1] == 0 and np.all(q[3, 32:64] == 0)
    # the scale is the group maximum over 127 to fp16 precision (normal fp16
    # scales; a scale below 2^-14 is subnormal and coarser, as fp16 is)
    amax = np.abs(v16).reshape(40, 8, 32).max(axis=2)
    normal = s.astype(np.float64) >= 2.0 ** -14
    assert normal.sum() > 200
    assert np.all(np.abs(s.astype(np.float64)[normal] * 127 / amax[normal] - 1) <= 2.0 ** -11)


def test_int8_ties_to_even_against_brute_force():
    """Brute force: for each value, the integer nearest to v/s by exhaustive
    search over -127..127 (ties broken to the even integer)."""
    rng = np.random.default_rng(6)
    w = rng.normal(0, 1, size=(6, 64)).astype(np.float32)
    w[:, 5] = np.float32(127.0) * 0.25  # group max fixes scale 0.25 ...
    w[:, 0] = 0.25 * np.array([0.5, 1.5, 2.5, -0.5, -1.5, -3.5])  # ... and ties at exact halves
    w[:, 1:5] = w[:, 6:10] = np.clip(w[:, 1:5], -30, 30)
    w[:, 32:] = np.clip(w[:, 32:], -30, 30)
    q, s = O.quantize_rows_int8(w)
    cand = np.arange(-127, 128)
    for r in range(w.shape[0]):
        for k in range(w.shape[1]):
            sc = np.float32(s[r, k // 32])
            x = np.float32(np.float16(w[r, k])) / sc
            d = np.abs(cand - np.float64(x))
            best = cand[d == d.min()]
            want = best[0] if len(best) == 1 else best[best % 2 == 0][0]
            assert q[r, k] == want, (r, k, x)
    assert q[:, 0].tolist() == [0, 2, 2, 0, -2, -4]


def test_int8_groups_are_input_channels_at_one_output_and_tap():
    """A single nonzero weight gives a nonzero scale to exactly its own group:
    32 consecutive input channels of one output channel at one tap."""
    cases = [("stages.0.blocks.0.0.conv1.weight", (8, 64, 3), (5, 40, 2)),   # Conv1d [out][in][k]
             ("stages.0.up.weight", (64, 6, 4), (50, 3, 1)),                  # ConvTranspose1d [in][out][k]
             ("layers.0.fc1.weight", (8, 64), (2, 33))]                        # Linear [out][in]
    for name, shape, pos in cases:
        w = np.zeros(shape)
        w[pos] = 127 / 256  # scale exactly 1/256: the value dequantizes exactly
        big = np.zeros((shape[0] * 4096,) + shape[1:])  # make it large enough to quantize
        big[: shape[0]] = w
        if O._is_transposed_conv(name):
            big = np.zeros((shape[0], shape[1] * 64, shape[2]))
            big[:, : shape[1]] = w
        assert O.int8_eligible(name, big.shape)
        out = O.quantize_weights_int8({name: big})[name]
        np.testing.assert_array_equal(out, big)
        rows, _ = O._rows_of(name, big)
        _, s = O.quantize_rows_int8(rows)
        assert np.count_nonzero(s) == 1
        r, grp = np.argwhere(s)[0]
        if len(shape) == 2:
            assert (r, grp) == (pos[0], pos[1] // 32)
        elif O._is_transposed_conv(name):
            cin, cout, k = big.shape
            assert (r, grp) == (pos[1] * k + pos[2], pos[0] // 32)
        else:
            cout, cin, k = big.shape
            assert (r, grp) == (pos[0] * k + pos[2], pos[1] // 32)


def test_int8_eligibility():
    el = {n for n, sh, _ in S.manifest(S.QWEN3) if O.int8_eligible(n, sh)}
    contraction = {n for n, sh, _ in S.manifest(S.QWEN3) if n.endswith(".weight") and len(sh) > 1
                   and not n.startswith("conv_post")}
    assert el == contraction and len(el) == 128
    assert not O.int8_eligible("conv_post.weight", (1, 96, 7))
    assert not O.int8_eligible("codebooks", (16, 2048, 512))
    mini = {n for n, sh, _ in S.manifest(S.MINI) if O.int8_eligible(n, sh)}
    assert "stages.1.blocks.0.0.conv1.weight" not in mini  # 64 x 64 x 3 = 12288 values
    assert "stages.1.blocks.1.0.conv1.weight" in mini      # 64 x 64 x 7
    assert "layers.0.q_proj.weight" not in mini            # 64 x 64
