"""Plain CPU oracle of the streaming code2wav decoder (numpy, float64 by default).

TEST INFRASTRUCTURE ONLY: imported by tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py, never by the product path.

What is computed, and where it is described
-------------------------------------------
"Edge TTS design (vLLM-Omni-compatible)", section 1.3 (Codec / vocoder): the
Qwen3-TTS-12Hz decoder is an RVQ embedding sum, a causal conv, an 8-layer
sliding-window (72-frame) transformer, 2x2 upsampling and a BigVGAN/Snake stack,
in fp32, 1920 samples per frame at 24 kHz, with cross-chunk state made of the
conv context and the 72-frame attention window.  Section 2.2 (IDecoderAdapter)
and 2.3 (state ownership) fix the chunked, stateful call shape; section 4
(ExecuTorch notes) asks for the state as explicit inputs and outputs.

"blixt/phonon", section Weights: rotary pairs are the two halves (j, j + hd/2)
of each head; transposed convolutions have kernel = 2 x stride.  Section Speed,
item 7: chunks of any size share one decoder state (a key/value ring and each
convolution's left context), and chunk size must not change the audio.

"Kokoro-82M ... ported to Core AI", ConvTranspose1d passage: a transposed
convolution equals zero insertion (stride - 1 zeros) followed by a plain
convolution with the flipped kernel.

Readings where the pages are silent (each also listed in the design notes):
every convolution is causal (left context only, the transposed convolutions
keep the first T*stride outputs); the embedding sum is a plain sum of the 16
selected codewords added in ascending codebook order; pre-norm LayerNorm with
eps 1e-5 and a final LayerNorm; 2-matrix GELU (erf) FFN; biases on every
linear; 1/sqrt(head_dim) score scale; keys at positions [t - W, t]; RoPE with
theta = 10000 on absolute frame positions counted from reset; the 2x2
upsampling is two ConvTranspose1d (stride 2, kernel 4) with no activation
between; BigVGAN stages are ConvTranspose1d then a multi-receptive-field mean
of AMP blocks, each block running, per dilation d, Snake -> conv(k, d) ->
Snake -> conv(k, 1) -> residual add; plain Snake x + sin^2(alpha x)/alpha with
no anti-aliasing filters; final Snake -> conv(k=7, C -> 1) -> tanh.

Pins (tests/test_oracle_*.py): brute-force loops on tiny shapes, the library
routines torch.nn.functional.conv1d / conv_transpose1d / layer_norm / gelu /
scaled_dot_product_attention on the CPU in float64, the zero-insertion +
flipped-kernel identity, closed-form special values of Snake, RoPE's relative
position invariance, and streamed == whole for several chunk schedules.  The
int8 weight quantizer: a hand-worked group, ties to even, the half-step error
bound, and the group layout.  The
decoder as a whole against the real Qwen3-TTS checkpoint is parity unpinned:
no trained weights or reference audio exist here.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
from scipy.special import erf


# ---------------------------------------------------------------------------
# layer primitives
# ---------------------------------------------------------------------------


def rvq_embed_sum(codebooks: np.ndarray, codes: np.ndarray) -> np.ndarray:
    """Residual-VQ decode: e[t] = sum over q of codebooks[q][codes[t, q]].

    Edge TTS design, section 1.3 (the decoder starts from the sum of the RVQ
    codewords) and section 1.2 (codebook 0 comes from the talker, 1..15 from
    the code predictor).  The sum is taken in
    ascending codebook order, one rounding per add, in the codebooks' dtype;
    numpy's pairwise np.sum is deliberately not used.  Codes outside
    [0, codebook_size) are an error.
    """
    codes = np.asarray(codes)
    Q, V, _ = codebooks.shape
    if codes.ndim != 2 or codes.shape[1] != Q:
        raise ValueError(f"codes must be [T][{Q}], got {codes.shape}")
    if codes.size and (codes.min() < 0 or codes.max() >= V):
        raise ValueError("code out of range")
    e = codebooks[0][codes[:, 0]].copy()
    for q in range(1, Q):
        e = e + codebooks[q][codes[:, q]]
    return e


def causal_conv1d(x, w, b, dilation=1, hist=None):
    """Causal dilated Conv1d on channels-last rows.

    x [N][Cin], w [Cout][Cin][k] (PyTorch layout), b [Cout].
    y[n] = b + sum_j w[:, :, j] . x[n - (k - 1 - j) * dilation], where rows before
    0 come from `hist` (the last (k-1)*dilation input rows of the previous chunk,
    oldest first) or are zero.  Returns (y, new_hist).
    """
    N, Cin = x.shape
    Cout, Cin2, k = w.shape
    assert Cin2 == Cin
    H = (k - 1) * dilation
    if hist is None:
        hist = np.zeros((H, Cin), dtype=x.dtype)
    assert hist.shape == (H, Cin)
    xp = np.concatenate([hist, x], axis=0)
    y = np.broadcast_to(b, (N, Cout)).astype(x.dtype, copy=True)
    for j in range(k):
        y += xp[j * dilation: j * dilation + N] @ np.ascontiguousarray(w[:, :, j].T)
    new_hist = xp[xp.shape[0] - H:].copy()
    return y, new_hist


def conv_transpose1d_causal(x, u, b, stride, hist=None):
    """Causal ConvTranspose1d, kernel = 2 x stride, by its scatter definition.

    x [N][Cin], u [Cin][Cout][2*stride] (PyTorch layout), b [Cout].  Every input
    row t scatters u[:, :, j]^T x[t] into output sample t*stride + j.  Output
    samples [0, N*stride) are kept: they need inputs up to row N-1 only, so no
    look-ahead is used.  Samples 0..stride-1 also receive the tail of the last
    input row of the previous chunk (`hist`, one row; zero at reset).
    Returns (y [N*stride][Cout], new_hist).
    """
    N, Cin = x.shape
    Cin2, Cout, K = u.shape
    assert Cin2 == Cin and K == 2 * stride
    s = stride
    if hist is None:
        hist = np.zeros((1, Cin), dtype=x.dtype)
    xp = np.concatenate([hist, x], axis=0)  # row i holds input time i - 1
    # z[m] holds output sample m - s
    z = np.zeros(((N + 1) * s + s, Cout), dtype=x.dtype)
    for j in range(K):
        z[j: j + (N + 1) * s: s] += xp @ np.ascontiguousarray(u[:, :, j])
    y = z[s: s + N * s] + b
    return y, xp[-1:].copy()


def snake(x, alpha):
    """Snake activation x + sin^2(alpha x) / alpha, one alpha per channel (last axis)."""
    return x + np.sin(alpha * x) ** 2 / alpha


def layer_norm(x, g, b, eps):
    """LayerNorm over the last axis with the biased variance."""
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    return (x - mu) / np.sqrt(var + eps) * g + b


def gelu(x):
    """Exact GELU: x/2 * (1 + erf(x / sqrt 2))."""
    return 0.5 * x * (1.0 + erf(x / math.sqrt(2.0)))


def rope_rotate(x, positions, theta):
    """Rotary embedding on the two halves of each head (blixt/phonon, Weights).

    x [T][H][hd]; positions [T] absolute frame indices.  For i < hd/2 with
    angle phi = p * theta^(-2i/hd):
      (x_i, x_{i+hd/2}) <- (x_i cos phi - x_{i+hd/2} sin phi,
                            x_i sin phi + x_{i+hd/2} cos phi).
    Angles, cosines and sines are evaluated in float64, then cast to x.dtype.
    """
    T, H, hd = x.shape
    half = hd // 2
    inv = theta ** (-2.0 * np.arange(half, dtype=np.float64) / hd)
    phi = np.asarray(positions, dtype=np.float64)[:, None] * inv[None, :]
    c = np.cos(phi).astype(x.dtype)[:, None, :]
    s = np.sin(phi).astype(x.dtype)[:, None, :]
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x1 * s + x2 * c], axis=-1)


def window_attention(q, k, v, qpos, kpos, window):
    """Sliding-window softmax attention.

    q [T][H][hd] at absolute positions qpos [T]; k, v [S][H][hd] at kpos [S].
    Query at position p attends the keys with position in [p - window, p]
    (the window's previous frames and itself); scores are q.k / sqrt(hd);
    softmax over those keys only.
    """
    T, H, hd = q.shape
    scores = np.einsum("thd,shd->hts", q, k) / math.sqrt(hd)
    qp = np.asarray(qpos)[:, None]
    kp = np.asarray(kpos)[None, :]
    allowed = (kp <= qp) & (kp >= qp - window)
    scores = np.where(allowed[None], scores, -np.inf)
    m = scores.max(axis=-1, keepdims=True)
    p = np.exp(scores - m)
    p = p / p.sum(axis=-1, keepdims=True)
    return np.einsum("hts,shd->thd", p, v)


def linear(x, w, b):
    return x @ w.T + b


def round_operand(a, operands):
    """Round a contraction operand to the operand format, keeping its dtype.

    operands=None leaves `a` unchanged; operands="f16" rounds every element to
    the nearest IEEE binary16 value (ties to even), the format the pages allow
    for the decoder at most ("Edge TTS design", section 1.5: quality row).
    Products and sums stay in the working dtype.
    """
    if operands is None:
        return a
    if operands != "f16":
        raise ValueError(f"unknown operand format {operands!r}")
    return np.asarray(a).astype(np.float16).astype(np.asarray(a).dtype)


# Contraction weights that the fp16-operand mode rounds: every conv, transposed
# conv and linear weight except the final C -> 1 conv (not a matrix product).
def _is_contraction_weight(name):
    return name.endswith(".weight") and not (
        ".ln" in name or name.startswith("final_ln") or name.startswith("conv_post"))


# ---------------------------------------------------------------------------
# decoder
# ---------------------------------------------------------------------------


@dataclass
class OracleState:
    """Everything one stream carries between chunks (Edge TTS design, 2.3).

    pos: frames decoded since reset.  kv[l]: (k, v) of the last `window` frames
    of layer l, RoPE already applied, oldest first ([n][H][hd], n <= window).
    hist[name]: the last rows of each convolution's input, oldest first.
    """

    pos: int = 0
    kv: list = field(default_factory=list)
    hist: dict = field(default_factory=dict)

    def copy(self):
        return OracleState(self.pos, [(k.copy(), v.copy()) for k, v in self.kv],
                           {n: h.copy() for n, h in self.hist.items()})


def new_state(cfg, dtype=np.float64) -> OracleState:
    """A fresh stream: position 0, no keys, zero conv context (Edge TTS design, 2.2 reset())."""
    H, hd = cfg["n_heads"], cfg["head_dim"]
    st = OracleState()
    st.kv = [(np.zeros((0, H, hd), dtype), np.zeros((0, H, hd), dtype)) for _ in range(cfg["n_layers"])]
    return st


def _get_hist(state, name, rows, ch, dtype):
    h = state.hist.get(name)
    if h is None:
        h = np.zeros((rows, ch), dtype)
    return h


def cast_weights(weights, dtype):
    return {k: np.asarray(v).astype(dtype, copy=False) for k, v in weights.items()}


def transformer_layer(h, W, l, cache, positions, cfg, operands=None):
    """One pre-norm layer: windowed self-attention with RoPE, then a GELU FFN.

    h [T][d] at absolute positions `positions`; cache = (k, v) of earlier
    frames.  Returns (h_out, new_cache) where new_cache keeps the last
    `window` frames.  operands="f16" rounds the inputs of the four linear
    products (their weights are expected already rounded).
    """
    r = lambda a: round_operand(a, operands)  # noqa: E731
    p = f"layers.{l}."
    T, d = h.shape
    H, hd, Wn = cfg["n_heads"], cfg["head_dim"], cfg["window"]
    eps = cfg["ln_eps"]
    u = layer_norm(h, W[p + "ln1.weight"], W[p + "ln1.bias"], eps)
    q = linear(r(u), W[p + "q_proj.weight"], W[p + "q_proj.bias"]).reshape(T, H, hd)
    k = linear(r(u), W[p + "k_proj.weight"], W[p + "k_proj.bias"]).reshape(T, H, hd)
    v = linear(r(u), W[p + "v_proj.weight"], W[p + "v_proj.bias"]).reshape(T, H, hd)
    q = rope_rotate(q, positions, cfg["rope_theta"])
    k = rope_rotate(k, positions, cfg["rope_theta"])
    kc, vc = cache
    K = np.concatenate([kc, k], axis=0)
    V = np.concatenate([vc, v], axis=0)
    p0 = int(positions[0])
    kpos = np.arange(p0 - kc.shape[0], p0 + T)
    o = window_attention(q, K, V, positions, kpos, Wn).reshape(T, d)
    h = h + linear(r(o), W[p + "o_proj.weight"], W[p + "o_proj.bias"])
    u = layer_norm(h, W[p + "ln2.weight"], W[p + "ln2.bias"], eps)
    f = gelu(linear(r(u), W[p + "fc1.weight"], W[p + "fc1.bias"]))
    h = h + linear(r(f), W[p + "fc2.weight"], W[p + "fc2.bias"])
    keep = min(Wn, K.shape[0])
    return h, (K[K.shape[0] - keep:].copy(), V[V.shape[0] - keep:].copy())


# ---------------------------------------------------------------------------
# int8 weights ("blixt/phonon", section Weights)
# ---------------------------------------------------------------------------

# A weight tensor of at least this many values is stored as int8 ...
INT8_MIN_VALUES = 16384
# ... with one fp16 scale per this many consecutive values of a row.
INT8_GROUP = 32


def quantize_rows_int8(rows):
    """int8 values and fp16 scales of a [n][K] matrix, one scale per 32
    consecutive values of a row (K a multiple of 32), as the phonon page's
    weight converter does: round the values to fp16; the scale is the largest
    magnitude of the 32 rounded values over 127, rounded to fp16; each value is
    the nearest integer to value / scale, ties to even.  The page does this in
    its offline weight converter and does not state the precision of the two
    divisions; here both are correctly rounded fp32 divisions, as in the
    device quantizer (where floating point decides an integer, both
    implementations decide in the same precision).  On the Qwen3-shaped
    decoder's weights float64 divisions give the same int8 values and scales
    for every one of the 242,862,080 quantized values.  A group of zeros gets
    scale 0 and values 0.

    Returns (q int8 [n][K], scale float16 [n][K/32])."""
    v = np.asarray(rows, dtype=np.float32).astype(np.float16).astype(np.float32)
    n, K = v.shape
    if K % INT8_GROUP:
        raise ValueError("row length must be a multiple of 32")
    g = v.reshape(n, K // INT8_GROUP, INT8_GROUP)
    amax = np.abs(g).max(axis=2)
    scale = (amax / np.float32(127)).astype(np.float16)
    s = scale.astype(np.float32)[:, :, None]
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.where(s > 0, np.rint(g / np.where(s > 0, s, np.float32(1))), np.float32(0))
    return q.astype(np.int8).reshape(n, K), scale


def dequantize_rows_int8(q, scale):
    """q * scale per group, in float64 (exact: 8-bit integer times fp16)."""
    n, K = q.shape
    out = q.astype(np.float64).reshape(n, K // INT8_GROUP, INT8_GROUP) * scale.astype(np.float64)[:, :, None]
    return out.reshape(n, K)


def _is_transposed_conv(name):
    return name.startswith("ups.") or name.endswith(".up.weight")


def int8_eligible(name, shape):
    """Whether a weight is stored as int8: a matrix-product weight of at least
    INT8_MIN_VALUES values whose rows (one output channel at one tap, along the
    input channels) split into whole groups of 32."""
    if not _is_contraction_weight(name) or int(np.prod(shape)) < INT8_MIN_VALUES:
        return False
    cin = shape[0] if _is_transposed_conv(name) else shape[1]
    return cin % INT8_GROUP == 0


def _rows_of(name, w):
    """The weight as [rows][in]: Linear [out][in] as is; Conv1d [out][in][k]
    and ConvTranspose1d [in][out][k] as [out][k][in] flattened to rows."""
    if w.ndim == 2:
        return w, lambda r: r
    if _is_transposed_conv(name):
        cin, cout, k = w.shape
        return (np.ascontiguousarray(w.transpose(1, 2, 0)).reshape(cout * k, cin),
                lambda r: r.reshape(cout, k, cin).transpose(2, 0, 1))
    cout, cin, k = w.shape
    return (np.ascontiguousarray(w.transpose(0, 2, 1)).reshape(cout * k, cin),
            lambda r: r.reshape(cout, k, cin).transpose(0, 2, 1))


def quantize_weights_int8(weights):
    """The weights with every int8-eligible tensor replaced by its dequantized
    values q * scale (float64, same shape); the others unchanged."""
    out = {}
    for name, w in weights.items():
        w = np.asarray(w)
        if int8_eligible(name, w.shape):
            rows, back = _rows_of(name, w)
            out[name] = np.ascontiguousarray(back(dequantize_rows_int8(*quantize_rows_int8(rows))))
        else:
            out[name] = w
    return out


def cast_operand_weights(weights, dtype, operands):
    """Weights in `dtype`, with every contraction weight rounded to the operand format."""
    W = cast_weights(weights, dtype)
    if operands is None:
        return W
    return {k: (round_operand(v, operands) if _is_contraction_weight(k) else v) for k, v in W.items()}


def decode_chunk(cfg, weights, codes, state: OracleState, dtype=np.float64, taps=None, operands=None):
    """Decode one chunk of T frames of one stream; returns (pcm [T*hop], state).

    `state` is updated in place and returned.  `taps`, if a dict, receives each
    stage's output (channels-last) for stage-by-stage comparison.
    operands="f16": every matrix product (convs, transposed convs, linears; not
    the final C -> 1 conv) takes fp16-rounded operands -- weights, inputs and
    history rows -- and sums the exact products in `dtype`; everything else
    (embedding sum, LayerNorm, attention, GELU, Snake, residuals, biases) stays
    in `dtype`.
    """
    W = cast_operand_weights(weights, dtype, operands)
    r = lambda a: round_operand(a, operands)  # noqa: E731
    codes = np.asarray(codes)
    T = codes.shape[0]

    def tap(name, val):
        if taps is not None:
            taps[name] = val.copy()

    e = rvq_embed_sum(W["codebooks"], codes)
    tap("embed", e)
    h, state.hist["pre_conv"] = causal_conv1d(
        r(e), W["pre_conv.weight"], W["pre_conv.bias"], 1,
        r(_get_hist(state, "pre_conv", cfg["pre_kernel"] - 1, cfg["embed_dim"], dtype)))
    tap("pre_conv", h)
    positions = state.pos + np.arange(T)
    for l in range(cfg["n_layers"]):
        h, state.kv[l] = transformer_layer(h, W, l, state.kv[l], positions, cfg, operands)
        tap(f"layer{l}", h)
    x = layer_norm(h, W["final_ln.weight"], W["final_ln.bias"], cfg["ln_eps"])
    tap("final_ln", x)
    d = cfg["model_dim"]
    for i, s in enumerate(cfg["up_strides"]):
        x, state.hist[f"ups.{i}"] = conv_transpose1d_causal(
            r(x), W[f"ups.{i}.weight"], W[f"ups.{i}.bias"], s, r(_get_hist(state, f"ups.{i}", 1, d, dtype)))
        tap(f"up{i}", x)
    x, state.hist["conv_pre"] = causal_conv1d(
        r(x), W["conv_pre.weight"], W["conv_pre.bias"], 1,
        r(_get_hist(state, "conv_pre", cfg["conv_pre_kernel"] - 1, d, dtype)))
    tap("conv_pre", x)
    chans = cfg["stage_channels"]
    n_res = len(cfg["res_kernels"])
    for si, rate in enumerate(cfg["rates"]):
        p = f"stages.{si}."
        cin, c = chans[si], chans[si + 1]
        x, state.hist[p + "up"] = conv_transpose1d_causal(
            r(x), W[p + "up.weight"], W[p + "up.bias"], rate, r(_get_hist(state, p + "up", 1, cin, dtype)))
        tap(f"stage{si}.up", x)
        acc = None
        for j, k in enumerate(cfg["res_kernels"]):
            y = x
            for i, dil in enumerate(cfg["dilations"]):
                q = p + f"blocks.{j}.{i}."
                a = snake(y, W[q + "act1.alpha"])
                t, state.hist[q + "conv1"] = causal_conv1d(
                    r(a), W[q + "conv1.weight"], W[q + "conv1.bias"], dil,
                    r(_get_hist(state, q + "conv1", (k - 1) * dil, c, dtype)))
                bb = snake(t, W[q + "act2.alpha"])
                uo, state.hist[q + "conv2"] = causal_conv1d(
                    r(bb), W[q + "conv2.weight"], W[q + "conv2.bias"], 1,
                    r(_get_hist(state, q + "conv2", k - 1, c, dtype)))
                y = y + uo
            acc = y if acc is None else acc + y
        x = acc / n_res
        tap(f"stage{si}", x)
    a = snake(x, W["act_post.alpha"])
    z, state.hist["conv_post"] = causal_conv1d(
        a, W["conv_post.weight"], W["conv_post.bias"], 1,
        _get_hist(state, "conv_post", cfg["post_kernel"] - 1, chans[-1], dtype))
    tap("pre_tanh", z[:, 0])
    pcm = np.tanh(z[:, 0])
    tap("pcm", pcm)
    state.pos += T
    return pcm, state


def decode_whole(cfg, weights, codes, dtype=np.float64, taps=None, operands=None):
    """Decode a whole sequence of one stream from a fresh state."""
    pcm, _ = decode_chunk(cfg, weights, codes, new_state(cfg, dtype), dtype, taps, operands)
    return pcm


def decode_schedule(cfg, weights, codes, schedule, dtype=np.float64, state=None, operands=None):
    """Decode one stream chunk by chunk (chunk lengths in `schedule`), concatenating the PCM."""
    W = cast_operand_weights(weights, dtype, operands)
    st = new_state(cfg, dtype) if state is None else state
    out, t0 = [], 0
    for n in schedule:
        pcm, st = decode_chunk(cfg, W, codes[t0:t0 + n], st, dtype, operands=operands)
        out.append(pcm)
        t0 += n
    return np.concatenate(out), st
