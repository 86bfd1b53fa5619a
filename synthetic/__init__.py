"""Seeded synthetic inputs for the streaming code2wav decoder.

This module is the only code shared by the CPU oracle, the tests and the
benchmark.  It describes the five decoder shapes, draws random-init weights and
random codec frames from fixed seeds, and lays weights out in the flat manifest
order the C ABI reads.  It holds none of the decoder's arithmetic: no layer is
evaluated here.

Shapes follow the code2wav description on the vLLM-Omni edge-TTS design page
("Qwen3TTSTokenizerV2Decoder", section 1.3: RVQ embedding sum, causal conv,
8-layer sliding-window transformer with a 72-frame window, 2x2 upsampling,
BigVGAN/Snake stack, 1920 samples per 12.5 Hz frame at 24 kHz), with the
channel widths, kernel sizes and rates of the five workloads named below.
"""
from __future__ import annotations

import math
from collections import OrderedDict

import numpy as np

# ---------------------------------------------------------------------------
# decoder shapes
# ---------------------------------------------------------------------------


def _cfg(**kw):
    base = dict(
        n_codebooks=16,
        rope_theta=10000.0,
        ln_eps=1e-5,
        pre_kernel=3,
        n_up=2,
        up_strides=(2, 2),
        conv_pre_kernel=7,
        post_kernel=7,
    )
    base.update(kw)
    base["head_dim"] = base["model_dim"] // base["n_heads"]
    base["hop"] = int(np.prod(base["up_strides"])) * int(np.prod(base["rates"]))
    chans = [base["voc_ch0"]]
    for _ in base["rates"]:
        chans.append(chans[-1] // 2)
    base["stage_channels"] = tuple(chans)  # input width of each stage, then the output width
    return base


TINY = _cfg(
    name="tiny",
    codebook_size=256,
    embed_dim=64,
    model_dim=64,
    n_layers=1,
    n_heads=4,
    window=8,
    ffn_dim=128,
    voc_ch0=64,
    rates=(4, 3),
    res_kernels=(3,),
    dilations=(1, 3),
    alpha_init="one",
)

QWEN3 = _cfg(
    name="qwen3_12hz",
    codebook_size=2048,
    embed_dim=512,
    model_dim=1024,
    n_layers=8,
    n_heads=16,
    window=72,
    ffn_dim=4096,
    voc_ch0=1536,
    rates=(8, 5, 4, 3),
    res_kernels=(3, 7, 11),
    dilations=(1, 3, 5),
    alpha_init="uniform",
)

# A narrow decoder with every structural feature of the Qwen3-shaped one (two
# layers, a window shorter than a chunk, four stages, three AMP kernels with
# three dilations each).  It keeps CPU invariant tests and small GPU parity
# cases fast.
MINI = _cfg(
    name="mini",
    codebook_size=64,
    embed_dim=32,
    model_dim=64,
    n_layers=2,
    n_heads=4,
    window=6,
    ffn_dim=128,
    voc_ch0=256,
    rates=(3, 2, 2, 2),
    res_kernels=(3, 7, 11),
    dilations=(1, 3, 5),
    alpha_init="uniform",
)

# The five workloads.  Each names the decoder, the batch, the frames per stream,
# the chunk schedule and the code distribution.  The streamed workload decodes
# the same codes as the whole-sequence one (same code seed), since its output
# must equal that whole-sequence output.
WORKLOADS = OrderedDict(
    [
        ("tiny_b1_t32", dict(model=TINY, batch=1, frames=32, schedule="whole",
                             codes="uniform", weight_seed=0, code_seed=100)),
        ("qwen3_b1_t250_whole", dict(model=QWEN3, batch=1, frames=250, schedule="whole",
                                     codes="uniform", weight_seed=1, code_seed=101)),
        ("qwen3_b1_t250_stream", dict(model=QWEN3, batch=1, frames=250,
                                      schedule=[1] + [25] * 9 + [24],
                                      codes="uniform", weight_seed=1, code_seed=101)),
        ("qwen3_b64_chunk25", dict(model=QWEN3, batch=64, frames=25, schedule="warm_then_25",
                                   codes="uniform", weight_seed=1, code_seed=103)),
        ("qwen3_b16_t1500_zipf", dict(model=QWEN3, batch=16, frames=1500, schedule=[25] * 60,
                                      codes="zipf", weight_seed=1, code_seed=104)),
        # small-chunk streaming: chunks of 1, 2, 4 and 8 frames, and a 4-4-8-16-25 ramp
        # over the 250-frame stream's codes (so it must reproduce the whole decode)
        ("qwen3_b1_chunks_1248", dict(model=QWEN3, batch=1, frames=60,
                                      schedule=[1] * 4 + [2] * 4 + [4] * 4 + [8] * 4,
                                      codes="uniform", weight_seed=1, code_seed=105)),
        ("qwen3_b1_t250_ramp", dict(model=QWEN3, batch=1, frames=250,
                                    schedule=[4, 4, 8, 16] + [25] * 8 + [18],
                                    codes="uniform", weight_seed=1, code_seed=101)),
        # voice-clone reference: a 75-frame (6 s) prefix decoded into the state
        # without audio, then the utterance streamed 1 + 25 x 3
        ("qwen3_b1_prefix75_stream", dict(model=QWEN3, batch=1, frames=76, prefix=75,
                                          schedule=[1] + [25] * 3,
                                          codes="uniform", weight_seed=1, code_seed=106)),
    ]
)

WORKLOAD_INDEX = list(WORKLOADS.keys())


def workload(i_or_name):
    key = WORKLOAD_INDEX[i_or_name] if isinstance(i_or_name, int) else i_or_name
    return WORKLOADS[key]


def batched_warmup_frames(b: int) -> int:
    """Frames stream b of the 64-stream workload decodes (untimed) before its timed chunk.

    Streams sit at different positions: 1 + 25*(3 + b mod 4) frames, i.e. 76, 101,
    126 or 151, so every attention window is full and positions differ.
    """
    return 1 + 25 * (3 + b % 4)


# ---------------------------------------------------------------------------
# weight manifest (PyTorch-native layouts)
# ---------------------------------------------------------------------------


def manifest(cfg):
    """Ordered (name, shape, init) list of every parameter.

    Layouts are the PyTorch-native ones: Linear [out][in], Conv1d [out][in][k],
    ConvTranspose1d [in][out][k], codebooks [codebook][entry][dim].
    init is one of: "normal" (N(0, 0.02)), "ln_gain" (1 + N(0, 0.02)), "alpha".
    """
    d, De, F = cfg["model_dim"], cfg["embed_dim"], cfg["ffn_dim"]
    m = []
    m.append(("codebooks", (cfg["n_codebooks"], cfg["codebook_size"], De), "normal"))
    m.append(("pre_conv.weight", (d, De, cfg["pre_kernel"]), "normal"))
    m.append(("pre_conv.bias", (d,), "normal"))
    for l in range(cfg["n_layers"]):
        p = f"layers.{l}."
        m += [
            (p + "ln1.weight", (d,), "ln_gain"),
            (p + "ln1.bias", (d,), "normal"),
            (p + "q_proj.weight", (d, d), "normal"),
            (p + "q_proj.bias", (d,), "normal"),
            (p + "k_proj.weight", (d, d), "normal"),
            (p + "k_proj.bias", (d,), "normal"),
            (p + "v_proj.weight", (d, d), "normal"),
            (p + "v_proj.bias", (d,), "normal"),
            (p + "o_proj.weight", (d, d), "normal"),
            (p + "o_proj.bias", (d,), "normal"),
            (p + "ln2.weight", (d,), "ln_gain"),
            (p + "ln2.bias", (d,), "normal"),
            (p + "fc1.weight", (F, d), "normal"),
            (p + "fc1.bias", (F,), "normal"),
            (p + "fc2.weight", (d, F), "normal"),
            (p + "fc2.bias", (d,), "normal"),
        ]
    m.append(("final_ln.weight", (d,), "ln_gain"))
    m.append(("final_ln.bias", (d,), "normal"))
    for i, s in enumerate(cfg["up_strides"]):
        m.append((f"ups.{i}.weight", (d, d, 2 * s), "normal"))
        m.append((f"ups.{i}.bias", (d,), "normal"))
    C0 = cfg["voc_ch0"]
    m.append(("conv_pre.weight", (C0, d, cfg["conv_pre_kernel"]), "normal"))
    m.append(("conv_pre.bias", (C0,), "normal"))
    chans = cfg["stage_channels"]
    for s, r in enumerate(cfg["rates"]):
        cin, cout = chans[s], chans[s + 1]
        p = f"stages.{s}."
        m.append((p + "up.weight", (cin, cout, 2 * r), "normal"))
        m.append((p + "up.bias", (cout,), "normal"))
        for j, k in enumerate(cfg["res_kernels"]):
            for i, _dil in enumerate(cfg["dilations"]):
                q = p + f"blocks.{j}.{i}."
                m += [
                    (q + "act1.alpha", (cout,), "alpha"),
                    (q + "conv1.weight", (cout, cout, k), "normal"),
                    (q + "conv1.bias", (cout,), "normal"),
                    (q + "act2.alpha", (cout,), "alpha"),
                    (q + "conv2.weight", (cout, cout, k), "normal"),
                    (q + "conv2.bias", (cout,), "normal"),
                ]
    m.append(("act_post.alpha", (chans[-1],), "alpha"))
    m.append(("conv_post.weight", (1, chans[-1], cfg["post_kernel"]), "normal"))
    m.append(("conv_post.bias", (1,), "normal"))
    return m


def n_params(cfg) -> int:
    return int(sum(math.prod(shape) for _, shape, _ in manifest(cfg)))


def make_weights(cfg, seed: int) -> "OrderedDict[str, np.ndarray]":
    """Random-init weights, drawn in manifest order from numpy's PCG64 stream.

    Every weight, bias and codeword ~ N(0, 0.02); LayerNorm gains 1 + N(0, 0.02);
    Snake alpha = 1 for the tiny decoder and U(0.5, 1.5) for the others.  Draws
    are float64, cast to float32.
    """
    rng = np.random.default_rng(seed)
    out = OrderedDict()
    for name, shape, init in manifest(cfg):
        n = math.prod(shape)
        if init == "normal":
            v = rng.standard_normal(n) * 0.02
        elif init == "ln_gain":
            v = 1.0 + rng.standard_normal(n) * 0.02
        elif init == "alpha":
            if cfg["alpha_init"] == "one":
                v = np.ones(n)
            else:
                v = rng.uniform(0.5, 1.5, n)
        else:  # pragma: no cover
            raise ValueError(init)
        out[name] = v.astype(np.float32).reshape(shape)
    return out


def flatten_weights(cfg, weights) -> np.ndarray:
    """Concatenate every tensor, C-contiguous, in manifest order, as one float32 vector."""
    parts = [np.ascontiguousarray(weights[name], dtype=np.float32).ravel() for name, _, _ in manifest(cfg)]
    return np.concatenate(parts)


# ---------------------------------------------------------------------------
# codec frames
# ---------------------------------------------------------------------------


def zipf_probs(V: int, s: float = 1.1) -> np.ndarray:
    """Zipf(s) over ranks 1..V, truncated and renormalised; code id = rank - 1."""
    ranks = np.arange(1, V + 1, dtype=np.float64)
    p = ranks ** (-s)
    return p / p.sum()


def make_codes(cfg, batch: int, frames: int, seed: int, dist: str = "uniform") -> np.ndarray:
    """int32 codes [batch][frames][n_codebooks], independent per (stream, frame, codebook)."""
    rng = np.random.default_rng(seed)
    V, Q = cfg["codebook_size"], cfg["n_codebooks"]
    if dist == "uniform":
        c = rng.integers(0, V, size=(batch, frames, Q))
    elif dist == "zipf":
        c = rng.choice(V, size=(batch, frames, Q), p=zipf_probs(V))
    else:
        raise ValueError(dist)
    return c.astype(np.int32)


def workload_codes(i_or_name) -> np.ndarray:
    """Codes of a workload (a reference prefix, if any, first).  For the 64-stream batched workload the array holds
    each stream's warm-up frames followed by its timed 25-frame chunk, padded to
    the longest stream (stream b uses its first batched_warmup_frames(b) + 25 rows)."""
    w = workload(i_or_name)
    cfg = w["model"]
    if w["schedule"] == "warm_then_25":
        total = max(batched_warmup_frames(b) for b in range(w["batch"])) + w["frames"]
        return make_codes(cfg, w["batch"], total, w["code_seed"], w["codes"])
    return make_codes(cfg, w["batch"], w.get("prefix", 0) + w["frames"], w["code_seed"], w["codes"])
