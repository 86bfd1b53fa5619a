"""Thin ctypes binding over libvocoder.so (include/vocoder.h).

The functions below carry the C entry points' names and only marshal
arguments: every step of the decoder runs in the library's HIP kernels.
PyTorch supplies device memory and the current stream.  If the shared
library is missing the import of this module still works, but every call
raises: there is no CPU fallback.
"""
from __future__ import annotations

import ctypes
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libvocoder.so")

VOCODER_OK = 0
VOCODER_EINVAL = -1
VOCODER_ESTATE = -2
VOCODER_EHIP = -3
VOCODER_ECODE = -4
VOCODER_ESCRATCH = -5

MAX_UP, MAX_STAGES, MAX_RES, MAX_DIL = 4, 8, 4, 4


class VocoderConfig(ctypes.Structure):
    _fields_ = [
        ("n_codebooks", ctypes.c_int32),
        ("codebook_size", ctypes.c_int32),
        ("embed_dim", ctypes.c_int32),
        ("model_dim", ctypes.c_int32),
        ("n_layers", ctypes.c_int32),
        ("n_heads", ctypes.c_int32),
        ("window", ctypes.c_int32),
        ("ffn_dim", ctypes.c_int32),
        ("rope_theta", ctypes.c_float),
        ("ln_eps", ctypes.c_float),
        ("pre_kernel", ctypes.c_int32),
        ("n_up", ctypes.c_int32),
        ("up_strides", ctypes.c_int32 * MAX_UP),
        ("voc_ch0", ctypes.c_int32),
        ("conv_pre_kernel", ctypes.c_int32),
        ("n_stages", ctypes.c_int32),
        ("rates", ctypes.c_int32 * MAX_STAGES),
        ("n_res", ctypes.c_int32),
        ("res_kernels", ctypes.c_int32 * MAX_RES),
        ("n_dil", ctypes.c_int32),
        ("dilations", ctypes.c_int32 * MAX_DIL),
        ("post_kernel", ctypes.c_int32),
        ("max_batch", ctypes.c_int32),
        ("max_frames", ctypes.c_int32),
        ("precision", ctypes.c_int32),
        ("weight_format", ctypes.c_int32),
    ]


PRECISIONS = {"f32": 0, "f16": 1, "split": 2}
WEIGHT_FORMATS = {"float": 0, "int8": 1}


class VocoderKernelStat(ctypes.Structure):
    _fields_ = [
        ("name", ctypes.c_char * 48),
        ("launches", ctypes.c_int32),
        ("total_ms", ctypes.c_double),
        ("flops", ctypes.c_double),
        ("bytes", ctypes.c_double),
    ]


class VocoderError(RuntimeError):
    def __init__(self, code, what):
        super().__init__(f"{what}: {vocoder_strerror(code)} ({code})")
        self.code = code


_lib = None


def lib():
    """Load libvocoder.so once; raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m vocoder_rvq_codebook_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER(VocoderConfig)
        vp, i32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
        for name in ("vocoder_raw_weights_count", "vocoder_packed_weights_bytes", "vocoder_weights_bytes",
                     "vocoder_workspace_bytes", "vocoder_state_bytes"):
            getattr(L, name).argtypes = [P]
            getattr(L, name).restype = sz
        L.vocoder_create.argtypes = [P, vp, vp, vp, vp, ctypes.POINTER(vp)]
        L.vocoder_create.restype = i32
        L.vocoder_reset.argtypes = [vp, vp, i32, vp]
        L.vocoder_reset.restype = i32
        L.vocoder_decode_chunk.argtypes = [vp, vp, i32, i32, vp, vp, vp, vp]
        L.vocoder_decode_chunk.restype = i32
        L.vocoder_decode_chunk_graph.argtypes = [vp, vp, i32, i32, vp, vp, vp, vp]
        L.vocoder_decode_chunk_graph.restype = i32
        L.vocoder_decode_chunk_noalloc.argtypes = [vp, vp, i32, i32, vp, vp, vp, vp]
        L.vocoder_decode_chunk_noalloc.restype = i32
        L.vocoder_graph_cache_size.argtypes = [vp]
        L.vocoder_graph_cache_size.restype = i32
        L.vocoder_quantize_int8.argtypes = [vp, ctypes.c_longlong, i32, vp, vp, vp]
        L.vocoder_quantize_int8.restype = i32
        L.vocoder_prefill.argtypes = [vp, vp, i32, i32, vp, vp, vp]
        L.vocoder_prefill.restype = i32
        L.vocoder_prefill_tail_frames.argtypes = [vp]
        L.vocoder_prefill_tail_frames.restype = i32
        L.vocoder_hop.argtypes = [vp]
        L.vocoder_hop.restype = i32
        L.vocoder_left_context_frames.argtypes = [vp]
        L.vocoder_left_context_frames.restype = i32
        L.vocoder_get_status.argtypes = [vp, vp]
        L.vocoder_get_status.restype = i32
        L.vocoder_set_tap.argtypes = [vp, ctypes.c_char_p, vp, sz]
        L.vocoder_set_tap.restype = i32
        L.vocoder_profile_begin.argtypes = [vp]
        L.vocoder_profile_begin.restype = i32
        L.vocoder_profile_end.argtypes = [vp, vp, ctypes.POINTER(VocoderKernelStat), i32, ctypes.POINTER(i32)]
        L.vocoder_profile_end.restype = i32
        L.vocoder_peak_mfma_flops.argtypes = [i32, i32, i32]
        L.vocoder_peak_mfma_flops.restype = ctypes.c_double
        L.vocoder_peak_mfma.argtypes = [i32, vp, i32, i32, vp]
        L.vocoder_peak_mfma.restype = i32
        L.vocoder_stream_read.argtypes = [vp, ctypes.c_longlong, vp, i32, vp]
        L.vocoder_stream_read.restype = i32
        L.vocoder_stream_copy.argtypes = [vp, vp, ctypes.c_longlong, i32, vp]
        L.vocoder_stream_copy.restype = i32
        L.vocoder_grid_barrier.argtypes = [vp, vp, vp, i32, i32, vp]
        L.vocoder_grid_barrier.restype = i32
        L.vocoder_empty_launches.argtypes = [vp, i32, i32, vp]
        L.vocoder_empty_launches.restype = i32
        L.vocoder_destroy.argtypes = [vp]
        L.vocoder_destroy.restype = None
        L.vocoder_strerror.argtypes = [i32]
        L.vocoder_strerror.restype = ctypes.c_char_p
        _lib = L
    return _lib


def make_config(model: dict, max_batch: int, max_frames: int) -> VocoderConfig:
    """Fill the C config from a decoder-shape dict (keys as in include/vocoder.h)."""
    c = VocoderConfig()
    for f in ("n_codebooks", "codebook_size", "embed_dim", "model_dim", "n_layers", "n_heads", "window",
              "ffn_dim", "pre_kernel", "voc_ch0", "conv_pre_kernel", "post_kernel"):
        setattr(c, f, int(model[f]))
    c.rope_theta = float(model["rope_theta"])
    c.ln_eps = float(model["ln_eps"])
    for lst, cnt, arr in (("up_strides", "n_up", c.up_strides), ("rates", "n_stages", c.rates),
                          ("res_kernels", "n_res", c.res_kernels), ("dilations", "n_dil", c.dilations)):
        vals = list(model[lst])
        if len(vals) > len(arr):
            raise ValueError(f"{lst}: at most {len(arr)} entries")
        setattr(c, cnt, len(vals))
        for i, v in enumerate(vals):
            arr[i] = int(v)
    c.max_batch = int(max_batch)
    c.max_frames = int(max_frames)
    prec = model.get("precision", "f32")
    if prec not in PRECISIONS:
        raise ValueError(f"precision must be one of {sorted(PRECISIONS)}")
    c.precision = PRECISIONS[prec]
    wf = model.get("weights", "float")
    if wf not in WEIGHT_FORMATS:
        raise ValueError(f"weights must be one of {sorted(WEIGHT_FORMATS)}")
    c.weight_format = WEIGHT_FORMATS[wf]
    return c


def _ptr(t) -> int | None:
    if t is None:
        return None
    if isinstance(t, torch.Tensor):
        if not t.is_cuda:
            raise ValueError("device tensor required")
        return t.data_ptr()
    return int(t)


def _stream(stream) -> int | None:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


# --- the C entry points, same names -----------------------------------------


def vocoder_raw_weights_count(cfg: VocoderConfig) -> int:
    return lib().vocoder_raw_weights_count(ctypes.byref(cfg))


def vocoder_packed_weights_bytes(cfg: VocoderConfig) -> int:
    return lib().vocoder_packed_weights_bytes(ctypes.byref(cfg))


def vocoder_weights_bytes(cfg: VocoderConfig) -> int:
    return lib().vocoder_weights_bytes(ctypes.byref(cfg))


def vocoder_workspace_bytes(cfg: VocoderConfig) -> int:
    return lib().vocoder_workspace_bytes(ctypes.byref(cfg))


def vocoder_state_bytes(cfg: VocoderConfig) -> int:
    return lib().vocoder_state_bytes(ctypes.byref(cfg))


def vocoder_create(cfg, raw_weights, packed_weights, workspace, stream=None):
    h = ctypes.c_void_p()
    rc = lib().vocoder_create(ctypes.byref(cfg), _ptr(raw_weights), _ptr(packed_weights), _ptr(workspace),
                              _stream(stream), ctypes.byref(h))
    if rc != VOCODER_OK:
        raise VocoderError(rc, "vocoder_create")
    return h.value


def vocoder_reset(handle, state, batch, stream=None) -> int:
    return lib().vocoder_reset(handle, _ptr(state), int(batch), _stream(stream))


def vocoder_decode_chunk(handle, codes, batch, n_frames, state_in, state_out, pcm, stream=None) -> int:
    return lib().vocoder_decode_chunk(handle, _ptr(codes), int(batch), int(n_frames), _ptr(state_in),
                                      _ptr(state_out), _ptr(pcm), _stream(stream))


def vocoder_decode_chunk_graph(handle, codes, batch, n_frames, state_in, state_out, pcm, stream=None) -> int:
    return lib().vocoder_decode_chunk_graph(handle, _ptr(codes), int(batch), int(n_frames), _ptr(state_in),
                                            _ptr(state_out), _ptr(pcm), _stream(stream))


def vocoder_decode_chunk_noalloc(handle, codes, batch, n_frames, state_in, state_out, pcm, stream=None) -> int:
    return lib().vocoder_decode_chunk_noalloc(handle, _ptr(codes), int(batch), int(n_frames), _ptr(state_in),
                                              _ptr(state_out), _ptr(pcm), _stream(stream))


def vocoder_graph_cache_size(handle) -> int:
    return lib().vocoder_graph_cache_size(handle)


def vocoder_quantize_int8(src, rows, K, q, scale, stream=None) -> int:
    return lib().vocoder_quantize_int8(_ptr(src), int(rows), int(K), _ptr(q), _ptr(scale), _stream(stream))


def vocoder_prefill(handle, codes, batch, n_frames, state_in, state_out, stream=None) -> int:
    return lib().vocoder_prefill(handle, _ptr(codes), int(batch), int(n_frames), _ptr(state_in), _ptr(state_out),
                                 _stream(stream))


def vocoder_prefill_tail_frames(handle) -> int:
    return lib().vocoder_prefill_tail_frames(handle)


def vocoder_hop(handle) -> int:
    return lib().vocoder_hop(handle)


def vocoder_left_context_frames(handle) -> int:
    return lib().vocoder_left_context_frames(handle)


def vocoder_get_status(handle, stream=None) -> int:
    return lib().vocoder_get_status(handle, _stream(stream))


def vocoder_set_tap(handle, name: str, dst, dst_floats: int = 0) -> int:
    return lib().vocoder_set_tap(handle, name.encode(), _ptr(dst), int(dst_floats))


def vocoder_profile_begin(handle) -> int:
    return lib().vocoder_profile_begin(handle)


def vocoder_profile_end(handle, stream=None, max_entries: int = 64):
    """Stop recording and return {kernel: dict(launches, total_ms, flops, bytes)}."""
    arr = (VocoderKernelStat * max_entries)()
    n = ctypes.c_int(0)
    rc = lib().vocoder_profile_end(handle, _stream(stream), arr, max_entries, ctypes.byref(n))
    if rc != VOCODER_OK:
        raise VocoderError(rc, "vocoder_profile_end")
    return {arr[i].name.decode(): dict(launches=arr[i].launches, total_ms=arr[i].total_ms, flops=arr[i].flops,
                                       bytes=arr[i].bytes) for i in range(min(n.value, max_entries))}


def vocoder_peak_mfma_flops(dtype: int, blocks: int, iters: int) -> float:
    return lib().vocoder_peak_mfma_flops(int(dtype), int(blocks), int(iters))


def vocoder_peak_mfma(dtype: int, out, blocks: int, iters: int, stream=None) -> int:
    return lib().vocoder_peak_mfma(int(dtype), _ptr(out), int(blocks), int(iters), _stream(stream))


def vocoder_stream_read(src, n: int, out, blocks: int, stream=None) -> int:
    return lib().vocoder_stream_read(_ptr(src), int(n), _ptr(out), int(blocks), _stream(stream))


def vocoder_stream_copy(src, dst, n: int, blocks: int, stream=None) -> int:
    return lib().vocoder_stream_copy(_ptr(src), _ptr(dst), int(n), int(blocks), _stream(stream))


def vocoder_grid_barrier(flags, slots, err, blocks: int, rounds: int, stream=None) -> int:
    return lib().vocoder_grid_barrier(_ptr(flags), _ptr(slots), _ptr(err), int(blocks), int(rounds), _stream(stream))


def vocoder_empty_launches(scratch, blocks: int, n: int, stream=None) -> int:
    return lib().vocoder_empty_launches(_ptr(scratch), int(blocks), int(n), _stream(stream))


def vocoder_destroy(handle) -> None:
    if handle:
        lib().vocoder_destroy(handle)


def vocoder_strerror(code: int) -> str:
    try:
        return lib().vocoder_strerror(int(code)).decode()
    except RuntimeError:
        return f"status {code}"


# --- convenience owner of the device buffers ---------------------------------


def _device(device) -> torch.device:
    """torch.device with an explicit index for a GPU ("cuda" -> the current one)."""
    device = torch.device(device)
    if device.type == "cuda" and device.index is None:
        device = torch.device("cuda", torch.cuda.current_device())
    return device


def check_decode_args(codes, state_in, state_out, pcm, *, n_codebooks: int, state_bytes: int, hop: int,
                      device, max_batch: int, max_frames: int) -> None:
    """Raise ValueError unless the tensors of one decode (or prefill, pcm=None)
    call are what the library will read and write: the library sees only raw
    pointers, so a buffer of the wrong type, layout, device or size would be
    read or written out of bounds on the device.

    codes: int32, contiguous, [batch][frames][n_codebooks], 1 <= batch <=
    max_batch, 1 <= frames <= max_frames.  States: uint8, contiguous,
    [>= batch][state_bytes], 256-byte aligned, and either the same buffer
    (in place) or disjoint.  pcm: float32, contiguous, >= batch * frames * hop
    elements."""
    device = _device(device)

    def on_device(t, what):
        if not isinstance(t, torch.Tensor):
            raise ValueError(f"{what} must be a torch tensor")
        if t.device != device:
            raise ValueError(f"{what} is on {t.device}, the decoder on {device}")
        if not t.is_contiguous():
            raise ValueError(f"{what} must be contiguous")

    on_device(codes, "codes")
    if codes.dtype != torch.int32 or codes.dim() != 3:
        raise ValueError("codes must be an int32 [batch][frames][codebooks] tensor")
    B, T, Q = codes.shape
    if Q != n_codebooks:
        raise ValueError(f"expected {n_codebooks} codebooks, got {Q}")
    if not (1 <= B <= max_batch) or not (1 <= T <= max_frames):
        raise ValueError(f"batch {B} / frames {T} outside [1, {max_batch}] / [1, {max_frames}]")
    for t, what in ((state_in, "state_in"), (state_out, "state_out")):
        on_device(t, what)
        if t.dtype != torch.uint8 or t.dim() != 2 or t.shape[1] != state_bytes:
            raise ValueError(f"{what} must be a uint8 [batch][{state_bytes}] tensor, got {t.dtype} "
                             f"{tuple(t.shape)}")
        if t.shape[0] < B:
            raise ValueError(f"{what} holds {t.shape[0]} states, the call decodes {B}")
        if t.data_ptr() % 256:
            raise ValueError(f"{what} must be 256-byte aligned")
    a, b, n = state_in.data_ptr(), state_out.data_ptr(), B * state_bytes
    if a != b and a < b + n and b < a + n:
        raise ValueError("state_out overlaps state_in without being the same buffer")
    if pcm is not None:
        on_device(pcm, "pcm")
        if pcm.dtype != torch.float32:
            raise ValueError("pcm must be float32")
        if pcm.numel() < B * T * hop:
            raise ValueError(f"pcm holds {pcm.numel()} samples, the call writes {B * T * hop}")


class Decoder:
    """A decoder instance with its packed weights and workspace held as torch
    device tensors.  States are [batch][state_bytes] uint8 tensors; a decode
    reads one and writes another, or updates one in place."""

    def __init__(self, model: dict, raw_weights, max_batch: int, max_frames: int, device="cuda"):
        self.model = model
        self.device = _device(device)
        self.cfg = make_config(model, max_batch, max_frames)
        n = vocoder_raw_weights_count(self.cfg)
        if n == 0:
            raise ValueError("unsupported decoder config")
        raw = torch.as_tensor(raw_weights, dtype=torch.float32).reshape(-1)
        if raw.numel() != n:
            raise ValueError(f"raw weights: expected {n} floats, got {raw.numel()}")
        raw = raw.to(self.device)
        self.packed = torch.empty(vocoder_packed_weights_bytes(self.cfg), dtype=torch.uint8, device=self.device)
        self.workspace = torch.empty(vocoder_workspace_bytes(self.cfg), dtype=torch.uint8, device=self.device)
        self.state_bytes = vocoder_state_bytes(self.cfg)
        with torch.cuda.device(self.device):
            self.handle = vocoder_create(self.cfg, raw, self.packed, self.workspace)
        del raw
        self.hop = vocoder_hop(self.handle)
        self.left_context_frames = vocoder_left_context_frames(self.handle)
        self._taps = {}

    def __del__(self):
        h = getattr(self, "handle", None)
        if h:
            vocoder_destroy(h)
            self.handle = None

    def new_state(self, batch: int) -> torch.Tensor:
        st = torch.empty((batch, self.state_bytes), dtype=torch.uint8, device=self.device)
        self.reset(st)
        return st

    def reset(self, state: torch.Tensor) -> None:
        if (not isinstance(state, torch.Tensor) or state.device != self.device or not state.is_contiguous()
                or state.dtype != torch.uint8 or state.dim() != 2 or state.shape[1] != self.state_bytes
                or state.shape[0] < 1 or state.data_ptr() % 256):
            raise ValueError(f"state must be a contiguous, 256-byte aligned uint8 [batch][{self.state_bytes}] "
                             f"tensor on {self.device}")
        rc = vocoder_reset(self.handle, state, state.shape[0])
        if rc != VOCODER_OK:
            raise VocoderError(rc, "vocoder_reset")

    def _check(self, codes, state_in, state_out, pcm):
        check_decode_args(codes, state_in, state_out, pcm, n_codebooks=self.cfg.n_codebooks,
                          state_bytes=self.state_bytes, hop=self.hop, device=self.device,
                          max_batch=self.cfg.max_batch, max_frames=self.cfg.max_frames)

    def decode(self, codes: torch.Tensor, state_in: torch.Tensor, state_out: torch.Tensor,
               pcm: torch.Tensor | None = None, graph: bool = False, noalloc: bool = False) -> torch.Tensor:
        """One chunk for codes.shape[0] streams.  state_out may be state_in
        itself (in place) or a disjoint buffer.  graph=True replays a HIP graph
        kept per (buffers, batch, frames): reuse the same code, state and PCM
        tensors across calls, and keep them alive while the decoder lives.
        noalloc=True runs vocoder_decode_chunk_noalloc (the call's buffers in
        the library's static scratch; pass pcm to allocate nothing here either)."""
        if pcm is None:
            self._check(codes, state_in, state_out, None)
            pcm = torch.empty((codes.shape[0], codes.shape[1] * self.hop), dtype=torch.float32, device=self.device)
        self._check(codes, state_in, state_out, pcm)
        B, T = codes.shape[0], codes.shape[1]
        if graph and noalloc:
            raise ValueError("graph and noalloc are separate entry points")
        fn = vocoder_decode_chunk_graph if graph else vocoder_decode_chunk_noalloc if noalloc else vocoder_decode_chunk
        rc = fn(self.handle, codes, B, T, state_in, state_out, pcm)
        if rc != VOCODER_OK:
            raise VocoderError(rc, fn.__name__)
        return pcm

    def prefill(self, codes: torch.Tensor, state_in: torch.Tensor, state_out: torch.Tensor) -> None:
        """Decode a reference prefix into state_out without producing audio."""
        self._check(codes, state_in, state_out, None)
        B, T = codes.shape[0], codes.shape[1]
        rc = vocoder_prefill(self.handle, codes, B, T, state_in, state_out)
        if rc != VOCODER_OK:
            raise VocoderError(rc, "vocoder_prefill")

    def status(self) -> int:
        return vocoder_get_status(self.handle)

    def set_tap(self, name: str, dst: torch.Tensor | None) -> None:
        if dst is None:
            vocoder_set_tap(self.handle, name, None, 0)
            self._taps.pop(name, None)
            return
        if dst.dtype != torch.float32 or not dst.is_cuda or not dst.is_contiguous():
            raise ValueError("tap destination must be a contiguous float32 device tensor")
        self._taps[name] = dst
        rc = vocoder_set_tap(self.handle, name, dst, dst.numel())
        if rc != VOCODER_OK:
            raise VocoderError(rc, "vocoder_set_tap")
