"""vocoder_decode_chunk_noalloc: the decode entry point for callers that cannot
allocate, whose per-call buffers live in the library's static device scratch.
Through the C ABI it must give what vocoder_decode_chunk gives on the same
inputs, bit for bit (the same kernels in the same order), on consecutive calls
whose second is smaller than the first, in place or not; a chunk too large for
the scratch is refused before any launch."""
import numpy as np
import pytest
import torch

import synthetic as S
from tests.gpu_util import decoder
from vocoder_rvq_codebook_amd import binding as vb

pytestmark = pytest.mark.gpu


def _call(fn, dec, codes, st_in, st_out, pcm):
    B, T = codes.shape[0], codes.shape[1]
    return fn(dec.handle, codes, B, T, st_in, st_out, pcm)


def _warm_states(dec, B, frames, seed):
    st = dec.new_state(B)
    codes = S.make_codes(dec.model, B, frames, seed) if frames else None
    for t0 in range(0, frames, 25):
        c = torch.from_numpy(np.ascontiguousarray(codes[:, t0:t0 + 25])).cuda()
        dec.decode(c, st, st)
    torch.cuda.synchronize()
    return st


@pytest.mark.parametrize("name,calls", [
    ("qwen3", [(2, 4, 30, False), (1, 1, 7, True)]),
    ("mini", [(3, 13, 11, False), (1, 2, 0, True)]),
    ("tiny", [(2, 9, 5, True), (1, 3, 20, False)]),
])
def test_noalloc_equals_decode_chunk(name, calls):
    model = {"qwen3": S.QWEN3, "mini": S.MINI, "tiny": S.TINY}[name]
    dec, _ = decoder(model, 1, 3, 25)
    for i, (B, T, warm, in_place) in enumerate(calls):
        print(f"\n[noalloc] {name} call {i}: batch {B}, frames {T}, warm {warm}, in place {in_place}", flush=True)
        st0 = _warm_states(dec, B, warm, 100 + i)
        codes = torch.from_numpy(S.make_codes(model, B, T, 200 + i)).cuda()
        ref_pcm = torch.full((B, T * dec.hop), float("nan"), device="cuda")
        ref_st = torch.zeros_like(st0)
        assert _call(vb.vocoder_decode_chunk, dec, codes, st0, ref_st, ref_pcm) == vb.VOCODER_OK
        pcm = torch.full((B, T * dec.hop), float("nan"), device="cuda")
        if in_place:
            st = st0.clone()
            rc = _call(vb.vocoder_decode_chunk_noalloc, dec, codes, st, st, pcm)
        else:
            st = torch.zeros_like(st0)
            rc = _call(vb.vocoder_decode_chunk_noalloc, dec, codes, st0, st, pcm)
        assert rc == vb.VOCODER_OK
        torch.cuda.synchronize()
        assert dec.status() == vb.VOCODER_OK
        assert torch.isfinite(ref_pcm).all()
        assert torch.equal(pcm, ref_pcm)
        assert torch.equal(st, ref_st)


def test_noalloc_refuses_chunks_beyond_its_scratch():
    dec, _ = decoder(S.QWEN3, 1, 3, 25)
    B, T = 3, 25  # about 1.9 GB of buffers at this shape: far beyond the scratch
    codes = torch.zeros((B, T, 16), dtype=torch.int32, device="cuda")
    st_in = dec.new_state(B)
    st_out = torch.full_like(st_in, 7)
    pcm = torch.full((B, T * dec.hop), 3.0, device="cuda")
    assert _call(vb.vocoder_decode_chunk_noalloc, dec, codes, st_in, st_out, pcm) == vb.VOCODER_ESCRATCH
    torch.cuda.synchronize()
    # nothing ran: the outputs are untouched
    assert torch.all(st_out == 7) and torch.all(pcm == 3.0)
    assert dec.status() == vb.VOCODER_OK
    # the largest one-stream chunk the header promises still fits
    codes = torch.zeros((1, 10, 16), dtype=torch.int32, device="cuda")
    pcm = torch.empty((1, 10 * dec.hop), device="cuda")
    assert _call(vb.vocoder_decode_chunk_noalloc, dec, codes, st_in[:1], st_out[:1], pcm) == vb.VOCODER_OK
    torch.cuda.synchronize()
    assert dec.status() == vb.VOCODER_OK
