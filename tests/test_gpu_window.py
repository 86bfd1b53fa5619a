"""The fp16 GEMMs that stage each 32-channel slab's input rows once for all of
its taps (the slab windows of conv_gemm_f16_dma_kernel): their tiles cover one
stream each, and the rows before a stream's first frame come from its state.

A window reads the same fp16 operands as the per-tap kernel and feeds the same
MFMA sequence, so the bits must not change.  The narrow test decoder (stage-2
and stage-3 launches of 64 and 32 channels) decodes three streams whole (1968
stage-3 rows per stream, the last tile of each stream partly idle, zero
history), as 9 + 32 frames (1536 rows: whole tiles, the first of each stream
reading the state the 9-frame chunk wrote) and as 10 + 31 frames (1488 rows:
state rows and a partly idle last tile).  Each must equal a schedule of short
chunks that never takes the windows, bit for bit, and the last stream must
match the oracle's fp16-operand decode.  The profile must
show the window launches, so the path cannot silently go unused."""
import pytest
import torch

import synthetic as S
from tests.gpu_util import check_close, decoder, oracle_stream, run_schedule
from tests.test_gpu_f16 import F16_VS_F16_ORACLE, half
from vocoder_rvq_codebook_amd import binding as vb

pytestmark = pytest.mark.gpu


def _profiled(dec, codes, schedule):
    vb.vocoder_profile_begin(dec.handle)
    pcm, st = run_schedule(dec, codes, schedule)
    prof = vb.vocoder_profile_end(dec.handle)
    assert dec.status() == vb.VOCODER_OK
    return pcm, st, sum(v.get("launches", 0) for k, v in prof.items() if k.endswith("_win"))


def test_f16_slab_windows_bitwise():
    model = half(S.MINI)
    B, T = 3, 41
    print(f"\n[window] mini fp16, {B} streams: 41 whole and 9 + 32 against short chunks", flush=True)
    dec, W = decoder(model, 9, B, T)
    codes = S.make_codes(model, B, T, 36)
    short, st_s, n_short = _profiled(dec, codes, [1, 1, 2, 4, 8, 8, 8, 8, 1])
    whole, st_w, n_whole = _profiled(dec, codes, [T])
    split, st_p, n_split = _profiled(dec, codes, [9, 32])
    cross, st_c, n_cross = _profiled(dec, codes, [10, 31])
    print(f"  window launches: short chunks {n_short}, whole {n_whole}, 9 + 32 {n_split}, 10 + 31 {n_cross}",
          flush=True)
    assert n_short == 0 and n_whole > 0 and n_split > 0 and n_cross > 0
    assert torch.equal(whole, short) and torch.equal(st_w, st_s)
    assert torch.equal(split, short) and torch.equal(st_p, st_s)
    assert torch.equal(cross, short) and torch.equal(st_c, st_s)
    ref = oracle_stream(model, W, codes[B - 1], [9, 32], operands="f16")
    check_close(split[B - 1].cpu().numpy(), ref, "windowed fp16 stream vs fp16-operand oracle", rel=F16_VS_F16_ORACLE)
