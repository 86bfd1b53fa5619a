"""The few-row GEMM path of short chunks (fp32 arithmetic, float and int8
weights): chunks of up to 4 frames send their at-most-16-row launches that
feed no LayerNorm through conv_gemm_rows_kernel instead of a split-K GEMM and
its fold.  Both paths reduce every output in the same order, so a stream
decoded in short chunks must equal its whole decode bit for bit; the profile
must show the few-row launches, so that the path cannot silently go unused."""
import pytest
import torch

import synthetic as S
from tests.gpu_util import decoder, run_schedule
from vocoder_rvq_codebook_amd import binding as vb

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("weights", ["float", "int8"])
def test_short_chunks_take_the_few_row_kernel_bitwise(weights):
    model = S.MINI if weights == "float" else dict(S.MINI, name="mini_q8_f32", weights="int8", precision="f32")
    print(f"\n[rows] mini, {weights} weights: 1+1+2+4+8+25 frames against 41 whole", flush=True)
    dec, _ = decoder(model, 9, 2, 41)
    codes = S.make_codes(model, 2, 41, 33)
    whole, st_w = run_schedule(dec, codes, [41])
    vb.vocoder_profile_begin(dec.handle)
    parts, st_p = run_schedule(dec, codes, [1, 1, 2, 4, 8, 25])
    prof = vb.vocoder_profile_end(dec.handle)
    assert dec.status() == vb.VOCODER_OK
    name = "conv_gemm_rows16_q8" if weights == "int8" else "conv_gemm_rows16"
    assert prof.get(name, {}).get("launches", 0) > 0, sorted(prof)
    assert torch.equal(whole, parts) and torch.equal(st_w, st_p)
