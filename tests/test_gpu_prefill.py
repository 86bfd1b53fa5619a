"""GPU tests of the reference-prefix prefill (vocoder_prefill): decoding a
prefix into the state without audio gives, bit for bit, the state that
decoding it with vocoder_decode_chunk gives, also when the stack after the
transformer runs over the prefix's last tail_frames frames only; the audio
decoded after a prefill matches the oracle's decode of prefix + utterance."""
import numpy as np
import pytest
import torch

import synthetic as S
from tests.gpu_util import check_close, decoder, oracle_stream, run_schedule
from vocoder_rvq_codebook_amd import binding as vb

pytestmark = pytest.mark.gpu


def tail_frames(model):
    """The prefill tail, walked back by hand from conv_post's carried rows."""
    need = model["post_kernel"] - 1
    for si in reversed(range(len(model["rates"]))):
        r = model["rates"][si]
        look = max(sum((k - 1) * (d + 1) for d in model["dilations"]) for k in model["res_kernels"])
        need = -(-(need + look) // r) + 1
    need += model["conv_pre_kernel"] - 1
    for s in reversed(model["up_strides"]):
        need = -(-need // s) + 1
    return need


def test_tail_frames_of_the_known_shapes():
    assert tail_frames(S.QWEN3) == 9
    assert tail_frames(S.MINI) == 23
    assert tail_frames(S.TINY) == 5


def _warm(dec, codes, warm):
    B = len(warm)
    st = dec.new_state(B)
    for b, nw in enumerate(warm):
        if nw:
            _, s2 = run_schedule(dec, codes[b:b + 1, :nw], [nw], state=st[b:b + 1].clone())
            st[b:b + 1].copy_(s2)
    return st


@pytest.mark.parametrize("model", [S.TINY, S.MINI, dict(S.MINI, name="mini_f16", precision="f16"),
                                   dict(S.MINI, name="mini_split", precision="split")],
                         ids=["tiny", "mini", "mini_f16", "mini_split"])
def test_prefill_state_equals_decode_state(model):
    tail = tail_frames(model)
    B, warm, utt = 2, [0, 9], 6
    frames = [tail + 7, tail, 3]
    dec, W = decoder(model, 31, B, max(frames))
    assert vb.vocoder_prefill_tail_frames(dec.handle) == tail
    codes = S.make_codes(model, B, max(warm) + max(frames) + utt, 71)
    for T in frames:
        st0 = _warm(dec, codes, warm)
        chunk = torch.from_numpy(np.stack([codes[b, nw:nw + T] for b, nw in enumerate(warm)])).cuda()
        st_dec, st_pre = torch.empty_like(st0), torch.empty_like(st0)
        dec.decode(chunk, st0, st_dec)
        dec.prefill(chunk, st0, st_pre)
        torch.cuda.synchronize()
        assert dec.status() == vb.VOCODER_OK
        assert torch.equal(st_pre, st_dec), f"T={T}"
        # the utterance after the prefix, against the oracle's decode of both
        nxt = np.stack([codes[b, nw + T:nw + T + utt] for b, nw in enumerate(warm)])
        pcm, _ = run_schedule(dec, nxt, [utt], state=st_pre)
        for b, nw in enumerate(warm):
            sched = [n for n in (nw, T, utt) if n]
            # fp16 operands: the oracle rounds the same operands; fp32 and split: the plain decoder
            ref = oracle_stream(model, W, codes[b, :nw + T + utt], sched,
                                operands="f16" if model.get("precision") == "f16" else None)
            rel = 2e-3 if model.get("precision") == "f16" else 1e-4
            check_close(pcm[b].cpu().numpy(), ref[(nw + T) * model["hop"]:], f"{model['name']} T={T} stream {b}",
                        rel=rel)


@pytest.mark.parametrize("precision", ["f32", "f16"])
def test_prefill_state_equals_decode_state_int8(precision):
    """int8 weights: the prefilled state is bitwise the decoded one (the
    decodes against the oracle on dequantized weights are tested with the
    int8 format itself)."""
    model = dict(S.MINI, name=f"mini_q8_{precision}", weights="int8", precision=precision)
    tail = tail_frames(model)
    B, warm = 2, [0, 9]
    dec, _ = decoder(model, 31, B, tail + 7)
    codes = S.make_codes(model, B, max(warm) + tail + 7, 72)
    for T in (tail + 7, 3):
        st0 = _warm(dec, codes, warm)
        chunk = torch.from_numpy(np.stack([codes[b, nw:nw + T] for b, nw in enumerate(warm)])).cuda()
        st_dec, st_pre = torch.empty_like(st0), torch.empty_like(st0)
        dec.decode(chunk, st0, st_dec)
        dec.prefill(chunk, st0, st_pre)
        torch.cuda.synchronize()
        assert dec.status() == vb.VOCODER_OK
        assert torch.equal(st_pre, st_dec), f"T={T}"


def test_prefill_rejects_bad_arguments_and_reports_bad_codes():
    model = S.TINY
    dec, _ = decoder(model, 0, 2, 8)
    st_a, st_b = dec.new_state(2), dec.new_state(2)
    codes = torch.zeros((2, 8, model["n_codebooks"]), dtype=torch.int32, device="cuda")
    assert vb.vocoder_prefill(dec.handle, codes, 2, 9, st_a, st_b) == vb.VOCODER_EINVAL
    assert vb.vocoder_prefill(dec.handle, codes, 3, 8, st_a, st_b) == vb.VOCODER_EINVAL
    st3 = dec.new_state(3)
    assert vb.vocoder_prefill(dec.handle, codes, 2, 8, st3[0:2], st3[1:3]) == vb.VOCODER_EINVAL  # overlap
    assert vb.vocoder_prefill(dec.handle, None, 2, 8, st_a, st_b) == vb.VOCODER_EINVAL
    codes[0, 7, 0] = -1
    dec.prefill(codes, st_a, st_b)
    assert dec.status() == vb.VOCODER_ECODE


def test_prefill_full_size():
    """Qwen3-shaped decoder: a 40-frame prefix (tail 9) from a fresh state and
    from a state 25 frames in gives decode_chunk's state bit for bit."""
    print("\n[prefill] full size", flush=True)
    model = S.QWEN3
    dec, _ = decoder(model, 1, 1, 250)
    assert vb.vocoder_prefill_tail_frames(dec.handle) == 9
    codes = S.workload_codes("qwen3_b1_t250_whole")
    for start in (0, 25):
        st0 = dec.new_state(1)
        if start:
            _, st0 = run_schedule(dec, codes[:, :start], [start])
        chunk = torch.from_numpy(np.ascontiguousarray(codes[:, start:start + 40])).cuda()
        st_dec, st_pre = torch.empty_like(st0), torch.empty_like(st0)
        dec.decode(chunk, st0, st_dec)
        dec.prefill(chunk, st0, st_pre)
        torch.cuda.synchronize()
        assert dec.status() == vb.VOCODER_OK
        assert torch.equal(st_pre, st_dec), f"start {start}"
