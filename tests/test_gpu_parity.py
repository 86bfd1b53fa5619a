"""GPU parity at small shapes: the HIP path through the C ABI against the
float64 oracle, stage by stage, on the tiny decoder and on a narrow decoder
with the full structure; bitwise chunking and batch invariance; device-side
error reporting.  Shapes span several tiles and ragged tails."""
import numpy as np
import pytest
import torch

import synthetic as S
from oracle import decoder as O
from tests.gpu_util import PCM_MAX_ABS, REL_L2, check_close, decoder, oracle_stream, run_schedule
from vocoder_rvq_codebook_amd import binding as vb

pytestmark = pytest.mark.gpu


def _stage_names(model):
    names = ["embed", "pre_conv"] + [f"layer{l}" for l in range(model["n_layers"])] + ["final_ln"]
    names += [f"up{i}" for i in range(len(model["up_strides"]))] + ["conv_pre"]
    for s in range(len(model["rates"])):
        names += [f"stage{s}.up", f"stage{s}"]
    return names + ["pre_tanh"]


def _tap_rows(model, name, T):
    up = int(np.prod(model["up_strides"]))
    if name in ("embed",):
        return T, model["embed_dim"]
    if name.startswith("layer") or name in ("pre_conv", "final_ln"):
        return T, model["model_dim"]
    if name.startswith("up"):
        i = int(name[2:])
        return T * int(np.prod(model["up_strides"][: i + 1])), model["model_dim"]
    if name == "conv_pre":
        return T * up, model["voc_ch0"]
    if name == "pre_tanh":
        return T * model["hop"], 1
    s = int(name[5:].split(".")[0])
    return T * up * int(np.prod(model["rates"][: s + 1])), model["stage_channels"][s + 1]


def test_tiny_workload_stage_by_stage():
    w = S.workload("tiny_b1_t32")
    model = w["model"]
    dec, W = decoder(model, w["weight_seed"], 1, 32)
    codes = S.workload_codes("tiny_b1_t32")
    T = codes.shape[1]
    taps = {}
    for name in _stage_names(model):
        rows, ch = _tap_rows(model, name, T)
        taps[name] = torch.full((rows * ch,), float("nan"), device="cuda")
        dec.set_tap(name, taps[name])
    pcm, _ = run_schedule(dec, codes, [T])
    assert dec.status() == vb.VOCODER_OK
    ref_taps = {}
    ref = oracle_stream(model, W, codes[0], taps=ref_taps)
    # the RVQ sum is exact: bitwise equal to the oracle's float32 ascending-codebook sum
    e32 = O.rvq_embed_sum(W["codebooks"], codes[0])
    np.testing.assert_array_equal(taps["embed"].cpu().numpy().reshape(e32.shape), e32)
    last = len(model["rates"]) - 1
    for name in _stage_names(model)[1:]:
        got = taps[name].cpu().numpy()
        r = ref_taps[name]
        if name == f"stage{last}":  # tapped after the final Snake
            r = O.snake(r, W["act_post.alpha"].astype(np.float64))
        check_close(got, r.reshape(-1), name)
    check_close(pcm.cpu().numpy()[0], ref, "pcm", max_abs=PCM_MAX_ABS)
    for name in taps:
        dec.set_tap(name, None)


@pytest.mark.parametrize("T", [1, 5, 13])
def test_mini_streams_at_different_positions(T):
    """Three streams warmed to positions 0, 7 and 20 (window 6), then one chunk of T."""
    model = S.MINI
    dec, W = decoder(model, 5, 3, 20)
    warm = [0, 7, 20]
    codes = S.make_codes(model, 3, max(warm) + T, 77)
    states = dec.new_state(3)
    for b, nw in enumerate(warm):
        if nw:
            st = states[b:b + 1]
            c = codes[b:b + 1, :nw]
            _, st2 = run_schedule(dec, c, [nw], state=st.clone())
            states[b:b + 1].copy_(st2)
    chunk = np.stack([codes[b, nw:nw + T] for b, nw in enumerate(warm)])
    taps = {}
    for name in _stage_names(model):
        rows, ch = _tap_rows(model, name, T)
        taps[name] = torch.full((3 * rows * ch,), float("nan"), device="cuda")
        dec.set_tap(name, taps[name])
    pcm, _ = run_schedule(dec, chunk, [T], state=states)
    assert dec.status() == vb.VOCODER_OK
    last = len(model["rates"]) - 1
    for b, nw in enumerate(warm):
        ref_taps = {}
        sched = [nw, T] if nw else [T]
        ref = oracle_stream(model, W, codes[b, : nw + T], sched, taps=ref_taps)
        for name in _stage_names(model):
            rows, ch = _tap_rows(model, name, T)
            got = taps[name].view(3, rows * ch)[b].cpu().numpy()
            r = ref_taps[name]
            if name == f"stage{last}":
                r = O.snake(r, W["act_post.alpha"].astype(np.float64))
            if name == "embed":
                np.testing.assert_array_equal(got, O.rvq_embed_sum(W["codebooks"], chunk[b]).reshape(-1))
            else:
                check_close(got, r.reshape(-1), f"stream {b} {name}")
        check_close(pcm[b].cpu().numpy(), ref[nw * model["hop"]:], f"stream {b} pcm", max_abs=PCM_MAX_ABS)
    for name in taps:
        dec.set_tap(name, None)


@pytest.mark.parametrize("model_name,schedule", [
    ("mini", [1] * 6 + [5, 13, 1, 14]),
    ("mini", [20, 20]),
    ("tiny", [1, 25, 6]),
    ("tiny", [8, 8, 8, 8]),
])
def test_streamed_equals_whole_bitwise(model_name, schedule):
    model = S.MINI if model_name == "mini" else S.TINY
    T = sum(schedule)
    dec, _ = decoder(model, 9, 2, 40)
    codes = S.make_codes(model, 2, T, 31)
    whole, st_w = run_schedule(dec, codes, [T])
    parts, st_p = run_schedule(dec, codes, schedule)
    assert torch.equal(whole, parts)
    # the carried states agree too (same rows, same position)
    assert torch.equal(st_w, st_p)


def test_batch_independence_bitwise():
    model = S.MINI
    dec, _ = decoder(model, 9, 4, 16)
    codes = S.make_codes(model, 4, 16, 41)
    both, _ = run_schedule(dec, codes, [16])
    for b in range(4):
        alone, _ = run_schedule(dec, codes[b:b + 1], [16])
        assert torch.equal(alone[0], both[b])


def test_out_of_range_code_is_reported():
    model = S.MINI
    dec, _ = decoder(model, 9, 2, 8)
    codes = S.make_codes(model, 2, 8, 5)
    run_schedule(dec, codes, [8])
    assert dec.status() == vb.VOCODER_OK
    bad = codes.copy()
    bad[1, 3, 7] = model["codebook_size"]
    pcm, _ = run_schedule(dec, bad, [8])
    assert dec.status() == vb.VOCODER_ECODE
    assert dec.status() == vb.VOCODER_OK  # reading clears it
    bad[1, 3, 7] = -5
    run_schedule(dec, bad, [8])
    assert dec.status() == vb.VOCODER_ECODE
    # the stream without a bad code is unaffected
    good, _ = run_schedule(dec, codes[:1], [8])
    assert torch.equal(good[0], pcm[0])


def test_foreign_state_is_reported_and_decoded_fresh():
    model = S.MINI
    dec, _ = decoder(model, 9, 1, 8)
    codes = S.make_codes(model, 1, 8, 6)
    fresh, _ = run_schedule(dec, codes, [8])
    st = dec.new_state(1)
    st[0, :4] = 0  # break the magic word
    got, _ = run_schedule(dec, codes, [8], state=st)
    assert dec.status() == vb.VOCODER_ESTATE
    assert torch.equal(got, fresh)
    # a state of another decoder shape is foreign too
    other, _ = decoder(S.TINY, 9, 1, 8)
    st_other = other.new_state(1)
    pad = torch.zeros((1, dec.state_bytes), dtype=torch.uint8, device="cuda")
    n = min(dec.state_bytes, other.state_bytes)
    pad[:, :n] = st_other[:, :n]
    got, _ = run_schedule(dec, codes, [8], state=pad)
    assert dec.status() == vb.VOCODER_ESTATE
    assert torch.equal(got, fresh)


def test_reset_after_abort_and_resume_from_saved_state():
    model = S.MINI
    dec, W = decoder(model, 9, 1, 16)
    codes = S.make_codes(model, 1, 30, 8)
    full, _ = run_schedule(dec, codes, [10, 10, 10])
    # decode 10 frames, save the state to the host, decode something else, abort
    _, st = run_schedule(dec, codes[:, :10], [10])
    saved = st.cpu()
    other = S.make_codes(model, 1, 7, 99)
    _, st2 = run_schedule(dec, other, [7], state=st)
    dec.reset(st2)  # abort: a reset state decodes like a fresh one
    fresh, _ = run_schedule(dec, codes, [10], state=st2)
    assert torch.equal(fresh[0], full[0, : 10 * model["hop"]])
    # a new decoder instance resumes from the saved state exactly
    dec2 = vb.Decoder(model, torch.from_numpy(S.flatten_weights(model, W)), 1, 16)
    resumed, _ = run_schedule(dec2, codes[:, 10:], [10, 10], state=saved.cuda())
    assert torch.equal(resumed[0], full[0, 10 * model["hop"]:])


def test_host_side_argument_errors():
    model = S.MINI
    dec, _ = decoder(model, 9, 2, 8)
    codes = torch.zeros((3, 4, 16), dtype=torch.int32, device="cuda")
    st = dec.new_state(3)
    st2 = dec.new_state(3)
    pcm = torch.empty((3, 4 * dec.hop), device="cuda")
    h = dec.handle
    assert vb.vocoder_decode_chunk(h, codes, 3, 4, st, st2, pcm) == vb.VOCODER_EINVAL  # batch > max
    assert vb.vocoder_decode_chunk(h, codes, 1, 9, st, st2, pcm) == vb.VOCODER_EINVAL  # frames > max
    assert vb.vocoder_decode_chunk(h, codes, 1, 0, st, st2, pcm) == vb.VOCODER_EINVAL
    assert vb.vocoder_decode_chunk(h, codes, 2, 4, st[0:2], st[1:3], pcm) == vb.VOCODER_EINVAL  # overlap
    assert vb.vocoder_prefill(h, codes, 2, 4, st[0:2], st[1:3]) == vb.VOCODER_EINVAL
    assert vb.vocoder_decode_chunk(h, codes, 2, 4, st[0:2], st2[0:2], pcm) == vb.VOCODER_OK
    assert vb.vocoder_decode_chunk(h, codes, 2, 4, st, st, pcm) == vb.VOCODER_OK  # in place
    assert dec.status() == vb.VOCODER_OK


@pytest.mark.parametrize("model_name,precision,graph", [
    ("mini", "f32", False),
    ("mini", "f32", True),
    ("mini", "f16", False),
    ("mini", "split", False),
    ("tiny", "f32", False),
])
def test_in_place_decode_equals_ping_pong(model_name, precision, graph):
    """state_out == state_in: chunks of 1, 25, 25 frames on two streams give
    the same PCM and the same final state, bit for bit, as decoding into a
    second buffer (the decoder adapter keeping one state across calls)."""
    base = S.MINI if model_name == "mini" else S.TINY
    model = dict(base, precision=precision, name=f"{base['name']}_{precision}")
    dec, _ = decoder(model, 9, 2, 25)
    sched = [1, 25, 25]
    codes = S.make_codes(model, 2, sum(sched), 53)
    ref, st_ref = run_schedule(dec, codes, sched)
    st = dec.new_state(2)
    out, t0 = [], 0
    for n in sched:
        c = torch.from_numpy(np.ascontiguousarray(codes[:, t0:t0 + n])).cuda()
        pcm = torch.empty((2, n * dec.hop), device="cuda")
        out.append(dec.decode(c, st, st, pcm, graph=graph).clone())
        t0 += n
    torch.cuda.synchronize()
    assert dec.status() == vb.VOCODER_OK
    assert torch.equal(torch.cat(out, dim=1), ref)
    assert torch.equal(st, st_ref)
    # a prefill in place leaves the same state as one into a second buffer
    st2, st3 = dec.new_state(2), dec.new_state(2)
    c = torch.from_numpy(np.ascontiguousarray(codes[:, :25])).cuda()
    dec.prefill(c, st2, st2)
    dec.prefill(c, st3.clone(), st3)
    torch.cuda.synchronize()
    assert torch.equal(st2, st3)
