"""The ordering-point microbenchmarks: a grid-wide barrier crossed inside one
cooperative kernel, against a dependent launch of an empty kernel.  The
barrier must order every block's writes before every other block's reads
(each round checks data another block wrote before the barrier), and every
wait in it is bounded, so a broken barrier reports an error instead of
hanging.  These price the ordering points of a small-chunk decode ("blixt/phonon",
Speed: the note on the cost of an empty dependent dispatch)."""
import pytest
import torch

from vocoder_rvq_codebook_amd import binding as vb

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("blocks", [2, 64, 256, 512])
def test_grid_barrier_orders_writes_before_reads(blocks):
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    print(f"\n[ordering] grid barrier, {blocks} blocks ({cus} CUs), 40 rounds", flush=True)
    flags = torch.zeros(blocks + 1, dtype=torch.int32, device="cuda")
    slots = torch.full((blocks * 64,), -1.0, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    assert vb.vocoder_grid_barrier(flags, slots, err, blocks, 40) == vb.VOCODER_OK
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    # 80 barriers: every block published round 80, and block 0 published it for all
    assert torch.all(flags == 80)
    # the last round's values: 39 * 7 + block
    assert torch.equal(slots.view(blocks, 64)[:, 0], 39 * 7 + torch.arange(blocks, device="cuda", dtype=torch.float32))


def test_grid_barrier_rejects_a_grid_that_cannot_be_resident():
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    flags = torch.zeros(64 * cus + 1, dtype=torch.int32, device="cuda")
    slots = torch.empty(64 * cus * 64, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    # more workgroups than the GPU holds at once: refused before any launch
    assert vb.vocoder_grid_barrier(flags, slots, err, 64 * cus, 1) == vb.VOCODER_EINVAL


def test_empty_launches():
    scratch = torch.zeros(2, dtype=torch.int32, device="cuda")
    assert vb.vocoder_empty_launches(scratch, 256, 100) == vb.VOCODER_OK
    torch.cuda.synchronize()
    assert scratch.tolist() == [0, 0]
