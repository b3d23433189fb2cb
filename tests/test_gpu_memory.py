"""GPU ring-buffer memory against the oracle's Tail_M (bit-exact).

The ring (txl_mem_update / txl_mem_reset_rows / txl_mem_read_logical) must
hold, for every row, exactly the states the oracle's variable-length memory
holds: the last valid[b] logical slots equal Tail_M of the row's history since
its last reset.
"""
import numpy as np
import pytest
import torch

import transformer_xl_relative_txl_amd as txl
from oracle import memory as om
from tests.gpu_helpers import say

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _logical(mem):
    out = torch.empty_like(mem.data)
    txl.txl_mem_read_logical(mem, out)
    torch.cuda.synchronize()
    return out.cpu()


def _check_rows(mem, ref_rows):
    logi = _logical(mem)
    valid = mem.valid.cpu().numpy()
    for b, ref in enumerate(ref_rows):
        assert valid[b] == ref.shape[0], (b, valid[b], ref.shape)
        got = logi[b, mem.M - valid[b]:].double().numpy()
        assert np.array_equal(got, ref), b


@pytest.mark.parametrize("n_rings", [1, 3])   # one ring takes its own kernel
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("B,M,L,d", [(1, 8, 4, 64), (3, 5, 2, 16), (2, 6, 6, 32),
                                      (2, 4, 7, 64), (8, 512, 512, 1024), (4, 640, 128, 64)])
def test_ring_matches_tail(dtype, B, M, L, d, n_rings):
    say(f"ring B{B} M{M} L{L} d{d} {dtype} rings {n_rings}")
    g = torch.Generator().manual_seed(B * 100 + M + L)
    mems = [txl.TxlMem.empty(B, M, d, dtype=dtype) for _ in range(n_rings)]
    ref = [[np.zeros((0, d)) for _ in range(B)] for _ in range(n_rings)]
    for s in range(5):
        hs = [torch.randn((B, L, d), generator=g).to(dtype) for _ in range(n_rings)]
        txl.txl_mem_update(mems, [h.to(DEV) for h in hs])
        for n in range(n_rings):
            ref[n] = om.update_rows(ref[n], hs[n].double().numpy(), M)
            assert mems[n].head == ((s + 1) * min(L, M)) % M
        for n in range(n_rings):
            _check_rows(mems[n], ref[n])


def test_reset_rows_then_grow():
    B, M, L, d = 4, 6, 4, 16
    g = torch.Generator().manual_seed(3)
    mems = [txl.TxlMem.empty(B, M, d, dtype=torch.float32) for _ in range(2)]
    ref = [[np.zeros((0, d)) for _ in range(B)] for _ in range(2)]
    for s in range(6):
        if s in (2, 4):
            flags = torch.tensor([1, 0, s == 4, 0], dtype=torch.uint8)
            txl.txl_mem_reset_rows(mems, flags.to(DEV))
            for n in range(2):
                ref[n] = [np.zeros((0, d)) if flags[b] else ref[n][b] for b in range(B)]
        hs = [torch.randn((B, L, d), generator=g) for _ in range(2)]
        txl.txl_mem_update(mems, [h.to(DEV) for h in hs])
        for n in range(2):
            ref[n] = om.update_rows(ref[n], hs[n].double().numpy(), M)
            _check_rows(mems[n], ref[n])
    txl.txl_mem_reset_rows(mems, None)
    torch.cuda.synchronize()
    for m in mems:
        assert (m.valid.cpu() == 0).all()


def test_zero_capacity_is_noop():
    mems = [txl.TxlMem.empty(2, 0, 16, dtype=torch.float32)]
    h = torch.randn((2, 3, 16), device=DEV)
    txl.txl_mem_update(mems, [h])
    torch.cuda.synchronize()
    assert mems[0].head == 0 and (mems[0].valid.cpu() == 0).all()


def test_many_rings_one_call():
    """More rings than one launch takes (the host splits the batch)."""
    B, M, L, d = 2, 5, 3, 8
    n = 40
    mems = [txl.TxlMem.empty(B, M, d, dtype=torch.float32) for _ in range(n)]
    hs = [torch.full((B, L, d), float(i), device=DEV) for i in range(n)]
    txl.txl_mem_update(mems, hs)
    txl.txl_mem_update(mems, hs)
    for i in (0, 31, 32, 39):
        logi = _logical(mems[i])
        assert (logi[:, M - 5:] == float(i)).all()
        assert (mems[i].valid.cpu() == 5).all()


def test_rejects_mismatched_rings():
    a = txl.TxlMem.empty(2, 4, 8, dtype=torch.float32)
    b = txl.TxlMem.empty(3, 4, 8, dtype=torch.float32)
    h = torch.zeros((2, 2, 8), device=DEV)
    with pytest.raises(txl.TxlError) as e:
        txl.txl_mem_update([a, b], [h, torch.zeros((3, 2, 8), device=DEV)])
    assert e.value.status_name == "TXL_ERR_INVALID_ARG"
    assert a.head == 0 and b.head == 0


@pytest.mark.parametrize("n_rings", [1, 3])
@pytest.mark.parametrize("B,M,L,d,extra", [(2, 6, 4, 16, 8), (3, 5, 7, 64, 64),
                                            (2, 384, 384, 512, 512), (1, 8, 3, 1024, 24)])
def test_strided_segment_view(B, M, L, d, extra, n_rings):
    """h_row_stride: each segment is the first d columns of a wider
    [B, L, d + extra] buffer (row stride d + extra); the ring must equal
    Tail_M of those d columns, and nothing of the extra columns may enter."""
    say(f"strided ring B{B} M{M} L{L} d{d} stride {d + extra} rings {n_rings}")
    g = torch.Generator().manual_seed(B * 7 + M + L + d)
    mems = [txl.TxlMem.empty(B, M, d, dtype=torch.bfloat16) for _ in range(n_rings)]
    ref = [[np.zeros((0, d)) for _ in range(B)] for _ in range(n_rings)]
    for s in range(4):
        wide = [torch.randn((B, L, d + extra), generator=g).to(torch.bfloat16)
                for _ in range(n_rings)]
        views = [w.to(DEV)[:, :, :d] for w in wide]
        assert views[0].stride(1) == d + extra
        txl.txl_mem_update(mems, views)
        for n in range(n_rings):
            ref[n] = om.update_rows(ref[n], wide[n][:, :, :d].double().numpy(), M)
            _check_rows(mems[n], ref[n])


def test_row_stride_below_width_is_rejected():
    a = txl.TxlMem.empty(2, 4, 16, dtype=torch.float32)
    import ctypes
    from transformer_xl_relative_txl_amd import _binding as bd
    h = torch.zeros((2, 3, 16), device=DEV)
    arr = bd._structs([a])
    ptrs = (ctypes.c_void_p * 1)(h.data_ptr())
    st = bd.lib().txl_mem_update(arr, 1, ptrs, 8, 3, None)
    assert st == 1 and a.head == 0
