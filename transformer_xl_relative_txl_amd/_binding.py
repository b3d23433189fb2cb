"""ctypes binding of libtxl (include/txl.h): argument marshalling only.

Every function here takes torch tensors that already live on the GPU, turns
them into the C structs of the header (pointers, sizes, element strides) and
calls the library on torch's current stream. No arithmetic of the method runs
in Python. If the library is missing the import fails loudly: there is no
fallback path.
"""
from __future__ import annotations

import ctypes
import os
from typing import List, Optional, Sequence

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtxl.so")

TXL_F32, TXL_BF16 = 0, 1
_STATUS = {0: "TXL_OK", 1: "TXL_ERR_INVALID_ARG", 2: "TXL_ERR_UNSUPPORTED",
           3: "TXL_ERR_WORKSPACE", 4: "TXL_ERR_HIP"}


class TxlError(RuntimeError):
    """A libtxl call returned a status other than TXL_OK."""

    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn}: {_STATUS.get(status, status)}: {msg}")
        self.status = status
        self.status_name = _STATUS.get(status, str(status))


class RelAttnArgs(ctypes.Structure):
    _fields_ = [
        ("dtype", ctypes.c_int),
        ("B", ctypes.c_int32), ("H", ctypes.c_int32), ("L", ctypes.c_int32),
        ("M", ctypes.c_int32), ("d_h", ctypes.c_int32),
        ("q", ctypes.c_void_p),
        ("q_sb", ctypes.c_int64), ("q_sh", ctypes.c_int64), ("q_sl", ctypes.c_int64),
        ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
        ("kv_sb", ctypes.c_int64), ("kv_sh", ctypes.c_int64), ("kv_sl", ctypes.c_int64),
        ("r", ctypes.c_void_p),
        ("r_sh", ctypes.c_int64), ("r_sl", ctypes.c_int64),
        ("u", ctypes.c_void_p), ("vb", ctypes.c_void_p),
        ("mem_valid", ctypes.c_void_p),
        ("scale", ctypes.c_float),
        ("out", ctypes.c_void_p),
        ("o_sb", ctypes.c_int64), ("o_sh", ctypes.c_int64), ("o_sl", ctypes.c_int64),
        ("lse", ctypes.c_void_p),
        ("out_f32", ctypes.c_void_p),
    ]


class RelAttnGrads(ctypes.Structure):
    _fields_ = [
        ("dout", ctypes.c_void_p),
        ("do_sb", ctypes.c_int64), ("do_sh", ctypes.c_int64), ("do_sl", ctypes.c_int64),
        ("dq", ctypes.c_void_p), ("dk", ctypes.c_void_p), ("dv", ctypes.c_void_p),
        ("dr", ctypes.c_void_p), ("du", ctypes.c_void_p), ("dvb", ctypes.c_void_p),
    ]


class TxlMemStruct(ctypes.Structure):
    _fields_ = [
        ("data", ctypes.c_void_p),
        ("valid", ctypes.c_void_p),
        ("head", ctypes.c_int64),
        ("B", ctypes.c_int32), ("M", ctypes.c_int32), ("d", ctypes.c_int32),
        ("dtype", ctypes.c_int),
    ]


class TxlKVCacheStruct(ctypes.Structure):
    _fields_ = [
        ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
        ("valid", ctypes.c_void_p),
        ("start", ctypes.c_int64),
        ("B", ctypes.c_int32), ("capacity", ctypes.c_int32), ("hd", ctypes.c_int32),
        ("dtype", ctypes.c_int),
    ]


class StackConfig(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("n_layer", "d", "n_head", "d_h", "d_ff", "vocab", "B", "L", "M")] + [
        ("ln_eps", ctypes.c_float), ("dtype", ctypes.c_int)]


LAYER_FIELDS = ("wq", "wk", "wv", "wo", "wr", "u", "vb", "ln1_g", "ln1_b", "w1", "w2",
                "ln2_g", "ln2_b")


class LayerWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in LAYER_FIELDS]


class StackWeights(ctypes.Structure):
    _fields_ = [("emb", ctypes.c_void_p), ("layers", ctypes.POINTER(LayerWeights))]


class LayerGrads(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in LAYER_FIELDS]


class StackGrads(ctypes.Structure):
    _fields_ = [("emb", ctypes.c_void_p), ("layers", ctypes.POINTER(LayerGrads))]


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"libtxl.so is not built at {LIB_PATH}; run "
            "`python -m transformer_xl_relative_txl_amd.build` (hipcc, gfx950)")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, st = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_int
    sz = ctypes.c_size_t
    lib.txl_status_str.argtypes = [st]
    lib.txl_status_str.restype = ctypes.c_char_p
    lib.txl_last_error.argtypes = []
    lib.txl_last_error.restype = ctypes.c_char_p
    lib.txl_version.argtypes = []
    lib.txl_version.restype = i32
    lib.txl_rel_pos_table.argtypes = [st, i32, i32, i32, i32, i32, vp, vp, vp]
    lib.txl_rel_pos_table.restype = st
    lib.txl_rel_attn_fwd.argtypes = [ctypes.POINTER(RelAttnArgs), vp]
    lib.txl_rel_attn_fwd.restype = st
    lib.txl_rel_attn_split_workspace_bytes.argtypes = [i32, i32, i32, i32]
    lib.txl_rel_attn_split_workspace_bytes.restype = sz
    lib.txl_rel_attn_fwd_split.argtypes = [ctypes.POINTER(RelAttnArgs), i32, vp, sz, vp]
    lib.txl_rel_attn_fwd_split.restype = st
    lib.txl_rel_attn_bwd_workspace_bytes.argtypes = [i32, i32, i32, i32]
    lib.txl_rel_attn_bwd_workspace_bytes.restype = sz
    lib.txl_rel_attn_bwd.argtypes = [ctypes.POINTER(RelAttnArgs), ctypes.POINTER(RelAttnGrads),
                                     vp, sz, vp]
    lib.txl_rel_attn_bwd.restype = st
    lib.txl_mem_update.argtypes = [ctypes.POINTER(TxlMemStruct), i32,
                                   ctypes.POINTER(vp), i64, i32, vp]
    lib.txl_mem_update.restype = st
    lib.txl_rel_attn_fwd_mem_update.argtypes = [ctypes.POINTER(RelAttnArgs),
                                                ctypes.POINTER(TxlMemStruct), vp, vp, sz, vp]
    lib.txl_rel_attn_fwd_mem_update.restype = st
    lib.txl_rel_attn_fwd_mem_update_noalloc.argtypes = [ctypes.POINTER(RelAttnArgs),
                                                        ctypes.POINTER(TxlMemStruct), vp, vp]
    lib.txl_rel_attn_fwd_mem_update_noalloc.restype = st
    lib.txl_rel_attn_mem_update_workspace_bytes.argtypes = [i32]
    lib.txl_rel_attn_mem_update_workspace_bytes.restype = sz
    lib.txl_mem_reset_rows.argtypes = [ctypes.POINTER(TxlMemStruct), i32, vp, vp]
    lib.txl_mem_reset_rows.restype = st
    lib.txl_mem_read_logical.argtypes = [ctypes.POINTER(TxlMemStruct), vp, vp]
    lib.txl_mem_read_logical.restype = st
    lib.txl_stack_persistent_bytes.argtypes = [ctypes.POINTER(StackConfig)]
    lib.txl_stack_persistent_bytes.restype = sz
    lib.txl_segment_step_workspace_bytes.argtypes = [ctypes.POINTER(StackConfig)]
    lib.txl_segment_step_workspace_bytes.restype = sz
    lib.txl_stack_create.argtypes = [ctypes.POINTER(StackConfig), ctypes.POINTER(StackWeights),
                                     vp, sz, vp, ctypes.POINTER(vp)]
    lib.txl_stack_create.restype = st
    lib.txl_segment_step.argtypes = [vp, vp, ctypes.POINTER(TxlMemStruct), vp, vp, sz, vp]
    lib.txl_segment_step.restype = st
    lib.txl_stack_destroy.argtypes = [vp]
    lib.txl_stack_destroy.restype = None
    lib.txl_segment_tape_bytes.argtypes = [ctypes.POINTER(StackConfig)]
    lib.txl_segment_tape_bytes.restype = sz
    lib.txl_segment_step_train.argtypes = [vp, vp, ctypes.POINTER(TxlMemStruct), vp, vp, sz,
                                           vp, sz, vp]
    lib.txl_segment_step_train.restype = st
    lib.txl_segment_backward_workspace_bytes.argtypes = [ctypes.POINTER(StackConfig)]
    lib.txl_segment_backward_workspace_bytes.restype = sz
    lib.txl_segment_backward.argtypes = [vp, vp, sz, vp, ctypes.POINTER(StackGrads), vp, sz, vp]
    lib.txl_segment_backward.restype = st
    lib.txl_kv_cache_min_capacity.argtypes = [ctypes.POINTER(StackConfig)]
    lib.txl_kv_cache_min_capacity.restype = i32
    lib.txl_segment_step_kv.argtypes = [vp, vp, ctypes.POINTER(TxlKVCacheStruct), vp, vp, sz, vp]
    lib.txl_segment_step_kv.restype = st
    lib.txl_kv_cache_reset_rows.argtypes = [ctypes.POINTER(TxlKVCacheStruct), i32, vp, vp]
    lib.txl_kv_cache_reset_rows.restype = st
    lib.txl_sampler_create.argtypes = [i32, i32, vp, vp, i32, vp, vp, i32, ctypes.POINTER(vp)]
    lib.txl_sampler_create.restype = st
    lib.txl_sampler_next.argtypes = [vp, vp, vp, vp, vp]
    lib.txl_sampler_next.restype = st
    lib.txl_sampler_destroy.argtypes = [vp]
    lib.txl_sampler_destroy.restype = None
    lib.txl_lm_loss_workspace_bytes.argtypes = [i32, i32]
    lib.txl_lm_loss_workspace_bytes.restype = sz
    lib.txl_lm_loss.argtypes = [vp, vp, vp, i32, i32, i32, vp, vp, sz, vp]
    lib.txl_lm_loss.restype = st
    return lib


_lib: Optional[ctypes.CDLL] = None


def lib() -> ctypes.CDLL:
    """The loaded library (loaded on first use)."""
    global _lib
    if _lib is None:
        _lib = _load()
    return _lib


def _check(fn: str, status: int) -> None:
    if status != 0:
        msg = lib().txl_last_error().decode(errors="replace")
        raise TxlError(fn, status, msg)


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _dtype(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return TXL_F32
    if t.dtype == torch.bfloat16:
        return TXL_BF16
    raise TypeError(f"libtxl serves float32 and bfloat16, got {t.dtype}")


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


# ----------------------------------------------------------------------------
def txl_version() -> int:
    return int(lib().txl_version())


def txl_rel_pos_table(w_r: torch.Tensor, M: int, L: int, H: int, d_h: int,
                      r: torch.Tensor, stream=None) -> torch.Tensor:
    """R [M+L, H*d_h] from W_R stored output-major [H*d_h, d] (contiguous)."""
    assert w_r.is_contiguous() and r.is_contiguous()
    d = w_r.shape[1]
    _check("txl_rel_pos_table",
           lib().txl_rel_pos_table(_dtype(w_r), M, L, d, H, d_h, _ptr(w_r), _ptr(r),
                                   _stream(stream)))
    return r


def txl_rel_attn_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                     r: torch.Tensor, u: torch.Tensor, vb: torch.Tensor,
                     out: torch.Tensor, mem_valid: Optional[torch.Tensor] = None,
                     lse: Optional[torch.Tensor] = None, scale: float = 0.0,
                     stream=None, kv_splits: int = 1,
                     workspace: Optional[torch.Tensor] = None,
                     out_f32: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Relative attention. q [B,H,L,d_h]; k, v [B,H,M+L,d_h] (same strides);
    r [H,M+L,d_h]; u, vb [H,d_h] contiguous; out [B,H,L,d_h]; mem_valid [B]
    int32; lse [B,H,L] float32; out_f32 [B,H,L,d_h] contiguous float32 (the
    unrounded output, bf16 only). Any element strides with a contiguous last
    dimension. kv_splits > 1 calls txl_rel_attn_fwd_split (workspace
    allocated here when not given)."""
    B, H, L, d_h = q.shape
    a = _attn_args(q, k, v, r, u, vb, out, mem_valid, lse, scale, out_f32)
    if kv_splits == 1:
        _check("txl_rel_attn_fwd", lib().txl_rel_attn_fwd(ctypes.byref(a), _stream(stream)))
        return out
    need = lib().txl_rel_attn_split_workspace_bytes(B, H, L, kv_splits)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _check("txl_rel_attn_fwd_split",
           lib().txl_rel_attn_fwd_split(ctypes.byref(a), kv_splits, _ptr(workspace),
                                        workspace.numel(), _stream(stream)))
    return out


def _attn_args(q, k, v, r, u, vb, out, mem_valid, lse, scale, out_f32=None) -> RelAttnArgs:
    B, H, L, d_h = q.shape
    M = k.shape[2] - L
    if k.stride() != v.stride():
        raise ValueError("k and v must share strides")
    a = RelAttnArgs()
    a.dtype = _dtype(q)
    a.B, a.H, a.L, a.M, a.d_h = B, H, L, M, d_h
    a.q = _ptr(q)
    a.q_sb, a.q_sh, a.q_sl = q.stride(0), q.stride(1), q.stride(2)
    a.k, a.v = _ptr(k), _ptr(v)
    a.kv_sb, a.kv_sh, a.kv_sl = k.stride(0), k.stride(1), k.stride(2)
    a.r = _ptr(r)
    a.r_sh, a.r_sl = r.stride(0), r.stride(1)
    a.u, a.vb = _ptr(u), _ptr(vb)
    a.mem_valid = _ptr(mem_valid)
    a.scale = float(scale)
    a.out = _ptr(out)
    a.o_sb, a.o_sh, a.o_sl = out.stride(0), out.stride(1), out.stride(2)
    a.lse = _ptr(lse)
    if out_f32 is not None:
        assert out_f32.dtype == torch.float32 and out_f32.is_contiguous()
        assert tuple(out_f32.shape) == tuple(out.shape)
    a.out_f32 = _ptr(out_f32)
    return a


def txl_rel_attn_bwd_workspace_bytes(B: int, H: int, L: int, M: int) -> int:
    return int(lib().txl_rel_attn_bwd_workspace_bytes(B, H, L, M))


def txl_rel_attn_bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                     r: torch.Tensor, u: torch.Tensor, vb: torch.Tensor,
                     out: torch.Tensor, lse: torch.Tensor, dout: torch.Tensor,
                     grads: dict, mem_valid: Optional[torch.Tensor] = None,
                     scale: float = 0.0, workspace: Optional[torch.Tensor] = None,
                     stream=None, out_f32: Optional[torch.Tensor] = None) -> dict:
    """Gradients of txl_rel_attn_fwd (bf16). q..lse are the forward call's
    tensors (out and lse as it wrote them, and out_f32 when it kept the
    unrounded output); dout [B,H,L,d_h] bf16; grads
    holds contiguous float32 outputs dq [B,H,L,d_h], dk, dv [B,H,M+L,d_h],
    dr [H,M+L,d_h], du, dvb [H,d_h] (allocated here when missing); the
    workspace is allocated here when not given."""
    B, H, L, d_h = q.shape
    M = k.shape[2] - L
    a = _attn_args(q, k, v, r, u, vb, out, mem_valid, lse, scale, out_f32)
    shapes = {"dq": (B, H, L, d_h), "dk": (B, H, M + L, d_h), "dv": (B, H, M + L, d_h),
              "dr": (H, M + L, d_h), "du": (H, d_h), "dvb": (H, d_h)}
    for name, shp in shapes.items():
        if name not in grads:
            grads[name] = torch.empty(shp, dtype=torch.float32, device=q.device)
        t = grads[name]
        if t.shape != shp or t.dtype != torch.float32 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous float32 tensor of shape {shp}")
    g = RelAttnGrads()
    g.dout = _ptr(dout)
    g.do_sb, g.do_sh, g.do_sl = dout.stride(0), dout.stride(1), dout.stride(2)
    for name in shapes:
        setattr(g, name, _ptr(grads[name]))
    if workspace is None:
        need = txl_rel_attn_bwd_workspace_bytes(B, H, L, M)
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _check("txl_rel_attn_bwd",
           lib().txl_rel_attn_bwd(ctypes.byref(a), ctypes.byref(g), _ptr(workspace),
                                  workspace.numel(), _stream(stream)))
    return grads


class TxlMem:
    """One ring-buffer memory: device tensors data [B,M,d] and valid [B]
    plus the host-side head (the C struct txl_mem)."""

    def __init__(self, data: torch.Tensor, valid: torch.Tensor, head: int = 0):
        assert data.dim() == 3 and data.is_contiguous()
        assert valid.dtype == torch.int32 and valid.shape == (data.shape[0],)
        self.data, self.valid, self.head = data, valid, int(head)

    @classmethod
    def empty(cls, B: int, M: int, d: int, dtype=torch.bfloat16, device="cuda"):
        """A fresh stream: zero-filled slots, no valid states, head 0."""
        return cls(torch.zeros((B, M, d), dtype=dtype, device=device),
                   torch.zeros((B,), dtype=torch.int32, device=device), 0)

    @property
    def B(self):
        return self.data.shape[0]

    @property
    def M(self):
        return self.data.shape[1]

    @property
    def d(self):
        return self.data.shape[2]

    def _struct(self) -> TxlMemStruct:
        s = TxlMemStruct()
        s.data, s.valid, s.head = _ptr(self.data), _ptr(self.valid), self.head
        s.B, s.M, s.d = self.B, self.M, self.d
        s.dtype = _dtype(self.data)
        return s


def _structs(mems: Sequence[TxlMem]):
    arr = (TxlMemStruct * max(1, len(mems)))()
    for i, m in enumerate(mems):
        arr[i] = m._struct()
    return arr


def txl_mem_update(mems: Sequence[TxlMem], hs: Sequence[torch.Tensor],
                   stream=None) -> None:
    """Append segment hs[n] ([B,L,d]) to ring mems[n]; heads advance. The
    segments may be views with any row stride (row (b, l) at
    (b*L + l) * stride(1) elements, so stride(0) must be L * stride(1)) and
    a contiguous last dimension; all share that row stride."""
    assert len(mems) == len(hs)
    L = hs[0].shape[1] if hs else 0
    row = hs[0].stride(1) if hs else 0
    for h in hs:
        assert h.dim() == 3 and h.shape[1] == L and h.stride(2) == 1 and h.stride(1) == row
        assert h.shape[0] <= 1 or h.stride(0) == L * row
    arr = _structs(mems)
    ptrs = (ctypes.c_void_p * max(1, len(hs)))(*[h.data_ptr() for h in hs])
    _check("txl_mem_update",
           lib().txl_mem_update(arr, len(mems), ptrs, row, L, _stream(stream)))
    for i, m in enumerate(mems):
        m.head = int(arr[i].head)


def txl_rel_attn_fwd_mem_update(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                                r: torch.Tensor, u: torch.Tensor, vb: torch.Tensor,
                                out: torch.Tensor, mem: TxlMem, h: torch.Tensor,
                                workspace: Optional[torch.Tensor] = None,
                                mem_valid: Optional[torch.Tensor] = None,
                                lse: Optional[torch.Tensor] = None, scale: float = 0.0,
                                stream=None) -> torch.Tensor:
    """txl_rel_attn_fwd followed by txl_mem_update([mem], [h]), as one launch.
    h [B,L,d] contiguous in the ring's dtype; workspace: the per-batch-row
    counters (txl_rel_attn_mem_update_workspace(B)), zero before the first
    call and left zero by each; allocated here when not given."""
    assert h.is_contiguous()
    if workspace is None:
        workspace = txl_rel_attn_mem_update_workspace(mem.B, device=h.device)
    a = _attn_args(q, k, v, r, u, vb, out, mem_valid, lse, scale)
    s = mem._struct()
    _check("txl_rel_attn_fwd_mem_update",
           lib().txl_rel_attn_fwd_mem_update(ctypes.byref(a), ctypes.byref(s), _ptr(h),
                                             _ptr(workspace),
                                             workspace.numel() * workspace.element_size(),
                                             _stream(stream)))
    mem.head = int(s.head)
    return out


def txl_rel_attn_fwd_mem_update_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                                        r: torch.Tensor, u: torch.Tensor, vb: torch.Tensor,
                                        out: torch.Tensor, mem: TxlMem, h: torch.Tensor,
                                        mem_valid: Optional[torch.Tensor] = None,
                                        lse: Optional[torch.Tensor] = None, scale: float = 0.0,
                                        stream=None) -> torch.Tensor:
    """txl_rel_attn_fwd_mem_update with the library's static counters: the
    call allocates nothing (for graph capture and serving loops). Calls that
    overlap on one GPU race."""
    assert h.is_contiguous()
    a = _attn_args(q, k, v, r, u, vb, out, mem_valid, lse, scale)
    s = mem._struct()
    _check("txl_rel_attn_fwd_mem_update_noalloc",
           lib().txl_rel_attn_fwd_mem_update_noalloc(ctypes.byref(a), ctypes.byref(s), _ptr(h),
                                                     _stream(stream)))
    mem.head = int(s.head)
    return out


def txl_rel_attn_mem_update_workspace(B: int, device="cuda") -> torch.Tensor:
    """Zeroed counters for txl_rel_attn_fwd_mem_update (keep and reuse them)."""
    n = int(lib().txl_rel_attn_mem_update_workspace_bytes(B))
    return torch.zeros(max(n, 4) // 4, dtype=torch.int32, device=device)


def txl_mem_reset_rows(mems: Sequence[TxlMem], reset: Optional[torch.Tensor] = None,
                       stream=None) -> None:
    """valid[b] = 0 in every ring for rows with reset[b] != 0 (uint8 [B]; None = all)."""
    if reset is not None:
        assert reset.dtype == torch.uint8
    arr = _structs(mems)
    _check("txl_mem_reset_rows",
           lib().txl_mem_reset_rows(arr, len(mems), _ptr(reset), _stream(stream)))


def txl_mem_read_logical(mem: TxlMem, out: torch.Tensor, stream=None) -> torch.Tensor:
    """Copy the ring out oldest-first into out [B,M,d]."""
    assert out.is_contiguous()
    s = mem._struct()
    _check("txl_mem_read_logical",
           lib().txl_mem_read_logical(ctypes.byref(s), _ptr(out), _stream(stream)))
    return out


class TxlKVCache:
    """Projected keys / values of one layer's memory (the C struct
    txl_kv_cache): device tensors k, v [B, capacity, H*d_h] and valid [B],
    plus the host-side window start."""

    def __init__(self, k: torch.Tensor, v: torch.Tensor, valid: torch.Tensor, start: int = 0):
        assert k.dim() == 3 and k.shape == v.shape and k.is_contiguous() and v.is_contiguous()
        assert valid.dtype == torch.int32 and valid.shape == (k.shape[0],)
        self.k, self.v, self.valid, self.start = k, v, valid, int(start)

    @classmethod
    def empty(cls, B: int, capacity: int, hd: int, dtype=torch.bfloat16, device="cuda"):
        """A fresh stream: no valid rows, window at row 0 (rows left uninitialised)."""
        return cls(torch.empty((B, capacity, hd), dtype=dtype, device=device),
                   torch.empty((B, capacity, hd), dtype=dtype, device=device),
                   torch.zeros((B,), dtype=torch.int32, device=device), 0)

    def _struct(self) -> TxlKVCacheStruct:
        s = TxlKVCacheStruct()
        s.k, s.v, s.valid, s.start = _ptr(self.k), _ptr(self.v), _ptr(self.valid), self.start
        s.B, s.capacity, s.hd = self.k.shape
        s.dtype = _dtype(self.k)
        return s


def _kv_structs(caches: Sequence[TxlKVCache]):
    arr = (TxlKVCacheStruct * max(1, len(caches)))()
    for i, c in enumerate(caches):
        arr[i] = c._struct()
    return arr


def txl_kv_cache_reset_rows(caches: Sequence[TxlKVCache], reset: Optional[torch.Tensor] = None,
                            stream=None) -> None:
    """valid[b] = 0 in every cache for rows with reset[b] != 0 (uint8 [B]; None = all)."""
    if reset is not None:
        assert reset.dtype == torch.uint8
    arr = _kv_structs(caches)
    _check("txl_kv_cache_reset_rows",
           lib().txl_kv_cache_reset_rows(arr, len(caches), _ptr(reset), _stream(stream)))


class TxlStack:
    """An N-layer stack (txl_stack_create): weights are torch tensors in the
    C layout (bf16, output-major, contiguous); the persistent R buffer and
    the step workspace are device tensors owned by this object."""

    def __init__(self, *, n_layer: int, d: int, n_head: int, d_h: int, d_ff: int, vocab: int,
                 B: int, L: int, M: int, emb: torch.Tensor, layers: Sequence[dict],
                 ln_eps: float = 1e-5, stream=None):
        self.cfg = StackConfig(n_layer, d, n_head, d_h, d_ff, vocab, B, L, M, ln_eps, TXL_BF16)
        self._keep = [emb] + [t for lw in layers for t in lw.values()]
        for t in self._keep:
            assert t.is_cuda and t.is_contiguous() and t.dtype == torch.bfloat16
        self._layers = (LayerWeights * n_layer)()
        for i, lw in enumerate(layers):
            self._layers[i] = LayerWeights(*[lw[n].data_ptr() for n in LAYER_FIELDS])
        self._weights = StackWeights(emb.data_ptr(), self._layers)
        pb = lib().txl_stack_persistent_bytes(ctypes.byref(self.cfg))
        wb = lib().txl_segment_step_workspace_bytes(ctypes.byref(self.cfg))
        if pb == 0 or wb == 0:
            raise TxlError("txl_stack_persistent_bytes", 2,
                           lib().txl_last_error().decode(errors="replace"))
        dev = emb.device
        self.persistent = torch.empty(pb, dtype=torch.uint8, device=dev)
        self.workspace = torch.empty(wb, dtype=torch.uint8, device=dev)
        h = ctypes.c_void_p()
        _check("txl_stack_create",
               lib().txl_stack_create(ctypes.byref(self.cfg), ctypes.byref(self._weights),
                                      self.persistent.data_ptr(), pb, _stream(stream),
                                      ctypes.byref(h)))
        self._h = h

    def r_table(self, layer: int) -> torch.Tensor:
        """Layer `layer`'s R as built by the library: [M+L, H*d_h] bf16 view."""
        c = self.cfg
        hd = c.n_head * c.d_h
        per = ((c.M + c.L) * hd * 2 + 255) // 256 * 256   # 256-byte aligned tables
        raw = self.persistent[layer * per: layer * per + (c.M + c.L) * hd * 2]
        return raw.view(torch.bfloat16).view(c.M + c.L, hd)

    def step(self, tokens: torch.Tensor, mems: Sequence[TxlMem], h_out: torch.Tensor,
             stream=None) -> torch.Tensor:
        """txl_segment_step: tokens [B, L] int32, n_layer + 1 rings, h_out [B, L, d]."""
        assert tokens.dtype == torch.int32 and tokens.is_contiguous()
        assert len(mems) == self.cfg.n_layer + 1 and h_out.is_contiguous()
        arr = _structs(mems)
        _check("txl_segment_step",
               lib().txl_segment_step(self._h, tokens.data_ptr(), arr, h_out.data_ptr(),
                                      self.workspace.data_ptr(), self.workspace.numel(),
                                      _stream(stream)))
        for i, m in enumerate(mems):
            m.head = int(arr[i].head)
        return h_out

    def tape_bytes(self) -> int:
        """txl_segment_tape_bytes of this stack's configuration."""
        return int(lib().txl_segment_tape_bytes(ctypes.byref(self.cfg)))

    def new_tape(self) -> torch.Tensor:
        """A device buffer of txl_segment_tape_bytes (uint8)."""
        return torch.empty(self.tape_bytes(), dtype=torch.uint8, device=self.persistent.device)

    def step_train(self, tokens: torch.Tensor, mems: Sequence[TxlMem], h_out: torch.Tensor,
                   tape: torch.Tensor, stream=None) -> torch.Tensor:
        """txl_segment_step_train: txl_segment_step that also fills `tape`."""
        assert tokens.dtype == torch.int32 and tokens.is_contiguous()
        assert len(mems) == self.cfg.n_layer + 1 and h_out.is_contiguous()
        assert tape.dtype == torch.uint8 and tape.is_contiguous()
        arr = _structs(mems)
        _check("txl_segment_step_train",
               lib().txl_segment_step_train(self._h, tokens.data_ptr(), arr, h_out.data_ptr(),
                                            tape.data_ptr(), tape.numel(),
                                            self.workspace.data_ptr(), self.workspace.numel(),
                                            _stream(stream)))
        for i, m in enumerate(mems):
            m.head = int(arr[i].head)
        return h_out

    def new_grads(self) -> dict:
        """fp32 device gradient buffers in the weights' layout:
        {"emb": [vocab, d], "layers": [ {name: tensor} per layer ]}."""
        c = self.cfg
        hd = c.n_head * c.d_h
        shapes = {"wq": (hd, c.d), "wk": (hd, c.d), "wv": (hd, c.d), "wr": (hd, c.d),
                  "wo": (c.d, hd), "u": (c.n_head, c.d_h), "vb": (c.n_head, c.d_h),
                  "ln1_g": (c.d,), "ln1_b": (c.d,), "ln2_g": (c.d,), "ln2_b": (c.d,),
                  "w1": (c.d_ff, c.d), "w2": (c.d, c.d_ff)}
        dev = self.persistent.device
        return {"emb": torch.empty(c.vocab, c.d, dtype=torch.float32, device=dev),
                "layers": [{n: torch.empty(*shapes[n], dtype=torch.float32, device=dev)
                            for n in LAYER_FIELDS} for _ in range(c.n_layer)]}

    def backward(self, tape: torch.Tensor, dy: torch.Tensor, grads: dict,
                 workspace: Optional[torch.Tensor] = None, stream=None) -> dict:
        """txl_segment_backward: dy [B, L, d] fp32 (gradient at h_out) and the
        tape of the matching step_train; fills `grads` (see new_grads)."""
        assert dy.dtype == torch.float32 and dy.is_contiguous()
        assert tape.dtype == torch.uint8 and tape.is_contiguous()
        if workspace is None:
            if getattr(self, "_bwd_ws", None) is None:
                nb = int(lib().txl_segment_backward_workspace_bytes(ctypes.byref(self.cfg)))
                self._bwd_ws = torch.empty(nb, dtype=torch.uint8, device=self.persistent.device)
            workspace = self._bwd_ws
        tensors = [grads["emb"]] + [t for lg in grads["layers"] for t in lg.values()]
        for t in tensors:
            assert t.is_cuda and t.is_contiguous() and t.dtype == torch.float32
        layers = (LayerGrads * self.cfg.n_layer)()
        for i, lg in enumerate(grads["layers"]):
            layers[i] = LayerGrads(*[lg[n].data_ptr() for n in LAYER_FIELDS])
        sg = StackGrads(grads["emb"].data_ptr(), layers)
        _check("txl_segment_backward",
               lib().txl_segment_backward(self._h, tape.data_ptr(), tape.numel(), dy.data_ptr(),
                                          ctypes.byref(sg), workspace.data_ptr(), workspace.numel(),
                                          _stream(stream)))
        return grads

    def kv_min_capacity(self) -> int:
        """txl_kv_cache_min_capacity: 2*M + L."""
        return int(lib().txl_kv_cache_min_capacity(ctypes.byref(self.cfg)))

    def step_kv(self, tokens: torch.Tensor, caches: Sequence["TxlKVCache"], h_out: torch.Tensor,
                stream=None) -> torch.Tensor:
        """txl_segment_step_kv: tokens [B, L] int32, n_layer caches, h_out [B, L, d]."""
        assert tokens.dtype == torch.int32 and tokens.is_contiguous()
        assert len(caches) == self.cfg.n_layer and h_out.is_contiguous()
        arr = _kv_structs(caches)
        _check("txl_segment_step_kv",
               lib().txl_segment_step_kv(self._h, tokens.data_ptr(), arr, h_out.data_ptr(),
                                         self.workspace.data_ptr(), self.workspace.numel(),
                                         _stream(stream)))
        for i, c in enumerate(caches):
            c.start = int(arr[i].start)
        return h_out

    def close(self):
        if getattr(self, "_h", None):
            lib().txl_stack_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class StreamSampler:
    """The per-row stream sampler (txl_sampler_*; host only): docs_per_row[b]
    is the list of documents (token id sequences) row b streams, in order."""

    def __init__(self, docs_per_row: Sequence[Sequence[Sequence[int]]], L: int, pad_id: int = 0):
        import numpy as np
        flat, offs, row_offs, row_docs = [], [0], [0], []
        for docs in docs_per_row:
            for doc in docs:
                flat.extend(int(t) for t in doc)
                offs.append(len(flat))
                row_docs.append(len(offs) - 2)
            row_offs.append(len(row_docs))
        self.B, self.L = len(docs_per_row), int(L)
        tok = np.asarray(flat, dtype=np.int32)
        off = np.asarray(offs, dtype=np.int64)
        ro = np.asarray(row_offs, dtype=np.int32)
        rd = np.asarray(row_docs, dtype=np.int32)
        h = ctypes.c_void_p()
        _check("txl_sampler_create",
               lib().txl_sampler_create(self.B, self.L, tok.ctypes.data, off.ctypes.data,
                                        len(offs) - 1, ro.ctypes.data, rd.ctypes.data,
                                        int(pad_id), ctypes.byref(h)))
        self._h = h

    def next(self):
        """(tokens [B, L] int32, targets [B, L] int32, reset [B] uint8,
        lengths [B] int32) as host numpy arrays."""
        import numpy as np
        tok = np.empty((self.B, self.L), dtype=np.int32)
        tgt = np.empty((self.B, self.L), dtype=np.int32)
        rst = np.empty((self.B,), dtype=np.uint8)
        ln = np.empty((self.B,), dtype=np.int32)
        _check("txl_sampler_next",
               lib().txl_sampler_next(self._h, tok.ctypes.data, tgt.ctypes.data, rst.ctypes.data,
                                      ln.ctypes.data))
        return tok, tgt, rst, ln

    def close(self):
        if getattr(self, "_h", None):
            lib().txl_sampler_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def txl_lm_loss(h: torch.Tensor, w_out: torch.Tensor, targets: torch.Tensor, nll: torch.Tensor,
                workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """nll[n] = logsumexp(w_out h[n]) - (w_out h[n])[targets[n]] (0 where the
    target is outside the vocabulary). h [n_tok, d] and w_out [vocab, d] bf16
    contiguous; targets int32 [n_tok]; nll fp32 [n_tok]."""
    assert h.is_contiguous() and w_out.is_contiguous() and targets.is_contiguous()
    assert targets.dtype == torch.int32 and nll.dtype == torch.float32
    n_tok, d = h.reshape(-1, h.shape[-1]).shape
    vocab = w_out.shape[0]
    need = lib().txl_lm_loss_workspace_bytes(n_tok, vocab)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=h.device)
    _check("txl_lm_loss",
           lib().txl_lm_loss(_ptr(h), _ptr(w_out), _ptr(targets), n_tok, d, vocab, _ptr(nll),
                             _ptr(workspace), workspace.numel(), _stream(stream)))
    return nll


def exported_symbols() -> List[str]:
    """Names of the C entry points this binding wraps."""
    return ["txl_rel_pos_table", "txl_rel_attn_fwd", "txl_rel_attn_split_workspace_bytes",
            "txl_rel_attn_fwd_split", "txl_rel_attn_bwd_workspace_bytes", "txl_rel_attn_bwd",
            "txl_mem_update", "txl_rel_attn_fwd_mem_update",
            "txl_rel_attn_fwd_mem_update_noalloc", "txl_rel_attn_mem_update_workspace_bytes",
            "txl_mem_reset_rows", "txl_mem_read_logical", "txl_stack_persistent_bytes",
            "txl_stack_create", "txl_segment_step_workspace_bytes", "txl_segment_step",
            "txl_stack_destroy", "txl_segment_tape_bytes", "txl_segment_step_train",
            "txl_segment_backward_workspace_bytes", "txl_segment_backward",
            "txl_kv_cache_min_capacity", "txl_segment_step_kv",
            "txl_kv_cache_reset_rows", "txl_sampler_create", "txl_sampler_next",
            "txl_sampler_destroy", "txl_lm_loss_workspace_bytes", "txl_lm_loss",
            "txl_status_str", "txl_last_error", "txl_version"]
