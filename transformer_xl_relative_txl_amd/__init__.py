"""libtxl for MI355X: Transformer-XL relative-position memory attention.

The HIP library (libtxl.so, built by ``transformer_xl_relative_txl_amd.build``)
holds every kernel; this package only marshals torch tensors into its C ABI.
"""
from ._binding import (  # noqa: F401
    LIB_PATH,
    StreamSampler,
    TXL_BF16,
    TXL_F32,
    TxlError,
    TxlKVCache,
    TxlMem,
    TxlStack,
    lib,
    txl_kv_cache_reset_rows,
    txl_lm_loss,
    txl_mem_read_logical,
    txl_mem_reset_rows,
    txl_mem_update,
    txl_rel_attn_bwd,
    txl_rel_attn_bwd_workspace_bytes,
    txl_rel_attn_fwd,
    txl_rel_attn_fwd_mem_update,
    txl_rel_attn_fwd_mem_update_noalloc,
    txl_rel_attn_mem_update_workspace,
    txl_rel_pos_table,
    txl_version,
)
