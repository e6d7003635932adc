"""Latent Sparse Attention hot path for AMD Instinct MI355X (gfx950).

The compute lives in ``liblsa_hip.so`` (hand-written HIP kernels behind the C
ABI of ``include/lsa.h``); ``binding`` is a thin ctypes layer over it.
"""
from .binding import (AttnParams, IndexInfo, IndexParams, LsaError, LsaIndex, SelectParams,  # noqa: F401
                      check, decode_selection, decode_step, decode_step_noalloc, dense_select, lib,
                      sparse_attn, sparse_attn_bwd,
                      sparse_attn_fwd, sparse_attn_grouped, sparse_attn_window,
                      workspace_bytes, EXPORTS,
                      LIB_PATH)
