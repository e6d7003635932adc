"""The C-ABI library loads and exports every entry point of include/lsa.h (no GPU needed)."""
import ctypes
import os
import re

import pytest

import hierarchical_sparse_attention_lsa_amd as L

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "lsa.h")


def _declared():
    txt = open(HEADER).read()
    return sorted(set(re.findall(r"LSA_API\s+[^;(]*?\b(lsa_\w+)\s*\(", txt)))


def test_library_exports_every_declared_symbol():
    if not os.path.exists(L.LIB_PATH):
        pytest.skip("library not built")
    lib = L.lib()
    names = _declared()
    assert len(names) >= 14
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(L.EXPORTS)


def test_host_validation_without_device():
    if not os.path.exists(L.LIB_PATH):
        pytest.skip("library not built")
    lib = L.lib()
    p = L.IndexParams(64, 4, 4096, 256, 4, 0, 0, 0, 10 * 2 ** 20)
    n = ctypes.c_size_t(0)
    assert lib.lsa_index_bytes(ctypes.byref(p), ctypes.byref(n)) == 0
    # pooled 160 MiB + centroids + CSR at 10M keys
    assert 160 * 2 ** 20 < n.value < 200 * 2 ** 20
    for field, bad, code in (("dim", 32, 2), ("block", 100, 2), ("buckets", 8, 2), ("iters", 0, 1),
                             ("pool", 0, 1)):
        q = L.IndexParams(64, 4, 4096, 256, 4, 0, 0, 0, 1 << 20)
        setattr(q, field, bad)
        assert lib.lsa_index_bytes(ctypes.byref(q), ctypes.byref(n)) == code, field
        assert lib.lsa_last_error()
    sp = L.SelectParams(4096, 512, 4, 0)
    ap = L.AttnParams(32, 8, 128, 0, 0.0)
    assert L.workspace_bytes(L.binding.OP_PREFILL, p, sp, ap, 32768) >= 32768 * 4612 * 4
    # a third Tree level needs the second one and MFMA-sized point counts
    for t2, code in (((2, 16, 2), 0), ((3, 16, 2), 2), ((2, 8, 2), 2), ((2, 16, 0), 1)):
        q = L.IndexParams(64, 4, 4096, 256, 4, 64, 32, 2, 1 << 20, *t2)
        assert lib.lsa_index_bytes(ctypes.byref(q), ctypes.byref(n)) == code, t2
    q = L.IndexParams(64, 4, 4096, 256, 4, 0, 0, 0, 1 << 20, 2, 16, 2)
    assert lib.lsa_index_bytes(ctypes.byref(q), ctypes.byref(n)) == 1
    # backward at a 128k training step: the (bucket -> queries) list alone
    # needs a slot for every (query, taken bucket)
    p128 = L.IndexParams(64, 4, 4096, 256, 4, 0, 0, 0, 2 ** 17)
    assert L.workspace_bytes(L.binding.OP_ATTN_BWD, p128, sp, ap, 2 ** 17) >= 2 ** 17 * 2048 * 8
    bad = L.AttnParams(32, 8, 96, 0, 0.0)
    with pytest.raises(L.LsaError):
        L.workspace_bytes(L.binding.OP_DECODE, p, sp, bad, 8)
    # descriptor init rejects a NULL arena and an uninitialised descriptor is refused
    desc = ctypes.create_string_buffer(lib.lsa_index_sizeof())
    assert lib.lsa_index_init(desc, ctypes.byref(p), None, 0) == 1
    info = L.IndexInfo()
    assert lib.lsa_index_get_info(desc, ctypes.byref(info)) == 4
    assert lib.lsa_select(desc, None, None, 0, ctypes.byref(sp), None, None, None, 0, None) == 4


def _fake_index(lib, p):
    """A descriptor over an aligned address that is never dereferenced: the
    calls below fail validation before anything is enqueued."""
    desc = ctypes.create_string_buffer(lib.lsa_index_sizeof())
    n = ctypes.c_size_t(0)
    assert lib.lsa_index_bytes(ctypes.byref(p), ctypes.byref(n)) == 0
    assert lib.lsa_index_init(desc, ctypes.byref(p), ctypes.c_void_p(1 << 40), n.value) == 0
    return desc


def test_grouped_attention_sizes_without_device():
    """Workspace sizing of the grouped attention: the union arrays hold 16/G x
    budget rows per group, the prefill workspace grows to hold the grouped
    attention only when the attention params are given and the shape takes
    it, and shapes it does not take are refused before anything runs."""
    if not os.path.exists(L.LIB_PATH):
        pytest.skip("library not built")
    lib = L.lib()
    sp = L.SelectParams(4096, 512, 4, 0)
    ap = L.AttnParams(32, 8, 128, 0, 0.0)
    nq = 32768
    g = L.workspace_bytes(L.binding.OP_ATTN_GROUPED, None, sp, ap, nq)
    ngrp = nq // 4
    # unions (4 B row + 1 B mask per slot) and the sinks-and-window partials
    assert g >= ngrp * 4 * 4096 * 5 + nq * 32 * (128 + 2) * 4
    assert g < 2 * (ngrp * 4 * 4096 * 5 + nq * 32 * (128 + 2) * 4)
    p = L.IndexParams(64, 4, 4096, 256, 4, 0, 0, 0, 10 * 2 ** 20)
    with_attn = L.workspace_bytes(L.binding.OP_PREFILL, p, sp, ap, nq)
    without = L.workspace_bytes(L.binding.OP_PREFILL, p, sp, None, nq)
    assert with_attn >= without and with_attn >= g
    g1 = L.AttnParams(8, 8, 128, 0, 0.0)              # G = 1: no grouping, no extra space
    assert L.workspace_bytes(L.binding.OP_PREFILL, p, sp, g1, nq) == without
    with pytest.raises(L.LsaError):
        L.workspace_bytes(L.binding.OP_ATTN_GROUPED, None, sp, ap, (1 << 26) + 1)
    fake = ctypes.c_void_p(16)
    n = ctypes.c_size_t(0)
    sp_big = L.SelectParams(8192, 512, 4, 0)          # 4 queries x 8192 rows: over the union cap
    for a, s_ in ((g1, sp), (L.AttnParams(32, 8, 96, 0, 0.0), sp), (ap, sp_big)):
        rc = lib.lsa_sparse_attn_grouped(fake, fake, fake, 1 << 20, fake, fake, s_.max_sel, 16, 0, fake,
                                         ctypes.byref(s_), ctypes.byref(a), fake, None, fake,
                                         ctypes.c_size_t(1 << 40), None)
        assert rc == 2, (a.Hq, a.Hkv, a.D, s_.budget)
    # a workspace below the size is refused, nothing enqueued
    rc = lib.lsa_sparse_attn_grouped(fake, fake, fake, 1 << 20, fake, fake, sp.max_sel, 16, 0, fake,
                                     ctypes.byref(sp), ctypes.byref(ap), fake, None, fake,
                                     ctypes.c_size_t(1024), None)
    assert rc == 3


def test_training_and_tree_argument_validation_without_device():
    if not os.path.exists(L.LIB_PATH):
        pytest.skip("library not built")
    lib = L.lib()
    fake = ctypes.c_void_p(1 << 40)
    p3 = L.IndexParams(64, 4, 256, 32, 2, 2, 16, 2, 1 << 16, 4, 16, 2)
    desc = _fake_index(lib, p3)
    # a three-level index needs tree2_top; a two-level one does not
    sp = L.SelectParams(100, 32, 4, 5)
    assert lib.lsa_select(desc, fake, fake, 1, ctypes.byref(sp), fake, fake, None, 0, None) == 1
    assert b"tree2_top" in lib.lsa_last_error()
    ap = L.AttnParams(8, 2, 128, 0, 0.0)
    args = lambda spp, nq, qpos0, kv: (desc, fake, fake, fake, kv, fake, fake, spp.max_sel, nq,
                                       qpos0, None, ctypes.byref(spp), ctypes.byref(ap), fake, fake,
                                       fake, fake, fake, fake, fake, 1 << 30, None)
    sp1 = L.SelectParams(100, 32, 65, 0)
    assert lib.lsa_sparse_attn_bwd(*args(sp1, 4, 0, 1000)) == 2          # sinks > 64
    sp2 = L.SelectParams(100, 32, 4, 0)
    assert lib.lsa_sparse_attn_bwd(*args(sp2, 4, 0, 1000)) == 1          # beyond the index's T = 0
    assert b"beyond" in lib.lsa_last_error()
    assert lib.lsa_sparse_attn_bwd(*args(sp2, 4, 999, 1000)) == 1        # beyond kv_rows
    assert lib.lsa_sparse_attn_bwd(*args(sp2, 0, 0, 1000)) == 0          # empty batch: nothing to do
    bad_ap = L.AttnParams(8, 3, 128, 0, 0.0)
    assert lib.lsa_sparse_attn_fwd(fake, fake, fake, 1000, fake, fake, sp2.max_sel, 4, 0,
                                   ctypes.byref(sp2), ctypes.byref(bad_ap), fake, fake, None) == 2
    assert lib.lsa_sparse_attn_fwd(fake, fake, fake, 1000, fake, fake, sp2.max_sel, 4, 0,
                                   ctypes.byref(sp2), ctypes.byref(ap), fake, None, None) == 1
    # early budget beyond the budget
    sp3 = L.SelectParams(100, 32, 4, 5, 200, 10, 2)
    assert lib.lsa_select(desc, fake, fake, 1, ctypes.byref(sp3), fake, fake, None, 0, None) == 1
    assert b"early_budget" in lib.lsa_last_error()
