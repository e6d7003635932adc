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
