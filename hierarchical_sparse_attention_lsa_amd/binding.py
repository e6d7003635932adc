"""Thin ctypes binding of the liblsa_hip C ABI (include/lsa.h).

Argument marshalling only: torch tensors provide device memory and
``torch.cuda.current_stream()`` provides the stream; every step of the hot
path runs in the HIP kernels of ``liblsa_hip.so``.  There is no fallback: if
the library is missing or a call fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional, Sequence

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liblsa_hip.so")

c_i32, c_i64, c_f32, c_vp, c_sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t

(OP_BUILD, OP_APPEND, OP_SELECT, OP_ATTN, OP_PREFILL, OP_DECODE, OP_DENSE, OP_ATTN_BWD,
 OP_ATTN_GROUPED) = range(9)


class IndexParams(ctypes.Structure):
    _fields_ = [("dim", c_i32), ("pool", c_i32), ("block", c_i32), ("buckets", c_i32),
                ("iters", c_i32), ("tree_group", c_i32), ("tree_super", c_i32),
                ("tree_iters", c_i32), ("max_tokens", c_i64), ("tree2_group", c_i32),
                ("tree2_super", c_i32), ("tree2_iters", c_i32)]


class SelectParams(ctypes.Structure):
    _fields_ = [("budget", c_i32), ("window", c_i32), ("sinks", c_i32), ("tree_top", c_i32),
                ("early_budget", c_i32), ("early_until", c_i32), ("tree2_top", c_i32)]

    @property
    def max_sel(self) -> int:
        return self.budget + self.window + self.sinks


class AttnParams(ctypes.Structure):
    _fields_ = [("Hq", c_i32), ("Hkv", c_i32), ("D", c_i32), ("out_f32", c_i32), ("scale", c_f32)]


class IndexInfo(ctypes.Structure):
    _fields_ = [(n, c_i64) for n in (
        "T", "n_pool", "n_full", "n_bkt", "n_grp", "n_sup",
        "off_pooled", "off_cent", "off_bcnt", "off_boff", "off_bmem", "off_bfirst", "off_blast",
        "off_scent", "off_scnt", "off_soff", "off_smem", "arena_bytes",
        "n_grp2", "n_top", "off_tcent", "off_tcnt", "off_toff", "off_tmem")]


EXPORTS = {
    "lsa_status_str": (ctypes.c_char_p, [c_i32]),
    "lsa_last_error": (ctypes.c_char_p, []),
    "lsa_check": (c_i32, [c_vp]),
    "lsa_index_sizeof": (c_sz, []),
    "lsa_index_bytes": (c_i32, [ctypes.POINTER(IndexParams), ctypes.POINTER(c_sz)]),
    "lsa_index_init": (c_i32, [c_vp, ctypes.POINTER(IndexParams), c_vp, c_sz]),
    "lsa_index_get_info": (c_i32, [c_vp, ctypes.POINTER(IndexInfo)]),
    "lsa_workspace_bytes": (c_i32, [c_i32, ctypes.POINTER(IndexParams), ctypes.POINTER(SelectParams),
                                    ctypes.POINTER(AttnParams), c_i64, ctypes.POINTER(c_sz)]),
    "lsa_build_index": (c_i32, [c_vp, c_vp, c_i64, c_vp, c_sz, c_vp]),
    "lsa_append_keys": (c_i32, [c_vp, c_vp, c_i64, c_vp, c_sz, c_vp]),
    "lsa_select": (c_i32, [c_vp, c_vp, c_vp, c_i32, ctypes.POINTER(SelectParams), c_vp, c_vp,
                           c_vp, c_sz, c_vp]),
    "lsa_sparse_attn": (c_i32, [c_vp, c_vp, c_vp, c_i64, c_vp, c_vp, c_i32, c_i32,
                                ctypes.POINTER(AttnParams), c_vp, c_vp, c_sz, c_vp]),
    "lsa_sparse_attn_window": (c_i32, [c_vp, c_vp, c_vp, c_i64, c_vp, c_vp, c_i32, c_i32, c_i64,
                                       ctypes.POINTER(SelectParams), ctypes.POINTER(AttnParams),
                                       c_vp, c_vp]),
    "lsa_sparse_attn_grouped": (c_i32, [c_vp, c_vp, c_vp, c_i64, c_vp, c_vp, c_i32, c_i32, c_i64,
                                        c_vp, ctypes.POINTER(SelectParams),
                                        ctypes.POINTER(AttnParams), c_vp, c_vp, c_vp, c_sz, c_vp]),
    "lsa_attn_grouped_prepare": (c_i32, [c_vp, c_vp, c_vp, c_i64, c_vp, c_vp, c_i32, c_i32, c_i64,
                                         c_vp, ctypes.POINTER(SelectParams),
                                         ctypes.POINTER(AttnParams), c_vp, c_sz, c_vp]),
    "lsa_attn_grouped_walk": (c_i32, [c_vp, c_vp, c_vp, c_i64, c_vp, c_vp, c_i32, c_i32, c_i64,
                                      ctypes.POINTER(SelectParams), ctypes.POINTER(AttnParams),
                                      c_vp, c_vp, c_vp, c_sz, c_vp]),
    "lsa_sparse_attn_fwd": (c_i32, [c_vp, c_vp, c_vp, c_i64, c_vp, c_vp, c_i32, c_i32, c_i64,
                                    ctypes.POINTER(SelectParams), ctypes.POINTER(AttnParams),
                                    c_vp, c_vp, c_vp]),
    "lsa_sparse_attn_bwd": (c_i32, [c_vp, c_vp, c_vp, c_vp, c_i64, c_vp, c_vp, c_i32, c_i32, c_i64,
                                    c_vp, ctypes.POINTER(SelectParams), ctypes.POINTER(AttnParams),
                                    c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_sz, c_vp]),
    "lsa_prefill_chunk": (c_i32, [c_vp, c_vp, c_i64, c_vp, c_vp, c_vp, c_vp, c_i64,
                                  ctypes.POINTER(SelectParams), ctypes.POINTER(AttnParams), c_vp,
                                  c_vp, c_vp, c_vp, c_sz, c_vp]),
    "lsa_decode_step": (c_i32, [ctypes.POINTER(c_vp), c_i32, c_vp, c_vp, c_vp, c_vp, c_vp, c_i64,
                                ctypes.POINTER(SelectParams), ctypes.POINTER(AttnParams), c_vp,
                                c_vp, c_sz, c_vp]),
    "lsa_dense_select": (c_i32, [c_vp, c_i64, c_vp, c_vp, c_i32, ctypes.POINTER(SelectParams),
                                 c_vp, c_vp, c_vp, c_sz, c_vp]),
    "lsa_decode_step_noalloc_max_bytes": (c_sz, []),
    "lsa_decode_step_noalloc": (c_i32, [ctypes.POINTER(c_vp), c_i32, c_vp, c_vp, c_vp, c_vp, c_vp,
                                        c_i64, ctypes.POINTER(SelectParams), ctypes.POINTER(AttnParams),
                                        c_vp, c_vp]),
}

_lib = None


class LsaError(RuntimeError):
    pass


def lib() -> ctypes.CDLL:
    """Load liblsa_hip.so (built in-tree); raise if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise LsaError(f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in EXPORTS.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _check(rc: int, what: str) -> None:
    if rc != 0:
        L = lib()
        raise LsaError(f"{what}: {L.lsa_status_str(rc).decode()}: {L.lsa_last_error().decode()}")


def check(stream=None) -> None:
    """Wait for the stream's work and raise LsaError if an earlier call's
    kernels failed on the device."""
    _check(lib().lsa_check(_stream(stream)), "lsa_check")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else c_vp(t.data_ptr())


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return c_vp(s.cuda_stream)


def _need(t: torch.Tensor, dtype, name: str, shape=None):
    if not t.is_cuda:
        raise LsaError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise LsaError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise LsaError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise LsaError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _bits(t: torch.Tensor) -> torch.Tensor:
    """bf16 tensors travel as their 16-bit patterns."""
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t


def workspace_bytes(op: int, iprm: Optional[IndexParams], sprm: Optional[SelectParams],
                    aprm: Optional[AttnParams], n: int) -> int:
    out = c_sz(0)
    _check(lib().lsa_workspace_bytes(op, ctypes.byref(iprm) if iprm else None,
                                     ctypes.byref(sprm) if sprm else None,
                                     ctypes.byref(aprm) if aprm else None, n, ctypes.byref(out)),
           "lsa_workspace_bytes")
    return out.value


class LsaIndex:
    """An LSA index over a device arena (caller-owned torch memory)."""

    def __init__(self, params: IndexParams, device="cuda"):
        L = lib()
        self.params = params
        nbytes = c_sz(0)
        _check(L.lsa_index_bytes(ctypes.byref(params), ctypes.byref(nbytes)), "lsa_index_bytes")
        self.arena = torch.empty(max(nbytes.value, 256), dtype=torch.uint8, device=device)
        self._desc = ctypes.create_string_buffer(L.lsa_index_sizeof())
        _check(L.lsa_index_init(self._desc, ctypes.byref(params), c_vp(self.arena.data_ptr()),
                                self.arena.numel()), "lsa_index_init")

    @property
    def handle(self):
        return ctypes.cast(self._desc, c_vp)

    def snapshot(self) -> bytes:
        """Host descriptor bytes (the device arena is not copied)."""
        return bytes(self._desc.raw)

    def restore(self, snap: bytes) -> None:
        ctypes.memmove(self._desc, snap, len(snap))

    def build(self, latk: torch.Tensor, stream=None) -> None:
        _need(latk, torch.int8, "latk")
        _check(lib().lsa_build_index(self._desc, _ptr(latk), latk.shape[0], None, 0,
                                     _stream(stream)), "lsa_build_index")

    def append(self, latk_new: torch.Tensor, stream=None) -> None:
        _need(latk_new, torch.int8, "latk_new")
        _check(lib().lsa_append_keys(self._desc, _ptr(latk_new), latk_new.shape[0], None, 0,
                                     _stream(stream)), "lsa_append_keys")

    def info(self) -> IndexInfo:
        out = IndexInfo()
        _check(lib().lsa_index_get_info(self._desc, ctypes.byref(out)), "lsa_index_get_info")
        return out

    def arrays(self) -> Dict[str, torch.Tensor]:
        """Views of the built index arrays inside the arena."""
        i = self.info()
        a = self.arena

        def view(off, n, dtype, width=1):
            esz = torch.empty((), dtype=dtype).element_size()
            return a[off: off + n * width * esz].view(dtype).view(n, width) if width > 1 else \
                a[off: off + n * esz].view(dtype)
        G = self.params.tree_group
        nsm = i.n_grp * G * self.params.buckets
        return {
            "pooled": view(i.off_pooled, i.n_pool, torch.int8, 64),
            "cent": view(i.off_cent, i.n_bkt, torch.int8, 64),
            "bcnt": view(i.off_bcnt, i.n_bkt, torch.int32),
            "boff": view(i.off_boff, i.n_bkt, torch.int32),
            "bmem": view(i.off_bmem, i.n_pool, torch.int32),
            "bfirst": view(i.off_bfirst, i.n_bkt, torch.int32),
            "blast": view(i.off_blast, i.n_bkt, torch.int32),
            "scent": view(i.off_scent, i.n_sup, torch.int8, 64),
            "scnt": view(i.off_scnt, i.n_sup, torch.int32),
            "soff": view(i.off_soff, i.n_sup, torch.int32),
            "smem": view(i.off_smem, nsm, torch.int32),
            "tcent": view(i.off_tcent, i.n_top, torch.int8, 64),
            "tcnt": view(i.off_tcnt, i.n_top, torch.int32),
            "toff": view(i.off_toff, i.n_top, torch.int32),
            "tmem": view(i.off_tmem, i.n_grp2 * self.params.tree2_group * self.params.tree_super,
                         torch.int32),
        }

    def select(self, latq: torch.Tensor, qpos: torch.Tensor, sp: SelectParams,
               idx: Optional[torch.Tensor] = None, cnt: Optional[torch.Tensor] = None,
               ws: Optional[torch.Tensor] = None, use_workspace: bool = True, stream=None):
        """Select keys for each query.  With a workspace (allocated here unless
        given) large Flat batches take the single-scan list path; without one
        (use_workspace=False) every query takes the exact refinement path."""
        nq = latq.shape[0]
        _need(latq, torch.int8, "latq", (nq, 64))
        _need(qpos, torch.int32, "qpos", (nq,))
        if idx is None:
            idx = torch.empty((nq, sp.max_sel), dtype=torch.int32, device=latq.device)
        if cnt is None:
            cnt = torch.empty((nq,), dtype=torch.int32, device=latq.device)
        _need(idx, torch.int32, "idx", (nq, sp.max_sel))
        _need(cnt, torch.int32, "cnt", (nq,))
        if use_workspace and ws is None:
            ws = torch.empty(max(workspace_bytes(OP_SELECT, self.params, sp, None, nq), 256),
                             dtype=torch.uint8, device=latq.device)
        if not use_workspace:
            ws = None
        _check(lib().lsa_select(self._desc, _ptr(latq), _ptr(qpos), nq, ctypes.byref(sp),
                                _ptr(idx), _ptr(cnt), _ptr(ws), ws.numel() if ws is not None else 0,
                                _stream(stream)), "lsa_select")
        return idx, cnt

    def prefill_chunk(self, latk_chunk: torch.Tensor, latq: torch.Tensor, q: torch.Tensor,
                      k: torch.Tensor, v: torch.Tensor, sp: SelectParams, ap: AttnParams,
                      out: Optional[torch.Tensor] = None, idx: Optional[torch.Tensor] = None,
                      cnt: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None,
                      stream=None) -> torch.Tensor:
        n = latk_chunk.shape[0]
        _need(latk_chunk, torch.int8, "latk_chunk", (n, 64))
        _need(latq, torch.int8, "latq", (n, 64))
        for name, t in (("q", q), ("k", k), ("v", v)):
            if t.dtype != torch.bfloat16:
                raise LsaError(f"{name} must be bfloat16")
            _need(t, torch.bfloat16, name)
        if out is None:
            out = torch.empty((n, ap.Hq, ap.D), dtype=torch.float32 if ap.out_f32 else torch.bfloat16,
                              device=q.device)
        if (idx is None) != (cnt is None):
            raise LsaError("pass both idx and cnt or neither")
        wsb = workspace_bytes(OP_PREFILL, self.params, sp, ap, n)
        if ws is None or ws.numel() < wsb:
            ws = torch.empty(wsb, dtype=torch.uint8, device=q.device)
        _check(lib().lsa_prefill_chunk(self._desc, _ptr(latk_chunk), n, _ptr(latq), _ptr(q),
                                       _ptr(k), _ptr(v), k.shape[0], ctypes.byref(sp),
                                       ctypes.byref(ap), _ptr(out), _ptr(idx), _ptr(cnt),
                                       _ptr(ws), ws.numel(), _stream(stream)), "lsa_prefill_chunk")
        return out


def sparse_attn(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, idx: torch.Tensor,
                cnt: torch.Tensor, ap: AttnParams, out: Optional[torch.Tensor] = None,
                stream=None) -> torch.Tensor:
    nq = q.shape[0]
    for name, t in (("q", q), ("k", k), ("v", v)):
        _need(t, torch.bfloat16, name)
    _need(idx, torch.int32, "idx")
    _need(cnt, torch.int32, "cnt", (nq,))
    if out is None:
        out = torch.empty((nq, ap.Hq, ap.D), dtype=torch.float32 if ap.out_f32 else torch.bfloat16,
                          device=q.device)
    _check(lib().lsa_sparse_attn(_ptr(q), _ptr(k), _ptr(v), k.shape[0], _ptr(idx), _ptr(cnt),
                                 idx.shape[1], nq, ctypes.byref(ap), _ptr(out), None, 0,
                                 _stream(stream)), "lsa_sparse_attn")
    return out


def sparse_attn_window(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, idx: torch.Tensor,
                       cnt: torch.Tensor, qpos0: int, sp: SelectParams, ap: AttnParams,
                       out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Attention of queries at positions qpos0.. over rows written by select
    with `sp`; the sinks and window are shared by consecutive queries."""
    nq = q.shape[0]
    for name, t in (("q", q), ("k", k), ("v", v)):
        _need(t, torch.bfloat16, name)
    _need(idx, torch.int32, "idx")
    _need(cnt, torch.int32, "cnt", (nq,))
    if out is None:
        out = torch.empty((nq, ap.Hq, ap.D), dtype=torch.float32 if ap.out_f32 else torch.bfloat16,
                          device=q.device)
    _check(lib().lsa_sparse_attn_window(_ptr(q), _ptr(k), _ptr(v), k.shape[0], _ptr(idx), _ptr(cnt),
                                        idx.shape[1], nq, qpos0, ctypes.byref(sp), ctypes.byref(ap),
                                        _ptr(out), _stream(stream)), "lsa_sparse_attn_window")
    return out


def sparse_attn_grouped(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, idx: torch.Tensor,
                        cnt: torch.Tensor, qpos0: int, sp: SelectParams, ap: AttnParams,
                        out: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None,
                        stream=None, part: str = "all", lse: Optional[torch.Tensor] = None,
                        latq: Optional[torch.Tensor] = None):
    """sparse_attn_window with each group of 16/G queries reading the union of
    its long-range keys once.  The queries are ordered by their latent
    nearest-neighbour components when `latq` (int8 [nq][64]) is given, else by
    their rows' first key and MinHash.  part: "all", or "prepare" then "walk"
    with the same workspace `ws` (the walk takes no latents).  With `lse`
    (float32 [nq][Hq]) the walk also stores the log-sum-exp, as
    sparse_attn_fwd does."""
    nq = q.shape[0]
    for name, t in (("q", q), ("k", k), ("v", v)):
        _need(t, torch.bfloat16, name)
    _need(idx, torch.int32, "idx")
    _need(cnt, torch.int32, "cnt", (nq,))
    if out is None and part != "prepare":
        out = torch.empty((nq, ap.Hq, ap.D), dtype=torch.float32 if ap.out_f32 else torch.bfloat16,
                          device=q.device)
    wsb = workspace_bytes(OP_ATTN_GROUPED, None, sp, ap, nq)
    if ws is None or ws.numel() < wsb:
        if part != "all":
            raise LsaError(f"sparse_attn_grouped part {part!r} needs a workspace of {wsb} bytes")
        ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device=q.device)
    if latq is not None:
        _need(latq, torch.int8, "latq", (nq, 64))
    head = (_ptr(q), _ptr(k), _ptr(v), k.shape[0], _ptr(idx), _ptr(cnt), idx.shape[1], nq, qpos0)
    params = (ctypes.byref(sp), ctypes.byref(ap))
    lat = (_ptr(latq) if latq is not None else None,)
    if lse is not None:
        _need(lse, torch.float32, "lse", (nq, ap.Hq))
    lp = _ptr(lse) if lse is not None else None
    if part == "all":
        _check(lib().lsa_sparse_attn_grouped(*head, *lat, *params, _ptr(out), lp, _ptr(ws), ws.numel(),
                                             _stream(stream)), "lsa_sparse_attn_grouped")
    elif part == "prepare":
        _check(lib().lsa_attn_grouped_prepare(*head, *lat, *params, _ptr(ws), ws.numel(),
                                              _stream(stream)), "lsa_attn_grouped_prepare")
    elif part == "walk":
        _check(lib().lsa_attn_grouped_walk(*head, *params, _ptr(out), lp, _ptr(ws), ws.numel(),
                                           _stream(stream)), "lsa_attn_grouped_walk")
    else:
        raise ValueError(f"part {part!r}")
    return out


def sparse_attn_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, idx: torch.Tensor,
                    cnt: torch.Tensor, qpos0: int, sp: SelectParams, ap: AttnParams,
                    out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                    stream=None):
    """Training forward: sparse_attn_window plus the log-sum-exp float32 [nq][Hq]."""
    nq = q.shape[0]
    for name, t in (("q", q), ("k", k), ("v", v)):
        _need(t, torch.bfloat16, name)
    _need(idx, torch.int32, "idx")
    _need(cnt, torch.int32, "cnt", (nq,))
    if out is None:
        out = torch.empty((nq, ap.Hq, ap.D), dtype=torch.float32 if ap.out_f32 else torch.bfloat16,
                          device=q.device)
    if lse is None:
        lse = torch.empty((nq, ap.Hq), dtype=torch.float32, device=q.device)
    _need(lse, torch.float32, "lse", (nq, ap.Hq))
    _check(lib().lsa_sparse_attn_fwd(_ptr(q), _ptr(k), _ptr(v), k.shape[0], _ptr(idx), _ptr(cnt),
                                     idx.shape[1], nq, qpos0, ctypes.byref(sp), ctypes.byref(ap),
                                     _ptr(out), _ptr(lse), _stream(stream)), "lsa_sparse_attn_fwd")
    return out, lse


def sparse_attn_bwd(index: "LsaIndex", q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                    idx: torch.Tensor, cnt: torch.Tensor, qpos0: int, sp: SelectParams,
                    ap: AttnParams, out: torch.Tensor, lse: torch.Tensor, dout: torch.Tensor,
                    dq: Optional[torch.Tensor] = None, dk: Optional[torch.Tensor] = None,
                    dv: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None,
                    stream=None, latq: Optional[torch.Tensor] = None):
    """Gradients (float32) of the sparse attention for queries at positions
    qpos0.. over rows that `index` selected with `sp`; returns (dq, dk, dv).
    With `latq` (int8 [nq][64]) dQ's grouped walk orders the queries by their
    latent neighbours, as sparse_attn_grouped does."""
    nq = q.shape[0]
    for name, t in (("q", q), ("k", k), ("v", v), ("dout", dout)):
        _need(t, torch.bfloat16, name)
    _need(idx, torch.int32, "idx")
    _need(cnt, torch.int32, "cnt", (nq,))
    _need(out, torch.float32 if ap.out_f32 else torch.bfloat16, "out", (nq, ap.Hq, ap.D))
    _need(lse, torch.float32, "lse", (nq, ap.Hq))
    dev = q.device
    if dq is None:
        dq = torch.empty((nq, ap.Hq, ap.D), dtype=torch.float32, device=dev)
    if dk is None:
        dk = torch.empty((k.shape[0], ap.Hkv, ap.D), dtype=torch.float32, device=dev)
    if dv is None:
        dv = torch.empty((k.shape[0], ap.Hkv, ap.D), dtype=torch.float32, device=dev)
    if ws is None:
        ws = torch.empty(max(workspace_bytes(OP_ATTN_BWD, index.params, sp, ap, nq), 256),
                         dtype=torch.uint8, device=dev)
    if latq is not None:
        _need(latq, torch.int8, "latq", (nq, 64))
    _check(lib().lsa_sparse_attn_bwd(index.handle, _ptr(q), _ptr(k), _ptr(v), k.shape[0], _ptr(idx),
                                     _ptr(cnt), idx.shape[1], nq, qpos0,
                                     _ptr(latq) if latq is not None else None, ctypes.byref(sp),
                                     ctypes.byref(ap), _ptr(out), _ptr(lse), _ptr(dout), _ptr(dq),
                                     _ptr(dk), _ptr(dv), _ptr(ws), ws.numel(), _stream(stream)),
           "lsa_sparse_attn_bwd")
    return dq, dk, dv


def dense_select(latk: torch.Tensor, latq: torch.Tensor, qpos: torch.Tensor, sp: SelectParams,
                 ws: Optional[torch.Tensor] = None, use_workspace: bool = True, stream=None):
    """The quadratic comparator.  With a workspace (allocated here unless given)
    batches of 64 or more queries take the single thresholded scan; without
    one (use_workspace=False) every query takes the exact kernel."""
    nq = latq.shape[0]
    _need(latk, torch.int8, "latk")
    _need(latq, torch.int8, "latq", (nq, 64))
    _need(qpos, torch.int32, "qpos", (nq,))
    idx = torch.empty((nq, sp.max_sel), dtype=torch.int32, device=latq.device)
    cnt = torch.empty((nq,), dtype=torch.int32, device=latq.device)
    if use_workspace and ws is None:
        ws = torch.empty(max(workspace_bytes(OP_DENSE, None, sp, None, nq), 256), dtype=torch.uint8,
                         device=latq.device)
    if not use_workspace:
        ws = None
    _check(lib().lsa_dense_select(_ptr(latk), latk.shape[0], _ptr(latq), _ptr(qpos), nq,
                                  ctypes.byref(sp), _ptr(idx), _ptr(cnt), _ptr(ws),
                                  ws.numel() if ws is not None else 0, _stream(stream)),
           "lsa_dense_select")
    return idx, cnt


def decode_step(indexes: Sequence[LsaIndex], latk_new: torch.Tensor, latq: torch.Tensor,
                q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, seq_stride_rows: int,
                sp: SelectParams, ap: AttnParams, out: Optional[torch.Tensor] = None,
                ws: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    n = len(indexes)
    _need(latk_new, torch.int8, "latk_new", (n, 64))
    _need(latq, torch.int8, "latq", (n, 64))
    for name, t in (("q", q), ("k", k), ("v", v)):
        _need(t, torch.bfloat16, name)
    if out is None:
        out = torch.empty((n, ap.Hq, ap.D), dtype=torch.float32 if ap.out_f32 else torch.bfloat16,
                          device=q.device)
    wsb = workspace_bytes(OP_DECODE, indexes[0].params, sp, ap, n)
    if ws is None or ws.numel() < wsb:
        ws = torch.empty(max(wsb, 256), dtype=torch.uint8, device=q.device)
    hs = (c_vp * n)(*[ctypes.cast(ix._desc, c_vp).value for ix in indexes])
    _check(lib().lsa_decode_step(hs, n, _ptr(latk_new), _ptr(latq), _ptr(q), _ptr(k), _ptr(v),
                                 seq_stride_rows, ctypes.byref(sp), ctypes.byref(ap), _ptr(out),
                                 _ptr(ws), ws.numel(), _stream(stream)), "lsa_decode_step")
    return out


def decode_step_noalloc(indexes: Sequence[LsaIndex], latk_new: torch.Tensor, latq: torch.Tensor,
                        q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, seq_stride_rows: int,
                        sp: SelectParams, ap: AttnParams, out: torch.Tensor, stream=None) -> torch.Tensor:
    """lsa_decode_step_noalloc: decode_step with the library's own device
    workspace; the caller passes the output buffer."""
    n = len(indexes)
    _need(latk_new, torch.int8, "latk_new", (n, 64))
    _need(latq, torch.int8, "latq", (n, 64))
    for name, t in (("q", q), ("k", k), ("v", v)):
        _need(t, torch.bfloat16, name)
    _need(out, torch.float32 if ap.out_f32 else torch.bfloat16, "out", (n, ap.Hq, ap.D))
    hs = (c_vp * n)(*[ctypes.cast(ix._desc, c_vp).value for ix in indexes])
    _check(lib().lsa_decode_step_noalloc(hs, n, _ptr(latk_new), _ptr(latq), _ptr(q), _ptr(k), _ptr(v),
                                         seq_stride_rows, ctypes.byref(sp), ctypes.byref(ap), _ptr(out),
                                         _stream(stream)), "lsa_decode_step_noalloc")
    return out


def decode_selection(ws: torch.Tensor, nseq: int, sp: SelectParams):
    """Views of the last decode step's selection at the head of its workspace."""
    ms = sp.max_sel
    a_idx = (nseq * ms * 4 + 255) // 256 * 256
    idx = ws[: nseq * ms * 4].view(torch.int32).view(nseq, ms)
    cnt = ws[a_idx: a_idx + nseq * 4].view(torch.int32)
    return idx, cnt
