"""Seeded synthetic inputs for the Latent Sparse Attention hot path.

This module is shared by the CPU oracle (test infrastructure) and by the GPU
path's tests and benchmark.  It holds no arithmetic of the method itself: no
pooling, clustering, scoring, selection or attention.  It only draws numbers.

Everything is counter-based, so any row of any tensor can be regenerated on
its own, on the host or on a device, with bit-identical results:

* ``_splitmix`` is the SplitMix64 output function (Steele, Lea, Flood,
  "Fast splittable pseudorandom number generators", OOPSLA 2014), evaluated
  with wrapping int64 torch arithmetic and masked (logical) right shifts, so
  the CPU and the GPU produce the same bits.
* One 64-bit hash yields four 16-bit uniforms.
* Normal variates come from fixed 65536-entry inverse-CDF tables evaluated at
  the cell midpoints ``(u + 0.5) / 65536``: a bf16 table for Q/K/V, and
  integer tables (in units of 1/64) for the latent mixtures.  Table lookups
  are exact on every device, so no transcendental function is evaluated on
  the device.

Workloads (the pages' prefill workload is the last 32k chunk of a 10M-token
context on one GPU; the latent index uses 64-d representations, 4096
long-range + 512 recent + 4 sink keys per query):

* latent keys: a Gaussian mixture with ``ncomp`` components; component means
  uniform in [-40, 40] (quantised to 1/64), per-key component uniform,
  per-dimension noise N(0, sigma=3); value = clamp(round(mean + noise)) in
  [-127, 127] with halves rounded up.
* latent queries: a uniformly drawn component's mean + N(0, 6) noise (6 is
  read as the standard deviation), same rounding and clamp.
* Q, K, V: bf16 values of N(0, 1) (tails truncated at about 4.3 sigma by the
  table).
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np
import torch

_MASK64 = (1 << 64) - 1


def _s64(x: int) -> int:
    """Reinterpret an unsigned 64-bit constant as a signed int64."""
    x &= _MASK64
    return x - (1 << 64) if x >= (1 << 63) else x


_GOLDEN = _s64(0x9E3779B97F4A7C15)
_M1 = _s64(0xBF58476D1CE4E5B9)
_M2 = _s64(0x94D049BB133111EB)


def _lsr(z: torch.Tensor, s: int) -> torch.Tensor:
    return (z >> s) & ((1 << (64 - s)) - 1)


def _splitmix(z: torch.Tensor) -> torch.Tensor:
    """SplitMix64 output mix of (z + golden gamma); wrapping int64 ops."""
    z = z + _GOLDEN
    z = (z ^ _lsr(z, 30)) * _M1
    z = (z ^ _lsr(z, 27)) * _M2
    return z ^ _lsr(z, 31)


def _key_scalar(*parts: int) -> int:
    """Combine integers into a 64-bit stream key (host-side, exact)."""
    z = 0x2026
    for p in parts:
        t = torch.tensor([_s64(z ^ (p * 0x100000001B3))], dtype=torch.int64)
        z = int(_splitmix(t)[0]) & _MASK64
    return _s64(z)


def hash64(key: int, counters: torch.Tensor) -> torch.Tensor:
    """64-bit hash of (stream key, counter) for an int64 counter tensor."""
    return _splitmix(counters * _GOLDEN + key)


def uniform16(key: int, idx: torch.Tensor) -> torch.Tensor:
    """16-bit uniforms (int64 in [0, 65535]) for element indices ``idx``."""
    h = hash64(key, idx >> 2)
    # shifts are at most 48, so sign extension never reaches the low 16 bits
    return (h >> (16 * (idx & 3))) & 0xFFFF


# --------------------------------------------------------------------------
# inverse-CDF tables (host computed once, identical wherever they are used)
# --------------------------------------------------------------------------
_TABLES: dict = {}


def _ndtri_mid() -> np.ndarray:
    from scipy.special import ndtri
    u = (np.arange(65536, dtype=np.float64) + 0.5) / 65536.0
    return ndtri(u)


def normal_bf16_table() -> torch.Tensor:
    """int16 bit patterns of bf16(N(0,1) quantile at the 65536 cell midpoints)."""
    t = _TABLES.get("bf16")
    if t is None:
        f32 = _ndtri_mid().astype(np.float32)
        bits = f32.view(np.uint32).astype(np.uint64)
        r = (bits + 0x7FFF + ((bits >> 16) & 1)) >> 16          # round to nearest even
        t = torch.from_numpy(r.astype(np.uint16).view(np.int16).copy())
        _TABLES["bf16"] = t
    return t


def normal_int_table(sigma: float) -> torch.Tensor:
    """int64 table of round(64 * sigma * N(0,1) quantile) at the cell midpoints."""
    k = ("int", float(sigma))
    t = _TABLES.get(k)
    if t is None:
        t = torch.from_numpy(np.rint(64.0 * sigma * _ndtri_mid()).astype(np.int64))
        _TABLES[k] = t
    return t


def _table_on(t: torch.Tensor, device) -> torch.Tensor:
    if t.device == torch.device(device):
        return t
    key = (id(t), str(device))
    c = _TABLES.get(key)
    if c is None:
        c = t.to(device)
        _TABLES[key] = c
    return c


# --------------------------------------------------------------------------
# workload presets
# --------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic workload: data recipe, index, selection and attention shapes."""
    name: str
    cfg_id: int
    T: int                 # context length (keys) the chunk ends at
    ncomp: int             # mixture components of the latent keys
    pool: int = 4
    block: int = 4096      # pooled vectors per block
    buckets: int = 256     # clusters per block
    iters: int = 4         # k-means iterations
    tree_group: int = 0    # blocks per super group (0 = Flat)
    tree_super: int = 0    # super clusters per group
    tree_iters: int = 0
    tree_top: int = 0      # super clusters taken per query
    tree2_group: int = 0   # third level: groups per top group
    tree2_super: int = 0   # top nodes per top group
    tree2_iters: int = 0
    tree2_top: int = 0     # top nodes taken per query
    chunk: int = 32768     # queries = the last ``chunk`` positions
    budget: int = 4096
    window: int = 512
    sinks: int = 4
    Hq: int = 32
    Hkv: int = 8
    D: int = 128
    nseq: int = 1          # independent sequences (decode)
    steps: int = 0         # decode steps
    dim: int = 64
    key_sigma: float = 3.0
    query_sigma: float = 6.0

    @property
    def max_sel(self) -> int:
        return self.budget + self.window + self.sinks


M = 1 << 20
WORKLOADS = {
    "tiny_flat": Workload("tiny_flat", 1, T=16384, ncomp=256, block=1024, buckets=64,
                          iters=3, chunk=128, budget=1024, window=128, sinks=4,
                          Hq=4, Hkv=1, D=64),
    "flat_1m": Workload("flat_1m", 2, T=M, ncomp=4096),
    "flat_10m": Workload("flat_10m", 3, T=10 * M, ncomp=16384),
    "decode_1m": Workload("decode_1m", 4, T=M, ncomp=4096, chunk=0, nseq=8, steps=256),
    "tree_10m": Workload("tree_10m", 5, T=10 * M, ncomp=16384, tree_group=64,
                         tree_super=64, tree_iters=4, tree_top=32),
    # three levels: top nodes over the supers of each run of 5 groups
    "tree3_10m": Workload("tree3_10m", 5, T=10 * M, ncomp=16384, tree_group=64,
                          tree_super=64, tree_iters=4, tree_top=32, tree2_group=5,
                          tree2_super=32, tree2_iters=4, tree2_top=16),
    # one attention layer's training step at 128k context: every position is a query
    "train_128k": Workload("train_128k", 6, T=M // 8, ncomp=1024, chunk=M // 8),
}

# stream ids
S_MEANS, S_KCOMP, S_KNOISE, S_QCOMP, S_QNOISE, S_Q, S_K, S_V, S_DO = range(9)


class Synth:
    """Seeded generator for one workload (and one sequence of it)."""

    def __init__(self, wl: Workload, seq: int = 0, data_cfg: Optional[int] = None):
        self.wl = wl
        self.seq = seq
        # the Tree workload shares the Flat 10M data
        cfg = data_cfg if data_cfg is not None else (3 if wl.cfg_id == 5 else wl.cfg_id)
        self.cfg = cfg
        self._keys = {s: _key_scalar(2026, cfg, s, seq) for s in range(9)}
        self._means = {}

    def key(self, stream: int) -> int:
        return self._keys[stream]

    # ---- mixture means: int64 [ncomp][dim] in units of 1/64 ----
    def means64(self, device="cpu") -> torch.Tensor:
        m = self._means.get(str(device))
        if m is None:
            n = self.wl.ncomp * self.wl.dim
            idx = torch.arange(n, dtype=torch.int64, device=device)
            h = _lsr(hash64(self.key(S_MEANS), idx), 1)
            m = (h % (80 * 64 + 1) - 40 * 64).reshape(self.wl.ncomp, self.wl.dim)
            self._means[str(device)] = m
        return m

    def _latent(self, rows: torch.Tensor, s_comp: int, s_noise: int, sigma: float,
                device) -> torch.Tensor:
        wl = self.wl
        rows = rows.to(device=device, dtype=torch.int64)
        comp = _lsr(hash64(self.key(s_comp), rows), 1) % wl.ncomp
        e = rows[:, None] * wl.dim + torch.arange(wl.dim, device=device, dtype=torch.int64)
        u = uniform16(self.key(s_noise), e)
        noise = _table_on(normal_int_table(sigma), device)[u]
        v = self.means64(device)[comp] + noise
        v = torch.div(v + 32, 64, rounding_mode="floor").clamp_(-127, 127)
        return v.to(torch.int8)

    def latk_rows(self, rows: torch.Tensor, device="cpu") -> torch.Tensor:
        """int8 [len(rows)][dim] latent keys at the given token positions."""
        return self._latent(rows, S_KCOMP, S_KNOISE, self.wl.key_sigma, device)

    def latk(self, t0: int, t1: int, device="cpu", chunk: int = 1 << 20) -> torch.Tensor:
        out = torch.empty((t1 - t0, self.wl.dim), dtype=torch.int8, device=device)
        for a in range(t0, t1, chunk):
            b = min(t1, a + chunk)
            out[a - t0:b - t0] = self.latk_rows(
                torch.arange(a, b, dtype=torch.int64, device=device), device)
        return out

    def latq_rows(self, rows: torch.Tensor, device="cpu") -> torch.Tensor:
        """int8 [len(rows)][dim] latent queries at the given token positions."""
        return self._latent(rows, S_QCOMP, S_QNOISE, self.wl.query_sigma, device)

    def latq(self, t0: int, t1: int, device="cpu") -> torch.Tensor:
        return self.latq_rows(torch.arange(t0, t1, dtype=torch.int64), device)

    # ---- bf16 tensors laid out [token][heads][D] ----
    def _bf16_rows(self, stream: int, rows: torch.Tensor, H: int, D: int, device) -> torch.Tensor:
        rows = rows.to(device=device, dtype=torch.int64)
        e = rows[:, None] * (H * D) + torch.arange(H * D, device=device, dtype=torch.int64)
        u = uniform16(self.key(stream), e)
        bits = _table_on(normal_bf16_table(), device)[u]
        return bits.view(torch.bfloat16).reshape(len(rows), H, D)

    def q_rows(self, rows, device="cpu"):
        return self._bf16_rows(S_Q, rows, self.wl.Hq, self.wl.D, device)

    def k_rows(self, rows, device="cpu"):
        return self._bf16_rows(S_K, rows, self.wl.Hkv, self.wl.D, device)

    def v_rows(self, rows, device="cpu"):
        return self._bf16_rows(S_V, rows, self.wl.Hkv, self.wl.D, device)

    def do_rows(self, rows, device="cpu"):
        """Upstream gradient of the attention output (training), [len(rows)][Hq][D]."""
        return self._bf16_rows(S_DO, rows, self.wl.Hq, self.wl.D, device)

    def fill_rows(self, which: str, out: torch.Tensor, t0: int, chunk: int = 1 << 16) -> None:
        """Fill ``out`` ([n][H][D] bf16, any device) with rows t0.. of Q, K, V or dO."""
        stream = {"q": S_Q, "k": S_K, "v": S_V, "do": S_DO}[which]
        n, H, D = out.shape
        dev = out.device
        for a in range(0, n, chunk):
            b = min(n, a + chunk)
            out[a:b] = self._bf16_rows(stream, torch.arange(t0 + a, t0 + b, dtype=torch.int64),
                                       H, D, dev)
