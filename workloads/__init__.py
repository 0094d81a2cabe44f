"""Seeded synthetic inputs for the table-batched embedding (TBE) workloads.

This module only draws inputs. It holds none of the method's arithmetic: no
pooling, no sort, no run-length encoding, no optimizer. Both the HIP path's
tests/benchmark and the CPU oracle take their inputs from here, so the same
seed gives the same batch on either side.

Workload shapes follow the FBTriton TBE tutorial (page 1, "Notation": T tables,
E rows, D columns, L bag size, B bags per table; the large-scenario statistics
of about 83M lookups, 3M unique rows and a hottest row near 125K lookups at
T*B = 4.2M, B = 128K) and the TorchEasyRec article (page 2, section 2: the
three demo tables of 1,141,730 / 461,498 / 846,812 rows).

Layout (the boundary's layout, table-major jagged like a KeyedJaggedTensor's
values/lengths):
  indices  int32 [N]        row index inside its own table
  offsets  int32 [T*B + 1]  bag i = t*B + b covers indices[offsets[i]:offsets[i+1]]
  psw      float32 [N] or None (per-sample weights)
  grad     float32 [B, T*D] upstream gradient of the pooled output; table t
           owns columns t*D .. t*D+D-1
  W        [sum(E), D] weights, tables stacked in order; dtype f32/f16/bf16
  m        float32 [sum(E)] row-wise Adagrad state

Weights and optimizer state are drawn on the device that holds them (the
table of the largest workload is 16 GiB), with torch's seeded generator.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

__all__ = ["Config", "WORKLOADS", "TINY", "DEMO3", "MEDIUM", "LARGE", "SMALL_TABLE", "Batch", "make_batch", "init_weights", "init_state",
           "torch_dtype", "table_offsets"]


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    T: int
    B: int
    D: int
    rows: tuple            # E_t per table
    dtype: str             # "f32" | "f16" | "bf16"
    bag: tuple             # ("fixed", L) | ("uniform", lo, hi) per table | ("poisson", mean)
    index: tuple           # ("uniform",) | ("zipf", alpha) | ("zipf_mandelbrot", alpha, q)
    weighted: bool
    preprocess_in_forward: bool
    seed: int
    lr: float = 0.01
    eps: float = 1e-8
    bag_per_table: Optional[tuple] = None   # overrides `bag` per table when set

    @property
    def sum_rows(self) -> int:
        return int(sum(self.rows))


# The five workloads, named by shape. Weight init U(-0.01, 0.01), state 0,
# lr 0.01 and eps 1e-8 throughout; the large skewed workload draws rows from a
# Zipf-Mandelbrot law whose draw reproduces page 1's statistics.
WORKLOADS = {
    "tiny_t2_e1k_d16_f32": Config("tiny_t2_e1k_d16_f32", T=2, B=64, D=16, rows=(1000, 1000), dtype="f32",
              bag=("fixed", 4), index=("uniform",), weighted=False,
              preprocess_in_forward=False, seed=1),
    "demo3_d16_f32_b4k": Config("demo3_d16_f32_b4k", T=3, B=4096, D=16, rows=(1141730, 461498, 846812),
              dtype="f32", bag=("fixed", 1), index=("zipf", 1.1), weighted=False,
              preprocess_in_forward=False, seed=2,
              bag_per_table=(("fixed", 1), ("uniform", 1, 20), ("uniform", 1, 20))),
    "t16_e1m_d128_f16_b16k": Config("t16_e1m_d128_f16_b16k", T=16, B=16384, D=128, rows=(1_000_000,) * 16,
              dtype="f16", bag=("poisson", 20.0), index=("zipf", 1.05),
              weighted=False, preprocess_in_forward=False, seed=3),
    "t32_e2m_d128_bf16_b128k": Config("t32_e2m_d128_bf16_b128k", T=32, B=131072, D=128, rows=(2_000_000,) * 32,
              dtype="bf16", bag=("poisson", 20.0),
              index=("zipf_mandelbrot", 1.404, 7.32), weighted=True,
              preprocess_in_forward=True, seed=4),
    "small_t64_e64_d128_f16_b32k": Config("small_t64_e64_d128_f16_b32k", T=64, B=32768, D=128, rows=(64,) * 64,
              dtype="f16", bag=("fixed", 64), index=("uniform",), weighted=False,
              preprocess_in_forward=False, seed=5),
}

# Short handles: the 2-table f32 toy, page 2's three demo tables, the
# 16-table f16 workload, the large skewed bf16 workload (page 1's statistics)
# and the small-table histogram workload.
TINY = WORKLOADS["tiny_t2_e1k_d16_f32"]
DEMO3 = WORKLOADS["demo3_d16_f32_b4k"]
MEDIUM = WORKLOADS["t16_e1m_d128_f16_b16k"]
LARGE = WORKLOADS["t32_e2m_d128_bf16_b128k"]
SMALL_TABLE = WORKLOADS["small_t64_e64_d128_f16_b32k"]


@dataclasses.dataclass
class Batch:
    cfg: Config
    indices: np.ndarray
    offsets: np.ndarray
    psw: Optional[np.ndarray]
    grad: Optional[np.ndarray]

    @property
    def N(self) -> int:
        return int(self.offsets[-1])


def table_offsets(rows) -> np.ndarray:
    """First stacked row of each table (int64 [T]); plain bookkeeping of the
    stacked weight layout, shared by generator callers."""
    r = np.asarray(rows, dtype=np.int64)
    out = np.zeros(len(r), dtype=np.int64)
    if len(r) > 1:
        out[1:] = np.cumsum(r)[:-1]
    return out


def _bag_lengths(spec, B, rng) -> np.ndarray:
    kind = spec[0]
    if kind == "fixed":
        return np.full(B, int(spec[1]), dtype=np.int64)
    if kind == "uniform":
        return rng.integers(int(spec[1]), int(spec[2]) + 1, size=B, dtype=np.int64)
    if kind == "poisson":
        return rng.poisson(float(spec[1]), size=B).astype(np.int64)
    raise ValueError(f"unknown bag-length spec {spec!r}")


def _rank_cdf(spec, E) -> Optional[np.ndarray]:
    kind = spec[0]
    if kind == "uniform":
        return None
    k = np.arange(1, E + 1, dtype=np.float64)
    if kind == "zipf":
        p = k ** (-float(spec[1]))
    elif kind == "zipf_mandelbrot":
        p = (k + float(spec[2])) ** (-float(spec[1]))
    else:
        raise ValueError(f"unknown index spec {spec!r}")
    cdf = np.cumsum(p)
    cdf /= cdf[-1]
    return cdf


def _draw_rows(spec, E, n, rng) -> np.ndarray:
    """Rows of one table: uniform, or a truncated Zipf-family rank drawn by
    inverse CDF on [1, E] and mapped to a row through a random permutation."""
    if spec[0] == "uniform":
        return rng.integers(0, E, size=n, dtype=np.int64)
    perm = rng.permutation(E)
    cdf = _rank_cdf(spec, E)
    u = rng.random(n)
    rank = np.searchsorted(cdf, u, side="right")        # 0-based rank
    np.minimum(rank, E - 1, out=rank)                    # guards u == cdf[-1]
    return perm[rank]


def make_batch(cfg: Config, *, with_grad: bool = True, B: Optional[int] = None,
               seed: Optional[int] = None) -> Batch:
    """Draw one batch. Draw order: per table the bag lengths; then per table the
    permutation and row draws; then per-sample weights; then the upstream
    gradient. `B` shrinks the batch for quick tests (same distributions)."""
    B = cfg.B if B is None else int(B)
    rng = np.random.default_rng(cfg.seed if seed is None else seed)
    T = cfg.T
    specs = cfg.bag_per_table or (cfg.bag,) * T
    lengths = np.empty(T * B, dtype=np.int64)
    for t in range(T):
        lengths[t * B:(t + 1) * B] = _bag_lengths(specs[t], B, rng)
    offsets = np.zeros(T * B + 1, dtype=np.int64)
    np.cumsum(lengths, out=offsets[1:])
    N = int(offsets[-1])
    if N >= 2 ** 31:
        raise ValueError("batch exceeds int32 offsets")
    indices = np.empty(N, dtype=np.int32)
    for t in range(T):
        a, b = int(offsets[t * B]), int(offsets[(t + 1) * B])
        indices[a:b] = _draw_rows(cfg.index, int(cfg.rows[t]), b - a, rng)
    psw = rng.random(N, dtype=np.float32) if cfg.weighted else None
    grad = None
    if with_grad:
        grad = rng.standard_normal((B, T * cfg.D), dtype=np.float32)
    return Batch(cfg=dataclasses.replace(cfg, B=B), indices=indices,
                 offsets=offsets.astype(np.int32), psw=psw, grad=grad)


# ---------------------------------------------------------------------------
# Weights and optimizer state: drawn on the target device with torch's seeded
# generator (uniform in float32, then rounded to nearest even into the weight
# type). Large tables (16 GiB at 64M rows) are filled in slices of rows so the
# float32 staging stays small. Callers that need the initial values of some
# rows on the host (the oracle) copy them from the tensor before any update.
# ---------------------------------------------------------------------------
_TORCH_DTYPES = {"f32": "float32", "f16": "float16", "bf16": "bfloat16"}


def torch_dtype(cfg: Config):
    import torch
    return getattr(torch, _TORCH_DTYPES[cfg.dtype])


def init_weights(cfg: Config, device, chunk_rows: int = 1 << 20):
    """W [sum(E), D] ~ U(-0.01, 0.01), deterministic for a device and seed."""
    import torch
    E = cfg.sum_rows
    gen = torch.Generator(device=device)
    gen.manual_seed(0x5EED0000 + cfg.seed)
    out = torch.empty((E, cfg.D), dtype=torch_dtype(cfg), device=device)
    for a in range(0, E, chunk_rows):
        b = min(E, a + chunk_rows)
        tmp = torch.empty((b - a, cfg.D), dtype=torch.float32, device=device)
        tmp.uniform_(-0.01, 0.01, generator=gen)
        out[a:b] = tmp
    return out


def init_state(cfg: Config, device, m0: str = "zeros"):
    """Row-wise Adagrad state [sum(E)]: zeros, or U(0, 1) when m0 == "uniform"."""
    import torch
    E = cfg.sum_rows
    if m0 == "zeros":
        return torch.zeros(E, dtype=torch.float32, device=device)
    gen = torch.Generator(device=device)
    gen.manual_seed(0xACC00000 + cfg.seed)
    return torch.empty(E, dtype=torch.float32, device=device).uniform_(0.0, 1.0, generator=gen)
