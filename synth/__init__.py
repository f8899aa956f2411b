"""Seeded synthetic inputs for the HyQuant decode path.

This module only draws numbers: it holds none of the method's arithmetic
(no quantization, no attention, no detection). Both the CPU oracle and the
HIP path take their inputs from here, so the two sides see identical data.

Every tensor slice is drawn from its own NumPy PCG64 stream keyed by
(workload seed, tensor id, batch, head), so any (b, h) slice can be
regenerated alone, e.g. to check one sampled output of a large workload.

Recipe (the stand-ins for the models and datasets the HyQuant pages evaluate
on; shapes follow Llama-3.1-8B, Qwen3-8B and GLM-4-9B attention layers):

* Values are drawn in float64 and rounded to the input dtype (float32 round to
  nearest even, then bfloat16 round to nearest even where the dtype is bf16).
* "grid" tensors (K and Q of the bf16 workloads) are rounded to multiples of
  2**-4 before the dtype rounding. Products of two such values are multiples
  of 2**-8, so the detector's column scores are exact in fp32/fp64.
* u_h is a unit vector per (batch, KV head). Planted vertical-line positions
  are token 0 plus round(frac * T) - 1 distinct uniform draws from
  [1, T - W), shared by all heads of a sequence. Planted keys get beta * u_h,
  every query of the group gets alpha * u_h.
* K has ``n_outlier`` channels per KV head scaled by ``outlier_scale``.
"""
from __future__ import annotations

import dataclasses
import math
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

# tensor ids for the per-slice streams
_T_Q, _T_K, _T_V, _T_QACC, _T_PLANT, _T_U, _T_OUTL, _T_QPRE = range(8)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    B: int
    Hq: int
    Hkv: int
    D: int
    T: int
    W: int
    k: int
    dtype: str            # "f32", "bf16" or "f16"
    group: int = 32
    R: int = 64           # detector accumulation depth (decode steps)
    alpha: float = 7.0    # query component along u
    beta: float = 7.0     # planted key component along u
    plant_frac: float = 0.02
    n_plant: int = -1     # overrides plant_frac when >= 0
    n_outlier: int = 4
    outlier_scale: float = 10.0
    grid: bool = True     # round K and Q to the 2**-4 grid

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def n_quant(self) -> int:
        """Positions covered by the INT4 planes: [0, T - W)."""
        return self.T - self.W

    def planted_count(self) -> int:
        if self.n_plant >= 0:
            return self.n_plant
        return int(round(self.plant_frac * self.T))

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


def _vl_budget(T: int) -> int:
    return int(math.floor(0.05 * T))


# The five workloads. 1: tiny fp32 decode; 2: Llama-3.1-8B-shaped decode at
# 32K; 3: Qwen3-8B-style batched decode at 128K; 4: GLM-4-9B-shaped detector;
# 5: causal prefill at 32K.
WORKLOADS = {
    "tiny": Workload("tiny", 1001, B=1, Hq=4, Hkv=1, D=64, T=512, W=32, k=8,
                     dtype="f32", alpha=3.0, beta=3.0, n_plant=4, n_outlier=0,
                     grid=False, R=1),
    "llama32k": Workload("llama32k", 1002, B=1, Hq=32, Hkv=8, D=128, T=32768,
                         W=128, k=_vl_budget(32768), dtype="bf16"),
    "qwen128k": Workload("qwen128k", 1003, B=16, Hq=32, Hkv=8, D=128,
                         T=131072, W=128, k=_vl_budget(131072), dtype="bf16"),
    "glm32k": Workload("glm32k", 1004, B=1, Hq=32, Hkv=2, D=128, T=32768,
                       W=128, k=_vl_budget(32768), dtype="bf16"),
    "prefill32k": Workload("prefill32k", 1005, B=1, Hq=32, Hkv=8, D=128,
                           T=32768, W=128, k=_vl_budget(32768), dtype="bf16"),
}


def _gen(seed: int, *key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(
        np.random.SeedSequence(seed, spawn_key=tuple(int(x) for x in key))))


# ---------------------------------------------------------------- rounding
def to_f32(x: np.ndarray) -> np.ndarray:
    return np.asarray(x, dtype=np.float64).astype(np.float32)


def f32_to_bf16_bits(x32: np.ndarray) -> np.ndarray:
    """bfloat16 bits of float32 values, round to nearest even (finite input)."""
    u = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def round_dtype(x: np.ndarray, dtype: str, grid: bool = False) -> np.ndarray:
    """Round float64 draws to the workload dtype. Returns float32 values that
    are exactly representable in ``dtype``."""
    if grid:
        x = np.rint(np.asarray(x, dtype=np.float64) * 16.0) / 16.0
    x32 = to_f32(x)
    if dtype == "f32":
        return x32
    if dtype == "bf16":
        return bf16_bits_to_f32(f32_to_bf16_bits(x32))
    if dtype == "f16":
        return x32.astype(np.float16).astype(np.float32)
    raise ValueError(dtype)


def to_device_bits(x32: np.ndarray, dtype: str) -> np.ndarray:
    """Raw storage of already-rounded values: uint16 bits for bf16, float32 for f32."""
    if dtype == "bf16":
        return f32_to_bf16_bits(x32)
    return np.ascontiguousarray(x32, dtype=np.float32)


# ---------------------------------------------------------------- pieces
def unit_vector(w: Workload, b: int, h: int) -> np.ndarray:
    v = _gen(w.seed, _T_U, b, h).standard_normal(w.D)
    return v / np.linalg.norm(v)


def planted_positions(w: Workload, b: int) -> np.ndarray:
    """Token 0 plus distinct uniform draws from [1, T - W), ascending."""
    n = w.planted_count()
    hi = w.T - w.W
    g = _gen(w.seed, _T_PLANT, b)
    extra = g.choice(np.arange(1, hi), size=max(0, min(n - 1, hi - 1)), replace=False)
    return np.sort(np.concatenate([[0], extra]).astype(np.int64))


def outlier_channels(w: Workload, b: int, h: int) -> np.ndarray:
    if w.n_outlier == 0:
        return np.zeros(0, dtype=np.int64)
    g = _gen(w.seed, _T_OUTL, b, h)
    return np.sort(g.choice(w.D, size=w.n_outlier, replace=False))


def keys(w: Workload, b: int, h: int, n: int | None = None) -> np.ndarray:
    """K for one (b, KV head): float32 values exact in the dtype, [T][D]."""
    T = w.T if n is None else n
    x = _gen(w.seed, _T_K, b, h).standard_normal((w.T, w.D))[:T]
    oc = outlier_channels(w, b, h)
    if len(oc):
        x[:, oc] *= w.outlier_scale
    pl = planted_positions(w, b)
    pl = pl[pl < T]
    x[pl] += w.beta * unit_vector(w, b, h)
    return round_dtype(x, w.dtype, grid=w.grid)


def values(w: Workload, b: int, h: int, n: int | None = None) -> np.ndarray:
    """V for one (b, KV head): N(0, 1) rounded to the dtype, [T][D]."""
    T = w.T if n is None else n
    x = _gen(w.seed, _T_V, b, h).standard_normal((w.T, w.D))[:T]
    return round_dtype(x, w.dtype, grid=False)


def query(w: Workload, b: int, i: int) -> np.ndarray:
    """Decode query of query head i: N(0, 1) + alpha * u_h, [D]."""
    h = i // w.G
    x = _gen(w.seed, _T_Q, b, i).standard_normal(w.D) + w.alpha * unit_vector(w, b, h)
    return round_dtype(x, w.dtype, grid=w.grid)


def query_history(w: Workload, b: int, i: int, R: int | None = None) -> np.ndarray:
    """R consecutive decode queries of query head i, [R][D] (detector input)."""
    R = w.R if R is None else R
    h = i // w.G
    x = _gen(w.seed, _T_QACC, b, i).standard_normal((R, w.D)) + w.alpha * unit_vector(w, b, h)
    return round_dtype(x, w.dtype, grid=w.grid)


def prefill_queries(w: Workload, b: int, i: int) -> np.ndarray:
    """Prompt queries of query head i for the causal prefill workload, [T][D]."""
    h = i // w.G
    x = _gen(w.seed, _T_QPRE, b, i).standard_normal((w.T, w.D)) + w.alpha * unit_vector(w, b, h)
    return round_dtype(x, w.dtype, grid=w.grid)


# ---------------------------------------------------------------- batched
def _parallel(fn, items, threads: int | None = None):
    threads = threads or min(16, os.cpu_count() or 1)
    if threads <= 1 or len(items) <= 1:
        return [fn(*it) for it in items]
    with ThreadPoolExecutor(threads) as ex:
        return list(ex.map(lambda it: fn(*it), items))


def all_keys(w: Workload, n: int | None = None, threads: int | None = None) -> np.ndarray:
    """K for every (b, KV head): float32 [B][Hkv][n][D]."""
    T = w.T if n is None else n
    out = np.empty((w.B, w.Hkv, T, w.D), dtype=np.float32)

    def fill(b, h):
        out[b, h] = keys(w, b, h, T)
    _parallel(fill, [(b, h) for b in range(w.B) for h in range(w.Hkv)], threads)
    return out


def all_values(w: Workload, n: int | None = None, threads: int | None = None) -> np.ndarray:
    T = w.T if n is None else n
    out = np.empty((w.B, w.Hkv, T, w.D), dtype=np.float32)

    def fill(b, h):
        out[b, h] = values(w, b, h, T)
    _parallel(fill, [(b, h) for b in range(w.B) for h in range(w.Hkv)], threads)
    return out


def all_queries(w: Workload) -> np.ndarray:
    return np.stack([np.stack([query(w, b, i) for i in range(w.Hq)]) for b in range(w.B)])


def all_query_histories(w: Workload, R: int | None = None) -> np.ndarray:
    """[B][Hq][R][D]"""
    return np.stack([np.stack([query_history(w, b, i, R) for i in range(w.Hq)])
                     for b in range(w.B)])


def random_vl_index(w: Workload, b: int, h: int, k: int | None = None,
                    cand_end: int | None = None, seed_extra: int = 0) -> np.ndarray:
    """A valid VL index list that is not chosen by any detector: k distinct
    positions of [0, cand_end), ascending. For tests of the decode path alone."""
    k = w.k if k is None else k
    ce = w.T - w.W if cand_end is None else cand_end
    g = _gen(w.seed + 7919 * (seed_extra + 1), 99, b, h)
    return np.sort(g.choice(ce, size=k, replace=False)).astype(np.int32)
