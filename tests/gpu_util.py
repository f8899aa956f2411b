"""Shared helpers of the GPU parity tests (no test cases here)."""
from __future__ import annotations

import sys

import numpy as np
import torch

import synth

TORCH_DT = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(x32: np.ndarray, dtype: str, device="cuda") -> torch.Tensor:
    """Upload values exactly representable in `dtype`."""
    if dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32)).to(device)
    if dtype == "bf16":
        bits = synth.f32_to_bf16_bits(x32)
        return torch.from_numpy(bits.view(np.int16)).to(device).view(torch.bfloat16)
    if dtype == "f16":
        return torch.from_numpy(np.asarray(x32, dtype=np.float16)).to(device)
    raise ValueError(dtype)


def from_dev(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy()


def rows_codes(plane: torch.Tensor) -> np.ndarray:
    """HQ_LAYOUT_ROWS plane [..., rows, D/2] -> bytes per logical row."""
    return plane.cpu().numpy()


def tile16_codes(plane: torch.Tensor) -> np.ndarray:
    """HQ_LAYOUT_TILE16 plane [..., rows/16, D/2, 16] -> [..., rows, D/2] bytes,
    following the layout stated in include/hq.h."""
    a = plane.cpu().numpy()
    # byte slot 4a + b holds row 4a + (0, 2, 1, 3)[b]; that order is its own inverse
    order = np.array([0, 2, 1, 3, 4, 6, 5, 7, 8, 10, 9, 11, 12, 14, 13, 15])
    a = a[..., order]
    a = np.swapaxes(a, -1, -2)                     # [..., rows/16, 16, D/2]
    return a.reshape(a.shape[:-3] + (a.shape[-3] * 16, a.shape[-1]))


def tile16_slot(r: int) -> int:
    """Byte slot of row r % 16 inside its TILE16 tile (runs of 4 rows are
    stored in the order 0, 2, 1, 3)."""
    r %= 16
    return (r & ~3) | ((r & 1) << 1) | ((r >> 1) & 1)


def sz_bits(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy().view(np.uint16)


def upload_kv(w: synth.Workload, n: int | None = None):
    """K, V of every (b, KV head) on the device, streamed one sequence at a time."""
    T = w.T if n is None else n
    dt = TORCH_DT[w.dtype]
    K = torch.empty((w.B, w.Hkv, T, w.D), dtype=dt, device="cuda")
    V = torch.empty_like(K)
    for b in range(w.B):
        kb = np.stack(synth._parallel(lambda h: synth.keys(w, b, h, T), [(h,) for h in range(w.Hkv)]))
        vb = np.stack(synth._parallel(lambda h: synth.values(w, b, h, T), [(h,) for h in range(w.Hkv)]))
        K[b].copy_(to_dev(kb, w.dtype))
        V[b].copy_(to_dev(vb, w.dtype))
    return K, V


def rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    rms = float(np.sqrt(np.mean(np.square(ref))))
    return float(np.max(np.abs(got - ref))) / rms


# ------------------------------------------------ matrix-core detector bounds
# The MFMA detector groups a unit's rows rho = i * R + r (query head i of the
# group, ring slot r) by rho mod 16 and accumulates each group in fp32 (the
# library header states this arithmetic). These helpers restate its
# consequences on the host, from the inputs alone.
N_RESIDUES = 16


def residue_abs_sums(q_acc: np.ndarray, K: np.ndarray, b: int, h: int, cand_end: int) -> np.ndarray:
    """[cand_end][16]: for column j and residue r, the sum over the rows
    rho = r mod 16 of the unit and all channels of |q[rho][d] k[j][d]|."""
    B, Hq, R, D = q_acc.shape
    G = Hq // K.shape[1]
    rows = np.abs(q_acc[b, h * G:(h + 1) * G].reshape(G * R, D).astype(np.float64))
    res = np.zeros((N_RESIDUES, D))
    for r in range(N_RESIDUES):
        res[r] = rows[r::N_RESIDUES].sum(axis=0)
    return np.abs(K[b, h, :cand_end].astype(np.float64)) @ res.T


def matmul_exact_precondition(q_acc: np.ndarray, K: np.ndarray, cand_end: int) -> float:
    """Largest residue absolute sum over all units and columns. Below 2^16
    (with grid inputs) every fp32 partial of the MFMA form is exact."""
    worst = 0.0
    for b in range(q_acc.shape[0]):
        for h in range(K.shape[1]):
            if cand_end:
                worst = max(worst, float(residue_abs_sums(q_acc, K, b, h, cand_end).max()))
    return worst


def matmul_score_bound_units(q_acc: np.ndarray, K: np.ndarray, cand_end: int) -> np.ndarray:
    """[B][Hkv][cand_end] bound, in score units of 2^-16, on |GPU - exact| for
    the MFMA form on inputs off the grid: each residue's fp32 chain of
    n = (G R / 16) D products (each exact in fp32) is off by at most
    2 n 2^-24 times its absolute sum (a factor 2 over round-to-nearest, so
    that truncating adds are covered too); the fp64 sum of the 16 residues
    adds at most 16 2^-53 of the total; the final rounding to units half a
    unit. One unit of slack."""
    B, Hq, R, D = q_acc.shape
    Hkv = K.shape[1]
    G = Hq // Hkv
    n = (G * R + N_RESIDUES - 1) // N_RESIDUES * D
    out = np.zeros((B, Hkv, cand_end))
    for b in range(B):
        for h in range(Hkv):
            s = residue_abs_sums(q_acc, K, b, h, cand_end)            # [n][16]
            tot = s.sum(axis=1)
            err = 2.0 * n * 2.0 ** -24 * tot + 16 * 2.0 ** -53 * tot
            out[b, h] = np.ceil(err * 65536.0) + 1.5
    return out
