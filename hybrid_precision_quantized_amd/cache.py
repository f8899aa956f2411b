"""Device buffers of one layer's hybrid KV cache and their C descriptor.

Torch allocates the memory; every byte of the cache is written by the
library's kernels (hq_quantize_kv, hq_vl_bitmap, hq_gather_rows).
Layouts are those of hq_hybrid_kv in include/hq.h.
"""
from __future__ import annotations

import torch

from . import (HQ_BF16, HQ_F16, HQ_F32, HQ_LAYOUT_ROWS, HQ_LAYOUT_TILE16, HybridKV,
               hq_gather_rows, hq_quantize_kv, hq_vl_bitmap)

_HP = {torch.float32: HQ_F32, torch.bfloat16: HQ_BF16, torch.float16: HQ_F16}


def round_up(x: int, m: int) -> int:
    return (x + m - 1) // m * m


class HybridCache:
    def __init__(self, B: int, Hkv: int, D: int, T: int, W: int, k: int,
                 hp_dtype: torch.dtype, t_cap: int | None = None, device="cuda"):
        if D % 32:
            raise ValueError("D must be a multiple of 32")
        self.B, self.Hkv, self.D, self.T, self.W, self.k = B, Hkv, D, T, W, k
        self.group = 32
        self.hp_dtype = hp_dtype
        self.t_cap = round_up(max(T - W, 1), 32) if t_cap is None else t_cap
        dev = torch.device(device)
        n = B * Hkv
        self.k_codes = torch.zeros((B, Hkv, self.t_cap, D // 2), dtype=torch.uint8, device=dev)
        self.v_codes = torch.zeros((B, Hkv, self.t_cap // 16, D // 2, 16), dtype=torch.uint8, device=dev)
        self.k_sz = torch.zeros((B, Hkv, self.t_cap, D // 32, 2), dtype=torch.int16, device=dev)
        self.v_sz = torch.zeros((B, Hkv, self.t_cap, D // 32, 2), dtype=torch.int16, device=dev)
        self.vl_bits = torch.zeros((B, Hkv, self.t_cap // 32), dtype=torch.int32, device=dev)
        self.vl_idx = torch.zeros((B, Hkv, max(k, 1)), dtype=torch.int32, device=dev)
        self.vl_k = torch.zeros((B, Hkv, max(k, 1), D), dtype=hp_dtype, device=dev)
        self.vl_v = torch.zeros_like(self.vl_k)
        self.win_k = torch.zeros((B, Hkv, max(W, 1), D), dtype=hp_dtype, device=dev)
        self.win_v = torch.zeros_like(self.win_k)
        self.win_offset = 0
        self.flags = 0
        self._n = n

    # ------------------------------------------------------------ building
    def quantize(self, K: torch.Tensor, V: torch.Tensor, stream=None):
        """INT4 planes for positions [0, T - W) of K, V [B][Hkv][T_src][D]."""
        nq = self.T - self.W
        Ts = K.shape[2]
        hq_quantize_kv(K, self._n, nq, self.D, Ts * self.D, self.D, self.k_codes, self.k_sz,
                       HQ_LAYOUT_ROWS, self.t_cap, 0, stream=stream)
        hq_quantize_kv(V, self._n, nq, self.D, Ts * self.D, self.D, self.v_codes, self.v_sz,
                       HQ_LAYOUT_TILE16, self.t_cap, 0, stream=stream)

    def set_vl(self, K: torch.Tensor, V: torch.Tensor, vl_idx: torch.Tensor, stream=None):
        """Install a VL set (int32 [B][Hkv][k], ascending): bitmap and 16-bit rows."""
        if self.k == 0:
            self.vl_bits.zero_()
            return
        self.vl_idx.copy_(vl_idx.to(torch.int32))
        Ts = K.shape[2]
        hq_vl_bitmap(self.vl_idx, self._n, self.k, self.t_cap, self.vl_bits, stream=stream)
        hq_gather_rows(K, self._n, Ts, self.D, self.vl_idx, self.k, self.vl_k, stream=stream)
        hq_gather_rows(V, self._n, Ts, self.D, self.vl_idx, self.k, self.vl_v, stream=stream)

    def set_window(self, K: torch.Tensor, V: torch.Tensor, stream=None):
        """Window rows [T - W, T) of K, V (copied by the gather kernel)."""
        if self.W == 0:
            return
        Ts = K.shape[2]
        idx = torch.arange(self.T - self.W, self.T, dtype=torch.int32).repeat(self._n, 1)
        idx = idx.to(K.device)
        hq_gather_rows(K, self._n, Ts, self.D, idx, self.W, self.win_k, stream=stream)
        hq_gather_rows(V, self._n, Ts, self.D, idx, self.W, self.win_v, stream=stream)
        self.win_offset = 0

    def build(self, K, V, vl_idx, stream=None):
        self.quantize(K, V, stream)
        self.set_vl(K, V, vl_idx, stream)
        self.set_window(K, V, stream)
        return self

    # ------------------------------------------------------------ descriptor
    def descriptor(self) -> HybridKV:
        d = HybridKV()
        d.B, d.Hkv, d.D, d.group = self.B, self.Hkv, self.D, self.group
        d.T, d.W, d.k, d.t_cap = self.T, self.W, self.k, self.t_cap
        d.k_codes, d.v_codes = self.k_codes.data_ptr(), self.v_codes.data_ptr()
        d.k_sz, d.v_sz = self.k_sz.data_ptr(), self.v_sz.data_ptr()
        d.vl_bits = self.vl_bits.data_ptr()
        d.vl_k, d.vl_v = self.vl_k.data_ptr(), self.vl_v.data_ptr()
        d.win_k, d.win_v = self.win_k.data_ptr(), self.win_v.data_ptr()
        d.win_offset = self.win_offset
        d.hp_dtype = _HP[self.hp_dtype]
        d.flags = self.flags
        return d

    def nbytes_algorithmic(self) -> int:
        """Bytes one decode step must read from this cache: INT4 codes and
        scale/zero of the non-VL quantized positions, the 16-bit VL and window
        rows, and the VL index list."""
        nq_eff = self.T - self.W - self.k
        per_tok = self.D + (self.D // 32) * 2 * 2 * 2      # K+V codes, K+V {s, z}
        hp = torch.tensor([], dtype=self.hp_dtype).element_size()
        n = self.B * self.Hkv
        return n * (nq_eff * per_tok + (self.k + self.W) * 2 * self.D * hp + self.k * 4)
