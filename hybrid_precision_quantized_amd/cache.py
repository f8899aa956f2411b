"""Device buffers of one layer's hybrid KV cache and their C descriptor.

Torch allocates the memory; every byte of the cache is written by the
library's kernels (hq_quantize_kv, hq_vl_bitmap, hq_gather_rows).
Layouts are those of hq_hybrid_kv in include/hq.h.
"""
from __future__ import annotations

import torch

from . import (HQ_BF16, HQ_F16, HQ_F32, HQ_LAYOUT_ROWS, HQ_LAYOUT_TILE16, HybridKV, hq_decode_step,
               hq_detect_vlines_cache, hq_detect_workspace_size, hq_gather_rows, hq_quantize_kv,
               hq_vl_bitmap, hq_vl_redetect, hq_vl_redetect_workspace_size, hq_vl_update)

_HP = {torch.float32: HQ_F32, torch.bfloat16: HQ_BF16, torch.float16: HQ_F16}


def round_up(x: int, m: int) -> int:
    return (x + m - 1) // m * m


class HybridCache:
    def __init__(self, B: int, Hkv: int, D: int, T: int, W: int, k: int,
                 hp_dtype: torch.dtype, t_cap: int | None = None, device="cuda", win_cap: int = 0):
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
        # the window ring: W rows, or win_cap >= W rows when it also keeps the
        # rows that left the window since the last VL update
        self.win_cap = win_cap if win_cap else W
        if self.win_cap < W:
            raise ValueError("win_cap must be 0 or >= W")
        self.win_k = torch.zeros((B, Hkv, max(self.win_cap, 1), D), dtype=hp_dtype, device=dev)
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
        """Ring rows of positions [T - win_cap, T) of K, V (copied by the gather
        kernel): position T - W + i in ring row (win_offset + i) % win_cap with
        win_offset = 0, so the window [T - W, T) fills rows 0 .. W - 1 and the
        older positions (those >= 0) the rows after them."""
        if self.W == 0:
            return
        Ts = K.shape[2]
        C = self.win_cap
        pos = [(self.T - self.W + r) if r < self.W else (self.T - self.W - (C - r)) for r in range(C)]
        idx = torch.tensor([p if p >= 0 else -1 for p in pos], dtype=torch.int32).repeat(self._n, 1)
        idx = idx.to(K.device)
        hq_gather_rows(K, self._n, Ts, self.D, idx, C, self.win_k, stream=stream)
        hq_gather_rows(V, self._n, Ts, self.D, idx, C, self.win_v, stream=stream)
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
        d.win_cap = self.win_cap if self.W else 0
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


class RollingCache(HybridCache):
    """One layer's hybrid cache as it rolls over decode steps.

    The 16-bit store is bounded: the VL rows and a window ring of W + R rows,
    whose R extra rows keep the positions that left the window since the last
    re-detection. Each step runs hq_decode_step (attention, the query into
    the detector ring, the oldest window row packed into INT4); every R-th
    step the detector scores the cache's INT4 keys (hq_detect_vlines_cache)
    and hq_vl_update re-chooses the VL set among the rows that still have
    16-bit copies. This class only holds the buffers and the integer
    bookkeeping (T, ring offset, first staged position); every step runs in
    the library's kernels, except writing the new token's K and V rows into
    the ring, which is the caller's projection output."""

    def __init__(self, B: int, Hkv: int, D: int, T0: int, W: int, k: int, hp_dtype: torch.dtype,
                 Hq: int, R: int = 64, t_cap: int | None = None, device="cuda"):
        if W < 1:
            raise ValueError("a rolling cache needs a window")
        super().__init__(B, Hkv, D, T0, W, k, hp_dtype, t_cap=t_cap, device=device, win_cap=W + R)
        dev = torch.device(device)
        self.Hq, self.R = Hq, R
        self.step_no = 0
        self.p0 = T0 - W
        self.q_acc = torch.zeros((B, Hq, R, D), dtype=hp_dtype, device=dev)
        self.scores = torch.zeros((B, Hkv, self.t_cap), dtype=torch.int64, device=dev)
        self.det_ws = torch.zeros(hq_detect_workspace_size(B, Hkv, self.t_cap, 0), dtype=torch.uint8, device=dev)
        self.redet_ws = torch.zeros(hq_vl_redetect_workspace_size(self.descriptor()), dtype=torch.uint8, device=dev)

    def decode_step(self, q, out, lse, ws, n_splits=0, stream=None):
        """Attention of this step's queries over [0, T); q goes into ring slot
        step % R and position T - W is packed into its INT4 row."""
        hq_decode_step(q, self.Hq, self.descriptor(), 0.0, n_splits, out, lse, ws, q_acc=self.q_acc,
                       R=self.R, step=self.step_no, evict=True, stream=stream)

    def advance(self, k_row, v_row):
        """Next step: T + 1, the ring offset moves on, and the new token's rows
        ([B][Hkv][D], the hp dtype) go into the ring row of position T."""
        if self.T - self.W + 1 > self.t_cap:
            raise ValueError("the INT4 planes are full")
        self.T += 1
        self.win_offset = (self.win_offset + 1) % self.win_cap
        row = (self.win_offset + self.W - 1) % self.win_cap
        self.win_k[:, :, row].copy_(k_row)
        self.win_v[:, :, row].copy_(v_row)
        self.step_no += 1

    def due(self) -> bool:
        """True after the step that fills the detector ring's last slot."""
        return self.step_no > 0 and (self.step_no - 1) % self.R == self.R - 1

    def redetect(self, stream=None, fused=True):
        """The new VL set among the current one and the positions that left
        the window since the last update, by their column scores from the
        INT4 keys and the R accumulated steps: the candidates' scores only,
        then the update (hq_vl_redetect), or, with fused=False, the detector's
        scores of every position (hq_detect_vlines_cache) then
        hq_vl_update."""
        cand_end = self.T - self.W
        kv = self.descriptor()
        if fused:
            hq_vl_redetect(kv, self.vl_idx, self.p0, self.q_acc, self.Hq, self.R, self.redet_ws, stream=stream)
        else:
            sc = self.scores.view(-1)[:self.B * self.Hkv * cand_end]
            hq_detect_vlines_cache(None, self.q_acc, self.Hq, self.R, max(self.step_no - 1, 0), True, kv, cand_end,
                                   0, None, sc, self.det_ws, stream=stream)
            hq_vl_update(kv, self.vl_idx, self.p0, sc, cand_end, stream=stream)
        self.p0 = cand_end

    def resident_bytes(self) -> int:
        """Device bytes this layer's cache holds: INT4 planes and scales at
        capacity, VL bitmap, VL rows and index list, the window ring, the
        detector's query ring and score buffer."""
        ts = (self.k_codes, self.v_codes, self.k_sz, self.v_sz, self.vl_bits, self.vl_idx, self.vl_k,
              self.vl_v, self.win_k, self.win_v, self.q_acc, self.scores)
        return int(sum(t.numel() * t.element_size() for t in ts))
