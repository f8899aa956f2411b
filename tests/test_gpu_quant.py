"""GPU parity of hq_quantize_kv, hq_gather_rows and hq_vl_bitmap against the
oracle: bit-exact codes, fp16 scale/zero bits, copied rows and bitmaps."""
import numpy as np
import pytest
import torch

import hybrid_precision_quantized_amd as hq
import synth
from oracle import quant
from tests.gpu_util import TORCH_DT, say, sz_bits, tile16_codes, to_dev

pytestmark = pytest.mark.gpu


def _values(rng, n_heads, n_rows, D, dtype):
    x = rng.standard_normal((n_heads, n_rows, D)) * rng.uniform(0.05, 8.0, (n_heads, n_rows, 1))
    x[..., 3] *= 10.0                                  # an outlier channel
    # special groups: constant, signed zeros, exact half-way ties
    if n_rows > 4:
        x[:, 0, :32] = 1.5
        x[:, 1, :] = 0.0
        x[:, 1, ::3] = -0.0
        s, z = 0.5, -2.0
        c = np.arange(32) % 16
        x[:, 2, :32] = z + c * s
        x[:, 2, 32:64] = z + (np.arange(32) % 15 + 0.5) * s
        x[:, 2, 32] = z
        x[:, 2, 33] = z + 15 * s
    if dtype == "bf16":
        x = synth.round_dtype(x, "bf16")
    elif dtype == "f16":
        x = np.asarray(x, np.float64).astype(np.float16).astype(np.float32)
    else:
        x = synth.round_dtype(x, "f32")
    return x


@pytest.mark.parametrize("dtype,D,n_heads,n_rows,row0,layout", [
    ("bf16", 128, 3, 1000, 0, hq.HQ_LAYOUT_ROWS),
    ("bf16", 128, 3, 1000, 5, hq.HQ_LAYOUT_TILE16),
    ("bf16", 64, 2, 333, 7, hq.HQ_LAYOUT_ROWS),
    ("bf16", 64, 2, 333, 16, hq.HQ_LAYOUT_TILE16),
    ("f32", 64, 1, 480, 0, hq.HQ_LAYOUT_ROWS),
    ("f32", 128, 2, 97, 3, hq.HQ_LAYOUT_TILE16),
    ("f16", 128, 2, 513, 1, hq.HQ_LAYOUT_ROWS),
    ("f16", 128, 1, 1, 31, hq.HQ_LAYOUT_TILE16),
])
def test_quantize_bit_exact(dtype, D, n_heads, n_rows, row0, layout):
    say(f"quantize dtype={dtype} D={D} heads={n_heads} rows={n_rows} row0={row0} layout={layout}")
    rng = np.random.default_rng(D * 1000 + n_rows)
    src_rows = n_rows + 3                       # source has extra rows: stride != n_rows * D
    x = _values(rng, n_heads, src_rows, D, dtype)
    xd = to_dev(x, dtype)
    cap = ((row0 + n_rows + 31) // 32) * 32
    codes = torch.full((n_heads, cap, D // 2), 0xA5, dtype=torch.uint8, device="cuda")
    sz = torch.full((n_heads, cap, D // 32, 2), 0x1234, dtype=torch.int16, device="cuda")
    if layout == hq.HQ_LAYOUT_TILE16:
        codes = codes.view(n_heads, cap // 16, D // 2, 16)
    hq.hq_quantize_kv(xd, n_heads, n_rows, D, src_rows * D, D, codes, sz, layout, cap, row0)
    torch.cuda.synchronize()
    got = tile16_codes(codes) if layout == hq.HQ_LAYOUT_TILE16 else codes.cpu().numpy()
    want_p, want_sz = quant.quantize_rows(x[:, :n_rows], 32)
    assert np.array_equal(got[:, row0:row0 + n_rows], want_p)
    assert np.array_equal(sz_bits(sz)[:, row0:row0 + n_rows], want_sz)
    # rows outside [row0, row0 + n_rows) untouched
    assert np.all(got[:, :row0] == 0xA5) and np.all(got[:, row0 + n_rows:] == 0xA5)


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("f32", 64), ("f16", 128)])
def test_gather_rows_exact(dtype, D):
    say(f"gather dtype={dtype} D={D}")
    rng = np.random.default_rng(3)
    n_heads, src_rows, k = 5, 700, 37
    x = synth.round_dtype(rng.standard_normal((n_heads, src_rows, D)), "f32")
    if dtype == "bf16":
        x = synth.round_dtype(x, "bf16")
    elif dtype == "f16":
        x = x.astype(np.float16).astype(np.float32)
    src = to_dev(x, dtype)
    idx = np.stack([np.sort(rng.choice(src_rows, k, replace=False)) for _ in range(n_heads)]).astype(np.int32)
    idx[1, 3] = -4
    idx[2, 5] = src_rows + 10                   # out of range -> zero row
    dst = torch.full((n_heads, k, D), 7.0, dtype=TORCH_DT[dtype], device="cuda")
    hq.hq_gather_rows(src, n_heads, src_rows, D, torch.from_numpy(idx).cuda(), k, dst)
    torch.cuda.synchronize()
    got = dst.float().cpu().numpy()
    for h in range(n_heads):
        for i in range(k):
            j = idx[h, i]
            ref = x[h, j] if 0 <= j < src_rows else np.zeros(D)
            assert np.array_equal(got[h, i], ref)


def test_vl_bitmap_exact():
    say("vl_bitmap")
    rng = np.random.default_rng(4)
    n_heads, t_cap, k = 6, 262144 + 4096, 500
    idx = np.stack([np.sort(rng.choice(t_cap, k, replace=False)) for _ in range(n_heads)]).astype(np.int32)
    bits = torch.full((n_heads, t_cap // 32), -1, dtype=torch.int32, device="cuda")
    hq.hq_vl_bitmap(torch.from_numpy(idx).cuda(), n_heads, k, t_cap, bits)
    torch.cuda.synchronize()
    want = np.zeros((n_heads, t_cap // 32), dtype=np.uint32)
    for h in range(n_heads):
        for t in idx[h]:
            want[h, t // 32] |= np.uint32(1) << np.uint32(t % 32)
    assert np.array_equal(bits.cpu().numpy().view(np.uint32), want)


@pytest.mark.parametrize("dtype,D,n_heads,n_rows,row0", [("bf16", 128, 8, 1, 32639), ("bf16", 64, 3, 40, 8),
                                                         ("f32", 64, 2, 17, 0), ("f16", 128, 4, 100, 28)])
def test_quantize_pair_matches_oracle(dtype, D, n_heads, n_rows, row0):
    say(f"quantize pair dtype={dtype} D={D} heads={n_heads} rows={n_rows} row0={row0}")
    rng = np.random.default_rng(n_rows + D)
    src_rows = n_rows + 5
    xk = _values(rng, n_heads, src_rows, D, dtype)
    xv = _values(rng, n_heads, src_rows, D, dtype)
    cap = ((row0 + n_rows + 31) // 32) * 32
    kc = torch.full((n_heads, cap, D // 2), 0x5A, dtype=torch.uint8, device="cuda")
    vc = torch.full((n_heads, cap // 16, D // 2, 16), 0x5A, dtype=torch.uint8, device="cuda")
    ks = torch.zeros((n_heads, cap, D // 32, 2), dtype=torch.int16, device="cuda")
    vs = torch.zeros_like(ks)
    hq.hq_quantize_kv_pair(to_dev(xk, dtype), to_dev(xv, dtype), n_heads, n_rows, D, src_rows * D, D,
                           kc, ks, vc, vs, cap, row0)
    torch.cuda.synchronize()
    kp, kz = quant.quantize_rows(xk[:, :n_rows], 32)
    vp, vz = quant.quantize_rows(xv[:, :n_rows], 32)
    assert np.array_equal(kc.cpu().numpy()[:, row0:row0 + n_rows], kp)
    assert np.array_equal(tile16_codes(vc)[:, row0:row0 + n_rows], vp)
    assert np.array_equal(sz_bits(ks)[:, row0:row0 + n_rows], kz)
    assert np.array_equal(sz_bits(vs)[:, row0:row0 + n_rows], vz)
    assert np.all(kc.cpu().numpy()[:, :row0] == 0x5A)
