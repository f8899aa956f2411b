"""C-ABI checks that need no GPU: the library loads, exports every function
declared in include/hq.h, and rejects bad arguments with the documented
status before anything is enqueued."""
import ctypes
import os
import re
import subprocess

import pytest

import hybrid_precision_quantized_amd as hq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hq.h")

FAKE = 0x100000          # a 256-byte aligned non-null address that is never dereferenced


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(hq_\w+)\s*\(", text)))


def test_header_declarations_are_exported():
    names = declared_functions()
    assert len(names) >= 11
    out = subprocess.run(["nm", "-D", "--defined-only", hq.library_path()],
                         capture_output=True, text=True, check=True).stdout
    exported = set(line.split()[-1] for line in out.splitlines() if line.strip())
    missing = [n for n in names if n not in exported]
    assert not missing, missing
    lib = hq.lib()
    for n in names:
        assert hasattr(lib, n)
    assert set(hq.EXPORTED) <= set(names) | {"hq_vl_bitmap"}


def test_version_and_strings():
    assert hq.hq_abi_version() == 2
    assert hq.hq_status_string(0) == "ok"
    assert "workspace" in hq.hq_status_string(3)


def _kv(**over):
    d = hq.HybridKV()
    d.B, d.Hkv, d.D, d.group = 1, 2, 128, 32
    d.T, d.W, d.k, d.t_cap = 1000, 128, 40, 896
    for f in ("k_codes", "v_codes", "k_sz", "v_sz", "vl_bits", "vl_k", "vl_v", "win_k", "win_v"):
        setattr(d, f, FAKE)
    d.win_offset, d.hp_dtype = 0, hq.HQ_BF16
    for k, v in over.items():
        setattr(d, k, v)
    return d


def _decode(kv, Hq=8, q=FAKE, qdt=hq.HQ_BF16, out=FAKE, ws=FAKE, ws_bytes=1 << 40, n_splits=0):
    return hq.lib().hq_decode_attn(q, qdt, Hq, ctypes.byref(kv) if kv is not None else None,
                                   0.0, n_splits, out, None, ws, ws_bytes, None)


@pytest.mark.parametrize("over,Hq,status", [
    ({"D": 96}, 8, hq.HQ_ERR_UNSUPPORTED),
    ({"group": 64}, 8, hq.HQ_ERR_UNSUPPORTED),
    ({"k": 900}, 8, hq.HQ_ERR_INVALID_ARG),          # k > T - W
    ({"W": 2000}, 8, hq.HQ_ERR_INVALID_ARG),         # W > T
    ({"t_cap": 800}, 8, hq.HQ_ERR_INVALID_ARG),      # t_cap < T - W
    ({"t_cap": 880}, 8, hq.HQ_ERR_INVALID_ARG),      # not a multiple of 32
    ({"win_offset": 128}, 8, hq.HQ_ERR_INVALID_ARG),
    ({"vl_bits": None}, 8, hq.HQ_ERR_INVALID_ARG),
    ({}, 7, hq.HQ_ERR_INVALID_ARG),                  # Hq % Hkv
    ({}, 64, hq.HQ_ERR_UNSUPPORTED),                 # G = 32
    ({"T": 0, "W": 0, "k": 0}, 8, hq.HQ_ERR_INVALID_ARG),
])
def test_decode_rejects(over, Hq, status):
    assert _decode(_kv(**over), Hq=Hq) == status
    assert hq.hq_last_error() != ""


def test_decode_rejects_null_and_dtype_and_workspace():
    assert _decode(None) == hq.HQ_ERR_INVALID_ARG
    assert _decode(_kv(), q=None) == hq.HQ_ERR_INVALID_ARG
    assert _decode(_kv(), qdt=hq.HQ_F16) == hq.HQ_ERR_UNSUPPORTED       # q dtype != rows dtype
    assert _decode(_kv(), qdt=7) == hq.HQ_ERR_INVALID_ARG
    kv = _kv()
    need = hq.hq_decode_workspace_size(kv, 8, 0)
    assert need > 0
    assert _decode(kv, ws_bytes=need - 1) == hq.HQ_ERR_WORKSPACE
    assert _decode(kv, ws=None) == hq.HQ_ERR_WORKSPACE
    assert _decode(kv, n_splits=-1) == hq.HQ_ERR_INVALID_ARG


def _step(kv, q_acc=FAKE, R=64, step=0, evict=1, ws_bytes=1 << 40):
    return hq.lib().hq_decode_step(FAKE, hq.HQ_BF16, 8, ctypes.byref(kv) if kv is not None else None,
                                   0.0, 0, FAKE, None, FAKE, ws_bytes, q_acc, R, step, evict, None)


def test_decode_step_rejects():
    # T - W = 872 needs t_cap >= 873 for the eviction: 896 is enough, 872 is not
    assert _step(_kv(t_cap=864)) == hq.HQ_ERR_INVALID_ARG             # also < T - W
    assert _step(_kv(T=1024, W=128, t_cap=896)) == hq.HQ_ERR_INVALID_ARG   # T - W = 896: no room
    assert "t_cap" in hq.hq_last_error()
    assert _step(_kv(), R=0) == hq.HQ_ERR_INVALID_ARG
    assert _step(_kv(), R=2000) == hq.HQ_ERR_INVALID_ARG
    assert _step(_kv(), step=-1) == hq.HQ_ERR_INVALID_ARG
    assert _step(_kv(), q_acc=FAKE + 4) == hq.HQ_ERR_INVALID_ARG      # misaligned ring
    assert _step(None) == hq.HQ_ERR_INVALID_ARG
    assert _step(_kv(), ws_bytes=1) == hq.HQ_ERR_WORKSPACE
    # without eviction the t_cap rule is that of hq_decode_attn
    assert _step(_kv(T=1024, W=128, t_cap=896), evict=0, ws_bytes=1) == hq.HQ_ERR_WORKSPACE


def test_decode_flags():
    assert _decode(_kv(flags=2)) == hq.HQ_ERR_INVALID_ARG                  # unknown flag
    assert "flags" in hq.hq_last_error()
    # dropping the INT4 set: the planes and the bitmap may be null (the call
    # then gets as far as the workspace check)
    kv = _kv(flags=hq.HQ_KV_DROP_INT4, k_codes=None, v_codes=None, k_sz=None, v_sz=None, vl_bits=None)
    assert _decode(kv, ws_bytes=1) == hq.HQ_ERR_WORKSPACE
    assert _decode(_kv(k_codes=None), ws_bytes=1) == hq.HQ_ERR_INVALID_ARG


def test_workspace_sizes():
    kv = _kv()
    s0 = hq.hq_decode_workspace_size(kv, 8, 0)
    s4 = hq.hq_decode_workspace_size(kv, 8, 4)
    s64 = hq.hq_decode_workspace_size(kv, 8, 64)
    assert 0 < s4 < s64 and s0 > 0
    assert hq.hq_decode_auto_splits(kv, 8) >= 1
    assert hq.hq_decode_workspace_size(_kv(D=96), 8, 0) == 0
    assert hq.hq_detect_workspace_size(1, 2, 32640, 1638) >= 2 * 32640 * 8


def test_quantize_rejects():
    L = hq.lib()
    ok = dict(x=FAKE, dt=hq.HQ_BF16, nh=2, nr=10, D=128, g=32, xh=1280 * 2, xr=128,
              codes=FAKE, sz=FAKE, lay=hq.HQ_LAYOUT_ROWS, dhr=64, d0=0)

    def call(**o):
        a = dict(ok, **o)
        return L.hq_quantize_kv(a["x"], a["dt"], a["nh"], a["nr"], a["D"], a["g"], a["xh"], a["xr"],
                                a["codes"], a["sz"], a["lay"], a["dhr"], a["d0"], None)
    assert call(g=16) == hq.HQ_ERR_UNSUPPORTED
    assert call(D=96) == hq.HQ_ERR_UNSUPPORTED
    assert call(dt=9) == hq.HQ_ERR_INVALID_ARG
    assert call(lay=5) == hq.HQ_ERR_INVALID_ARG
    assert call(d0=60) == hq.HQ_ERR_INVALID_ARG          # rows past dst_head_rows
    assert call(lay=hq.HQ_LAYOUT_TILE16, dhr=72) == hq.HQ_ERR_INVALID_ARG
    assert call(x=None) == hq.HQ_ERR_INVALID_ARG
    assert call(xr=100) == hq.HQ_ERR_INVALID_ARG         # rows not 16-byte aligned
    assert call(nr=0) == hq.HQ_OK                        # empty: no-op, nothing enqueued


def test_gather_and_bitmap_reject():
    L = hq.lib()
    assert L.hq_gather_rows(FAKE, hq.HQ_BF16, 2, 100, 128, None, 5, FAKE, None) == hq.HQ_ERR_INVALID_ARG
    assert L.hq_gather_rows(FAKE, hq.HQ_BF16, 2, 100, 4, FAKE, 5, FAKE, None) == hq.HQ_ERR_UNSUPPORTED
    assert L.hq_gather_rows(FAKE, hq.HQ_BF16, 2, 100, 128, FAKE, 0, FAKE, None) == hq.HQ_OK
    assert L.hq_vl_bitmap(FAKE, 2, 5, 100, FAKE, None) == hq.HQ_ERR_INVALID_ARG   # t_cap % 32
    assert L.hq_vl_bitmap(FAKE, 0, 5, 128, FAKE, None) == hq.HQ_OK


def test_detect_rejects_and_accumulate_only_path():
    L = hq.lib()
    ran = ctypes.c_int(7)

    def call(**o):
        a = dict(q_new=None, q_acc=FAKE, dt=hq.HQ_BF16, B=1, Hq=32, Hkv=2, D=128, R=64, step=0,
                 force=0, k=FAKE, k_rows=1000, ce=900, kt=45, m=hq.HQ_DETECT_MATMUL, idx=FAKE,
                 sc=None, ws=FAKE, wsb=1 << 30)
        a.update(o)
        return L.hq_detect_vlines(a["q_new"], a["q_acc"], a["dt"], a["B"], a["Hq"], a["Hkv"], a["D"],
                                  a["R"], a["step"], a["force"], a["k"], a["k_rows"], a["ce"], a["kt"],
                                  a["m"], a["idx"], a["sc"], ctypes.byref(ran), a["ws"], a["wsb"], None)
    assert call(Hq=31) == hq.HQ_ERR_INVALID_ARG
    assert call(D=96) == hq.HQ_ERR_UNSUPPORTED
    assert call(R=0) == hq.HQ_ERR_INVALID_ARG
    assert call(kt=901) == hq.HQ_ERR_INVALID_ARG
    assert call(ce=1001) == hq.HQ_ERR_INVALID_ARG
    assert call(m=3) == hq.HQ_ERR_INVALID_ARG
    assert call(dt=hq.HQ_F32, step=63) == hq.HQ_ERR_UNSUPPORTED     # fp32 needs the QSUM form
    assert call(step=63, wsb=16) == hq.HQ_ERR_WORKSPACE
    # no q_new and not the last slot: nothing to do, nothing enqueued
    assert call(step=5) == hq.HQ_OK and ran.value == 0
