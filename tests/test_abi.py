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
    assert hq.hq_abi_version() == 3
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


def test_decode_rejects_empty_softmax_and_misaligned_words():
    # dropping the INT4 set with no VL rows and no window leaves nothing to attend to
    kv = _kv(flags=hq.HQ_KV_DROP_INT4, T=800, k=0, W=0, win_offset=0)
    assert _decode(kv) == hq.HQ_ERR_INVALID_ARG
    assert "empty" in hq.hq_last_error()
    # the scale planes and the VL bitmap are read as 32-bit words
    for f in ("k_sz", "v_sz", "vl_bits"):
        assert _decode(_kv(**{f: FAKE + 2})) == hq.HQ_ERR_INVALID_ARG, f
        assert "4-byte" in hq.hq_last_error()
    assert _decode(_kv(k_sz=FAKE + 4), ws_bytes=1) == hq.HQ_ERR_WORKSPACE   # 4-byte aligned is enough


def test_quantize_pair_rejects():
    L = hq.lib()
    ok = dict(xk=FAKE, xv=FAKE, dt=hq.HQ_BF16, nh=2, nr=10, D=128, g=32, xh=1280, xr=128,
              kc=FAKE, ks=FAKE, vc=FAKE, vs=FAKE, dhr=64, d0=0)

    def call(**o):
        a = dict(ok, **o)
        return L.hq_quantize_kv_pair(a["xk"], a["xv"], a["dt"], a["nh"], a["nr"], a["D"], a["g"], a["xh"],
                                     a["xr"], a["kc"], a["ks"], a["vc"], a["vs"], a["dhr"], a["d0"], None)
    assert call(dt=5) == hq.HQ_ERR_INVALID_ARG
    assert call(g=64) == hq.HQ_ERR_UNSUPPORTED
    assert call(D=256) == hq.HQ_ERR_UNSUPPORTED
    assert call(nr=-1) == hq.HQ_ERR_INVALID_ARG
    assert call(d0=60) == hq.HQ_ERR_INVALID_ARG          # rows past dst_head_rows
    assert call(dhr=72) == hq.HQ_ERR_INVALID_ARG         # not a multiple of 16 (TILE16 values)
    assert call(xv=None) == hq.HQ_ERR_INVALID_ARG
    assert call(vs=None) == hq.HQ_ERR_INVALID_ARG
    assert call(xr=100) == hq.HQ_ERR_INVALID_ARG         # rows not 16-byte aligned
    assert call(ks=FAKE + 2) == hq.HQ_ERR_INVALID_ARG    # scale plane not 4-byte aligned
    assert call(nr=0) == hq.HQ_OK                        # empty: no-op


@pytest.mark.parametrize("entry", ["hq_prefill_attn", "hq_prefill_attn_i8"])
def test_prefill_rejects(entry):
    L = hq.lib()
    fn = getattr(L, entry)
    ok = dict(q=FAKE, k=FAKE, v=FAKE, dt=hq.HQ_BF16, B=1, Hq=8, Hkv=2, T=1000, D=128, g=32, W=128,
              vl=FAKE, kvl=50, out=FAKE, lse=None, ws=FAKE, wsb=1 << 40)

    def call(**o):
        a = dict(ok, **o)
        return fn(a["q"], a["k"], a["v"], a["dt"], a["B"], a["Hq"], a["Hkv"], a["T"], a["D"], a["g"], a["W"],
                  a["vl"], a["kvl"], 0.0, a["out"], a["lse"], a["ws"], a["wsb"], None)
    assert call(dt=hq.HQ_F32) == hq.HQ_ERR_UNSUPPORTED
    assert call(D=64) == hq.HQ_ERR_UNSUPPORTED
    assert call(g=16) == hq.HQ_ERR_UNSUPPORTED
    assert call(T=0) == hq.HQ_ERR_INVALID_ARG
    assert call(Hq=7) == hq.HQ_ERR_INVALID_ARG
    assert call(W=-1) == hq.HQ_ERR_INVALID_ARG
    assert call(kvl=1001) == hq.HQ_ERR_INVALID_ARG        # more VL columns than positions
    assert call(q=None) == hq.HQ_ERR_INVALID_ARG
    assert call(out=FAKE + 8) == hq.HQ_ERR_INVALID_ARG    # misaligned
    need = hq.hq_prefill_workspace_size(1, 8, 2, 1000, 128, 50)
    assert need > 0
    assert call(wsb=need - 1) == hq.HQ_ERR_WORKSPACE
    assert call(ws=FAKE + 16) == hq.HQ_ERR_INVALID_ARG    # workspace not 256-byte aligned
    assert call(T=1 << 23, Hq=2, kvl=0) == hq.HQ_ERR_UNSUPPORTED   # one head's planes past 2^31 bytes
    assert entry in hq.hq_last_error()


def test_vl_update_and_redetect_reject():
    """Both in-place VL updates reject what they cannot do before launching
    anything: p0 outside [max(0, T - win_cap), T - W] (rows no longer in the
    ring), too many recent positions or candidates, a bad head dim, the
    fused form's query arguments; p0 == T - W is a no-op."""
    L = hq.lib()
    ok = dict(kv=_kv(win_cap=192), idx=FAKE, p0=808, sc=FAKE, stride=872, q=FAKE, qdt=hq.HQ_BF16, Hq=8, R=64,
              ws=FAKE, wsb=1 << 30)

    def upd(**o):
        a = dict(ok, **o)
        kv = a["kv"]
        return L.hq_vl_update(ctypes.byref(kv) if kv is not None else None, a["idx"], a["p0"], a["sc"],
                              a["stride"], None)

    def red(**o):
        a = dict(ok, **o)
        kv = a["kv"]
        return L.hq_vl_redetect(ctypes.byref(kv) if kv is not None else None, a["idx"], a["p0"], a["q"], a["qdt"],
                                a["Hq"], a["R"], a["ws"], a["wsb"], None)
    for call in (upd, red):
        assert call(kv=None) == hq.HQ_ERR_INVALID_ARG
        assert call(p0=873) == hq.HQ_ERR_INVALID_ARG                  # past T - W
        assert call(p0=807) == hq.HQ_ERR_INVALID_ARG                  # its row left the ring
        assert call(kv=_kv(win_cap=192, D=96)) == hq.HQ_ERR_UNSUPPORTED
        assert call(kv=_kv(T=3000, t_cap=2880, win_cap=3000), p0=100, stride=2872) == hq.HQ_ERR_UNSUPPORTED
        assert call(kv=_kv(T=10000, t_cap=9888, k=8200, win_cap=192), p0=9808, stride=9872) == \
            hq.HQ_ERR_UNSUPPORTED                                       # more than 8192 candidates
        assert call(idx=None) == hq.HQ_ERR_INVALID_ARG
        assert call(kv=_kv(win_cap=192, vl_k=FAKE + 8)) == hq.HQ_ERR_INVALID_ARG
        assert call(p0=872) == hq.HQ_OK                                # no position left the window
    assert upd(stride=871) == hq.HQ_ERR_INVALID_ARG
    assert upd(sc=None) == hq.HQ_ERR_INVALID_ARG
    assert red(qdt=hq.HQ_F16) == hq.HQ_ERR_INVALID_ARG                # not the cache's 16-bit dtype
    assert red(Hq=7) == hq.HQ_ERR_INVALID_ARG
    assert red(R=0) == hq.HQ_ERR_INVALID_ARG and red(R=1025) == hq.HQ_ERR_INVALID_ARG
    assert red(q=None) == hq.HQ_ERR_INVALID_ARG
    assert red(q=FAKE + 8) == hq.HQ_ERR_INVALID_ARG
    assert red(kv=_kv(win_cap=192, k_codes=None)) == hq.HQ_ERR_INVALID_ARG
    need = hq.hq_vl_redetect_workspace_size(_kv(win_cap=192))
    assert need == 2 * (40 + 1024) * 8
    assert red(wsb=need - 1) == hq.HQ_ERR_WORKSPACE and red(ws=None) == hq.HQ_ERR_WORKSPACE
    assert red(ws=FAKE + 4) == hq.HQ_ERR_INVALID_ARG
    assert "hq_vl_redetect" in hq.hq_last_error()


def test_detect_cache_and_mass_reject():
    L = hq.lib()
    ran = ctypes.c_int(7)
    kv = _kv()

    def cache(**o):
        a = dict(q_new=None, q_acc=FAKE, dt=hq.HQ_BF16, Hq=8, R=64, step=63, force=0, kv=kv, ce=800,
                 kt=40, idx=FAKE, sc=None, ws=FAKE, wsb=1 << 30)
        a.update(o)
        return L.hq_detect_vlines_cache(a["q_new"], a["q_acc"], a["dt"], a["Hq"], a["R"], a["step"], a["force"],
                                        ctypes.byref(a["kv"]) if a["kv"] is not None else None, a["ce"],
                                        a["kt"], a["idx"], a["sc"], ctypes.byref(ran), a["ws"], a["wsb"], None)
    assert cache(kv=None) == hq.HQ_ERR_INVALID_ARG
    assert cache(dt=9) == hq.HQ_ERR_INVALID_ARG
    assert cache(Hq=7) == hq.HQ_ERR_INVALID_ARG
    assert cache(kv=_kv(D=96)) == hq.HQ_ERR_UNSUPPORTED
    assert cache(R=0) == hq.HQ_ERR_INVALID_ARG
    assert cache(step=-1) == hq.HQ_ERR_INVALID_ARG
    assert cache(ce=1001) == hq.HQ_ERR_INVALID_ARG       # beyond T
    assert cache(kt=801) == hq.HQ_ERR_INVALID_ARG        # k_top > cand_end
    assert cache(q_acc=None) == hq.HQ_ERR_INVALID_ARG
    assert cache(wsb=8) == hq.HQ_ERR_WORKSPACE
    assert cache(step=5) == hq.HQ_OK and ran.value == 0  # not the ring's last slot: nothing to do

    def mass(**o):
        a = dict(q_new=None, q_acc=FAKE, dt=hq.HQ_BF16, B=1, Hq=32, Hkv=2, D=128, R=64, step=63, force=0,
                 k=FAKE, k_rows=1000, ce=900, kt=45, idx=FAKE, sc=None, ws=FAKE, wsb=1 << 30)
        a.update(o)
        return L.hq_detect_vlines_mass(a["q_new"], a["q_acc"], a["dt"], a["B"], a["Hq"], a["Hkv"], a["D"],
                                       a["R"], a["step"], a["force"], a["k"], a["k_rows"], a["ce"], a["kt"], 0.0,
                                       a["idx"], a["sc"], ctypes.byref(ran), a["ws"], a["wsb"], None)
    assert mass(dt=hq.HQ_F32) == hq.HQ_ERR_UNSUPPORTED
    assert mass(Hq=31) == hq.HQ_ERR_INVALID_ARG
    assert mass(D=96) == hq.HQ_ERR_UNSUPPORTED
    assert mass(R=2000) == hq.HQ_ERR_INVALID_ARG
    assert mass(ce=1001) == hq.HQ_ERR_INVALID_ARG
    assert mass(kt=901) == hq.HQ_ERR_INVALID_ARG
    assert mass(k=None) == hq.HQ_ERR_INVALID_ARG
    assert mass(wsb=8) == hq.HQ_ERR_WORKSPACE
    assert mass(k=FAKE + 8) == hq.HQ_ERR_INVALID_ARG     # misaligned keys
    assert mass(step=5) == hq.HQ_OK and ran.value == 0


def test_stream_read_rejects():
    L = hq.lib()
    assert L.hq_stream_read(None, 4096, FAKE, None) == hq.HQ_ERR_INVALID_ARG
    assert L.hq_stream_read(FAKE, 4096, None, None) == hq.HQ_ERR_INVALID_ARG
    assert L.hq_stream_read(FAKE + 8, 4096, FAKE, None) == hq.HQ_ERR_INVALID_ARG
    assert L.hq_stream_read(FAKE, 4100, FAKE, None) == hq.HQ_ERR_INVALID_ARG
    assert L.hq_stream_read(FAKE, 0, FAKE, None) == hq.HQ_OK
    assert hq.lib().hq_stream_read_sink_bytes() > 0


_NO_DEVICE_SCRIPT = r"""
import ctypes, sys
import hybrid_precision_quantized_amd as hq
L = hq.lib()
F = 0x100000
kv = hq.HybridKV()
kv.B, kv.Hkv, kv.D, kv.group, kv.T, kv.W, kv.k, kv.t_cap = 1, 2, 128, 32, 1000, 128, 40, 896
for f in ("k_codes", "v_codes", "k_sz", "v_sz", "vl_bits", "vl_k", "vl_v", "win_k", "win_v"):
    setattr(kv, f, F)
kv.hp_dtype = hq.HQ_BF16
calls = {
    "hq_decode_attn": lambda: L.hq_decode_attn(F, hq.HQ_BF16, 8, ctypes.byref(kv), 0.0, 0, F, None, F, 1 << 40, None),
    "hq_quantize_kv": lambda: L.hq_quantize_kv(F, hq.HQ_BF16, 2, 10, 128, 32, 2560, 128, F, F, 0, 64, 0, None),
    "hq_gather_rows": lambda: L.hq_gather_rows(F, hq.HQ_BF16, 2, 100, 128, F, 5, F, None),
    "hq_vl_bitmap": lambda: L.hq_vl_bitmap(F, 2, 5, 128, F, None),
    "hq_stream_read": lambda: L.hq_stream_read(F, 4096, F, None),
}
for name, fn in calls.items():
    s = fn()
    msg = hq.hq_last_error()
    print(name, s, msg)
    assert s == hq.HQ_ERR_HIP, (name, s)
    assert msg, name
print("NO_DEVICE_OK")
"""


def test_no_device_reports_hip_error():
    """Without a GPU every valid call fails with HQ_ERR_HIP and a message
    instead of crashing. Run in a child process (no HIP state leaks into this
    one) and only where no device is visible: with a GPU present the same
    calls would launch kernels on the fake addresses."""
    import sys
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("a GPU is visible: this check runs only where none is")
    r = subprocess.run([sys.executable, "-c", _NO_DEVICE_SCRIPT], capture_output=True, text=True,
                       cwd=ROOT, timeout=300)
    assert r.returncode == 0 and "NO_DEVICE_OK" in r.stdout, r.stdout + r.stderr


def test_decode_noalloc_rejects_before_touching_a_device():
    L = hq.lib()

    def call(kv, Hq=8, n_splits=0, q=FAKE, out=FAKE):
        return L.hq_decode_attn_noalloc(q, hq.HQ_BF16, Hq, ctypes.byref(kv) if kv is not None else None,
                                        0.0, n_splits, out, None, None)
    assert call(None) == hq.HQ_ERR_INVALID_ARG
    assert call(_kv(D=96)) == hq.HQ_ERR_UNSUPPORTED
    assert call(_kv(), q=None) == hq.HQ_ERR_INVALID_ARG
    assert call(_kv(), n_splits=-1) == hq.HQ_ERR_INVALID_ARG
    # more split partials than the fixed array holds: 16 x 32 heads x 256 splits
    big = _kv(B=16, Hkv=8, T=4096, W=128, k=100, t_cap=4096)
    assert hq.hq_decode_workspace_size(big, 32, 256) > hq.HQ_DECODE_SCRATCH_BYTES
    assert call(big, Hq=32, n_splits=256) == hq.HQ_ERR_WORKSPACE
    assert "fixed" in hq.hq_last_error()
