"""The C ABI on the CPU: libpa.so loads, exports every function include/pa.h
declares, and its host-side argument checks return the documented status
codes before anything is launched (no GPU is touched by these tests)."""

import ctypes
import glob
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pa.h")
HEADERS = sorted(glob.glob(os.path.join(ROOT, "include", "*.h")))

pa = pytest.importorskip("paged_kv_attention_07_amd")
lib = pa.lib

OK, INVALID, UNSUPPORTED, WORKSPACE, SCRATCH = 0, -1, -2, -3, -5
FAKE = ctypes.c_void_p(0x10000)     # never dereferenced: checks fail before use
FAKE_WS = ctypes.c_void_p(0x100000)  # 256-byte aligned


def declared_functions():
    names = set()
    for path in HEADERS:
        text = open(path, encoding="utf-8").read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names |= set(re.findall(r"\b(pa_[a-z_0-9]+)\s*\(", text))
    return sorted(names)


def test_header_declares_the_boundary():
    names = declared_functions()
    for want in ("pa_reshape_and_cache", "pa_attention_decode", "pa_attention_mixed",
                 "pa_compute_slot_mapping", "pa_attention_workspace_size", "pa_status_string",
                 "pa_copy_blocks", "pa_sched_create", "pa_sched_schedule", "pa_sched_update",
                 "pa_xxh64"):
        assert want in names


def test_every_declared_symbol_is_exported():
    out = subprocess.run(["nm", "-D", "--defined-only", pa.library_path], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    for name in declared_functions():
        assert name in exported, name
        assert hasattr(lib, name)


def test_no_torch_types_in_header():
    for path in HEADERS:
        text = open(path, encoding="utf-8").read()
        assert "at::" not in text and "torch::" not in text and "c10::" not in text
        assert "extern \"C\"" in text


def test_status_strings():
    assert pa.pa_status_string(OK) == "ok"
    for s in (INVALID, UNSUPPORTED, WORKSPACE, -4, SCRATCH):
        assert pa.pa_status_string(s) not in ("", "ok", "unknown status")
    assert pa.pa_status_string(12345) == "unknown status"
    assert pa.pa_version() >= 100


def rac(**kw):
    a = dict(key=FAKE, value=FAKE, kv=FAKE, slots=FAKE, T=4, NB=64, B=16, Hkv=2, D=64, dtype=0)
    a.update(kw)
    return lib.pa_reshape_and_cache(a["key"], a["value"], a["kv"], a["slots"], a["T"], a["NB"],
                                    a["B"], a["Hkv"], a["D"], a["dtype"], None)


def test_reshape_and_cache_checks():
    assert rac(key=None) == INVALID
    assert rac(slots=None) == INVALID
    assert rac(kv=None) == INVALID
    assert rac(T=-1) == INVALID
    assert rac(NB=0) == INVALID
    assert rac(B=32) == UNSUPPORTED
    assert rac(D=96) == UNSUPPORTED
    assert rac(dtype=9) == UNSUPPORTED
    assert rac(key=ctypes.c_void_p(0x10008)) == INVALID   # not 16-byte aligned
    assert rac(T=0) == OK                                 # nothing to do, nothing launched


def test_copy_blocks_checks():
    f = lib.pa_copy_blocks
    assert f(None, FAKE, 2, 64, 16, 2, 64, 1, None) == INVALID
    assert f(FAKE, None, 2, 64, 16, 2, 64, 1, None) == INVALID
    assert f(FAKE, FAKE, -1, 64, 16, 2, 64, 1, None) == INVALID
    assert f(FAKE, FAKE, 2, 0, 16, 2, 64, 1, None) == INVALID
    assert f(FAKE, FAKE, 2, 64, 8, 2, 64, 1, None) == UNSUPPORTED
    assert f(FAKE, FAKE, 2, 64, 16, 2, 96, 1, None) == UNSUPPORTED
    assert f(FAKE, FAKE, 2, 64, 16, 2, 64, 7, None) == UNSUPPORTED
    assert f(FAKE, None, 0, 64, 16, 2, 64, 1, None) == OK   # nothing to copy


def ws_size(R=4, T=4, Hq=4, Hkv=2, D=64, L=100, Q=1, S=0):
    return lib.pa_attention_workspace_size(R, T, Hq, Hkv, D, L, Q, S)


def test_workspace_size_pure_and_rejecting():
    a = ws_size()
    assert a > 0 and a == ws_size() and a % 256 == 0
    assert ws_size(S=3) > 0 and ws_size(S=3) != ws_size(S=300)
    assert ws_size(Hq=6, Hkv=4) == 0        # not a multiple
    assert ws_size(Hq=6, Hkv=2) == 0        # group 3 unsupported
    assert ws_size(D=80) == 0
    assert ws_size(R=0) == 0
    # grows with the batch and with the split count
    assert ws_size(R=64, L=4096) > ws_size(R=4, L=4096)
    assert ws_size(S=64) > ws_size(S=8)


def decode(**kw):
    a = dict(out=FAKE, q=FAKE, kv=FAKE, NB=64, B=16, Hkv=2, D=64, dtype=0, bt=FAKE, stride=7,
             sl=FAKE, R=4, L=100, Hq=4, scale=0.125, ws=FAKE_WS, wsb=None, S=0)
    a.update(kw)
    if a["wsb"] is None:
        a["wsb"] = ws_size(R=a["R"], T=a["R"], Hq=a["Hq"], Hkv=a["Hkv"], D=a["D"], L=a["L"], S=a["S"])
    return lib.pa_attention_decode(a["out"], a["q"], a["kv"], a["NB"], a["B"], a["Hkv"], a["D"],
                                   a["dtype"], a["bt"], a["stride"], a["sl"], a["R"], a["L"],
                                   a["Hq"], a["scale"], a["ws"], a["wsb"], a["S"], None)


def test_decode_checks():
    assert decode(out=None) == INVALID
    assert decode(q=None) == INVALID
    assert decode(bt=None) == INVALID
    assert decode(sl=None) == INVALID
    assert decode(B=8) == UNSUPPORTED
    assert decode(D=256) == UNSUPPORTED
    assert decode(dtype=3) == UNSUPPORTED
    assert decode(Hq=5) == INVALID
    assert decode(Hq=6) == UNSUPPORTED and decode(Hq=6, Hkv=2) == UNSUPPORTED
    assert decode(Hq=32, Hkv=2) == UNSUPPORTED            # group 16
    assert decode(stride=3) == INVALID                    # table narrower than max_seq_len
    assert decode(scale=float("nan")) == INVALID
    assert decode(scale=float("inf")) == INVALID
    assert decode(scale=0.0) == INVALID                   # the scale is a positive temperature
    assert decode(scale=-0.125) == INVALID
    assert decode(S=-1) == INVALID
    assert decode(ws=None) == WORKSPACE
    assert decode(wsb=16) == WORKSPACE
    assert decode(ws=ctypes.c_void_p(0x100010)) == WORKSPACE  # misaligned workspace
    assert decode(R=0) == OK
    assert decode(L=0) == OK


def mixed(**kw):
    a = dict(out=FAKE, q=FAKE, kv=FAKE, NB=64, B=16, Hkv=2, D=64, dtype=1, bt=FAKE, stride=7,
             sl=FAKE, qsl=FAKE, nc=FAKE, R=4, T=20, Q=17, L=100, Hq=4, scale=0.125,
             ws=FAKE_WS, wsb=1 << 30, S=0)
    a.update(kw)
    return lib.pa_attention_mixed(a["out"], a["q"], a["kv"], a["NB"], a["B"], a["Hkv"], a["D"],
                                  a["dtype"], a["bt"], a["stride"], a["sl"], a["qsl"], a["nc"],
                                  a["R"], a["T"], a["Q"], a["L"], a["Hq"], a["scale"], a["ws"],
                                  a["wsb"], a["S"], None)


def test_mixed_checks():
    assert mixed(qsl=None) == INVALID
    assert mixed(nc=None) == INVALID
    assert mixed(T=-1) == INVALID
    assert mixed(Q=-1) == INVALID
    assert mixed(dtype=0, wsb=8) == WORKSPACE  # fp32 chunks are accepted (vector-ALU tiles)
    assert mixed(wsb=8) == WORKSPACE
    assert mixed(T=0) == OK


def cache_decode(**kw):
    a = dict(out=FAKE, q=FAKE, k=FAKE, v=FAKE, kv=FAKE, NB=64, B=16, Hkv=2, D=64, dtype=1,
             bt=FAKE, stride=7, sl=FAKE, slots=None, R=4, L=100, Hq=4, scale=0.125,
             ws=FAKE_WS, wsb=1 << 30, S=0)
    a.update(kw)
    return lib.pa_cache_and_attend_decode(
        a["out"], a["q"], a["k"], a["v"], a["kv"], a["NB"], a["B"], a["Hkv"], a["D"],
        a["dtype"], a["bt"], a["stride"], a["sl"], a["slots"], a["R"], a["L"], a["Hq"],
        a["scale"], a["ws"], a["wsb"], a["S"], None)


def cache_mixed(**kw):
    a = dict(out=FAKE, q=FAKE, k=FAKE, v=FAKE, kv=FAKE, NB=64, B=16, Hkv=2, D=64, dtype=1,
             bt=FAKE, stride=7, sl=FAKE, qsl=FAKE, nc=FAKE, slots=None, R=4, T=20, Q=17, L=100,
             Hq=4, scale=0.125, ws=FAKE_WS, wsb=1 << 30, S=0)
    a.update(kw)
    return lib.pa_cache_and_attend_mixed(
        a["out"], a["q"], a["k"], a["v"], a["kv"], a["NB"], a["B"], a["Hkv"], a["D"],
        a["dtype"], a["bt"], a["stride"], a["sl"], a["qsl"], a["nc"], a["slots"], a["R"],
        a["T"], a["Q"], a["L"], a["Hq"], a["scale"], a["ws"], a["wsb"], a["S"], None)


def test_cache_and_attend_checks():
    """The one-launch steps check the new-token inputs on top of the
    attention call's own checks."""
    for f in (cache_decode, cache_mixed):
        assert f(k=None) == INVALID
        assert f(v=None) == INVALID
        assert f(k=ctypes.c_void_p(0x10008)) == INVALID        # not 16-byte aligned
        assert f(out=None) == INVALID
        assert f(B=8) == UNSUPPORTED
        assert f(D=256) == UNSUPPORTED
        assert f(wsb=16) == WORKSPACE
    assert cache_decode(R=0, k=None, v=None) == OK             # nothing to store or attend
    assert cache_mixed(T=0, k=None, v=None) == OK
    assert cache_mixed(dtype=0, wsb=8) == WORKSPACE            # fp32 chunks are accepted


def no_workspace(**kw):
    a = dict(out=FAKE, q=FAKE, k=FAKE, v=FAKE, kv=FAKE, NB=64, B=16, Hkv=2, D=64, dtype=1,
             bt=FAKE, stride=7, sl=FAKE, qsl=FAKE, nc=FAKE, slots=None, R=4, T=20, Q=17, L=100,
             Hq=4, scale=0.125, S=0)
    a.update(kw)
    return lib.pa_cache_and_attend_mixed_no_workspace(
        a["out"], a["q"], a["k"], a["v"], a["kv"], a["NB"], a["B"], a["Hkv"], a["D"],
        a["dtype"], a["bt"], a["stride"], a["sl"], a["qsl"], a["nc"], a["slots"], a["R"],
        a["T"], a["Q"], a["L"], a["Hq"], a["scale"], a["S"], None)


def test_no_workspace_host_checks():
    """The no-workspace step rejects a call whose workspace would exceed the
    built-in scratch array, and every host-argument error, before it touches
    the device (these calls need no GPU)."""
    ws = lib.pa_attention_workspace_size
    # 32 heads of 128 dims: a few hundred requests fit, ten thousand do not
    assert ws(256, 256, 32, 8, 128, 4096, 1, 0) <= pa.NO_WORKSPACE_MAX_BYTES
    assert ws(10000, 10000, 32, 8, 128, 4096, 1, 0) > pa.NO_WORKSPACE_MAX_BYTES
    big = dict(R=10000, T=10000, Q=1, L=4096, Hq=32, Hkv=8, D=128, stride=256)
    assert no_workspace(**big) == SCRATCH
    assert no_workspace(**big, S=3) == SCRATCH
    assert ws(10000, 10000, 32, 8, 128, 4096, 1, 3) > pa.NO_WORKSPACE_MAX_BYTES
    assert no_workspace(out=None) == INVALID
    assert no_workspace(k=None) == INVALID
    assert no_workspace(qsl=None) == INVALID
    assert no_workspace(B=8) == UNSUPPORTED
    assert no_workspace(D=256) == UNSUPPORTED
    assert no_workspace(Hq=6) == UNSUPPORTED
    assert no_workspace(S=-1) == INVALID
    assert no_workspace(R=0, T=0) == OK                        # nothing to launch
    assert no_workspace(T=0, k=None, v=None) == OK


def shared_prefix(**kw):
    a = dict(out=FAKE, q=FAKE, kv=FAKE, NB=64, B=16, Hkv=2, D=64, dtype=1, bt=FAKE, stride=7,
             sl=FAKE, R=4, L=100, Hq=4, scale=0.125, P=2, ws=FAKE_WS, wsb=1 << 30, S=0)
    a.update(kw)
    return lib.pa_attention_decode_shared_prefix(
        a["out"], a["q"], a["kv"], a["NB"], a["B"], a["Hkv"], a["D"], a["dtype"], a["bt"],
        a["stride"], a["sl"], a["R"], a["L"], a["Hq"], a["scale"], a["P"], a["ws"], a["wsb"],
        a["S"], None)


def test_shared_prefix_checks():
    f = lib.pa_attention_decode_shared_prefix_workspace_size
    assert f(4, 4, 2, 64, 100, 2, 0) > 0
    assert f(4, 4, 2, 64, 100, 2, 0) >= f(4, 4, 2, 64, 100, 0, 0)  # covers the plain plan
    assert f(4, 4, 2, 64, 100, -1, 0) == 0
    assert f(4, 4, 2, 64, 100, 7, 0) == 0                          # 16 P > max_seq_len
    assert shared_prefix(P=-1) == INVALID
    assert shared_prefix(P=7) == INVALID                           # prefix longer than L
    assert shared_prefix(q=None) == INVALID
    assert shared_prefix(ws=None) == WORKSPACE
    assert shared_prefix(wsb=16) == WORKSPACE
    assert shared_prefix(R=0) == OK


def test_cache_and_attend_shared_prefix_checks():
    f = lib.pa_cache_and_attend_decode_shared_prefix

    def call(**kw):
        a = dict(out=FAKE, q=FAKE, k=FAKE, v=FAKE, kv=FAKE, NB=64, B=16, Hkv=2, D=64, dtype=1,
                 bt=FAKE, stride=7, sl=FAKE, slots=None, R=4, L=100, Hq=4, scale=0.125, P=2,
                 ws=FAKE_WS, wsb=1 << 30, S=0)
        a.update(kw)
        return f(a["out"], a["q"], a["k"], a["v"], a["kv"], a["NB"], a["B"], a["Hkv"], a["D"],
                 a["dtype"], a["bt"], a["stride"], a["sl"], a["slots"], a["R"], a["L"], a["Hq"],
                 a["scale"], a["P"], a["ws"], a["wsb"], a["S"], None)
    assert call(k=None) == INVALID
    assert call(v=ctypes.c_void_p(0x10008)) == INVALID          # not 16-byte aligned
    assert call(P=-1) == INVALID
    assert call(P=7) == INVALID                                  # prefix longer than L
    assert call(q=None) == INVALID
    assert call(ws=None) == WORKSPACE
    assert call(B=8) == UNSUPPORTED
    assert call(R=0, k=None, v=None) == OK


def test_plan_follows_device_geometry():
    """The split is planned from the device's CU count: 3 wavefronts per CU
    over the KV heads, beside concurrent tiles the slots they leave (4-6
    waves per CU), never ranges under 4 blocks; a fixed split is kept as
    given."""
    f = pa.pa_plan_decode_ranges
    for cus in (256, 304, 128, 80, 64, 32):
        assert f(64, 32, 8, 128, "bf16", 4096, num_cus=cus) == cus * 3 // 8   # decode rows alone
        beside = f(64, 32, 8, 128, "bf16", 2048, max_query_len=512, num_cus=cus)
        assert cus * 4 // 8 <= beside <= cus * 6 // 8
        assert f(64, 32, 8, 128, "bf16", 4096, num_splits=7, num_cus=cus) == 7
    # the partitioned device gets proportionally fewer ranges
    assert f(64, 32, 8, 128, "bf16", 4096, num_cus=32) * 8 == f(64, 32, 8, 128, "bf16", 4096,
                                                               num_cus=256)
    # fp32 rows of 128 dims take two query heads per wave: twice the waves per
    # KV head, half the ranges
    assert f(64, 32, 8, 128, "f32", 4096, num_cus=256) == 48
    # short batches: no range under 4 blocks
    assert f(2, 32, 8, 128, "bf16", 64, num_cus=256) == 2
    with pytest.raises(pa.PAError):
        f(64, 32, 8, 128, "bf16", 4096, num_cus=0)
    with pytest.raises(pa.PAError):
        f(64, 30, 8, 128, "bf16", 4096)


def test_planned_mixed_checks():
    """The planned mixed entries reject plan fields out of range before any
    launch (null plan = library choice)."""
    plan_t = pa._MixedPlan

    def call(plan, **kw):
        a = dict(out=FAKE, q=FAKE, kv=FAKE, NB=64, B=16, Hkv=2, D=64, dtype=1, bt=FAKE,
                 stride=7, sl=FAKE, qsl=FAKE, nc=FAKE, R=4, T=20, Q=17, L=100, Hq=4,
                 scale=0.125, ws=FAKE_WS, wsb=16)
        a.update(kw)
        return lib.pa_attention_mixed_planned(
            a["out"], a["q"], a["kv"], a["NB"], a["B"], a["Hkv"], a["D"], a["dtype"], a["bt"],
            a["stride"], a["sl"], a["qsl"], a["nc"], a["R"], a["T"], a["Q"], a["L"], a["Hq"],
            a["scale"], a["ws"], a["wsb"], None if plan is None else ctypes.byref(plan), None)
    assert call(plan_t(0, 2, -1)) == INVALID
    assert call(plan_t(0, -1, 3)) == INVALID
    assert call(plan_t(-1, -1, -1)) == INVALID
    assert call(plan_t(0, 1, 0)) == WORKSPACE        # valid plan: gets to the workspace check
    assert call(None) == WORKSPACE


def test_slot_mapping_checks():
    f = lib.pa_compute_slot_mapping
    assert f(None, FAKE, 7, FAKE, FAKE, 4, 4, 16, None) == INVALID
    assert f(FAKE, FAKE, 7, FAKE, FAKE, 4, 4, 32, None) == UNSUPPORTED
    assert f(FAKE, FAKE, 7, FAKE, FAKE, 0, 4, 16, None) == INVALID
    assert f(FAKE, FAKE, 7, FAKE, FAKE, 4, 0, 16, None) == OK


def test_binding_rejects_host_tensors():
    torch = pytest.importorskip("torch")
    kv = torch.zeros(4, 2, 16, 1, 64)
    k = torch.zeros(2, 1, 64)
    with pytest.raises(ValueError):
        pa.pa_reshape_and_cache(k, k, kv, torch.zeros(2, dtype=torch.int64))


def test_single_hip_runtime_in_process():
    """Importing the binding maps exactly one HIP runtime: torch's.  (With the
    library loaded before torch, two HIP/HSA runtimes shared the process and
    torch's device memory was handed to the wrong one.)"""
    code = ("import paged_kv_attention_07_amd, torch\n"
            "m = open('/proc/self/maps').read()\n"
            "print(len({l.split()[-1] for l in m.splitlines() if 'libamdhip64' in l}))\n")
    out = subprocess.run(["python", "-c", code], capture_output=True, text=True, cwd=ROOT,
                         check=True).stdout.strip()
    assert out == "1"


def test_engine_checks():
    """pa_engine_* validate their arguments before touching the GPU."""
    from paged_kv_attention_07_amd.engine import _Geometry
    from paged_kv_attention_07_amd.sched import _Config
    cfg = _Config(64, 16, 256, 8, 1024, 0, 1, 1)
    geo = _Geometry(32, 8, 128, 1, 0.088, 0)
    size = lib.pa_engine_device_bytes(ctypes.byref(cfg), ctypes.byref(geo))
    assert size > 0 and size % 256 == 0
    bad_cfg = _Config(64, 8, 256, 8, 1024, 0, 1, 1)            # block size 8
    assert lib.pa_engine_device_bytes(ctypes.byref(bad_cfg), ctypes.byref(geo)) == 0
    bad_geo = _Geometry(32, 8, 96, 1, 0.088, 0)                # head_dim 96
    assert lib.pa_engine_device_bytes(ctypes.byref(cfg), ctypes.byref(bad_geo)) == 0
    h = ctypes.c_void_p()
    assert lib.pa_engine_create(ctypes.byref(cfg), ctypes.byref(geo), None, FAKE_WS, size,
                                ctypes.byref(h)) == INVALID
    assert lib.pa_engine_create(ctypes.byref(cfg), ctypes.byref(geo), FAKE, FAKE_WS, 16,
                                ctypes.byref(h)) == WORKSPACE
    assert lib.pa_engine_create(ctypes.byref(cfg), ctypes.byref(geo), FAKE,
                                ctypes.c_void_p(0x100010), size, ctypes.byref(h)) == INVALID


def check_meta(**kw):
    a = dict(flags=FAKE, bt=FAKE, stride=7, sl=FAKE, qsl=FAKE, nc=FAKE, slots=None, R=4, T=20,
             Q=17, L=100, NB=64, B=16, P=0)
    a.update(kw)
    return lib.pa_check_metadata(a["flags"], a["bt"], a["stride"], a["sl"], a["qsl"], a["nc"],
                                 a["slots"], a["R"], a["T"], a["Q"], a["L"], a["NB"], a["B"],
                                 a["P"], None)


def test_check_metadata_host_checks():
    """Host arguments of the device metadata check are validated before any
    launch."""
    assert check_meta(flags=None) == INVALID
    assert check_meta(B=8) == UNSUPPORTED
    assert check_meta(R=-1) == INVALID and check_meta(T=-1) == INVALID
    assert check_meta(nc=None) == INVALID                # offsets without computed counts
    assert check_meta(qsl=None, nc=None) == INVALID      # decode batch: T must equal R
    assert check_meta(bt=None) == INVALID and check_meta(sl=None) == INVALID
    assert check_meta(P=8) == INVALID                    # prefix wider than the table
    assert check_meta(R=0) == INVALID                    # tokens without requests
    assert check_meta(R=0, T=0) == OK                    # nothing to check


def test_workspace_size_covers_every_shorter_call():
    """A buffer sized for (R, T, max_seq_len, max_query_len) serves any call
    within those bounds: the size never shrinks as a bound grows (a call
    with a shorter chunk leaves its decode rows more waves, so more ranges)."""
    ws = lib.pa_attention_workspace_size
    for hq, hkv, d in ((32, 8, 128), (8, 2, 64), (4, 4, 128), (64, 8, 128)):
        for R in (1, 2, 7, 64, 256, 1024):
            for L in (1, 17, 600, 4096, 32768):
                sizes = [ws(R, 4096, hq, hkv, d, L, q, 0) for q in (1, 2, 3, 17, 100, 512, 2048, 8192)]
                assert all(s > 0 for s in sizes)
                assert sizes == sorted(sizes), (hq, hkv, d, R, L, sizes)
                # and it covers the plans of smaller batches and shorter contexts
                for R2 in (1, max(1, R // 2), R):
                    for L2 in (1, max(1, L // 3), L):
                        assert ws(R2, 4096, hq, hkv, d, L2, 2, 0) <= ws(R, 4096, hq, hkv, d, L, 2, 0)
