"""The C-ABI library loads, exports every symbol include/mk.h declares, and
rejects bad arguments synchronously, before any HIP call (no GPU needed)."""
import ctypes as C
import os
import re

import pytest

from tile_pipelined_gemm_amd import mk

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x10000          # a 16-byte aligned, never dereferenced "device pointer"


@pytest.fixture(scope="module")
def lib():
    return mk.load()


def declared_symbols():
    text = open(os.path.join(ROOT, "include", "mk.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mk_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported(lib):
    decl = declared_symbols()
    assert set(decl) == set(mk.EXPORTS)
    for name in decl:
        assert hasattr(lib, name), name


def test_support_functions(lib):
    assert lib.mk_version() >= 1
    assert lib.mk_status_string(mk.MK_ERR_TIMEOUT) == b"watchdog timeout"
    assert mk.mk_tile_name(0) == "auto" and mk.mk_tile_name(1) == "256x256"
    assert [mk.mk_tile_name(i) for i in range(5, 12)] == ["256x256dma", "128x128dma", "256x128dma", "128x256dma",
                                                         "128x128dma8", "256x256dma_w8", "128x128pc"]
    assert mk.mk_tile_name(99) is None


def _ag(lib, R=2, m=64, K=128, N=64, c_dtype=mk.MK_BF16, arrival=None, ws_bytes=1 << 20, ws=FAKE,
        shards=None, launch=None):
    sh = (C.c_void_p * R)(*([FAKE] * R)) if shards is None else shards
    return lib.mk_ag_gemm(sh, R, m, K, FAKE, N, FAKE, c_dtype, FAKE, arrival, launch, ws, ws_bytes, None)


def test_ag_validation(lib):
    assert _ag(lib, R=0) == mk.MK_ERR_UNSUPPORTED
    assert _ag(lib, K=100) == mk.MK_ERR_UNSUPPORTED
    assert _ag(lib, N=12) == mk.MK_ERR_UNSUPPORTED
    assert _ag(lib, c_dtype=7) == mk.MK_ERR_INVALID
    assert _ag(lib, shards=(C.c_void_p * 2)(FAKE, None)) == mk.MK_ERR_INVALID
    assert _ag(lib, shards=(C.c_void_p * 2)(FAKE, FAKE + 2)) == mk.MK_ERR_INVALID   # misaligned
    assert _ag(lib, ws=None) == mk.MK_ERR_WORKSPACE
    assert _ag(lib, ws_bytes=16) == mk.MK_ERR_WORKSPACE
    assert b"workspace" in lib.mk_last_error()


@pytest.mark.parametrize("order,delays,n_units,unit_rows,withhold", [
    ([0, 0, 1, 2], None, 4, 32, -1),          # not a permutation
    ([0, 1, 2, 4], None, 4, 32, -1),          # id out of range
    ([0, 1, 2, 3], None, 4, 16, -1),          # does not cover M = 128
    ([0, 1, 2, 3], [0, 5, 2_000_000_000, 1], 4, 32, -1),   # delay above 1 s
    ([0, 1, 2, 3], None, 4, 32, 9),           # withheld unit out of range
])
def test_ag_schedule_rejected(lib, order, delays, n_units, unit_rows, withhold):
    arr, keep = mk.make_arrival(order, delays, unit_rows, withhold)
    arr.n_units = n_units
    assert _ag(lib, arrival=C.byref(arr)) == mk.MK_ERR_SCHEDULE


def test_ag_too_many_units(lib):
    arr, keep = mk.make_arrival(list(range(512)), None, 1)
    assert _ag(lib, R=4, m=128, arrival=C.byref(arr)) == mk.MK_ERR_UNSUPPORTED


def test_ag_bad_launch_options(lib):
    lau = mk.make_launch(mode=4)
    assert _ag(lib, launch=C.byref(lau)) == mk.MK_ERR_INVALID
    lau = mk.make_launch(copy_kib=-1)
    assert _ag(lib, launch=C.byref(lau)) == mk.MK_ERR_INVALID
    lau = mk.make_launch(queue_mode=3)
    assert _ag(lib, launch=C.byref(lau)) == mk.MK_ERR_INVALID
    lau = mk.make_launch(tile=42)
    rc = _ag(lib, launch=C.byref(lau))
    assert rc in (mk.MK_ERR_INVALID, mk.MK_ERR_HIP)   # device query may come first without a GPU


def test_valid_call_without_gpu_reports_hip_error(lib):
    # Everything validates; the first HIP call then fails cleanly (no device here).
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert _ag(lib) == mk.MK_ERR_HIP


def test_ag_workspace_holds_packed_a_for_a_single_tile_row(lib):
    # header + 256 unit counters; a single 128-row tile row with K % 128 == 0
    # adds the packed copy of A (128 x K bf16) at a 256-byte aligned offset
    base = lib.mk_ag_gemm_workspace(8, 1024, 8192, 3584, 0)
    assert base == 256 + 256 * 4
    assert lib.mk_ag_gemm_workspace(8, 16, 8192, 28672, 0) == 1280 + 128 * 8192 * 2
    assert lib.mk_ag_gemm_workspace(3, 40, 640, 392, 0) == 1280 + 128 * 640 * 2
    assert lib.mk_ag_gemm_workspace(1, 128, 256, 512, 0) == 1280 + 128 * 256 * 2
    assert lib.mk_ag_gemm_workspace(1, 129, 256, 512, 0) == base       # two tile rows
    assert lib.mk_ag_gemm_workspace(8, 16, 8192 + 64, 28672, 0) == base  # K % 128 != 0


def _ag_noalloc(lib, R=2, m=64, K=128, N=64, c_dtype=mk.MK_BF16, arrival=None, shards=None, launch=None):
    sh = (C.c_void_p * R)(*([FAKE] * R)) if shards is None else shards
    return lib.mk_ag_gemm_noalloc(sh, R, m, K, FAKE, N, FAKE, c_dtype, FAKE, arrival, launch, None)


def test_ag_noalloc_validation(lib):
    # the same argument checks as mk_ag_gemm, before any HIP call
    assert _ag_noalloc(lib, R=0) == mk.MK_ERR_UNSUPPORTED
    assert _ag_noalloc(lib, K=100) == mk.MK_ERR_UNSUPPORTED
    assert _ag_noalloc(lib, c_dtype=7) == mk.MK_ERR_INVALID
    assert _ag_noalloc(lib, shards=(C.c_void_p * 2)(FAKE, FAKE + 2)) == mk.MK_ERR_INVALID
    arr, keep = mk.make_arrival([0, 1, 1, 3], None, 32, -1)
    assert _ag_noalloc(lib, arrival=C.byref(arr)) == mk.MK_ERR_SCHEDULE
    # a withheld unit could only be reported through a workspace's status
    arr, keep = mk.make_arrival([0, 1, 2, 3], None, 32, 2)
    assert _ag_noalloc(lib, arrival=C.byref(arr)) == mk.MK_ERR_INVALID
    assert b"withhold" in lib.mk_last_error()
    lau = mk.make_launch(mode=4)
    assert _ag_noalloc(lib, launch=C.byref(lau)) == mk.MK_ERR_INVALID
    import torch
    if not torch.cuda.is_available():                  # valid: the first HIP call fails cleanly
        assert _ag_noalloc(lib) == mk.MK_ERR_HIP


def _rs(lib, M=512, K=64, N=64, R=4, out_dtype=mk.MK_F32, ws_bytes=1 << 24, partials=True, lau=None,
        arrival=None, landing=None):
    P = (C.c_void_p * R)(*([FAKE] * R))
    O = (C.c_void_p * R)(*([FAKE] * R))
    return lib.mk_gemm_rs(FAKE, FAKE, M, K, N, P if partials else None, R, O, out_dtype, arrival, landing, lau,
                          FAKE, ws_bytes, None)


def test_rs_validation(lib):
    assert _rs(lib, M=510) == mk.MK_ERR_INVALID              # M % R
    assert _rs(lib, K=60) == mk.MK_ERR_UNSUPPORTED
    assert _rs(lib, R=65) == mk.MK_ERR_UNSUPPORTED
    assert _rs(lib, out_dtype=5) == mk.MK_ERR_INVALID
    assert _rs(lib, partials=False) == mk.MK_ERR_INVALID
    assert _rs(lib, M=4 * 96) == mk.MK_ERR_UNSUPPORTED       # 96 rows per owner: not a tile multiple
    lau = mk.make_launch(tile=3)
    assert _rs(lib, lau=C.byref(lau)) == mk.MK_ERR_UNSUPPORTED   # 128 rows per owner: not a 256-row tile multiple
    lau = mk.make_launch(tile=1)
    assert _rs(lib, M=1024, lau=C.byref(lau)) == mk.MK_ERR_UNSUPPORTED   # register 256x256 tile not built for RS
    lau = mk.make_launch(tile=5)
    assert _rs(lib, M=1024, K=136, lau=C.byref(lau)) == mk.MK_ERR_UNSUPPORTED   # direct-to-LDS tile needs K % 128 == 0
    assert _rs(lib, ws_bytes=64) == mk.MK_ERR_WORKSPACE
    lau = mk.make_launch(n_reduce=-5)
    assert _rs(lib, lau=C.byref(lau)) == mk.MK_ERR_INVALID
    for qm in (-1, 2):                                        # 0 one queue, 1 per-XCD band queues
        lau = mk.make_launch(queue_mode=qm)
        assert _rs(lib, lau=C.byref(lau)) == mk.MK_ERR_INVALID, qm
        assert _ar(lib, lau=C.byref(lau)) == mk.MK_ERR_INVALID, qm


def _ar(lib, M=510, K=64, N=64, R=4, out_dtype=mk.MK_F32, ws_bytes=1 << 24, partials=True, lau=None, outs=True):
    P = (C.c_void_p * R)(*([FAKE] * R))
    O = (C.c_void_p * R)(*([FAKE] * R))
    return lib.mk_gemm_ar(FAKE, FAKE, M, K, N, P if partials else None, R, O if outs else None, out_dtype, None,
                          None, lau, FAKE, ws_bytes, None)


def test_ar_validation(lib):
    # M = 510 is not a multiple of R: fine for the all-reduce (the first HIP call then fails without a GPU)
    import torch
    if not torch.cuda.is_available():
        assert _ar(lib) == mk.MK_ERR_HIP
    assert _ar(lib, K=60) == mk.MK_ERR_UNSUPPORTED
    assert _ar(lib, R=65) == mk.MK_ERR_UNSUPPORTED
    assert _ar(lib, out_dtype=5) == mk.MK_ERR_INVALID
    assert _ar(lib, partials=False) == mk.MK_ERR_INVALID
    assert _ar(lib, outs=False) == mk.MK_ERR_INVALID
    lau = mk.make_launch(tile=1)
    assert _ar(lib, lau=C.byref(lau)) == mk.MK_ERR_UNSUPPORTED    # register 256x256 tile not built
    assert _ar(lib, ws_bytes=64) == mk.MK_ERR_WORKSPACE
    assert lib.mk_gemm_ar_workspace(8192, 3584, 8192, 8, mk.MK_F32) == lib.mk_gemm_rs_workspace(
        8192, 3584, 8192, 8, mk.MK_F32)


def _rs_arrival(n_units, unit_rows, order=None, delays=None, withhold=-1):
    order = list(range(n_units)) if order is None else order
    arr, keep = mk.make_arrival(order, delays, unit_rows, withhold)
    return C.byref(arr), keep


@pytest.mark.parametrize("order,delays,n_units,unit_rows,R,withhold", [
    ([0, 1, 2, 3, 4, 5], None, 6, 256, 4, -1),          # 3 peers x 2 blocks = 6 units: fine on the host
    ([0, 1, 2, 3, 4, 4], None, 6, 256, 4, -1),          # not a permutation
    ([0, 1, 2, 3, 4, 5], None, 6, 200, 4, -1),          # 6 x 200 rows != 3 x 512
    ([0, 1], None, 2, 512, 4, -1),                      # 2 units of 512 rows: 3 peers need 3
    ([0, 1, 2, 3, 4, 5], [0, 0, 0, 2_000_000_000, 0, 0], 6, 256, 4, -1),   # delay over 1 s
    ([0, 1, 2, 3, 4, 5], None, 6, 256, 4, 6),           # withheld unit out of range
    ([0, 1, 2, 3], None, 4, 384, 4, -1),                # 4 x 384 = 3 x 512 rows but 384 does not divide M
    ([0], None, 1, 512, 1, -1),                         # R = 1: no partial sums to schedule
])
def test_rs_schedule_rejected(lib, order, delays, n_units, unit_rows, R, withhold):
    M = 512
    arr, keep = _rs_arrival(n_units, unit_rows, order, delays, withhold)
    if order == [0, 1, 2, 3, 4, 5] and delays is None and withhold == -1 and unit_rows == 256:
        import torch
        if torch.cuda.is_available():
            pytest.skip("a GPU is present")
        assert _rs(lib, M=M, R=R, arrival=arr) == mk.MK_ERR_HIP   # valid: only the first HIP call fails
        return
    assert _rs(lib, M=M, R=R, arrival=arr) == mk.MK_ERR_SCHEDULE


def test_rs_landing_rules(lib):
    L = (C.c_void_p * 3)(*([FAKE] * 3))
    assert _rs(lib, landing=L) == mk.MK_ERR_INVALID                 # landing buffers need a schedule
    arr, keep = _rs_arrival(6, 256)
    bad = (C.c_void_p * 3)(FAKE, None, FAKE)
    assert _rs(lib, arrival=arr, landing=bad) == mk.MK_ERR_INVALID  # a NULL landing buffer
    mis = (C.c_void_p * 3)(FAKE, FAKE + 4, FAKE)
    assert _rs(lib, arrival=arr, landing=mis) == mk.MK_ERR_INVALID  # misaligned
    lau = mk.make_launch(n_copy=-1)
    assert _rs(lib, arrival=arr, lau=C.byref(lau)) == mk.MK_ERR_INVALID
    lau = mk.make_launch(mode=2)                                   # one phase alone: no schedule
    assert _rs(lib, arrival=arr, lau=C.byref(lau)) == mk.MK_ERR_INVALID
    lau = mk.make_launch(mode=4)
    assert _rs(lib, lau=C.byref(lau)) == mk.MK_ERR_INVALID


def test_peak_probe_validation(lib):
    f, n, b = C.c_double(0), C.c_int(0), C.c_double(0)
    assert lib.mk_peak_mfma(0, FAKE, 1 << 20, C.byref(f), C.byref(n), None) == mk.MK_ERR_INVALID
    assert lib.mk_peak_mfma(10, None, 1 << 20, C.byref(f), C.byref(n), None) == mk.MK_ERR_WORKSPACE
    assert lib.mk_peak_hbm(FAKE, FAKE, 1 << 30, 2, FAKE, 4096, C.byref(b), None) == mk.MK_ERR_INVALID
    assert lib.mk_peak_hbm(None, FAKE, 1 << 30, 0, FAKE, 4096, C.byref(b), None) == mk.MK_ERR_INVALID
    assert lib.mk_peak_hbm(FAKE, None, 1 << 30, 1, FAKE, 4096, C.byref(b), None) == mk.MK_ERR_INVALID
    assert lib.mk_peak_workspace() >= 256


def test_rs_workspace_sizes(lib):
    f32 = lib.mk_gemm_rs_workspace(8192, 3584, 8192, 8, mk.MK_F32)
    bf = lib.mk_gemm_rs_workspace(8192, 3584, 8192, 8, mk.MK_BF16)
    assert bf - f32 == 8192 * 8192 * 4


def _moe(lib, T=256, H=128, E=64, k=4, eb=0, L=8, F=128, y=mk.MK_BF16, arrival=None, lau=None, ws_bytes=1 << 24):
    W = (C.c_void_p * L)(*([FAKE] * L))
    return lib.mk_moe_dispatch_gemm(FAKE, FAKE, T, H, E, k, W, eb, L, F, FAKE, FAKE, FAKE, FAKE, FAKE,
                                    FAKE, FAKE, y, arrival, lau, FAKE, ws_bytes, None)


def test_moe_validation(lib):
    assert _moe(lib, k=65) == mk.MK_ERR_INVALID
    assert _moe(lib, k=17, E=64) == mk.MK_ERR_INVALID
    assert _moe(lib, E=2048) == mk.MK_ERR_UNSUPPORTED
    assert _moe(lib, eb=60, L=8) == mk.MK_ERR_INVALID
    assert _moe(lib, H=100) == mk.MK_ERR_UNSUPPORTED
    assert _moe(lib, L=0) == mk.MK_ERR_UNSUPPORTED
    assert _moe(lib, y=3) == mk.MK_ERR_INVALID
    assert _moe(lib, ws_bytes=100) == mk.MK_ERR_WORKSPACE
    # the receive buffer (T x H bf16) is read through 32-bit offsets
    assert _moe(lib, T=1 << 16, H=1 << 14) == mk.MK_ERR_UNSUPPORTED
    arr, keep = mk.make_arrival([0, 1, 1, 3], None, 64)
    assert _moe(lib, arrival=C.byref(arr)) == mk.MK_ERR_SCHEDULE
    # launch options are checked before any HIP call
    for bad in (dict(mode=4), dict(mode=-1), dict(grid=-1), dict(n_copy=-1), dict(queue_mode=6), dict(queue_mode=-1)):
        lau = mk.make_launch(**bad)
        assert _moe(lib, lau=C.byref(lau)) == mk.MK_ERR_INVALID, bad


def _ring(lib, R=4, H=2, S=300, D=128, o=mk.MK_BF16, recv=True, arrival=None, lau=None, ws_bytes=1 << 20):
    K = (C.c_void_p * R)(*([FAKE] * R))
    V = (C.c_void_p * R)(*([FAKE] * R))
    rv = FAKE if recv else None
    return lib.mk_ring_attn(FAKE, K, V, R, H, S, D, FAKE, o, rv, rv, arrival, lau, FAKE, ws_bytes, None)


def test_ring_validation(lib):
    import torch
    if not torch.cuda.is_available():
        assert _ring(lib) == mk.MK_ERR_HIP                      # valid: the first HIP call fails
        assert _ring(lib, R=1, recv=False) == mk.MK_ERR_HIP     # one rank needs no receive buffers
    assert _ring(lib, D=64) == mk.MK_ERR_UNSUPPORTED
    assert _ring(lib, R=0) == mk.MK_ERR_UNSUPPORTED
    assert _ring(lib, R=65) == mk.MK_ERR_UNSUPPORTED
    assert _ring(lib, H=0) == mk.MK_ERR_INVALID
    assert _ring(lib, S=0) == mk.MK_ERR_INVALID
    assert _ring(lib, H=40, R=8) == mk.MK_ERR_UNSUPPORTED    # 280 units > MK_MAX_UNITS
    assert _ring(lib, o=7) == mk.MK_ERR_INVALID
    assert _ring(lib, recv=False) == mk.MK_ERR_INVALID
    assert _ring(lib, ws_bytes=64) == mk.MK_ERR_WORKSPACE
    lau = mk.make_launch(mode=2)
    assert _ring(lib, lau=C.byref(lau)) == mk.MK_ERR_INVALID
    # arrival: a permutation of (R-1)*H units of one "row" each
    arr, keep = mk.make_arrival([0, 1, 2, 3, 4, 5], None, 1)
    if not torch.cuda.is_available():
        assert _ring(lib, arrival=C.byref(arr)) == mk.MK_ERR_HIP
    arr, keep = mk.make_arrival([0, 1, 2, 3, 4, 4], None, 1)
    assert _ring(lib, arrival=C.byref(arr)) == mk.MK_ERR_SCHEDULE
    arr, keep = mk.make_arrival([0, 1, 2, 3, 4], None, 1)
    assert _ring(lib, arrival=C.byref(arr)) == mk.MK_ERR_SCHEDULE
    arr, keep = mk.make_arrival([0, 1, 2], None, 2)
    assert _ring(lib, arrival=C.byref(arr)) == mk.MK_ERR_SCHEDULE
    arr, keep = mk.make_arrival([0], None, 1)
    assert _ring(lib, R=1, recv=False, arrival=C.byref(arr)) == mk.MK_ERR_SCHEDULE
    assert lib.mk_ring_attn_workspace(16, 4096, 8) >= 256 + 4 * 112


def _combine(lib, T=64, E=32, k=4, eb=0, L=8, rows=256, F=64, o=mk.MK_BF16, ws_bytes=1 << 20, yl=True):
    return lib.mk_moe_combine(FAKE, T, E, k, FAKE, FAKE, FAKE, eb, L, FAKE if yl else None, rows, FAKE, F, FAKE, o,
                              FAKE, ws_bytes, None)


def test_moe_combine_validation(lib):
    import torch
    if not torch.cuda.is_available():
        assert _combine(lib) == mk.MK_ERR_HIP                   # valid: the first HIP call fails
    assert _combine(lib, yl=False) == mk.MK_ERR_INVALID
    assert _combine(lib, T=0) == mk.MK_ERR_INVALID
    assert _combine(lib, k=0) == mk.MK_ERR_INVALID
    assert _combine(lib, k=17, E=64) == mk.MK_ERR_INVALID
    assert _combine(lib, E=2000) == mk.MK_ERR_UNSUPPORTED
    assert _combine(lib, eb=30, L=8) == mk.MK_ERR_INVALID
    assert _combine(lib, F=60) == mk.MK_ERR_UNSUPPORTED
    assert _combine(lib, o=9) == mk.MK_ERR_INVALID
    assert _combine(lib, ws_bytes=16) == mk.MK_ERR_WORKSPACE
    assert lib.mk_moe_combine_workspace(4096, 8) == 4096 * 8 * 4


def _run_py(code):
    import subprocess
    import sys
    return subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True, timeout=300)


def test_load_binds_to_torch_hip_runtime():
    # mk.load() imports torch first, so one HIP runtime is mapped
    r = _run_py("from tile_pipelined_gemm_amd import mk; mk.load(); print(mk._hip_runtimes_mapped())")
    assert r.returncode == 0, r.stderr
    assert r.stdout.count("libamdhip64") == 1, r.stdout


def test_load_after_foreign_runtime_raises():
    # the library loaded before torch by other code: two runtimes are mapped,
    # and mk.load() refuses instead of letting the first call fail
    r = _run_py("import ctypes; ctypes.CDLL('tile_pipelined_gemm_amd/libmk.so'); "
                "from tile_pipelined_gemm_amd import mk; mk.load()")
    assert r.returncode != 0
    assert "two HIP runtimes" in r.stderr


def test_moe_gate_validation(lib):
    g = lambda T=256, H=256, E=64, x=FAKE, ws=FAKE, wb=1 << 26: lib.mk_moe_gate(x, FAKE, T, H, E, FAKE, ws, wb, None)
    assert g(T=0) == mk.MK_ERR_INVALID
    assert g(H=4) == mk.MK_ERR_INVALID
    assert g(H=100) == mk.MK_ERR_UNSUPPORTED
    assert g(E=12) == mk.MK_ERR_UNSUPPORTED
    assert g(E=2048) == mk.MK_ERR_UNSUPPORTED
    assert g(x=None) == mk.MK_ERR_INVALID
    assert g(x=FAKE + 2) == mk.MK_ERR_INVALID
    assert g(ws=None) == mk.MK_ERR_WORKSPACE
    import torch
    if not torch.cuda.is_available():
        assert g() == mk.MK_ERR_HIP                                 # valid: the device query fails
    assert lib.mk_moe_gate_workspace(4096, 7168, 256) >= 256


def test_plan_reports_the_per_shape_defaults(lib):
    # the five workloads' shapes (no GPU here: the AG item size assumes 256 CUs)
    ag = mk.mk_plan(mk.MK_OP_AG_GEMM, 8192, 3584, 8192, 8)
    assert (ag.tile, ag.copy_kib, ag.n_copy, ag.n_reduce, ag.queue_mode) == (mk.TILE_256x256_DMA_W8, 512, 0, 0, 0)
    sk = mk.mk_plan(mk.MK_OP_AG_GEMM, 128, 28672, 8192, 8)
    assert (sk.tile, sk.copy_kib) == (mk.TILE_128x128_PC, 16)          # one 16 KiB row per item
    assert mk.mk_plan(mk.MK_OP_AG_GEMM, 256, 96, 128, 4).tile == mk.TILE_128x128
    # below one round of 256x256 tiles the half-size direct-to-LDS tile spreads the work
    for M, N, K in [(1024, 3584, 8192), (2048, 3584, 8192), (2048, 4096, 4096), (3072, 2048, 8192)]:
        assert mk.mk_plan(mk.MK_OP_AG_GEMM, M, N, K, 8).tile == mk.TILE_128x256_DMA, (M, N, K)
    for M, N, K in [(4096, 3584, 8192), (4096, 8192, 4096), (4096, 4352, 512)]:
        assert mk.mk_plan(mk.MK_OP_AG_GEMM, M, N, K, 8).tile == mk.TILE_256x256_DMA_W8, (M, N, K)
    assert mk.mk_plan(mk.MK_OP_AG_GEMM, 1024, 3584, 8200, 8).tile == mk.TILE_128x128   # K % 128 != 0
    assert mk.mk_plan(mk.MK_OP_AG_GEMM, 128, 28672, 8192 + 128, 8).tile == mk.TILE_128x128_PC
    assert mk.mk_plan(mk.MK_OP_AG_GEMM, 128, 28672, 8192 + 64, 8).tile == mk.TILE_128x128
    rs = mk.mk_plan(mk.MK_OP_GEMM_RS, 8192, 8192, 3584, 8)
    assert (rs.tile, rs.copy_kib) == (mk.TILE_256x256_DMA, 1024)
    assert mk.mk_plan(mk.MK_OP_GEMM_RS, 8192 - 1024, 8192, 3584, 7).tile == mk.TILE_256x256_DMA
    assert mk.mk_plan(mk.MK_OP_GEMM_RS, 8 * 200, 512, 384, 8).tile == mk.TILE_128x128   # 200-row owner blocks
    assert mk.mk_plan(mk.MK_OP_GEMM_AR, 8 * 200, 512, 384, 8).tile == mk.TILE_128x256_DMA  # 14 tiles: spread
    # below one round of 256x256 tiles the 128x256 tile spreads the work
    assert mk.mk_plan(mk.MK_OP_GEMM_RS, 2048, 4096, 4096, 8).tile == mk.TILE_128x256_DMA
    assert mk.mk_plan(mk.MK_OP_GEMM_AR, 2048, 4096, 4096, 8).tile == mk.TILE_128x256_DMA
    assert mk.mk_plan(mk.MK_OP_GEMM_RS, 4096, 4096, 3584, 8).tile == mk.TILE_256x256_DMA
    assert mk.mk_plan(mk.MK_OP_GEMM_RS, 8 * 384, 8192, 512, 8).tile == mk.TILE_128x256_DMA   # 384-row owners
    assert mk.mk_plan(mk.MK_OP_MOE, 0, 2048, 7168).tile == mk.TILE_256x256_DMA
    assert mk.mk_plan(mk.MK_OP_MOE, 0, 200, 384).tile == mk.TILE_128x128
    assert mk.mk_plan(mk.MK_OP_MOE, 0, 2048, 136).tile == mk.TILE_256x256
    assert [mk.mk_plan(7, 1, 1, 1, 1, check=False), mk.mk_plan(0, 0, 1, 1, 1, check=False),
            mk.mk_plan(1, 8, 8, 8, 0, check=False)] == [mk.MK_ERR_INVALID] * 3
    assert lib.mk_plan(0, 8, 8, 8, 1, None) == mk.MK_ERR_INVALID


def _greedy_finish(wide, narrow, grid, cost=0.8):
    """Finishing time of the one tile queue on `grid` workgroups, simulated
    tile by tile: wide tiles (cost 1) first, then narrow ones, each taken by
    the first free workgroup."""
    import heapq
    free = [0.0] * grid
    end = 0.0
    for c in [1.0] * wide + [cost] * narrow:
        t = heapq.heappop(free) + c
        end = max(end, t)
        heapq.heappush(free, t)
    return end


def _column_plan(M, N, grid):
    tm, a0 = -(-M // 256), -(-N // 256)
    if tm * a0 > 8 * grid:
        return (a0, 0), False
    best, plan, close = _greedy_finish(tm * a0, 0, grid), (a0, 0), False
    for a in range(a0 - 1, max(-1, a0 - 65), -1):
        b = -(-(N - 256 * a) // 192)
        m = _greedy_finish(tm * a, tm * b, grid)
        close |= abs(m - 0.97 * best) < 1e-9
        if m < 0.97 * best:
            best, plan = m, (a, b)
    return plan, close


def test_ag_column_plan(lib):
    # the AG workload on 256 workgroups: 8 wide and 8 narrow tiles per tile row
    assert mk.mk_ag_column_plan(8192, 3584, 256) == (8, 8)
    assert 8 * 256 + 8 * 192 == 3584
    # on fewer workgroups, or other widths (the GPU tests run these)
    assert mk.mk_ag_column_plan(2048, 3584, 64) == (8, 8)
    assert mk.mk_ag_column_plan(2048, 3000, 64) == (0, 16)
    assert mk.mk_ag_column_plan(4096, 4352, 256) == (14, 4)         # 14 x 256 + 4 x 192 = 4352
    # fewer tiles than workgroups: 19 narrow tiles per row spread the work over
    # 152 workgroups instead of 112; many rounds: the plan is not searched
    assert mk.mk_ag_column_plan(2048, 3584, 256) == (0, 19)
    assert mk.mk_ag_column_plan(65536, 3584, 256) == (14, 0)
    assert mk.mk_ag_column_plan(8192, 2048, 256) == (8, 0)           # 256 tiles: one full round
    # every plan covers N with no empty tile and matches a tile-by-tile
    # simulation of the queue (shapes whose comparison is a tie are skipped)
    import random
    rng = random.Random(7)
    for _ in range(150):
        M, N, grid = 256 * rng.randint(1, 48), 8 * rng.randint(1, 900), rng.choice([16, 64, 100, 256])
        a, b = mk.mk_ag_column_plan(M, N, grid)
        assert 256 * a + 192 * b >= N and (b == 0 or 256 * a + 192 * (b - 1) < N) and 256 * a < N + 256
        want, close = _column_plan(M, N, grid)
        if not close:
            assert (a, b) == want, (M, N, grid)
    for bad in [(0, 8, 1), (8, 0, 1), (8, 8, 0)]:
        assert mk.mk_ag_column_plan(*bad, check=False) == mk.MK_ERR_INVALID
    assert lib.mk_ag_column_plan(8, 8, 1, None, None) == mk.MK_ERR_INVALID


def test_litmus_validation(lib):
    assert lib.mk_litmus_workspace(4, 1024) == 256 + 4 * 4 + 4 * 4 + 4 * 8 + (256 - (256 + 64) % 256) % 256 + 4 * 1024 * 4 \
        or lib.mk_litmus_workspace(4, 1024) >= 256 + 4 * 1024 * 4
    ws = lib.mk_litmus_workspace(4, 1024)
    assert lib.mk_litmus_mp(0, 1024, 10, 1, FAKE, FAKE, ws, 0, None) == mk.MK_ERR_INVALID       # pairs
    assert lib.mk_litmus_mp(65, 1024, 10, 1, FAKE, FAKE, ws, 0, None) == mk.MK_ERR_INVALID
    assert lib.mk_litmus_mp(4, 0, 10, 1, FAKE, FAKE, ws, 0, None) == mk.MK_ERR_INVALID          # words
    assert lib.mk_litmus_mp(4, 1024, 0, 1, FAKE, FAKE, ws, 0, None) == mk.MK_ERR_INVALID        # rounds
    assert lib.mk_litmus_mp(4, 1024, 10, 2, FAKE, FAKE, ws, 0, None) == mk.MK_ERR_INVALID       # fenced
    assert lib.mk_litmus_mp(4, 1024, 10, 1, None, FAKE, ws, 0, None) == mk.MK_ERR_INVALID       # result
    assert lib.mk_litmus_mp(4, 1024, 10, 1, FAKE, FAKE, ws - 4, 0, None) == mk.MK_ERR_WORKSPACE
