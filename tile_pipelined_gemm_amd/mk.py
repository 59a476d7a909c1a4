"""Thin ctypes binding of libmk.so (declared in include/mk.h).

Every function here only marshals arguments -- torch tensors become device
pointers, Python lists become host pointer arrays, the current torch stream
becomes the hipStream_t -- and calls the C entry point of the same name.  All
computation runs in the HIP kernels of libmk.so; there is no fallback: if the
library is missing, ``load()`` raises.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Optional, Sequence

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmk.so")

MK_BF16, MK_F32 = 0, 1
MK_OK, MK_ERR_INVALID, MK_ERR_UNSUPPORTED, MK_ERR_WORKSPACE, MK_ERR_HIP, MK_ERR_TIMEOUT, MK_ERR_SCHEDULE = \
    0, -1, -2, -3, -4, -5, -6
MK_MAX_UNITS = 256
TILE_256x256, TILE_128x128, TILE_256x128, TILE_128x256, TILE_256x256_DMA = 1, 2, 3, 4, 5
TILE_128x128_DMA, TILE_256x128_DMA, TILE_128x256_DMA = 6, 7, 8
TILE_128x128_DMA8 = 9
TILE_256x256_DMA_W8 = 10
TILE_128x128_PC = 11

# Symbols declared in include/mk.h (checked by the CPU tests).
EXPORTS = [
    "mk_ag_gemm_workspace", "mk_ag_gemm", "mk_ag_gemm_noalloc", "mk_gemm_rs_workspace", "mk_gemm_rs",
    "mk_gemm_ar_workspace", "mk_gemm_ar",
    "mk_moe_dispatch_gemm_workspace", "mk_moe_dispatch_gemm", "mk_moe_combine_workspace", "mk_moe_combine",
    "mk_moe_gate_workspace", "mk_moe_gate",
    "mk_ring_attn_workspace", "mk_ring_attn",
    "mk_workspace_init",
    "mk_poll_status", "mk_status_string", "mk_last_error", "mk_tile_name", "mk_version", "mk_plan",
    "mk_ag_column_plan",
    "mk_wall_clock_khz", "mk_peak_workspace", "mk_peak_mfma", "mk_peak_hbm", "mk_litmus_workspace", "mk_litmus_mp",
]


class MkError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"mk error {code}: {msg}")
        self.code = code


class mk_arrival(C.Structure):
    _fields_ = [("order", C.POINTER(C.c_int32)), ("delay_ns", C.POINTER(C.c_uint32)),
                ("n_units", C.c_int32), ("unit_rows", C.c_int32), ("withhold", C.c_int32)]


class mk_launch(C.Structure):
    _fields_ = [("mode", C.c_int32), ("grid", C.c_int32), ("n_copy", C.c_int32),
                ("n_reduce", C.c_int32), ("tile", C.c_int32), ("spin_limit_us", C.c_uint32),
                ("tile_log", C.c_void_p), ("copy_kib", C.c_int32), ("copy_policy", C.c_int32),
                ("copy_log", C.c_void_p), ("queue_mode", C.c_int32)]


_lib = None


def _hip_runtimes_mapped():
    """Distinct HIP runtime files mapped into this process (Linux)."""
    try:
        with open("/proc/self/maps") as f:
            return sorted({ln.split()[-1] for ln in f if "libamdhip64" in ln})
    except OSError:
        return []


def load(path: Optional[str] = None):
    """Load libmk.so (once).  Raises if it has not been built.

    torch is imported first: it carries its own HIP runtime, and libmk.so must
    bind to that same runtime (the dynamic loader reuses an already loaded
    libamdhip64.so.7).  Loaded the other way round, the process would map two
    runtimes, and the streams and device pointers torch hands over would be
    foreign to the one libmk calls (stream synchronisation then fails).  The
    check after loading turns that state into an error instead of a failed
    first call.
    """
    global _lib
    if _lib is not None:
        return _lib
    path = path or LIB_PATH
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: run `python -m tile_pipelined_gemm_amd.build`")
    import torch  # noqa: F401  (binds the process to torch's HIP runtime first)
    lib = C.CDLL(path)
    runtimes = _hip_runtimes_mapped()
    if len(runtimes) > 1:
        raise RuntimeError("two HIP runtimes are mapped into this process " + ", ".join(runtimes) +
                           ": libmk.so was loaded before torch by other code; import torch first")
    vp, i32, i64, sz = C.c_void_p, C.c_int, C.c_int64, C.c_size_t
    pp = C.POINTER(C.c_void_p)
    lib.mk_ag_gemm_workspace.restype = sz
    lib.mk_ag_gemm_workspace.argtypes = [i32, i64, i64, i64, C.c_int32]
    lib.mk_ag_gemm.restype = i32
    lib.mk_ag_gemm.argtypes = [pp, i32, i64, i64, vp, i64, vp, i32, vp,
                               C.POINTER(mk_arrival), C.POINTER(mk_launch), vp, sz, vp]
    lib.mk_ag_gemm_noalloc.restype = i32
    lib.mk_ag_gemm_noalloc.argtypes = [pp, i32, i64, i64, vp, i64, vp, i32, vp,
                                       C.POINTER(mk_arrival), C.POINTER(mk_launch), vp]
    lib.mk_gemm_rs_workspace.restype = sz
    lib.mk_gemm_rs_workspace.argtypes = [i64, i64, i64, i32, i32]
    lib.mk_gemm_rs.restype = i32
    lib.mk_gemm_rs.argtypes = [vp, vp, i64, i64, i64, pp, i32, pp, i32,
                               C.POINTER(mk_arrival), pp, C.POINTER(mk_launch), vp, sz, vp]
    lib.mk_gemm_ar_workspace.restype = sz
    lib.mk_gemm_ar_workspace.argtypes = [i64, i64, i64, i32, i32]
    lib.mk_gemm_ar.restype = i32
    lib.mk_gemm_ar.argtypes = [vp, vp, i64, i64, i64, pp, i32, pp, i32,
                               C.POINTER(mk_arrival), pp, C.POINTER(mk_launch), vp, sz, vp]
    lib.mk_moe_dispatch_gemm_workspace.restype = sz
    lib.mk_moe_dispatch_gemm_workspace.argtypes = [i64, i64, i32, i32, i32, i64]
    lib.mk_moe_dispatch_gemm.restype = i32
    lib.mk_moe_dispatch_gemm.argtypes = [vp, vp, i64, i64, i32, i32, pp, i32, i32, i64,
                                         vp, vp, vp, vp, vp, vp, vp, i32,
                                         C.POINTER(mk_arrival), C.POINTER(mk_launch), vp, sz, vp]
    lib.mk_moe_gate_workspace.restype = sz
    lib.mk_moe_gate_workspace.argtypes = [i64, i64, i32]
    lib.mk_moe_gate.restype = i32
    lib.mk_moe_gate.argtypes = [vp, vp, i64, i64, i32, vp, vp, sz, vp]
    lib.mk_moe_combine_workspace.restype = sz
    lib.mk_moe_combine_workspace.argtypes = [i64, i32]
    lib.mk_moe_combine.restype = i32
    lib.mk_moe_combine.argtypes = [vp, i64, i32, i32, vp, vp, vp, i32, i32, vp, i64, vp, i64, vp, i32, vp, sz, vp]
    lib.mk_ring_attn_workspace.restype = sz
    lib.mk_ring_attn_workspace.argtypes = [i32, i64, i32]
    lib.mk_ring_attn.restype = i32
    lib.mk_ring_attn.argtypes = [vp, pp, pp, i32, i32, i64, i32, vp, i32, vp, vp,
                                 C.POINTER(mk_arrival), C.POINTER(mk_launch), vp, sz, vp]
    lib.mk_workspace_init.restype = i32
    lib.mk_workspace_init.argtypes = [vp, sz, vp]
    lib.mk_poll_status.restype = i32
    lib.mk_poll_status.argtypes = [vp, vp]
    lib.mk_status_string.restype = C.c_char_p
    lib.mk_status_string.argtypes = [i32]
    lib.mk_last_error.restype = C.c_char_p
    lib.mk_last_error.argtypes = []
    lib.mk_tile_name.restype = C.c_char_p
    lib.mk_tile_name.argtypes = [i32]
    lib.mk_plan.restype = i32
    lib.mk_plan.argtypes = [i32, i64, i64, i64, i32, C.POINTER(mk_launch)]
    lib.mk_ag_column_plan.restype = i32
    lib.mk_ag_column_plan.argtypes = [i64, i64, i32, C.POINTER(C.c_int), C.POINTER(C.c_int)]
    lib.mk_version.restype = i32
    lib.mk_version.argtypes = []
    lib.mk_wall_clock_khz.restype = i32
    lib.mk_wall_clock_khz.argtypes = []
    lib.mk_peak_workspace.restype = sz
    lib.mk_peak_workspace.argtypes = []
    lib.mk_peak_mfma.restype = i32
    lib.mk_peak_mfma.argtypes = [i32, vp, sz, C.POINTER(C.c_double), C.POINTER(C.c_int), vp]
    lib.mk_litmus_workspace.restype = sz
    lib.mk_litmus_workspace.argtypes = [i32, i32]
    lib.mk_litmus_mp.restype = i32
    lib.mk_litmus_mp.argtypes = [i32, i32, i32, i32, vp, vp, sz, C.c_uint32, vp]
    lib.mk_peak_hbm.restype = i32
    lib.mk_peak_hbm.argtypes = [vp, vp, sz, i32, vp, sz, C.POINTER(C.c_double), vp]
    _lib = lib
    return lib


def _check(rc: int):
    if rc != MK_OK:
        raise MkError(rc, _lib.mk_last_error().decode())
    return rc


# ---------------------------------------------------------------- marshalling
def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _ptr_array(ts: Sequence) -> C.Array:
    return (C.c_void_p * max(1, len(ts)))(*[_ptr(t) for t in ts])


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return MK_BF16
    if t.dtype == torch.float32:
        return MK_F32
    raise ValueError(f"unsupported output dtype {t.dtype}")


def make_arrival(order=None, delay_ns=None, unit_rows=0, withhold=-1):
    """Build an mk_arrival from Python sequences (None when order is None)."""
    if order is None:
        return None, ()
    order = list(int(x) for x in order)
    o = (C.c_int32 * len(order))(*order)
    d = None
    if delay_ns is not None:
        d = (C.c_uint32 * len(order))(*[int(x) for x in delay_ns])
    a = mk_arrival(C.cast(o, C.POINTER(C.c_int32)),
                   C.cast(d, C.POINTER(C.c_uint32)) if d is not None else None,
                   len(order), int(unit_rows), int(withhold))
    return a, (o, d)


def mk_litmus_mp(pairs, words, rounds, *, fenced=True, spin_limit_us=0, stream=None, check=True):
    """Cross-XCD message-passing litmus run; returns (stale words, cross-XCD
    pairs, producer XCD mask, consumer XCD mask) or the error code."""
    import torch
    lib = load()
    ws = workspace(lib.mk_litmus_workspace(pairs, words))
    res = torch.zeros(4, dtype=torch.int32, device="cuda")
    rc = lib.mk_litmus_mp(pairs, words, rounds, 1 if fenced else 0, _ptr(res), _ptr(ws), ws.numel(), spin_limit_us,
                          _stream(stream))
    if rc != MK_OK:
        return _check(rc) if check else rc
    st = mk_poll_status(ws, stream)
    if st != MK_OK:
        return _check(st) if check else st
    return tuple(int(x) & 0xffffffff for x in res.cpu().tolist())


def mk_peak_mfma(iters, ws, *, stream=None):
    """Launch the MFMA-only loop; returns (flops of the launch, waves).  The
    per-wave {core ticks, wall ticks} pairs land in ws at byte 256."""
    f, n = C.c_double(0.0), C.c_int(0)
    _check(load().mk_peak_mfma(int(iters), _ptr(ws), ws.numel() * ws.element_size(), C.byref(f), C.byref(n),
                               _stream(stream)))
    return f.value, n.value


def mk_peak_hbm(src, dst, mode, ws, *, stream=None) -> float:
    """Launch the HBM read (mode 0) or copy (mode 1) stream over src's bytes;
    returns the bytes it moves (read plus written)."""
    b = C.c_double(0.0)
    _check(load().mk_peak_hbm(_ptr(src), _ptr(dst), src.numel() * src.element_size(), int(mode), _ptr(ws),
                              ws.numel() * ws.element_size(), C.byref(b), _stream(stream)))
    return b.value


def mk_wall_clock_khz() -> int:
    """Rate of the device wall clock that stamps the tile and copy logs (kHz)."""
    return _check_pos(load().mk_wall_clock_khz())


def _check_pos(v: int) -> int:
    if v < 0:
        raise MkError(v, load().mk_last_error().decode())
    return v


def make_launch(mode=0, grid=0, n_copy=0, n_reduce=0, tile=0, spin_limit_us=0, tile_log=None, copy_kib=0,
                copy_log=None, copy_policy=0, queue_mode=0):
    return mk_launch(mode, grid, n_copy, n_reduce, tile, spin_limit_us, _ptr(tile_log), copy_kib, copy_policy,
                     _ptr(copy_log), queue_mode)


# ---------------------------------------------------------------- entry points
def mk_ag_gemm_workspace(R, m_shard, K, N, unit_rows=0) -> int:
    return load().mk_ag_gemm_workspace(R, m_shard, K, N, unit_rows)


def mk_gemm_rs_workspace(M, K, N, R, out_dtype=MK_F32) -> int:
    return load().mk_gemm_rs_workspace(M, K, N, R, out_dtype)


def mk_moe_dispatch_gemm_workspace(T, H, E, k, L, F) -> int:
    return load().mk_moe_dispatch_gemm_workspace(T, H, E, k, L, F)


def mk_moe_gate_workspace(T, H, E) -> int:
    return load().mk_moe_gate_workspace(T, H, E)


def mk_moe_gate(X, W_gate, logits, ws, *, stream=None, check=True) -> int:
    """X [T, H] and W_gate [H, E] bf16; logits [T, E] float32 (written)."""
    T, H = X.shape
    E = W_gate.shape[1]
    rc = load().mk_moe_gate(_ptr(X), _ptr(W_gate), T, H, E, _ptr(logits), _ptr(ws), ws.numel() * ws.element_size(),
                            _stream(stream))
    return _check(rc) if check else rc


def mk_moe_combine_workspace(T, k) -> int:
    return load().mk_moe_combine_workspace(T, k)


def mk_moe_combine(logits, topk, offsets, perm, expert_begin, L, y_local, y_peer, out, ws, *, stream=None,
                   check=True) -> int:
    """logits [T, E] float32; topk [T, k], offsets [E+1], perm [T*k] int32 (the
    dispatch outputs); y_local [rows, F], y_peer [T*k, F] bf16; out [T, F]."""
    T, E = logits.shape
    k = topk.shape[1]
    F = out.shape[1]
    rc = load().mk_moe_combine(_ptr(logits), T, E, k, _ptr(topk), _ptr(offsets), _ptr(perm), expert_begin, L,
                               _ptr(y_local), y_local.shape[0], _ptr(y_peer), F, _ptr(out), _dtype_code(out),
                               _ptr(ws), ws.numel() * ws.element_size(), _stream(stream))
    return _check(rc) if check else rc


def mk_ring_attn_workspace(H, S, R) -> int:
    return load().mk_ring_attn_workspace(H, S, R)


def mk_ring_attn(Q, k_shards, v_shards, O, k_recv, v_recv, ws, *, order=None, delay_ns=None, withhold=-1,
                 launch=None, stream=None, check=True) -> int:
    """Q, k_shards[r], v_shards[r]: [H, S, 128] bf16; O: [H, S, 128] bf16 or
    float32; k_recv, v_recv: [(R-1), H, S, 128] bf16 receive buffers (None for
    R = 1)."""
    lib = load()
    R = len(k_shards)
    H, S, D = Q.shape
    arr, keep = make_arrival(order if R > 1 else None, delay_ns, 1, withhold)
    lau = launch if launch is not None else make_launch()
    rc = lib.mk_ring_attn(_ptr(Q), _ptr_array(k_shards), _ptr_array(v_shards), R, H, S, D, _ptr(O),
                          _dtype_code(O), _ptr(k_recv), _ptr(v_recv),
                          C.byref(arr) if arr is not None else None, C.byref(lau),
                          _ptr(ws), ws.numel() * ws.element_size(), _stream(stream))
    del keep
    return _check(rc) if check else rc


def mk_workspace_init(ws, stream=None):
    return _check(load().mk_workspace_init(_ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))


def mk_poll_status(ws, stream=None) -> int:
    """Synchronise and return the sticky device status (MK_OK or MK_ERR_TIMEOUT)."""
    return load().mk_poll_status(_ptr(ws), _stream(stream))


def mk_ag_gemm(shards, B, C_out, a_gathered, ws, *, order=None, delay_ns=None, unit_rows=0,
               withhold=-1, launch=None, stream=None, check=True) -> int:
    lib = load()
    R = len(shards)
    m_shard, K = shards[0].shape
    N = B.shape[1]
    arr, keep = make_arrival(order, delay_ns, unit_rows or m_shard, withhold)
    lau = launch if launch is not None else make_launch()
    rc = lib.mk_ag_gemm(_ptr_array(shards), R, m_shard, K, _ptr(B), N, _ptr(C_out), _dtype_code(C_out),
                        _ptr(a_gathered), C.byref(arr) if arr is not None else None, C.byref(lau),
                        _ptr(ws), ws.numel() * ws.element_size(), _stream(stream))
    del keep
    return _check(rc) if check else rc


def mk_ag_gemm_noalloc(shards, B, C_out, a_gathered, *, order=None, delay_ns=None, unit_rows=0, launch=None,
                       stream=None, check=True) -> int:
    """mk_ag_gemm with the library's built-in scratch instead of a workspace."""
    lib = load()
    R = len(shards)
    m_shard, K = shards[0].shape
    N = B.shape[1]
    arr, keep = make_arrival(order, delay_ns, unit_rows or m_shard, -1)
    lau = launch if launch is not None else make_launch()
    rc = lib.mk_ag_gemm_noalloc(_ptr_array(shards), R, m_shard, K, _ptr(B), N, _ptr(C_out), _dtype_code(C_out),
                                _ptr(a_gathered), C.byref(arr) if arr is not None else None, C.byref(lau),
                                _stream(stream))
    del keep
    return _check(rc) if check else rc


def _gemm_reduce(fn, A, B, partials, outs, ws, order, delay_ns, unit_rows, withhold, landing, launch, stream,
                 check):
    M, K = A.shape
    N = B.shape[1]
    R = len(outs)
    arr, keep = make_arrival(order, delay_ns, unit_rows, withhold)
    lau = launch if launch is not None else make_launch()
    land = _ptr_array(landing) if landing is not None else None
    rc = fn(_ptr(A), _ptr(B), M, K, N, _ptr_array(partials), R, _ptr_array(outs), _dtype_code(outs[0]),
            C.byref(arr) if arr is not None else None, land, C.byref(lau), _ptr(ws),
            ws.numel() * ws.element_size(), _stream(stream))
    del keep
    return _check(rc) if check else rc


def mk_gemm_rs(A, B, partials, out_owner, ws, *, order=None, delay_ns=None, unit_rows=0, withhold=-1,
               landing=None, launch=None, stream=None, check=True) -> int:
    """order/delay_ns/unit_rows: optional arrival schedule of the partial sums
    (units of unit_rows rows of one peer); landing: optional R-1 fp32 [M, N]
    buffers the copy workgroups move the units into."""
    return _gemm_reduce(load().mk_gemm_rs, A, B, partials, out_owner, ws, order, delay_ns, unit_rows, withhold,
                        landing, launch, stream, check)


def mk_gemm_ar_workspace(M, K, N, R, out_dtype=MK_F32) -> int:
    return load().mk_gemm_ar_workspace(M, K, N, R, out_dtype)


def mk_gemm_ar(A, B, partials, out_rank, ws, *, order=None, delay_ns=None, unit_rows=0, withhold=-1,
               landing=None, launch=None, stream=None, check=True) -> int:
    return _gemm_reduce(load().mk_gemm_ar, A, B, partials, out_rank, ws, order, delay_ns, unit_rows, withhold,
                        landing, launch, stream, check)


def mk_moe_dispatch_gemm(X, logits, W, k, expert_begin, topk_idx, counts, offsets, perm, n_local_rows,
                         Xs, Y, ws, *, order=None, delay_ns=None, block_tokens=0, withhold=-1,
                         launch=None, stream=None, check=True) -> int:
    lib = load()
    T, H = X.shape
    E = logits.shape[1]
    L = len(W)
    F = W[0].shape[1]
    # the receive buffer holds row t for token t; Y one row per local pair
    if Xs.numel() < T * H or Y.numel() < T * min(k, L) * F:
        raise ValueError(f"Xs needs {T} x {H} elements and Y {T * min(k, L)} x {F}")
    arr, keep = make_arrival(order, delay_ns, block_tokens, withhold)
    lau = launch if launch is not None else make_launch()
    rc = lib.mk_moe_dispatch_gemm(_ptr(X), _ptr(logits), T, H, E, k, _ptr_array(W), expert_begin, L, F,
                                  _ptr(topk_idx), _ptr(counts), _ptr(offsets), _ptr(perm), _ptr(n_local_rows),
                                  _ptr(Xs), _ptr(Y), _dtype_code(Y),
                                  C.byref(arr) if arr is not None else None, C.byref(lau),
                                  _ptr(ws), ws.numel() * ws.element_size(), _stream(stream))
    del keep
    return _check(rc) if check else rc


MK_OP_AG_GEMM, MK_OP_GEMM_RS, MK_OP_GEMM_AR, MK_OP_MOE = 0, 1, 2, 3


def mk_plan(op: int, M: int, N: int, K: int, R: int = 1, check=True):
    """The per-shape default launch of an operation (see include/mk.h); a
    mk_launch that can be passed back as `launch`."""
    out = mk_launch()
    rc = load().mk_plan(op, M, N, K, R, C.byref(out))
    if check:
        _check(rc)
    return out if rc == MK_OK else rc


def mk_ag_column_plan(M: int, N: int, grid: int, check=True):
    """(tn_wide, tn_narrow): the 256- and 192-wide column tiles per tile row
    that mk_ag_gemm uses with tile 10 on `grid` workgroups (see include/mk.h)."""
    a, b = C.c_int(), C.c_int()
    rc = load().mk_ag_column_plan(M, N, grid, C.byref(a), C.byref(b))
    if check:
        _check(rc)
    return (a.value, b.value) if rc == MK_OK else rc


def mk_tile_name(i: int):
    r = load().mk_tile_name(i)
    return r.decode() if r is not None else None


def workspace(nbytes: int, device="cuda"):
    """A zero-filled workspace tensor (bytes rounded up to 256)."""
    import torch
    nbytes = (int(nbytes) + 255) // 256 * 256
    return torch.zeros(nbytes, dtype=torch.uint8, device=device)
