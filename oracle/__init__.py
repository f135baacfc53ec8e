"""CPU oracle for the fused MoE FFN layer -- TEST INFRASTRUCTURE ONLY.

Only tests/, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never imports, links or calls it, and the oracle never
imports the product: the two share nothing but the seeded input generator.

The arithmetic lives in ``moe_oracle.c`` (plain C, fp64 accumulation; the
INT8 quantiser decides its codes in fp32 like the kernels do).  This wrapper
only compiles it with gcc when the shared object is missing or older than the
source, and marshals NumPy arrays through ctypes.

Pins: see the header of ``moe_oracle.c``; every function is pinned by a
``-m "not gpu"`` test.
"""
from __future__ import annotations

import concurrent.futures
import ctypes
import os
import subprocess
import threading

import numpy as np

_DIR = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_DIR, "moe_oracle.c")
_SO = os.path.join(_DIR, "liboracle.so")
_lock = threading.Lock()
_lib = None

BF16, FP8, INT8 = 0, 1, 2
INT4 = 3      # weight-only 4-bit codes [K, N/2] bytes, fp32 scales [K/128, N]
FP8_ACT8 = 4  # FP8 weights with FP8 (E4M3, per-128-block power-of-two) activations


def _inter(w13, wdtype: int) -> int:
    """Intermediate size I from a w13 array [.., H, 2I] (INT4: [.., H, I] bytes)."""
    return w13.shape[-1] if wdtype == INT4 else w13.shape[-1] // 2
SOFTMAX, SIGMOID = 0, 1


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (no fast-math, no FP contraction)."""
    if not force and os.path.exists(_SO) and os.path.getmtime(_SO) >= os.path.getmtime(_SRC):
        return _SO
    tmp = _SO + f".tmp{os.getpid()}"
    cmd = ["gcc", "-O2", "-fPIC", "-shared", "-std=c11", "-fno-fast-math", "-ffp-contract=off",
           "-Wall", "-Wno-unused-function", "-Wno-maybe-uninitialized", _SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _SO)
    return _SO


def _load():
    global _lib
    with _lock:
        if _lib is None:
            lib = ctypes.CDLL(build())
            P = ctypes.c_void_p
            i32, i64, f32, f64 = ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_double
            lib.oracle_bf16_to_double.argtypes = [ctypes.c_uint16]
            lib.oracle_bf16_to_double.restype = f64
            lib.oracle_e4m3fn_to_double.argtypes = [ctypes.c_uint8]
            lib.oracle_e4m3fn_to_double.restype = f64
            lib.oracle_double_to_bf16.argtypes = [f64]
            lib.oracle_double_to_bf16.restype = ctypes.c_uint16
            lib.oracle_quant_int8_row.argtypes = [P, i32, P, P]
            lib.oracle_quant_int8_row.restype = None
            lib.oracle_topk.argtypes = [P, i32, i32, i32, i32, i32, P, P]
            lib.oracle_topk.restype = i32
            lib.oracle_align_capacity.argtypes = [i64, i32, i32]
            lib.oracle_align_capacity.restype = i64
            lib.oracle_align.argtypes = [P, i64, i32, i32, P, P, P]
            lib.oracle_align.restype = i32
            lib.oracle_float_ffn.argtypes = [i32, P, i32, i32, P, P, P, P, P, P]
            lib.oracle_float_ffn.restype = None
            lib.oracle_int8_ffn.argtypes = [P, f32, i32, i32, P, P, P, P, P, P, P, P, P, P]
            lib.oracle_int8_ffn.restype = None
            lib.oracle_double_to_e4m3fn.argtypes = [f64]
            lib.oracle_double_to_e4m3fn.restype = ctypes.c_uint8
            lib.oracle_fp8_block_exponent.argtypes = [f64]
            lib.oracle_fp8_block_exponent.restype = i32
            lib.oracle_quant_fp8_act_row.argtypes = [P, i32, P, P, P]
            lib.oracle_quant_fp8_act_row.restype = None
            lib.oracle_float_ffn_act8.argtypes = [P, i32, i32, P, P, P, P, P, P]
            lib.oracle_float_ffn_act8.restype = None
            lib.oracle_int4_code.argtypes = [P, i32, i64, i64]
            lib.oracle_int4_code.restype = i32
            lib.oracle_moe.argtypes = [i32, P, i32, i32, i32, i32, i32, P, P, P, P, P, P, P, P,
                                       P, P, i32, P, i32, P, P]
            lib.oracle_moe.restype = i32
            _lib = lib
    return _lib


def _np(a, dtype):
    """Contiguous NumPy view/copy with the given dtype; accepts torch CPU tensors."""
    if a is None:
        return None
    if hasattr(a, "detach"):  # torch tensor -> numpy without importing torch here
        a = a.detach().cpu()
        if str(a.dtype) == "torch.bfloat16":
            import torch  # local: only for the bit view
            a = a.view(torch.uint16) if hasattr(torch, "uint16") else a.view(torch.int16)
        elif str(a.dtype) == "torch.float8_e4m3fn":
            import torch
            a = a.view(torch.uint8)
        a = a.numpy()
    a = np.asarray(a)
    if a.dtype != np.dtype(dtype):
        if np.dtype(dtype).itemsize == a.dtype.itemsize and a.dtype.kind in "iu" and \
                np.dtype(dtype).kind in "iu":
            a = a.view(dtype)
        else:
            a = a.astype(dtype)
    return np.ascontiguousarray(a)


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"oracle {what} failed with code {rc}")


def bf16_to_double(bits: int) -> float:
    return _load().oracle_bf16_to_double(int(bits))


def e4m3fn_to_double(code: int) -> float:
    return _load().oracle_e4m3fn_to_double(int(code))


def double_to_bf16(v: float) -> int:
    return int(_load().oracle_double_to_bf16(float(v)))


def double_to_e4m3fn(v: float) -> int:
    return int(_load().oracle_double_to_e4m3fn(float(v)))


def fp8_block_exponent(amax: float) -> int:
    return int(_load().oracle_fp8_block_exponent(float(amax)))


def int4_code(w_bytes, N: int, k: int, n: int) -> int:
    """Signed code of element (k, n) of an INT4 matrix stored as [K, N/2] bytes."""
    w = _np(w_bytes, np.uint8)
    return int(_load().oracle_int4_code(_ptr(w), N, k, n))


def quant_fp8_act_row(x):
    """-> (E4M3FN codes uint8 [n], block exponents int32 [n/128], values fp64 [n])."""
    x = _np(x, np.float64).reshape(-1)
    codes = np.empty(x.size, np.uint8)
    exps = np.empty(x.size // 128, np.int32)
    xq = np.empty(x.size, np.float64)
    _load().oracle_quant_fp8_act_row(_ptr(x), x.size, _ptr(codes), _ptr(exps), _ptr(xq))
    return codes, exps, xq


def float_ffn_act8(x_row, w13, w13_scale, w2, w2_scale):
    """One FP8 expert with FP8 activations on one token. -> (h fp64 [2I], y fp64 [H])."""
    xr = _np(x_row, np.float64)
    H = xr.size
    a13 = _np(w13, np.uint8)
    a2 = _np(w2, np.uint8)
    I = a13.shape[-1] // 2
    s13 = _np(w13_scale, np.float32)
    s2 = _np(w2_scale, np.float32)
    h = np.empty(2 * I, np.float64)
    y = np.empty(H, np.float64)
    _load().oracle_float_ffn_act8(_ptr(xr), H, I, _ptr(a13), _ptr(s13), _ptr(a2), _ptr(s2),
                                  _ptr(h), _ptr(y))
    return h, y


def quant_int8_row(x):
    x = _np(x, np.float32)
    q = np.empty(x.shape[-1], np.int8)
    s = np.zeros(1, np.float32)
    _load().oracle_quant_int8_row(_ptr(x), x.shape[-1], _ptr(q), _ptr(s))
    return q, float(s[0])


def quant_int8_rows(x):
    x = _np(x, np.float32)
    q = np.empty(x.shape, np.int8)
    s = np.empty(x.shape[0], np.float32)
    for r in range(x.shape[0]):
        q[r], s[r] = quant_int8_row(x[r])
    return q, s


def topk(logits, k: int, score: int, renorm: int):
    """-> (weights fp64 [T, k], ids int32 [T, k])."""
    lg = _np(logits, np.float32)
    T, E = lg.shape
    w = np.empty((T, k), np.float64)
    ids = np.empty((T, k), np.int32)
    _check(_load().oracle_topk(_ptr(lg), T, E, k, score, renorm, _ptr(w), _ptr(ids)), "topk")
    return w, ids


def align_capacity(P: int, E: int, B: int) -> int:
    return int(_load().oracle_align_capacity(P, E, B))


def align(topk_ids, E: int, B: int):
    """-> (sorted_ids int32 [cap], expert_ids int32 [ceil(cap/B)], num_tokens_post_pad int)."""
    ids = _np(topk_ids, np.int32).reshape(-1)
    P = ids.size
    cap = align_capacity(P, E, B)
    sorted_ids = np.empty(cap, np.int32)
    expert_ids = np.empty((cap + B - 1) // B, np.int32)
    npp = np.zeros(1, np.int32)
    _check(_load().oracle_align(_ptr(ids) if P else None, P, E, B, _ptr(sorted_ids),
                                _ptr(expert_ids), _ptr(npp)), "align")
    return sorted_ids, expert_ids, int(npp[0])


def float_ffn(wdtype: int, x_row, w13, w13_scale, w2, w2_scale):
    """One BF16/FP8 expert on one token (x_row as float64 values).
    -> (h fp64 [2I], y fp64 [H])."""
    xr = _np(x_row, np.float64)
    H = xr.size
    wd = np.uint16 if wdtype == BF16 else np.uint8
    a13 = _np(w13, wd)
    a2 = _np(w2, wd)
    I = _inter(a13, wdtype)
    s13 = _np(w13_scale, np.float32)
    s2 = _np(w2_scale, np.float32)
    h = np.empty(2 * I, np.float64)
    y = np.empty(H, np.float64)
    _load().oracle_float_ffn(wdtype, _ptr(xr), H, I, _ptr(a13), _ptr(s13), _ptr(a2), _ptr(s2),
                             _ptr(h), _ptr(y))
    return h, y


def int8_ffn(xq, sx: float, w13, w13_scale, w2, w2_scale):
    """One INT8 expert on one quantised token, with its full trace.
    -> dict(h_int, a, qa, sa, y_int, y)."""
    xq = _np(xq, np.int8)
    H = xq.size
    a13 = _np(w13, np.int8)
    a2 = _np(w2, np.int8)
    I = a13.shape[-1] // 2
    s13 = _np(w13_scale, np.float32)
    s2 = _np(w2_scale, np.float32)
    out = dict(h_int=np.empty(2 * I, np.int64), a=np.empty(I, np.float64),
               qa=np.empty(I, np.int8), sa=np.zeros(1, np.float32),
               y_int=np.empty(H, np.int64), y=np.empty(H, np.float64))
    _load().oracle_int8_ffn(_ptr(xq), float(sx), H, I, _ptr(a13), _ptr(s13), _ptr(a2), _ptr(s2),
                            _ptr(out["y"]), _ptr(out["h_int"]), _ptr(out["a"]), _ptr(out["qa"]),
                            _ptr(out["sa"]), _ptr(out["y_int"]))
    out["sa"] = float(out["sa"][0])
    return out


def host_threads() -> int:
    """Host threads the oracle may use: the CPUs this process may run on,
    at most 16."""
    try:
        n = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def moe(wdtype: int, x, w13, w13_scale, w2, w2_scale, topk_w, topk_ids, sh13=None,
        sh13_scale=None, sh2=None, sh2_scale=None, tokens=None, want_acc=False, threads=None):
    """The layer.  x: bf16 bits (uint16) or torch bf16 [T, H]; weights logical.
    topk_w is taken as fp32 (the precision the library's boundary carries).
    threads: host threads (default host_threads()); the token list is cut
    into that many contiguous shards, each evaluated by the same C loop on
    its own thread (tokens are independent, so the bits do not depend on it).
    -> out bf16 bits uint16 [n, H] (and fp64 pre-rounding sums if want_acc)."""
    xb = _np(x, np.uint16)
    T, H = xb.shape
    wd = np.uint16 if wdtype == BF16 else (np.int8 if wdtype == INT8 else np.uint8)
    a13 = _np(w13, wd)
    a2 = _np(w2, wd)
    E = a13.shape[0]
    I = _inter(a13, wdtype)
    s13 = _np(w13_scale, np.float32)
    s2 = _np(w2_scale, np.float32)
    tw = _np(topk_w, np.float32)
    ti = _np(topk_ids, np.int32)
    k = ti.shape[-1]
    h13 = _np(sh13, wd)
    h2 = _np(sh2, wd)
    hs13 = _np(sh13_scale, np.float32)
    hs2 = _np(sh2_scale, np.float32)
    shI = 0 if h13 is None else _inter(h13, wdtype)
    tok = np.arange(T, dtype=np.int32) if tokens is None else _np(tokens, np.int32).reshape(-1)
    n = tok.size
    out = np.empty((n, H), np.uint16)
    acc = np.empty((n, H), np.float64) if want_acc else None
    lib = _load()
    nthr = max(1, min(host_threads() if threads is None else int(threads), n))
    bounds = [n * s // nthr for s in range(nthr + 1)]

    def shard(s):
        lo, hi = bounds[s], bounds[s + 1]
        if lo == hi:
            return 0
        o = out[lo:hi]
        a = None if acc is None else acc[lo:hi]
        return lib.oracle_moe(wdtype, _ptr(xb), T, H, I, E, k, _ptr(a13), _ptr(s13), _ptr(a2),
                              _ptr(s2), _ptr(tw), _ptr(ti), _ptr(h13), _ptr(hs13), _ptr(h2),
                              _ptr(hs2), shI, _ptr(tok[lo:hi]), hi - lo, _ptr(a), _ptr(o))

    if nthr == 1:
        rcs = [shard(0)]
    else:  # ctypes releases the GIL during each call
        with concurrent.futures.ThreadPoolExecutor(max_workers=nthr) as ex:
            rcs = list(ex.map(shard, range(nthr)))
    for rc in rcs:
        _check(rc, "moe")
    return (out, acc) if want_acc else out


def bf16_bits_to_f64(bits) -> np.ndarray:
    """Vectorised bf16 bit pattern -> float64 (exact), for test comparisons."""
    b = np.asarray(bits).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)
