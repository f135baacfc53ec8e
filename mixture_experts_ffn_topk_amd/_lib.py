"""ctypes binding of libmoe (include/moe.h): argument marshalling only.

Every function takes torch tensors that already live on the GPU, passes their
device pointers and the current HIP stream to the C ABI, and raises on a
non-OK status.  No computation happens here, and there is no fallback: if
libmoe.so is missing or cannot be loaded, importing this module's functions
raises.  Build the library with ``python -m mixture_experts_ffn_topk_amd.build``.
"""
from __future__ import annotations

import ctypes
import os
import threading
from typing import Optional

import torch

from . import synth

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoe.so")

MOE_OK = 0
PATH_AUTO, PATH_DECODE, PATH_PREFILL = 0, 1, 2
W_BF16, W_FP8, W_INT8, W_INT4 = (synth.WDTYPE_BF16, synth.WDTYPE_FP8, synth.WDTYPE_INT8,
                                  synth.WDTYPE_INT4)
SCORE_SOFTMAX, SCORE_SIGMOID = synth.SCORE_SOFTMAX, synth.SCORE_SIGMOID

_lock = threading.Lock()
_lib = None


class MoEError(RuntimeError):
    def __init__(self, fn: str, status: int, detail: str):
        super().__init__(f"{fn} failed: status {status} ({detail})")
        self.status = status


class _DenseExpert(ctypes.Structure):
    _fields_ = [("w13", ctypes.c_void_p), ("w13_scale", ctypes.c_void_p),
                ("w2", ctypes.c_void_p), ("w2_scale", ctypes.c_void_p), ("inter", ctypes.c_int)]


class _Layout(ctypes.Structure):
    _fields_ = [("path", ctypes.c_int), ("block_size", ctypes.c_int),
                ("chunk_rows", ctypes.c_int), ("max_chunks", ctypes.c_int),
                ("cap", ctypes.c_int64), ("rows", ctypes.c_int64),
                ("sorted_ids", ctypes.c_size_t), ("meta", ctypes.c_size_t),
                ("chunks", ctypes.c_size_t), ("xq", ctypes.c_size_t), ("xs", ctypes.c_size_t),
                ("xs_stride", ctypes.c_int), ("total", ctypes.c_size_t), ("sched", ctypes.c_size_t)]


class _Options(ctypes.Structure):
    _fields_ = [("path", ctypes.c_int), ("split_k", ctypes.c_int),
                ("prefill_span", ctypes.c_int), ("fp8_activations", ctypes.c_int),
                ("tiny_fusion", ctypes.c_int), ("reserved", ctypes.c_int * 3)]


EXPORTS = [
    "moe_status_str", "moe_last_error", "moe_version", "moe_topk", "moe_align_capacity",
    "moe_align_block_size", "moe_quant_int8_rows", "moe_packed_bytes", "moe_prepack",
    "moe_prepack_bf16", "moe_prepack_fp8", "moe_prepack_int8", "moe_prepack_int4",
    "moe_dequant_fp8",
    "fused_moe_workspace_bytes", "fused_moe_workspace_bytes_ex", "fused_moe_workspace_layout",
    "fused_moe_bf16",
    "fused_moe_fp8", "fused_moe_int8", "fused_moe_int4", "fused_moe_ex", "fused_moe_routed",
    "fused_moe_routed_noalloc", "moe_profile_enable",
    "moe_profile_collect", "moe_profile_stage_name",
]


def load():
    """Load libmoe.so (raises if it is missing)."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m mixture_experts_ffn_topk_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        P, i32, i64, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t
        sig = {
            "moe_status_str": ([i32], ctypes.c_char_p),
            "moe_last_error": ([], ctypes.c_char_p),
            "moe_version": ([], i32),
            "moe_topk": ([P, i32, i32, i32, i32, i32, P, P, P], i32),
            "moe_align_capacity": ([i64, i32, i32], i64),
            "moe_align_block_size": ([P, i32, i32, i32, i32, P, P, P, P], i32),
            "moe_quant_int8_rows": ([P, i32, i32, P, P, P], i32),
            "moe_packed_bytes": ([i32, i32, i32, i32], sz),
            "moe_prepack": ([i32, P, i32, i32, i32, i32, P, P], i32),
            "moe_dequant_fp8": ([P, P, i32, i32, i32, P, P], i32),
            "fused_moe_workspace_bytes": ([i32, i32, i32, i32, i32, i32, i32], sz),
            "fused_moe_workspace_bytes_ex": ([i32, i32, i32, i32, i32, i32, i32, P], sz),
            "fused_moe_workspace_layout": ([i32, i32, i32, i32, i32, i32, i32, P, P], i32),
            "fused_moe_ex": ([i32, P, P, P, P, P, P, P, i32, i32, i32, i32, i32, P, P, sz, P, P,
                              P], i32),
            "fused_moe_routed": ([i32, P, i32, i32, P, P, P, P, P, P, P, i32, i32, i32, i32, i32,
                                  P, P, sz, P, P, P], i32),
            "fused_moe_routed_noalloc": ([i32, P, i32, i32, P, P, P, P, P, P, P, i32, i32, i32,
                                          i32, i32, P, P, P, P], i32),
            "fused_moe_bf16": ([P, P, P, P, P, i32, i32, i32, i32, i32, P, P, sz, P, P], i32),
            "fused_moe_fp8": ([P, P, P, P, P, P, P, i32, i32, i32, i32, i32, P, P, sz, P, P], i32),
            "fused_moe_int8": ([P, P, P, P, P, P, P, i32, i32, i32, i32, i32, P, P, sz, P, P],
                               i32),
            "fused_moe_int4": ([P, P, P, P, P, P, P, i32, i32, i32, i32, i32, P, P, sz, P, P],
                               i32),
            "moe_prepack_int4": ([P, i32, i32, i32, i32, P, P], i32),
            "moe_profile_enable": ([i32], i32),
            "moe_profile_collect": ([P, P, i32], i32),
            "moe_profile_stage_name": ([i32], ctypes.c_char_p),
        }
        for name, (args, res) in sig.items():
            f = getattr(lib, name)
            f.argtypes = args
            f.restype = res
        _lib = lib
        return lib


def _check(fn: str, status: int):
    if status != MOE_OK:
        lib = load()
        raise MoEError(fn, status, lib.moe_last_error().decode())


def _dev(t: Optional[torch.Tensor], name: str):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


# ---------------------------------------------------------------------------
# Entry points (same names as the C ABI, without the moe_ prefix where short)
# ---------------------------------------------------------------------------

def topk(logits: torch.Tensor, k: int, score: int, renormalize: int = 1, out=None, stream=None):
    T, E = logits.shape
    dev = logits.device
    w, ids = out if out is not None else (torch.empty(T, k, dtype=torch.float32, device=dev),
                                          torch.empty(T, k, dtype=torch.int32, device=dev))
    _check("moe_topk", load().moe_topk(_dev(logits, "logits"), T, E, k, score, renormalize,
                                        _dev(w, "w"), _dev(ids, "ids"), _stream(stream)))
    return w, ids


def align_capacity(P: int, E: int, block_size: int) -> int:
    return int(load().moe_align_capacity(P, E, block_size))


def align_block_size(topk_ids: torch.Tensor, E: int, block_size: int, stream=None):
    T, k = topk_ids.shape
    cap = align_capacity(T * k, E, block_size)
    dev = topk_ids.device
    sorted_ids = torch.empty(max(cap, 1), dtype=torch.int32, device=dev)
    expert_ids = torch.empty(max((cap + block_size - 1) // block_size, 1), dtype=torch.int32,
                             device=dev)
    npp = torch.empty(1, dtype=torch.int32, device=dev)
    _check("moe_align_block_size", load().moe_align_block_size(
        _dev(topk_ids, "topk_ids"), T, k, E, block_size, _dev(sorted_ids, "sorted_ids"),
        _dev(expert_ids, "expert_ids"), _dev(npp, "npp"), _stream(stream)))
    return sorted_ids[:cap], expert_ids[:(cap + block_size - 1) // block_size], npp


def quant_int8_rows(x: torch.Tensor, stream=None):
    rows, cols = x.shape
    q = torch.empty(rows, cols, dtype=torch.int8, device=x.device)
    s = torch.empty(rows, dtype=torch.float32, device=x.device)
    _check("moe_quant_int8_rows", load().moe_quant_int8_rows(
        _dev(x, "x"), rows, cols, _dev(q, "q"), _dev(s, "scale"), _stream(stream)))
    return q, s


def _inter(w13p: torch.Tensor, wdtype: int) -> int:
    """Intermediate size I of a (packed) w13 [.., H, 2I] (INT4: [.., H, I] bytes)."""
    return w13p.shape[-1] if wdtype == W_INT4 else w13p.shape[-1] // 2


def prepack(wdtype: int, w: torch.Tensor, is_w13: bool, stream=None) -> torch.Tensor:
    """Logical [E, K, N] (or [K, N]) weights -> packed buffer of the same dtype/shape
    (INT4: [E, K, N/2] bytes of nibble pairs)."""
    w3 = w if w.dim() == 3 else w.unsqueeze(0)
    E, K, N = w3.shape
    if wdtype == W_INT4:
        N *= 2
    out = torch.empty_like(w3)
    _check("moe_prepack", load().moe_prepack(wdtype, _dev(w3, "w"), E, K, N, int(bool(is_w13)),
                                             _dev(out, "packed"), _stream(stream)))
    return out if w.dim() == 3 else out[0]


def dequant_fp8(codes: torch.Tensor, scale: Optional[torch.Tensor], mode: int = 0, stream=None):
    K, N = codes.shape
    out = torch.empty(K, N, dtype=torch.float32, device=codes.device)
    _check("moe_dequant_fp8", load().moe_dequant_fp8(
        _dev(codes, "codes"), _dev(scale, "scale"), K, N, mode, _dev(out, "out"), _stream(stream)))
    return out


def _opts(path: int, split_k: int, span: int = 0, fp8_act: int = 0, tiny_fusion: int = 0):
    o = _Options()
    o.path = path
    o.split_k = split_k
    o.prefill_span = span
    o.fp8_activations = int(bool(fp8_act))
    o.tiny_fusion = int(tiny_fusion)
    return o


def workspace_bytes(wdtype: int, T: int, H: int, I: int, E: int, k: int, has_shared: bool,
                    path: int = PATH_AUTO, split_k: int = 0, fp8_act: int = 0, tiny_fusion: int = 0) -> int:
    lib = load()
    if path == PATH_AUTO and split_k == 0 and not fp8_act and not tiny_fusion:
        return int(lib.fused_moe_workspace_bytes(wdtype, T, H, I, E, k, int(has_shared)))
    o = _opts(path, split_k, 0, fp8_act, tiny_fusion)
    return int(lib.fused_moe_workspace_bytes_ex(wdtype, T, H, I, E, k, int(has_shared),
                                                ctypes.byref(o)))


def workspace_layout(wdtype: int, T: int, H: int, I: int, E: int, k: int, has_shared: bool,
                     path: int = PATH_AUTO, split_k: int = 0, span: int = 0, fp8_act: int = 0,
                     tiny_fusion: int = 0) -> dict:
    """Byte offsets of the alignment inside the workspace of the matching
    fused_moe call (fused_moe_workspace_layout), as a dict."""
    o = _opts(path, split_k, span, fp8_act, tiny_fusion)
    lay = _Layout()
    _check("fused_moe_workspace_layout", load().fused_moe_workspace_layout(
        wdtype, T, H, I, E, k, int(has_shared), ctypes.byref(o), ctypes.byref(lay)))
    return {name: getattr(lay, name) for name, _ in _Layout._fields_}


def fused_moe(wdtype: int, x: torch.Tensor, w13p: torch.Tensor, w13_scale, w2p: torch.Tensor,
              w2_scale, topk_w: torch.Tensor, topk_ids: torch.Tensor, shared=None,
              workspace: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
              path: int = PATH_AUTO, split_k: int = 0, stream=None, span: int = 0,
              fp8_act: int = 0, tiny_fusion: int = 0) -> torch.Tensor:
    """shared: None or (w13p [H, 2I], w13_scale, w2p [I, H], w2_scale) packed with E=1.
    span: BF16 / INT8 prefill column groups per workgroup (0 = auto).
    fp8_act: FP8 weights on the tile kernels: FP8 activations (opt in).
    tiny_fusion: 1 keeps the alignment of tiny decode batches in a launch of
    its own (0: inside the first GEMM; same results)."""
    T, H = x.shape
    E = w13p.shape[0]
    I = _inter(w13p, wdtype)
    k = topk_ids.shape[1]
    if out is None:
        out = torch.empty(T, H, dtype=torch.bfloat16, device=x.device)
    need = workspace_bytes(wdtype, T, H, I, E, k, shared is not None, path, split_k, fp8_act, tiny_fusion)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    sh = None
    if shared is not None:
        s13, s13s, s2, s2s = shared
        sh = _DenseExpert(_dev(s13, "shared w13").value, _dev(s13s, "shared w13_scale").value
                          if s13s is not None else None, _dev(s2, "shared w2").value,
                          _dev(s2s, "shared w2_scale").value if s2s is not None else None, I)
    o = _opts(path, split_k, span, fp8_act, tiny_fusion)
    _check("fused_moe_ex", load().fused_moe_ex(
        wdtype, _dev(x, "x"), _dev(w13p, "w13"), _dev(w13_scale, "w13_scale"), _dev(w2p, "w2"),
        _dev(w2_scale, "w2_scale"), _dev(topk_w, "topk_weights"), _dev(topk_ids, "topk_ids"),
        T, H, I, E, k, ctypes.byref(sh) if sh is not None else None,
        _dev(workspace, "workspace"), workspace.numel(), _dev(out, "out"), ctypes.byref(o),
        _stream(stream)))
    return out


def fused_moe_routed(wdtype: int, logits: torch.Tensor, k: int, score: int, renorm: int,
                     x: torch.Tensor, w13p: torch.Tensor, w13_scale, w2p: torch.Tensor, w2_scale,
                     topk_w: torch.Tensor, topk_ids: torch.Tensor, shared=None,
                     workspace: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                     path: int = PATH_AUTO, split_k: int = 0, stream=None, span: int = 0,
                     fp8_act: int = 0, tiny_fusion: int = 0) -> torch.Tensor:
    """Router top-k of `logits` into topk_w / topk_ids, then the fused layer,
    in one library call (same results as topk() followed by fused_moe())."""
    T, H = x.shape
    E = w13p.shape[0]
    I = _inter(w13p, wdtype)
    if tuple(logits.shape) != (T, E) or logits.dtype != torch.float32:
        raise ValueError(f"logits must be fp32 [{T}, {E}]")
    if tuple(topk_w.shape) != (T, k) or tuple(topk_ids.shape) != (T, k):
        raise ValueError(f"topk outputs must be [{T}, {k}]")
    if out is None:
        out = torch.empty(T, H, dtype=torch.bfloat16, device=x.device)
    need = workspace_bytes(wdtype, T, H, I, E, k, shared is not None, path, split_k, fp8_act, tiny_fusion)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    sh = None
    if shared is not None:
        s13, s13s, s2, s2s = shared
        sh = _DenseExpert(_dev(s13, "shared w13").value, _dev(s13s, "shared w13_scale").value
                          if s13s is not None else None, _dev(s2, "shared w2").value,
                          _dev(s2s, "shared w2_scale").value if s2s is not None else None, I)
    o = _opts(path, split_k, span, fp8_act, tiny_fusion)
    _check("fused_moe_routed", load().fused_moe_routed(
        wdtype, _dev(logits, "logits"), score, int(bool(renorm)), _dev(x, "x"),
        _dev(w13p, "w13"), _dev(w13_scale, "w13_scale"), _dev(w2p, "w2"),
        _dev(w2_scale, "w2_scale"), _dev(topk_w, "topk_weights"), _dev(topk_ids, "topk_ids"),
        T, H, I, E, k, ctypes.byref(sh) if sh is not None else None,
        _dev(workspace, "workspace"), workspace.numel(), _dev(out, "out"), ctypes.byref(o),
        _stream(stream)))
    return out


NOALLOC_SCRATCH_BYTES = 64 << 20  # MOE_NOALLOC_SCRATCH_BYTES in include/moe.h


def fused_moe_routed_noalloc(wdtype: int, logits: torch.Tensor, k: int, score: int, renorm: int,
                             x: torch.Tensor, w13p: torch.Tensor, w13_scale, w2p: torch.Tensor,
                             w2_scale, topk_w: torch.Tensor, topk_ids: torch.Tensor, out: torch.Tensor,
                             shared=None, path: int = PATH_AUTO, split_k: int = 0, stream=None,
                             span: int = 0, tiny_fusion: int = 0) -> torch.Tensor:
    """fused_moe_routed without a workspace argument: the library's static
    per-GPU scratch is used (callers that cannot allocate).  Every output
    tensor must be passed in."""
    T, H = x.shape
    E = w13p.shape[0]
    I = _inter(w13p, wdtype)
    if tuple(logits.shape) != (T, E) or logits.dtype != torch.float32:
        raise ValueError(f"logits must be fp32 [{T}, {E}]")
    if tuple(topk_w.shape) != (T, k) or tuple(topk_ids.shape) != (T, k):
        raise ValueError(f"topk outputs must be [{T}, {k}]")
    if tuple(out.shape) != (T, H):
        raise ValueError(f"out must be [{T}, {H}]")
    sh = None
    if shared is not None:
        s13, s13s, s2, s2s = shared
        sh = _DenseExpert(_dev(s13, "shared w13").value, _dev(s13s, "shared w13_scale").value
                          if s13s is not None else None, _dev(s2, "shared w2").value,
                          _dev(s2s, "shared w2_scale").value if s2s is not None else None, I)
    o = _opts(path, split_k, span, 0, tiny_fusion)
    _check("fused_moe_routed_noalloc", load().fused_moe_routed_noalloc(
        wdtype, _dev(logits, "logits"), score, int(bool(renorm)), _dev(x, "x"),
        _dev(w13p, "w13"), _dev(w13_scale, "w13_scale"), _dev(w2p, "w2"),
        _dev(w2_scale, "w2_scale"), _dev(topk_w, "topk_weights"), _dev(topk_ids, "topk_ids"),
        T, H, I, E, k, ctypes.byref(sh) if sh is not None else None, _dev(out, "out"),
        ctypes.byref(o), _stream(stream)))
    return out


def profile_enable(on: bool):
    load().moe_profile_enable(int(bool(on)))


def profile_collect():
    """-> {stage name: (total ms, launches)} for every kernel timed since the last collect."""
    lib = load()
    n = 32
    ms = (ctypes.c_double * n)()
    cnt = (ctypes.c_int64 * n)()
    ns = lib.moe_profile_collect(ms, cnt, n)
    res = {}
    for i in range(min(ns, n)):
        if cnt[i]:
            res[lib.moe_profile_stage_name(i).decode()] = (ms[i], int(cnt[i]))
    return res


class MoELayer:
    """Device-resident weights of one layer plus a reusable workspace.

    Holds the packed expert weights (prepacked once, outside any timing) and
    runs one step of the hot path: router top-k, then the fused layer.
    """

    def __init__(self, inp: synth.MoEInputs, path: int = PATH_AUTO, split_k: int = 0, span: int = 0,
                 packed_from: Optional["MoELayer"] = None, fp8_act: int = 0, tiny_fusion: int = 0):
        """packed_from: a layer over the same weights (another batch size)
        whose packed buffers are shared instead of prepacking again.
        fp8_act: FP8 weights on the tile kernels: FP8 activations (opt in).
        tiny_fusion: 1 = tiny decode batches align in a launch of their own."""
        cfg = inp.cfg
        self.cfg = cfg
        self.path = path
        self.split_k = split_k
        self.span = span
        self.fp8_act = int(bool(fp8_act))
        self.tiny_fusion = int(tiny_fusion)
        wd = cfg.wdtype
        view = {W_BF16: torch.uint16, W_FP8: torch.uint8, W_INT8: torch.int8, W_INT4: torch.uint8}[wd]
        if packed_from is not None:
            self.w13, self.w2, self.shared = packed_from.w13, packed_from.w2, packed_from.shared
        else:
            self.w13 = prepack(wd, inp.w13.view(view), True)
            self.w2 = prepack(wd, inp.w2.view(view), False)
            self.shared = None
            if cfg.shared:
                self.shared = (prepack(wd, inp.sh13.view(view), True), inp.sh13_scale,
                               prepack(wd, inp.sh2.view(view), False), inp.sh2_scale)
        self.s13, self.s2 = inp.w13_scale, inp.w2_scale
        dev = inp.x.device
        need = workspace_bytes(wd, cfg.T, cfg.H, cfg.I, cfg.E, cfg.k, cfg.shared, path, split_k,
                               self.fp8_act, self.tiny_fusion)
        self.ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
        self.out = torch.empty(cfg.T, cfg.H, dtype=torch.bfloat16, device=dev)
        self.tw = torch.empty(cfg.T, cfg.k, dtype=torch.float32, device=dev)
        self.ti = torch.empty(cfg.T, cfg.k, dtype=torch.int32, device=dev)

    def route(self, logits):
        return topk(logits, self.cfg.k, self.cfg.score, self.cfg.renorm, out=(self.tw, self.ti))

    def ffn(self, x, tw, ti):
        return fused_moe(self.cfg.wdtype, x, self.w13, self.s13, self.w2, self.s2, tw, ti,
                         self.shared, self.ws, self.out, self.path, self.split_k, span=self.span,
                         fp8_act=self.fp8_act, tiny_fusion=self.tiny_fusion)

    def step(self, logits, x):
        """One layer step in one library call (router top-k into self.tw /
        self.ti, then the fused layer into self.out)."""
        c = self.cfg
        return fused_moe_routed(c.wdtype, logits, c.k, c.score, c.renorm, x, self.w13, self.s13,
                                self.w2, self.s2, self.tw, self.ti, self.shared, self.ws, self.out,
                                self.path, self.split_k, span=self.span, fp8_act=self.fp8_act,
                                tiny_fusion=self.tiny_fusion)

    def layout(self) -> dict:
        """Where this layer's calls keep the alignment in self.ws."""
        c = self.cfg
        return workspace_layout(c.wdtype, c.T, c.H, c.I, c.E, c.k, c.shared, self.path,
                                self.split_k, self.span, self.fp8_act, self.tiny_fusion)

    def step_two_calls(self, logits, x):
        """The same step as moe_topk followed by the fused layer."""
        tw, ti = self.route(logits)
        return self.ffn(x, tw, ti)
