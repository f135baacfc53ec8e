"""Seeded synthetic inputs for the fused MoE FFN layer.

This module only *draws* inputs: router logits, bf16 activations and expert
weights, the latter stored the way a quantised checkpoint stores them (FP8
E4M3FN codes with one fp32 scale per 128x128 block, or INT8 codes with one fp32
scale per output channel).  It holds none of the layer's own arithmetic
(routing, alignment, GEMMs, activation quantisation, combine), imports neither
the HIP binding nor the oracle, and serves both sides of every parity check.

Workload shapes follow the models the pages name: a tiny BF16 layer, a
DeepSeek-R1-shaped FP8 layer (hidden 7168, intermediate 2048, 256 routed
experts, top-8, one shared expert) and a Qwen3-235B-A22B-shaped INT8 layer
(hidden 4096, intermediate 1536, 128 experts, top-8).  Weights are N(0, 0.02)
and activations / logits N(0, 1), all drawn with torch's seeded generator on
the requested device (so a given (seed, device) pair is reproducible; CPU and
GPU streams differ).

Logical layouts (row-major, last index contiguous):
  logits  fp32 [T, E]
  x       bf16 [T, H]
  w13     [E, H, 2I]   columns [0, I) = gate (goes through SiLU), [I, 2I) = up
  w2      [E, I, H]
  FP8 scales  fp32 [E, K/128, N/128]   (W ~= code * scale, per 128x128 block)
  INT8 scales fp32 [E, N]              (W ~= code * scale, per output channel)
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import torch

SCORE_SOFTMAX = 0
SCORE_SIGMOID = 1

WDTYPE_BF16 = 0
WDTYPE_FP8 = 1
WDTYPE_INT8 = 2
WDTYPE_INT4 = 3

_FP8_MAX = 448.0  # largest finite E4M3FN magnitude
_FP8_BLOCK = 128


@dataclasses.dataclass(frozen=True)
class MoEConfig:
    name: str
    T: int
    H: int
    I: int
    E: int
    k: int
    wdtype: int
    score: int
    renorm: int
    shared: bool = False
    routing: str = "normal"  # "normal" | "zipf"
    zipf_s: float = 1.1
    seed: int = 0

    def with_T(self, T: int) -> "MoEConfig":
        return dataclasses.replace(self, T=T, name=f"{self.name.split('@')[0]}@T{T}")

    def small(self, T: int, H: int, I: int, E: Optional[int] = None) -> "MoEConfig":
        """Same routing / dtype recipe at reduced sizes (for oracle-speed parity)."""
        return dataclasses.replace(self, T=T, H=H, I=I, E=E if E is not None else self.E,
                                   name=f"{self.name.split('@')[0]}@small{T}x{H}x{I}")


# The five workloads (names describe the shape; sizes as the workload list fixes them).
TINY_BF16 = MoEConfig("tiny_bf16_T16", T=16, H=256, I=128, E=8, k=2,
                      wdtype=WDTYPE_BF16, score=SCORE_SOFTMAX, renorm=1)
DSR1_FP8_DECODE_T4 = MoEConfig("dsr1_fp8_decode_T4", T=4, H=7168, I=2048, E=256, k=8,
                               wdtype=WDTYPE_FP8, score=SCORE_SIGMOID, renorm=1, shared=True)
DSR1_FP8_DECODE_T64_ZIPF = MoEConfig("dsr1_fp8_decode_T64_zipf", T=64, H=7168, I=2048, E=256,
                                     k=8, wdtype=WDTYPE_FP8, score=SCORE_SIGMOID, renorm=1,
                                     shared=True, routing="zipf")
DSR1_FP8_PREFILL_T4096 = MoEConfig("dsr1_fp8_prefill_T4096", T=4096, H=7168, I=2048, E=256,
                                   k=8, wdtype=WDTYPE_FP8, score=SCORE_SIGMOID, renorm=1,
                                   shared=True)
QWEN3_INT8 = MoEConfig("qwen3_int8", T=1, H=4096, I=1536, E=128, k=8,
                       wdtype=WDTYPE_INT8, score=SCORE_SOFTMAX, renorm=1)

# The DeepSeek-R1-shaped decode batch with 4-bit weight-only experts (the
# INT4 decode path; no workload of the list uses INT4 weights).
DSR1_INT4_DECODE_T4 = MoEConfig("dsr1_int4_decode_T4", T=4, H=7168, I=2048, E=256, k=8,
                                wdtype=WDTYPE_INT4, score=SCORE_SIGMOID, renorm=1, shared=True)
EXTRA_CONFIGS = {"c2_int4": DSR1_INT4_DECODE_T4}

CONFIGS = {
    "c1": TINY_BF16,
    "c2": DSR1_FP8_DECODE_T4,
    "c3": DSR1_FP8_DECODE_T64_ZIPF,
    "c4": DSR1_FP8_PREFILL_T4096,
    "c5_T1": QWEN3_INT8.with_T(1),
    "c5_T32": QWEN3_INT8.with_T(32),
    "c5_T2048": QWEN3_INT8.with_T(2048),
}


def _gen(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


# Stream ids: each tensor draws from its own child seed so shapes can change
# independently and large weights can be drawn one expert at a time.
_S_LOGITS, _S_X, _S_W13, _S_W2, _S_SH13, _S_SH2, _S_PERM, _S_GUMBEL = range(8)


def _child_seed(seed: int, stream: int, sub: int = 0) -> int:
    return (seed * 1_000_003 + stream * 7919 + sub * 104_729) % (2**63 - 1)


def draw_logits(cfg: MoEConfig, device="cpu", seed: Optional[int] = None) -> torch.Tensor:
    """Router logits fp32 [T, E].

    "normal": N(0,1).  "zipf": log p_e + Gumbel(0,1) noise where p_e is
    proportional to (rank(e)+1)^-s and rank comes from a seeded permutation
    of the experts, so the first choice of each token is Zipf-distributed.
    """
    seed = cfg.seed if seed is None else seed
    g = _gen(device, _child_seed(seed, _S_LOGITS))
    if cfg.routing == "normal":
        return torch.randn(cfg.T, cfg.E, generator=g, device=device, dtype=torch.float32)
    if cfg.routing == "zipf":
        gp = _gen("cpu", _child_seed(seed, _S_PERM))
        rank = torch.randperm(cfg.E, generator=gp)  # rank[e]
        logp = -cfg.zipf_s * torch.log(rank.to(torch.float64) + 1.0)
        logp = logp - torch.logsumexp(logp, 0)
        u = torch.rand(cfg.T, cfg.E, generator=g, device=device, dtype=torch.float64)
        u = u.clamp_(1e-300, 1.0 - 1e-16)
        gumbel = -torch.log(-torch.log(u))
        return (logp.to(device).unsqueeze(0) + gumbel).to(torch.float32)
    raise ValueError(cfg.routing)


def draw_x(cfg: MoEConfig, device="cpu", seed: Optional[int] = None) -> torch.Tensor:
    """Hidden states bf16 [T, H], N(0,1) rounded to bf16."""
    seed = cfg.seed if seed is None else seed
    g = _gen(device, _child_seed(seed, _S_X))
    return torch.randn(cfg.T, cfg.H, generator=g, device=device,
                       dtype=torch.float32).to(torch.bfloat16)


def _normal_matrix(K: int, N: int, device, seed: int, stream: int, sub: int, std=0.02):
    g = _gen(device, _child_seed(seed, stream, sub))
    return torch.randn(K, N, generator=g, device=device, dtype=torch.float32) * std


def encode_fp8_blocks(w: torch.Tensor):
    """fp32 [K, N] -> (E4M3FN codes uint8 [K, N], fp32 scales [K/128, N/128]).

    Checkpoint-style block quantisation of a synthetic weight: scale = block
    amax / 448, code = E4M3FN(w / scale) via torch's float8 cast.  Input
    preparation only; the layer never quantises weights at run time.
    """
    K, N = w.shape
    assert K % _FP8_BLOCK == 0 and N % _FP8_BLOCK == 0
    b = w.reshape(K // _FP8_BLOCK, _FP8_BLOCK, N // _FP8_BLOCK, _FP8_BLOCK)
    amax = b.abs().amax(dim=(1, 3)).clamp_min(1e-30)
    scale = (amax / _FP8_MAX).to(torch.float32)
    q = (b / scale[:, None, :, None]).clamp_(-_FP8_MAX, _FP8_MAX)
    codes = q.reshape(K, N).to(torch.float8_e4m3fn).view(torch.uint8)
    return codes, scale


def encode_int8_channels(w: torch.Tensor):
    """fp32 [K, N] -> (int8 codes [K, N], fp32 scales [N]); symmetric per output channel."""
    amax = w.abs().amax(dim=0).clamp_min(1e-30)
    scale = (amax / 127.0).to(torch.float32)
    q = torch.round(w / scale[None, :]).clamp_(-127, 127).to(torch.int8)
    return q, scale


def encode_int4_groups(w: torch.Tensor):
    """fp32 [K, N] -> (4-bit codes packed two per byte uint8 [K, N/2], fp32 scales
    [K/128, N]).  Checkpoint-style symmetric quantisation per output column and
    128-row K group: scale = group amax / 7, code = round(w / scale) in [-7, 7],
    stored as a two's-complement nibble, column 2j in the low nibble of byte j."""
    K, N = w.shape
    assert K % 128 == 0 and N % 2 == 0
    g = w.reshape(K // 128, 128, N)
    amax = g.abs().amax(dim=1).clamp_min(1e-30)
    scale = (amax / 7.0).to(torch.float32)
    q = torch.round(g / scale[:, None, :]).clamp_(-7, 7).to(torch.int32).reshape(K, N)
    nib = (q & 15).to(torch.uint8)
    codes = nib[:, 0::2] | (nib[:, 1::2] << 4)
    return codes.contiguous(), scale


def _draw_expert(cfg: MoEConfig, K: int, N: int, device, seed, stream, e):
    w = _normal_matrix(K, N, device, seed, stream, e)
    if cfg.wdtype == WDTYPE_BF16:
        return w.to(torch.bfloat16).view(torch.uint16), None
    if cfg.wdtype == WDTYPE_FP8:
        return encode_fp8_blocks(w)
    if cfg.wdtype == WDTYPE_INT8:
        return encode_int8_channels(w)
    if cfg.wdtype == WDTYPE_INT4:
        return encode_int4_groups(w)
    raise ValueError(cfg.wdtype)


def draw_weight_stack(cfg: MoEConfig, which: str, device="cpu", seed: Optional[int] = None,
                      experts=None):
    """Expert weights in logical layout.

    which = "w13" -> [E, H, 2I]; "w2" -> [E, I, H]; "sh13" / "sh2" -> the
    shared expert's [H, 2I] / [I, H] (no leading E axis).
    Returns (codes, scales) where codes is uint16 (bf16 bits), uint8 (E4M3FN,
    or INT4 nibble pairs [.., K, N/2]) or int8, and scales is None (bf16), fp32
    [E, K/128, N/128] (FP8), fp32 [E, N] (INT8) or fp32 [E, K/128, N] (INT4).
    experts: optional list of expert indices to draw (others are not drawn);
    then the leading axis has len(experts) entries.  Each expert has its own
    stream, so a subset draws exactly the same values as the full stack.
    """
    seed = cfg.seed if seed is None else seed
    if which in ("w13", "sh13"):
        K, N = cfg.H, 2 * cfg.I
    elif which in ("w2", "sh2"):
        K, N = cfg.I, cfg.H
    else:
        raise ValueError(which)
    stream = {"w13": _S_W13, "w2": _S_W2, "sh13": _S_SH13, "sh2": _S_SH2}[which]
    if which.startswith("sh"):
        return _draw_expert(cfg, K, N, device, seed, stream, 0)
    idx = list(range(cfg.E)) if experts is None else list(experts)
    codes0, scale0 = None, None
    codes = None
    scales = None
    for n, e in enumerate(idx):
        c, s = _draw_expert(cfg, K, N, device, seed, stream, e)
        if codes is None:
            codes = torch.empty((len(idx),) + tuple(c.shape), dtype=c.dtype, device=device)
            if s is not None:
                scales = torch.empty((len(idx),) + tuple(s.shape), dtype=s.dtype, device=device)
        codes[n].copy_(c)
        if s is not None:
            scales[n].copy_(s)
    return codes, scales


@dataclasses.dataclass
class MoEInputs:
    cfg: MoEConfig
    logits: torch.Tensor
    x: torch.Tensor
    w13: torch.Tensor
    w13_scale: Optional[torch.Tensor]
    w2: torch.Tensor
    w2_scale: Optional[torch.Tensor]
    sh13: Optional[torch.Tensor] = None
    sh13_scale: Optional[torch.Tensor] = None
    sh2: Optional[torch.Tensor] = None
    sh2_scale: Optional[torch.Tensor] = None


def draw_inputs(cfg: MoEConfig, device="cpu", seed: Optional[int] = None) -> MoEInputs:
    """All inputs of one layer invocation for a workload."""
    w13, s13 = draw_weight_stack(cfg, "w13", device, seed)
    w2, s2 = draw_weight_stack(cfg, "w2", device, seed)
    inp = MoEInputs(cfg, draw_logits(cfg, device, seed), draw_x(cfg, device, seed),
                    w13, s13, w2, s2)
    if cfg.shared:
        inp.sh13, inp.sh13_scale = draw_weight_stack(cfg, "sh13", device, seed)
        inp.sh2, inp.sh2_scale = draw_weight_stack(cfg, "sh2", device, seed)
    return inp


def bytes_per_expert(cfg: MoEConfig) -> int:
    """Stored bytes of one expert's w13 + w2 (codes + scales)."""
    n = cfg.H * 2 * cfg.I + cfg.I * cfg.H
    if cfg.wdtype == WDTYPE_INT4:
        return n // 2 + 4 * ((cfg.H // 128) * 2 * cfg.I + (cfg.I // 128) * cfg.H)
    elem = {WDTYPE_BF16: 2, WDTYPE_FP8: 1, WDTYPE_INT8: 1}[cfg.wdtype]
    b = n * elem
    if cfg.wdtype == WDTYPE_FP8:
        b += 4 * ((cfg.H // 128) * (2 * cfg.I // 128) + (cfg.I // 128) * (cfg.H // 128))
    elif cfg.wdtype == WDTYPE_INT8:
        b += 4 * (2 * cfg.I + cfg.H)
    return b
