"""GPU: INT4 weight-only layers on the decode (weight-streaming) kernels
against the oracle (ORC_INT4), through the C ABI: several tiles per
dimension, ragged token counts, every K split, a shared expert, a hot
expert over many chunks, zero group scales, zero input, and the
DeepSeek-R1-shaped decode batch with INT4 experts (every token)."""
import numpy as np
import pytest
import torch

from mixture_experts_ffn_topk_amd import _lib as moe
from mixture_experts_ffn_topk_amd import synth
from helpers import check_close, oracle_layer, oracle_routed_layer

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _say(*a):
    print(*a, flush=True)


def _cfg(name, T, H, I, E, k, shared=True, score=1, routing="normal"):
    return synth.MoEConfig(name, T=T, H=H, I=I, E=E, k=k, wdtype=synth.WDTYPE_INT4, score=score,
                           renorm=1, shared=shared, routing=routing)


CASES = {
    "ragged_shared": _cfg("i4_r", T=37, H=640, I=384, E=6, k=2),
    "many_experts_zipf": _cfg("i4_z", T=40, H=512, I=256, E=32, k=8, routing="zipf"),
    "single_token": _cfg("i4_1", T=1, H=1024, I=512, E=64, k=8, shared=False, score=0),
    "rows_per_expert_8": _cfg("i4_8", T=64, H=256, I=256, E=8, k=1),
}


@pytest.mark.parametrize("name", list(CASES))
def test_int4_layer(name):
    cfg = CASES[name]
    _say("int4 layer", name)
    inp = synth.draw_inputs(cfg, DEV)
    layer = moe.MoELayer(inp)
    out = layer.step(inp.logits, inp.x).clone()
    torch.cuda.synchronize()
    assert layer.layout()["path"] == moe.PATH_DECODE
    rel, mx = check_close(out, oracle_routed_layer(inp), f"int4 {name}")
    _say(f"  {name}: rel-L2 {rel:.2e}, max-abs/max|ref| {mx:.2e}")


@pytest.mark.parametrize("split_k", [1, 2, 3, 5])
def test_int4_split_k(split_k):
    """Five 128-row K blocks in GEMM1 (H = 640): splits of 1, 2, 3 and 5."""
    cfg = CASES["ragged_shared"]
    _say("int4 split", split_k)
    inp = synth.draw_inputs(cfg, DEV)
    layer = moe.MoELayer(inp, path=moe.PATH_DECODE, split_k=split_k)
    tw, ti = layer.route(inp.logits)
    tw, ti = tw.clone(), ti.clone()
    out = layer.ffn(inp.x, tw, ti).clone()
    torch.cuda.synchronize()
    check_close(out, oracle_layer(inp, tw, ti), f"int4 split {split_k}")


def test_int4_hot_expert_zero_scales_zero_rows():
    """One expert takes every token (many 64-row chunks), zero group scales
    in w13 and w2, two all-zero token rows."""
    cfg = _cfg("i4_h", T=300, H=256, I=256, E=9, k=2)
    _say("int4 hot expert")
    inp = synth.draw_inputs(cfg, DEV)
    inp.logits[:, 4] += 20.0
    inp.w13_scale[4, 1, 7] = 0.0
    inp.w2_scale[4, 0, 100] = 0.0
    inp.sh13_scale[0, 300] = 0.0
    inp.x[3] = 0
    inp.x[250] = 0
    layer = moe.MoELayer(inp)
    out = layer.step(inp.logits, inp.x).clone()
    torch.cuda.synchronize()
    check_close(out, oracle_routed_layer(inp), "int4 hot")


def test_int4_zero_input():
    cfg = _cfg("i4_0", T=9, H=256, I=128, E=4, k=2)
    inp = synth.draw_inputs(cfg, DEV)
    inp.x.zero_()
    out = moe.MoELayer(inp).step(inp.logits, inp.x)
    torch.cuda.synchronize()
    assert torch.all(out.float() == 0.0)


def test_int4_prefill_path_refused():
    cfg = _cfg("i4_p", T=64, H=256, I=128, E=4, k=2)
    inp = synth.draw_inputs(cfg, DEV)
    layer = moe.MoELayer(inp, path=moe.PATH_PREFILL)
    with pytest.raises(moe.MoEError) as ei:
        layer.step(inp.logits, inp.x)
    assert ei.value.status == 2 and "decode kernels only" in str(ei.value)


@pytest.mark.slow
def test_int4_workload_dsr1_decode():
    """DeepSeek-R1-shaped decode batch (T = 4, 256 experts top-8 + shared)
    with INT4 experts, as the benchmark runs it; every token."""
    cfg = synth.EXTRA_CONFIGS["c2_int4"]
    _say("int4 workload", cfg.name)
    inp = synth.draw_inputs(cfg, DEV)
    layer = moe.MoELayer(inp)
    out = layer.step(inp.logits, inp.x).clone()
    torch.cuda.synchronize()
    rel, mx = check_close(out, oracle_routed_layer(inp), cfg.name)
    _say(f"  {cfg.name}: rel-L2 {rel:.2e}, max-abs/max|ref| {mx:.2e}")
