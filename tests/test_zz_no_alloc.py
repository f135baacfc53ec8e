"""GPU: fused_moe_routed_noalloc (no workspace argument; the library's static
per-GPU scratch) gives exactly what fused_moe_routed gives with a caller
workspace, on two calls in a row (the second with fewer tokens, so the
scratch holds the first call's larger contents), and matches the oracle to
the output tolerance."""
import numpy as np
import pytest
import torch

from mixture_experts_ffn_topk_amd import _lib as moe
from mixture_experts_ffn_topk_amd import synth
from helpers import check_close, oracle_layer

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _noalloc_step(layer, logits, x):
    c = layer.cfg
    tw = torch.empty(c.T, c.k, dtype=torch.float32, device=DEV)
    ti = torch.empty(c.T, c.k, dtype=torch.int32, device=DEV)
    out = torch.empty(c.T, c.H, dtype=torch.bfloat16, device=DEV)
    moe.fused_moe_routed_noalloc(c.wdtype, logits, c.k, c.score, c.renorm, x, layer.w13, layer.s13,
                                 layer.w2, layer.s2, tw, ti, out, layer.shared, layer.path,
                                 layer.split_k)
    return out, tw, ti


# (T of the two calls, I, E, k): a 48-token batch then 5 tokens; and a tiny
# INT8 batch (at most 8 pairs, GEMM2 unsplit: GEMM2 takes the combine) of
# 3 tokens then 1
SHAPES = {"T48": ((48, 5), 512, 64, 8), "tiny": ((3, 1), 128, 16, 2)}


@pytest.mark.parametrize("wd,path,shape", [(synth.WDTYPE_FP8, moe.PATH_AUTO, "T48"),
                                           (synth.WDTYPE_INT8, moe.PATH_AUTO, "T48"),
                                           (synth.WDTYPE_BF16, moe.PATH_PREFILL, "T48"),
                                           (synth.WDTYPE_INT8, moe.PATH_AUTO, "tiny")])
def test_noalloc_equals_workspace_entry(wd, path, shape):
    Ts, I, E, k = SHAPES[shape]
    big = synth.MoEConfig("noalloc", T=Ts[0], H=1024, I=I, E=E, k=k, wdtype=wd, score=1, renorm=1,
                          shared=wd != synth.WDTYPE_INT8)
    print("noalloc", wd, path, shape, flush=True)
    inp = synth.draw_inputs(big, DEV)
    first = None
    for T in Ts:  # second call smaller than the first
        cfg = big.with_T(T)
        sub = synth.MoEInputs(cfg, inp.logits[:T].contiguous(), inp.x[:T].contiguous(), inp.w13,
                              inp.w13_scale, inp.w2, inp.w2_scale, inp.sh13, inp.sh13_scale,
                              inp.sh2, inp.sh2_scale)
        layer = moe.MoELayer(sub, path=path, packed_from=first)
        first = first or layer
        got, tw, ti = _noalloc_step(layer, sub.logits, sub.x)
        torch.cuda.synchronize()
        want = layer.step(sub.logits, sub.x)
        torch.cuda.synchronize()
        assert torch.equal(ti, layer.ti), f"T={T}: top-k ids differ"
        assert torch.equal(tw, layer.tw), f"T={T}: top-k weights differ"
        assert torch.equal(got.view(torch.int16), want.view(torch.int16)), f"T={T}: outputs differ"
        check_close(got, oracle_layer(sub, tw, ti), f"noalloc T={T}")
