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


@pytest.mark.parametrize("wd,path", [(synth.WDTYPE_FP8, moe.PATH_AUTO),
                                     (synth.WDTYPE_INT8, moe.PATH_AUTO),
                                     (synth.WDTYPE_BF16, moe.PATH_PREFILL)])
def test_noalloc_equals_workspace_entry(wd, path):
    big = synth.MoEConfig("noalloc", T=48, H=1024, I=512, E=64, k=8, wdtype=wd, score=1, renorm=1,
                          shared=wd != synth.WDTYPE_INT8)
    print("noalloc", wd, path, flush=True)
    inp = synth.draw_inputs(big, DEV)
    first = None
    for T in (48, 5):  # second call smaller than the first
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
