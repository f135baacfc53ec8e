"""GPU: the opt-in FP8-activation variant of the FP8 tile kernels (moe_options
fp8_activations = 1).  Both GEMM inputs are quantised to E4M3FN per row and
128-element K block with power-of-two scales, each product is one FP8 MFMA.

- The token rows' codes and scale bytes the call leaves in its workspace equal
  oracle.quant_fp8_act_row bit for bit (the same decision in the same
  precision: bf16 values times a power of two, rounded to nearest even).
- The layer output matches the FP8-activation oracle (ORC_FP8_ACT8) to the
  output tolerance; the intermediate is rounded to bf16 before it is
  quantised, the oracle quantises its fp64 value, so a few codes may differ.
- Against the bf16-activation (weight-only) oracle the variant is a few
  percent off in relative L2, as 3-bit-mantissa activations are: the
  tolerance report asserts it stays in that band."""
import numpy as np
import pytest
import torch

import oracle
from mixture_experts_ffn_topk_amd import _lib as moe
from mixture_experts_ffn_topk_amd import synth
from helpers import check_close, oracle_layer, oracle_routing, tile_tokens, read_alignment

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _say(*a):
    print(*a, flush=True)


def _act8_ref(inp, tw, ti, tokens=None):
    """Oracle output with FP8 activations for `tokens` (bf16 bits)."""
    cfg = inp.cfg
    cpu = lambda t: None if t is None else t.cpu()
    toks = np.arange(cfg.T) if tokens is None else np.asarray(tokens)
    return oracle.moe(oracle.FP8_ACT8, inp.x.cpu(), inp.w13.cpu(), inp.w13_scale.cpu(),
                      inp.w2.cpu(), inp.w2_scale.cpu(), np.asarray(tw.cpu(), np.float32),
                      ti.cpu().numpy(), cpu(inp.sh13), cpu(inp.sh13_scale), cpu(inp.sh2),
                      cpu(inp.sh2_scale), tokens=np.asarray(toks, np.int32))


def _check_token_codes(layer, x):
    """Records [T, H/64, 64 B] and scale bytes [T, stride] in the workspace vs
    the oracle's quantiser, bit for bit."""
    lay = layer.layout()
    T, H = x.shape
    rec = layer.ws[lay["xq"]:lay["xq"] + T * H].cpu().numpy().reshape(T, H // 64, 4, 16)
    stride = lay["xs_stride"]
    assert stride >= H // 128 and stride % 16 == 0
    ex = layer.ws[lay["xs"]:lay["xs"] + T * stride].cpu().numpy().reshape(T, stride)
    # record part p of stage st: k = 64 st + 8p .. +7, then 64 st + 32 + 8p .. +7
    k_of = np.empty((H // 64, 4, 16), np.int64)
    for st in range(H // 64):
        for p in range(4):
            k_of[st, p, :8] = 64 * st + 8 * p + np.arange(8)
            k_of[st, p, 8:] = 64 * st + 32 + 8 * p + np.arange(8)
    xf = x.float().cpu().numpy().astype(np.float64)
    for t in range(T):
        codes, exps, _ = oracle.quant_fp8_act_row(xf[t])
        got = np.empty(H, np.uint8)
        got[k_of.reshape(-1)] = rec[t].reshape(-1)
        assert np.array_equal(got, codes), f"token {t}: codes differ"
        assert np.array_equal(ex[t, :H // 128].astype(np.int64), 127 - exps.astype(np.int64)), \
            f"token {t}: scale bytes differ"


CASES = {
    # several row blocks, column groups and K blocks; ragged T; a half-full last
    # 256-column group (H = 640); scale-byte rows of 16 and 128 bytes
    "ragged_shared": synth.MoEConfig("a8_r", T=70, H=640, I=384, E=6, k=2, wdtype=synth.WDTYPE_FP8,
                                     score=1, renorm=1, shared=True),
    "zipf_many_experts": synth.MoEConfig("a8_z", T=200, H=1024, I=256, E=32, k=8,
                                         wdtype=synth.WDTYPE_FP8, score=1, renorm=1, shared=True,
                                         routing="zipf"),
    "wide_k": synth.MoEConfig("a8_w", T=40, H=16384, I=128, E=4, k=1, wdtype=synth.WDTYPE_FP8,
                              score=0, renorm=1, shared=False),
}


@pytest.mark.parametrize("name", list(CASES))
def test_fp8_act_layer_matches_act8_oracle(name):
    cfg = CASES[name]
    _say("fp8 act layer", name)
    inp = synth.draw_inputs(cfg, DEV)
    layer = moe.MoELayer(inp, path=moe.PATH_PREFILL, fp8_act=1)
    out = layer.step(inp.logits, inp.x).clone()
    torch.cuda.synchronize()
    _check_token_codes(layer, inp.x)
    tw, ti = oracle_routing(inp)
    np.testing.assert_array_equal(layer.ti.cpu().numpy(), ti)
    rel, mx = check_close(out, _act8_ref(inp, torch.from_numpy(tw), torch.from_numpy(ti)), name)
    _say(f"  {name}: vs FP8-activation oracle rel-L2 {rel:.2e}, max-abs/max|ref| {mx:.2e}")


def test_fp8_act_special_block_scales_and_zero_rows():
    """Zero, subnormal and scaled-up weight block scales, an all-zero token row
    (its blocks take e = 0 and zero codes) and an all-zero 128-block inside a
    row."""
    cfg = synth.MoEConfig("a8_sc", T=64, H=512, I=256, E=6, k=2, wdtype=synth.WDTYPE_FP8,
                          score=1, renorm=1, shared=True)
    _say("fp8 act special scales")
    inp = synth.draw_inputs(cfg, DEV)
    inp.w13_scale[0, 1, 0] = 0.0
    inp.w13_scale[2, 0, 1] = 1e-40
    inp.w13_scale[3, 3, 2] *= 256.0
    inp.w2_scale[4, 0, 1] = 0.0
    inp.sh2_scale[1, 0] *= 256.0
    inp.x[5] = 0
    inp.x[9, 128:256] = 0
    layer = moe.MoELayer(inp, path=moe.PATH_PREFILL, fp8_act=1)
    out = layer.step(inp.logits, inp.x).clone()
    torch.cuda.synchronize()
    _check_token_codes(layer, inp.x)
    tw, ti = oracle_routing(inp)
    check_close(out, _act8_ref(inp, torch.from_numpy(tw), torch.from_numpy(ti)), "act8 scales")


def test_fp8_act_zero_input():
    cfg = synth.MoEConfig("a8_0", T=33, H=256, I=256, E=8, k=2, wdtype=synth.WDTYPE_FP8,
                          score=1, renorm=1, shared=True)
    inp = synth.draw_inputs(cfg, DEV)
    inp.x.zero_()
    layer = moe.MoELayer(inp, path=moe.PATH_PREFILL, fp8_act=1)
    out = layer.step(inp.logits, inp.x)
    torch.cuda.synchronize()
    assert torch.all(out.float() == 0.0)


def test_fp8_act_ignored_by_decode_kernels():
    """The decode kernels stream FP8 weights against bf16 activations with or
    without the option: the same bits."""
    cfg = synth.MoEConfig("a8_d", T=4, H=512, I=256, E=16, k=4, wdtype=synth.WDTYPE_FP8,
                          score=1, renorm=1, shared=True)
    inp = synth.draw_inputs(cfg, DEV)
    a = moe.MoELayer(inp, path=moe.PATH_DECODE).step(inp.logits, inp.x).clone()
    b = moe.MoELayer(inp, path=moe.PATH_DECODE, fp8_act=1).step(inp.logits, inp.x).clone()
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.slow
def test_fp8_act_workload_c4():
    """The DeepSeek-R1-shaped prefill (T = 4096) with FP8 activations: the
    token of the last real row of every (expert, chunk) tile plus spread
    tokens against the FP8-activation oracle (output tolerance), and the
    tolerance report against the bf16-activation oracle."""
    cfg = synth.CONFIGS["c4"]
    _say("fp8 act c4")
    inp = synth.draw_inputs(cfg, DEV)
    layer = moe.MoELayer(inp, fp8_act=1)
    out = layer.step(inp.logits, inp.x).clone()
    torch.cuda.synchronize()
    _check_token_codes(layer, inp.x)
    tw, ti = oracle_routing(inp)
    np.testing.assert_array_equal(layer.ti.cpu().numpy(), ti)
    sorted_ids, _, chunks, _ = read_alignment(layer)
    toks = tile_tokens(sorted_ids, chunks, cfg, np.linspace(0, cfg.T - 1, 16).round())
    _say(f"  c4 act8: oracle on {len(toks)} tokens")
    tw_t, ti_t = torch.from_numpy(tw), torch.from_numpy(ti)
    got = out[torch.from_numpy(toks).to(DEV)]
    rel, mx = check_close(got, _act8_ref(inp, tw_t, ti_t, toks), "c4 act8")
    _say(f"  c4 act8 vs FP8-activation oracle: rel-L2 {rel:.2e}, max-abs/max|ref| {mx:.2e}")
    ref16 = oracle_layer(inp, tw_t, ti_t, toks)
    g = got.double().cpu().numpy()
    r = oracle.bf16_bits_to_f64(ref16)
    rel16 = np.linalg.norm(g - r) / np.linalg.norm(r)
    _say(f"  c4 act8 vs bf16-activation oracle (tolerance report): rel-L2 {rel16:.3e}")
    assert 0.005 < rel16 < 0.08
