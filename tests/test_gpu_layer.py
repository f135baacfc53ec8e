"""GPU parity of the fused layer (top-k -> align -> GEMM1+SiLU -> GEMM2 ->
combine) against the oracle, through the C ABI.

Small cases run the oracle on every output element (several tiles per
dimension, ragged token counts, both kernel families forced, split-K
variants); the workload-sized cases run exactly what the benchmark times and
compare sampled tokens that the oracle evaluates one by one.  Tolerance:
relative L2 <= 1e-2 and max-abs <= 2e-2 * max|ref| (tests/helpers.py)."""
import numpy as np
import pytest
import torch

import oracle
from mixture_experts_ffn_topk_amd import _lib as moe
from mixture_experts_ffn_topk_amd import synth
from helpers import (check_alignment, check_close, oracle_layer, oracle_quant_check,
                     oracle_routed_layer, oracle_routing, tile_tokens)

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
PATHS = {"auto": moe.PATH_AUTO, "decode": moe.PATH_DECODE, "prefill": moe.PATH_PREFILL}


def _say(*a):
    print(*a, flush=True)


def _run(inp, path=moe.PATH_AUTO, split_k=0, tw=None, ti=None):
    layer = moe.MoELayer(inp, path=path, split_k=split_k)
    if tw is None:
        tw, ti = layer.route(inp.logits)
        tw, ti = tw.clone(), ti.clone()
    out = layer.ffn(inp.x, tw, ti).clone()
    torch.cuda.synchronize()
    return out, tw, ti, layer


SMALL = {
    # name: config (several tiles in H and I, a ragged T)
    "bf16_tiny": synth.CONFIGS["c1"],
    "bf16_ragged": synth.MoEConfig("bf16_ragged", T=37, H=384, I=256, E=6, k=2,
                                   wdtype=synth.WDTYPE_BF16, score=0, renorm=1, shared=True),
    "fp8_sigmoid_shared": synth.MoEConfig("fp8_s", T=29, H=512, I=256, E=16, k=4,
                                          wdtype=synth.WDTYPE_FP8, score=1, renorm=1,
                                          shared=True),
    "fp8_zipf": synth.MoEConfig("fp8_z", T=40, H=256, I=384, E=32, k=8, wdtype=synth.WDTYPE_FP8,
                                score=1, renorm=1, shared=True, routing="zipf"),
    "int8_softmax": synth.MoEConfig("int8_s", T=33, H=512, I=384, E=12, k=3,
                                    wdtype=synth.WDTYPE_INT8, score=0, renorm=1),
    "int8_shared_norenorm": synth.MoEConfig("int8_n", T=9, H=256, I=256, E=5, k=2,
                                            wdtype=synth.WDTYPE_INT8, score=0, renorm=0,
                                            shared=True),
    # H = 384: the INT8 prefill GEMM2's last 256-column group is half full
    "int8_partial_cols": synth.MoEConfig("int8_p", T=70, H=384, I=128, E=4, k=2,
                                         wdtype=synth.WDTYPE_INT8, score=1, renorm=1,
                                         shared=True),
}


@pytest.mark.parametrize("path", list(PATHS))
@pytest.mark.parametrize("name", list(SMALL))
def test_layer_small_all_outputs(name, path):
    cfg = SMALL[name]
    _say("layer small", name, path)
    inp = synth.draw_inputs(cfg, DEV)
    out, tw, ti, _ = _run(inp, PATHS[path])
    ref = oracle_layer(inp, tw, ti)
    check_close(out, ref, f"{name}/{path}")


# five 128-row K blocks: K splits of 3+2 and 2+2+1 blocks, so a split runs the
# stream's steady loop and its tail, or the tail alone, with and without loads
K5 = {wd: synth.MoEConfig(f"k5_{wd}", T=37, H=640, I=256, E=6, k=2, wdtype=wd, score=0, renorm=1,
                          shared=(wd != synth.WDTYPE_INT8))
      for wd in (synth.WDTYPE_BF16, synth.WDTYPE_FP8, synth.WDTYPE_INT8)}


@pytest.mark.parametrize("split_k", [1, 2, 3, 4])
@pytest.mark.parametrize("name", ["fp8_sigmoid_shared", "int8_softmax", "bf16_ragged",
                                  "k5_bf16", "k5_fp8", "k5_int8"])
def test_layer_decode_split_k(name, split_k):
    cfg = SMALL[name] if name in SMALL else K5[{"k5_bf16": synth.WDTYPE_BF16, "k5_fp8": synth.WDTYPE_FP8,
                                                "k5_int8": synth.WDTYPE_INT8}[name]]
    _say("layer split-k", name, split_k)
    inp = synth.draw_inputs(cfg, DEV)
    out, tw, ti, _ = _run(inp, moe.PATH_DECODE, split_k)
    check_close(out, oracle_layer(inp, tw, ti), f"{name}/split{split_k}")


# BF16 / INT8 prefill workgroups running several column groups back to back:
# H = 640 gives INT8 2.5 groups of 256 columns in GEMM2 (a half-full last
# group) and BF16 5 groups of 128; I = 384 gives 3 (INT8) or 6 (BF16) GEMM1
# groups, so spans of 2 and 3 leave a shorter last workgroup; 99 is clamped.
SPAN = {wd: synth.MoEConfig(f"span_{wd}", T=70, H=640, I=384, E=4, k=2, wdtype=wd, score=1, renorm=1,
                            shared=True)
        for wd in (synth.WDTYPE_BF16, synth.WDTYPE_INT8)}


@pytest.mark.parametrize("span", [1, 2, 3, 99])
@pytest.mark.parametrize("wd", [synth.WDTYPE_BF16, synth.WDTYPE_INT8])
def test_layer_prefill_group_span(wd, span):
    cfg = SPAN[wd]
    _say("layer prefill span", wd, span)
    inp = synth.draw_inputs(cfg, DEV)
    layer = moe.MoELayer(inp, path=moe.PATH_PREFILL, span=span)
    tw, ti = layer.route(inp.logits)
    tw, ti = tw.clone(), ti.clone()
    out = layer.ffn(inp.x, tw, ti).clone()
    torch.cuda.synchronize()
    check_close(out, oracle_layer(inp, tw, ti), f"span{span}/{wd}")


@pytest.mark.parametrize("wd", [synth.WDTYPE_BF16, synth.WDTYPE_FP8, synth.WDTYPE_INT8])
def test_layer_prefill_partial_column_group(wd):
    """H = 640 on the prefill kernels: FP8 and INT8 GEMM2 end in a half-full
    256-column group (BF16: five 128-column groups)."""
    cfg = K5[wd]
    _say("layer prefill partial group", wd)
    inp = synth.draw_inputs(cfg, DEV)
    out, tw, ti, _ = _run(inp, moe.PATH_PREFILL)
    check_close(out, oracle_layer(inp, tw, ti), f"prefill partial/{wd}")


@pytest.mark.parametrize("span", [1, 2])
@pytest.mark.parametrize("kb", [1, 2, 3, 4, 5, 6, 7, 8, 9, 10])
def test_layer_int8_prefill_stage_counts(kb, span):
    """INT8 prefill with H = 128 * kb (2 * kb stages of 64 per column group)
    and one or two groups per workgroup: every count of stages modulo the
    weight waves' register-ring unroll, so every tail of that ring runs."""
    cfg = synth.MoEConfig(f"i8_kb{kb}", T=40, H=128 * kb, I=256, E=4, k=2, wdtype=synth.WDTYPE_INT8,
                          score=0, renorm=1, shared=(kb % 2 == 0))
    _say("layer int8 prefill stages", kb, span)
    inp = synth.draw_inputs(cfg, DEV)
    layer = moe.MoELayer(inp, path=moe.PATH_PREFILL, span=span)
    tw, ti = layer.route(inp.logits)
    tw, ti = tw.clone(), ti.clone()
    out = layer.ffn(inp.x, tw, ti).clone()
    torch.cuda.synchronize()
    check_close(out, oracle_layer(inp, tw, ti), f"int8 prefill kb={kb} span={span}")


@pytest.mark.parametrize("path", ["decode", "prefill"])
@pytest.mark.parametrize("wd", [synth.WDTYPE_BF16, synth.WDTYPE_FP8, synth.WDTYPE_INT8])
def test_layer_hot_expert_many_chunks(wd, path):
    """One expert takes every token (rows >> chunk size), one gets a single
    token, the rest none: multi-chunk experts, lone rows, empty experts."""
    cfg = synth.MoEConfig("hot", T=300, H=256, I=256, E=9, k=2, wdtype=wd, score=1, renorm=1,
                          shared=(wd != synth.WDTYPE_INT8))
    _say("layer hot expert", wd, path)
    inp = synth.draw_inputs(cfg, DEV)
    inp.logits[:, 4] += 20.0
    inp.logits[0, 7] += 40.0
    inp.logits[1:, 6] += 10.0
    out, tw, ti, _ = _run(inp, PATHS[path])
    assert int((ti == 4).sum()) == cfg.T
    check_close(out, oracle_layer(inp, tw, ti), f"hot/{wd}/{path}")


@pytest.mark.parametrize("path", ["decode", "prefill"])
def test_layer_single_token_single_expert(path):
    cfg = synth.MoEConfig("one", T=1, H=128, I=128, E=1, k=1, wdtype=synth.WDTYPE_FP8,
                          score=0, renorm=1)
    _say("layer T=1 E=1", path)
    inp = synth.draw_inputs(cfg, DEV)
    out, tw, ti, _ = _run(inp, PATHS[path])
    check_close(out, oracle_layer(inp, tw, ti), "one")


@pytest.mark.parametrize("path", ["decode", "prefill"])
def test_layer_fp8_special_block_scales(path):
    """Zero, subnormal and large 128x128 block scales (codes left as drawn):
    a zero scale contributes nothing, a subnormal one keeps its tiny value,
    a scaled-up block neither overflows nor disturbs its neighbours.  The
    prefill path splits every scale into an MFMA exponent and a rescaled
    mantissa, so these are its edge cases."""
    cfg = synth.MoEConfig("fp8_sc", T=64, H=512, I=256, E=6, k=2, wdtype=synth.WDTYPE_FP8,
                          score=1, renorm=1, shared=True)
    _say("layer fp8 block scales", path)
    inp = synth.draw_inputs(cfg, DEV)
    inp.w13_scale[0, 1, 0] = 0.0        # gate block, K block 1
    inp.w13_scale[1, 2, 3] = 0.0        # up block
    inp.w13_scale[2, 0, 1] = 1e-40      # subnormal fp32
    inp.w13_scale[3, 3, 2] *= 256.0
    inp.w2_scale[4, 0, 1] = 0.0
    inp.w2_scale[5, 1, 3] = 3e-39       # subnormal fp32
    inp.sh13_scale[2, 1] = 0.0
    inp.sh2_scale[1, 0] *= 256.0
    out, tw, ti, _ = _run(inp, PATHS[path])
    check_close(out, oracle_layer(inp, tw, ti), f"fp8 scales/{path}")


@pytest.mark.parametrize("path", ["decode", "prefill"])
def test_layer_graph_replay(path):
    """One layer step captured in a HIP graph: every replay, with eager steps
    on other routings and host synchronisations in between, reproduces the
    eager output bit for bit (the call path records no memsets and no
    allocations)."""
    cfg = SMALL["fp8_zipf"]
    _say("layer graph replay", path)
    inp = synth.draw_inputs(cfg, DEV)
    layer = moe.MoELayer(inp, path=PATHS[path])
    other = synth.draw_logits(cfg, DEV, seed=cfg.seed + 11)
    want = layer.step(inp.logits, inp.x).clone()
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        layer.step(inp.logits, inp.x)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        layer.step(inp.logits, inp.x)
    torch.cuda.synchronize()
    for rep in range(4):
        layer.step(other, inp.x)  # eager work on another routing in between
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(layer.out, want), f"replay {rep} differs from the eager step"
    check_close(want, oracle_layer(inp, layer.tw.clone(), layer.ti.clone()), f"graph/{path}")


def test_layer_graph_replay_many_pairs():
    """The many-workgroup alignment (9900 pairs) and INT8 prefill workgroups
    running two column groups each, captured in a HIP graph: every replay
    equals the eager step bit for bit."""
    cfg = synth.MoEConfig("graph_many", T=1100, H=640, I=384, E=16, k=8, wdtype=synth.WDTYPE_INT8,
                          score=1, renorm=1, shared=True)
    _say("layer graph replay many pairs")
    inp = synth.draw_inputs(cfg, DEV)
    layer = moe.MoELayer(inp, path=moe.PATH_PREFILL, span=2)
    other = synth.draw_logits(cfg, DEV, seed=cfg.seed + 13)
    want = layer.step(inp.logits, inp.x).clone()
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        layer.step(inp.logits, inp.x)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        layer.step(inp.logits, inp.x)
    torch.cuda.synchronize()
    for rep in range(3):
        layer.step(other, inp.x)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(layer.out, want), f"replay {rep} differs from the eager step"
    toks = np.unique(np.linspace(0, cfg.T - 1, 24).round().astype(int))
    check_close(want[torch.from_numpy(toks).to(DEV)],
                oracle_layer(inp, layer.tw.clone(), layer.ti.clone(), toks), "graph many pairs")


ROUTED = [
    # (T, H, I, E, k, wdtype, score, renorm, shared): both sides of the
    # one-workgroup top-k + alignment threshold (16 tokens), every weight type,
    # up to 1000 experts (16 logits per lane) and k = 32
    (1, 256, 128, 128, 8, synth.WDTYPE_INT8, 0, 1, False),
    (4, 512, 256, 256, 8, synth.WDTYPE_FP8, 1, 1, True),
    (16, 256, 128, 8, 2, synth.WDTYPE_BF16, 0, 1, False),
    (32, 256, 256, 64, 6, synth.WDTYPE_FP8, 0, 0, True),
    (33, 256, 128, 64, 4, synth.WDTYPE_INT8, 1, 1, True),
    (64, 256, 128, 1000, 8, synth.WDTYPE_BF16, 1, 1, False),
    (7, 128, 128, 1000, 32, synth.WDTYPE_FP8, 0, 1, True),
]


@pytest.mark.parametrize("case", ROUTED, ids=[f"T{c[0]}_E{c[3]}_k{c[4]}_w{c[5]}" for c in ROUTED])
def test_layer_routed_equals_two_calls(case):
    """fused_moe_routed (top-k and alignment in one workgroup for T <= 16)
    gives exactly the top-k weights, ids and layer output of moe_topk
    followed by fused_moe_ex."""
    T, H, I, E, k, wd, score, renorm, shared = case
    cfg = synth.MoEConfig("routed", T=T, H=H, I=I, E=E, k=k, wdtype=wd, score=score,
                          renorm=renorm, shared=shared)
    _say("layer routed", case)
    inp = synth.draw_inputs(cfg, DEV)
    layer = moe.MoELayer(inp)
    out1 = layer.step(inp.logits, inp.x).clone()
    tw1, ti1 = layer.tw.clone(), layer.ti.clone()
    out2 = layer.step_two_calls(inp.logits, inp.x).clone()
    torch.cuda.synchronize()
    assert torch.equal(ti1, layer.ti), "top-k ids differ"
    assert torch.equal(tw1, layer.tw), "top-k weights differ"
    assert torch.equal(out1, out2), "layer output differs"
    rw, rids = oracle.topk(inp.logits.cpu(), k, score, renorm)
    np.testing.assert_array_equal(ti1.cpu().numpy(), rids)
    check_close(out1, oracle_layer(inp, tw1, ti1), f"routed {case}")


def test_layer_dropped_slot_ids():
    """Out-of-range expert ids are dropped, as documented, and nothing faults."""
    cfg = SMALL["fp8_sigmoid_shared"]
    _say("layer dropped ids")
    inp = synth.draw_inputs(cfg, DEV)
    layer = moe.MoELayer(inp)
    tw, ti = layer.route(inp.logits)
    tw, ti = tw.clone(), ti.clone()
    ti[3, 1] = cfg.E + 5
    ti[4, 0] = -1
    out = layer.ffn(inp.x, tw, ti).clone()
    torch.cuda.synchronize()
    tw_ref = tw.clone()
    ti_ref = ti.clone()
    tw_ref[3, 1] = 0.0
    tw_ref[4, 0] = 0.0
    ti_ref[3, 1] = 0
    ti_ref[4, 0] = 0
    check_close(out, oracle_layer(inp, tw_ref, ti_ref), "dropped")


@pytest.mark.parametrize("wd", [synth.WDTYPE_BF16, synth.WDTYPE_INT8])
def test_layer_prefill_span_bit_identical(wd):
    """The span only changes which workgroup computes a column group, not the
    arithmetic: every span gives the same bits."""
    cfg = SPAN[wd]
    _say("layer prefill span bits", wd)
    inp = synth.draw_inputs(cfg, DEV)
    outs = []
    for span in (1, 2, 3):
        layer = moe.MoELayer(inp, path=moe.PATH_PREFILL, span=span)
        tw, ti = layer.route(inp.logits)
        outs.append(layer.ffn(inp.x, tw, ti).clone())
    torch.cuda.synchronize()
    for o in outs[1:]:
        assert torch.equal(o.view(torch.int16), outs[0].view(torch.int16))


# 9900 pairs (>= 8192 with the shared expert): the alignment runs over many
# workgroups (blocks of 2048 pairs, a short last block).  Every output is
# checked, so a pair dropped or placed twice by the alignment shows up.
MANY_PAIRS = {
    "uniform": synth.MoEConfig("many_u", T=1100, H=256, I=128, E=16, k=8, wdtype=synth.WDTYPE_INT8,
                               score=0, renorm=1, shared=True),
    "zipf": synth.MoEConfig("many_z", T=1100, H=256, I=128, E=40, k=8, wdtype=synth.WDTYPE_BF16,
                            score=1, renorm=1, shared=True, routing="zipf"),
    # 1000 experts: the scan's one thread per expert near its 1024 limit
    "many_experts": synth.MoEConfig("many_e", T=1100, H=128, I=128, E=1000, k=8,
                                    wdtype=synth.WDTYPE_INT8, score=0, renorm=1, shared=False),
}


def test_layer_huge_pair_count_sampled():
    """576,000 pairs: more than 256 blocks of 2048, so the alignment doubles
    its block to 4096 pairs; sampled tokens against the oracle."""
    cfg = synth.MoEConfig("huge_p", T=72000, H=128, I=128, E=64, k=8, wdtype=synth.WDTYPE_INT8,
                          score=0, renorm=1, shared=False)
    _say("layer huge pair count")
    inp = synth.draw_inputs(cfg, DEV)
    layer = moe.MoELayer(inp)
    out = layer.step(inp.logits, inp.x).clone()
    torch.cuda.synchronize()
    tw, ti = layer.tw.clone(), layer.ti.clone()
    toks = np.unique(np.linspace(0, cfg.T - 1, 24).round().astype(int))
    check_close(out[torch.from_numpy(toks).to(DEV)], oracle_layer(inp, tw, ti, toks), "huge pairs")


@pytest.mark.parametrize("name", list(MANY_PAIRS))
def test_layer_many_pairs_alignment(name):
    cfg = MANY_PAIRS[name]
    _say("layer many pairs", name)
    inp = synth.draw_inputs(cfg, DEV)
    inp.logits[:, 3] += 4.0  # one expert far above the rest: several chunks
    layer = moe.MoELayer(inp)
    tw, ti = layer.route(inp.logits)
    tw, ti = tw.clone(), ti.clone()
    # a few dropped slots, spread over the pair blocks
    for t, j in ((5, 1), (400, 0), (700, 7), (1099, 3)):
        ti[t, j] = -1 if t % 2 else cfg.E + 3
    out = layer.ffn(inp.x, tw, ti).clone()
    torch.cuda.synchronize()
    tw_ref, ti_ref = tw.clone(), ti.clone()
    bad = (ti_ref < 0) | (ti_ref >= cfg.E)
    tw_ref[bad] = 0.0
    ti_ref[bad] = 0
    check_close(out, oracle_layer(inp, tw_ref, ti_ref), f"many pairs {name}")


def test_layer_deterministic_and_workspace_reuse():
    cfg = SMALL["fp8_zipf"]
    _say("layer determinism")
    inp = synth.draw_inputs(cfg, DEV)
    for path in (moe.PATH_DECODE, moe.PATH_PREFILL):
        layer = moe.MoELayer(inp, path=path, split_k=3 if path == moe.PATH_DECODE else 0)
        first = layer.step(inp.logits, inp.x).clone()
        for _ in range(4):
            layer.ws.fill_(0xA5)  # garbage workspace must not matter
            again = layer.step(inp.logits, inp.x)
            assert torch.equal(first, again)


def test_expert_id_probe():
    """Each expert's output is a known multiple of its id: a misrouted block
    shows the wrong number.  Gate column reads x0 (large, SiLU ~ identity),
    up column reads x1 = 1, W2 writes (e+1)/64 into every output column."""
    E, H, I, T, k = 12, 128, 128, 23, 2
    w13 = torch.zeros(E, H, 2 * I)
    w2 = torch.zeros(E, I, H)
    for e in range(E):
        w13[e, 0, :I] = 1.0
        w13[e, 1, I:] = 1.0
        w2[e, 0, :] = (e + 1) / 64.0
    x = torch.zeros(T, H)
    x[:, 0] = 16.0
    x[:, 1] = 1.0
    cfg = synth.MoEConfig("probe", T=T, H=H, I=I, E=E, k=k, wdtype=synth.WDTYPE_BF16, score=0,
                          renorm=1)
    inp = synth.MoEInputs(cfg, synth.draw_logits(cfg, DEV), x.to(torch.bfloat16).to(DEV),
                          w13.to(torch.bfloat16).view(torch.uint16).to(DEV), None,
                          w2.to(torch.bfloat16).view(torch.uint16).to(DEV), None)
    _say("expert id probe")
    for path in (moe.PATH_DECODE, moe.PATH_PREFILL):
        out, tw, ti, _ = _run(inp, path)
        silu16 = 16.0 / (1.0 + np.exp(-16.0))
        expect = (tw.cpu().double() * ((ti.cpu().double() + 1) / 64.0)).sum(1) * silu16
        got = out.cpu().double()
        np.testing.assert_allclose(got.numpy(), np.repeat(expect.numpy()[:, None], H, 1),
                                   rtol=1e-2)
        check_close(out, oracle_layer(inp, tw, ti), "probe")


# ---------------------------------------------------------------------------
# Workload sizes, as the benchmark runs them; sampled tokens against the oracle
# ---------------------------------------------------------------------------

_WEIGHTS = {}


def _workload_inputs(name):
    cfg = synth.CONFIGS[name]
    key = (cfg.wdtype, cfg.H, cfg.I, cfg.E, cfg.shared)
    if key not in _WEIGHTS:
        _WEIGHTS.clear()
        torch.cuda.empty_cache()
        w13, s13 = synth.draw_weight_stack(cfg, "w13", DEV)
        w2, s2 = synth.draw_weight_stack(cfg, "w2", DEV)
        sh = (synth.draw_weight_stack(cfg, "sh13", DEV) + synth.draw_weight_stack(cfg, "sh2", DEV)
              if cfg.shared else (None,) * 4)
        _WEIGHTS[key] = (w13, s13, w2, s2) + tuple(sh)
    w13, s13, w2, s2, a, b, c, d = _WEIGHTS[key]
    return synth.MoEInputs(cfg, synth.draw_logits(cfg, DEV), synth.draw_x(cfg, DEV), w13, s13,
                           w2, s2, a, b, c, d)


@pytest.mark.slow
@pytest.mark.parametrize("name", ["c1", "c2", "c3", "c4", "c5_T1", "c5_T32", "c5_T2048"])
def test_layer_workload(name):
    """Each workload exactly as the benchmark times it (one fused_moe_routed
    call, automatic kernel choice).  Bit-exact: the top-k ids, and the
    alignment the call wrote into its workspace (sorted_ids, npp, every
    16-row block's expert, the chunk list; for INT8 also the token rows'
    codes and scales) against the oracle -- these are the variants the timed
    layer runs: the one-workgroup top-k + alignment up to 16 tokens, the
    one-workgroup alignment with shared pairs and chunks, and the
    count/scan/scatter kernels from 8192 pairs.  Outputs: every token up to
    T = 64; at T = 2048 / 4096 the token of the last real row of every
    (expert, chunk) tile the GEMMs run, plus 32 spread tokens, against the
    oracle with its own routing."""
    _say("workload", name)
    inp = _workload_inputs(name)
    cfg = inp.cfg
    layer = moe.MoELayer(inp)
    out = layer.step(inp.logits, inp.x).clone()
    torch.cuda.synchronize()
    tw, ti = layer.tw.clone(), layer.ti.clone()
    rw, rids = oracle_routing(inp)
    np.testing.assert_array_equal(ti.cpu().numpy(), rids)
    np.testing.assert_allclose(tw.cpu().numpy(), rw, rtol=2e-6, atol=0)
    sorted_ids, chunks = check_alignment(layer, ti, name)
    if cfg.wdtype == synth.WDTYPE_INT8:
        oracle_quant_check(layer, inp.x)
    if cfg.T <= 64:
        toks = np.arange(cfg.T)
    else:
        toks = tile_tokens(sorted_ids, chunks, cfg, np.linspace(0, cfg.T - 1, 32).round())
    _say(f"  {name}: {len(chunks)} chunks, oracle on {len(toks)} tokens")
    ref = oracle_routed_layer(inp, toks)
    rel, mx = check_close(out[torch.from_numpy(toks).to(DEV)], ref, name)
    _say(f"  {name}: rel-L2 {rel:.2e}, max-abs/max|ref| {mx:.2e}")
    del layer


@pytest.mark.parametrize("path", ["decode", "prefill"])
@pytest.mark.parametrize("wd", [synth.WDTYPE_BF16, synth.WDTYPE_FP8, synth.WDTYPE_INT8])
def test_layer_zero_input(wd, path):
    """x = 0 gives out = 0 exactly (SiLU(0) * 0 = 0 in every expert; the INT8
    rows quantise with scale 0), as the oracle does."""
    cfg = synth.MoEConfig("zero", T=37, H=256, I=256, E=8, k=2, wdtype=wd, score=1, renorm=1,
                          shared=True)
    _say("layer zero input", wd, path)
    inp = synth.draw_inputs(cfg, DEV)
    inp.x.zero_()
    out, tw, ti, layer = _run(inp, PATHS[path])
    assert torch.all(out.float() == 0.0), "non-zero output for zero input"
    ref = oracle_routed_layer(inp)
    assert np.all(oracle.bf16_bits_to_f64(ref) == 0.0)
    if wd == synth.WDTYPE_INT8:
        oracle_quant_check(layer, inp.x)


@pytest.mark.parametrize("path", ["decode", "prefill"])
def test_layer_int8_all_zero_token_rows(path):
    """INT8: token rows that are all zero quantise to scale 0 and codes 0
    (the amax = 0 case of the quantiser); with no shared expert their outputs
    are exactly 0, and the other rows match the oracle."""
    cfg = synth.MoEConfig("zrow", T=40, H=512, I=256, E=12, k=3, wdtype=synth.WDTYPE_INT8,
                          score=0, renorm=1)
    _say("layer int8 zero rows", path)
    inp = synth.draw_inputs(cfg, DEV)
    zero_rows = [0, 7, 8, 39]
    inp.x[zero_rows] = 0
    layer = moe.MoELayer(inp, path=PATHS[path])
    out = layer.step(inp.logits, inp.x).clone()
    torch.cuda.synchronize()
    oracle_quant_check(layer, inp.x)
    assert torch.all(out[zero_rows].float() == 0.0)
    check_close(out, oracle_routed_layer(inp), f"int8 zero rows/{path}")
