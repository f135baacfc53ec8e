"""GPU parity of the routing-side entry points against the oracle, through the
C ABI: top-k ids bit-exact (weights to fp32 rounding), alignment bit-exact,
INT8 row quantiser bit-exact, FP8 converters on all 256 codes."""
import itertools
import math

import numpy as np
import pytest
import torch

import oracle
from mixture_experts_ffn_topk_amd import _lib as moe
from mixture_experts_ffn_topk_amd import synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _say(*a):
    print(*a, flush=True)


@pytest.mark.parametrize("name", list(synth.CONFIGS))
def test_topk_matches_oracle(name):
    cfg = synth.CONFIGS[name]
    _say("topk", name)
    lg = synth.draw_logits(cfg, DEV)
    w, ids = moe.topk(lg, cfg.k, cfg.score, cfg.renorm)
    torch.cuda.synchronize()
    rw, rids = oracle.topk(lg.cpu(), cfg.k, cfg.score, cfg.renorm)
    np.testing.assert_array_equal(ids.cpu().numpy(), rids)
    np.testing.assert_allclose(w.cpu().numpy().astype(np.float64), rw, rtol=2e-6, atol=1e-7)


@pytest.mark.parametrize("E,k,score,renorm", [(8, 2, 0, 1), (256, 8, 1, 1), (128, 8, 0, 0),
                                              (1, 1, 0, 1), (5, 5, 1, 0), (1000, 32, 0, 1),
                                              (64, 3, 1, 1), (65, 7, 0, 1)])
def test_topk_shapes_and_ties(E, k, score, renorm):
    _say("topk", E, k, score, renorm)
    g = torch.Generator(device=DEV).manual_seed(E * 31 + k)
    T = 77
    lg = torch.randn(T, E, generator=g, device=DEV)
    lg[0, :] = 0.5                       # all equal
    lg[1, : min(E, 9)] = 2.0             # leading ties
    lg[2] = torch.round(lg[2] * 2) / 2   # many ties
    w, ids = moe.topk(lg, k, score, renorm)
    torch.cuda.synchronize()
    rw, rids = oracle.topk(lg.cpu(), k, score, renorm)
    np.testing.assert_array_equal(ids.cpu().numpy(), rids)
    np.testing.assert_allclose(w.cpu().numpy().astype(np.float64), rw, rtol=2e-6, atol=1e-7)


def _align_case(flat, T, k, E, B):
    ids = torch.from_numpy(np.asarray(flat, np.int32).reshape(T, k)).to(DEV)
    s, eids, npp = moe.align_block_size(ids, E, B)
    torch.cuda.synchronize()
    rs, re, rn = oracle.align(np.asarray(flat, np.int32).reshape(T, k), E, B)
    assert int(npp.item()) == rn
    np.testing.assert_array_equal(s.cpu().numpy(), rs)
    np.testing.assert_array_equal(eids.cpu().numpy(), re)


def test_align_exhaustive_tiny():
    _say("align exhaustive tiny")
    n = 0
    for T, k, E, B in itertools.product([1, 2, 3], [1, 2], [1, 2, 3], [1, 2, 4]):
        if k > E:
            continue
        rows = list(itertools.permutations(range(E), k))
        for c in itertools.product(rows, repeat=T):
            _align_case(np.array(c).reshape(-1), T, k, E, B)
            n += 1
    assert n > 300


@pytest.mark.parametrize("B", [1, 2, 16, 64, 128, 256])
@pytest.mark.parametrize("name", ["c1", "c2", "c3", "c4", "c5_T1", "c5_T32", "c5_T2048"])
def test_align_matches_oracle_on_workloads(name, B):
    cfg = synth.CONFIGS[name]
    _say("align", name, B)
    lg = synth.draw_logits(cfg, DEV)
    _, ids = moe.topk(lg, cfg.k, cfg.score, cfg.renorm)
    _align_case(ids.cpu().numpy().reshape(-1), cfg.T, cfg.k, cfg.E, B)


def test_align_skewed_and_large():
    _say("align skewed")
    rng = np.random.default_rng(0)
    # all pairs on two experts, one untouched expert in between; P > one wave segment
    T, k, E = 5000, 2, 7
    flat = np.stack([np.full(T, 3), np.full(T, 5)], 1).reshape(-1)
    _align_case(flat, T, k, E, 16)
    # random large, many experts (E > 512 exercises the 8-wave layout)
    for E, T, k, B in [(1024, 3000, 8, 16), (600, 2048, 6, 4), (300, 12000, 8, 64)]:
        flat = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).reshape(-1)
        _align_case(flat, T, k, E, B)


def test_align_deterministic():
    _say("align determinism")
    cfg = synth.CONFIGS["c4"]
    lg = synth.draw_logits(cfg, DEV)
    _, ids = moe.topk(lg, cfg.k, cfg.score, cfg.renorm)
    first = [t.clone() for t in moe.align_block_size(ids, cfg.E, 16)]
    for _ in range(5):
        again = moe.align_block_size(ids, cfg.E, 16)
        for a, b in zip(first, again):
            assert torch.equal(a, b)


def test_quant_rows_bit_exact():
    _say("quant rows")
    g = torch.Generator(device=DEV).manual_seed(3)
    x = (torch.randn(300, 4096, generator=g, device=DEV) *
         torch.logspace(-30, 30, 300, device=DEV)[:, None]).to(torch.bfloat16)
    x[5] = 0
    x[6, 7] = 3.0e38
    x[7, :8] = torch.tensor([127.0, 63.5, -0.5, 1.5, 2.5, -126.5, 0.0, 1.0])
    x[7, 8:] = 0
    q, s = moe.quant_int8_rows(x)
    torch.cuda.synchronize()
    rq, rs = oracle.quant_int8_rows(x.float().cpu())
    np.testing.assert_array_equal(s.cpu().numpy(), rs)
    np.testing.assert_array_equal(q.cpu().numpy(), rq)


def test_quant_rows_golden():
    _say("quant golden")
    import json, os
    gold = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "quant_int8.json")))
    for case in gold["cases"]:
        xs = case["x"] + [0.0] * (-len(case["x"]) % 8)
        x = torch.tensor([xs], dtype=torch.float32).to(torch.bfloat16).to(DEV)
        if not torch.equal(x.float().cpu()[0, : len(case["x"])],
                           torch.tensor(case["x"], dtype=torch.float32)):
            continue  # value not representable in bf16: covered by the oracle pins
        q, s = moe.quant_int8_rows(x)
        assert q.cpu().numpy()[0, : len(case["q"])].tolist() == case["q"]


def test_fp8_decode_all_codes():
    _say("fp8 codes")
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8).reshape(2, 128).to(DEV)
    got = moe.dequant_fp8(codes, None, mode=0).cpu().numpy().reshape(-1)
    for c in range(256):
        ref = oracle.e4m3fn_to_double(c)
        if math.isnan(ref):
            assert math.isnan(got[c]), c
        else:
            assert got[c] == ref and math.copysign(1, got[c]) == math.copysign(1, ref), c


def test_fp8_block_dequant_both_converters():
    _say("fp8 block dequant")
    g = torch.Generator(device=DEV).manual_seed(9)
    K, N = 256, 384
    codes = torch.randint(0, 256, (K, N), generator=g, device=DEV, dtype=torch.int32)
    codes = codes.to(torch.uint8)
    codes[codes == 0x7F] = 0x7E
    codes[codes == 0xFF] = 0xFE
    scale = torch.rand(K // 128, N // 128, generator=g, device=DEV) * 1e-3 + 1e-4
    exact = moe.dequant_fp8(codes, scale, mode=0).cpu().numpy().astype(np.float64)
    rounded = moe.dequant_fp8(codes, scale, mode=1).cpu().numpy().astype(np.float64)
    cn = codes.cpu().numpy()
    sn = scale.cpu().numpy().astype(np.float64)
    lut = np.array([oracle.e4m3fn_to_double(c) for c in range(256)])
    ref = lut[cn] * np.repeat(np.repeat(sn, 128, 0), 128, 1)
    np.testing.assert_allclose(exact, ref, rtol=2 ** -24, atol=0)  # one fp32 rounding
    refb = oracle.bf16_bits_to_f64(np.vectorize(oracle.double_to_bf16)(ref))
    ulp = np.abs(refb) * 2.0 ** -7
    assert np.all(np.abs(rounded - refb) <= ulp + 1e-45)
    assert np.mean(rounded == refb) > 0.999
