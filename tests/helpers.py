"""Shared pieces of the GPU parity tests: the output tolerance and running the
oracle on the experts a subset of tokens needs."""
import numpy as np
import torch

import oracle
from mixture_experts_ffn_topk_amd import synth

# Output tolerance of the fused layer against the oracle: relative L2 error over
# all compared elements (fp64) <= 1e-2 and max |err| <= 2e-2 * max |ref|.
REL_L2 = 1e-2
MAX_ABS_FRAC = 2e-2


def bf16_to_f64(t) -> np.ndarray:
    if isinstance(t, torch.Tensor):
        return t.detach().to("cpu").to(torch.float64).numpy()
    return oracle.bf16_bits_to_f64(t)


def check_close(got, ref, what=""):
    g = bf16_to_f64(got).reshape(-1)
    r = bf16_to_f64(ref).reshape(-1)
    assert np.all(np.isfinite(g)), f"{what}: non-finite output"
    err = g - r
    nref = np.linalg.norm(r)
    rel = np.linalg.norm(err) / max(nref, 1e-300)
    mx = np.abs(err).max() if err.size else 0.0
    lim = MAX_ABS_FRAC * max(np.abs(r).max(), 1e-300)
    assert rel <= REL_L2, f"{what}: rel-L2 {rel:.3e} > {REL_L2}"
    assert mx <= lim, f"{what}: max-abs {mx:.3e} > {lim:.3e}"
    return rel, mx / max(np.abs(r).max(), 1e-300)


def oracle_layer(inp: synth.MoEInputs, topk_w, topk_ids, tokens=None):
    """Oracle output (bf16 bits, [n, H]) for `tokens` (default all), fetching
    only the experts those tokens route to."""
    cfg = inp.cfg
    ids = np.asarray(topk_ids.cpu() if isinstance(topk_ids, torch.Tensor) else topk_ids)
    tw = np.asarray(topk_w.cpu() if isinstance(topk_w, torch.Tensor) else topk_w,
                    dtype=np.float32)
    toks = np.arange(cfg.T) if tokens is None else np.asarray(tokens)
    used = sorted(set(int(e) for e in ids[toks].reshape(-1)))
    remap = {e: n for n, e in enumerate(used)}
    sub_ids = np.vectorize(lambda e: remap.get(int(e), 0))(ids).astype(np.int32)
    sel = torch.tensor(used, dtype=torch.long, device=inp.w13.device)

    def pick(w):  # index_select has no uint16 kernel: go through int16
        if w.dtype == torch.uint16:
            return w.view(torch.int16).index_select(0, sel).view(torch.uint16).cpu()
        return w.index_select(0, sel).cpu()

    w13 = pick(inp.w13)
    w2 = pick(inp.w2)
    s13 = None if inp.w13_scale is None else inp.w13_scale.index_select(0, sel).cpu()
    s2 = None if inp.w2_scale is None else inp.w2_scale.index_select(0, sel).cpu()
    cpu = lambda t: None if t is None else t.cpu()
    x = inp.x.cpu()
    return oracle.moe(cfg.wdtype, x, w13, s13, w2, s2, tw, sub_ids, cpu(inp.sh13),
                      cpu(inp.sh13_scale), cpu(inp.sh2), cpu(inp.sh2_scale),
                      tokens=np.asarray(toks, np.int32))
