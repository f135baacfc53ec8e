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


def oracle_routed_layer(inp: synth.MoEInputs, tokens=None):
    """Oracle output for `tokens` with the oracle's own routing (its top-k
    ids and weights, the weights cast to fp32)."""
    tw, ti = oracle_routing(inp)
    return oracle_layer(inp, tw, ti, tokens)


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


def oracle_routing(inp: synth.MoEInputs):
    """The oracle's own top-k of inp.logits: (weights as fp32 -- the precision
    the library's boundary carries -- [T, k], ids int32 [T, k])."""
    cfg = inp.cfg
    w, ids = oracle.topk(inp.logits.cpu(), cfg.k, cfg.score, cfg.renorm)
    return w.astype(np.float32), ids


def read_alignment(layer):
    """The alignment a finished fused call left in layer.ws, located through
    fused_moe_workspace_layout: (sorted_ids[:npp], npp, chunks int32 [n, 4],
    layout dict)."""
    lay = layer.layout()
    ws = layer.ws
    meta = ws[lay["meta"]:lay["meta"] + 8].view(torch.int32).cpu().numpy()
    npp, nch = int(meta[0]), int(meta[1])
    assert 0 <= npp <= lay["rows"] and npp % lay["block_size"] == 0, (npp, lay)
    assert 0 <= nch <= lay["max_chunks"], (nch, lay)
    s0 = lay["sorted_ids"]
    sorted_ids = ws[s0:s0 + 4 * npp].view(torch.int32).cpu().numpy()
    c0 = lay["chunks"]
    chunks = ws[c0:c0 + 16 * nch].view(torch.int32).cpu().numpy().reshape(nch, 4)
    if lay["sched"] != 2 ** 64 - 1:
        # the tile kernels' copy: the same chunks, largest first
        q0 = lay["sched"]
        sched = ws[q0:q0 + 16 * nch].view(torch.int32).cpu().numpy().reshape(nch, 4)
        assert np.all(np.diff(sched[:, 2]) <= 0), "schedule not in order of non-increasing rows"
        key = lambda c: c[np.lexsort(c[:, ::-1].T)]
        assert np.array_equal(key(sched), key(chunks)), "schedule is not a permutation of the chunk list"
    return sorted_ids, npp, chunks, lay


def expected_alignment(topk_ids, E: int, shared: bool, B: int, chunk_rows: int):
    """What the fused layer's alignment must be, from oracle.align: the routed
    pairs, then (shared expert) one pair per token as expert E; slots whose id
    lies outside [0, E) are dropped.  Dropped pairs are routed to an extra last
    expert for the oracle, whose group is then cut off the end (every other
    slot, the sentinel and the padding are unaffected).
    -> (sorted_ids[:npp], per-block expert [npp/B], npp, chunks [n, 3])."""
    ids = np.asarray(topk_ids).reshape(-1).astype(np.int64)
    T = np.asarray(topk_ids).shape[0]
    E_tot = E + (1 if shared else 0)
    drop = (ids < 0) | (ids >= E)
    flat = np.where(drop, E_tot, ids)
    if shared:
        flat = np.concatenate([flat, np.full(T, E, np.int64)])
    n_drop = int(drop.sum())
    s, eids, npp = oracle.align(flat.astype(np.int32), E_tot + (1 if n_drop else 0), B)
    npp -= (n_drop + B - 1) // B * B
    blocks = eids[:npp // B]
    chunks = []
    b = 0
    while b < blocks.size:
        e = blocks[b]
        end = b
        while end < blocks.size and blocks[end] == e:
            end += 1
        for r in range(b * B, end * B, chunk_rows):
            chunks.append((int(e), r, min(chunk_rows, end * B - r)))
        b = end
    return s[:npp], blocks, npp, np.asarray(chunks, np.int64).reshape(-1, 3)


def check_alignment(layer, topk_ids, what=""):
    """Bit-exact comparison of the alignment a fused call wrote (sorted_ids,
    num_tokens_post_pad, each 16-row block's expert, the chunk list) with
    oracle.align.  -> (sorted_ids[:npp], chunks) for choosing sample rows."""
    cfg = layer.cfg
    got_s, npp, chunks, lay = read_alignment(layer)
    want_s, want_blk, want_npp, want_ch = expected_alignment(
        topk_ids.cpu().numpy() if isinstance(topk_ids, torch.Tensor) else topk_ids, cfg.E,
        cfg.shared, lay["block_size"], lay["chunk_rows"])
    assert npp == want_npp, f"{what}: num_tokens_post_pad {npp} != {want_npp}"
    bad = np.flatnonzero(got_s != want_s)
    assert bad.size == 0, f"{what}: sorted_ids differ at {bad[:8]} ({got_s[bad[:8]]} vs {want_s[bad[:8]]})"
    blk = np.full(npp // lay["block_size"], -1, np.int64)
    for e, r0, n, _ in chunks:
        blk[r0 // lay["block_size"]:(r0 + n) // lay["block_size"]] = e
    assert np.array_equal(blk, want_blk), f"{what}: block experts differ"
    assert np.array_equal(chunks[:, :3].astype(np.int64), want_ch), f"{what}: chunk list differs"
    return got_s, chunks


def tile_tokens(sorted_ids, chunks, cfg, extra=()):
    """Tokens whose rows touch every (expert, chunk) tile the GEMMs run: the
    token of each chunk's last real row (so ragged chunk tails are included),
    plus `extra`."""
    P = cfg.T * cfg.k
    P_tot = P + (cfg.T if cfg.shared else 0)
    toks = set(int(t) for t in extra)
    for _, r0, n, _ in chunks:
        rows = sorted_ids[r0:r0 + n]
        real = rows[rows < P_tot]
        assert real.size, "a chunk without a real row"
        pid = int(real[-1])
        toks.add(pid // cfg.k if pid < P else pid - P)
    return np.asarray(sorted(toks), np.int64)


def oracle_quant_check(layer, x):
    """INT8 weights: the token rows' codes and scales the fused call wrote
    into its workspace equal the oracle's quantiser bit for bit."""
    lay = layer.layout()
    T, H = x.shape
    q = layer.ws[lay["xq"]:lay["xq"] + T * H].view(torch.int8).cpu().numpy().reshape(T, H)
    s = layer.ws[lay["xs"]:lay["xs"] + 4 * T].view(torch.float32).cpu().numpy()
    rq, rs = oracle.quant_int8_rows(x.float().cpu().numpy())
    assert np.array_equal(s.view(np.uint32), rs.view(np.uint32)), "token row scales differ"
    assert np.array_equal(q, rq), "token row codes differ"
