"""The C-ABI library on a host without a GPU: it loads, exports every entry
point include/moe.h declares, and its host-side logic (capacities, workspace
plan, argument validation) answers without launching anything."""
import ctypes
import os
import re

import pytest

from mixture_experts_ffn_topk_amd import _lib, synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")

MOE_OK, MOE_ERR_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE = 0, 1, 2, 3
FAKE = ctypes.c_void_p(0x10000)  # never dereferenced: validation fails first


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*([a-z_][a-z0-9_]*)\s*\(",
                       src, flags=re.M)
    return sorted(set(n for n in names if n.startswith(("moe_", "fused_moe"))))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        from mixture_experts_ffn_topk_amd import build
        build.build(verbose=False)
    return _lib.load()


def test_header_declarations_are_exported(lib):
    decl = _declared()
    assert len(decl) >= 20, decl
    for name in decl:
        assert hasattr(lib, name), f"{name} declared in moe.h but not exported"
    assert sorted(_lib.EXPORTS) == decl


def test_status_strings_and_version(lib):
    assert lib.moe_status_str(0) == b"ok"
    assert lib.moe_status_str(3) == b"workspace too small"
    assert lib.moe_version() >= 100


def test_align_capacity(lib):
    assert lib.moe_align_capacity(32, 256, 16) == 32 + 256 * 15
    assert lib.moe_align_capacity(0, 8, 1) == 0
    assert lib.moe_align_capacity(5, 3, 4) == 14


def test_validation_rejects_without_launch(lib):
    s = ctypes.c_void_p(0)
    # top-k: k > E, bad score, E too large
    assert lib.moe_topk(FAKE, 4, 8, 9, 0, 1, FAKE, FAKE, s) == MOE_ERR_ARG
    assert lib.moe_topk(FAKE, 4, 8, 2, 7, 1, FAKE, FAKE, s) == MOE_ERR_ARG
    assert lib.moe_topk(FAKE, 4, 2048, 2, 0, 1, FAKE, FAKE, s) == MOE_ERR_ARG
    assert lib.moe_topk(None, 0, 8, 2, 0, 1, None, None, s) == MOE_OK  # T == 0: no-op
    # alignment: block size not a power of two / too large, null outputs
    assert lib.moe_align_block_size(FAKE, 4, 2, 8, 12, FAKE, FAKE, FAKE, s) == MOE_ERR_ARG
    assert lib.moe_align_block_size(FAKE, 4, 2, 8, 512, FAKE, FAKE, FAKE, s) == MOE_ERR_ARG
    assert lib.moe_align_block_size(FAKE, 4, 2, 8, 16, None, FAKE, FAKE, s) == MOE_ERR_ARG
    # quant: cols not a multiple of 8
    assert lib.moe_quant_int8_rows(FAKE, 2, 12, FAKE, FAKE, s) == MOE_ERR_ARG
    # prepack: K not a multiple of 64, in place
    assert lib.moe_prepack(1, FAKE, 2, 100, 256, 1, ctypes.c_void_p(0x20000), s) == MOE_ERR_ARG
    assert lib.moe_prepack(1, FAKE, 2, 128, 256, 1, FAKE, s) == MOE_ERR_ARG


def _fused(lib, wd=1, T=4, H=256, I=128, E=8, k=2, ws_bytes=1 << 40, shared=None, **null):
    ptr = {n: (None if null.get(n) else FAKE)
           for n in ["x", "w13", "s13", "w2", "s2", "tw", "ti", "ws", "out"]}
    return lib.fused_moe_ex(wd, ptr["x"], ptr["w13"], ptr["s13"], ptr["w2"], ptr["s2"],
                            ptr["tw"], ptr["ti"], T, H, I, E, k, shared, ptr["ws"], ws_bytes,
                            ptr["out"], None, ctypes.c_void_p(0))


def test_fused_validation(lib):
    assert _fused(lib, H=200) == MOE_ERR_ARG          # not a multiple of 128
    assert _fused(lib, I=64) == MOE_ERR_ARG
    assert _fused(lib, k=9) == MOE_ERR_ARG            # k > E
    assert _fused(lib, E=1024) == MOE_ERR_ARG
    assert _fused(lib, T=1 << 22, k=8) == MOE_ERR_ARG  # T*k > 2^24
    assert _fused(lib, x=True) == MOE_ERR_ARG
    assert _fused(lib, s13=True) == MOE_ERR_ARG       # FP8 needs scales
    assert _fused(lib, wd=0, s13=True, s2=True, ws_bytes=1) == MOE_ERR_WORKSPACE
    assert _fused(lib, ws_bytes=16) == MOE_ERR_WORKSPACE
    assert b"workspace" in lib.moe_last_error()
    sh = _lib._DenseExpert(0x10000, 0x10000, 0x10000, 0x10000, 64)  # inter != I
    assert _fused(lib, shared=ctypes.byref(sh)) == MOE_ERR_UNSUPPORTED
    sh = _lib._DenseExpert(0x10000, None, 0x10000, 0x10000, 128)    # missing scale
    assert _fused(lib, shared=ctypes.byref(sh)) == MOE_ERR_ARG
    assert _fused(lib, T=0) == MOE_OK                 # empty batch: no-op


def test_decode_path_activation_limit(lib):
    """The decode kernels address activations with 32-bit buffer offsets: a
    forced decode path whose token rows reach 2 GiB is refused before any
    launch (AUTO picks the prefill kernels there)."""
    o = _lib._Options()
    o.path = 1  # decode
    T, H, I, E, k = 150000, 8192, 128, 1000, 1  # T*H*2 > 2 GiB, T*k/E <= 8
    st = lib.fused_moe_ex(1, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, T, H, I, E, k, None, FAKE,
                          1 << 40, FAKE, ctypes.byref(o), ctypes.c_void_p(0))
    assert st == MOE_ERR_UNSUPPORTED
    assert b"2 GiB" in lib.moe_last_error()


def test_negative_prefill_span(lib):
    """A negative column-group span is an argument error, refused before any
    launch."""
    o = _lib._Options()
    o.path = 2  # prefill
    o.prefill_span = -1
    st = lib.fused_moe_ex(1, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4, 256, 128, 8, 2, None, FAKE,
                          1 << 40, FAKE, ctypes.byref(o), ctypes.c_void_p(0))
    assert st == MOE_ERR_ARG
    assert b"prefill_span" in lib.moe_last_error()


def _routed(lib, logits=FAKE, score=1, T=4, k=2, E=8):
    return lib.fused_moe_routed(1, logits, score, 1, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, T,
                                256, 128, E, k, None, FAKE, 1 << 40, FAKE, None,
                                ctypes.c_void_p(0))


def test_routed_validation(lib):
    assert _routed(lib, logits=None) == MOE_ERR_ARG
    assert _routed(lib, score=5) == MOE_ERR_ARG
    assert _routed(lib, k=9) == MOE_ERR_ARG           # k > E
    assert _routed(lib, T=0) == MOE_OK                # empty batch: no-op


@pytest.mark.parametrize("name", list(synth.CONFIGS))
def test_workspace_plan_sizes(lib, name):
    cfg = synth.CONFIGS[name]
    ws = lib.fused_moe_workspace_bytes(cfg.wdtype, cfg.T, cfg.H, cfg.I, cfg.E, cfg.k,
                                       int(cfg.shared))
    assert ws > 0
    for path in (1, 2):
        o = _lib._Options()
        o.path = path
        ex = lib.fused_moe_workspace_bytes_ex(cfg.wdtype, cfg.T, cfg.H, cfg.I, cfg.E, cfg.k,
                                              int(cfg.shared), ctypes.byref(o))
        assert 0 < ex <= ws
    # activations dominate nothing unreasonable: bounded by a few GiB even at prefill sizes
    assert ws < 8 << 30
    assert lib.fused_moe_workspace_bytes(cfg.wdtype, 0, cfg.H, cfg.I, cfg.E, cfg.k, 0) == 0


def test_prefill_workspace_grows_with_tokens(lib):
    """On the prefill kernels the workspace never shrinks as T grows, also
    across the 8192-pair threshold (T = 911 here, 9 pairs per token with the
    shared expert) where the many-workgroup alignment adds its block-count
    segment, for every weight type.  (The decode plan is not monotonic: few
    tokens split K more ways and keep larger fp32 partial sums.)"""
    o = _lib._Options()
    o.path = 2  # prefill
    for wd in (0, 1, 2):
        prev = 0
        for T in (1, 16, 512, 910, 911, 912, 2048, 4096, 65536):
            ws = lib.fused_moe_workspace_bytes_ex(wd, T, 1024, 512, 64, 8, 1, ctypes.byref(o))
            assert ws >= prev, (wd, T, ws, prev)
            prev = ws


def test_packed_bytes(lib):
    assert lib.moe_packed_bytes(1, 3, 256, 512) == 3 * 256 * 512
    assert lib.moe_packed_bytes(0, 3, 256, 512) == 2 * 3 * 256 * 512
    assert lib.moe_packed_bytes(2, 0, 256, 512) == 0


def test_profile_stage_names(lib):
    names = [lib.moe_profile_stage_name(i).decode() for i in range(16)]
    for n in ["topk", "align", "gemm1", "gemm2", "combine", "topk_align"]:
        assert n in names
    assert lib.moe_profile_stage_name(99) == b""


@pytest.mark.parametrize("name", list(synth.CONFIGS))
@pytest.mark.parametrize("path", [0, 1, 2])
def test_workspace_layout(lib, name, path):
    """fused_moe_workspace_layout describes the plan the call makes: its
    total equals the reported workspace size, every segment lies inside it,
    and the per-row buffers hold P' + 15 * min(E', P') rows (at most that
    many slots survive the 16-row padding), never more than sorted_ids' cap;
    the prefill path also holds the size-ordered copy of the chunk list."""
    cfg = synth.CONFIGS[name]
    lay = _lib.workspace_layout(cfg.wdtype, cfg.T, cfg.H, cfg.I, cfg.E, cfg.k, cfg.shared,
                                path=path)
    o = _lib._Options()
    o.path = path
    total = lib.fused_moe_workspace_bytes_ex(cfg.wdtype, cfg.T, cfg.H, cfg.I, cfg.E, cfg.k,
                                             int(cfg.shared), ctypes.byref(o))
    assert lay["total"] == total
    P_tot = cfg.T * cfg.k + (cfg.T if cfg.shared else 0)
    E_tot = cfg.E + (1 if cfg.shared else 0)
    assert lay["block_size"] == 16
    assert lay["cap"] == P_tot + E_tot * 15
    assert lay["rows"] == min(lay["cap"], P_tot + 15 * min(E_tot, P_tot))
    assert lay["path"] in (1, 2) and (path == 0 or lay["path"] == path)
    assert lay["chunk_rows"] % 16 == 0 and lay["max_chunks"] >= 1
    assert lay["sorted_ids"] + 4 * lay["cap"] <= total
    assert lay["meta"] + 8 <= total and lay["chunks"] + 16 * lay["max_chunks"] <= total
    if cfg.wdtype == synth.WDTYPE_INT8:
        assert lay["xq"] + cfg.T * cfg.H <= total and lay["xs"] + 4 * cfg.T <= total
    for key in ("sorted_ids", "meta", "chunks", "xq", "xs"):
        assert lay[key] % 256 == 0
    # the tile kernels' size-ordered chunk list exists on the prefill path only
    if lay["path"] == 2:
        assert lay["sched"] % 256 == 0 and lay["sched"] + 16 * lay["max_chunks"] <= total
        assert lay["sched"] >= lay["chunks"] + 16 * lay["max_chunks"]
    else:
        assert lay["sched"] == 2 ** 64 - 1


def test_workspace_layout_rejects(lib):
    lay = _lib._Layout()
    assert lib.fused_moe_workspace_layout(1, 4, 256, 128, 8, 2, 0, None, None) == MOE_ERR_ARG
    assert lib.fused_moe_workspace_layout(1, 0, 256, 128, 8, 2, 0, None,
                                          ctypes.byref(lay)) == MOE_ERR_ARG
    assert lib.fused_moe_workspace_layout(1, 4, 200, 128, 8, 2, 0, None,
                                          ctypes.byref(lay)) == MOE_ERR_ARG
    assert lib.fused_moe_workspace_layout(1, 4, 256, 128, 8, 9, 0, None,
                                          ctypes.byref(lay)) == MOE_ERR_ARG
    assert lib.fused_moe_workspace_layout(7, 4, 256, 128, 8, 2, 0, None,
                                          ctypes.byref(lay)) == MOE_ERR_ARG


def test_decode_workspace_small_batches(lib):
    """Few tokens no longer pay for a sorted-table-sized row capacity: the
    decode plan of one token needs far less than the cap-sized buffers
    (cap = P' + 15 E' slots) would take."""
    for name in ("c2", "c5_T1"):
        cfg = synth.CONFIGS[name].with_T(1)
        o = _lib._Options()
        o.path = 1
        ws = lib.fused_moe_workspace_bytes_ex(cfg.wdtype, 1, cfg.H, cfg.I, cfg.E, cfg.k,
                                              int(cfg.shared), ctypes.byref(o))
        E_tot = cfg.E + (1 if cfg.shared else 0)
        cap = cfg.k + (1 if cfg.shared else 0) + 15 * E_tot
        assert ws < cap * cfg.I * 2, (name, ws)


def test_noalloc_rejects_oversized_batch_without_a_device(lib):
    """fused_moe_routed_noalloc refuses a batch whose workspace exceeds its
    static scratch before touching any device, with a clear message."""
    assert _lib.NOALLOC_SCRATCH_BYTES == 64 << 20
    c = synth.CONFIGS["c4"]
    st = lib.fused_moe_routed_noalloc(c.wdtype, FAKE, 1, 1, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                      FAKE, c.T, c.H, c.I, c.E, c.k, None, FAKE, None,
                                      ctypes.c_void_p(0))
    assert st == MOE_ERR_UNSUPPORTED
    assert b"static maximum" in lib.moe_last_error()
    assert lib.fused_moe_routed_noalloc(c.wdtype, None, 1, 1, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                        FAKE, 4, c.H, c.I, c.E, c.k, None, FAKE, None,
                                        ctypes.c_void_p(0)) == MOE_ERR_ARG
    assert lib.fused_moe_routed_noalloc(c.wdtype, FAKE, 1, 1, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                        FAKE, 0, c.H, c.I, c.E, c.k, None, FAKE, None,
                                        ctypes.c_void_p(0)) == MOE_OK


def test_int4_host_side(lib):
    """INT4: packed size is half a byte per weight, prepack wants K % 128,
    and forcing the tile kernels is refused before any launch."""
    assert lib.moe_packed_bytes(3, 2, 256, 512) == 2 * 256 * 512 // 2
    s = ctypes.c_void_p(0)
    assert lib.moe_prepack(3, FAKE, 2, 192, 512, 1, ctypes.c_void_p(0x20000), s) == MOE_ERR_ARG
    o = _lib._Options()
    o.path = 2
    st = lib.fused_moe_ex(3, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 64, 256, 128, 4, 2, None,
                          FAKE, 1 << 40, FAKE, ctypes.byref(o), ctypes.c_void_p(0))
    assert st == MOE_ERR_UNSUPPORTED and b"decode kernels only" in lib.moe_last_error()
    assert lib.fused_moe_ex(4, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4, 256, 128, 4, 2, None,
                            FAKE, 1 << 40, FAKE, None, ctypes.c_void_p(0)) == MOE_ERR_ARG
