"""The C ABI without a GPU: the library loads, exports exactly what include/nabla.h
declares, sizes workspaces, and rejects bad arguments with status codes before
any GPU work is enqueued (only validation paths are exercised here)."""

import ctypes
import os
import re
import subprocess

import pytest

import block_sparse_attention_nabla_amd as nb

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nabla.h")

OK, INVALID, UNSUPPORTED, WORKSPACE, HIPERR = 0, 1, 2, 3, 4


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(nb.LIB_PATH):
        pytest.fail("libnabla.so is not built (run python -m block_sparse_attention_nabla_amd.build)")
    return nb.load_library()


def _declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"NABLA_API\s+[\w\s\*]+?\b(nabla_\w+)\s*\(", text)))


def test_exports_match_header(lib):
    declared = _declared_functions()
    assert declared == sorted(nb.EXPORTED_SYMBOLS)
    out = subprocess.run(["nm", "-D", "--defined-only", nb.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = sorted({ln.split()[-1] for ln in out.splitlines() if " T " in ln and "nabla" in ln})
    assert exported == declared
    for name in declared:
        assert hasattr(lib, name)


def test_status_strings(lib):
    assert nb.nabla_status_string(0) == "NABLA_OK"
    assert nb.nabla_status_string(3) == "NABLA_ERR_WORKSPACE"
    assert nb.nabla_status_string(99) == "NABLA_ERR_UNKNOWN"


def test_workspace_sizes(lib):
    B, H, S, D = 1, 2, 1024, 64
    n = S // 64
    mask = nb.nabla_workspace_size(nb.NABLA_OP_MASK, B, H, S, D)
    assert mask >= 2 * B * H * n * D * 4 + B * H * n * n * 4
    assert nb.nabla_workspace_size(nb.NABLA_OP_FWD, B, H, S, D) >= B * H * n * 4
    assert nb.nabla_workspace_size(nb.NABLA_OP_BWD, B, H, S, D) >= B * H * S * 4 + 2 * B * H * n * 4
    assert nb.nabla_workspace_size(nb.NABLA_OP_MASK, B, H, 1000, D) == 0  # S % N != 0
    assert nb.nabla_workspace_size(nb.NABLA_OP_MASK, B, H, S, 96) == 0    # unsupported D
    assert nb.nabla_workspace_size(7, B, H, S, D) == 0


def test_mask_workspace_holds_the_logit_map_for_a_chunk_of_heads(lib):
    # Linear terms per head row: fp32 + fp64 means of Q and K, two norms; plus
    # bitmask words. The n x n fp32 map is held for as many heads as fit
    # 256 MiB, at least one.
    def linear(B, H, S, D):
        n = S // 64
        return B * H * n * (2 * D * 4 + 2 * D * 8 + 2 * 4 + ((n + 31) // 32) * 4)

    cap = 256 << 20
    for B, H, S, D in [(1, 40, 80640, 128), (2, 16, 61440, 128), (1, 2, 64 * 6144, 64),
                       (1, 40, 64 * 8192, 128)]:
        n = S // 64
        head_map = n * n * 4
        heads = max(1, min(B * H, cap // head_map))
        size = nb.nabla_workspace_size(nb.NABLA_OP_MASK, B, H, S, D)
        want = linear(B, H, S, D) + heads * head_map
        assert want <= size <= want + 16 * 256 + B * H * 4, (B, H, S, D, size, want)
    # 720p (40 heads, n = 1260) keeps its whole map in one chunk; n = 8192 with
    # 40 heads needs one head's map (268 MB), not all forty (10.7 GB).
    assert nb.nabla_workspace_size(nb.NABLA_OP_MASK, 1, 40, 80640, 128) > 40 * 1260 * 1260 * 4
    assert nb.nabla_workspace_size(nb.NABLA_OP_MASK, 1, 40, 64 * 8192, 128) < 2 * 8192 * 8192 * 4 + (2 << 30)


# Fake, 256-aligned, never-dereferenced device addresses: every call below
# fails validation before anything touches them.
P = ctypes.c_void_p(0x7F0000000000)
P2 = ctypes.c_void_p(0x7F0000100000)
BIG = 1 << 40


def _mask(lib, B=1, H=2, S=1024, D=64, N=64, thr=0.5, sta=None, q=P, k=P, cnt=P, idx=P,
          qc=None, qi=None, ws=P2, wsb=BIG):
    return lib.nabla_build_mask(q, k, B, H, S, D, N, thr, sta, cnt, idx, qc, qi, None, ws, wsb, None)


def test_build_mask_validation(lib):
    assert _mask(lib, S=1000) == INVALID
    assert _mask(lib, B=0) == INVALID
    assert _mask(lib, N=32, S=1024) == UNSUPPORTED
    assert _mask(lib, D=96) == UNSUPPORTED
    assert _mask(lib, S=64 * (8192 + 1)) == UNSUPPORTED
    assert _mask(lib, thr=float("nan")) == INVALID
    assert _mask(lib, thr=-0.01) == INVALID
    assert _mask(lib, thr=float("inf")) == INVALID
    assert _mask(lib, q=None) == INVALID
    assert _mask(lib, idx=None) == INVALID
    assert _mask(lib, q=ctypes.c_void_p(0x7F0000000008)) == INVALID  # not 16-byte aligned
    assert _mask(lib, qc=P, qi=None) == INVALID
    assert _mask(lib, ws=None) == WORKSPACE
    assert _mask(lib, wsb=16) == WORKSPACE


def test_build_mask_sta_validation(lib):
    good = dict(T=4, Hs=16, Ws=16, P=8, win_t=3, win_h=8, win_w=8)

    def sta(**over):
        d = dict(good, **over)
        return ctypes.pointer(nb.StaWindow(*(d[f] for f in ("T", "Hs", "Ws", "P", "win_t", "win_h", "win_w"))))

    # S = 4*16*16 = 1024 matches; every bad field is rejected.
    assert _mask(lib, sta=sta(T=5)) == INVALID         # T*Hs*Ws != S
    assert _mask(lib, sta=sta(P=4)) == INVALID         # P*P != N
    assert _mask(lib, sta=sta(win_h=12)) == INVALID    # not a multiple of P
    assert _mask(lib, sta=sta(win_t=0)) == INVALID
    assert _mask(lib, sta=sta(win_w=0)) == INVALID
    assert _mask(lib, sta=sta(Hs=12, Ws=16 * 16 // 12)) == INVALID


def test_fwd_validation(lib):
    f = lib.nabla_sparse_attn_fwd

    def call(S=1024, D=64, scale=0.125, v=P, o=P, odt=0, ws=P2, wsb=BIG, fb=0):
        return f(P, P, v, 1, 2, S, D, 64, P, P, scale, fb, o, odt, None, ws, wsb, None)

    assert call(S=1000) == INVALID
    assert call(D=256) == UNSUPPORTED
    assert call(scale=0.0) == INVALID
    assert call(scale=float("nan")) == INVALID
    assert call(scale=float("inf")) == INVALID
    assert call(v=None) == INVALID
    assert call(o=None) == INVALID
    assert call(odt=2) == INVALID
    assert call(fb=-1) == INVALID
    assert call(fb=5) == INVALID        # n = 16 blocks is not a multiple of 5
    assert call(ws=None) == WORKSPACE
    assert call(wsb=4) == WORKSPACE


def test_bwd_validation(lib):
    f = lib.nabla_sparse_attn_bwd

    def call(S=1024, lse=P, qc=P, scale=0.125, odt=0, ws=P2, wsb=BIG):
        return f(P, P, P, P, odt, P, lse, 1, 2, S, 64, 64, P, P, qc, P, scale, P, P, P, ws, wsb, None)

    assert call(S=1000) == INVALID
    assert call(lse=None) == INVALID
    assert call(qc=None) == INVALID
    assert call(scale=-1.0) == INVALID
    assert call(odt=5) == INVALID
    assert call(wsb=8) == WORKSPACE


def test_binding_requires_the_library(tmp_path):
    # The binding never falls back to anything else: a missing library raises.
    import importlib
    mod = importlib.import_module("block_sparse_attention_nabla_amd")
    saved = mod._lib
    try:
        mod._lib = None
        with pytest.raises(RuntimeError, match="missing"):
            mod.load_library(str(tmp_path / "nope.so"))
    finally:
        mod._lib = saved


def test_reorder_validation(lib):
    f = lib.nabla_reorder_tokens

    def call(src=P, dst=P2, B=1, T=2, Hs=16, Ws=16, Pt=8, row=256, inv=0):
        return f(src, dst, B, T, Hs, Ws, Pt, row, inv, None)

    assert call(Hs=12) == INVALID                      # Hs not a multiple of P
    assert call(Ws=20) == INVALID
    assert call(row=24) == INVALID                     # row not a multiple of 16
    assert call(row=0) == INVALID
    assert call(Pt=0) == INVALID
    assert call(B=-1) == INVALID
    assert call(inv=2) == INVALID
    assert call(src=None) == INVALID
    assert call(dst=ctypes.c_void_p(0x7F0000100008)) == INVALID  # misaligned
    assert call(dst=ctypes.c_void_p(0x7F0000000000 + 4096)) == INVALID  # overlaps src
    assert call(B=1 << 20, T=1 << 10, Hs=64, Ws=64, Pt=1, row=16) == UNSUPPORTED
    # Empty permutations enqueue nothing and need no pointers.
    assert call(src=None, dst=None, B=0) == OK
    assert call(src=None, dst=None, T=0) == OK
    assert call(src=None, dst=None, Hs=0) == OK


def test_topk_validation(lib):
    f = lib.nabla_build_topk_mask

    def call(S=1024, D=64, topk=4, q=P, sta=None, ws=P2, wsb=BIG):
        return f(q, P, 1, 2, S, D, 64, topk, sta, P, P, None, None, None, ws, wsb, None)

    assert call(topk=0) == INVALID
    assert call(topk=-3) == INVALID
    assert call(S=1000) == INVALID
    assert call(D=96) == UNSUPPORTED
    assert call(q=None) == INVALID
    assert call(wsb=16) == WORKSPACE


def test_sta_mask_validation(lib):
    f = lib.nabla_build_sta_mask
    good = dict(T=4, Hs=16, Ws=16, P=8, win_t=3, win_h=8, win_w=8)

    def sta(**over):
        d = dict(good, **over)
        return ctypes.pointer(nb.StaWindow(*(d[k] for k in ("T", "Hs", "Ws", "P", "win_t", "win_h", "win_w"))))

    def call(S=1024, s=None, cnt=P, ws=P2, wsb=BIG, qc=None, qi=None):
        return f(1, 2, S, 64, s, cnt, P, qc, qi, None, ws, wsb, None)

    assert call(s=None) == INVALID                       # the window is required
    assert call(s=sta(T=5)) == INVALID                   # T*Hs*Ws != S
    assert call(s=sta(win_h=12)) == INVALID
    assert call(s=sta(), cnt=None) == INVALID
    assert call(s=sta(), qc=P) == INVALID                # q_count without q_idx
    assert call(s=sta(), ws=None) == WORKSPACE
    assert call(s=sta(), wsb=16) == WORKSPACE
    # The STA workspace ignores D and holds one bitmask row per query block.
    size = nb.nabla_workspace_size(nb.NABLA_OP_STA_MASK, 1, 2, 1024, 0)
    assert size >= 2 * 16 * 4 and size == nb.nabla_workspace_size(nb.NABLA_OP_STA_MASK, 1, 2, 1024, 128)


def test_fidelity_validation(lib):
    bm = lib.nabla_block_mass
    assert bm(P, P, P, 1, 2, 1000, 64, 64, 0.125, P, None) == INVALID      # S % N
    assert bm(P, P, None, 1, 2, 1024, 64, 64, 0.125, P, None) == INVALID   # lse required
    assert bm(P, P, P, 1, 2, 1024, 64, 64, 0.125, None, None) == INVALID   # mass required
    assert bm(P, P, P, 1, 2, 1024, 64, 64, 0.0, P, None) == INVALID
    assert bm(P, P, P, 1, 2, 1024, 96, 64, 0.125, P, None) == UNSUPPORTED
    rc = lib.nabla_mask_recall
    assert rc(P, 1, 2, 1000, 64, P, P, P, P, None) == INVALID
    assert rc(None, 1, 2, 1024, 64, P, P, P, P, None) == INVALID
    assert rc(P, 1, 2, 1024, 64, P, P, P, None, None) == INVALID
    assert rc(P, 1, 2, 1024, 32, P, P, P, P, None) == UNSUPPORTED


def test_static_forward_rejects_shapes_beyond_its_scratch(lib):
    # No GPU needed: the shape check fails before any HIP call (dummy aligned pointers).
    p = ctypes.c_void_p(1 << 20)
    st = lib.nabla_sparse_attn_fwd_static(p, p, p, 1, 129, 64 * 8192, 64, 64, p, p, 0.125, 0, p, 0,
                                          None, None)
    assert st == WORKSPACE
    st = lib.nabla_sparse_attn_fwd_static(p, p, p, 1, 1, 100, 64, 64, p, p, 0.125, 0, p, 0, None, None)
    assert st == INVALID  # S % N != 0


def test_check_lists_validation(lib):
    cl = lib.nabla_check_lists
    assert cl(P, P, 1, 2, 1000, 64, P, None) == INVALID   # S % N
    assert cl(None, P, 1, 2, 1024, 64, P, None) == INVALID
    assert cl(P, None, 1, 2, 1024, 64, P, None) == INVALID
    assert cl(P, P, 1, 2, 1024, 64, None, None) == INVALID
    assert cl(P, P, 1, 2, 1024, 32, P, None) == UNSUPPORTED
