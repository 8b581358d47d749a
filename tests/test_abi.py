"""The C ABI library: loads, exports every declared symbol, validates on the host.

No test here launches a kernel: every call below is rejected by host-side
validation before the library touches the GPU, so these run on a machine
without one.
"""

import ctypes
import os
import re

import pytest

from sparse_causal_attention_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "scfa.h")

# fake, aligned, never-dereferenced device addresses
P = 0x7F0000000000
P2 = 0x7F0000100000


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"\b(scfa_\w+)\s*\(", text)


def test_header_and_binding_agree():
    names = _declared()
    assert sorted(names) == sorted(_lib.EXPORTED)


def test_library_exports_every_declared_symbol():
    lib = _lib.load()
    for name in _declared():
        assert hasattr(lib, name), name
    # also visible to a plain dlopen, independent of the binding
    raw = ctypes.CDLL(_lib.LIB_PATH)
    for name in _declared():
        getattr(raw, name)


def _fwd(**kw):
    a = dict(q=P, k=P, v=P, qi=P2, ki=P2, o=P, lse=P2, B=1, H=2, Tq=100, Tk=100, d=64, block=64, scale=0.125,
             dtype=0, flags=0, ws=P, nws=1 << 30, stream=None)
    a.update(kw)
    lib = _lib.load()
    return lib.scfa_qk_sparse_fwd(a["q"], a["k"], a["v"], a["qi"], a["ki"], a["o"], a["lse"], a["B"], a["H"],
                                  a["Tq"], a["Tk"], a["d"], a["block"], a["scale"], a["dtype"], a["flags"],
                                  a["ws"], a["nws"], a["stream"])


@pytest.mark.parametrize(
    "kw,status",
    [
        (dict(d=96), _lib.ERR_UNSUPPORTED),
        (dict(d=32), _lib.ERR_UNSUPPORTED),
        (dict(block=32), _lib.ERR_UNSUPPORTED),
        (dict(dtype=7), _lib.ERR_UNSUPPORTED),
        (dict(B=0), _lib.ERR_INVALID_ARGUMENT),
        (dict(H=-1), _lib.ERR_INVALID_ARGUMENT),
        (dict(Tq=-5), _lib.ERR_INVALID_ARGUMENT),
        (dict(scale=0.0), _lib.ERR_INVALID_ARGUMENT),
        (dict(scale=float("inf")), _lib.ERR_INVALID_ARGUMENT),
        (dict(scale=float("nan")), _lib.ERR_INVALID_ARGUMENT),
        (dict(q=None), _lib.ERR_INVALID_ARGUMENT),
        (dict(o=None), _lib.ERR_INVALID_ARGUMENT),
        (dict(lse=None), _lib.ERR_INVALID_ARGUMENT),
        (dict(q=P + 8), _lib.ERR_INVALID_ARGUMENT),  # not 16-byte aligned
        (dict(qi=P2 + 2), _lib.ERR_INVALID_ARGUMENT),  # not 4-byte aligned
        (dict(ki=None), _lib.ERR_INVALID_ARGUMENT),  # only one of q_idx / k_idx
        (dict(flags=1 << 7), _lib.ERR_INVALID_ARGUMENT),
        (dict(ws=None), _lib.ERR_INVALID_ARGUMENT),
        (dict(ws=P + 16), _lib.ERR_INVALID_ARGUMENT),  # workspace alignment
        (dict(nws=16), _lib.ERR_WORKSPACE_TOO_SMALL),
        (dict(B=40000, H=40000), _lib.ERR_INVALID_ARGUMENT),  # too large
    ],
)
def test_invalid_arguments_are_rejected_before_launch(kw, status):
    assert _fwd(**kw) == status
    msg = _lib.load().scfa_last_error().decode()
    assert msg


def test_hash_entry_points_require_hashes_and_positions():
    lib = _lib.load()
    common = (1, 1, 64, 64, 64, 64, 0.125, 0, 0, P, 1 << 30, None)
    # q_hash NULL
    assert lib.scfa_hash_sparse_fwd(P, P, P, P2, P2, None, P2, P, P2, *common) == _lib.ERR_INVALID_ARGUMENT
    # q_idx NULL (positions are mandatory in Hash-sparse mode)
    assert lib.scfa_hash_sparse_fwd(P, P, P, None, P2, P2, P2, P, P2, *common) == _lib.ERR_INVALID_ARGUMENT
    # backward: dout NULL
    assert lib.scfa_hash_sparse_bwd(P, P, P, P, P2, None, P2, P2, P2, P2, P, P, P, *common) == \
        _lib.ERR_INVALID_ARGUMENT
    assert lib.scfa_qk_sparse_bwd(P, P, P, P, P2, P, P2, P2, P, P, None, *common) == _lib.ERR_INVALID_ARGUMENT


def test_lsh_sort_validation():
    lib = _lib.load()

    def call(nb=16, d=64, dtype=0, flags=0, x=P, R=P2, comp=None, comp_s=None, nws=1 << 30, x_rows=None, T_x=0,
             xs=P):
        return lib.scfa_lsh_bucket_sort(x, x_rows, T_x, None, R, nb, 1, 2, 1000, d, dtype, flags, P2, P2, P2, xs,
                                        comp, comp_s, P, nws, None)

    assert call(nb=3) == _lib.ERR_UNSUPPORTED
    assert call(nb=0) == _lib.ERR_UNSUPPORTED
    assert call(nb=2048) == _lib.ERR_UNSUPPORTED
    assert call(d=80) == _lib.ERR_UNSUPPORTED
    assert call(dtype=2) == _lib.ERR_UNSUPPORTED
    assert call(flags=1) == _lib.ERR_INVALID_ARGUMENT  # NO_PRUNE is not a sort flag
    assert call(x=None) == _lib.ERR_INVALID_ARGUMENT
    assert call(R=P2 + 2) == _lib.ERR_INVALID_ARGUMENT
    assert call(comp=P) == _lib.ERR_INVALID_ARGUMENT  # companion without output
    assert call(nws=100) == _lib.ERR_WORKSPACE_TOO_SMALL
    # row indirection into a longer x: needs x_rows, no row copies, 4-byte aligned rows
    assert call(T_x=5000) == _lib.ERR_INVALID_ARGUMENT
    assert call(T_x=-1) == _lib.ERR_INVALID_ARGUMENT
    assert call(x_rows=P2, T_x=5000) == _lib.ERR_UNSUPPORTED  # x_sorted requested
    assert call(x_rows=P2 + 2, T_x=5000, xs=None) == _lib.ERR_INVALID_ARGUMENT


def test_block_meta_validation():
    lib = _lib.load()
    assert lib.scfa_block_meta(P2, P2, P2, None, 1, 1, 100, 100, 64, P, P, P2, P2, None, None, None) == \
        _lib.ERR_INVALID_ARGUMENT
    assert lib.scfa_block_meta(P2, P2, None, None, 1, 1, 100, 100, 48, P, P, P2, P2, None, None, None) == \
        _lib.ERR_UNSUPPORTED
    assert lib.scfa_block_meta(P2, P2, None, None, 1, 1, 100, 100, 64, P + 4, P, P2, P2, None, None, None) == \
        _lib.ERR_INVALID_ARGUMENT  # stats need 16-byte alignment
    assert lib.scfa_block_meta(P2, P2, None, None, 1, 1, 100, 100, 64, P, P, P2, P2, P2, None, None) == \
        _lib.ERR_INVALID_ARGUMENT  # col_count without col_list


def test_block_meta_exact_validation():
    lib = _lib.load()
    f = lib.scfa_block_meta_exact
    need = lib.scfa_workspace_size(_lib.OP_BLOCK_META_EXACT, 1, 1, 100, 100, 0, 64, 0)
    assert need > 0
    # hash mode needs its workspace, 256-byte aligned and large enough
    assert f(P2, P2, P2, P2, 1, 1, 100, 100, 64, P, P, P2, P2, None, None, None, 0, None) == \
        _lib.ERR_INVALID_ARGUMENT
    assert f(P2, P2, P2, P2, 1, 1, 100, 100, 64, P, P, P2, P2, None, None, P + 16, need, None) == \
        _lib.ERR_INVALID_ARGUMENT
    assert f(P2, P2, P2, P2, 1, 1, 100, 100, 64, P, P, P2, P2, None, None, P, need - 1, None) == \
        _lib.ERR_WORKSPACE_TOO_SMALL
    assert f(P2, P2, P2, None, 1, 1, 100, 100, 64, P, P, P2, P2, None, None, P, need, None) == \
        _lib.ERR_INVALID_ARGUMENT
    assert f(P2, P2, P2, P2, 1, 1, 100, 100, 96, P, P, P2, P2, None, None, P, need, None) == \
        _lib.ERR_UNSUPPORTED


def test_row_indirection_validation():
    lib = _lib.load()

    def fwd(q_rows=None, k_rows=None, dtype=0, tqs=0, tks=0, B=1):
        return lib.scfa_attn_fwd_lists(P, P, P, P2, P2, None, None, q_rows, k_rows, tqs, tks, P2, P2, P, P2, B, 1,
                                       100, 100, 64, 64, 0.125, dtype, 0, None)

    assert fwd(q_rows=P2 + 2) == _lib.ERR_INVALID_ARGUMENT  # 4-byte alignment
    assert fwd(k_rows=P2 + 1) == _lib.ERR_INVALID_ARGUMENT
    assert fwd(q_rows=P2, dtype=1) == _lib.ERR_UNSUPPORTED  # bf16 only
    assert lib.scfa_attn_bwd_dkdv_lists(P, P, P, P2, P, P2, P2, P2, None, None, None, P2 + 3, 0, 0, P2, P2, P, P, 1,
                                        1, 100, 100, 64, 64, 0.125, 0, 0, None) == _lib.ERR_INVALID_ARGUMENT
    # caller tensors of another length need the matching rows array, and sizes >= 0 within the 2^31 bound
    assert fwd(tqs=400) == _lib.ERR_INVALID_ARGUMENT
    assert fwd(k_rows=P2, tqs=400) == _lib.ERR_INVALID_ARGUMENT
    assert fwd(q_rows=P2, k_rows=P2, tqs=-3) == _lib.ERR_INVALID_ARGUMENT
    assert fwd(q_rows=P2, k_rows=P2, tqs=1 << 26, B=64) == _lib.ERR_INVALID_ARGUMENT
    assert lib.scfa_attn_bwd_prep(P, P2, P, None, 400, P2, 1, 1, 100, 64, 0, 0, None) == _lib.ERR_INVALID_ARGUMENT


def test_workspace_sizes():
    lib = _lib.load()
    ws = lib.scfa_workspace_size
    r = lambda n: (n + 255) // 256 * 256  # noqa: E731
    BH, nq, nk, Tq = 2 * 3, 4, 2, 200
    segs = r(BH * nq * 64 * 16) + r(BH * nk * 64 * 16) + r(BH * nq * 4) + r(BH * nk * 4)  # one record per row
    fwd = r(BH * nq * 16) + r(BH * nk * 16) + r(BH * nq * 4) + r(BH * nq * nk * 4) + segs
    bwd = fwd + r(BH * nk * 4) + r(BH * nk * nq * 4) + r(2 * BH * Tq * 4)
    assert ws(_lib.OP_QK_FWD, 2, 3, 200, 100, 64, 64, 0) == fwd
    assert ws(_lib.OP_HASH_BWD, 2, 3, 200, 100, 64, 64, 0) == bwd
    assert ws(_lib.OP_QK_FWD, 0, 3, 200, 100, 64, 64, 0) == 0
    assert ws(_lib.OP_QK_FWD, 1, 3, 200, 100, 64, 96, 0) == 0
    assert ws(_lib.OP_BLOCK_META_EXACT, 2, 3, 200, 100, 0, 64, 0) == segs
    assert ws(_lib.OP_LSH_SORT, 1, 1, 5000, 0, 64, 0, 16) > 0
    assert ws(_lib.OP_LSH_SORT, 1, 1, 5000, 0, 64, 0, 15) == 0
    assert ws(99, 1, 1, 5, 5, 64, 64, 0) == 0


def test_noalloc_rejects_oversize_shapes_on_the_host():
    lib = _lib.load()
    cap = lib.scfa_noalloc_scratch_bytes()
    assert cap == 32 << 20
    # 48 heads of 16,384 tokens at block 64 need more scratch than the static array holds
    assert lib.scfa_workspace_size(_lib.OP_HASH_FWD, 2, 24, 16384, 16384, 64, 64, 0) > cap
    rc = lib.scfa_hash_sparse_fwd_noalloc(P, P, P, P2, P2, P2, P2, P, P2, 2, 24, 16384, 16384, 64, 64, 0.125, 0, 0,
                                          None)
    assert rc == _lib.ERR_WORKSPACE_TOO_SMALL
    assert b"static scratch" in lib.scfa_last_error()
    # the benchmark's 24 heads fit
    assert lib.scfa_workspace_size(_lib.OP_HASH_FWD, 2, 12, 16384, 16384, 64, 64, 0) <= cap


def test_stored_ds_validation():
    lib = _lib.load()

    def dq(qi=P2, dtype=0, flags=0, tiles=10, ds=P):
        return lib.scfa_attn_bwd_dq_ds_lists(P, P, P, P, P2, P, qi, qi, None, None, None, None, 0, 0, P2, P2, P2, P2,
                                             ds, tiles, P, P2, 1, 1, 100, 100, 64, 64, 0.125, dtype, flags, None)

    assert dq(qi=None) == _lib.ERR_UNSUPPORTED  # dense: no lists, no slots
    assert dq(dtype=1) == _lib.ERR_UNSUPPORTED  # bf16 only
    assert dq(flags=_lib.FLAG_NO_PRUNE) == _lib.ERR_UNSUPPORTED
    assert dq(tiles=-1) == _lib.ERR_INVALID_ARGUMENT
    assert dq(ds=P + 8) == _lib.ERR_INVALID_ARGUMENT  # 16-byte alignment
    assert lib.scfa_tile_slots(P2, P2, P2, P2, 1, 1, 100, 100, 96, P2, P2, None) == _lib.ERR_UNSUPPORTED
    assert lib.scfa_tile_slots(P2, P2, P2, P2, 1, 1, 100, 100, 64, None, P2, None) == _lib.ERR_INVALID_ARGUMENT
    assert lib.scfa_attn_bwd_prep(P, P2, P, None, 0, P2, 1, 1, 100, 64, 1, 0, None) == _lib.ERR_UNSUPPORTED
    assert lib.scfa_attn_bwd_prep(P, P2, P, None, 0, P2, 1, 1, 100, 64, 0, _lib.FLAG_ORIG_ROWS, None) == \
        _lib.ERR_INVALID_ARGUMENT  # caller rows need q_rows


def test_orig_rows_flag_validation():
    lib = _lib.load()

    def fwd(q_rows=None, k_rows=None, flags=_lib.FLAG_ORIG_ROWS):
        return lib.scfa_attn_fwd_lists(P, P, P, P2, P2, None, None, q_rows, k_rows, 0, 0, P2, P2, P, P2, 1, 1, 100,
                                       100, 64, 64, 0.125, 0, flags, None)

    assert fwd() == _lib.ERR_INVALID_ARGUMENT  # no row indirection
    assert fwd(q_rows=P2) == _lib.ERR_INVALID_ARGUMENT  # both needed
    # not a flag of the one-call entry points
    assert lib.scfa_qk_sparse_fwd(P, P, P, P2, P2, P, P2, 1, 2, 100, 100, 64, 64, 0.125, 0, _lib.FLAG_ORIG_ROWS,
                                  P, 1 << 30, None) == _lib.ERR_INVALID_ARGUMENT


def test_varlen_validation():
    lib = _lib.load()

    def fwd(qo=P2, ko=P2, tq=1000, tk=900, q_rows_fn=None, d=64):
        return lib.scfa_attn_fwd_varlen(P, P, P, qo, ko, tq, tk, P2, P2, None, None, P2, P2, P, P2, 2, 3, 300, 300,
                                        d, 64, 0.125, 0, 0, None)

    assert fwd(qo=None) == _lib.ERR_INVALID_ARGUMENT
    assert fwd(ko=P2 + 2) == _lib.ERR_INVALID_ARGUMENT  # alignment
    assert fwd(tq=-1) == _lib.ERR_INVALID_ARGUMENT
    assert fwd(d=80) == _lib.ERR_UNSUPPORTED
    assert lib.scfa_block_meta_varlen(None, P2, 10, 10, P2, P2, None, None, 1, 1, 64, 64, 64, P, P, P2, P2, None, None,
                                      None, 0, None) == _lib.ERR_INVALID_ARGUMENT


def test_binding_fails_loudly_without_library(tmp_path, monkeypatch):
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(_lib, "_LIB", None)
    with pytest.raises(ImportError):
        _lib.load()


def test_row_gather_scatter_validation():
    lib = _lib.load()

    def g(**kw):
        a = dict(src=P, index=P2, dst=P + (1 << 24), B=1, H=2, Ts=100, Td=80, d=64, dtype=0)
        a.update(kw)
        return lib.scfa_gather_rows(a["src"], a["index"], a["dst"], a["B"], a["H"], a["Ts"], a["Td"], a["d"],
                                    a["dtype"], None)

    def s(flags=0, **kw):
        a = dict(src=P, index=P2, dst=P + (1 << 24), B=1, H=2, Ts=100, Td=80, d=64, dtype=0)
        a.update(kw)
        return lib.scfa_scatter_rows(a["src"], a["index"], a["dst"], a["B"], a["H"], a["Ts"], a["Td"], a["d"],
                                     a["dtype"], flags, None)

    assert g(dtype=3) == _lib.ERR_UNSUPPORTED
    assert g(d=4) == _lib.ERR_UNSUPPORTED  # 8-byte rows
    assert g(B=0) == _lib.ERR_INVALID_ARGUMENT
    assert g(src=None) == _lib.ERR_INVALID_ARGUMENT
    assert g(index=P2 + 2) == _lib.ERR_INVALID_ARGUMENT
    assert g(dst=P + 8) == _lib.ERR_INVALID_ARGUMENT
    assert g(dst=P + 1024) == _lib.ERR_INVALID_ARGUMENT  # overlaps src
    assert s(flags=1) == _lib.ERR_INVALID_ARGUMENT  # not a scatter flag
    assert s(flags=_lib.FLAG_ZERO_FILL, dst=None) == _lib.ERR_INVALID_ARGUMENT
    assert g(d=4096) == _lib.ERR_UNSUPPORTED  # 8 KiB rows: more than 256 pieces per row
    assert s(B=256, H=256) == _lib.ERR_UNSUPPORTED  # B*H beyond the grid's second dimension
    assert lib.scfa_last_error().decode()

    def z(dst=P, index=P2, B=1, H=2, n=50, T=100, d=64, dtype=0):
        return lib.scfa_zero_rows(dst, index, B, H, n, T, d, dtype, None)

    assert z(dtype=3) == _lib.ERR_UNSUPPORTED
    assert z(d=4) == _lib.ERR_UNSUPPORTED  # 8-byte rows
    assert z(n=-1) == _lib.ERR_INVALID_ARGUMENT
    assert z(dst=None) == _lib.ERR_INVALID_ARGUMENT
    assert z(dst=P + 8) == _lib.ERR_INVALID_ARGUMENT
    assert z(index=P2 + 2) == _lib.ERR_INVALID_ARGUMENT
    assert z(B=256, H=256) == _lib.ERR_UNSUPPORTED
