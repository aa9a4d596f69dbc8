"""The C-ABI library: it loads, exports every symbol include/calibattn.h declares
with the binding's signatures, and rejects invalid arguments on the host before
any launch (these calls never reach the GPU).  CPU only."""
import ctypes
import os
import re

import pytest

from calibrated_block_sparse_calib_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "calibattn.h")

EINVAL, EUNSUPPORTED = 1, 2


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(?:cba_status|const char\*|int32_t)\s+(\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def test_header_declares_every_call():
    names = _declared_functions()
    for n in ["calib_block_energy", "select_blocks_by_energy", "build_block_csr", "sparse_attn_fwd",
              "rep_row_broadcast", "dense_attn_fwd", "spatial_rep_similarity", "select_rep_heads",
              "build_block_intervals", "sparse_attn_fwd_intervals", "block_energy_from_lse",
              "select_blocks_by_energy_heads", "order_heavy_rows_first", "calib_block_energy_ws",
              "cba_status_str", "cba_version"]:
        assert n in names
    assert set(names) == set(_lib.SIGNATURES)


def test_library_exports_every_declared_symbol(lib):
    for name in _declared_functions():
        assert hasattr(lib, name), name


def test_desc_struct_matches_header_layout():
    # int32 x 10, float, then three int64 (8-aligned): 44 bytes + 4 padding + 24.
    assert ctypes.sizeof(_lib.AttnDesc) == 72
    assert _lib.AttnDesc.stride_b.offset == 48


def test_status_strings_and_version(lib):
    assert lib.cba_status_str(0) == b"ok"
    assert lib.cba_status_str(1) == b"invalid argument"
    assert lib.cba_status_str(99) == b"unknown status"
    assert lib.cba_version() == 100


def _desc(**kw):
    base = dict(dtype=1, batch=1, heads=2, seq_len=256, head_dim=128, block=128, n_prefix=0,
                grid_f=0, grid_h=0, grid_w=0, scale=0.0, stride_b=2 * 256 * 128, stride_h=256 * 128,
                stride_n=128)
    base.update(kw)
    return _lib.AttnDesc(**base)


FAKE = ctypes.c_void_p(0x10000)  # 16-byte aligned, never dereferenced: validation fails first


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=5), EUNSUPPORTED),
    (dict(head_dim=96), EUNSUPPORTED),
    (dict(block=48), EUNSUPPORTED),
    (dict(batch=0), EINVAL),
    (dict(heads=0), EINVAL),
    (dict(seq_len=0), EINVAL),
    (dict(seq_len=-1), EINVAL),
    (dict(n_prefix=100), EINVAL),  # not a multiple of block
    (dict(grid_f=2, grid_h=2, grid_w=2), EINVAL),  # grid does not cover seq_len - n_prefix
    (dict(stride_n=64), EINVAL),  # rows overlap
    (dict(stride_n=130), EINVAL),  # row stride not 16-byte aligned
    (dict(scale=float("inf")), EINVAL),
])
def test_dense_rejects_bad_descriptors(lib, kw, code):
    d = _desc(**kw)
    assert lib.dense_attn_fwd(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, None, None) == code


def test_null_and_misaligned_pointers_rejected(lib):
    d = _desc()
    assert lib.dense_attn_fwd(None, FAKE, FAKE, FAKE, FAKE, None, None) == EINVAL
    assert lib.dense_attn_fwd(ctypes.byref(d), None, FAKE, FAKE, FAKE, None, None) == EINVAL
    assert lib.dense_attn_fwd(ctypes.byref(d), ctypes.c_void_p(0x10008), FAKE, FAKE, FAKE, None, None) == EINVAL
    # energy needs lse and energy; v and o come together
    assert lib.calib_block_energy(ctypes.byref(d), FAKE, FAKE, None, None, None, FAKE, None) == EINVAL
    assert lib.calib_block_energy(ctypes.byref(d), FAKE, FAKE, FAKE, None, FAKE, FAKE, None) == EINVAL


def test_sparse_rejects_bad_skip_list_and_repetition(lib):
    d = _desc()
    rep = (ctypes.c_uint8 * 2)(0, 1)
    # no row_ptr
    assert lib.sparse_attn_fwd(ctypes.byref(d), FAKE, FAKE, FAKE, None, FAKE, 4, None, None, 1, 0, FAKE, None,
                               None) == EINVAL
    # negative col_idx length
    assert lib.sparse_attn_fwd(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, -1, None, None, 1, 0, FAKE, None,
                               None) == EINVAL
    # a repetition head without a token grid
    assert lib.sparse_attn_fwd(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, 4, None, rep, 4, 1, FAKE, None,
                               None) == EINVAL
    # anchor stride below 1
    dg = _desc(grid_f=1, grid_h=16, grid_w=16)
    assert lib.sparse_attn_fwd(ctypes.byref(dg), FAKE, FAKE, FAKE, FAKE, FAKE, 4, None, rep, 0, 1, FAKE, None,
                               None) == EINVAL
    assert lib.rep_row_broadcast(ctypes.byref(dg), FAKE, None, 4, None) == EINVAL


def test_select_and_csr_reject_bad_sizes(lib):
    assert lib.select_blocks_by_energy(FAKE, 1, 1, 5000, 0.9, 0.5, 1, 0, FAKE, None, None) == EINVAL
    assert lib.select_blocks_by_energy(FAKE, 0, 1, 8, 0.9, 0.5, 1, 0, FAKE, None, None) == EINVAL
    assert lib.select_blocks_by_energy(None, 1, 1, 8, 0.9, 0.5, 1, 0, FAKE, None, None) == EINVAL
    assert lib.select_blocks_by_energy(FAKE, 1, 1, 8, float("nan"), 0.5, 1, 0, FAKE, None, None) == EINVAL
    assert lib.select_blocks_by_energy(FAKE, 1, 1, 8, 0.9, 0.5, 1, 9, FAKE, None, None) == EINVAL
    assert lib.build_block_csr(None, 4, 4, FAKE, None, 0, None, None) == EINVAL
    assert lib.build_block_csr(FAKE, 0, 4, FAKE, None, 0, None, None) == EINVAL
    assert lib.build_block_csr(FAKE, 4, 4, FAKE, FAKE, -1, None, None) == EINVAL
    assert lib.build_block_csr(FAKE, 1 << 20, 1 << 12, FAKE, None, 0, None, None) == EINVAL
    # empty problems are rejected, not silently accepted
    assert lib.build_block_csr(FAKE, 4, 0, FAKE, None, 0, None, None) == EINVAL
    assert lib.build_block_intervals(FAKE, 0, 4, FAKE, None, 0, None) == EINVAL
    assert lib.build_block_intervals(FAKE, 4, 0, FAKE, None, 0, None) == EINVAL
    assert lib.order_heavy_rows_first(FAKE, 0, 4, 2.0, FAKE, None) == EINVAL
    assert lib.select_blocks_by_energy(FAKE, 1, 0, 8, 0.9, 0.5, 1, 0, FAKE, None, None) == EINVAL
    assert lib.select_blocks_by_energy(FAKE, 1, 1, 0, 0.9, 0.5, 1, 0, FAKE, None, None) == EINVAL


def test_missing_library_raises(monkeypatch, tmp_path):
    monkeypatch.setattr(_lib, "_lib", None)
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "absent.so"))
    with pytest.raises(_lib.LibraryMissing):
        _lib.load()


def test_repetition_detection_rejects_bad_arguments(lib):
    grid = dict(grid_f=1, grid_h=16, grid_w=16)
    d = _desc(**grid)
    ok = (FAKE, FAKE, FAKE, 4, FAKE, FAKE, None)
    # no token grid
    assert lib.spatial_rep_similarity(ctypes.byref(_desc()), *ok) == EINVAL
    # stride below 2, or a single image row: no follower rows
    assert lib.spatial_rep_similarity(ctypes.byref(d), FAKE, FAKE, FAKE, 1, FAKE, FAKE, None) == EINVAL
    d1 = _desc(grid_f=16, grid_h=1, grid_w=16)
    assert lib.spatial_rep_similarity(ctypes.byref(d1), *ok) == EINVAL
    # missing or misaligned outputs / lse
    assert lib.spatial_rep_similarity(ctypes.byref(d), FAKE, FAKE, None, 4, FAKE, FAKE, None) == EINVAL
    assert lib.spatial_rep_similarity(ctypes.byref(d), FAKE, FAKE, FAKE, 4, None, FAKE, None) == EINVAL
    assert lib.spatial_rep_similarity(ctypes.byref(d), FAKE, FAKE, FAKE, 4, FAKE, ctypes.c_void_p(0x10002),
                                      None) == EINVAL
    # unsupported head_dim; q misaligned
    assert lib.spatial_rep_similarity(ctypes.byref(_desc(head_dim=96, **grid)), *ok) == EUNSUPPORTED
    assert lib.spatial_rep_similarity(ctypes.byref(d), ctypes.c_void_p(0x10008), *ok[1:]) == EINVAL
    # select_rep_heads
    assert lib.select_rep_heads(None, 1, 4, 0.5, FAKE, None) == EINVAL
    assert lib.select_rep_heads(FAKE, 0, 4, 0.5, FAKE, None) == EINVAL
    assert lib.select_rep_heads(FAKE, 1, 0, 0.5, FAKE, None) == EINVAL
    assert lib.select_rep_heads(FAKE, 1, 4, float("nan"), FAKE, None) == EINVAL
    assert lib.select_rep_heads(FAKE, 1, 4, 0.5, None, None) == EINVAL


def test_intervals_reject_bad_arguments(lib):
    assert lib.build_block_intervals(None, 4, 4, FAKE, None, 0, None) == EINVAL
    assert lib.build_block_intervals(FAKE, 0, 4, FAKE, None, 0, None) == EINVAL
    assert lib.build_block_intervals(FAKE, 4, 70000, FAKE, None, 0, None) == EINVAL  # runs need 16-bit blocks
    assert lib.build_block_intervals(FAKE, 4, 4, None, None, 0, None) == EINVAL
    assert lib.build_block_intervals(FAKE, 4, 4, FAKE, FAKE, -1, None) == EINVAL
    d = _desc()
    # no iv_ptr; negative length; a length without runs
    assert lib.sparse_attn_fwd_intervals(ctypes.byref(d), FAKE, FAKE, FAKE, None, FAKE, 4, None, None, 1, 0, FAKE,
                                         None, None) == EINVAL
    assert lib.sparse_attn_fwd_intervals(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, -1, None, None, 1, 0, FAKE,
                                         None, None) == EINVAL
    assert lib.sparse_attn_fwd_intervals(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, None, 4, None, None, 1, 0, FAKE,
                                         None, None) == EINVAL
    assert lib.sparse_attn_fwd_intervals(ctypes.byref(_desc(block=48)), FAKE, FAKE, FAKE, FAKE, FAKE, 4, None, None,
                                         1, 0, FAKE, None, None) == EUNSUPPORTED


def test_online_search_calls_reject_bad_arguments(lib):
    d = _desc()
    assert lib.block_energy_from_lse(ctypes.byref(d), FAKE, FAKE, None, FAKE, None) == EINVAL
    assert lib.block_energy_from_lse(ctypes.byref(d), FAKE, FAKE, FAKE, None, None) == EINVAL
    assert lib.block_energy_from_lse(ctypes.byref(d), None, FAKE, FAKE, FAKE, None) == EINVAL
    assert lib.block_energy_from_lse(ctypes.byref(_desc(head_dim=80)), FAKE, FAKE, FAKE, FAKE, None) == EUNSUPPORTED
    taus = (ctypes.c_double * 2)(0.9, 0.8)
    bad = (ctypes.c_double * 2)(0.9, float("nan"))
    neg = (ctypes.c_double * 2)(0.9, -0.1)
    f = lib.select_blocks_by_energy_heads
    assert f(FAKE, 1, 2, 8, None, 0.5, 1, 0, FAKE, None, None) == EINVAL
    assert f(FAKE, 1, 2, 8, bad, 0.5, 1, 0, FAKE, None, None) == EINVAL
    assert f(FAKE, 1, 2, 8, neg, 0.5, 1, 0, FAKE, None, None) == EINVAL
    assert f(FAKE, 1, 300, 8, taus, 0.5, 1, 0, FAKE, None, None) == EINVAL  # beyond 256 heads
    assert f(FAKE, 1, 2, 5000, taus, 0.5, 1, 0, FAKE, None, None) == EINVAL
    assert f(None, 1, 2, 8, taus, 0.5, 1, 0, FAKE, None, None) == EINVAL


def test_heavy_order_rejects_bad_arguments(lib):
    f = lib.order_heavy_rows_first
    assert f(None, 4, 4, 2.0, FAKE, None) == EINVAL
    assert f(FAKE, 4, 4, 2.0, None, None) == EINVAL
    assert f(FAKE, 0, 4, 2.0, FAKE, None) == EINVAL
    assert f(FAKE, 4, 4, -1.0, FAKE, None) == EINVAL
    assert f(FAKE, 4, 4, float("inf"), FAKE, None) == EINVAL


def test_energy_ws_rejects_bad_arguments(lib):
    d = _desc()  # bf16, 2 heads, 256 tokens, block 128: nb = 2, workspace 2*2*2*128*4 = 4096 bytes
    f = lib.calib_block_energy_ws
    assert f(ctypes.byref(d), FAKE, FAKE, None, None, FAKE, FAKE, None, 4096, None) == EINVAL  # no workspace
    # smaller than one workgroup's rows (two query blocks x nb x block floats = 2048 bytes): ECAPACITY
    assert f(ctypes.byref(d), FAKE, FAKE, None, None, FAKE, FAKE, FAKE, 2047, None) == 4
    # with V one query block per workgroup (1024 bytes)
    assert f(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1023, None) == 4
    assert f(ctypes.byref(d), FAKE, FAKE, None, None, FAKE, FAKE, FAKE, -1, None) == EINVAL
    assert f(ctypes.byref(d), FAKE, FAKE, None, None, None, FAKE, FAKE, 4096, None) == EINVAL  # no lse
    assert f(ctypes.byref(d), FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, 4096, None) == EINVAL  # v without o
    assert f(ctypes.byref(d), FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, 4096, None) == EINVAL  # o without v
    assert f(ctypes.byref(d), FAKE, FAKE, None, None, FAKE, FAKE, ctypes.c_void_p(0x10004), 4096, None) == EINVAL
    assert f(ctypes.byref(_desc(block=48)), FAKE, FAKE, None, None, FAKE, FAKE, FAKE, 1 << 20, None) == EUNSUPPORTED