"""The Python binding refuses caller-supplied output buffers of the wrong dtype,
shape or layout before anything reaches the library (which takes bare pointers and
would write past a short buffer).  CPU only: the GPU-residency check is bypassed and
the library is replaced by a stub that records being reached."""
import pytest
import torch

import calibrated_block_sparse_calib_amd as cba
from calibrated_block_sparse_calib_amd import _lib, api


class Reached(Exception):
    pass


@pytest.fixture(autouse=True)
def no_library(monkeypatch):
    monkeypatch.setattr(api, "_require_gpu", lambda *ts: None)

    def load():
        raise Reached()

    monkeypatch.setattr(_lib, "load", load)


B, H, N, D, BLK = 1, 2, 40, 64, 32
NB = (N + BLK - 1) // BLK


def qkv():
    return [torch.zeros(B, H, N, D, dtype=torch.bfloat16) for _ in range(3)]


def f32(*shape):
    return torch.zeros(*shape, dtype=torch.float32)


def test_correct_outputs_reach_the_library():
    q, k, v = qkv()
    with pytest.raises(Reached):
        cba.calib_block_energy(q, k, v, block=BLK, lse=f32(B, H, N), energy=f32(B, H, NB, NB), o=torch.zeros_like(q))
    with pytest.raises(Reached):
        cba.select_blocks_by_energy(f32(1, H, NB, NB), 0.9, mask=torch.zeros(H, NB, NB, dtype=torch.uint8),
                                    votes=torch.zeros(H, NB, NB, dtype=torch.int32))
    with pytest.raises(Reached):
        cba.dense_attn_fwd(q, k, v, block=BLK, lse=f32(B, H, N))


@pytest.mark.parametrize("kw", [
    {"lse": f32(B, H, N - 1)},
    {"lse": torch.zeros(B, H, N, dtype=torch.float64)},
    {"energy": f32(B, H, NB, NB - 1)},
    {"energy": f32(B, H, NB, NB).transpose(2, 3)},
    {"o": torch.zeros(B, H, N, D, dtype=torch.float32)},
    {"o": torch.zeros(B, H, N + 1, D, dtype=torch.bfloat16)},
])
def test_energy_calls_refuse_bad_outputs(kw):
    q, k, v = qkv()
    with pytest.raises(cba.CalibAttnError):
        cba.calib_block_energy(q, k, v, block=BLK, **kw)
    kw_ws = {key: val for key, val in kw.items() if key != "o"}
    if kw_ws:
        with pytest.raises(cba.CalibAttnError):
            cba.calib_block_energy_ws(q, k, block=BLK, workspace=torch.zeros(16, dtype=torch.uint8), **kw_ws)
    if "energy" in kw:
        with pytest.raises(cba.CalibAttnError):
            cba.block_energy_from_lse(q, k, f32(B, H, N), block=BLK, **kw)


@pytest.mark.parametrize("kw", [
    {"mask": torch.zeros(H, NB, NB - 1, dtype=torch.uint8)},
    {"mask": torch.zeros(H, NB, NB, dtype=torch.int32)},
    {"votes": torch.zeros(H, NB, NB, dtype=torch.uint8)},
    {"votes": torch.zeros(H, NB + 1, NB, dtype=torch.int32)},
])
def test_selection_refuses_bad_outputs(kw):
    e = f32(1, H, NB, NB)
    with pytest.raises(cba.CalibAttnError):
        cba.select_blocks_by_energy(e, 0.9, **kw)
    with pytest.raises(cba.CalibAttnError):
        cba.select_blocks_by_energy_heads(e, [0.9] * H, **kw)


def test_attention_calls_refuse_bad_lse_and_skip_lists():
    q, k, v = qkv()
    rows = H * NB
    row_ptr = torch.zeros(rows + 1, dtype=torch.int32)
    col_idx = torch.zeros(rows * NB, dtype=torch.int32)
    bad_lse = f32(B, H, N + 3)
    with pytest.raises(cba.CalibAttnError):
        cba.dense_attn_fwd(q, k, v, block=BLK, lse=bad_lse)
    with pytest.raises(cba.CalibAttnError):
        cba.sparse_attn_fwd(q, k, v, row_ptr, col_idx, block=BLK, lse=bad_lse)
    with pytest.raises(cba.CalibAttnError):
        cba.sparse_attn_fwd_intervals(q, k, v, row_ptr, col_idx, block=BLK, lse=bad_lse)
    strided = torch.zeros(2 * rows * NB, dtype=torch.int32)[::2]
    with pytest.raises(cba.CalibAttnError):
        cba.sparse_attn_fwd(q, k, v, row_ptr, strided, block=BLK)
    with pytest.raises(cba.CalibAttnError):
        cba.sparse_attn_fwd(q, k, v, row_ptr, col_idx, block=BLK, work_order=torch.zeros(2 * rows, dtype=torch.int32)[::2])
    with pytest.raises(Reached):
        cba.sparse_attn_fwd(q, k, v, row_ptr, col_idx, block=BLK, lse=f32(B, H, N))
