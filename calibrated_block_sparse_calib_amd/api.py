"""Python binding of libcalibattn.so: one function per C entry point, same names.

Argument marshalling only -- every step runs in the library's HIP kernels.
PyTorch provides device memory and the current stream.  Attention tensors are
[batch, heads, seq_len, head_dim] (head_dim contiguous) in float32 or bfloat16 on
the GPU; q, k, v and o must share one stride pattern.
"""
import ctypes
from typing import Optional, Sequence, Tuple

import numpy as np
import torch

from . import _lib

_DTYPES = {torch.float32: 0, torch.bfloat16: 1}


class CalibAttnError(RuntimeError):
    pass


def _check(status: int, what: str):
    if status != 0:
        msg = _lib.load().cba_status_str(status).decode()
        raise CalibAttnError(f"{what} failed: status {status} ({msg})")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _require_gpu(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise CalibAttnError("tensors must be on the GPU")


def make_desc(q: torch.Tensor, block: int, n_prefix: int = 0, grid: Optional[Sequence[int]] = None,
              scale: float = 0.0) -> _lib.AttnDesc:
    """Descriptor of a [batch, heads, seq_len, head_dim] attention problem."""
    if q.dim() != 4:
        raise CalibAttnError("expected a [batch, heads, seq_len, head_dim] tensor")
    if q.dtype not in _DTYPES:
        raise CalibAttnError(f"unsupported dtype {q.dtype}")
    if q.stride(3) != 1:
        raise CalibAttnError("head_dim must be contiguous")
    b, h, n, d = q.shape
    gf, gh, gw = (0, 0, 0) if grid is None else (int(x) for x in grid)
    return _lib.AttnDesc(
        _DTYPES[q.dtype], b, h, n, d, int(block), int(n_prefix), gf, gh, gw, float(scale),
        q.stride(0), q.stride(1), q.stride(2),
    )


def _same_layout(ref: torch.Tensor, *ts):
    for t in ts:
        if t is None:
            continue
        if t.shape != ref.shape or t.stride() != ref.stride() or t.dtype != ref.dtype:
            raise CalibAttnError("q, k, v and o must share shape, strides and dtype")


def _check_out(t: Optional[torch.Tensor], shape, dtype, name: str):
    """A caller-supplied buffer the library writes (or reads) by pointer alone: its
    dtype, shape and contiguity must be exactly the documented ones."""
    if t is None:
        return
    if t.dtype != dtype or tuple(t.shape) != tuple(shape) or not t.is_contiguous():
        raise CalibAttnError(f"{name} must be a contiguous {dtype} tensor of shape {tuple(shape)}")


def _out_like(q: torch.Tensor) -> torch.Tensor:
    """A new output tensor with exactly q's shape and strides (the library writes O
    with the strides it reads Q with)."""
    return torch.empty_strided(q.shape, q.stride(), dtype=q.dtype, device=q.device)


def _rep_array(rep_heads, heads):
    if rep_heads is None:
        return None, None
    arr = np.ascontiguousarray(np.asarray(rep_heads, dtype=np.uint8).reshape(-1))
    if arr.shape[0] != heads:
        raise CalibAttnError("rep_heads needs one flag per head")
    return arr, arr.ctypes.data_as(ctypes.c_void_p)


def n_blocks(seq_len: int, block: int) -> int:
    return (seq_len + block - 1) // block


def calib_block_energy(q, k, v=None, *, block: int, n_prefix: int = 0, grid=None, scale: float = 0.0,
                       lse: Optional[torch.Tensor] = None, energy: Optional[torch.Tensor] = None,
                       o: Optional[torch.Tensor] = None):
    """Dense pass (LSE cached, O when v is given) then block energies.
    The batch index is the calibration draw.  Returns (energy, lse, o)."""
    _require_gpu(q, k, v, lse, energy, o)
    _same_layout(q, k, v, o)
    desc = make_desc(q, block, n_prefix, grid, scale)
    b, h, n, _ = q.shape
    nb = n_blocks(n, block)
    _check_out(lse, (b, h, n), torch.float32, "lse")
    _check_out(energy, (b, h, nb, nb), torch.float32, "energy")
    if lse is None:
        lse = torch.empty((b, h, n), dtype=torch.float32, device=q.device)
    if energy is None:
        energy = torch.empty((b, h, nb, nb), dtype=torch.float32, device=q.device)
    if v is not None and o is None:
        o = _out_like(q)
    _check(_lib.load().calib_block_energy(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(o),
                                          _ptr(lse), _ptr(energy), _stream()), "calib_block_energy")
    return energy, lse, o


def select_blocks_by_energy(energy: torch.Tensor, tau: float, rho: float = 0.5, force_diag: bool = True,
                            n_dense_prefix_blocks: int = 0, mask: Optional[torch.Tensor] = None,
                            votes: Optional[torch.Tensor] = None, return_votes: bool = False):
    """energy: fp32 [draws, heads, nb, nb] -> mask uint8 [heads, nb, nb] (and votes)."""
    _require_gpu(energy)
    if energy.dtype != torch.float32 or energy.dim() != 4 or not energy.is_contiguous():
        raise CalibAttnError("energy must be contiguous fp32 [draws, heads, nb, nb]")
    d, h, nb, nb2 = energy.shape
    if nb != nb2:
        raise CalibAttnError("energy must be square per head")
    _require_gpu(mask, votes)
    _check_out(mask, (h, nb, nb), torch.uint8, "mask")
    _check_out(votes, (h, nb, nb), torch.int32, "votes")
    if mask is None:
        mask = torch.empty((h, nb, nb), dtype=torch.uint8, device=energy.device)
    if return_votes and votes is None:
        votes = torch.empty((h, nb, nb), dtype=torch.int32, device=energy.device)
    _check(_lib.load().select_blocks_by_energy(_ptr(energy), d, h, nb, float(tau), float(rho), int(bool(force_diag)),
                                               int(n_dense_prefix_blocks), _ptr(mask), _ptr(votes), _stream()),
           "select_blocks_by_energy")
    return (mask, votes) if return_votes else mask


def energy_workspace_bytes(q: torch.Tensor, block: int) -> int:
    """Workspace size calib_block_energy_ws needs for q's shape."""
    b, h, n, _ = q.shape
    nb = n_blocks(n, block)
    return b * h * nb * nb * block * 4


def calib_block_energy_ws(q, k, v=None, *, block: int, n_prefix: int = 0, grid=None, scale: float = 0.0,
                          workspace: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                          energy: Optional[torch.Tensor] = None, o: Optional[torch.Tensor] = None):
    """calib_block_energy in one pass over the keys, using a workspace of
    energy_workspace_bytes(q, block) bytes (allocated here when not given).  A
    smaller workspace runs the pass in several launches with the same results; it
    must hold at least one workgroup's rows (up to 8 query blocks x nb x block
    floats).
    Returns (energy, lse, o); o is None without v."""
    _require_gpu(q, k, v, workspace, lse, energy, o)
    _same_layout(q, k, v, o)
    desc = make_desc(q, block, n_prefix, grid, scale)
    b, h, n, _ = q.shape
    nb = n_blocks(n, block)
    _check_out(lse, (b, h, n), torch.float32, "lse")
    _check_out(energy, (b, h, nb, nb), torch.float32, "energy")
    if lse is None:
        lse = torch.empty((b, h, n), dtype=torch.float32, device=q.device)
    if energy is None:
        energy = torch.empty((b, h, nb, nb), dtype=torch.float32, device=q.device)
    if v is not None and o is None:
        o = _out_like(q)
    need = energy_workspace_bytes(q, block)
    if workspace is None:
        workspace = torch.empty(need if q.dtype == torch.bfloat16 else 16, dtype=torch.uint8, device=q.device)
    if not workspace.is_contiguous():
        raise CalibAttnError("workspace must be contiguous")
    _check(_lib.load().calib_block_energy_ws(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                                             _ptr(energy), _ptr(workspace),
                                             workspace.numel() * workspace.element_size(), _stream()),
           "calib_block_energy_ws")
    return energy, lse, o


NOALLOC_MAX_BYTES = 256 << 20  # the library's fixed per-GPU array behind calib_block_energy_noalloc


def calib_block_energy_noalloc(q, k, v=None, *, block: int, n_prefix: int = 0, grid=None, scale: float = 0.0,
                               lse: Optional[torch.Tensor] = None, energy: Optional[torch.Tensor] = None,
                               o: Optional[torch.Tensor] = None):
    """calib_block_energy_ws with no workspace: the library keeps the one-pass
    log-sums in a fixed device array of its own (NOALLOC_MAX_BYTES per GPU) and
    allocates nothing.  Outputs not given are allocated here, by torch, before the
    call.  Calls that overlap on one GPU share that array and must not run
    concurrently.  Returns (energy, lse, o); o is None without v."""
    _require_gpu(q, k, v, lse, energy, o)
    _same_layout(q, k, v, o)
    desc = make_desc(q, block, n_prefix, grid, scale)
    b, h, n, _ = q.shape
    nb = n_blocks(n, block)
    _check_out(lse, (b, h, n), torch.float32, "lse")
    _check_out(energy, (b, h, nb, nb), torch.float32, "energy")
    if lse is None:
        lse = torch.empty((b, h, n), dtype=torch.float32, device=q.device)
    if energy is None:
        energy = torch.empty((b, h, nb, nb), dtype=torch.float32, device=q.device)
    if v is not None and o is None:
        o = _out_like(q)
    _check(_lib.load().calib_block_energy_noalloc(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(o),
                                                  _ptr(lse), _ptr(energy), _stream()),
           "calib_block_energy_noalloc")
    return energy, lse, o


def block_energy_from_lse(q, k, lse, *, block: int, n_prefix: int = 0, grid=None, scale: float = 0.0,
                          energy: Optional[torch.Tensor] = None):
    """Energy sweep alone from a given (possibly cached) LSE fp32 [batch, heads, seq_len].
    Returns energy fp32 [batch, heads, nb, nb]."""
    _require_gpu(q, k, lse, energy)
    _same_layout(q, k)
    desc = make_desc(q, block, n_prefix, grid, scale)
    b, h, n, _ = q.shape
    nb = n_blocks(n, block)
    if lse.dtype != torch.float32 or tuple(lse.shape) != (b, h, n) or not lse.is_contiguous():
        raise CalibAttnError("lse must be contiguous fp32 [batch, heads, seq_len]")
    if energy is None:
        energy = torch.empty((b, h, nb, nb), dtype=torch.float32, device=q.device)
    _check_out(energy, (b, h, nb, nb), torch.float32, "energy")
    _check(_lib.load().block_energy_from_lse(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(lse), _ptr(energy),
                                             _stream()), "block_energy_from_lse")
    return energy


def select_blocks_by_energy_heads(energy: torch.Tensor, tau_heads, rho: float = 0.5, force_diag: bool = True,
                                  n_dense_prefix_blocks: int = 0, mask: Optional[torch.Tensor] = None,
                                  votes: Optional[torch.Tensor] = None, return_votes: bool = False):
    """select_blocks_by_energy with one threshold per head (tau_heads: a sequence of
    heads floats, kept on the host)."""
    _require_gpu(energy)
    if energy.dtype != torch.float32 or energy.dim() != 4 or not energy.is_contiguous():
        raise CalibAttnError("energy must be contiguous fp32 [draws, heads, nb, nb]")
    d, h, nb, nb2 = energy.shape
    if nb != nb2:
        raise CalibAttnError("energy must be square per head")
    taus = np.ascontiguousarray(np.asarray(tau_heads, dtype=np.float64).reshape(-1))
    if taus.shape[0] != h:
        raise CalibAttnError("tau_heads needs one threshold per head")
    _require_gpu(mask, votes)
    _check_out(mask, (h, nb, nb), torch.uint8, "mask")
    _check_out(votes, (h, nb, nb), torch.int32, "votes")
    if mask is None:
        mask = torch.empty((h, nb, nb), dtype=torch.uint8, device=energy.device)
    if return_votes and votes is None:
        votes = torch.empty((h, nb, nb), dtype=torch.int32, device=energy.device)
    _check(_lib.load().select_blocks_by_energy_heads(_ptr(energy), d, h, nb, taus.ctypes.data_as(ctypes.c_void_p),
                                                     float(rho), int(bool(force_diag)), int(n_dense_prefix_blocks),
                                                     _ptr(mask), _ptr(votes), _stream()),
           "select_blocks_by_energy_heads")
    return (mask, votes) if return_votes else mask


def build_block_csr(mask: torch.Tensor, with_order: bool = True, exact: bool = False, count_only: bool = False,
                    ) -> Tuple[torch.Tensor, Optional[torch.Tensor], Optional[torch.Tensor]]:
    """mask uint8 [..., nkb] (rows = all leading dims) -> (row_ptr, col_idx, work_order).

    exact=False: one call with capacity rows * nkb (no host synchronisation); the
    first row_ptr[-1] entries of col_idx are the skip list.  exact=True: a count
    pass, a host read of nnz, then the fill into a tensor of exactly nnz entries.
    count_only=True: the count pass alone, returning (row_ptr, None, None)."""
    _require_gpu(mask)
    if mask.dtype != torch.uint8 or not mask.is_contiguous():
        raise CalibAttnError("mask must be contiguous uint8")
    nkb = mask.shape[-1]
    rows = mask.numel() // nkb
    lib = _lib.load()
    row_ptr = torch.empty(rows + 1, dtype=torch.int32, device=mask.device)
    if count_only:
        _check(lib.build_block_csr(_ptr(mask), rows, nkb, _ptr(row_ptr), None, 0, None, _stream()),
               "build_block_csr(count)")
        return row_ptr, None, None
    order = torch.empty(rows, dtype=torch.int32, device=mask.device) if with_order else None
    if exact:
        _check(lib.build_block_csr(_ptr(mask), rows, nkb, _ptr(row_ptr), None, 0, None, _stream()),
               "build_block_csr(count)")
        cap = int(row_ptr[-1].item())
    else:
        cap = rows * nkb
    col_idx = torch.empty(max(cap, 1), dtype=torch.int32, device=mask.device)
    _check(lib.build_block_csr(_ptr(mask), rows, nkb, _ptr(row_ptr), _ptr(col_idx), cap, _ptr(order), _stream()),
           "build_block_csr")
    return row_ptr, col_idx, order


def order_heavy_rows_first(row_ptr: torch.Tensor, nkb: int, factor: float = 2.0,
                           work_order: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Row order with the rows holding more than factor x the mean kept blocks first
    (longest first), then the other rows in place.  row_ptr from build_block_csr."""
    _require_gpu(row_ptr, work_order)
    if row_ptr.dtype != torch.int32 or not row_ptr.is_contiguous():
        raise CalibAttnError("row_ptr must be contiguous int32")
    rows = row_ptr.numel() - 1
    if work_order is None:
        work_order = torch.empty(rows, dtype=torch.int32, device=row_ptr.device)
    if work_order.dtype != torch.int32 or work_order.numel() != rows or not work_order.is_contiguous():
        raise CalibAttnError("work_order must be contiguous int32 [rows]")
    _check(_lib.load().order_heavy_rows_first(_ptr(row_ptr), rows, int(nkb), float(factor), _ptr(work_order),
                                              _stream()), "order_heavy_rows_first")
    return work_order


def build_block_intervals(mask: torch.Tensor, exact: bool = False) -> Tuple[torch.Tensor, torch.Tensor]:
    """mask uint8 [..., nkb] (rows = all leading dims) -> (iv_ptr int32 [rows + 1],
    ivs [capacity]): the maximal runs of kept blocks of every row, each packed as
    first | count << 16 (uint32 bits, held in an int32 tensor).

    exact=False: one call with the capacity that can never be exceeded (rows *
    ceil(nkb / 2)); the first iv_ptr[-1] entries are the runs.  exact=True: a count
    pass, a host read of the total, then the fill into exactly that many entries."""
    _require_gpu(mask)
    if mask.dtype != torch.uint8 or not mask.is_contiguous():
        raise CalibAttnError("mask must be contiguous uint8")
    nkb = mask.shape[-1]
    rows = mask.numel() // nkb
    lib = _lib.load()
    iv_ptr = torch.empty(rows + 1, dtype=torch.int32, device=mask.device)
    if exact:
        _check(lib.build_block_intervals(_ptr(mask), rows, nkb, _ptr(iv_ptr), None, 0, _stream()),
               "build_block_intervals(count)")
        cap = int(iv_ptr[-1].item())
    else:
        cap = rows * ((nkb + 1) // 2)
    ivs = torch.empty(max(cap, 1), dtype=torch.int32, device=mask.device)
    _check(lib.build_block_intervals(_ptr(mask), rows, nkb, _ptr(iv_ptr), _ptr(ivs), cap, _stream()),
           "build_block_intervals")
    return iv_ptr, ivs


def sparse_attn_fwd_intervals(q, k, v, iv_ptr, ivs, *, block: int, work_order=None, rep_heads=None,
                              anchor_stride: int = 1, fuse_broadcast: bool = True, n_prefix: int = 0, grid=None,
                              scale: float = 0.0, o: Optional[torch.Tensor] = None,
                              lse: Optional[torch.Tensor] = None, return_lse: bool = False):
    """sparse_attn_fwd with the skip list as block intervals (build_block_intervals)."""
    _require_gpu(q, k, v, iv_ptr, ivs, work_order, o, lse)
    if o is None:
        o = _out_like(q)
    _same_layout(q, k, v, o)
    desc = make_desc(q, block, n_prefix, grid, scale)
    b, h, n, _ = q.shape
    _check_out(lse, (b, h, n), torch.float32, "lse")
    if return_lse and lse is None:
        lse = torch.empty((b, h, n), dtype=torch.float32, device=q.device)
    if iv_ptr.dtype != torch.int32 or ivs.dtype not in (torch.int32, torch.uint32):
        raise CalibAttnError("iv_ptr must be int32 and ivs 32-bit")
    if not (iv_ptr.is_contiguous() and ivs.is_contiguous()):
        raise CalibAttnError("iv_ptr and ivs must be contiguous")
    if iv_ptr.numel() != h * n_blocks(n, block) + 1:
        raise CalibAttnError("iv_ptr must have heads * nb + 1 entries")
    if work_order is not None and (work_order.dtype != torch.int32 or work_order.numel() != h * n_blocks(n, block)
                                   or not work_order.is_contiguous()):
        raise CalibAttnError("work_order must be contiguous int32 [heads * nb]")
    rep_arr, rep_ptr = _rep_array(rep_heads, h)
    _check(_lib.load().sparse_attn_fwd_intervals(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(iv_ptr),
                                                 _ptr(ivs), ivs.numel(), _ptr(work_order), rep_ptr,
                                                 int(anchor_stride), int(bool(fuse_broadcast)), _ptr(o), _ptr(lse),
                                                 _stream()),
           "sparse_attn_fwd_intervals")
    del rep_arr
    return (o, lse) if return_lse else o


def sparse_attn_fwd(q, k, v, row_ptr, col_idx, *, block: int, work_order=None, rep_heads=None,
                    anchor_stride: int = 1, fuse_broadcast: bool = True, n_prefix: int = 0, grid=None,
                    scale: float = 0.0, o: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                    return_lse: bool = False):
    """Block-sparse attention over the kept blocks in (row_ptr, col_idx)."""
    _require_gpu(q, k, v, row_ptr, col_idx, work_order, o, lse)
    if o is None:
        o = _out_like(q)
    _same_layout(q, k, v, o)
    desc = make_desc(q, block, n_prefix, grid, scale)
    b, h, n, _ = q.shape
    _check_out(lse, (b, h, n), torch.float32, "lse")
    if return_lse and lse is None:
        lse = torch.empty((b, h, n), dtype=torch.float32, device=q.device)
    if row_ptr.dtype != torch.int32 or col_idx.dtype != torch.int32:
        raise CalibAttnError("row_ptr and col_idx must be int32")
    if not (row_ptr.is_contiguous() and col_idx.is_contiguous()):
        raise CalibAttnError("row_ptr and col_idx must be contiguous")
    if row_ptr.numel() != h * n_blocks(n, block) + 1:
        raise CalibAttnError("row_ptr must have heads * nb + 1 entries")
    if work_order is not None and (work_order.dtype != torch.int32 or work_order.numel() != h * n_blocks(n, block)
                                   or not work_order.is_contiguous()):
        raise CalibAttnError("work_order must be contiguous int32 [heads * nb]")
    rep_arr, rep_ptr = _rep_array(rep_heads, h)
    _check(_lib.load().sparse_attn_fwd(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(row_ptr), _ptr(col_idx),
                                       col_idx.numel(), _ptr(work_order), rep_ptr, int(anchor_stride),
                                       int(bool(fuse_broadcast)), _ptr(o), _ptr(lse), _stream()),
           "sparse_attn_fwd")
    del rep_arr
    return (o, lse) if return_lse else o


def rep_row_broadcast(o: torch.Tensor, rep_heads, anchor_stride: int, *, block: int, n_prefix: int = 0,
                      grid=None):
    """Copy anchor-row outputs to their follower rows, in place.  Returns o."""
    _require_gpu(o)
    desc = make_desc(o, block, n_prefix, grid)
    rep_arr, rep_ptr = _rep_array(rep_heads, o.shape[1])
    _check(_lib.load().rep_row_broadcast(ctypes.byref(desc), _ptr(o), rep_ptr, int(anchor_stride), _stream()),
           "rep_row_broadcast")
    del rep_arr
    return o


def dense_attn_fwd(q, k, v, *, block: int = 128, scale: float = 0.0, o: Optional[torch.Tensor] = None,
                   lse: Optional[torch.Tensor] = None, return_lse: bool = False):
    """Dense attention over every key (the baseline)."""
    _require_gpu(q, k, v, o, lse)
    if o is None:
        o = _out_like(q)
    _same_layout(q, k, v, o)
    desc = make_desc(q, block, 0, None, scale)
    b, h, n, _ = q.shape
    _check_out(lse, (b, h, n), torch.float32, "lse")
    if return_lse and lse is None:
        lse = torch.empty((b, h, n), dtype=torch.float32, device=q.device)
    _check(_lib.load().dense_attn_fwd(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _stream()),
           "dense_attn_fwd")
    return (o, lse) if return_lse else o


def spatial_rep_similarity(q, k, lse, anchor_stride: int, *, n_prefix: int = 0, grid=None, scale: float = 0.0,
                           token_cos: Optional[torch.Tensor] = None, head_sim: Optional[torch.Tensor] = None):
    """Cosine similarity between each follower token's attention row and its
    anchor's, and its mean per (batch item, head).  lse: fp32 [batch, heads, seq_len]
    of the same q and k (calib_block_energy or dense_attn_fwd).  Returns
    (head_sim [batch, heads], token_cos [batch, heads, seq_len]); token_cos is only
    written at follower tokens (a new tensor starts as NaN)."""
    _require_gpu(q, k, lse, token_cos, head_sim)
    _same_layout(q, k)
    desc = make_desc(q, 128, n_prefix, grid, scale)
    b, h, n, _ = q.shape
    if lse.dtype != torch.float32 or tuple(lse.shape) != (b, h, n) or not lse.is_contiguous():
        raise CalibAttnError("lse must be contiguous fp32 [batch, heads, seq_len]")
    if token_cos is None:
        token_cos = torch.full((b, h, n), float("nan"), dtype=torch.float32, device=q.device)
    if head_sim is None:
        head_sim = torch.empty((b, h), dtype=torch.float32, device=q.device)
    for t, shape in ((token_cos, (b, h, n)), (head_sim, (b, h))):
        if t.dtype != torch.float32 or tuple(t.shape) != shape or not t.is_contiguous():
            raise CalibAttnError("token_cos and head_sim must be contiguous fp32 of the documented shapes")
    _check(_lib.load().spatial_rep_similarity(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(lse), int(anchor_stride),
                                              _ptr(token_cos), _ptr(head_sim), _stream()),
           "spatial_rep_similarity")
    return head_sim, token_cos


def select_rep_heads(head_sim: torch.Tensor, gamma: float, rep_heads: Optional[torch.Tensor] = None):
    """head_sim fp32 [draws, heads] -> uint8 [heads] on the GPU: 1 where the mean over
    the draws is strictly above gamma."""
    _require_gpu(head_sim, rep_heads)
    if head_sim.dtype != torch.float32 or head_sim.dim() != 2 or not head_sim.is_contiguous():
        raise CalibAttnError("head_sim must be contiguous fp32 [draws, heads]")
    d, h = head_sim.shape
    if rep_heads is None:
        rep_heads = torch.empty(h, dtype=torch.uint8, device=head_sim.device)
    if rep_heads.dtype != torch.uint8 or rep_heads.numel() != h or not rep_heads.is_contiguous():
        raise CalibAttnError("rep_heads must be contiguous uint8 [heads]")
    _check(_lib.load().select_rep_heads(_ptr(head_sim), d, h, float(gamma), _ptr(rep_heads), _stream()),
           "select_rep_heads")
    return rep_heads


def version() -> int:
    return int(_lib.load().cba_version())
