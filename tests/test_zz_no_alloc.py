"""calib_block_energy_noalloc (the call that allocates nothing) against
calib_block_energy_ws with a caller workspace: energies, LSE and O bit-identical,
on two calls in a row, the second on a smaller input.  The first input's
workspace (338 MiB) exceeds the library's 256 MiB array, so that call runs in
several launches; the second covers a batch of two, block 64 (two query blocks
per workgroup) and a ragged last block.  One call is also captured in a HIP graph
and replayed, the use the entry point is for."""
import numpy as np
import pytest
import torch

import calibrated_block_sparse_calib_amd as cba
from tests.gpu_util import log

pytestmark = pytest.mark.gpu


def _inputs(batch, heads, n, d, seed):
    g = torch.Generator().manual_seed(seed)
    x = [torch.randn((batch, heads, n, d), generator=g) for _ in range(3)]
    x[1] = x[1] * 1.5  # sharper rows than N(0,1) keys give
    return [t.to(torch.bfloat16).cuda() for t in x]


def _check_pair(batch, heads, n, d, block, seed, with_v):
    q, k, v = _inputs(batch, heads, n, d, seed)
    v = v if with_v else None
    need = cba.energy_workspace_bytes(q, block)
    log(f"noalloc: batch {batch} heads {heads} n {n} d {d} B {block} V {with_v}: workspace {need / 2**20:.1f} MiB "
        f"(array {cba.api.NOALLOC_MAX_BYTES / 2**20:.0f} MiB)")
    e_ref, l_ref, o_ref = cba.calib_block_energy_ws(q, k, v, block=block)
    e, l, o = cba.calib_block_energy_noalloc(q, k, v, block=block)
    torch.cuda.synchronize()
    assert torch.equal(e, e_ref), float((e - e_ref).abs().max())
    assert torch.equal(l, l_ref)
    if with_v:
        assert torch.equal(o, o_ref)
    assert torch.isfinite(e).all()
    return need


def test_noalloc_matches_workspace_call_twice():
    big = _check_pair(batch=1, heads=3, n=60000, d=128, block=128, seed=1, with_v=False)
    assert big > cba.api.NOALLOC_MAX_BYTES  # several launches
    small = _check_pair(batch=2, heads=2, n=3001, d=64, block=64, seed=2, with_v=True)
    assert small < big


def test_noalloc_block32_and_repeat():
    # block 32 groups several query blocks per workgroup; a ragged group at each head's end
    _check_pair(batch=1, heads=3, n=1000, d=128, block=32, seed=3, with_v=False)
    _check_pair(batch=1, heads=3, n=1000, d=128, block=32, seed=3, with_v=False)


def test_noalloc_rejects_bad_arguments():
    q, k, _ = _inputs(1, 1, 256, 128, 4)
    with pytest.raises(cba.CalibAttnError):
        cba.calib_block_energy_noalloc(q, k[:, :, :200], block=128)


def test_noalloc_under_graph_capture():
    """The callers this entry point is for: one call captured in a HIP graph (after
    an eager call, which looks up the array's address), replayed three times with
    eager work between the replays (a fill of the outputs, and an eager call on
    other inputs that reuses the array); every replay bit-identical to the eager
    result."""
    q, k, v = _inputs(1, 2, 3000, 128, 5)
    e0, l0, o0 = cba.calib_block_energy_noalloc(q, k, v, block=128)
    e, l, o = torch.empty_like(e0), torch.empty_like(l0), torch.empty_like(o0)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        cba.calib_block_energy_noalloc(q, k, v, block=128, lse=l, energy=e, o=o)
    torch.cuda.synchronize()
    for i in range(3):
        e.fill_(-1.0)
        l.fill_(-1.0)
        o.fill_(-1.0)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(e, e0) and torch.equal(l, l0) and torch.equal(o, o0), f"replay {i}"
        cba.calib_block_energy_noalloc(k, q, None, block=128)
        torch.cuda.synchronize()
    log("  noalloc graph: 3 replays bit-identical to the eager call")
