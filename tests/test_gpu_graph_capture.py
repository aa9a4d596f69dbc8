"""The inference step under HIP graph capture: the skip-list build (one call,
no host synchronisation) and sparse attention with repetition heads and the
fused anchor broadcast, captured once and replayed.  Between replays new Q, K, V
and a new block mask are written into the captured buffers (as a denoising loop
would per step), with other eager work in between; every replay must equal,
bit for bit, the same calls made eagerly on the same inputs.  The library
allocates nothing and synchronises nothing, so its calls can be captured.
(tests/test_gpu_parity.py captures the C calls directly, with the separate
broadcast, and replays them on unchanged inputs.)"""
import numpy as np
import pytest
import torch

import calibrated_block_sparse_calib_amd as cba
from tests.gpu_util import log

pytestmark = pytest.mark.gpu

GRID = (5, 16, 24)  # 1920 tokens: 15 blocks of 128
HEADS, D, B, STRIDE = 4, 128, 128, 4
REP = np.array([0, 1, 0, 1], np.uint8)


def _fill(qd, kd, vd, md, seed):
    g = torch.Generator().manual_seed(seed)
    for t in (qd, kd, vd):
        t.copy_(torch.randn(t.shape, generator=g).to(t.dtype))
    nb = md.shape[-1]
    m = (torch.rand((HEADS, nb, nb), generator=g) < 0.4).to(torch.uint8)
    m[:, torch.arange(nb), torch.arange(nb)] = 1
    md.copy_(m)


def _step(qd, kd, vd, md, o):
    rp, ci, wo = cba.build_block_csr(md)
    cba.sparse_attn_fwd(qd, kd, vd, rp, ci, block=B, work_order=wo, rep_heads=REP, anchor_stride=STRIDE,
                        fuse_broadcast=True, grid=GRID, o=o)


def test_inference_step_replays_bit_identical():
    n = int(np.prod(GRID))
    nb = (n + B - 1) // B
    shape = (1, HEADS, n, D)
    qd, kd, vd = (torch.empty(shape, dtype=torch.bfloat16, device="cuda") for _ in range(3))
    md = torch.empty((HEADS, nb, nb), dtype=torch.uint8, device="cuda")
    o_graph = torch.zeros(shape, dtype=torch.bfloat16, device="cuda")
    o_eager = torch.zeros_like(o_graph)
    _fill(qd, kd, vd, md, seed=0)
    _step(qd, kd, vd, md, o_eager)  # warm-up outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _step(qd, kd, vd, md, o_graph)
    torch.cuda.synchronize()
    for i in range(4):
        _fill(qd, kd, vd, md, seed=10 + i)
        o_graph.fill_(7.0)
        g.replay()
        torch.cuda.synchronize()
        o_eager.fill_(-7.0)
        _step(qd, kd, vd, md, o_eager)
        torch.cuda.synchronize()
        assert torch.isfinite(o_graph).all(), f"replay {i}"
        assert torch.equal(o_graph, o_eager), f"replay {i}: max {float((o_graph.float() - o_eager.float()).abs().max())}"
    log("  graph: 4 replays on new inputs and masks, bit-identical to the eager step")
