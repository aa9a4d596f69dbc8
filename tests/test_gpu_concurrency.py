"""The library keeps no state between calls: two host threads, each enqueueing the
skip-list build, sparse attention with a repetition head and the one-pass energies
on its own stream (default priority) and its own problem, get the same bits as the
same calls made one after the other."""
import threading

import numpy as np
import pytest
import torch

import calibrated_block_sparse_calib_amd as cba
from tests.gpu_util import log
from workloads import AttnConfig, make_qkv, random_block_mask, rep_head_flags

pytestmark = pytest.mark.gpu


def _problem(seed, grid):
    cfg = AttnConfig(name=f"conc{seed}", heads=3, head_dim=128, grid=grid, block=128, dtype="bf16", seed=seed,
                     n_prefix=0, lt=3.0, ls=8.0, density_range=(0.3, 0.6), rep_heads_fixed=(1,), anchor_stride=4)
    q, k, v = make_qkv(cfg, draw=0)
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x))[None].to(torch.bfloat16).cuda()
    p = dict(cfg=cfg, q=dev(q), k=dev(k), v=dev(v), mask=torch.from_numpy(random_block_mask(cfg)).cuda(),
             rep=rep_head_flags(cfg))
    p["ws"] = torch.empty(cba.energy_workspace_bytes(p["q"], cfg.block), dtype=torch.uint8, device="cuda")
    return p


def _run(p):
    cfg = p["cfg"]
    row_ptr, col_idx, order = cba.build_block_csr(p["mask"])
    o = cba.sparse_attn_fwd(p["q"], p["k"], p["v"], row_ptr, col_idx, block=cfg.block, work_order=order,
                            rep_heads=p["rep"], anchor_stride=cfg.anchor_stride, fuse_broadcast=True,
                            n_prefix=cfg.n_prefix, grid=cfg.grid)
    e, lse, _ = cba.calib_block_energy_ws(p["q"], p["k"], block=cfg.block, n_prefix=cfg.n_prefix, grid=cfg.grid,
                                          workspace=p["ws"])
    return [row_ptr, col_idx, order, o, e, lse]


def test_two_threads_on_two_streams_match_serial_calls():
    probs = [_problem(31, (3, 9, 40)), _problem(32, (2, 12, 33))]
    ref = [_run(p) for p in probs]
    torch.cuda.synchronize()
    results = [[None] * 3 for _ in probs]
    errors = []

    def worker(i):
        try:
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                for it in range(3):
                    results[i][it] = _run(probs[i])
            s.synchronize()
        except Exception as exc:  # reported by the main thread
            errors.append(exc)

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(len(probs))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    torch.cuda.synchronize()
    assert not errors, errors
    for i, p in enumerate(probs):
        nnz = int(ref[i][0][-1])
        for it in range(3):
            got = results[i][it]
            assert got is not None
            assert torch.equal(got[0], ref[i][0]) and torch.equal(got[1][:nnz], ref[i][1][:nnz])
            assert torch.equal(got[2], ref[i][2])
            for a, b in zip(got[3:], ref[i][3:]):
                assert torch.equal(a, b)
        log(f"  problem {i}: 3 concurrent runs bit-identical to the serial run (nnz {nnz})")
