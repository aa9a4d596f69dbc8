"""The calibrated mask dictionary on the GPU, at the Mochi workload's full size:
three timestep buckets calibrated with a schedule that is stricter early
(tau = 0.98, 0.95, 0.92) and two layers, then saved, reloaded and used.

  * each entry's mask: bit-exact against the oracle's selection on the GPU's own
    energies (the oracle's rule applied to the same fp32 values), and its runs
    bit-exact against the oracle's block intervals of that mask;
  * the processing order: the oracle's heavy-rows-first order;
  * the output of the reloaded entry: bit-identical to the in-memory entry's and
    to sparse_attn_fwd over the CSR skip list of the same mask, and within the
    bf16 bars of the oracle on sampled query blocks.
"""
import dataclasses

import numpy as np
import pytest
import torch

import calibrated_block_sparse_calib_amd as cba
import oracle
from calibrated_block_sparse_calib_amd.mask_dict import MaskDictionary
from workloads import get_config, make_qkv
from tests.gpu_util import check_bf16_outputs, log, to_host

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(900)]

SCHEDULE = (0.98, 0.95, 0.92)


def _dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16).cuda()


def test_mochi_schedule_dictionary_round_trip(tmp_path):
    base = get_config("mochi")
    md = MaskDictionary(SCHEDULE, block=base.block, rho=base.rho)
    masks, evals = {}, {}
    for layer in range(2):
        # a second layer: the same shapes, other seeds
        cfg = base if layer == 0 else dataclasses.replace(base, seed=base.seed + 100)
        for bucket in range(3):
            log(f"calibrating mochi layer {layer} bucket {bucket} at tau {SCHEDULE[bucket]}")
            draws = [make_qkv(cfg, draw=d, bucket=bucket, with_v=False) for d in range(cfg.calib_draws)]
            q = _dev(np.stack([x[0] for x in draws]))
            k = _dev(np.stack([x[1] for x in draws]))
            entry, energy, mask = md.calibrate(bucket, layer, q, k, n_prefix=cfg.n_prefix, grid=cfg.grid,
                                               return_energy=True)
            torch.cuda.synchronize()
            m = mask.cpu().numpy()
            ref_m, _ = oracle.select_blocks(to_host(energy), SCHEDULE[bucket], cfg.rho, True, cfg.n_prefix_blocks)
            np.testing.assert_array_equal(m, ref_m)
            ip, first, count, _ = oracle.build_intervals(m.reshape(-1, cfg.nb))
            packed = (first.astype(np.uint32) | (count.astype(np.uint32) << np.uint32(16))).view(np.int32)
            np.testing.assert_array_equal(entry.iv_ptr.cpu().numpy(), ip)
            np.testing.assert_array_equal(entry.ivs.cpu().numpy(), packed)
            counts = m.reshape(-1, cfg.nb).sum(axis=1)
            np.testing.assert_array_equal(entry.order.cpu().numpy(), oracle.heavy_first_order(counts, 2.0))
            log(f"  density {m.mean():.3f}, {entry.runs} runs for {int(m.sum())} kept blocks")
            masks[(bucket, layer)] = m
            del q, k, energy, mask
            evals[(bucket, layer)] = make_qkv(cfg, draw=cfg.calib_draws, bucket=bucket)
    path = str(tmp_path / "mochi_masks.npz")
    md.save(path)
    md2 = MaskDictionary.load(path, device="cuda")
    assert md2.keys() == md.keys() and md2.tau_schedule == list(SCHEDULE)
    n_steps = 30
    for step in (0, 12, 29):
        bucket = step * 3 // n_steps
        for layer in range(2):
            q, k, v = evals[(bucket, layer)]
            qd, kd, vd = _dev(q[None]), _dev(k[None]), _dev(v[None])
            kw = dict(step=step, n_steps=n_steps, layer=layer, n_prefix=base.n_prefix, grid=base.grid)
            o_mem = md.attention(qd, kd, vd, **kw)
            o_load = md2.attention(qd, kd, vd, **kw)
            m = masks[(bucket, layer)]
            row_ptr, col_idx, _ = cba.build_block_csr(torch.from_numpy(m).cuda())
            o_csr = cba.sparse_attn_fwd(qd, kd, vd, row_ptr, col_idx, block=base.block, n_prefix=base.n_prefix,
                                        grid=base.grid)
            torch.cuda.synchronize()
            assert torch.equal(o_load, o_mem), f"step {step} layer {layer}: reloaded entry differs"
            assert torch.equal(o_load, o_csr), f"step {step} layer {layer}: intervals differ from CSR"
            got = to_host(o_load)[0]
            rng = np.random.default_rng(step * 10 + layer)
            gots, refs = [], []
            for h in rng.choice(base.heads, 3, replace=False):
                for qb in sorted({0, base.nb - 1, int(rng.integers(0, base.nb))}):
                    rows = np.zeros(base.seq_len, dtype=bool)
                    rows[qb * base.block:(qb + 1) * base.block] = True
                    ref, _ = oracle.sparse_attention(q[h], k[h], v[h], m[h], base.block, None, rows)
                    gots.append(got[h][rows])
                    refs.append(ref[rows])
            mx, exc, mean = check_bf16_outputs(np.concatenate(gots), np.concatenate(refs), f"step {step} l{layer}")
            log(f"  step {step} (bucket {bucket}) layer {layer}: bit-identical after reload; oracle max {mx:.2e} "
                f"(beyond rounding {exc:.2e}) mean {mean:.2e}")
