"""Benchmark of calibrated block-sparse attention on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload wan14_720p]

Workload (default): Wan-2.1-14B-like 720p self-attention -- 40 heads, head_dim 128,
token grid 21x45x80 = 75600 tokens, bf16, block 128; per-head Bernoulli block masks
with density uniform in 20-50% and the diagonal kept; 10 spatial-repetition heads
with anchors every 4 image rows.  Inputs are synthetic (seeded generator) and
resident in HBM before the timed region.

A step is the inference path: build_block_csr (mask -> skip list and work order)
then sparse_attn_fwd (kept blocks only, anchor rows of repetition heads, fused
broadcast).  value = kept-block FLOPs / step time.  The other entry points
(calib_block_energy, calib_block_energy_ws, select_blocks_by_energy, spatial_rep_similarity,
select_rep_heads, rep_row_broadcast, dense_attn_fwd) are timed in the same run and
reported under "rows"; dense_attn_fwd gives the speedup.  The fp64 CPU oracle is timed on a bounded sample of query blocks of the
same workload (cpu_baseline) and its outputs are compared with the GPU's.

Prints one JSON line.
"""
import argparse
import ctypes
import hashlib
import json
import os
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "kept-block attn TFLOP/s & % bf16 MFMA peak; speedup vs dense, Wan-14B 720p"
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0
KERNEL_SOURCE = os.path.join(ROOT, "calibrated_block_sparse_calib_amd", "csrc", "attn_bf16.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "sparse_attn_fwd_wan14_720p_traffic.json")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kept_flops(mask, cfg, rep, computed):
    """4 d * sum over heads and computed query rows of the kept key tokens of the row's block."""
    n, B, nb = cfg.seq_len, cfg.block, cfg.nb
    sizes = np.minimum(B, n - np.arange(nb) * B).astype(np.int64)  # tokens per block
    kept_tokens = mask.astype(np.int64) @ sizes  # [H, nb]
    total = 0
    for h in range(cfg.heads):
        rows = computed[1] if rep[h] else computed[0]  # computed rows per query block
        total += int((rows * kept_tokens[h]).sum())
    return 4 * cfg.head_dim * total


def rows_per_block(cfg, is_rep):
    """Computed query rows per query block: all rows, or for a repetition head the
    text rows and the image rows with y % anchor_stride == 0."""
    r = np.ones(cfg.seq_len, bool)
    if is_rep:
        f_, h_, w_ = cfg.grid
        t = np.arange(cfg.n_prefix, cfg.seq_len)
        r[cfg.n_prefix:] = (((t - cfg.n_prefix) // w_) % h_) % cfg.anchor_stride == 0
    pad = cfg.nb * cfg.block - cfg.seq_len
    return np.concatenate([r, np.zeros(pad, bool)]).reshape(cfg.nb, cfg.block).sum(1).astype(np.int64)


KERNEL_UNIT = ("attn_bf16.hip", "mfma_util.h")  # the sparse kernel's own sources


def source_hash():
    """Hash of the sources compiled into the sparse kernel (its file, the device
    helpers, its compile flags and the parameter block it reads from the shared
    header): byte counters taken on another version of them are not reported."""
    import re

    h = hashlib.sha256()
    csrc = os.path.dirname(KERNEL_SOURCE)
    for name in KERNEL_UNIT:
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + f.read())
    from calibrated_block_sparse_calib_amd.build import EXTRA

    h.update(" ".join(EXTRA.get(KERNEL_UNIT[0], [])).encode())  # its compile flags
    with open(os.path.join(csrc, "cba_internal.h")) as f:
        hdr = f.read()
    for pat in (r"struct AttnParams \{.*?\n\};", r"inline bool rep_head\(.*?\n\}", r"constexpr int kMaxRepHeads = \d+;"):
        m = re.search(pat, hdr, re.S)
        h.update(m.group(0).encode() if m else b"?")
    return h.hexdigest()[:16]


def traffic_from_profile():
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except OSError:
        return None
    return t.get("bytes_per_launch") if t.get("source_hash") == source_hash() else None


def cpu_baseline(cfg, q, k, v, mask, rep, got_o, budget_s, step_flops, seed=0):
    """Time the fp64 oracle on sampled query blocks of the same workload; the time of
    a whole step (step_flops kept FLOPs) is extrapolated from the sample's rate."""
    import oracle

    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count() or 1
    rng = np.random.default_rng(seed)
    nb, B = cfg.nb, cfg.block
    picks = [(h, qb) for h in range(cfg.heads) for qb in (0, nb - 1)]  # first and ragged last blocks
    picks += [(int(h), int(qb)) for h, qb in zip(rng.integers(0, cfg.heads, 4096), rng.integers(0, nb, 4096))]
    comp_all = np.ones(cfg.seq_len, bool)
    comp_rep = oracle.computed_rows(cfg.seq_len, cfg.n_prefix, cfg.grid, cfg.anchor_stride, True)
    flops, errs, done = 0, [], 0
    t0 = time.perf_counter()
    for h, qb in picks:
        if time.perf_counter() - t0 > budget_s:
            break
        lo, hi = qb * B, min(cfg.seq_len, (qb + 1) * B)
        rows = np.zeros(cfg.seq_len, bool)
        rows[lo:hi] = (comp_rep if rep[h] else comp_all)[lo:hi]
        o, _ = oracle.sparse_attention(q[h], k[h], v[h], mask[h], B, None, rows)
        kept = sum(min(B, cfg.seq_len - kb * B) for kb in np.nonzero(mask[h, qb])[0])
        flops += 4 * cfg.head_dim * int(rows.sum()) * kept
        errs.append(np.abs(got_o[h][rows] - o[rows]))
        done += 1
    dt = time.perf_counter() - t0
    err = np.concatenate(errs)
    return {
        "value": flops / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": cores,
        "kind": "oracle",
        "sample": f"{done} query blocks ({done * B} rows max) of {cfg.name}, fp64 NumPy, {dt:.1f} s",
        "sec_per_block": dt / done,
        "extrapolated_step_s": step_flops / (flops / dt),  # by kept-work ratio, not measured
    }, {"rows_checked": int(err.shape[0]), "max_abs": float(err.max()), "mean_abs": float(err.mean())}


def skip_list_bytes(rows, nkb, nnz, runs):
    """Storage of one (timestep, layer) mask entry: bitmask, CSR, block intervals."""
    return {"bitmask": rows * ((nkb + 7) // 8), "csr": 4 * (rows + 1 + nnz), "intervals": 4 * (rows + 1 + runs)}


def rep_rows_per_head(cfg):
    """Query rows spatial_rep_similarity computes per head: every row of the row
    groups that hold a follower row (anchor row plus followers)."""
    f_, h_, w_ = cfg.grid
    s = cfg.anchor_stride
    groups = (h_ - 1 + s - 1) // s
    return f_ * w_ * min(groups * s, h_)


def rep_sampled_parity(cfg, q, k, token_cos, n_tokens=96, seed=0):
    """Oracle cosines of sampled follower tokens (the last one always) of a few heads
    against the GPU's token_cos."""
    import oracle

    rng = np.random.default_rng(seed)
    f_, h_, w_ = cfg.grid
    t = np.arange(cfg.n_prefix, cfg.seq_len)
    fol = t[((t - cfg.n_prefix) // w_) % h_ % cfg.anchor_stride != 0]
    errs = []
    for h in sorted({0, cfg.heads - 1, int(rng.integers(0, cfg.heads))}):
        pick = np.unique(np.append(rng.choice(fol, n_tokens, replace=False), fol[-1]))
        _, ref = oracle.repetition_cosines(q[h], k[h], cfg.n_prefix, cfg.grid, cfg.anchor_stride, tokens=pick)
        errs.append(np.abs(token_cos[h][pick].astype(np.float64) - ref))
    err = np.concatenate(errs)
    return {"tokens_checked": int(err.shape[0]), "max_abs": float(err.max()), "mean_abs": float(err.mean())}


def density_sweep(cfg, lib, desc, qd, kd, vd, od, row_ptr, col_idx, timeit, P, S,
                  densities=(0.10, 0.20, 0.35, 0.50, 1.0)):
    """sparse_attn_fwd on the same shape with one seeded Bernoulli density for every
    head (diagonal kept, no repetition heads); least-squares fit of time against
    kept FLOPs shows whether time scales with the kept work."""
    import dataclasses

    import torch
    from workloads import random_block_mask

    points = []
    full_rows = rows_per_block(cfg, False)
    no_rep = np.zeros(cfg.heads, bool)
    for dens in densities:
        c = dataclasses.replace(cfg, density_range=(dens, dens))
        m = random_block_mask(c) if dens < 1.0 else np.ones((cfg.heads, cfg.nb, cfg.nb), np.uint8)
        md = torch.from_numpy(m).cuda()
        st = lib.build_block_csr(P(md), cfg.heads * cfg.nb, cfg.nb, P(row_ptr), P(col_idx), col_idx.numel(), None, S)
        assert st == 0, st

        def run():
            st = lib.sparse_attn_fwd(ctypes.byref(desc), P(qd), P(kd), P(vd), P(row_ptr), P(col_idx),
                                     col_idx.numel(), None, None, cfg.anchor_stride, 0, P(od), None, S)
            assert st == 0, st

        ms = timeit(run)
        fl = kept_flops(m, cfg, no_rep, (full_rows, full_rows))
        points.append({"density": round(float(m.mean()), 4), "ms": ms, "kept_flops": fl,
                       "tflops": fl / ms / 1e9})
        del md
    x = np.array([p["kept_flops"] for p in points], float)
    y = np.array([p["ms"] for p in points], float)
    slope, icpt = np.polyfit(x, y, 1)
    r2 = 1.0 - float(((y - (slope * x + icpt)) ** 2).sum() / ((y - y.mean()) ** 2).sum())
    log("density sweep: " + ", ".join(f"{p['density']:.2f}: {p['ms']:.2f} ms" for p in points) +
        f"; fit r2 {r2:.5f}")
    return {"points": points, "fit_ms_per_tflop": slope * 1e12, "fit_intercept_ms": icpt, "fit_r2": r2,
            "marginal_tflops": 1e-9 / slope}


def calibrated_workload(name, reps=2, tau_schedule=None):
    """One calibrated workload end to end: calib_block_energy_ws over every draw
    (energies and LSE in one sweep; the two-sweep calib_block_energy is timed beside
    it), select_blocks_by_energy, build_block_csr,
    the heavy-rows-first order, and sparse_attn_fwd on a held-out draw (also in
    natural order, and through block intervals), plus dense_attn_fwd for the
    speedup.  Per timestep bucket when the workload has
    several; tau_schedule gives each bucket its own energy threshold (early
    buckets first), else every bucket uses the workload's tau."""
    import torch

    import calibrated_block_sparse_calib_amd as cba
    from workloads import get_config, make_qkv

    cfg = get_config(name)
    B, n, H, d = cfg.block, cfg.seq_len, cfg.heads, cfg.head_dim
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16).cuda()
    ev = lambda: torch.cuda.Event(enable_timing=True)

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            a, b_ = ev(), ev()
            a.record()
            fn()
            b_.record()
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b_))
        return statistics.median(ts)

    out = []
    for bucket in range(cfg.buckets):
        t0 = time.perf_counter()
        draws = [make_qkv(cfg, draw=i, bucket=bucket, with_v=False) for i in range(cfg.calib_draws)]
        qc = dev(np.stack([x[0] for x in draws]))
        kc = dev(np.stack([x[1] for x in draws]))
        del draws
        q, k, v = make_qkv(cfg, draw=cfg.calib_draws, bucket=bucket)
        qd, kd, vd = dev(q[None]), dev(k[None]), dev(v[None])
        del q, k, v
        log(f"{name} bucket {bucket}: inputs generated in {time.perf_counter() - t0:.1f} s")
        res = {}
        ws = torch.empty(cba.energy_workspace_bytes(qc, B), dtype=torch.uint8, device="cuda")
        energy, lse, _ = cba.calib_block_energy_ws(qc, kc, block=B, n_prefix=cfg.n_prefix, grid=cfg.grid, workspace=ws)
        e_ms = timed(lambda: cba.calib_block_energy_ws(qc, kc, block=B, n_prefix=cfg.n_prefix, grid=cfg.grid,
                                                      workspace=ws, lse=lse, energy=energy))
        del ws
        e2, l2, _ = cba.calib_block_energy(qc, kc, None, block=B, n_prefix=cfg.n_prefix, grid=cfg.grid)
        e2_ms = timed(lambda: cba.calib_block_energy(qc, kc, None, block=B, n_prefix=cfg.n_prefix, grid=cfg.grid,
                                                    lse=l2, energy=e2))
        e2_diff = float((e2 - energy).abs().max())
        del e2, l2
        cal_flops = 2 * n * n * d * H * cfg.calib_draws  # QK^T, once per draw
        tau = cfg.tau if tau_schedule is None else tau_schedule[min(bucket, len(tau_schedule) - 1)]
        mask = cba.select_blocks_by_energy(energy, tau, cfg.rho, True, cfg.n_prefix_blocks)
        s_ms = timed(lambda: cba.select_blocks_by_energy(energy, tau, cfg.rho, True, cfg.n_prefix_blocks,
                                                        mask=mask))
        row_ptr, col_idx, _ = cba.build_block_csr(mask, with_order=False)
        c_ms = timed(lambda: cba.build_block_csr(mask, with_order=False))
        # heavy rows (the dense text rows) first, the rest in natural order
        order = cba.order_heavy_rows_first(row_ptr, cfg.nb, 2.0)
        o_ms = timed(lambda: cba.order_heavy_rows_first(row_ptr, cfg.nb, 2.0, work_order=order))
        o = torch.empty_like(qd)
        spn_ms = timed(lambda: cba.sparse_attn_fwd(qd, kd, vd, row_ptr, col_idx, block=B, n_prefix=cfg.n_prefix,
                                                   grid=cfg.grid, o=o))
        sp_ms = timed(lambda: cba.sparse_attn_fwd(qd, kd, vd, row_ptr, col_idx, block=B, n_prefix=cfg.n_prefix,
                                                  grid=cfg.grid, o=o, work_order=order))
        iv_ptr, ivs = cba.build_block_intervals(mask)
        ivb_ms = timed(lambda: cba.build_block_intervals(mask))
        o_iv = torch.empty_like(qd)
        iv_ms = timed(lambda: cba.sparse_attn_fwd_intervals(qd, kd, vd, iv_ptr, ivs, block=B, n_prefix=cfg.n_prefix,
                                                            grid=cfg.grid, o=o_iv, work_order=order))
        same = bool(torch.equal(o, o_iv))
        n_runs = int(iv_ptr[-1].item())
        del o_iv, iv_ptr, ivs
        de_ms = timed(lambda: cba.dense_attn_fwd(qd, kd, vd, block=B, o=o))
        m = mask.cpu().numpy()
        kept = kept_flops(m, cfg, np.zeros(H, bool), (rows_per_block(cfg, False),) * 2)
        dens = m.mean(axis=(1, 2))
        res.update({"bucket": bucket, "tau": tau, "draws": cfg.calib_draws, "calib_ms": e_ms,
                    "calib_tflops": cal_flops / e_ms / 1e9, "calib_two_sweep_ms": e2_ms,
                    "calib_two_sweep_max_abs_diff": e2_diff, "select_ms": s_ms, "csr_ms": c_ms,
                    "mask_density": float(m.mean()), "head_density_min": float(dens.min()),
                    "head_density_max": float(dens.max()), "order_ms": o_ms, "sparse_natural_order_ms": spn_ms,
                    "sparse_ms": sp_ms, "sparse_tflops": kept / sp_ms / 1e9,
                    "dense_ms": de_ms, "speedup_vs_dense": de_ms / sp_ms,
                    "intervals_build_ms": ivb_ms, "sparse_intervals_ms": iv_ms, "intervals_same_output": same,
                    "runs": n_runs, "kept_blocks": int(m.sum()),
                    "skip_list_bytes": skip_list_bytes(H * cfg.nb, cfg.nb, int(m.sum()), n_runs)})
        log(f"{name} bucket {bucket}: calibration {e_ms:.1f} ms ({res['calib_tflops']:.0f} TFLOP/s; two sweeps "
            f"{e2_ms:.1f} ms, max |dE| {e2_diff:.1e}), select "
            f"{s_ms:.2f} ms, density {res['mask_density']:.3f}, sparse {sp_ms:.2f} ms (natural order {spn_ms:.2f}) "
            f"({res['sparse_tflops']:.0f} TFLOP/s kept), dense {de_ms:.2f} ms; intervals: {n_runs} runs for "
            f"{int(m.sum())} blocks, sparse {iv_ms:.2f} ms")
        out.append(res)
        del qc, kc, qd, kd, vd, energy, lse, mask, row_ptr, col_idx, o
        torch.cuda.empty_cache()
    return out if len(out) > 1 else out[0]


def online_search(name, n_steps=8, search_steps=(0, 4)):
    """Online search on one workload (the search-and-reuse schedule of AdaSpa's
    method): at step 0 one dense pass (calib_block_energy_ws) gives the step's output,
    the LSE and the energies, then selection and the skip list; the following steps reuse the mask
    with sparse attention; at each later search step the output comes from the
    current mask and the energies from: the LSE cached at step 0 (the pages' reuse of
    the cache), the LSE that the step's own sparse pass writes over its kept blocks,
    or the step's own full LSE, which the one-pass sweep without V computes along with
    the energies ("own": the same mask as a search with a dense pass).  Each step's input is a fresh seeded
    draw of the workload.  Reports per-step times against dense attention, the output
    error against dense at every step, and the mask agreement of each later search
    with a search from the step's own dense LSE."""
    import torch

    import calibrated_block_sparse_calib_amd as cba
    from workloads import get_config, make_qkv

    cfg = get_config(name)
    B, H = cfg.block, cfg.heads
    taus = [cfg.tau] * H
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16).cuda()
    ev = lambda: torch.cuda.Event(enable_timing=True)
    kw = dict(block=B, n_prefix=cfg.n_prefix, grid=cfg.grid)
    t0 = time.perf_counter()
    inputs = []
    for st in range(n_steps):
        q, k, v = make_qkv(cfg, draw=st)
        inputs.append((dev(q[None]), dev(k[None]), dev(v[None])))
    log(f"online search {name}: {n_steps} steps of inputs in {time.perf_counter() - t0:.1f} s")
    o = torch.empty_like(inputs[0][0])
    od = torch.empty_like(o)
    lse_now = torch.empty(inputs[0][0].shape[:3], dtype=torch.float32, device="cuda")
    dense_ms, own_masks = [], {}
    for st, (q, k, v) in enumerate(inputs):  # the dense reference of every step
        c, d_ = ev(), ev()
        c.record()
        cba.dense_attn_fwd(q, k, v, block=B, o=od)
        d_.record()
        torch.cuda.synchronize()
        dense_ms.append(c.elapsed_time(d_))
        if st in search_steps and st > 0:
            e_own, _, _ = cba.calib_block_energy(q, k, None, **kw)
            own_masks[st] = cba.select_blocks_by_energy_heads(e_own, taus, cfg.rho, True, cfg.n_prefix_blocks)
            del e_own
    out = {"search_steps": list(search_steps), "tau": cfg.tau, "dense_ms": dense_ms}
    ws = torch.empty(cba.energy_workspace_bytes(o, B), dtype=torch.uint8, device="cuda")
    for source in ("cached", "sparse", "own"):
        lse = None
        row_ptr = col_idx = None
        steps = []
        for st, (q, k, v) in enumerate(inputs):
            a, b_ = ev(), ev()
            search = st in search_steps
            torch.cuda.synchronize()
            a.record()
            if st == 0:
                energy, lse, _ = cba.calib_block_energy_ws(q, k, v, o=o, workspace=ws, **kw)
            elif search and source == "sparse":
                cba.sparse_attn_fwd(q, k, v, row_ptr, col_idx, o=o, lse=lse_now, **kw)
                energy = cba.block_energy_from_lse(q, k, lse_now, **kw)
            elif search and source == "own":
                cba.sparse_attn_fwd(q, k, v, row_ptr, col_idx, o=o, **kw)
                energy, _, _ = cba.calib_block_energy_ws(q, k, workspace=ws, lse=lse_now, **kw)
            else:
                cba.sparse_attn_fwd(q, k, v, row_ptr, col_idx, o=o, **kw)
                if search:
                    energy = cba.block_energy_from_lse(q, k, lse, **kw)
            if search:
                mask = cba.select_blocks_by_energy_heads(energy, taus, cfg.rho, True, cfg.n_prefix_blocks)
                row_ptr, col_idx, _ = cba.build_block_csr(mask, with_order=False)
            b_.record()
            torch.cuda.synchronize()
            cba.dense_attn_fwd(q, k, v, block=B, o=od)
            rel = float((o.float() - od.float()).norm() / od.float().norm())
            rec = {"step": st, "kind": "search" if search else "reuse", "ms": a.elapsed_time(b_),
                   "rel_err_vs_dense": rel}
            if search:
                rec["density"] = float(mask.float().mean())
                if st in own_masks:
                    rec["mask_agreement_vs_own_lse"] = float((own_masks[st] == mask).float().mean())
            steps.append(rec)
            log(f"  [{source} LSE] step {st} {rec['kind']}: {rec['ms']:.1f} ms (dense {dense_ms[st]:.1f} ms), "
                f"rel err {rel:.2e}" + (f", density {rec['density']:.3f}" if search else "")
                + (f", mask agreement {rec['mask_agreement_vs_own_lse']:.4f}"
                   if "mask_agreement_vs_own_lse" in rec else ""))
        tot = sum(r["ms"] for r in steps)
        out[source + "_lse"] = {"steps": steps, "total_ms": tot, "speedup_vs_dense": sum(dense_ms) / tot}
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="wan14_720p")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle time for cpu_baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-rows", action="store_true", help="time only the step (profiling runs)")
    ap.add_argument("--order", choices=["lpt", "natural"], default="natural",
                    help="lpt: work_order from build_block_csr (longest rows first); natural: no work_order "
                         "(rows in head-major order)")
    ap.add_argument("--no-sweep", action="store_true", help="skip the density sweep")
    ap.add_argument("--calibrated", default="",
                    help="comma-separated calibrated workloads (wan13_480p, mochi, hunyuan, or 'all') to also time "
                         "end to end: calibration over all draws, selection, skip list, sparse attention")
    ap.add_argument("--tau-schedule", default="",
                    help="comma-separated energy thresholds, one per timestep bucket of the calibrated workloads "
                         "(early buckets first); default: each workload's own tau")
    ap.add_argument("--online-search", default="",
                    help="a calibrated workload (e.g. hunyuan) to run the online search-and-reuse schedule on "
                         "(8 steps, searches at steps 0 and 4)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="also run a plain device copy of this size (calibrates HBM byte counters)")
    ap.add_argument("--only", choices=["step", "dense"], default="step",
                    help="dense: time only dense_attn_fwd (warmup + steps launches) and print its rate "
                         "(profiling runs of the dense kernel)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch

    import calibrated_block_sparse_calib_amd as cba
    from workloads import get_config, make_qkv, random_block_mask, rep_head_flags

    cfg = get_config(args.workload)
    if cfg.mask_mode != "bernoulli":
        raise SystemExit("bench.py times the seeded-mask workloads; calibrated workloads are parity cases")
    cba.load_library()
    torch.cuda.set_device(0)
    t0 = time.perf_counter()
    q, k, v = make_qkv(cfg, draw=cfg.calib_draws)
    mask = random_block_mask(cfg)
    rep = rep_head_flags(cfg)
    log(f"generated {cfg.name} inputs in {time.perf_counter() - t0:.1f} s")
    dev = lambda x: torch.from_numpy(x)[None].to(torch.bfloat16).cuda()
    qd, kd, vd = dev(q), dev(k), dev(v)
    md = torch.from_numpy(mask).cuda()
    od = torch.empty_like(qd)
    B, nb, n = cfg.block, cfg.nb, cfg.seq_len
    row_ptr = torch.empty(cfg.heads * nb + 1, dtype=torch.int32, device="cuda")
    col_idx = torch.empty(cfg.heads * nb * nb, dtype=torch.int32, device="cuda")
    order = torch.empty(cfg.heads * nb, dtype=torch.int32, device="cuda")
    comp = (rows_per_block(cfg, False), rows_per_block(cfg, True))
    flops = kept_flops(mask, cfg, rep, comp)
    dense_flops = 4 * cfg.head_dim * n * n * cfg.heads
    density = float(mask.mean())
    lib = cba.load_library()
    desc = cba.make_desc(qd, B, cfg.n_prefix, cfg.grid)
    rep_arr = np.ascontiguousarray(rep)
    stream = torch.cuda.current_stream()
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    S = ctypes.c_void_p(stream.cuda_stream)
    wo = P(order) if args.order == "lpt" else None

    def csr():
        st = lib.build_block_csr(P(md), cfg.heads * nb, nb, P(row_ptr), P(col_idx), col_idx.numel(),
                                 P(order) if args.order == "lpt" else None, S)
        assert st == 0, st

    def sparse(fuse=1):
        st = lib.sparse_attn_fwd(ctypes.byref(desc), P(qd), P(kd), P(vd), P(row_ptr), P(col_idx), col_idx.numel(),
                                 wo, rep_arr.ctypes.data_as(ctypes.c_void_p), cfg.anchor_stride, fuse, P(od),
                                 None, S)
        assert st == 0, st

    ev = lambda: torch.cuda.Event(enable_timing=True)
    if args.only == "dense":
        for _ in range(args.warmup):
            cba.dense_attn_fwd(qd, kd, vd, block=B, o=od)
        torch.cuda.synchronize()
        marks = [(ev(), ev()) for _ in range(args.steps)]
        for a, b_ in marks:
            a.record(stream)
            cba.dense_attn_fwd(qd, kd, vd, block=B, o=od)
            b_.record(stream)
        torch.cuda.synchronize()
        d_ms = statistics.mean(a.elapsed_time(b_) for a, b_ in marks)
        print(json.dumps({"kernel": "dense_attn_fwd", "workload": cfg.name, "launches": args.steps, "ms": d_ms,
                          "tflops": dense_flops / d_ms / 1e9,
                          "frac_bf16_peak": dense_flops / d_ms / 1e9 / PEAK_BF16_TFLOPS}), flush=True)
        return
    for _ in range(args.warmup):
        csr()
        sparse()
    torch.cuda.synchronize()
    marks = [(ev(), ev(), ev()) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for a, b_, c in marks:
        a.record(stream)
        csr()
        b_.record(stream)
        sparse()
        c.record(stream)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t_start) * 1e3 / args.steps
    csr_ms = [a.elapsed_time(b_) for a, b_, _ in marks]
    sparse_ms = [b_.elapsed_time(c) for _, b_, c in marks]
    step_ms = [a.elapsed_time(c) for a, _, c in marks]
    sp_avg = statistics.mean(sparse_ms)
    value = flops / (wall_ms * 1e-3) / 1e12
    achieved = flops / (sp_avg * 1e-3) / 1e12
    log(f"step {wall_ms:.3f} ms wall, sparse_attn_fwd {sp_avg:.3f} ms avg ({achieved:.1f} TFLOP/s kept), "
        f"csr {statistics.mean(csr_ms):.3f} ms")
    got_o = od[0].float().cpu().numpy()
    if args.copy_probe_mib:
        src_t = torch.empty(args.copy_probe_mib << 20, dtype=torch.uint8, device="cuda")
        dst_t = torch.empty_like(src_t)
        for _ in range(2):
            dst_t.copy_(src_t)
        torch.cuda.synchronize()
        log(f"copy probe: {args.copy_probe_mib} MiB read + {args.copy_probe_mib} MiB written per copy, 2 copies")
        del src_t, dst_t

    rows = {}
    if not args.no_rows:
        def timeit(fn, reps=3):
            fn()
            torch.cuda.synchronize()
            ts = []
            for _ in range(reps):
                a, b_ = ev(), ev()
                a.record(stream)
                fn()
                b_.record(stream)
                torch.cuda.synchronize()
                ts.append(a.elapsed_time(b_))
            return statistics.median(ts)

        do = torch.empty_like(qd)
        dense_ms = timeit(lambda: cba.dense_attn_fwd(qd, kd, vd, block=B, o=do))
        rows["dense_attn_fwd"] = {"ms": dense_ms, "tflops": dense_flops / dense_ms / 1e9}
        rows["sparse_attn_fwd"] = {"ms": sp_avg, "tflops": achieved, "kept_flops": flops, "density": density}
        rows["build_block_csr"] = {"ms": statistics.mean(csr_ms),
                                   "algorithmic_bytes": int(mask.size + 4 * (row_ptr.numel() + 2 * int(mask.sum())
                                                                             + order.numel()))}
        rows["build_block_csr"]["gbs"] = rows["build_block_csr"]["algorithmic_bytes"] / rows["build_block_csr"]["ms"] / 1e6
        bc_ms = timeit(lambda: cba.rep_row_broadcast(od, rep, cfg.anchor_stride, block=B, n_prefix=cfg.n_prefix,
                                                     grid=cfg.grid))
        f_, h_, w_ = cfg.grid
        followers = int(rep.sum()) * f_ * (h_ - len(range(0, h_, cfg.anchor_stride))) * w_
        bc_bytes = 2 * followers * cfg.head_dim * 2
        rows["rep_row_broadcast"] = {"ms": bc_ms, "algorithmic_bytes": bc_bytes, "gbs": bc_bytes / bc_ms / 1e6}
        unfused_ms = timeit(lambda: sparse(fuse=0))
        rows["sparse_attn_fwd_unfused"] = {"ms": unfused_ms}
        # the same mask as block intervals (runs of kept blocks): build, then attention through the runs
        iv_ptr, ivs = cba.build_block_intervals(md)
        ivb_ms = timeit(lambda: cba.build_block_intervals(md))
        iv_o = torch.empty_like(qd)
        iv_ms = timeit(lambda: cba.sparse_attn_fwd_intervals(qd, kd, vd, iv_ptr, ivs, block=B, rep_heads=rep,
                                                             anchor_stride=cfg.anchor_stride, n_prefix=cfg.n_prefix,
                                                             grid=cfg.grid, o=iv_o))
        n_runs = int(iv_ptr[-1].item())
        rows["build_block_intervals"] = {"ms": ivb_ms, "runs": n_runs,
                                         "algorithmic_bytes": int(2 * mask.size + 4 * (iv_ptr.numel() + n_runs))}
        rows["sparse_attn_fwd_intervals"] = {"ms": iv_ms, "tflops": flops / iv_ms / 1e9,
                                             "same_output_as_csr": bool(torch.equal(iv_o, od))}
        rows["skip_list_bytes"] = skip_list_bytes(cfg.heads * nb, nb, int(mask.sum()), n_runs)
        del iv_o, iv_ptr, ivs
        energy = torch.empty((1, cfg.heads, nb, nb), dtype=torch.float32, device="cuda")
        lse = torch.empty((1, cfg.heads, n), dtype=torch.float32, device="cuda")
        eo = torch.empty_like(qd)
        en_ms = timeit(lambda: cba.calib_block_energy(qd, kd, vd, block=B, lse=lse, energy=energy, o=eo), reps=2)
        rows["calib_block_energy"] = {"ms": en_ms, "draws": 1, "tflops": 1.5 * dense_flops / en_ms / 1e9}
        # energies, LSE and O in one sweep over the keys, with its workspace; also without V
        ws = torch.empty(cba.energy_workspace_bytes(qd, B), dtype=torch.uint8, device="cuda")
        e1, l1, o1 = torch.empty_like(energy), torch.empty_like(lse), torch.empty_like(eo)
        e1_ms = timeit(lambda: cba.calib_block_energy_ws(qd, kd, vd, block=B, workspace=ws, lse=l1, energy=e1,
                                                         o=o1), reps=2)
        same_o = bool(torch.equal(o1, eo)) and bool(torch.equal(l1, lse))
        e1k_ms = timeit(lambda: cba.calib_block_energy_ws(qd, kd, block=B, workspace=ws, lse=l1, energy=e1), reps=2)
        rows["calib_block_energy_ws"] = {"ms": e1_ms, "draws": 1, "tflops": dense_flops / e1_ms / 1e9,
                                         "without_v_ms": e1k_ms,
                                         "without_v_tflops": 0.5 * dense_flops / e1k_ms / 1e9,
                                         "workspace_bytes": ws.numel(), "o_lse_same_as_two_sweep": same_o,
                                         "max_abs_diff_vs_two_sweep": float((e1 - energy).abs().max())}
        log(f"calib_block_energy_ws {e1_ms:.2f} ms ({dense_flops / e1_ms / 1e9:.0f} TFLOP/s; two sweeps "
            f"{en_ms:.2f} ms); without V {e1k_ms:.2f} ms; O and LSE identical {same_o}, max |dE| "
            f"{rows['calib_block_energy_ws']['max_abs_diff_vs_two_sweep']:.2e}")
        del ws, e1, l1, o1
        sel_ms = timeit(lambda: cba.select_blocks_by_energy(energy, 0.95, 0.5))
        rows["select_blocks_by_energy"] = {"ms": sel_ms, "draws": 1}
        # repetition detection on the same draw, from the LSE of the energy pass
        rs_head, rs_tok = cba.spatial_rep_similarity(qd, kd, lse, cfg.anchor_stride, n_prefix=cfg.n_prefix,
                                                     grid=cfg.grid)
        rs_ms = timeit(lambda: cba.spatial_rep_similarity(qd, kd, lse, cfg.anchor_stride, n_prefix=cfg.n_prefix,
                                                          grid=cfg.grid, token_cos=rs_tok, head_sim=rs_head))
        rs_flops = 2 * rep_rows_per_head(cfg) * n * cfg.head_dim * cfg.heads  # QK^T of the computed rows
        srh_ms = timeit(lambda: cba.select_rep_heads(rs_head, 0.9))
        hs = rs_head[0].cpu().numpy()
        rows["spatial_rep_similarity"] = {"ms": rs_ms, "tflops": rs_flops / rs_ms / 1e9,
                                          "rows_per_head": rep_rows_per_head(cfg), "draws": 1,
                                          "head_sim_min": float(hs.min()), "head_sim_max": float(hs.max()),
                                          "select_rep_heads_ms": srh_ms}
        log(f"spatial_rep_similarity {rs_ms:.2f} ms ({rs_flops / rs_ms / 1e9:.0f} TFLOP/s), head scores "
            f"{hs.min():.3f}..{hs.max():.3f}")
        rep_tok_host = rs_tok[0].cpu().numpy()
        del rs_tok
        del do, eo, energy
        if not args.no_sweep:
            rows["density_sweep"] = density_sweep(cfg, lib, desc, qd, kd, vd, od, row_ptr, col_idx, timeit, P, S)

    if args.calibrated:
        names = ["wan13_480p", "mochi", "hunyuan"] if args.calibrated == "all" else args.calibrated.split(",")
        del qd, kd, vd, od, md, row_ptr, col_idx, order
        torch.cuda.empty_cache()
        sched = [float(x) for x in args.tau_schedule.split(",")] if args.tau_schedule else None
        rows["calibrated"] = {name: calibrated_workload(name, tau_schedule=sched) for name in names}

    if args.online_search:
        rows["online_search"] = online_search(args.online_search)

    cpu, parity = None, None
    if not args.no_cpu_baseline:
        cpu, parity = cpu_baseline(cfg, q, k, v, mask, rep, got_o, args.cpu_budget, flops)
        log(f"cpu baseline {cpu['value']:.4f} TFLOP/s on {cpu['cores']} cores; sampled parity {parity}")
        if "spatial_rep_similarity" in rows:
            rows["spatial_rep_similarity"]["parity_sample"] = rep_sampled_parity(cfg, q, k, rep_tok_host)
            log(f"spatial_rep_similarity sampled parity {rows['spatial_rep_similarity']['parity_sample']}")

    traffic = traffic_from_profile()
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded token-grid generator; random-init, no model weights)",
        "config": {"workload": cfg.name, "heads": cfg.heads, "seq_len": n, "head_dim": cfg.head_dim,
                   "grid": list(cfg.grid), "block": B, "mask_density": round(density, 4),
                   "rep_heads": int(rep.sum()), "anchor_stride": cfg.anchor_stride,
                   "schedule": args.order},
        "pct_bf16_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "speedup_vs_dense": round(rows["dense_attn_fwd"]["ms"] / wall_ms, 3) if "dense_attn_fwd" in rows else None,
        "roofline": {"bound": "mfma", "kernel": "sparse_attn_fwd", "achieved": round(achieved, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic},
        "cpu_baseline": cpu,
        "parity_sample": parity,
        "rows": rows,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
