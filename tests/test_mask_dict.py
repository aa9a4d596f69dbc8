"""Host logic of the calibrated mask dictionary (CPU only): the timestep buckets,
the threshold schedule, and the .npz round trip of entries built from the
oracle's block intervals, including the refusal of damaged files."""
import json

import numpy as np
import pytest
import torch

import oracle
from calibrated_block_sparse_calib_amd.mask_dict import MaskDictionary, MaskEntry, bucket_of_step


def _entry(heads, nb, block, tau, seed, stride=1, rep=None):
    rng = np.random.default_rng(seed)
    mask = (rng.random((heads * nb, nb)) < 0.3).astype(np.uint8)
    ip, first, count, _ = oracle.build_intervals(mask)
    ivs = (first.astype(np.uint32) | (count.astype(np.uint32) << np.uint32(16))).view(np.int32)
    order = rng.permutation(heads * nb).astype(np.int32)
    rep = np.zeros(heads, np.uint8) if rep is None else np.asarray(rep, np.uint8)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32))
    return MaskEntry(heads, nb, block, tau, stride, t(ip), t(ivs), t(order), rep), mask


def test_bucket_of_step():
    # 50 steps in 3 buckets: steps 0-16, 17-33, 34-49
    got = [bucket_of_step(s, 50, 3) for s in range(50)]
    assert got[0] == 0 and got[16] == 0 and got[17] == 1 and got[33] == 1 and got[34] == 2 and got[49] == 2
    assert all(a <= b for a, b in zip(got, got[1:]))
    assert [bucket_of_step(s, 2, 3) for s in range(2)] == [0, 1]
    with pytest.raises(ValueError):
        bucket_of_step(5, 5, 3)


def test_schedule_is_stricter_early():
    MaskDictionary([0.98, 0.95, 0.92], block=128)
    with pytest.raises(ValueError):
        MaskDictionary([0.9, 0.95], block=128)
    MaskDictionary([0.9, 0.95], block=128, allow_rising=True)
    with pytest.raises(ValueError):
        MaskDictionary([1.2], block=128)


def test_round_trip(tmp_path):
    md = MaskDictionary([0.98, 0.95, 0.92], block=64)
    entries = {}
    for b in range(3):
        for l in range(2):
            e, _ = _entry(heads=3, nb=9, block=64, tau=md.tau_schedule[b], seed=10 * b + l, stride=4,
                          rep=[0, 1, 0] if l else None)
            md.put(b, l, e)
            entries[(b, l)] = e
    path = str(tmp_path / "masks.npz")
    md.save(path)
    md2 = MaskDictionary.load(path, device="cpu")
    assert md2.tau_schedule == md.tau_schedule and md2.block == 64 and md2.rho == 0.5
    assert md2.keys() == md.keys()
    for key, e in entries.items():
        e2 = md2.get(*key)
        assert (e2.heads, e2.nb, e2.block, e2.tau, e2.anchor_stride) == (3, 9, 64, e.tau, 4)
        for a, b in ((e.iv_ptr, e2.iv_ptr), (e.ivs, e2.ivs), (e.order, e2.order)):
            assert a.dtype == b.dtype and torch.equal(a, b)
        np.testing.assert_array_equal(e.rep_heads, e2.rep_heads)
    # the step -> bucket lookup picks the entry of its bucket
    assert md2.entry_for_step(0, 30, 1) is md2.get(0, 1)
    assert md2.entry_for_step(29, 30, 0) is md2.get(2, 0)


def test_kept_blocks_counts_the_runs():
    e, mask = _entry(heads=2, nb=11, block=32, tau=0.9, seed=3)
    assert e.kept_blocks() == int(mask.sum())


def _damage(path, out, key, fn):
    with np.load(path, allow_pickle=False) as z:
        arrays = {k: z[k] for k in z.files}
    arrays[key] = fn(arrays[key])
    with open(out, "wb") as f:
        np.savez(f, **arrays)


@pytest.mark.parametrize("key,fn", [
    ("b0_l0_iv_ptr", lambda a: a[:-1]),                                   # wrong length
    ("b0_l0_iv_ptr", lambda a: np.concatenate([a[:1], a[1:] + 1])),      # offsets past the runs
    ("b0_l0_ivs", lambda a: (a.view(np.uint32) + np.uint32(40)).view(np.int32)),  # runs past nb
    ("b0_l0_order", lambda a: np.zeros_like(a)),                          # not a permutation
    ("b0_l0_rep", lambda a: a.astype(np.int32)),                          # wrong dtype
    ("meta", lambda a: np.frombuffer(json.dumps({"format": 99}).encode(), np.uint8)),
])
def test_damaged_files_are_refused(tmp_path, key, fn):
    md = MaskDictionary([0.95], block=32)
    e, _ = _entry(heads=2, nb=7, block=32, tau=0.95, seed=1)
    md.put(0, 0, e)
    path, bad = str(tmp_path / "ok.npz"), str(tmp_path / "bad.npz")
    md.save(path)
    MaskDictionary.load(path, device="cpu")
    _damage(path, bad, key, fn)
    with pytest.raises((ValueError, KeyError)):
        MaskDictionary.load(bad, device="cpu")


def test_put_checks_bucket_and_block():
    md = MaskDictionary([0.95, 0.9], block=32)
    e, _ = _entry(heads=1, nb=4, block=32, tau=0.95, seed=2)
    with pytest.raises(KeyError):
        md.put(2, 0, e)
    e64, _ = _entry(heads=1, nb=4, block=64, tau=0.95, seed=2)
    with pytest.raises(ValueError):
        md.put(0, 0, e64)
