"""The calibrated mask dictionary of CalibAtt's offline stage and its use at
inference.

Calibration runs dense attention on a few inputs per (timestep, layer, head),
keeps per query block the fewest key blocks that reach an energy threshold, votes
over the inputs, and stores the result -- with the heads found to repeat across
the image rows of a frame -- in a dictionary keyed by (timestep, layer, head); the
threshold depends on the timestep and is stricter (keeps more energy) at early
denoising steps.  At inference each attention call loads the skip list of its
(timestep, layer) and computes only the listed blocks (CalibAtt, zh section 2.2A
"cross-prompt aggregation" and section 2.2B; de section 2A; fr sections 2B and 2C).

Here one entry covers one (timestep bucket, layer) and holds, for all its heads:

  * the skip list as block intervals (build_block_intervals: the compact form,
    a few runs per row for banded masks),
  * the processing order of the rows (order_heavy_rows_first),
  * the repetition flags and the anchor stride.

Every step runs in libcalibattn.so through the binding; this module only keeps
the entries and moves them to and from a .npz file.  The file is plain arrays
plus a JSON header and is read with numpy's allow_pickle=False, so loading it
executes nothing from the file.
"""
import json
from dataclasses import dataclass
from typing import Dict, Optional, Sequence, Tuple

import numpy as np
import torch

from . import api

FORMAT_VERSION = 1


@dataclass
class MaskEntry:
    """Skip lists of every head of one (timestep bucket, layer).

    iv_ptr: int32 [heads * nb + 1] run offsets per row (row = head * nb + qb).
    ivs: int32 [runs], each run packed as first | count << 16 (uint32 bits).
    order: int32 [heads * nb] processing order of the rows.
    rep_heads: uint8 [heads] on the host; 1 marks a spatial repetition head.
    """
    heads: int
    nb: int
    block: int
    tau: float
    anchor_stride: int
    iv_ptr: torch.Tensor
    ivs: torch.Tensor
    order: torch.Tensor
    rep_heads: np.ndarray

    @property
    def runs(self) -> int:
        return int(self.ivs.numel())

    def kept_blocks(self) -> int:
        """Number of kept (head, query block, key block) triples."""
        iv = self.ivs.cpu().numpy().view(np.uint32)
        return int((iv >> np.uint32(16)).astype(np.int64).sum())

    def to(self, device) -> "MaskEntry":
        return MaskEntry(self.heads, self.nb, self.block, self.tau, self.anchor_stride, self.iv_ptr.to(device),
                         self.ivs.to(device), self.order.to(device), self.rep_heads.copy())


def bucket_of_step(step: int, n_steps: int, n_buckets: int) -> int:
    """Timestep bucket of denoising step `step` (0 = first) of n_steps: n_buckets
    equal spans of consecutive steps, the first bucket holding the earliest steps."""
    if not (0 <= step < n_steps) or n_buckets < 1:
        raise ValueError("need 0 <= step < n_steps and n_buckets >= 1")
    return min(step * n_buckets // n_steps, n_buckets - 1)


class MaskDictionary:
    """Calibrated skip lists keyed by (timestep bucket, layer).

    tau_schedule: one energy threshold per timestep bucket, earliest first.  The
        pages ask for stricter thresholds at early steps; a schedule that rises
        later is refused unless allow_rising=True.
    rho: vote threshold (a block is kept when more than rho of the inputs keep it).
    """

    def __init__(self, tau_schedule: Sequence[float], *, block: int, rho: float = 0.5,
                 allow_rising: bool = False):
        taus = [float(t) for t in tau_schedule]
        if not taus or any(not (0.0 <= t <= 1.0) for t in taus):
            raise ValueError("tau_schedule needs one threshold in [0, 1] per bucket")
        if not allow_rising and any(b > a for a, b in zip(taus, taus[1:])):
            raise ValueError("tau_schedule must not rise from early to late buckets")
        self.tau_schedule = taus
        self.block = int(block)
        self.rho = float(rho)
        self.entries: Dict[Tuple[int, int], MaskEntry] = {}

    @property
    def n_buckets(self) -> int:
        return len(self.tau_schedule)

    def keys(self):
        return sorted(self.entries)

    def put(self, bucket: int, layer: int, entry: MaskEntry):
        if not 0 <= bucket < self.n_buckets:
            raise KeyError(f"bucket {bucket} outside the schedule")
        if entry.block != self.block:
            raise ValueError("entry block size differs from the dictionary's")
        self.entries[(int(bucket), int(layer))] = entry

    def get(self, bucket: int, layer: int) -> MaskEntry:
        return self.entries[(int(bucket), int(layer))]

    def entry_for_step(self, step: int, n_steps: int, layer: int) -> MaskEntry:
        return self.get(bucket_of_step(step, n_steps, self.n_buckets), layer)

    # ------------------------------------------------------------ calibration

    def calibrate(self, bucket: int, layer: int, q: torch.Tensor, k: torch.Tensor, *, n_prefix: int = 0,
                  grid=None, force_diag: bool = True, n_dense_prefix_blocks: Optional[int] = None,
                  anchor_stride: int = 1, rep_gamma: Optional[float] = None, heavy_factor: float = 2.0,
                  return_energy: bool = False):
        """Calibrate one entry from calibration inputs q, k [draws, heads, N, d]
        (bf16 or fp32, on the GPU) and store it under (bucket, layer).

        Energies: one pass over the keys per input (calib_block_energy_ws, one
        input at a time so the workspace is one input's); selection at the bucket's
        tau with the vote over the inputs; the skip list as runs; the heavy-rows-
        first order; with rep_gamma, the repetition flags of the heads whose mean
        follower cosine over the inputs is above rep_gamma (anchor_stride >= 2).
        Returns the entry (and, with return_energy, (entry, energy, mask))."""
        draws, heads, n, _ = q.shape
        block = self.block
        nb = api.n_blocks(n, block)
        tau = self.tau_schedule[bucket]
        if n_dense_prefix_blocks is None:
            n_dense_prefix_blocks = n_prefix // block
        energy = torch.empty((draws, heads, nb, nb), dtype=torch.float32, device=q.device)
        lse = torch.empty((draws, heads, n), dtype=torch.float32, device=q.device)
        ws = None
        if q.dtype == torch.bfloat16:
            ws = torch.empty(api.energy_workspace_bytes(q[:1], block), dtype=torch.uint8, device=q.device)
        for d in range(draws):
            api.calib_block_energy_ws(q[d:d + 1], k[d:d + 1], block=block, n_prefix=n_prefix, grid=grid,
                                      workspace=ws, lse=lse[d:d + 1], energy=energy[d:d + 1])
        del ws
        mask = api.select_blocks_by_energy(energy, tau, self.rho, force_diag, n_dense_prefix_blocks)
        iv_ptr, ivs = api.build_block_intervals(mask, exact=True)
        row_ptr, _, _ = api.build_block_csr(mask, count_only=True)
        order = api.order_heavy_rows_first(row_ptr, nb, heavy_factor)
        rep = np.zeros(heads, dtype=np.uint8)
        if rep_gamma is not None:
            head_sim, _ = api.spatial_rep_similarity(q, k, lse, anchor_stride, n_prefix=n_prefix, grid=grid)
            rep = api.select_rep_heads(head_sim, rep_gamma).cpu().numpy()
        entry = MaskEntry(heads, nb, block, tau, int(anchor_stride), iv_ptr, ivs[:int(iv_ptr[-1].item())], order,
                          rep)
        self.put(bucket, layer, entry)
        if return_energy:
            return entry, energy, mask
        return entry

    # ------------------------------------------------------------- inference

    def attention(self, q, k, v, *, step: int, n_steps: int, layer: int, n_prefix: int = 0, grid=None,
                  fuse_broadcast: bool = True, o: Optional[torch.Tensor] = None):
        """Sparse attention of one layer at one denoising step with the entry of its
        (timestep bucket, layer)."""
        e = self.entry_for_step(step, n_steps, layer)
        return self.attention_with(e, q, k, v, n_prefix=n_prefix, grid=grid, fuse_broadcast=fuse_broadcast, o=o)

    @staticmethod
    def attention_with(e: MaskEntry, q, k, v, *, n_prefix: int = 0, grid=None, fuse_broadcast: bool = True,
                       o: Optional[torch.Tensor] = None):
        if q.shape[1] != e.heads or api.n_blocks(q.shape[2], e.block) != e.nb:
            raise api.CalibAttnError("entry does not match the attention shape")
        rep = e.rep_heads if e.rep_heads.any() else None
        return api.sparse_attn_fwd_intervals(q, k, v, e.iv_ptr, e.ivs, block=e.block, work_order=e.order,
                                             rep_heads=rep, anchor_stride=e.anchor_stride,
                                             fuse_broadcast=fuse_broadcast, n_prefix=n_prefix, grid=grid, o=o)

    # ----------------------------------------------------------- persistence

    def save(self, path: str):
        """Write every entry to a .npz file (arrays plus a JSON header)."""
        meta = {"format": FORMAT_VERSION, "tau_schedule": self.tau_schedule, "block": self.block, "rho": self.rho,
                "entries": []}
        arrays = {}
        for (b, l) in self.keys():
            e = self.entries[(b, l)]
            key = f"b{b}_l{l}"
            meta["entries"].append({"bucket": b, "layer": l, "key": key, "heads": e.heads, "nb": e.nb,
                                    "tau": e.tau, "anchor_stride": e.anchor_stride})
            arrays[key + "_iv_ptr"] = e.iv_ptr.cpu().numpy().astype(np.int32)
            arrays[key + "_ivs"] = e.ivs.cpu().numpy().astype(np.int32)
            arrays[key + "_order"] = e.order.cpu().numpy().astype(np.int32)
            arrays[key + "_rep"] = np.asarray(e.rep_heads, dtype=np.uint8)
        arrays["meta"] = np.frombuffer(json.dumps(meta).encode(), dtype=np.uint8)
        with open(path, "wb") as f:
            np.savez(f, **arrays)

    @classmethod
    def load(cls, path: str, device="cuda") -> "MaskDictionary":
        """Read a file written by save(); the skip lists go to `device`."""
        with np.load(path, allow_pickle=False) as z:
            meta = json.loads(bytes(z["meta"]).decode())
            if meta.get("format") != FORMAT_VERSION:
                raise ValueError(f"unknown mask dictionary format {meta.get('format')}")
            md = cls(meta["tau_schedule"], block=meta["block"], rho=meta["rho"], allow_rising=True)
            for m in meta["entries"]:
                key, heads, nb = m["key"], int(m["heads"]), int(m["nb"])
                iv_ptr, ivs = z[key + "_iv_ptr"], z[key + "_ivs"]
                order, rep = z[key + "_order"], z[key + "_rep"]
                _validate(iv_ptr, ivs, order, rep, heads, nb, key)
                t = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(device)
                md.put(m["bucket"], m["layer"], MaskEntry(heads, nb, int(meta["block"]), float(m["tau"]),
                                                          int(m["anchor_stride"]), t(iv_ptr), t(ivs), t(order),
                                                          np.ascontiguousarray(rep, dtype=np.uint8)))
        return md


def _validate(iv_ptr, ivs, order, rep, heads, nb, key):
    """Structural checks of one stored entry, so a damaged file is refused before
    its offsets reach a kernel."""
    rows = heads * nb
    if iv_ptr.dtype != np.int32 or ivs.dtype != np.int32 or order.dtype != np.int32 or rep.dtype != np.uint8:
        raise ValueError(f"{key}: wrong array dtypes")
    if iv_ptr.shape != (rows + 1,) or order.shape != (rows,) or rep.shape != (heads,):
        raise ValueError(f"{key}: wrong array shapes")
    if iv_ptr[0] != 0 or np.any(np.diff(iv_ptr) < 0) or iv_ptr[-1] != ivs.shape[0]:
        raise ValueError(f"{key}: run offsets are not a valid prefix sum")
    u = ivs.view(np.uint32)
    first, count = u & np.uint32(0xFFFF), u >> np.uint32(16)
    if np.any(count < 1) or np.any(first.astype(np.int64) + count > nb):
        raise ValueError(f"{key}: runs outside the key blocks")
    if not np.array_equal(np.sort(order), np.arange(rows, dtype=np.int32)):
        raise ValueError(f"{key}: order is not a permutation of the rows")
