"""Host-side bookkeeping for one or more requests: which token ranges are
cached, where the seam windows start, and the per-request entry lists that
hypic_compose walks.

Seam placement (HYPIC, codernav.top article, section on full-attention
layers and seam windows): every internal segment, i.e. every segment after a
request's first, keeps its first w tokens out of the cache; they are
recomputed at reuse.  So a request with boundaries b_0 < b_1 < ... < b_m has
cached bodies [b_0, b_1) and [b_j + w, b_{j+1}) for j >= 1, and seam windows
[b_j, b_j + w) for j >= 1.  A segment not longer than w is rejected.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import List, Sequence

import numpy as np


@dataclass
class Plan:
    seg_begin: np.ndarray   # [n_slots] int64, cached body start (global token index)
    seg_end: np.ndarray     # [n_slots] int64
    list_off: np.ndarray    # [n_req + 1] int32
    pair_id: np.ndarray     # [n_entries] int32, pair slot of each entry
    seam_begin: np.ndarray  # [n_entries] int64, first seam token, -1 for a request's first entry
    w: int
    seg_index: np.ndarray   # [n_slots] int64, the segment (numbered in request order) each slot holds

    @property
    def n_slots(self) -> int:
        return len(self.seg_begin)

    @property
    def n_req(self) -> int:
        return len(self.list_off) - 1

    @property
    def max_seg_len(self) -> int:
        return int((self.seg_end - self.seg_begin).max()) if self.n_slots else 0

    @property
    def max_list_len(self) -> int:
        return int(np.diff(self.list_off).max()) if self.n_req else 0


def request_plan(requests: Sequence[np.ndarray], w: int, slot_order: str = "request") -> Plan:
    """One pair slot per segment of every request.

    slot_order "request": slots in request order.  "longest_first": slots
    numbered by decreasing body length (ties in request order).  The build
    launches one workgroup per (slot, chain) in slot order and the GPU hands
    them out in that order, so longest-first is the longest-processing-time
    rule: the long segments start first and the short ones fill in behind
    them, which evens out the work per compute unit.  Entries reach their
    slots through pair_id either way, so results do not depend on the order."""
    if slot_order not in ("request", "longest_first"):
        raise ValueError(f"unknown slot order {slot_order!r}")
    sb, se, po, pid, seam = [], [], [0], [], []
    for b in requests:
        b = np.asarray(b, dtype=np.int64)
        m = len(b) - 1
        for j in range(m):
            start, end = int(b[j]), int(b[j + 1])
            if j > 0 and end - start <= w:
                raise ValueError(f"segment {j} of length {end - start} is not longer than the seam width {w}")
            body = start + (w if j > 0 else 0)
            pid.append(len(sb))
            sb.append(body)
            se.append(end)
            seam.append(start if (j > 0 and w > 0) else -1)
        po.append(len(pid))
    sb, se, pid = np.asarray(sb, np.int64), np.asarray(se, np.int64), np.asarray(pid, np.int32)
    order = np.arange(len(sb), dtype=np.int64)
    if slot_order == "longest_first" and len(sb):
        order = np.argsort(-(se - sb), kind="stable")  # new slot i holds segment order[i]
        rank = np.empty_like(order)
        rank[order] = np.arange(len(order))
        sb, se, pid = sb[order], se[order], rank[pid].astype(np.int32)
    return Plan(sb, se, np.asarray(po, np.int32), pid, np.asarray(seam, np.int64), w, order)
