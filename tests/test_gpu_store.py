"""Cache misses forced from the host (codernav.top, segment parallelism:
misses are inevitable as the corpus changes and rarely used documents are
evicted): pairs kept in a pool indexed by the pair store, segments evicted
and rebuilt, a launch failure injected during a rebuild; every compose must
give bitwise the same states and seam outputs as the run where every pair
was present, and match the oracle."""
import os

import numpy as np
import pytest
import torch

import workloads
import state_caching_segment_amd as hy
from gpu_harness import TOL, oracle_request
from state_caching_segment_amd.plan import request_plan

pytestmark = pytest.mark.gpu


class Pool:
    """Pairs of one layer in a device pool of n_slots, indexed by content key."""

    def __init__(self, wl, plan, n_slots):
        self.wl, self.plan = wl, plan
        d, C = wl.dk, wl.n_chains
        self.L = hy.layout(wl.family, wl.dtype, C, d)
        self.x = hy.tokens(wl.q, wl.k, wl.v, wl.g, wl.beta, wl.gamma)
        self.T = torch.full((n_slots, C, hy.hypic_t_elems(wl.family, d)), float("nan"), device="cuda")
        self.S = torch.full((n_slots, C, d, d), float("nan"), device="cuda")
        self.store = hy.Store(n_slots)
        # content key of each body: its tokens' keys and values (token ids in a real system)
        self.keys = [hy.hypic_content_key(np.concatenate([
            wl.k[int(b):int(e)].float().cpu().numpy().ravel(), wl.v[int(b):int(e)].float().cpu().numpy().ravel()]))
            for b, e in zip(plan.seg_begin, plan.seg_end)]
        self.built = 0

    def request(self, r):
        """Acquire the slots of request r's bodies, build the misses into them,
        compose with seams; -> (state, seam outputs)."""
        p, wl = self.plan, self.wl
        e0, e1 = int(p.list_off[r]), int(p.list_off[r + 1])
        segs = [int(p.pair_id[e]) for e in range(e0, e1)]
        slots, miss = self.store.acquire([self.keys[s] for s in segs])
        todo = [(s, int(sl)) for s, sl, m in zip(segs, slots, miss) if m]
        if todo:
            sb = torch.tensor([int(p.seg_begin[s]) for s, _ in todo], dtype=torch.int64, device="cuda")
            se = torch.tensor([int(p.seg_end[s]) for s, _ in todo], dtype=torch.int64, device="cuda")
            tT = torch.empty(len(todo), *self.T.shape[1:], device="cuda")
            tS = torch.empty(len(todo), *self.S.shape[1:], device="cuda")
            hy.hypic_segment_build(self.L, self.x, len(todo), sb, se, int((se - sb).max()), tT, tS)
            idx = torch.tensor([sl for _, sl in todo], dtype=torch.long, device="cuda")
            self.T.index_copy_(0, idx, tT)
            self.S.index_copy_(0, idx, tS)
            self.built += len(todo)
        n = e1 - e0
        C, d, w = wl.n_chains, wl.dk, wl.w
        state = torch.zeros(1, C, d, d, device="cuda")
        o = torch.zeros(n, w, C, d, device="cuda")
        hy.hypic_compose(self.L, hy.SEQ, 1, n, torch.tensor([0, n], dtype=torch.int32, device="cuda"),
                         torch.from_numpy(slots).cuda(), self.T.shape[0], self.T, self.S, self.x,
                         torch.from_numpy(p.seam_begin[e0:e1]).cuda(), w, state, o)
        torch.cuda.synchronize()
        return state, o, int(miss.sum())


def _workload():
    # two requests over the same document collection: request 1 reuses three
    # of request 0's segments (same tokens at other positions) and adds two
    lens0 = [90, 70, 75, 110, 66, 81]
    wl = workloads.make("store", config_id=64, family="gdn", dtype="bf16", n_chains=3, d=64,
                        lens=[lens0, [70, 75, 66, 120, 95]], w=8, laws=workloads.GDN_LAWS, device="cuda")
    b0, b1 = wl.requests
    # copy request 0's segments 1, 2, 4 into request 1's first three segments
    for dst, src in ((0, 1), (1, 2), (2, 4)):
        for t in (wl.q, wl.k, wl.v, wl.g, wl.beta):
            t[int(b1[dst]):int(b1[dst + 1])] = t[int(b0[src]):int(b0[src + 1])]
    return wl


def test_forced_miss_evict_rebuild_bitwise():
    wl = _workload()
    plan = request_plan(wl.requests, wl.w)
    ref = oracle_request(wl, list(range(wl.n_chains)))
    # every pair present: a pool as large as the collection
    big = Pool(wl, plan, 16)
    st0, o0, m0 = big.request(0)
    st1, o1, m1 = big.request(1)
    assert m0 == 6
    # request 1's first body starts at its segment start (no seam): it is not
    # the same body as request 0's segment 1 (seam cut), so it misses; its
    # other two shared bodies hit
    assert m1 == 3, m1
    for r, (st, o) in enumerate(((st0, o0), (st1, o1))):
        for c in range(wl.n_chains):
            a = st[0, c].double().cpu().numpy()
            assert np.linalg.norm(a - ref[r]["state"][c]) / np.linalg.norm(ref[r]["state"][c]) <= TOL["bf16"]
    # evict three bodies, then compose again: they are rebuilt into free slots
    for s in (1, 3, 5):
        assert big.store.evict(big.keys[s])
    built = big.built
    st0b, o0b, m = big.request(0)
    assert m == 3 and big.built == built + 3
    assert torch.equal(st0b, st0) and torch.equal(o0b, o0)
    # a pool too small for both requests: LFU eviction between them, every
    # compose still bitwise the all-hit result
    small = Pool(wl, plan, 6)
    for r, (st, o) in ((0, (st0, o0)), (1, (st1, o1)), (0, (st0, o0)), (1, (st1, o1))):
        stx, ox, _ = small.request(r)
        assert torch.equal(stx, st) and torch.equal(ox, o), r
    stats = small.store.stats()
    assert stats["evictions"] > 0 and stats["hits"] > 0, stats


def test_injected_launch_failure_during_rebuild():
    """A rebuild whose launch fails (HYPIC_FAULT_INJECT=build) raises
    HYPIC_E_DEVICE; dropping the entries it claimed and retrying gives the
    all-hit result bitwise."""
    wl = _workload()
    plan = request_plan(wl.requests, wl.w)
    pool = Pool(wl, plan, 16)
    st0, o0, _ = pool.request(0)
    for s in (2, 4):
        pool.store.evict(pool.keys[s])
    os.environ["HYPIC_FAULT_INJECT"] = "build"
    try:
        with pytest.raises(hy.HypicError) as e:
            pool.request(0)
        assert e.value.status == -4
    finally:
        del os.environ["HYPIC_FAULT_INJECT"]
    # the failed call's misses hold slots whose pairs were never built
    for s in (2, 4):
        assert pool.store.evict(pool.keys[s])
    st, o, m = pool.request(0)
    assert m == 2 and torch.equal(st, st0) and torch.equal(o, o0)
