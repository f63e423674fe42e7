"""GPU checks of the C ABI's options: the state after every entry
(d_prefix_states), resuming a compose from a saved state in either mode, the
HYPIC_VALIDATE read-back, the HYPIC_DEBUG synchronous launches, and
composition time that does not grow with segment length (codernav.top,
section on linear layers: merging a cached segment is a constant-time step)."""
import os

import numpy as np
import pytest
import torch

import oracle
import workloads
import state_caching_segment_amd as hy
from gpu_harness import TOL, chain_inputs, gpu_request, oracle_request
from state_caching_segment_amd.plan import request_plan

pytestmark = pytest.mark.gpu

LAWS = {"gdn": workloads.GDN_LAWS, "deltanet": workloads.GDN_LAWS, "kda": workloads.KDA_LAWS}


def _wl(fam, dtype, d, lens, n_chains=3, cid=88, w=8):
    return workloads.make(f"{fam}_{dtype}_{d}", config_id=cid, family=fam, dtype=dtype, n_chains=n_chains, d=d,
                          lens=lens, w=w, laws=LAWS.get(fam, workloads.DIAG_LAWS),
                          gamma=workloads.retnet_gammas(n_chains) if fam == "retnet" else None, device="cuda")


def _sequential_state(wl, chain, t0, t1):
    """The oracle's token-by-token recurrence over [t0, t1) from zero."""
    q, k, v, g, beta, gam = chain_inputs(wl, [chain], t0, t1)
    S, _ = oracle.run(wl.family, q[0], k[0], v[0], None if g is None else g[0], None if beta is None else beta[0],
                      1.0 if gam is None else gam[0])
    return S


@pytest.mark.parametrize("fam,dtype,d", [("gdn", "bf16", 128), ("kda", "bf16", 128), ("deltanet", "f32", 16),
                                         ("gla", "bf16", 64), ("retnet", "f32", 64), ("gdn", "bf16", 32)])
@pytest.mark.parametrize("mode", ["seq", "tree"])
def test_prefix_states(fam, dtype, d, mode):
    """Every entry's state (its seam window and pair applied) equals the
    sequential recurrence over the request's tokens up to that entry's end."""
    lens = [[70, 40, 33, 90, 25, 61, 44, 30, 52, 19, 27], [130, 60, 45], [50], [40, 31, 29, 66, 73, 20, 18]]
    wl = _wl(fam, dtype, d, lens)
    m = hy.TREE if mode == "tree" else hy.SEQ
    gpu = gpu_request(wl, mode=m, prefix=True)
    plain = gpu_request(wl, mode=m)
    plan = gpu["plan"]
    pre = gpu["prefix"].double().cpu().numpy()
    assert torch.isfinite(gpu["prefix"]).all()
    worst = 0.0
    for r, b in enumerate(wl.requests):
        e0 = int(plan.list_off[r])
        for j in range(len(b) - 1):
            for c in range(wl.n_chains):
                ref = _sequential_state(wl, c, int(b[0]), int(b[j + 1]))
                worst = max(worst, oracle.rel_fro(pre[e0 + j, c], ref))
        # the last entry's state is the request's final state (in tree mode
        # the final state comes from the scan, the entry's from the second
        # pass: equal to rounding)
        last, fin = gpu["prefix"][int(plan.list_off[r + 1]) - 1], gpu["state"][r]
        if mode == "seq":
            assert torch.equal(last, fin)
        else:
            assert float((last - fin).double().norm() / fin.double().norm()) <= TOL[dtype]
    print(f"prefix {fam} {dtype} {d} {mode}: {worst:.2e}", flush=True)
    assert worst <= TOL[dtype]
    # the option changes nothing else: seam outputs within tolerance of the
    # plain call (tree mode writes them from its second pass), final states
    # equal in sequential mode
    if mode == "seq":
        assert torch.equal(gpu["state"], plain["state"]) and torch.equal(gpu["O"], plain["O"])
    else:
        for key in ("state", "O"):
            a, p = gpu[key].double(), plain[key].double()
            assert float((a - p).norm() / p.norm()) <= TOL[dtype], key


@pytest.mark.parametrize("fam,d", [("gdn", 128), ("gla", 64), ("kda", 128)])
@pytest.mark.parametrize("mode", ["seq", "tree"])
def test_resume_from_saved_state(fam, d, mode):
    """compose(first entries) then compose(rest) from the saved state equals
    the oracle's whole request: the second call starts from a nonzero state,
    which the tree's scan and seam fix-up take as their starting point."""
    wl = _wl(fam, "bf16", d, [100, 90, 75, 140, 66, 81, 95], n_chains=4, cid=89)
    full = gpu_request(wl)
    plan = full["plan"]
    dev = "cuda"
    L = hy.layout(fam, "bf16", wl.n_chains, d)
    x = hy.tokens(wl.q, wl.k, wl.v, wl.g, wl.beta, wl.gamma)
    state = torch.zeros(1, wl.n_chains, d, d, device=dev)
    o = torch.zeros(len(plan.pair_id), wl.w, wl.n_chains, d, device=dev)
    pid = torch.from_numpy(plan.pair_id).to(dev)
    seam = torch.from_numpy(plan.seam_begin).to(dev)
    m = hy.TREE if mode == "tree" else hy.SEQ
    for lo in ([0, 2], [2, 7]):
        n = lo[1] - lo[0]
        lst = torch.tensor([0, n], dtype=torch.int32, device=dev)
        ws, nws = None, 0
        if m == hy.TREE:
            nws = hy.hypic_workspace_bytes(L, hy.OP_COMPOSE_TREE, 1, n, wl.w)
            ws = torch.empty(nws, dtype=torch.uint8, device=dev)
        hy.hypic_compose(L, m, 1, n, lst, pid[lo[0]:], plan.n_slots, full["T"], full["S"], x, seam[lo[0]:], wl.w,
                         state, o[lo[0]:], ws=ws, ws_bytes=nws)
    torch.cuda.synchronize()
    if m == hy.SEQ:
        assert torch.equal(state, full["state"])
        assert torch.equal(o[1:], full["O"][1:])
    ref = oracle_request(wl, list(range(wl.n_chains)))[0]
    st = state.double().cpu().numpy()
    oo = o.double().cpu().numpy()
    for c in range(wl.n_chains):
        assert oracle.rel_fro(st[0, c], ref["state"][c]) <= TOL["bf16"]
        for j in range(1, len(plan.pair_id)):
            assert oracle.rel_fro(oo[j, :, c], ref["O"][j, :, c]) <= TOL["bf16"], (c, j)


def test_validate_reads_back_offsets():
    """HYPIC_VALIDATE=1: bad device-resident offsets and slot ids are refused
    with HYPIC_E_INVALID before anything is launched; good ones give the same
    results as without the check."""
    wl = _wl("gdn", "bf16", 64, [70, 40, 33, 90], n_chains=2, cid=90)
    plan = request_plan(wl.requests, wl.w)
    dev = "cuda"
    L = hy.layout("gdn", "bf16", wl.n_chains, 64)
    x = hy.tokens(wl.q, wl.k, wl.v, wl.g, wl.beta)
    T = torch.full((plan.n_slots, 2, 64 * 64), float("nan"), device=dev)
    S = torch.full((plan.n_slots, 2, 64, 64), float("nan"), device=dev)
    sb = torch.from_numpy(plan.seg_begin).to(dev)
    se = torch.from_numpy(plan.seg_end).to(dev)
    lo = torch.from_numpy(plan.list_off).to(dev)
    pid = torch.from_numpy(plan.pair_id).to(dev)
    seam = torch.from_numpy(plan.seam_begin).to(dev)
    state = torch.zeros(1, 2, 64, 64, device=dev)
    o = torch.zeros(len(plan.pair_id), wl.w, 2, 64, device=dev)
    os.environ["HYPIC_VALIDATE"] = "1"
    try:
        def bad(fn, *args, **kw):
            with pytest.raises(hy.HypicError) as e:
                fn(*args, **kw)
            assert e.value.status == -1 and "HYPIC_VALIDATE" in str(e.value), str(e.value)

        bad(hy.hypic_segment_build, L, x, plan.n_slots, se, sb, plan.max_seg_len, T, S)       # reversed ranges
        bad(hy.hypic_segment_build, L, x, plan.n_slots, sb, se, plan.max_seg_len - 1, T, S)   # longer than max
        assert torch.isnan(T).all(), "a refused build enqueued work"
        hy.hypic_segment_build(L, x, plan.n_slots, sb, se, plan.max_seg_len, T, S)
        bad_pid = pid.clone()
        bad_pid[2] = plan.n_slots
        bad(hy.hypic_compose, L, hy.SEQ, 1, plan.max_list_len, lo, bad_pid, plan.n_slots, T, S, x, seam, wl.w,
            state, o)
        bad(hy.hypic_compose, L, hy.SEQ, 1, plan.max_list_len - 1, lo, pid, plan.n_slots, T, S, x, seam, wl.w,
            state, o)
        bad_seam = seam.clone()
        bad_seam[1] = -5
        bad(hy.hypic_compose, L, hy.SEQ, 1, plan.max_list_len, lo, pid, plan.n_slots, T, S, x, bad_seam, wl.w,
            state, o)
        bad(hy.hypic_seam_advance, L, x, 2, torch.tensor([3, -1], dtype=torch.int64, device=dev), wl.w,
            torch.zeros(2, 2, 64, 64, device=dev), torch.zeros(2, wl.w, 2, 64, device=dev))
        assert torch.count_nonzero(state) == 0 and torch.count_nonzero(o) == 0, "a refused call enqueued work"
        hy.hypic_compose(L, hy.SEQ, 1, plan.max_list_len, lo, pid, plan.n_slots, T, S, x, seam, wl.w, state, o)
        torch.cuda.synchronize()
    finally:
        del os.environ["HYPIC_VALIDATE"]
    ref = gpu_request(wl)
    assert torch.equal(T, ref["T"]) and torch.equal(S, ref["S"])
    assert torch.equal(state, ref["state"]) and torch.equal(o[1:], ref["O"][1:])


def test_compose_time_independent_of_segment_length():
    """The compose reads one cached pair per segment whatever the segment's
    length: two requests with the same number of segments, of 520 and of
    8200 tokens each, compose in the same time (medians within 20%)."""
    n_chains, d, m = 256, 128, 12
    times = {}
    for seg in (520, 8200):
        wl = workloads.make(f"const_{seg}", config_id=91, family="gdn", dtype="bf16", n_chains=n_chains, d=d,
                            lens=[seg] * m, w=8, laws=workloads.GDN_LAWS, device="cuda")
        plan = request_plan(wl.requests, wl.w)
        dev = "cuda"
        L = hy.layout("gdn", "bf16", n_chains, d)
        x = hy.tokens(wl.q, wl.k, wl.v, wl.g, wl.beta)
        T = torch.empty(plan.n_slots, n_chains, d * d, device=dev)
        S = torch.empty(plan.n_slots, n_chains, d, d, device=dev)
        hy.hypic_segment_build(L, x, plan.n_slots, torch.from_numpy(plan.seg_begin).to(dev),
                               torch.from_numpy(plan.seg_end).to(dev), plan.max_seg_len, T, S)
        lo = torch.from_numpy(plan.list_off).to(dev)
        pid = torch.from_numpy(plan.pair_id).to(dev)
        seam = torch.from_numpy(plan.seam_begin).to(dev)
        state = torch.zeros(1, n_chains, d, d, device=dev)
        o = torch.zeros(m, wl.w, n_chains, d, device=dev)
        ms = []
        for it in range(25):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            hy.hypic_compose(L, hy.SEQ, 1, m, lo, pid, plan.n_slots, T, S, x, seam, wl.w, state, o)
            b.record()
            torch.cuda.synchronize()
            if it >= 5:
                ms.append(a.elapsed_time(b))
        times[seg] = float(np.median(ms))
        del wl, T, S, x
        torch.cuda.empty_cache()
    print("compose ms by segment length:", times, flush=True)
    assert 1 / 1.2 <= times[8200] / times[520] <= 1.2, times


@pytest.mark.parametrize("fam,dtype,d,mode", [("gdn", "bf16", 128, "seq"), ("kda", "bf16", 64, "tree"),
                                              ("gla", "bf16", 64, "tree")])
def test_debug_synchronous_launches_change_nothing(fam, dtype, d, mode):
    """HYPIC_DEBUG=1 synchronizes after every launch: pairs, states and seam
    outputs are bitwise those of the asynchronous run, and every call still
    returns success."""
    wl = _wl(fam, dtype, d, [[70, 150, 64, 9, 90]], cid=91)
    m = hy.TREE if mode == "tree" else hy.SEQ
    ref = gpu_request(wl, mode=m)
    os.environ["HYPIC_DEBUG"] = "1"
    try:
        dbg = gpu_request(wl, mode=m)
    finally:
        del os.environ["HYPIC_DEBUG"]
    for key in ("T", "S", "state", "O"):
        assert torch.equal(ref[key], dbg[key]), key
