"""GPU parity on the method's degenerate cases, through the C ABI: empty and
one-token segments (an empty segment's pair is exactly (I, 0)); requests with
one entry and with none (the state passes through); the same cached pair
named several times in one request (a document repeated); seam windows on some
entries and not others; nonzero incoming states.  Expected values are the
oracle's own pairs composed entry by entry, with the seam windows run by its
token recurrence from the running state."""
import numpy as np
import pytest
import torch

import oracle
import workloads
import state_caching_segment_amd as hy
from gpu_harness import TOL, chain_inputs, dense_T

pytestmark = pytest.mark.gpu

LAWS = {"gdn": workloads.GDN_LAWS, "deltanet": workloads.GDN_LAWS, "kda": workloads.KDA_LAWS}
# slot token ranges over a 193-token stream (40 + 70 + 33 + 50): empty and one-token segments included
SLOTS = [(0, 40), (40, 40), (40, 110), (110, 111), (111, 111), (111, 143)]
# requests: one entry; none; one pair three times; empty and one-token pairs; seam starts per entry (-1: none)
LISTS = [[2], [], [0, 0, 0], [1, 4, 3, 5]]
SEAMS = [[-1], [], [-1, 150, -1], [150, -1, 10, 180]]


@pytest.mark.parametrize("fam,dtype,d", [("gdn", "bf16", 128), ("kda", "bf16", 64), ("gla", "bf16", 64),
                                         ("deltanet", "f32", 32), ("mamba2", "f32", 16), ("retnet", "bf16", 64),
                                         ("linear", "f32", 32)])
@pytest.mark.parametrize("mode", ["seq", "tree"])
def test_degenerate_segments_and_lists(fam, dtype, d, mode):
    C, w = 2, 8
    wl = workloads.make(f"deg_{fam}_{dtype}_{d}", config_id=94, family=fam, dtype=dtype, n_chains=C, d=d,
                        lens=[40, 70, 33, 50], w=w, laws=LAWS.get(fam, workloads.DIAG_LAWS),
                        gamma=workloads.retnet_gammas(C) if fam == "retnet" else None, device="cuda")
    dev = "cuda"
    L = hy.layout(fam, dtype, C, d)
    x = hy.tokens(wl.q, wl.k, wl.v, wl.g, wl.beta, wl.gamma)
    te = hy.hypic_t_elems(fam, d)
    n_slots = len(SLOTS)
    T = torch.full((n_slots, C, te), float("nan"), device=dev)
    S = torch.full((n_slots, C, d, d), float("nan"), device=dev)
    sb = torch.tensor([b for b, _ in SLOTS], dtype=torch.int64, device=dev)
    se = torch.tensor([e for _, e in SLOTS], dtype=torch.int64, device=dev)
    hy.hypic_segment_build(L, x, n_slots, sb, se, max(e - b for b, e in SLOTS), T, S)
    lo = torch.tensor(np.concatenate([[0], np.cumsum([len(l) for l in LISTS])]), dtype=torch.int32, device=dev)
    pid = torch.tensor([p for l in LISTS for p in l], dtype=torch.int32, device=dev)
    seam = torch.tensor([s for l in SEAMS for s in l], dtype=torch.int64, device=dev)
    n_req, n_ent = len(LISTS), int(pid.numel())
    rng = np.random.default_rng(94)
    init = rng.standard_normal((n_req, C, d, d)) * 0.5
    state = torch.tensor(init, dtype=torch.float32, device=dev)
    o = torch.full((n_ent, w, C, d), float("nan"), device=dev)
    tree = mode == "tree"
    nws = hy.hypic_workspace_bytes(L, hy.OP_COMPOSE_TREE, n_req, max(len(l) for l in LISTS), w) if tree else 0
    ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=dev) if tree else None
    hy.hypic_compose(L, hy.TREE if tree else hy.SEQ, n_req, max(len(l) for l in LISTS), lo, pid, n_slots, T, S, x,
                     seam, w, state, o, None, ws, nws)
    torch.cuda.synchronize()
    tol = TOL[dtype]
    for c in range(C):
        def inp(b, e):
            q, k, v, g, beta, gam = chain_inputs(wl, [c], b, e)
            return (q[0], k[0], v[0], None if g is None else g[0], None if beta is None else beta[0],
                    1.0 if gam is None else float(gam[0]))
        pairs = []
        for s, (b, e) in enumerate(SLOTS):
            q, k, v, g, beta, gam = inp(b, e)
            Tr, Sr = oracle.pair(fam, k, v, g, beta, gam) if e > b else (np.eye(d), np.zeros((d, d)))
            pairs.append((Tr, Sr))
            Tg = dense_T(T[s, c].double().cpu().numpy(), d)
            Sg = S[s, c].double().cpu().numpy()
            if e == b:   # an empty segment: exactly the identity pair
                assert np.array_equal(Tg, np.eye(d)) and not Sg.any(), (fam, s)
            else:
                assert oracle.rel_fro(Tg, Tr) <= tol and oracle.rel_fro(Sg, Sr) <= tol, (fam, s)
        e0 = 0
        for r, (lst, sms) in enumerate(zip(LISTS, SEAMS)):
            st = init[r, c].copy()
            for j, (p, s0) in enumerate(zip(lst, sms)):
                if s0 >= 0:
                    q, k, v, g, beta, gam = inp(s0, s0 + w)
                    st, O = oracle.run(fam, q, k, v, g, beta, gam, S0=st)
                    Og = o[e0 + j, :, c].double().cpu().numpy()
                    assert oracle.rel_fro(Og, O) <= tol, (fam, mode, r, j, "seam outputs")
                st = oracle.compose(pairs[p][0], pairs[p][1], st)
            got = state[r, c].double().cpu().numpy()
            assert oracle.rel_fro(got, st) <= tol, (fam, mode, r, oracle.rel_fro(got, st))
            e0 += len(lst)
