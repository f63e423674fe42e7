"""Runs one workload through the HIP library (via the C ABI binding) and
through the fp64 oracle, and compares them object by object.

Error metric: relative Frobenius norm per object (each cached T and S per
(segment, chain), each final state per (request, chain), each w x dv seam
output block per (entry, chain)); the max over objects is held to the
tolerance.  A reference T below 2^-100 in norm is checked instead for
||T_gpu|| <= 2^-100 sqrt(dk) (fp32 cannot hold it with headroom).
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
import state_caching_segment_amd as hy
from state_caching_segment_amd.plan import request_plan

FLOOR = 2.0 ** -100
TOL = {"f32": 1e-4, "bf16": 5e-3}


def gpu_request(wl, w=None, stream=None, mode=None, slot_order="request", prefix=False):
    """Build every segment body's pair, then compose each request with its seams
    (sequential compose, or the tree scan with mode=hy.TREE); with prefix=True
    the state after every entry is returned too."""
    mode = hy.SEQ if mode is None else mode
    w = wl.w if w is None else w
    plan = request_plan(wl.requests, w, slot_order=slot_order)
    dev = wl.k.device
    L = hy.layout(wl.family, wl.dtype, wl.n_chains, wl.dk)
    x = hy.tokens(wl.q, wl.k, wl.v, wl.g, wl.beta, wl.gamma)
    te = hy.hypic_t_elems(wl.family, wl.dk)
    T = torch.full((plan.n_slots, wl.n_chains, te), float("nan"), device=dev)
    S = torch.full((plan.n_slots, wl.n_chains, wl.dk, wl.dv), float("nan"), device=dev)
    sb = torch.from_numpy(plan.seg_begin).to(dev)
    se = torch.from_numpy(plan.seg_end).to(dev)
    hy.hypic_segment_build(L, x, plan.n_slots, sb, se, plan.max_seg_len, T, S, stream=stream)
    state = torch.zeros(plan.n_req, wl.n_chains, wl.dk, wl.dv, device=dev)
    o = torch.zeros(len(plan.pair_id), max(w, 1), wl.n_chains, wl.dv, device=dev)
    lo = torch.from_numpy(plan.list_off).to(dev)
    pid = torch.from_numpy(plan.pair_id).to(dev)
    seam = torch.from_numpy(plan.seam_begin).to(dev)
    ws, nws = None, 0
    if mode == hy.TREE:
        nws = hy.hypic_workspace_bytes(L, hy.OP_COMPOSE_TREE, plan.n_req, plan.max_list_len, w)
        ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=dev)
    pre = (torch.full((len(plan.pair_id), wl.n_chains, wl.dk, wl.dv), float("nan"), device=dev) if prefix
           else None)
    hy.hypic_compose(L, mode, plan.n_req, plan.max_list_len, lo, pid, plan.n_slots, T, S,
                     x if w > 0 else None, seam, w, state, o, pre, ws, nws, stream=stream)
    torch.cuda.synchronize()
    return {"plan": plan, "T": T, "S": S, "state": state, "O": o, "prefix": pre}


def chain_inputs(wl, chains, t0, t1):
    """fp64 chain-major copies of the token range [t0, t1) for the given chains."""
    def cm(x):
        if x is None:
            return None
        y = x[t0:t1][:, chains].double().cpu().numpy()
        return np.ascontiguousarray(np.moveaxis(y, 1, 0))
    gam = None if wl.gamma is None else wl.gamma[chains].double().cpu().numpy()
    return cm(wl.q), cm(wl.k), cm(wl.v), cm(wl.g), cm(wl.beta), gam


def oracle_request(wl, chains, w=None, nthreads=0, reqs=None, parallel=1):
    """The oracle's reuse path for every request (or the requests listed in
    reqs), on the given chains; `parallel` requests at a time (the oracle's
    calls release the interpreter lock)."""
    w = wl.w if w is None else w
    rs = list(range(len(wl.requests)) if reqs is None else reqs)
    inputs = []
    for r in rs:
        b = wl.requests[r]
        inputs.append((b, chain_inputs(wl, chains, int(b[0]), int(b[-1]))))

    def one(item):
        b, (q, k, v, g, beta, gam) = item
        return oracle.request_batch(wl.family, b - b[0], w, q, k, v, g, beta, gam, nthreads=nthreads)
    if parallel <= 1:
        return [one(it) for it in inputs]
    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(max_workers=parallel) as ex:
        return list(ex.map(one, inputs))


def dense_T(Tc: np.ndarray, dk: int) -> np.ndarray:
    """Expand a stored T (scalar, diagonal or dense) to dk x dk."""
    Tc = np.asarray(Tc, dtype=np.float64).reshape(-1)
    if Tc.size == 1:
        return Tc[0] * np.eye(dk)
    if Tc.size == dk:
        return np.diag(Tc)
    return Tc.reshape(dk, dk)


def _rel(x, ref):
    # a non-finite value (an unwritten NaN output, an overflow) is an infinite
    # error: max() over objects would silently pass over a NaN
    if not np.isfinite(x).all():
        return float("inf")
    nr = np.linalg.norm(ref)
    return float(np.linalg.norm(x - ref) / nr) if nr > 0 else float(np.linalg.norm(x))


def compare(wl, gpu, ref, chains, w=None, reqs=None):
    """Max relative Frobenius errors per object kind; ref from oracle_request
    (with the same reqs)."""
    w = wl.w if w is None else w
    plan = gpu["plan"]
    T = gpu["T"].double().cpu().numpy()
    S = gpu["S"].double().cpu().numpy()
    st = gpu["state"].double().cpu().numpy()
    O = gpu["O"].double().cpu().numpy()
    err = {"T": 0.0, "S": 0.0, "state": 0.0, "O": 0.0, "T_floor": 0}
    for r, res in zip(range(len(ref)) if reqs is None else reqs, ref):
        e0 = int(plan.list_off[r])
        m = int(plan.list_off[r + 1]) - e0
        for j in range(m):
            slot = int(plan.pair_id[e0 + j])
            for ci, c in enumerate(chains):
                Tr = res["T"][j, ci]
                Tg = dense_T(T[slot, c], wl.dk)
                if np.linalg.norm(Tr) < FLOOR:
                    err["T_floor"] += 1
                    assert np.linalg.norm(Tg) <= FLOOR * np.sqrt(wl.dk)
                else:
                    err["T"] = max(err["T"], _rel(Tg, Tr))
                err["S"] = max(err["S"], _rel(S[slot, c], res["S"][j, ci]))
                if j > 0 and w > 0:
                    err["O"] = max(err["O"], _rel(O[e0 + j, :w, c], res["O"][j, :w, ci]))
        for ci, c in enumerate(chains):
            err["state"] = max(err["state"], _rel(st[r, c], res["state"][ci]))
    return err


def assert_close(err, tol, label=""):
    bad = {k: v for k, v in err.items() if k != "T_floor" and not (v <= tol)}
    assert not bad, f"{label}: errors above {tol}: {bad} (all: {err})"
