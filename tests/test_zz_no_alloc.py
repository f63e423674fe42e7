"""The tree compose with the library's own workspace
(hypic_compose_tree_noalloc), called through the C ABI, against the same
compose with a caller workspace (hypic_compose, HYPIC_TREE): bitwise equal on
two calls in a row, the second smaller than the first, so that it runs over
what the first left in the shared workspace."""
import numpy as np
import pytest
import torch

import workloads
import state_caching_segment_amd as hy
from state_caching_segment_amd.plan import request_plan

pytestmark = pytest.mark.gpu


def _case(fam, dtype, d, lens, n_chains, cid):
    laws = {"gdn": workloads.GDN_LAWS, "kda": workloads.KDA_LAWS}.get(fam, workloads.DIAG_LAWS)
    wl = workloads.make(f"noalloc_{fam}", config_id=cid, family=fam, dtype=dtype, n_chains=n_chains, d=d, lens=lens,
                        w=8, laws=laws, device="cuda")
    plan = request_plan(wl.requests, wl.w)
    dev = "cuda"
    L = hy.layout(fam, dtype, n_chains, d)
    x = hy.tokens(wl.q, wl.k, wl.v, wl.g, wl.beta, wl.gamma)
    te = hy.hypic_t_elems(fam, d)
    T = torch.empty(plan.n_slots, n_chains, te, device=dev)
    S = torch.empty(plan.n_slots, n_chains, d, d, device=dev)
    hy.hypic_segment_build(L, x, plan.n_slots, torch.from_numpy(plan.seg_begin).to(dev),
                           torch.from_numpy(plan.seg_end).to(dev), plan.max_seg_len, T, S)
    args = dict(L=L, n_req=plan.n_req, max_list_len=plan.max_list_len, list_off=torch.from_numpy(plan.list_off).to(dev),
                pair_id=torch.from_numpy(plan.pair_id).to(dev), n_slots=plan.n_slots, T=T, S=S, seam=x,
                seam_begin=torch.from_numpy(plan.seam_begin).to(dev), w=wl.w)
    return wl, plan, args


def _run(args, plan, n_chains, d, noalloc, w):
    dev = "cuda"
    rng = np.random.default_rng(3)
    state = torch.tensor(rng.normal(size=(plan.n_req, n_chains, d, d)) * 0.1, dtype=torch.float32, device=dev)
    o = torch.zeros(len(plan.pair_id), w, n_chains, d, device=dev)
    pre = torch.zeros(len(plan.pair_id), n_chains, d, d, device=dev)
    a = dict(args)
    L = a.pop("L")
    if noalloc:
        hy.hypic_compose_tree_noalloc(L, *a.values(), state, o, pre)
    else:
        nws = hy.hypic_workspace_bytes(L, hy.OP_COMPOSE_TREE, plan.n_req, plan.max_list_len, w)
        assert 0 < nws <= hy.NOALLOC_WORKSPACE_BYTES
        ws = torch.empty(nws, dtype=torch.uint8, device=dev)
        hy.hypic_compose(L, hy.TREE, *a.values(), state, o, pre, ws=ws, ws_bytes=nws)
    torch.cuda.synchronize()
    return state, o, pre


@pytest.mark.parametrize("fam,dtype,d", [("gdn", "bf16", 128), ("kda", "bf16", 64), ("gla", "bf16", 64)])
def test_noalloc_tree_matches_caller_workspace(fam, dtype, d):
    big = [[70, 40, 33, 90, 25, 61, 44, 30, 52, 19, 27], [130, 60, 45], [40, 31, 29, 66, 73, 20, 18]]
    small = [[50, 40, 33], [30, 29]]
    for lens, n_chains, cid in ((big, 6, 95), (small, 3, 96)):
        wl, plan, args = _case(fam, dtype, d, lens, n_chains, cid)
        for use_prefix in (False, True):
            a = dict(args)
            ref = _run(a, plan, n_chains, d, False, wl.w)
            got = _run(a, plan, n_chains, d, True, wl.w)
            for name, x, y in zip(("state", "O", "prefix"), got, ref):
                assert torch.isfinite(y).all(), name
                assert torch.equal(x, y), (fam, name, len(plan.pair_id))


def test_noalloc_rejects_oversize_before_any_launch():
    """A request whose tree workspace exceeds the library's own is refused with
    HYPIC_E_WORKSPACE, naming both sizes."""
    L = hy.layout("kda", "bf16", 32, 128)
    need = hy.hypic_workspace_bytes(L, hy.OP_COMPOSE_TREE, 16, 128, 8)
    assert need > hy.NOALLOC_WORKSPACE_BYTES
    with pytest.raises(hy.HypicError) as e:
        # (device pointers are never dereferenced here; they only need the
        # alignment the call checks first)
        hy.hypic_compose_tree_noalloc(L, 16, 128, 16, 16, 10, 16, 16, None, None, 0, 16, None)
    assert e.value.status == -3 and str(hy.NOALLOC_WORKSPACE_BYTES) in str(e.value)
