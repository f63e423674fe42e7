"""Compact pairs on the GPU: hypic_pair_compact's bf16 T^ and power-of-two
scale reproduce T to bf16 rounding, and hypic_compose_compact over them
matches the oracle's reuse path within the bf16 tolerance, at the full
960-chain request under the headline gates and under the two stressors in
which T carries real weight (no decay; slow gates)."""
import numpy as np
import pytest
import torch

import workloads
import state_caching_segment_amd as hy
from gpu_harness import TOL, gpu_request, oracle_request

pytestmark = pytest.mark.gpu


def _compact(L, T, n_slots):
    C, d2 = T.shape[1], T.shape[2]
    Tc = torch.empty(n_slots, C, d2, dtype=torch.bfloat16, device="cuda")
    sc = torch.empty(n_slots, C, device="cuda")
    hy.hypic_pair_compact(L, n_slots, T, Tc, sc)
    torch.cuda.synchronize()
    return Tc, sc


def _compose_compact(wl, gpu, Tc, sc, prefix=False):
    plan = gpu["plan"]
    dev = "cuda"
    L = hy.layout(wl.family, wl.dtype, wl.n_chains, wl.dk)
    x = hy.tokens(wl.q, wl.k, wl.v, wl.g, wl.beta)
    state = torch.zeros(plan.n_req, wl.n_chains, wl.dk, wl.dk, device=dev)
    o = torch.zeros(len(plan.pair_id), wl.w, wl.n_chains, wl.dk, device=dev)
    pre = torch.zeros(len(plan.pair_id), wl.n_chains, wl.dk, wl.dk, device=dev) if prefix else None
    hy.hypic_compose_compact(L, plan.n_req, plan.max_list_len, torch.from_numpy(plan.list_off).to(dev),
                             torch.from_numpy(plan.pair_id).to(dev), plan.n_slots, Tc, sc, gpu["S"], x,
                             torch.from_numpy(plan.seam_begin).to(dev), wl.w, state, o, pre)
    torch.cuda.synchronize()
    return state, o, pre


def test_compaction_is_exact_scaling_and_bf16_rounding():
    """Long segments under the headline gates leave T in fp32's subnormal
    range (the 2048-token body): those too are scaled exactly."""
    wl = workloads.make("cpt", config_id=70, family="gdn", dtype="bf16", n_chains=4, d=128,
                        lens=[130, 513, 9, 64, 700, 2048], w=8, laws=workloads.GDN_LAWS, device="cuda")
    gpu = gpu_request(wl)
    L = hy.layout("gdn", "bf16", 4, 128)
    n = gpu["plan"].n_slots
    Tc, sc = _compact(L, gpu["T"], n)
    assert torch.isfinite(Tc).all() and torch.isfinite(sc).all()
    T = gpu["T"].double()
    s = sc.double()
    mant, _ = np.frexp(s.cpu().numpy())
    assert (mant == 0.5).all(), "scales are powers of two"
    rec = Tc.double() * s[..., None]
    for i in range(n):
        for c in range(4):
            t = T[i, c]
            mx = t.abs().max().item()
            if mx == 0:
                assert sc[i, c].item() == 1.0 and torch.count_nonzero(Tc[i, c]) == 0
                continue
            assert 0.5 <= (Tc[i, c].double().abs().max().item()) <= 1.0
            # bf16 round to nearest (8 significant bits): relative 2^-8 at most per element
            assert ((rec[i, c] - t).abs() <= 2.0 ** -8 * t.abs() + 1e-45).all()


@pytest.mark.parametrize("name", ["c4", "c4_deltanet", "c4_slowgdn"])
def test_compact_compose_full_request_sampled(name):
    wl = workloads.config(name, device="cuda")
    gpu = gpu_request(wl)
    L = hy.layout(wl.family, wl.dtype, wl.n_chains, wl.dk)
    Tc, sc = _compact(L, gpu["T"], gpu["plan"].n_slots)
    state, o, _ = _compose_compact(wl, gpu, Tc, sc)
    rng = np.random.default_rng(407)
    chains = sorted(set([0, 959]) | set(rng.choice(np.arange(1, 959), 14, replace=False).tolist()))
    ref = oracle_request(wl, chains)[0]
    st, oo = state.double().cpu().numpy(), o.double().cpu().numpy()
    assert np.isfinite(st).all() and np.isfinite(oo).all() and torch.isfinite(Tc).all()
    full_st = gpu["state"].double().cpu().numpy()
    err_state = err_o = err_fp32 = 0.0
    for ci, c in enumerate(chains):
        r = ref["state"][ci]
        err_state = max(err_state, np.linalg.norm(st[0, c] - r) / np.linalg.norm(r))
        err_fp32 = max(err_fp32, np.linalg.norm(full_st[0, c] - r) / np.linalg.norm(r))
        for j in range(1, len(gpu["plan"].pair_id)):
            ro = ref["O"][j, :, ci]
            err_o = max(err_o, np.linalg.norm(oo[j, :, c] - ro) / np.linalg.norm(ro))
    print(f"compact {name}: state {err_state:.2e} (fp32 pairs {err_fp32:.2e}), seam outputs {err_o:.2e}", flush=True)
    assert err_state <= TOL["bf16"] and err_o <= TOL["bf16"]


def test_compact_prefix_states_and_ragged():
    """Ragged lists, two requests, with prefix states: every entry's state
    within tolerance of the fp32-pair compose's."""
    lens = [[70, 40, 33, 90, 25, 61], [130, 60, 45, 81]]
    wl = workloads.make("cpt2", config_id=71, family="deltanet", dtype="bf16", n_chains=3, d=64, lens=lens, w=8,
                        laws=workloads.GDN_LAWS, device="cuda")
    gpu = gpu_request(wl, prefix=True)
    L = hy.layout("deltanet", "bf16", 3, 64)
    Tc, sc = _compact(L, gpu["T"], gpu["plan"].n_slots)
    state, o, pre = _compose_compact(wl, gpu, Tc, sc, prefix=True)
    for a, b in ((state, gpu["state"]), (pre, gpu["prefix"])):
        for i in range(a.shape[0]):
            for c in range(3):
                assert float((a[i, c] - b[i, c]).double().norm() / b[i, c].double().norm()) <= TOL["bf16"]
