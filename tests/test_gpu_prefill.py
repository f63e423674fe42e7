"""GPU parity of the fused cold prefill (hypic_segment_prefill): every body
token's output of the segment read from a zero state, and the segment's pair,
against the fp64 oracle's token-by-token recurrence over the same tokens.

Per object: the n x dv output block of each (segment, chain) and its T and S,
relative Frobenius error <= 5e-3 (bf16 inputs, fp32 state, bf16 outputs).  The
pair must also agree with the one hypic_segment_build writes to fp32 rounding
(relative 1e-4 for T and 1e-5 for S per segment): the same chunk arithmetic
runs in both."""
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import oracle
import workloads
import state_caching_segment_amd as hy
from gpu_harness import FLOOR, TOL, chain_inputs, dense_T
from state_caching_segment_amd.plan import request_plan

pytestmark = pytest.mark.gpu

RAGGED = [130, 200, 9, 72, 73, 513, 64, 1]


def _prefill(wl, plan):
    dev = wl.k.device
    L = hy.layout(wl.family, wl.dtype, wl.n_chains, wl.dk)
    x = hy.tokens(wl.q, wl.k, wl.v, wl.g, wl.beta, wl.gamma)
    te = hy.hypic_t_elems(wl.family, wl.dk)
    T = torch.full((plan.n_slots, wl.n_chains, te), float("nan"), device=dev)
    S = torch.full((plan.n_slots, wl.n_chains, wl.dk, wl.dv), float("nan"), device=dev)
    out = torch.full((wl.n_tok, wl.n_chains, wl.dv), float("nan"), dtype=wl.k.dtype, device=dev)
    sb = torch.from_numpy(plan.seg_begin).to(dev)
    se = torch.from_numpy(plan.seg_end).to(dev)
    hy.hypic_segment_prefill(L, x, plan.n_slots, sb, se, plan.max_seg_len, T, S, out)
    T2, S2 = torch.empty_like(T), torch.empty_like(S)
    hy.hypic_segment_build(L, x, plan.n_slots, sb, se, plan.max_seg_len, T2, S2)
    torch.cuda.synchronize()
    # The same chunk arithmetic with another assignment of columns to waves
    # (and S rounds e^{Gamma_c - Gamma_t} v_t once less in the prefill: the
    # decay is applied where the value is consumed): both pairs agree to fp32
    # rounding, segment by segment; a long segment's T, the product of all its
    # transitions, accumulates the most (1e-4 relative; S 1e-5).
    for s in range(plan.n_slots):
        for a, b, tol in ((T[s], T2[s], 1e-4), (S[s], S2[s], 1e-5)):
            assert torch.isfinite(a).all()
            assert float((a - b).double().norm()) <= tol * float(b.double().norm()) + 1e-30, s
    return T, S, out


def _check(wl, plan, T, S, out, chains, label):
    def one(c):
        err = {"T": 0.0, "S": 0.0, "O": 0.0, "T_floor": 0}
        for s in range(plan.n_slots):
            b, e = int(plan.seg_begin[s]), int(plan.seg_end[s])
            if e == b:
                continue
            q, k, v, g, beta, gam = chain_inputs(wl, [c], b, e)
            Sr, Or = oracle.run(wl.family, q[0], k[0], v[0], None if g is None else g[0],
                                None if beta is None else beta[0])
            Tr, _ = oracle.pair(wl.family, k[0], v[0], None if g is None else g[0], None if beta is None else beta[0])
            Tg = dense_T(T[s, c].double().cpu().numpy(), wl.dk)
            if np.linalg.norm(Tr) < FLOOR:
                err["T_floor"] += 1
                assert np.linalg.norm(Tg) <= FLOOR * np.sqrt(wl.dk)
            else:
                err["T"] = max(err["T"], oracle.rel_fro(Tg, Tr))
            err["S"] = max(err["S"], oracle.rel_fro(S[s, c].double().cpu().numpy(), Sr))
            Og = out[b:e, c].double().cpu().numpy()
            assert np.isfinite(Og).all(), (s, c)
            err["O"] = max(err["O"], oracle.rel_fro(Og, Or))
        return err
    with ThreadPoolExecutor(max_workers=16) as ex:
        errs = list(ex.map(one, chains))
    worst = {k: max(e[k] for e in errs) for k in ("T", "S", "O")}
    worst["T_floor"] = sum(e["T_floor"] for e in errs)
    print(label, {k: (f"{v:.2e}" if isinstance(v, float) else v) for k, v in worst.items()}, flush=True)
    for k in ("T", "S", "O"):
        assert worst[k] <= TOL[wl.dtype], (label, worst)


@pytest.mark.parametrize("fam", ["gdn", "deltanet"])
@pytest.mark.parametrize("d", [128, 64, 32, 16])
@pytest.mark.parametrize("laws", ["gdn", "slow"])
def test_prefill_ragged(fam, d, laws):
    """Lengths below, at and past one 64-token chunk, one token, several
    chunks with a ragged tail; gates of the headline law and slow gates."""
    lw = workloads.SLOW_GDN_LAWS if laws == "slow" else workloads.GDN_LAWS
    wl = workloads.make(f"pf_{fam}_{d}", config_id=60, family=fam, dtype="bf16", n_chains=3, d=d, lens=RAGGED, w=8,
                        laws=lw, device="cuda")
    plan = request_plan(wl.requests, 0)   # every segment whole: bodies from token 0 of each
    T, S, out = _prefill(wl, plan)
    _check(wl, plan, T, S, out, list(range(wl.n_chains)), f"prefill {fam} d={d} {laws}")


def test_prefill_other_families_refused():
    wl = workloads.make("pf_gla", config_id=61, family="gla", dtype="bf16", n_chains=2, d=64, lens=[70], w=8,
                        laws=workloads.DIAG_LAWS, device="cuda")
    plan = request_plan(wl.requests, 0)
    with pytest.raises(hy.HypicError) as e:
        _prefill(wl, plan)
    assert e.value.status == -2


@pytest.mark.parametrize("name", ["c4", "c4_slowgdn"])
def test_prefill_full_request_sampled(name):
    """960 chains (30 layers x 32 heads), the 32768-token request's 48 cached
    bodies (w = 8 seams left out), every output written on the GPU; a seeded
    16-chain sample with the first and last chain against the oracle."""
    wl = workloads.config(name, device="cuda")
    plan = request_plan(wl.requests, wl.w, slot_order="longest_first")
    T, S, out = _prefill(wl, plan)
    rng = np.random.default_rng(406)
    chains = sorted(set([0, 959]) | set(rng.choice(np.arange(1, 959), 14, replace=False).tolist()))
    # seam tokens are not part of any body: their rows stay untouched
    sb = plan.seam_begin[plan.seam_begin >= 0]
    assert torch.isnan(out[int(sb[0]):int(sb[0]) + wl.w, 0].float()).all()
    _check(wl, plan, T, S, out, chains, f"prefill {name} sampled")
