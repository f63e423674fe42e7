"""GPU parity of the variant patches (codernav.top, section on linear layers,
last paragraph): hypic_rerotate against the oracle's re-rotation, and
hypic_conv_warmup against the oracle's causal convolution; then both in the
reuse path, against the oracle's recurrence over the whole request with keys
rotated at their absolute positions, or with the whole sequence convolved."""
import numpy as np
import pytest
import torch

import oracle
import workloads
import state_caching_segment_amd as hy
from gpu_harness import TOL
from state_caching_segment_amd.plan import request_plan

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("fam,d", [("gdn", 128), ("deltanet", 64), ("gdn", 32), ("gdn", 16), ("retnet", 64),
                                   ("mamba2", 128)])
def test_rerotate_matches_oracle(fam, d):
    """Random pairs, slots in a shuffled order, offsets from 0 to 3e6
    (angles reduced in fp64): every (item, chain) within 1e-5 of the oracle;
    in place gives the same."""
    rng = np.random.default_rng(d)
    n_slots, n_chains = 6, 5
    te = hy.hypic_t_elems(fam, d)
    T = torch.tensor(rng.normal(size=(n_slots, n_chains, te)), dtype=torch.float32, device="cuda")
    S = torch.tensor(rng.normal(size=(n_slots, n_chains, d, d)), dtype=torch.float32, device="cuda")
    slot = np.array([3, 0, 5, 1, 4, 2], np.int32)
    offs = np.array([0, 5, 517, 32768, 100003, 3_000_001], np.int64)
    To, So = torch.empty_like(T), torch.empty_like(S)
    L = hy.layout(fam, "f32", n_chains, d)
    hy.hypic_rerotate(L, n_slots, torch.from_numpy(slot).cuda(), torch.from_numpy(offs).cuda(), 10000.0, T, S,
                      To, So)
    torch.cuda.synchronize()
    Tn, Sn = T.double().cpu().numpy(), S.double().cpu().numpy()
    worst = 0.0
    for i in range(n_slots):
        for c in range(n_chains):
            t = Tn[slot[i], c]
            Td = t[0] * np.eye(d) if te == 1 else t.reshape(d, d)
            Tr, Sr = oracle.rerotate(Td, Sn[slot[i], c], float(offs[i]))
            got_T = To[i, c].double().cpu().numpy()
            got_T = got_T[0] * np.eye(d) if te == 1 else got_T.reshape(d, d)
            worst = max(worst, oracle.rel_fro(got_T, Tr), oracle.rel_fro(So[i, c].double().cpu().numpy(), Sr))
    print(f"rerotate {fam} d={d}: {worst:.2e}", flush=True)
    assert worst <= 1e-5
    # in place (slot i -> item i)
    ident = torch.arange(n_slots, dtype=torch.int32, device="cuda")
    T2, S2 = T[torch.from_numpy(slot).long().cuda()].clone(), S[torch.from_numpy(slot).long().cuda()].clone()
    hy.hypic_rerotate(L, n_slots, ident, torch.from_numpy(offs).cuda(), 10000.0, T2, S2, T2, S2)
    torch.cuda.synchronize()
    assert torch.equal(T2, To) and torch.equal(S2, So)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("K,act,w,d", [(4, 1, 8, 64), (1, 0, 8, 64), (8, 1, 8, 64), (3, 0, 8, 64), (4, 1, 5, 64),
                                       (8, 0, 13, 64), (3, 1, 20, 64), (8, 1, 13, 16), (2, 0, 9, 128)])
def test_conv_warmup_matches_oracle(dtype, K, act, w, d):
    """Windows at token 0, 2 (history partly before the sequence) and inside
    it; every window's q, k, v against the oracle's convolution of the whole
    raw sequence at those positions.  Windows shorter than the kernel's
    eight-token round and spanning two and three rounds (the history carried
    from one round to the next)."""
    rng = np.random.default_rng(K)
    n_tok, n_chains = 300, 3
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16}[dtype]
    raw = [torch.tensor(rng.normal(size=(n_tok, n_chains, d)), dtype=tdt, device="cuda") for _ in range(3)]
    taps = rng.normal(size=(3, n_chains, d, K)) / K
    starts = np.array([0, 2, 101, n_tok - w], np.int64)  # (the last window ends at the last token)
    outs = [torch.full((len(starts), w, n_chains, d), float("nan"), dtype=tdt, device="cuda") for _ in range(3)]
    L = hy.layout("gdn", dtype, n_chains, d)
    hy.hypic_conv_warmup(L, hy.tokens(q=raw[0], k=raw[1], v=raw[2]), torch.tensor(taps, dtype=torch.float32,
                         device="cuda"), K, act, len(starts), torch.from_numpy(starts).cuda(), w, *outs)
    torch.cuda.synchronize()
    tol = TOL[dtype]
    worst = 0.0
    for which in range(3):
        for c in range(n_chains):
            x = raw[which][:, c].double().cpu().numpy()
            full = oracle.conv(x, taps[which, c], act)
            for i, s in enumerate(starts):
                got = outs[which][i, :, c].double().cpu().numpy()
                worst = max(worst, oracle.rel_fro(got, full[s: s + w]))
    print(f"conv warm-up {dtype} K={K} act={act} w={w} d={d}: {worst:.2e}", flush=True)
    assert worst <= tol


def _rope_keys(x, p0):
    """Rows t of x [n][d] rotated to positions p0 + t (the oracle's R)."""
    return np.stack([oracle.rope_matrix(x.shape[1], p0 + t) @ x[t] for t in range(len(x))])


@pytest.mark.parametrize("fam", ["gdn", "deltanet"])
def test_rerotated_pairs_in_the_reuse_path(fam):
    """RoPE model, fp32 inputs: each body's pair is built with its keys at
    local positions, re-rotated to the body's absolute start, and composed
    with seam windows whose q and k sit at their absolute positions; the final
    state and every seam output match the oracle's recurrence over the whole
    request with absolutely rotated keys and queries.  Without the
    re-rotation the state is far off."""
    lens = [90, 70, 75, 110]
    d, C, w = 32, 2, 8
    wl = workloads.make("rope", config_id=62, family=fam, dtype="f32", n_chains=C, d=d, lens=lens, w=w,
                        laws=workloads.GDN_LAWS, device="cuda")
    plan = request_plan(wl.requests, w)
    q0, k0 = wl.q.double().cpu().numpy(), wl.k.double().cpu().numpy()
    n = wl.n_tok
    # absolute positions everywhere (seams and the oracle), local positions per body (the cache)
    q_abs, k_abs, k_loc = np.empty_like(q0), np.empty_like(k0), np.empty_like(k0)
    for c in range(C):
        q_abs[:, c], k_abs[:, c] = _rope_keys(q0[:, c], 0), _rope_keys(k0[:, c], 0)
        for s in range(plan.n_slots):
            b, e = int(plan.seg_begin[s]), int(plan.seg_end[s])
            k_loc[b:e, c] = _rope_keys(k0[b:e, c], 0)
    dev = "cuda"
    f32 = lambda a: torch.tensor(a, dtype=torch.float32, device=dev).contiguous()
    L = hy.layout(fam, "f32", C, d)
    kl_t = f32(k_loc)   # (held: hy.tokens keeps only its address)
    x_loc = hy.tokens(wl.q, kl_t, wl.v, wl.g, wl.beta)
    te = hy.hypic_t_elems(fam, d)
    T = torch.empty(plan.n_slots, C, te, device=dev)
    S = torch.empty(plan.n_slots, C, d, d, device=dev)
    hy.hypic_segment_build(L, x_loc, plan.n_slots, torch.from_numpy(plan.seg_begin).to(dev),
                           torch.from_numpy(plan.seg_end).to(dev), plan.max_seg_len, T, S)
    Tr, Sr = torch.empty_like(T), torch.empty_like(S)
    hy.hypic_rerotate(L, plan.n_slots, torch.arange(plan.n_slots, dtype=torch.int32, device=dev),
                      torch.from_numpy(plan.seg_begin).to(dev), 10000.0, T, S, Tr, Sr)
    qa, ka = f32(q_abs), f32(k_abs)
    x_abs = hy.tokens(qa, ka, wl.v, wl.g, wl.beta)
    out = {}
    for name, (TT, SS) in {"rerotated": (Tr, Sr), "as_cached": (T, S)}.items():
        state = torch.zeros(1, C, d, d, device=dev)
        o = torch.zeros(len(plan.pair_id), w, C, d, device=dev)
        hy.hypic_compose(L, hy.SEQ, 1, plan.max_list_len, torch.from_numpy(plan.list_off).to(dev),
                         torch.from_numpy(plan.pair_id).to(dev), plan.n_slots, TT, SS, x_abs,
                         torch.from_numpy(plan.seam_begin).to(dev), w, state, o)
        torch.cuda.synchronize()
        out[name] = (state.double().cpu().numpy(), o.double().cpu().numpy())
    g = None if wl.g is None else wl.g.double().cpu().numpy()
    beta = wl.beta.double().cpu().numpy()
    for c in range(C):
        Sref, Oref = oracle.run(fam, q_abs[:, c], k_abs[:, c], wl.v[:, c].double().cpu().numpy(),
                                None if g is None else g[:, c], beta[:, c])
        st, o = out["rerotated"]
        assert oracle.rel_fro(st[0, c], Sref) <= TOL["f32"]
        for j in range(1, len(lens)):
            sb = int(plan.seam_begin[j])
            assert oracle.rel_fro(o[j, :, c], Oref[sb: sb + w]) <= TOL["f32"], (c, j)
        assert oracle.rel_fro(out["as_cached"][0][0, c], Sref) > 1e-2


def test_conv_warmup_in_the_reuse_path():
    """Short-convolution model, fp32 inputs: bodies are cached from their
    segment's own convolution (zero history at the segment start; the seam
    tokens ahead of each body supply its taps), seams take the warm-up from
    raw inputs; the final state and seam outputs match the oracle's
    recurrence over the whole request convolved as one sequence.  With cold
    seam windows (no warm-up) the seam outputs are off."""
    rng = np.random.default_rng(63)
    lens = [80, 66, 95, 70]
    d, C, w, K = 32, 2, 8, 4
    fam = "gdn"
    wl = workloads.make("conv", config_id=63, family=fam, dtype="f32", n_chains=C, d=d, lens=lens, w=w,
                        laws=workloads.GDN_LAWS, device="cuda")
    plan = request_plan(wl.requests, w)
    raw = [t.double().cpu().numpy() for t in (wl.q, wl.k, wl.v)]
    taps = rng.normal(size=(3, C, d, K)) / K
    full = [np.stack([oracle.conv(raw[i][:, c], taps[i, c], 1) for c in range(C)], 1) for i in range(3)]
    seg_local = [np.empty_like(r) for r in raw]
    b_all = wl.requests[0]
    for j in range(len(lens)):
        b, e = int(b_all[j]), int(b_all[j + 1])
        for i in range(3):
            for c in range(C):
                seg_local[i][b:e, c] = oracle.conv(raw[i][b:e, c], taps[i, c], 1)
    dev = "cuda"
    f32 = lambda a: torch.tensor(a, dtype=torch.float32, device=dev).contiguous()
    L = hy.layout(fam, "f32", C, d)
    ql, kl, vl = (f32(a) for a in seg_local)
    xl = hy.tokens(ql, kl, vl, wl.g, wl.beta)
    T = torch.empty(plan.n_slots, C, d * d, device=dev)
    S = torch.empty(plan.n_slots, C, d, d, device=dev)
    hy.hypic_segment_build(L, xl, plan.n_slots, torch.from_numpy(plan.seg_begin).to(dev),
                           torch.from_numpy(plan.seg_end).to(dev), plan.max_seg_len, T, S)
    # seam windows: warm-up from raw inputs, laid out one window after another
    seams = plan.seam_begin[plan.seam_begin >= 0]
    ns = len(seams)
    wq, wk, wv = (torch.empty(ns, w, C, d, device=dev) for _ in range(3))
    rq, rk, rv = (f32(a) for a in raw)
    taps_t = f32(taps)
    hy.hypic_conv_warmup(L, hy.tokens(q=rq, k=rk, v=rv), taps_t, K, 1, ns, torch.from_numpy(seams).to(dev), w,
                         wq, wk, wv)
    # gates and beta of the seam tokens, gathered to the same layout
    idx = torch.from_numpy((seams[:, None] + np.arange(w)[None, :]).reshape(-1)).to(dev)
    sg, sbeta = wl.g[idx].contiguous(), wl.beta[idx].contiguous()
    xs = hy.tokens(wq.view(ns * w, C, d), wk.view(ns * w, C, d), wv.view(ns * w, C, d), sg, sbeta)
    seam_begin = np.where(plan.seam_begin >= 0, np.cumsum(plan.seam_begin >= 0) * w - w, -1).astype(np.int64)
    results = {}
    for name, x_seam in (("warm", xs), ("cold", hy.tokens(ql, kl, vl, wl.g, wl.beta))):
        sbg = seam_begin if name == "warm" else plan.seam_begin
        state = torch.zeros(1, C, d, d, device=dev)
        o = torch.zeros(len(plan.pair_id), w, C, d, device=dev)
        hy.hypic_compose(L, hy.SEQ, 1, plan.max_list_len, torch.from_numpy(plan.list_off).to(dev),
                         torch.from_numpy(plan.pair_id).to(dev), plan.n_slots, T, S, x_seam,
                         torch.from_numpy(sbg).to(dev), w, state, o)
        torch.cuda.synchronize()
        results[name] = (state.double().cpu().numpy(), o.double().cpu().numpy())
    g, beta = wl.g.double().cpu().numpy(), wl.beta.double().cpu().numpy()
    cold_err = 0.0
    for c in range(C):
        Sref, Oref = oracle.run(fam, full[0][:, c], full[1][:, c], full[2][:, c], g[:, c], beta[:, c])
        st, o = results["warm"]
        assert oracle.rel_fro(st[0, c], Sref) <= TOL["f32"]
        for j in range(1, len(lens)):
            s0 = int(plan.seam_begin[j])
            assert oracle.rel_fro(o[j, :, c], Oref[s0: s0 + w]) <= TOL["f32"], (c, j)
            cold_err = max(cold_err, oracle.rel_fro(results["cold"][1][j, :, c], Oref[s0: s0 + w]))
    assert cold_err > 1e-2
