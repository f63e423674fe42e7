"""Benchmark of the linear-layer segment state caching hot path on one GPU.

One step = the whole path over one synthetic request:
  1. hypic_segment_build: the cached pair (T_C, S(C|0)) of every segment body
     on every chain;
  2. hypic_compose: the request's running state assembled from those pairs,
     advancing through the w = 8 seam tokens of every internal segment and
     emitting their outputs.
Default workload: Gated DeltaNet, bf16 inputs with fp32 state, 30 layers x 32
heads = 960 chains, d = 128, one 32768-token request in 48 segments
(lognormal lengths, min 512, mean ~683), seams of 8 tokens on the 47 internal
segments.  Inputs are seeded synthetic tensors generated on the GPU and
resident in HBM before timing starts.

Printed: one JSON line with build tokens/s (request tokens / build time) as
`value`, the compose latency, each kernel's roofline fraction, and the fp64
oracle timed on the host on a bounded sample of chains.
"""
import argparse
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads  # noqa: E402
import state_caching_segment_amd as hy  # noqa: E402
from state_caching_segment_amd.plan import request_plan  # noqa: E402

METRIC = "(T_C,S0) build tokens/s + 32k-request state-compose latency (ms), 1 GPU"
HBM_PEAK = 8.0e12        # B/s, MI355X HBM3E
BF16_PEAK = 2.5e15       # FLOP/s, dense bf16 MFMA
FP32_MFMA_PEAK = 157.3e12
CH = 64


DENSE = ("deltanet", "gdn", "kda")


def _gate_elems(family, d):
    """Log-gate values per token: a dk-vector (GLA, KDA), a scalar (Mamba2,
    GDN) or none."""
    return d if family in ("gla", "kda") else (1 if family in ("mamba2", "gdn") else 0)


def _t_elems(family, d):
    return d * d if family in DENSE else (d if family == "gla" else 1)


def build_cost(family, lens, d, n_chains, in_bytes):
    """Algorithmic flops and HBM bytes of building the pairs of segments with
    the given lengths.
    Dense families (chunked UT/WY form, c = 64), per chunk of c tokens: carry
    of [T|S] 8 c d^2 (4 c d^2 for a segment's first chunk, which starts from
    [I|0]), Gram c(c-1)d, unit-lower inverse c^3/3, W and U 2 c^2 d.
    Diagonal families: 2 d^2 per token (the k~ v^T accumulation).
    Bytes: k, v (d each), the log-gates and beta per token read once, and the
    fp32 pair (T and S) written once."""
    flops = 0.0
    for n in lens:
        if family in DENSE:
            for j, c0 in enumerate(range(0, int(n), CH)):
                c = min(CH, int(n) - c0)
                carry = 8 * c * d * d if j > 0 else 4 * c * d * d
                flops += carry + c * (c - 1) * d + c ** 3 / 3 + 2 * c * c * d
        else:
            flops += 2.0 * d * d * int(n)
    tokens = float(np.sum(lens))
    per_tok = 2 * d + _gate_elems(family, d) + (1 if family in DENSE else 0)
    byts = tokens * per_tok * in_bytes + len(lens) * (_t_elems(family, d) + d * d) * 4
    return flops * n_chains, byts * n_chains


def compose_cost(family, n_entries, n_seams, w, d, n_chains, in_bytes):
    """Algorithmic flops and bytes of one sequential compose with seams: every
    pair read once (fp32 T and S), per seam token q, k, v (d each), the gates
    and beta read and o (d, fp32) written, initial and final state; flops
    2 d^3 per dense pair after the first (T S; 2 d^2 for diagonal T) and
    about 7 d^2 per seam token."""
    pair_flops = 2 * d ** 3 if family in DENSE else 2 * d * d
    flops = (n_entries - 1) * pair_flops + n_seams * w * 7 * d * d
    seam_in = 3 * d + _gate_elems(family, d) + (1 if family in DENSE else 0)
    byts = n_entries * (_t_elems(family, d) + d * d) * 4 + n_seams * w * (seam_in * in_bytes + d * 4) + 2 * d * d * 4
    return flops * n_chains, byts * n_chains


def build_kernel(family, dtype):
    """The build kernel the library dispatches for a family and input dtype,
    and the sources whose hash keys its stored counter readings."""
    if family == "kda":
        return "k_build_kda", ["build_kda.hip", "common.h"]
    if family in ("deltanet", "gdn"):
        if dtype == "bf16":
            return "k_build_dense_pipe", ["build_dense_pipe.hip", "common.h"]
        return "k_build_dense", ["build_dense.hip", "common.h"]
    return "k_build_diag", ["build_diag.hip", "common.h"]


def compose_kernel(family, in_bf16=True, d=128):
    """The sequential compose kernel the library dispatches for a family, and
    the sources whose hash keys its stored counter readings."""
    files = ["compose.hip", "compose_common.h", "common.h"]
    if family in ("deltanet", "gdn") and in_bf16 and d >= 64:
        return "k_compose_lean", files
    return ("k_compose_dense" if family in ("deltanet", "gdn", "kda") else "k_compose_seq"), files


def measured_traffic(key, files):
    """HBM bytes per launch from the committed rocprofv3 FETCH_SIZE / WRITE_SIZE
    passes (profiles/counters.json), or None when the kernel's source changed
    since they were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "counters.json")
    if not os.path.exists(path):
        return None
    c = json.load(open(path)).get(key)
    if c is None:
        return None
    h = hashlib.sha256()
    for f in files:
        h.update(open(os.path.join(ROOT, "state_caching_segment_amd", "csrc", f), "rb").read())
    if h.hexdigest()[:16] != c["source_sha"]:
        return None
    return c["fetch_bytes"] + c["write_bytes"]


def cpu_baseline(wl, n_chains_sample, w):
    """The fp64 oracle (build every pair token by token, compose, seams) on a
    sample of chains, all host threads; scaled to request tokens/s for all
    chains."""
    import oracle
    chains = list(range(n_chains_sample))
    b = wl.requests[0]

    def cm(x):
        if x is None:
            return None
        return np.ascontiguousarray(np.moveaxis(x[:, chains].double().cpu().numpy(), 1, 0))

    q, k, v, g, beta = cm(wl.q), cm(wl.k), cm(wl.v), cm(wl.g), cm(wl.beta)
    gam = None if wl.gamma is None else wl.gamma[chains].double().cpu().numpy()
    threads = oracle.max_threads()
    t0 = time.perf_counter()
    oracle.request_batch(wl.family, b - b[0], w, q, k, v, g, beta, gam, want_pairs=False, nthreads=threads)
    dt = time.perf_counter() - t0
    tok = float(b[-1] - b[0])
    return {"value": tok * n_chains_sample / (wl.n_chains * dt), "unit": "tokens/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{n_chains_sample} of {wl.n_chains} chains, full {int(tok)}-token request "
                      f"(all pairs + compose + seams), {dt:.1f} s; scaled by chains"}


def workload_text(name, wl, plan, C, d, w, req_tokens, n_build, hits, mode_name):
    n_req = len(wl.requests)
    heads = "30 layers x 32 heads" if C == 960 else f"{C} heads"
    req = (f"one {req_tokens}-token request" if n_req == 1 else f"{n_req} requests, {req_tokens} tokens")
    if hits:
        return (f"{wl.family} {wl.dtype}: build of {n_build} cold segment bodies + {mode_name} compose with w={w} "
                f"seams over all {plan.n_slots} cached pairs: {C} chains ({heads}), d={d}, {req}")
    return (f"{wl.family} pair build + {mode_name} compose with w={w} seams: {C} chains ({heads}), d={d}, {req}, "
            f"{plan.n_slots} segments")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="c4")
    ap.add_argument("--calib-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB (5 times), to scale HBM counters")
    ap.add_argument("--compose", choices=("auto", "seq", "tree"), default="auto",
                    help="compose mode; auto: the tree scan where the workload asks for it (cache hits) or where the "
                         "request's chains are fewer than the compute units and its list has at least 16 entries "
                         "(latency-bound), else sequential")
    ap.add_argument("--cpu-chains", type=int, default=-1,
                    help="chains in the oracle's CPU-baseline sample (-1: four per host thread, about 13 s of "
                         "host work at the default workload; 0: skip)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (the path shards by chain with no "
              f"exchange, so N GPUs would each run this same per-GPU workload).", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)
    if args.calib_copy > 0:
        n = args.calib_copy * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calib_copy_bytes_read": n * 4, "calib_copy_bytes_written": n * 4, "launches": 5}))
        return
    hy.load()

    wl = workloads.config(args.config, device="cuda")
    w = wl.w
    plan = request_plan(wl.requests, w, slot_order="longest_first")
    d, C = wl.dk, wl.n_chains
    dev = "cuda"
    L = hy.layout(wl.family, wl.dtype, C, d)
    x = hy.tokens(wl.q, wl.k, wl.v, wl.g, wl.beta, wl.gamma)
    te = hy.hypic_t_elems(wl.family, d)
    T = torch.empty(plan.n_slots, C, te, device=dev)
    S = torch.empty(plan.n_slots, C, d, d, device=dev)
    sb = torch.from_numpy(plan.seg_begin).to(dev)
    se = torch.from_numpy(plan.seg_end).to(dev)
    lo = torch.from_numpy(plan.list_off).to(dev)
    pid = torch.from_numpy(plan.pair_id).to(dev)
    seam = torch.from_numpy(plan.seam_begin).to(dev)
    state = torch.zeros(plan.n_req, C, d, d, device=dev)
    o = torch.zeros(len(plan.pair_id), w, C, d, device=dev)
    stream = torch.cuda.current_stream()
    # Workloads with cache hits (n_cold set) time the build of the cold
    # segment bodies only, into their own pair buffers, and compose with the
    # associative tree scan over the full pair cache, which is built once
    # beforehand (untimed); the others time the build of every segment and
    # the sequential compose.
    cold = (np.concatenate([c for c in wl.cold])[plan.seg_index] if wl.cold
            else np.ones(plan.n_slots, bool))  # per slot
    hits = not cold.all()
    if args.compose == "auto":
        n_cu = torch.cuda.get_device_properties(dev).multi_processor_count
        # with too few chains to fill the GPU the tree's parallel blocks pay
        # from lists of 8 entries: 32 entries on 16 GLA chains (0.20 ms against
        # 0.44), 8 entries on 8 RetNet chains (0.042 ms against 0.048)
        mode = hy.TREE if hits or (plan.n_req * C < n_cu and plan.max_list_len >= 8) else hy.SEQ
    else:
        mode = hy.TREE if args.compose == "tree" else hy.SEQ
    if hits:
        hy.hypic_segment_build(L, x, plan.n_slots, sb, se, plan.max_seg_len, T, S, stream=stream)
        cb_idx = np.nonzero(cold)[0]
        bsb = torch.from_numpy(plan.seg_begin[cb_idx]).to(dev)
        bse = torch.from_numpy(plan.seg_end[cb_idx]).to(dev)
        n_build = len(cb_idx)
        bT = torch.empty(n_build, C, te, device=dev)
        bS = torch.empty(n_build, C, d, d, device=dev)
        build_lens = plan.seg_end[cb_idx] - plan.seg_begin[cb_idx]
    else:
        bsb, bse, n_build, bT, bS = sb, se, plan.n_slots, T, S
        build_lens = plan.seg_end - plan.seg_begin
    max_build = int(build_lens.max())
    nws = hy.hypic_workspace_bytes(L, hy.OP_COMPOSE_TREE, plan.n_req, plan.max_list_len, w)
    ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=dev)

    def step(ev=None, cmode=mode):
        if ev:
            ev[0].record(stream)
        hy.hypic_segment_build(L, x, n_build, bsb, bse, max_build, bT, bS, stream=stream)
        if ev:
            ev[1].record(stream)
        state.zero_()
        if ev:
            ev[2].record(stream)
        hy.hypic_compose(L, cmode, plan.n_req, plan.max_list_len, lo, pid, plan.n_slots, T, S, x, seam, w, state,
                         o, ws=ws if cmode == hy.TREE else None, ws_bytes=nws if cmode == hy.TREE else 0,
                         stream=stream)
        if ev:
            ev[3].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # the other compose mode on the same lists, for comparison
    alt_mode = hy.SEQ if mode == hy.TREE else hy.TREE
    sev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    for i in range(args.steps):
        step(sev[i], alt_mode)
    torch.cuda.synchronize()
    alt_ms = float(np.median([e[2].elapsed_time(e[3]) for e in sev]))
    b_ms = np.array([e[0].elapsed_time(e[1]) for e in evs])
    c_ms = np.array([e[2].elapsed_time(e[3]) for e in evs])
    step_ms = wall * 1e3 / args.steps

    in_bytes = 2 if wl.dtype == "bf16" else 4
    req_tokens = int(sum(int(b[-1] - b[0]) for b in wl.requests))
    build_tokens = int(build_lens.sum())
    bf, bb = build_cost(wl.family, build_lens, d, C, in_bytes)
    n_seams = int((plan.seam_begin >= 0).sum())
    cf, cb = compose_cost(wl.family, len(plan.pair_id), n_seams, w, d, C, in_bytes)
    tb, tc = float(np.median(b_ms)) * 1e-3, float(np.median(c_ms)) * 1e-3
    # the build's binding roof is the larger of its HBM and bf16-MFMA times
    b_hbm, b_mfma = bb / tb, bf / tb
    b_bound = "hbm" if bb / HBM_PEAK >= bf / BF16_PEAK else "mfma"
    roof_build = ({"bound": "hbm", "achieved": b_hbm / 1e9, "peak": HBM_PEAK / 1e9, "unit": "GB/s",
                   "frac": b_hbm / HBM_PEAK} if b_bound == "hbm" else
                  {"bound": "mfma", "achieved": b_mfma / 1e12, "peak": BF16_PEAK / 1e12, "unit": "TFLOP/s",
                   "frac": b_mfma / BF16_PEAK})
    bk_name, bk_files = build_kernel(wl.family, wl.dtype)
    key = "" if args.config == "c4" else "_" + args.config  # stored counters per workload
    roof_build.update({"traffic": measured_traffic("build" + key, bk_files),
                       "kernel": bk_name, "alg_bytes": bb, "alg_flops": bf,
                       "mfma_frac_alg": b_mfma / BF16_PEAK, "hbm_frac_alg": b_hbm / HBM_PEAK})
    ck_name, ck_files = compose_kernel(wl.family, wl.dtype == "bf16", d)
    if mode == hy.TREE:
        ck_name = "k_compose_dense (tree block phase) + k_tree_scan + k_tree_fix"
    roof_comp = {"bound": "hbm", "achieved": cb / tc / 1e9, "peak": HBM_PEAK / 1e9, "unit": "GB/s",
                 "frac": cb / tc / HBM_PEAK, "traffic": measured_traffic("compose" + key, ck_files),
                 "kernel": ck_name, "alg_bytes": cb,
                 "alg_flops": cf}
    out = {
        "metric": METRIC,
        "value": build_tokens / tb,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": step_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if wl.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": workload_text(args.config, wl, plan, C, d, w, req_tokens, n_build, hits,
                                               "tree" if mode == hy.TREE else "seq"),
                   "chains": C, "d": d, "request_tokens": req_tokens, "segments": plan.n_slots, "w": w,
                   "built_segments": n_build, "built_tokens": build_tokens, "compose_mode": "tree" if mode == hy.TREE else "seq",
                   "state_dtype": "f32", "slot_order": "longest_first"},
        "build_ms": float(np.median(b_ms)),
        "build_ms_p10_p90": [float(np.percentile(b_ms, 10)), float(np.percentile(b_ms, 90))],
        "compose_latency_ms": float(np.median(c_ms)),
        "compose_ms_p10_p90": [float(np.percentile(c_ms, 10)), float(np.percentile(c_ms, 90))],
        "chain_tokens_per_s_build": build_tokens * C / tb,
        "roofline": roof_build,
        "roofline_compose": roof_comp,
    }
    out["compose_alt"] = {"mode": "seq" if alt_mode == hy.SEQ else "tree", "ms": alt_ms}
    if args.cpu_chains != 0:
        import oracle
        n_cpu = 4 * oracle.max_threads() if args.cpu_chains < 0 else args.cpu_chains
        out["cpu_baseline"] = cpu_baseline(wl, min(n_cpu, C), w)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
