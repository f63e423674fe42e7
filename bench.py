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
`value`, the compose latency, each kernel's roofline fraction, the fused cold
prefill (outputs of every body token and the pairs in one pass) for the
dense families, a measured device copy bandwidth beside the vendor peak, and
the fp64 oracle timed on the host on a bounded sample of chains.

Workloads with cache hits (the KDA layer: 13 cold segments of 128 per
request) time the build of the cold bodies only and compose with the tree
scan over the full pair cache; --layers N repeats that for N layers, each on
fresh inputs generated untimed, and reports the per-layer times and their
sum.  --ab PATH alternates steps between this library and another build of
it in the same process (a same-box A/B comparison).
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
    Dense families (chunked UT/WY form, c = 64; KDA c = 32), per chunk of c tokens: carry
    of [T|S] 8 c d^2 (4 c d^2 for a segment's first chunk, which starts from
    [I|0]), Gram c(c-1)d, unit-lower inverse c^3/3, W and U 2 c^2 d.
    Diagonal families: 2 d^2 per token (the k~ v^T accumulation).
    Bytes: k, v (d each), the log-gates and beta per token read once, and the
    fp32 pair (T and S) written once."""
    flops = 0.0
    for n in lens:
        if family in DENSE:
            ch = 32 if family == "kda" else CH
            for j, c0 in enumerate(range(0, int(n), ch)):
                c = min(ch, int(n) - c0)
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
        if dtype == "bf16":
            return "k_build_kda_pipe", ["build_kda_pipe.hip", "common.h"]
        return "k_build_kda", ["build_kda.hip", "common.h"]
    if family in ("deltanet", "gdn"):
        if dtype == "bf16":
            return "k_build_dense_pipe", ["build_dense_pipe.hip", "common.h"]
        return "k_build_dense", ["build_dense.hip", "common.h"]
    if dtype == "bf16":
        return "k_build_diag_slices", ["build_diag.hip", "common.h", "compose_common.h"]
    return "k_build_diag", ["build_diag.hip", "common.h", "compose_common.h"]


def compose_kernel(family, in_bf16=True, d=128, tree=False):
    """The compose kernels the library dispatches for a family and mode, and
    the sources whose hash keys their stored counter readings."""
    files = ["compose.hip", "compose_common.h", "common.h"]
    dense = family in DENSE
    if tree:
        block = "k_compose_dense (tree block)" if dense else "k_tree_block"
        scan = "k_compose_lean (scan)" if dense and in_bf16 and d >= 64 else "k_tree_scan"
        fix = "k_tree_fix_mma" if in_bf16 and d >= 64 else "k_tree_fix"
        return f"{block} + {scan} + {fix}", files
    if family in ("deltanet", "gdn") and in_bf16 and d >= 64:
        return "k_compose_lean", files
    return ("k_compose_dense" if dense else "k_compose_seq"), files


def prefill_cost(family, lens, d, n_chains, in_bytes):
    """Algorithmic flops and bytes of the fused cold prefill: the pair build
    plus, per chunk of c tokens, the outputs from the chunk-start state
    (2 c d^2, none for a segment's first chunk, which starts from zero) and
    within the chunk (tril(Q K^T): c(c+1) d; times the solved rows: c(c+1) d);
    bytes add q read and o written (d each, input dtype) per token."""
    flops, byts = build_cost(family, lens, d, n_chains, in_bytes)
    extra = 0.0
    for n in lens:
        for j, c0 in enumerate(range(0, int(n), CH)):
            c = min(CH, int(n) - c0)
            extra += (2 * c * d * d if j > 0 else 0) + 2 * c * (c + 1) * d
    tokens = float(np.sum(lens))
    return flops + extra * n_chains, byts + tokens * 2 * d * in_bytes * n_chains


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


def _chain_major(x, chains, t0=None, t1=None):
    if x is None:
        return None
    y = x if t0 is None else x[t0:t1]
    return np.ascontiguousarray(np.moveaxis(y[:, chains].double().cpu().numpy(), 1, 0))


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(wl, plan, cold, n_chains_sample, w):
    """The fp64 oracle timed on the host on a bounded sample of chains, on the
    work `value` counts, scaled to all chains:
      - without cache hits: the whole request (every pair built token by
        token with explicit T, then the compose and the seams);
      - with cache hits: the pairs of request 0's cold bodies.
    Threads: all host threads, plus one single-thread time on one chain."""
    import oracle
    threads = oracle.max_threads()

    def run(chains, nthreads):
        if cold.all():
            b = wl.requests[0]
            q, k, v, g, beta = (_chain_major(t, chains) for t in (wl.q, wl.k, wl.v, wl.g, wl.beta))
            gam = None if wl.gamma is None else wl.gamma[chains].double().cpu().numpy()
            t0 = time.perf_counter()
            oracle.request_batch(wl.family, b - b[0], w, q, k, v, g, beta, gam, want_pairs=False, nthreads=nthreads)
            return time.perf_counter() - t0, float(b[-1] - b[0])
        # cold bodies of request 0, one oracle pair per (body, chain), chains on host threads
        e0, e1 = int(plan.list_off[0]), int(plan.list_off[1])
        slots = [int(plan.pair_id[e]) for e in range(e0, e1) if cold[int(plan.pair_id[e])]]
        jobs = []
        for sl in slots:
            b, e = int(plan.seg_begin[sl]), int(plan.seg_end[sl])
            ins = [_chain_major(t, chains, b, e) for t in (wl.k, wl.v, wl.g, wl.beta)]
            for ci in range(len(chains)):
                jobs.append([None if t is None else t[ci] for t in ins])
        from concurrent.futures import ThreadPoolExecutor
        t0 = time.perf_counter()
        with ThreadPoolExecutor(max_workers=nthreads) as ex:
            list(ex.map(lambda j: oracle.pair(wl.family, j[0], j[1], j[2], j[3]), jobs))
        return time.perf_counter() - t0, float(sum(plan.seg_end[s] - plan.seg_begin[s] for s in slots))

    chains = list(range(n_chains_sample))
    dt, tok = run(chains, threads)
    dt1, _ = run([0], 1)
    what = ("full {}-token request (all pairs + compose + seams)".format(int(tok)) if cold.all() else
            "the cold bodies of request 0 ({} tokens, their pairs)".format(int(tok)))
    return {"value": tok * n_chains_sample / (wl.n_chains * dt), "unit": "tokens/s", "cores": threads,
            "kind": "oracle", "cpu_model": cpu_model(),
            "single_thread_value": tok / (wl.n_chains * dt1),
            "sample": f"{n_chains_sample} of {wl.n_chains} chains, {what}, {dt:.1f} s on {threads} threads "
                      f"(one chain on one thread: {dt1:.1f} s); scaled by chains"}


def workload_text(name, wl, plan, C, d, w, req_tokens, n_build, hits, mode_name, layers=1):
    n_req = len(wl.requests)
    heads = "30 layers x 32 heads" if C == 960 else f"{C} heads"
    req = (f"one {req_tokens}-token request" if n_req == 1 else f"{n_req} requests, {req_tokens} tokens")
    if hits:
        lay = f", per layer, {layers} layers" if layers > 1 else ", one layer"
        return (f"{wl.family} {wl.dtype}: build of {n_build} cold segment bodies + {mode_name} compose with w={w} "
                f"seams over all {plan.n_slots} cached pairs: {C} chains ({heads}), d={d}, {req}{lay}")
    return (f"{wl.family} pair build + {mode_name} compose with w={w} seams: {C} chains ({heads}), d={d}, {req}, "
            f"{plan.n_slots} segments")


def copy_bandwidth(stream, gib=2, reps=5):
    """A plain device-to-device copy of `gib` GiB, timed with events:
    (read + write bytes) / time, the best of `reps`."""
    n = gib * (1 << 30) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    best = 0.0
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        dst.copy_(src)
        b.record(stream)
        b.synchronize()
        best = max(best, 2 * n * 4 / (a.elapsed_time(b) * 1e-3))
    del src, dst
    torch.cuda.empty_cache()
    return best


def roof(bytes_, flops, t, bound=None):
    hbm, mf = bytes_ / t, flops / t
    if bound is None:
        bound = "hbm" if bytes_ / HBM_PEAK >= flops / BF16_PEAK else "mfma"
    r = ({"bound": "hbm", "achieved": hbm / 1e9, "peak": HBM_PEAK / 1e9, "unit": "GB/s", "frac": hbm / HBM_PEAK}
         if bound == "hbm" else
         {"bound": "mfma", "achieved": mf / 1e12, "peak": BF16_PEAK / 1e12, "unit": "TFLOP/s", "frac": mf / BF16_PEAK})
    r.update({"alg_bytes": bytes_, "alg_flops": flops, "mfma_frac_alg": mf / BF16_PEAK, "hbm_frac_alg": hbm / HBM_PEAK})
    return r


def _median_ms(fn, steps, stream):
    fn()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    for e in evs:
        e[0].record(stream)
        fn()
        e[1].record(stream)
    torch.cuda.synchronize()
    return float(np.median([e[0].elapsed_time(e[1]) for e in evs]))


def variant_leg(lay, steps, stream):
    """Times of the variant patches on the layer's shapes, with their HBM
    rooflines: re-rotation reads and writes every pair once; the warm-up
    reads K - 1 + w raw tokens and writes w tokens of q, k, v per window."""
    wl, plan = lay.wl, lay.plan
    d, C, w, K = wl.dk, wl.n_chains, lay.w, 4
    res = {}
    in_bytes = 2 if wl.dtype == "bf16" else 4
    if wl.family not in ("gla", "kda"):
        te = hy.hypic_t_elems(wl.family, d)
        Tr, Sr = torch.empty_like(lay.T), torch.empty_like(lay.S)
        ident = torch.arange(plan.n_slots, dtype=torch.int32, device="cuda")
        offs = torch.from_numpy(plan.seg_begin).cuda()
        ms = _median_ms(lambda: hy.hypic_rerotate(lay.L, plan.n_slots, ident, offs, 10000.0, lay.T, lay.S, Tr, Sr,
                                                  stream=stream), steps, stream)
        byts = 2.0 * plan.n_slots * C * (te + d * d) * 4
        res["rerotate"] = {"ms": ms, "pairs": plan.n_slots * C,
                           "roofline": roof(byts, 0.0, ms * 1e-3, "hbm") | {"kernel": "k_rerotate"}}
        del Tr, Sr
    seams = plan.seam_begin[plan.seam_begin >= 0]
    if len(seams):
        ns = len(seams)
        outs = [torch.empty(ns, w, C, d, dtype=wl.k.dtype, device="cuda") for _ in range(3)]
        taps = torch.randn(3, C, d, K, device="cuda") / K
        sb = torch.from_numpy(seams).cuda()
        raw = hy.tokens(q=wl.q, k=wl.k, v=wl.v)
        ms = _median_ms(lambda: hy.hypic_conv_warmup(lay.L, raw, taps, K, 1, ns, sb, w, *outs, stream=stream),
                        steps, stream)
        byts = ns * C * 3.0 * d * in_bytes * (K - 1 + 2 * w) + 3 * C * d * K * 4
        res["conv_warmup"] = {"ms": ms, "windows": ns * C, "taps": K,
                              "roofline": roof(byts, 0.0, ms * 1e-3, "hbm") | {"kernel": "k_conv_warmup"}}
    return res


class Layer:
    """One layer's inputs, plan and buffers on the GPU, and the timed step."""

    def __init__(self, config, layer, compose, stream):
        dev = "cuda"
        self.wl = wl = workloads.config(config, device=dev, layer=layer)
        self.w = w = wl.w
        self.plan = plan = request_plan(wl.requests, w, slot_order="longest_first")
        d, C = wl.dk, wl.n_chains
        self.stream = stream
        self.L = L = hy.layout(wl.family, wl.dtype, C, d)
        self.x = x = hy.tokens(wl.q, wl.k, wl.v, wl.g, wl.beta, wl.gamma)
        te = hy.hypic_t_elems(wl.family, d)
        self.T = torch.empty(plan.n_slots, C, te, device=dev)
        self.S = torch.empty(plan.n_slots, C, d, d, device=dev)
        sb = torch.from_numpy(plan.seg_begin).to(dev)
        se = torch.from_numpy(plan.seg_end).to(dev)
        self.lo = torch.from_numpy(plan.list_off).to(dev)
        self.pid = torch.from_numpy(plan.pair_id).to(dev)
        self.seam = torch.from_numpy(plan.seam_begin).to(dev)
        self.state = torch.zeros(plan.n_req, C, d, d, device=dev)
        self.o = torch.zeros(len(plan.pair_id), w, C, d, device=dev)
        # Workloads with cache hits time the build of the cold bodies only,
        # into their own pair buffers, and compose over the full pair cache,
        # which is built once beforehand (untimed); the others time the build
        # of every segment.
        self.cold = cold = (np.concatenate([c for c in wl.cold])[plan.seg_index] if wl.cold
                            else np.ones(plan.n_slots, bool))  # per slot
        self.hits = not cold.all()
        if compose == "auto":
            n_cu = torch.cuda.get_device_properties(dev).multi_processor_count
            # with too few chains to fill the GPU the tree's parallel blocks pay
            # from lists of 8 entries: 32 entries on 16 GLA chains (0.20 ms against
            # 0.44), 8 entries on 8 RetNet chains (0.042 ms against 0.048)
            self.mode = hy.TREE if self.hits or (plan.n_req * C < n_cu and plan.max_list_len >= 8) else hy.SEQ
        else:
            self.mode = hy.TREE if compose == "tree" else hy.SEQ
        if self.hits:
            hy.hypic_segment_build(L, x, plan.n_slots, sb, se, plan.max_seg_len, self.T, self.S, stream=stream)
            idx = np.nonzero(cold)[0]
            self.bsb = torch.from_numpy(plan.seg_begin[idx]).to(dev)
            self.bse = torch.from_numpy(plan.seg_end[idx]).to(dev)
            self.n_build = len(idx)
            self.bT = torch.empty(self.n_build, C, te, device=dev)
            self.bS = torch.empty(self.n_build, C, d, d, device=dev)
            self.build_lens = plan.seg_end[idx] - plan.seg_begin[idx]
        else:
            self.bsb, self.bse, self.n_build, self.bT, self.bS = sb, se, plan.n_slots, self.T, self.S
            self.build_lens = plan.seg_end - plan.seg_begin
        self.max_build = int(self.build_lens.max())
        self.nws = hy.hypic_workspace_bytes(L, hy.OP_COMPOSE_TREE, plan.n_req, plan.max_list_len, w)
        self.ws = torch.empty(max(self.nws, 1), dtype=torch.uint8, device=dev)

    def step(self, ev=None, cmode=None):
        cmode = self.mode if cmode is None else cmode
        st, p = self.stream, self.plan
        if ev:
            ev[0].record(st)
        hy.hypic_segment_build(self.L, self.x, self.n_build, self.bsb, self.bse, self.max_build, self.bT, self.bS,
                               stream=st)
        if ev:
            ev[1].record(st)
        self.state.zero_()
        if ev:
            ev[2].record(st)
        tree = cmode == hy.TREE
        hy.hypic_compose(self.L, cmode, p.n_req, p.max_list_len, self.lo, self.pid, p.n_slots, self.T, self.S,
                         self.x, self.seam, self.w, self.state, self.o, ws=self.ws if tree else None,
                         ws_bytes=self.nws if tree else 0, stream=st)
        if ev:
            ev[3].record(st)

    def timed(self, steps, cmode=None, libs=None):
        """Median build and compose times (ms) over `steps` steps; with libs,
        the steps alternate over the libraries and one pair of lists per
        library comes back."""
        libs = libs or [None]
        evs = [[[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)] for _ in libs]
        for i in range(steps):
            for li, lib in enumerate(libs):
                if lib is not None:
                    hy.hypic.use(lib)
                self.step(evs[li][i], cmode)
        torch.cuda.synchronize()
        res = []
        for ev in evs:
            res.append((np.array([e[0].elapsed_time(e[1]) for e in ev]), np.array([e[2].elapsed_time(e[3]) for e in ev])))
        return res


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
                         "request's chains are fewer than the compute units and its list has at least 8 entries "
                         "(latency-bound), else sequential")
    ap.add_argument("--cpu-chains", type=int, default=-1,
                    help="chains in the oracle's CPU-baseline sample (-1: four per host thread, about 13 s of "
                         "host work at the default workload; 0: skip)")
    ap.add_argument("--layers", type=int, default=1,
                    help="layers to run one after another, each on fresh inputs generated untimed (workloads "
                         "with cache hits); the per-layer times and their sum are reported")
    ap.add_argument("--no-prefill", action="store_true", help="skip the fused cold prefill leg")
    ap.add_argument("--ab", default=None, metavar="LIB[,LIB...]",
                    help="other builds of libhypic.so: steps alternate between this one and them in this process")
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
    lib_a = hy.load()
    libs = None
    if args.ab:
        libs = [lib_a] + [hy.hypic.load(os.path.abspath(p), cache=False) for p in args.ab.split(",")]
    stream = torch.cuda.current_stream()
    copy_bw = copy_bandwidth(stream)

    lay = Layer(args.config, 0, args.compose, stream)
    wl, plan, w, mode = lay.wl, lay.plan, lay.w, lay.mode
    d, C = wl.dk, wl.n_chains
    for _ in range(args.warmup):
        lay.step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    (b_ms, c_ms), *ab = lay.timed(args.steps, libs=libs)
    wall = time.perf_counter() - t0
    step_ms = wall * 1e3 / (args.steps * (2 if libs else 1))
    hy.hypic.use(lib_a)
    # the other compose mode on the same lists, for comparison
    alt_mode = hy.SEQ if mode == hy.TREE else hy.TREE
    (_, alt_c), = lay.timed(args.steps, alt_mode)

    in_bytes = 2 if wl.dtype == "bf16" else 4
    req_tokens = int(sum(int(b[-1] - b[0]) for b in wl.requests))
    build_tokens = int(lay.build_lens.sum())
    bf, bb = build_cost(wl.family, lay.build_lens, d, C, in_bytes)
    n_seams = int((plan.seam_begin >= 0).sum())
    cf, cb = compose_cost(wl.family, len(plan.pair_id), n_seams, w, d, C, in_bytes)
    tb, tc = float(np.median(b_ms)) * 1e-3, float(np.median(c_ms)) * 1e-3
    roof_build = roof(bb, bf, tb)
    bk_name, bk_files = build_kernel(wl.family, wl.dtype)
    key = "" if args.config == "c4" else "_" + args.config  # stored counters per workload
    roof_build.update({"traffic": measured_traffic("build" + key, bk_files), "kernel": bk_name,
                       "measured_copy_GBps": copy_bw / 1e9, "frac_of_measured_copy": bb / tb / copy_bw})
    tree = mode == hy.TREE
    ck_name, ck_files = compose_kernel(wl.family, wl.dtype == "bf16", d, tree)
    roof_comp = roof(cb, cf, tc, "hbm")
    roof_comp.update({"traffic": None if tree else measured_traffic("compose" + key, ck_files), "kernel": ck_name,
                      "frac_of_measured_copy": cb / tc / copy_bw})
    # value: request tokens per second of build (all chains); with cache hits
    # only the cold bodies are built, and value counts those tokens
    v_tokens = build_tokens if lay.hits else req_tokens
    out = {
        "metric": METRIC,
        "value": v_tokens / tb,
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
        "config": {"workload": workload_text(args.config, wl, plan, C, d, w, req_tokens, lay.n_build, lay.hits,
                                               "tree" if tree else "seq", args.layers),
                   "chains": C, "d": d, "request_tokens": req_tokens, "segments": plan.n_slots, "w": w,
                   "built_segments": lay.n_build, "built_tokens": build_tokens,
                   "value_tokens": "cold body tokens" if lay.hits else "request tokens (seam tokens included)",
                   "compose_mode": "tree" if tree else "seq", "state_dtype": "f32", "slot_order": "longest_first"},
        "build_ms": float(np.median(b_ms)),
        "build_ms_p10_p90": [float(np.percentile(b_ms, 10)), float(np.percentile(b_ms, 90))],
        "compose_latency_ms": float(np.median(c_ms)),
        "compose_ms_p10_p90": [float(np.percentile(c_ms, 10)), float(np.percentile(c_ms, 90))],
        "chain_tokens_per_s_build": build_tokens * C / tb,
        "roofline": roof_build,
        "roofline_compose": roof_comp,
        "compose_alt": {"mode": "tree" if alt_mode == hy.TREE else "seq", "ms": float(np.median(alt_c))},
        "hbm_copy_measured_GBps": copy_bw / 1e9,
    }
    if libs:
        out["ab"] = {"libs": ["this"] + args.ab.split(","),
                     "build_ms": [float(np.median(b_ms))] + [float(np.median(x[0])) for x in ab],
                     "compose_ms": [float(np.median(c_ms))] + [float(np.median(x[1])) for x in ab]}
    # fused cold prefill of the same bodies (outputs of every body token and the pairs)
    if not args.no_prefill and wl.family in ("deltanet", "gdn") and wl.dtype == "bf16":
        pout = torch.empty(wl.n_tok, C, d, dtype=wl.k.dtype, device="cuda")
        pT, pS = torch.empty_like(lay.bT), torch.empty_like(lay.bS)
        pf = lambda: hy.hypic_segment_prefill(lay.L, lay.x, lay.n_build, lay.bsb, lay.bse, lay.max_build, pT, pS,
                                              pout, stream=stream)
        for _ in range(max(1, args.warmup)):
            pf()
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
        for e in evs:
            e[0].record(stream)
            pf()
            e[1].record(stream)
        torch.cuda.synchronize()
        p_ms = np.array([e[0].elapsed_time(e[1]) for e in evs])
        tp = float(np.median(p_ms)) * 1e-3
        pfl, pby = prefill_cost(wl.family, lay.build_lens, d, C, in_bytes)
        rp = roof(pby, pfl, tp)
        rp.update({"kernel": "k_build_dense_pipe (prefill instantiation)", "traffic": None})
        out["prefill"] = {"ms": float(np.median(p_ms)), "ms_p10_p90": [float(np.percentile(p_ms, 10)),
                                                                        float(np.percentile(p_ms, 90))],
                          "tokens_per_s": v_tokens / tp, "ms_over_build": tp / tb, "roofline": rp}
        if libs:
            # the same prefill alternating over the libraries, step by step
            pab = [[] for _ in libs]
            for _ in range(args.steps):
                for li, lib in enumerate(libs):
                    hy.hypic.use(lib)
                    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
                    ev[0].record(stream)
                    pf()
                    ev[1].record(stream)
                    torch.cuda.synchronize()
                    pab[li].append(ev[0].elapsed_time(ev[1]))
            hy.hypic.use(lib_a)
            out["ab"]["prefill_ms"] = [float(np.median(x)) for x in pab]
        del pout, pT, pS
        torch.cuda.empty_cache()
    # compact pairs (bf16 T^ with a power-of-two scale): the same compose over them
    if wl.family in ("deltanet", "gdn") and wl.dtype == "bf16" and d >= 64 and not tree:
        Tc = torch.empty(plan.n_slots, C, d * d, dtype=torch.bfloat16, device="cuda")
        sc = torch.empty(plan.n_slots, C, device="cuda")
        hy.hypic_pair_compact(lay.L, plan.n_slots, lay.T, Tc, sc, stream=stream)

        def cc():
            lay.state.zero_()
            hy.hypic_compose_compact(lay.L, plan.n_req, plan.max_list_len, lay.lo, lay.pid, plan.n_slots, Tc, sc,
                                     lay.S, lay.x, lay.seam, w, lay.state, lay.o, stream=stream)
        ms = _median_ms(cc, args.steps, stream) - _median_ms(lambda: lay.state.zero_(), args.steps, stream)
        cbc = cb - len(plan.pair_id) * C * d * d * 2.0   # T read in bf16: half its fp32 bytes
        out["compose_compact"] = {"ms": ms, "roofline": roof(cbc, cf, ms * 1e-3, "hbm") |
                                  {"kernel": "k_compose_lean (compact pairs)", "traffic": None}}
        # the compaction itself: T read in fp32, T^ written in bf16, one scale per (slot, chain)
        pc_ms = _median_ms(lambda: hy.hypic_pair_compact(lay.L, plan.n_slots, lay.T, Tc, sc, stream=stream),
                           args.steps, stream)
        pcb = plan.n_slots * C * (d * d * 6.0 + 4.0)
        out["compose_compact"]["pair_compact"] = {"ms": pc_ms, "roofline": roof(pcb, 0.0, pc_ms * 1e-3, "hbm") |
                                                  {"kernel": "k_pair_compact", "traffic": None}}
        del Tc, sc
    # variant patches at this shape: every cached pair re-rotated to its body's
    # absolute offset (rotary embeddings), and the seam windows' convolved
    # q, k, v from raw inputs (short convolution, 4 taps, SiLU)
    if not args.no_prefill:
        out["variants"] = variant_leg(lay, args.steps, stream)
    if args.layers > 1:
        # every further layer on fresh inputs (generated and its pair cache
        # built untimed), then its timed steps; the first layer is the one above
        per_b, per_c = [float(np.median(b_ms))], [float(np.median(c_ms))]
        toks = [build_tokens]
        del lay
        torch.cuda.empty_cache()
        for layer in range(1, args.layers):
            ly = Layer(args.config, layer, args.compose, stream)
            ly.step()
            torch.cuda.synchronize()
            (bl, cl), = ly.timed(max(3, args.steps // 2))
            per_b.append(float(np.median(bl)))
            per_c.append(float(np.median(cl)))
            toks.append(int(ly.build_lens.sum()))
            print(f"layer {layer}: build {per_b[-1]:.3f} ms, compose {per_c[-1]:.3f} ms", file=sys.stderr, flush=True)
            del ly
            torch.cuda.empty_cache()
        out["layers"] = {"n": args.layers, "build_ms": per_b, "compose_ms": per_c,
                         "build_ms_sum": float(np.sum(per_b)), "compose_ms_sum": float(np.sum(per_c)),
                         "total_ms_sum": float(np.sum(per_b) + np.sum(per_c)),
                         "build_tokens_per_s_all_layers": float(np.sum(toks)) / (np.sum(per_b) * 1e-3)}
        lay = None
    if args.cpu_chains != 0:
        import oracle
        n_cpu = 4 * oracle.max_threads() if args.cpu_chains < 0 else args.cpu_chains
        if lay is None:
            lay = Layer(args.config, 0, args.compose, stream)
        out["cpu_baseline"] = cpu_baseline(lay.wl, lay.plan, lay.cold, min(n_cpu, C), w)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
