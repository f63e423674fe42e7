// libhypic C ABI: argument validation, dispatch to the gfx950 kernels,
// status reporting.  Every check that can be made on the host runs before
// the first HIP call, so a rejected call enqueues nothing.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "../../include/hypic.h"
#include "kernels.h"

namespace {

thread_local std::string g_last_error;

int fail(int status, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return status;
}

int ok() {
    g_last_error.clear();
    return HYPIC_OK;
}

constexpr int64_t kMaxTokStride = int64_t(1) << 24;

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

int esize(int dtype) { return dtype == HYPIC_BF16 ? 2 : 4; }

// Padded state size the kernels are instantiated for.
int padded_d(int dk) { return dk <= 32 ? 32 : dk; }

int check_layout(const hypic_layout *L) {
    if (!L) return fail(HYPIC_E_INVALID, "layout is NULL");
    if (L->family < HYPIC_LINEAR || L->family > HYPIC_KDA) return fail(HYPIC_E_INVALID, "unknown family %d", L->family);
    if (L->in_dtype != HYPIC_F32 && L->in_dtype != HYPIC_BF16)
        return fail(HYPIC_E_INVALID, "unknown input dtype %d", L->in_dtype);
    if (L->n_chains < 1) return fail(HYPIC_E_INVALID, "n_chains must be >= 1 (got %d)", L->n_chains);
    if (L->dk != 16 && L->dk != 32 && L->dk != 64 && L->dk != 128)
        return fail(HYPIC_E_INVALID, "dk must be 16, 32, 64 or 128 (got %d)", L->dk);
    if (L->dv != L->dk) return fail(HYPIC_E_UNSUPPORTED, "dv != dk is not supported (dk=%d dv=%d)", L->dk, L->dv);
    return HYPIC_OK;
}

bool needs_g(int f) { return f == HYPIC_MAMBA2 || f == HYPIC_GDN || f == HYPIC_GLA || f == HYPIC_KDA; }
bool needs_beta(int f) { return f == HYPIC_DELTANET || f == HYPIC_GDN || f == HYPIC_KDA; }
bool vec_gate(int f) { return f == HYPIC_GLA || f == HYPIC_KDA; }

// need_q: the op reads q (seam outputs).
int check_tokens(const hypic_layout *L, const hypic_tokens *x, bool need_q) {
    if (!x) return fail(HYPIC_E_INVALID, "token tensors are NULL");
    const int es = esize(L->in_dtype);
    if (!x->k || !x->v) return fail(HYPIC_E_INVALID, "k and v are required");
    if (need_q && !x->q) return fail(HYPIC_E_INVALID, "q is required for seam outputs");
    if (needs_g(L->family) && !x->g) return fail(HYPIC_E_INVALID, "this family needs log-gates g");
    if (needs_beta(L->family) && !x->beta) return fail(HYPIC_E_INVALID, "this family needs beta");
    if (L->family == HYPIC_RETNET && !x->gamma) return fail(HYPIC_E_INVALID, "RetNet needs gamma");
    if (x->chain_stride < L->dk) return fail(HYPIC_E_INVALID, "chain_stride %lld < dk", (long long)x->chain_stride);
    if (x->tok_stride < (int64_t)L->dk) return fail(HYPIC_E_INVALID, "tok_stride %lld < dk", (long long)x->tok_stride);
    if (((x->tok_stride * es) & 15) || ((x->chain_stride * es) & 15))
        return fail(HYPIC_E_INVALID, "q/k/v strides must be multiples of 16 bytes");
    if (!aligned16(x->k) || !aligned16(x->v) || (need_q && !aligned16(x->q)))
        return fail(HYPIC_E_INVALID, "q/k/v must be 16-byte aligned");
    if (needs_g(L->family)) {
        if (x->g_tok_stride < 0 || x->g_chain_stride < 0) return fail(HYPIC_E_INVALID, "negative g stride");
        if (vec_gate(L->family) && (x->g_chain_stride < L->dk && L->n_chains > 1))
            return fail(HYPIC_E_INVALID, "g_chain_stride < dk for a per-channel gate");
    }
    if (needs_beta(L->family) && (x->b_tok_stride < 0 || x->b_chain_stride < 0))
        return fail(HYPIC_E_INVALID, "negative beta stride");
    // token offsets inside a chunk or seam window are 32-bit in the kernels
    if (x->tok_stride > kMaxTokStride || (needs_g(L->family) && x->g_tok_stride > kMaxTokStride) ||
        (needs_beta(L->family) && x->b_tok_stride > kMaxTokStride))
        return fail(HYPIC_E_UNSUPPORTED, "token strides above 2^24 elements are not supported");
    return HYPIC_OK;
}

hy::Tok to_tok(const hypic_tokens *x) {
    hy::Tok t;
    t.q = x->q;
    t.k = x->k;
    t.v = x->v;
    t.g = x->g;
    t.beta = x->beta;
    t.gamma = x->gamma;
    t.ts = x->tok_stride;
    t.cs = x->chain_stride;
    t.gts = x->g_tok_stride;
    t.gcs = x->g_chain_stride;
    t.bts = x->b_tok_stride;
    t.bcs = x->b_chain_stride;
    return t;
}

// HYPIC_DEBUG=1: every call synchronizes its stream after launching, so that
// an error in the kernel's execution is reported by the call that launched
// it, with the launch's name (normally it surfaces at the caller's next
// synchronization, from whichever call that is).
bool debug_on() {
    const char *e = getenv("HYPIC_DEBUG");
    return e && e[0] && strcmp(e, "0") != 0;
}

int launched(hipError_t e, const char *what, hipStream_t st) {
    if (e != hipSuccess) return fail(HYPIC_E_DEVICE, "%s: %s", what, hipGetErrorString(e));
    if (debug_on()) {
        e = hipStreamSynchronize(st);
        if (e == hipSuccess) e = hipGetLastError();
        if (e != hipSuccess) return fail(HYPIC_E_DEVICE, "%s (HYPIC_DEBUG, at the stream synchronization): %s", what,
                                         hipGetErrorString(e));
    }
    return ok();
}

bool dense(int f) { return f == HYPIC_DELTANET || f == HYPIC_GDN || f == HYPIC_KDA; }

// HYPIC_VALIDATE=1: device-resident offsets and slot ids are read back (a
// synchronous copy on the caller's stream) and checked before any launch.
bool validate_on() {
    const char *e = getenv("HYPIC_VALIDATE");
    return e && e[0] == '1';
}

// HYPIC_FAULT_INJECT: "1" or "all" fails every call that would launch, one of
// "build", "compose", "seam", "rerotate", "conv", "compact" only that call, with HYPIC_E_DEVICE after its
// arguments have been validated; nothing is enqueued.  A host-side stand-in
// for a failed launch, so that callers can test their error paths without
// making the GPU fail.
int injected(const char *op) {
    const char *e = getenv("HYPIC_FAULT_INJECT");
    if (!e || !e[0] || !strcmp(e, "0")) return HYPIC_OK;
    if (!strcmp(e, "1") || !strcmp(e, "all") || !strcmp(e, op))
        return fail(HYPIC_E_DEVICE, "%s launch: fault injected (HYPIC_FAULT_INJECT=%s)", op, e);
    return HYPIC_OK;
}

template <typename T>
int read_back(std::vector<T> &h, const T *d, size_t n, hipStream_t st, const char *what) {
    h.resize(n);
    if (n == 0) return HYPIC_OK;
    hipError_t e = hipMemcpyAsync(h.data(), d, n * sizeof(T), hipMemcpyDeviceToHost, st);
    if (e == hipSuccess) e = hipStreamSynchronize(st);
    if (e != hipSuccess) return fail(HYPIC_E_DEVICE, "HYPIC_VALIDATE: reading %s: %s", what, hipGetErrorString(e));
    return HYPIC_OK;
}

int validate_segments(int n_seg, const int64_t *d_b, const int64_t *d_e, int64_t max_len, hipStream_t st) {
    std::vector<int64_t> b, e;
    int rc = read_back(b, d_b, n_seg, st, "d_seg_begin");
    if (!rc) rc = read_back(e, d_e, n_seg, st, "d_seg_end");
    if (rc) return rc;
    for (int s = 0; s < n_seg; ++s) {
        if (b[s] < 0 || e[s] < b[s])
            return fail(HYPIC_E_INVALID, "HYPIC_VALIDATE: segment %d has range [%lld, %lld)", s, (long long)b[s],
                        (long long)e[s]);
        if (e[s] - b[s] > max_len)
            return fail(HYPIC_E_INVALID, "HYPIC_VALIDATE: segment %d is %lld tokens, above max_seg_len %lld", s,
                        (long long)(e[s] - b[s]), (long long)max_len);
    }
    return HYPIC_OK;
}

int validate_lists(int n_req, int max_list, const int32_t *d_off, const int32_t *d_pid, int64_t n_slots,
                   const int64_t *d_sb, hipStream_t st) {
    std::vector<int32_t> off, pid;
    std::vector<int64_t> sb;
    int rc = read_back(off, d_off, (size_t)n_req + 1, st, "d_list_off");
    if (rc) return rc;
    if (off[0] < 0) return fail(HYPIC_E_INVALID, "HYPIC_VALIDATE: d_list_off[0] = %d < 0", off[0]);
    for (int r = 0; r < n_req; ++r) {
        const int len = off[r + 1] - off[r];
        if (len < 0 || len > max_list)
            return fail(HYPIC_E_INVALID, "HYPIC_VALIDATE: request %d has %d entries (max_list_len %d)", r, len, max_list);
    }
    const int e0 = off[0], n = off[n_req] - off[0];
    if (n == 0) return HYPIC_OK;
    if (!d_pid) return fail(HYPIC_E_INVALID, "HYPIC_VALIDATE: entries but no d_pair_id");
    if ((rc = read_back(pid, d_pid + e0, n, st, "d_pair_id"))) return rc;
    for (int i = 0; i < n; ++i)
        if (pid[i] < 0 || pid[i] >= n_slots)
            return fail(HYPIC_E_INVALID, "HYPIC_VALIDATE: entry %d names slot %d (n_slots %lld)", e0 + i, pid[i],
                        (long long)n_slots);
    if (d_sb) {
        if ((rc = read_back(sb, d_sb + e0, n, st, "d_seam_begin"))) return rc;
        for (int i = 0; i < n; ++i)
            if (sb[i] < -1)
                return fail(HYPIC_E_INVALID, "HYPIC_VALIDATE: entry %d has seam start %lld", e0 + i, (long long)sb[i]);
    }
    return HYPIC_OK;
}

}  // namespace

extern "C" {

int64_t hypic_t_elems(int32_t family, int32_t dk) {
    switch (family) {
    case HYPIC_LINEAR:
    case HYPIC_RETNET:
    case HYPIC_MAMBA2: return 1;
    case HYPIC_GLA: return dk;
    case HYPIC_DELTANET:
    case HYPIC_GDN:
    case HYPIC_KDA: return (int64_t)dk * dk;
    }
    return 0;
}

}  // extern "C"

namespace {

// Tree-mode blocking, for the MI355X's 256 compute units.  About sqrt(m)
// entries per block (m = list length) balances the parallel block phase
// against the sequential scan over block aggregates.  Two cases shift it:
// - Too few block workgroups to fill the GPU: blocks of about sqrt(m / 2)
//   entries.  A block entry costs more than a scan step, so this pays until
//   the scan grows long.
// - The chains alone (n_req x n_chains) give surplus parallelism: fewer,
//   longer blocks (less aggregate traffic, scan and fix-up work), as long as
//   at least 8 block workgroups remain per compute unit.
// Blocks are then evened out, at most 64 entries.
int tree_block(int max_list, int64_t chains) {
    if (max_list <= 0) return 1;
    constexpr int64_t kCUs = 256;
    int b = 1;
    while (b * b < max_list) ++b;
    int nb = (max_list + b - 1) / b;
    if (chains * nb < kCUs) {
        b = 1;
        while (2 * b * b < max_list) ++b;
        nb = (max_list + b - 1) / b;
    } else {
        while (nb > 1 && chains * (nb - 1) >= 8 * kCUs) --nb;
    }
    b = (max_list + nb - 1) / nb;
    return b > 64 ? 64 : b;
}

struct TreeLayout {
    int B, NB;
    size_t off_aggT, off_aggS, off_sin, off_pvec, off_blk, total;
};

TreeLayout tree_layout(const hypic_layout *L, int n_req, int max_list, int w) {
    TreeLayout t;
    t.B = tree_block(max_list, (int64_t)n_req * L->n_chains);
    t.NB = max_list > 0 ? (max_list + t.B - 1) / t.B : 0;
    auto al = [](size_t x) { return (x + 255) / 256 * 256; };
    const size_t agg = (size_t)n_req * t.NB * L->n_chains * L->dk * L->dk * sizeof(float);
    const size_t pv = w > 0 ? (size_t)n_req * max_list * w * L->n_chains * L->dk * sizeof(float) : 0;
    t.off_aggT = 0;
    t.off_aggS = al(agg);
    t.off_sin = t.off_aggS + al(agg);
    t.off_pvec = t.off_sin + al(agg);
    t.off_blk = t.off_pvec + al(pv);
    t.total = t.off_blk + al(((size_t)n_req * t.NB + 1) * sizeof(int32_t));
    return t;
}

}  // namespace

extern "C" {

size_t hypic_workspace_bytes(const hypic_layout *L, int32_t op, int32_t n_items, int64_t max_len, int32_t w) {
    if (check_layout(L) || n_items < 0 || max_len < 0 || w < 0) return 0;
    if (op == HYPIC_OP_COMPOSE_TREE) return tree_layout(L, n_items, (int)max_len, w).total;
    return 0;
}

int hypic_segment_build(const hypic_layout *L, const hypic_tokens *x, int32_t n_seg, const int64_t *d_seg_begin,
                        const int64_t *d_seg_end, int64_t max_seg_len, float *d_T, float *d_S, void *d_ws,
                        size_t ws_bytes, void *stream) {
    (void)d_ws;
    (void)ws_bytes;
    int rc = check_layout(L);
    if (rc) return rc;
    if ((rc = check_tokens(L, x, false))) return rc;
    if (n_seg < 0) return fail(HYPIC_E_INVALID, "n_seg < 0");
    if (max_seg_len < 0) return fail(HYPIC_E_INVALID, "max_seg_len < 0");
    if (n_seg == 0) return ok();
    if (!d_seg_begin || !d_seg_end || !d_T || !d_S) return fail(HYPIC_E_INVALID, "NULL segment or output pointer");
    if ((int64_t)n_seg * L->n_chains > 0x7fffffff) return fail(HYPIC_E_INVALID, "n_seg * n_chains too large");
    if (L->family == HYPIC_KDA &&
        (!aligned16(x->g) || ((x->g_tok_stride * esize(L->in_dtype)) & 15) || ((x->g_chain_stride * esize(L->in_dtype)) & 15)))
        return fail(HYPIC_E_INVALID, "KDA log-gate rows must be 16-byte aligned");
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    if (validate_on() && (rc = validate_segments(n_seg, d_seg_begin, d_seg_end, max_seg_len, st))) return rc;
    if ((rc = injected("build"))) return rc;
    hy::BuildArgs a{};
    a.x = to_tok(x);
    a.n_chains = L->n_chains;
    a.dk = L->dk;
    a.seg_begin = d_seg_begin;
    a.seg_end = d_seg_end;
    a.T = d_T;
    a.S = d_S;
    const int D = padded_d(L->dk);
    const bool bf = L->in_dtype == HYPIC_BF16;
    if (L->family == HYPIC_KDA)
        return launched(bf ? hy::build_kda_pipe(a, D, n_seg, st) : hy::build_kda(a, bf, D, n_seg, st),
                        "KDA build launch", st);
    if (dense(L->family)) {
        if (bf) return launched(hy::build_dense_pipe(a, L->family, D, n_seg, st), "dense build launch", st);
        return launched(hy::build_dense(a, L->family, bf, D, n_seg, st), "dense build launch", st);
    }
    return launched(hy::build_diag(a, L->family, bf, D, n_seg, st), "diagonal build launch", st);
}

}  // extern "C"

namespace {

// hypic_compose; lib_ws: the tree's workspace is the library's own (d_ws and
// ws_bytes unused), whose address is taken only once a launch is due.
int compose_call(const hypic_layout *L, int32_t mode, int32_t n_req, int32_t max_list_len, const int32_t *d_list_off,
                 const int32_t *d_pair_id, int64_t n_slots, const float *d_T, const float *d_S,
                 const hypic_tokens *seam, const int64_t *d_seam_begin, int32_t w, float *d_state, float *d_o,
                 float *d_prefix_states, void *d_ws, size_t ws_bytes, bool lib_ws, void *stream) {
    int rc = check_layout(L);
    if (rc) return rc;
    if (mode != HYPIC_SEQ && mode != HYPIC_TREE) return fail(HYPIC_E_INVALID, "unknown mode %d", mode);
    if (n_req < 0 || max_list_len < 0 || n_slots < 0) return fail(HYPIC_E_INVALID, "negative size");
    if (w < 0) return fail(HYPIC_E_INVALID, "w < 0");
    if (n_req == 0) return ok();
    if (!d_list_off || !d_state) return fail(HYPIC_E_INVALID, "NULL list or state pointer");
    if (max_list_len > 0 && (!d_pair_id || !d_T || !d_S)) return fail(HYPIC_E_INVALID, "NULL pair pointer");
    if ((int64_t)n_req * L->n_chains > 0x7fffffff) return fail(HYPIC_E_INVALID, "n_req * n_chains too large");
    const bool has_seam = seam != nullptr && w > 0;
    if (has_seam) {
        if ((rc = check_tokens(L, seam, true))) return rc;
        if (!d_seam_begin || !d_o) return fail(HYPIC_E_INVALID, "seams need d_seam_begin and d_o");
    }
    // (pairs are read 16 bytes at a time; states and outputs are fp32)
    if ((max_list_len > 0 && (!aligned16(d_T) || !aligned16(d_S))) || !aligned4(d_state) ||
        (has_seam && !aligned4(d_o)) || !aligned4(d_prefix_states))
        return fail(HYPIC_E_INVALID, "pairs must be 16-byte aligned, states and outputs 4-byte aligned");
    hy::ComposeArgs a{};
    a.x = has_seam ? to_tok(seam) : hy::Tok{};
    a.n_chains = L->n_chains;
    a.dk = L->dk;
    a.w = has_seam ? w : 0;
    a.has_seam = has_seam ? 1 : 0;
    a.list_off = d_list_off;
    a.pair_id = d_pair_id;
    a.T = d_T;
    a.S = d_S;
    a.t_elems = hypic_t_elems(L->family, L->dk);
    a.seam_begin = d_seam_begin;
    a.state = d_state;
    a.o = d_o;
    a.prefix = d_prefix_states;
    const bool bf = L->in_dtype == HYPIC_BF16;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    TreeLayout tl{};
    if (mode == HYPIC_TREE) {
        tl = tree_layout(L, n_req, max_list_len, has_seam ? w : 0);
        if (lib_ws && tl.total > hy::kStaticWorkspaceBytes)
            return fail(HYPIC_E_WORKSPACE,
                        "tree compose of %d requests x %d chains, %d entries, w=%d needs %zu workspace bytes; the "
                        "library's own workspace holds %zu (hypic_compose takes a caller workspace)",
                        n_req, L->n_chains, max_list_len, has_seam ? w : 0, tl.total, hy::kStaticWorkspaceBytes);
        if (!lib_ws && (!d_ws || ws_bytes < tl.total))
            return fail(HYPIC_E_WORKSPACE, "tree compose needs %zu workspace bytes (got %zu)", tl.total, ws_bytes);
    }
    if (validate_on() &&
        (rc = validate_lists(n_req, max_list_len, d_list_off, d_pair_id, n_slots, has_seam ? d_seam_begin : nullptr, st)))
        return rc;
    if ((rc = injected("compose"))) return rc;
    if (mode == HYPIC_SEQ) return launched(hy::compose_seq(a, L->family, bf, padded_d(L->dk), n_req, st), "compose launch", st);
    if (max_list_len == 0) return ok();
    if (lib_ws) {
        const hipError_t e = hy::static_workspace(&d_ws);
        if (e != hipSuccess) return fail(HYPIC_E_DEVICE, "library workspace address: %s", hipGetErrorString(e));
    }
    hy::TreeArgs t;
    t.c = a;
    t.B = tl.B;
    t.NB = tl.NB;
    t.max_list = max_list_len;
    char *base = static_cast<char *>(d_ws);
    t.aggT = reinterpret_cast<float *>(base + tl.off_aggT);
    t.aggS = reinterpret_cast<float *>(base + tl.off_aggS);
    t.sin = reinterpret_cast<float *>(base + tl.off_sin);
    t.pvec = reinterpret_cast<float *>(base + tl.off_pvec);
    t.blk_off = reinterpret_cast<int32_t *>(base + tl.off_blk);
    return launched(hy::compose_tree(t, L->family, bf, padded_d(L->dk), n_req, st), "tree compose launch", st);
}

}  // namespace

extern "C" {

int hypic_segment_prefill(const hypic_layout *L, const hypic_tokens *x, int32_t n_seg, const int64_t *d_seg_begin,
                          const int64_t *d_seg_end, int64_t max_seg_len, float *d_T, float *d_S, void *d_out,
                          int64_t out_tok_stride, int64_t out_chain_stride, void *stream) {
    int rc = check_layout(L);
    if (rc) return rc;
    if ((rc = check_tokens(L, x, true))) return rc;
    if (n_seg < 0) return fail(HYPIC_E_INVALID, "n_seg < 0");
    if (max_seg_len < 0) return fail(HYPIC_E_INVALID, "max_seg_len < 0");
    if (out_chain_stride < L->dv || out_tok_stride < L->dv)
        return fail(HYPIC_E_INVALID, "output strides (%lld, %lld) below dv", (long long)out_tok_stride,
                    (long long)out_chain_stride);
    if (!(L->family == HYPIC_DELTANET || L->family == HYPIC_GDN) || L->in_dtype != HYPIC_BF16)
        return fail(HYPIC_E_UNSUPPORTED, "fused prefill is implemented for DeltaNet and GDN with bf16 inputs");
    if (n_seg == 0) return ok();
    if (!d_seg_begin || !d_seg_end || !d_T || !d_S || !d_out)
        return fail(HYPIC_E_INVALID, "NULL segment or output pointer");
    // (the outputs leave as four-element row pieces)
    if ((out_tok_stride & 3) || (out_chain_stride & 3) || (reinterpret_cast<uintptr_t>(d_out) & 7))
        return fail(HYPIC_E_INVALID, "prefill output: strides must be multiples of 4 elements, d_out 8-byte aligned");
    if ((int64_t)n_seg * L->n_chains > 0x7fffffff) return fail(HYPIC_E_INVALID, "n_seg * n_chains too large");
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    if (validate_on() && (rc = validate_segments(n_seg, d_seg_begin, d_seg_end, max_seg_len, st))) return rc;
    if ((rc = injected("build"))) return rc;
    hy::BuildArgs a{};
    a.x = to_tok(x);
    a.n_chains = L->n_chains;
    a.dk = L->dk;
    a.seg_begin = d_seg_begin;
    a.seg_end = d_seg_end;
    a.T = d_T;
    a.S = d_S;
    a.o = d_out;
    a.ots = out_tok_stride;
    a.ocs = out_chain_stride;
    return launched(hy::build_dense_pipe(a, L->family, padded_d(L->dk), n_seg, st), "prefill launch", st);
}

int hypic_compose(const hypic_layout *L, int32_t mode, int32_t n_req, int32_t max_list_len, const int32_t *d_list_off,
                  const int32_t *d_pair_id, int64_t n_slots, const float *d_T, const float *d_S,
                  const hypic_tokens *seam, const int64_t *d_seam_begin, int32_t w, float *d_state, float *d_o,
                  float *d_prefix_states, void *d_ws, size_t ws_bytes, void *stream) {
    return compose_call(L, mode, n_req, max_list_len, d_list_off, d_pair_id, n_slots, d_T, d_S, seam, d_seam_begin, w,
                        d_state, d_o, d_prefix_states, d_ws, ws_bytes, false, stream);
}

static_assert(hy::kStaticWorkspaceBytes == HYPIC_NOALLOC_WORKSPACE_BYTES, "header and library disagree");

int hypic_compose_tree_noalloc(const hypic_layout *L, int32_t n_req, int32_t max_list_len, const int32_t *d_list_off,
                               const int32_t *d_pair_id, int64_t n_slots, const float *d_T, const float *d_S,
                               const hypic_tokens *seam, const int64_t *d_seam_begin, int32_t w, float *d_state,
                               float *d_o, float *d_prefix_states, void *stream) {
    return compose_call(L, HYPIC_TREE, n_req, max_list_len, d_list_off, d_pair_id, n_slots, d_T, d_S, seam,
                        d_seam_begin, w, d_state, d_o, d_prefix_states, nullptr, 0, true, stream);
}

int hypic_pair_compact(const hypic_layout *L, int32_t n_slots, const float *d_T, void *d_Tc, float *d_Tscale,
                       void *stream) {
    int rc = check_layout(L);
    if (rc) return rc;
    if (!dense(L->family)) return fail(HYPIC_E_UNSUPPORTED, "compact pairs are for dense transitions");
    if (n_slots < 0) return fail(HYPIC_E_INVALID, "n_slots < 0");
    if (n_slots == 0) return ok();
    if (!d_T || !d_Tc || !d_Tscale) return fail(HYPIC_E_INVALID, "NULL pointer");
    if (!aligned16(d_T) || (reinterpret_cast<uintptr_t>(d_Tc) & 7))
        return fail(HYPIC_E_INVALID, "T must be 16-byte and the compact T 8-byte aligned");
    if ((int64_t)n_slots * L->n_chains > 0x7fffffff) return fail(HYPIC_E_INVALID, "n_slots * n_chains too large");
    if ((rc = injected("compact"))) return rc;
    return launched(hy::pair_compact(d_T, static_cast<hy::bf16 *>(d_Tc), d_Tscale, L->dk, (int64_t)n_slots * L->n_chains,
                                     reinterpret_cast<hipStream_t>(stream)),
                    "pair compaction launch", reinterpret_cast<hipStream_t>(stream));
}

int hypic_compose_compact(const hypic_layout *L, int32_t n_req, int32_t max_list_len, const int32_t *d_list_off,
                          const int32_t *d_pair_id, int64_t n_slots, const void *d_Tc, const float *d_Tscale,
                          const float *d_S, const hypic_tokens *seam, const int64_t *d_seam_begin, int32_t w,
                          float *d_state, float *d_o, float *d_prefix_states, void *stream) {
    int rc = check_layout(L);
    if (rc) return rc;
    if (!(L->family == HYPIC_DELTANET || L->family == HYPIC_GDN) || L->in_dtype != HYPIC_BF16 || L->dk < 64)
        return fail(HYPIC_E_UNSUPPORTED, "compact-pair compose is implemented for DeltaNet and GDN, bf16, dk >= 64");
    if (n_req < 0 || max_list_len < 0 || n_slots < 0 || w < 0) return fail(HYPIC_E_INVALID, "negative size");
    if (n_req == 0) return ok();
    if (!d_list_off || !d_state) return fail(HYPIC_E_INVALID, "NULL list or state pointer");
    if (max_list_len > 0 && (!d_pair_id || !d_Tc || !d_Tscale || !d_S))
        return fail(HYPIC_E_INVALID, "NULL pair pointer");
    if ((int64_t)n_req * L->n_chains > 0x7fffffff) return fail(HYPIC_E_INVALID, "n_req * n_chains too large");
    const bool has_seam = seam != nullptr && w > 0;
    if (has_seam) {
        if ((rc = check_tokens(L, seam, true))) return rc;
        if (!d_seam_begin || !d_o) return fail(HYPIC_E_INVALID, "seams need d_seam_begin and d_o");
    }
    if ((max_list_len > 0 && ((reinterpret_cast<uintptr_t>(d_Tc) & 7u) || !aligned16(d_S))) || !aligned4(d_state) ||
        (has_seam && !aligned4(d_o)) || !aligned4(d_prefix_states))
        return fail(HYPIC_E_INVALID, "compact T must be 8-byte, S 16-byte, states and outputs 4-byte aligned");
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    if (validate_on() &&
        (rc = validate_lists(n_req, max_list_len, d_list_off, d_pair_id, n_slots, has_seam ? d_seam_begin : nullptr, st)))
        return rc;
    if ((rc = injected("compose"))) return rc;
    hy::ComposeArgs a{};
    a.x = has_seam ? to_tok(seam) : hy::Tok{};
    a.n_chains = L->n_chains;
    a.dk = L->dk;
    a.w = has_seam ? w : 0;
    a.has_seam = has_seam ? 1 : 0;
    a.list_off = d_list_off;
    a.pair_id = d_pair_id;
    a.T = static_cast<const float *>(d_Tc);
    a.t_scale = d_Tscale;
    a.S = d_S;
    a.t_elems = (int64_t)L->dk * L->dk;
    a.seam_begin = d_seam_begin;
    a.state = d_state;
    a.o = d_o;
    a.prefix = d_prefix_states;
    return launched(hy::compose_seq_compact(a, L->family, L->dk, n_req, st), "compact compose launch", st);
}

int hypic_rerotate(const hypic_layout *L, int32_t n_items, const int32_t *d_slot, const int64_t *d_offset,
                   double rope_base, const float *d_T, const float *d_S, float *d_T_out, float *d_S_out,
                   void *stream) {
    int rc = check_layout(L);
    if (rc) return rc;
    if (n_items < 0) return fail(HYPIC_E_INVALID, "n_items < 0");
    if (!(rope_base > 1.0)) return fail(HYPIC_E_INVALID, "rope_base must be above 1 (got %g)", rope_base);
    if (L->family == HYPIC_GLA || L->family == HYPIC_KDA)
        return fail(HYPIC_E_UNSUPPORTED,
                    "re-rotation is exact only when the decay commutes with the rotation; per-channel gates do "
                    "not (unless both channels of every pair decay alike)");
    if (n_items == 0) return ok();
    if (!d_slot || !d_offset || !d_T || !d_S || !d_T_out || !d_S_out) return fail(HYPIC_E_INVALID, "NULL pointer");
    if (!aligned16(d_T) || !aligned16(d_S) || !aligned16(d_T_out) || !aligned16(d_S_out))
        return fail(HYPIC_E_INVALID, "pairs must be 16-byte aligned");
    if ((int64_t)n_items * L->n_chains > 0x7fffffff) return fail(HYPIC_E_INVALID, "n_items * n_chains too large");
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    if (validate_on()) {
        std::vector<int32_t> sl;
        if ((rc = read_back(sl, d_slot, n_items, st, "d_slot"))) return rc;
        for (int i = 0; i < n_items; ++i)
            if (sl[i] < 0) return fail(HYPIC_E_INVALID, "HYPIC_VALIDATE: item %d names slot %d", i, sl[i]);
    }
    if ((rc = injected("rerotate"))) return rc;
    hy::RerotateArgs a{};
    a.n_chains = L->n_chains;
    a.dk = L->dk;
    a.t_elems = hypic_t_elems(L->family, L->dk);
    a.slot = d_slot;
    a.offset = d_offset;
    a.base = rope_base;
    a.T = d_T;
    a.S = d_S;
    a.T_out = d_T_out;
    a.S_out = d_S_out;
    return launched(hy::rerotate(a, n_items, st), "re-rotation launch", st);
}

int hypic_conv_warmup(const hypic_layout *L, const hypic_tokens *raw, const float *d_taps, int32_t conv_k,
                      int32_t act, int32_t n_items, const int64_t *d_tok_begin, int32_t w, void *d_q_out,
                      void *d_k_out, void *d_v_out, void *stream) {
    int rc = check_layout(L);
    if (rc) return rc;
    if (!raw || !raw->q || !raw->k || !raw->v) return fail(HYPIC_E_INVALID, "raw q, k and v are required");
    if (raw->chain_stride < L->dk || raw->tok_stride < L->dk)
        return fail(HYPIC_E_INVALID, "raw strides below dk");
    if (conv_k < 1 || conv_k > 8) return fail(HYPIC_E_UNSUPPORTED, "conv_k must be 1 .. 8 (got %d)", conv_k);
    if (act != 0 && act != 1) return fail(HYPIC_E_INVALID, "act must be 0 (none) or 1 (SiLU)");
    if (n_items < 0 || w < 0) return fail(HYPIC_E_INVALID, "negative n_items or w");
    if (n_items == 0 || w == 0) return ok();
    if (!d_taps || !d_tok_begin || !d_q_out || !d_k_out || !d_v_out) return fail(HYPIC_E_INVALID, "NULL pointer");
    if ((int64_t)n_items * L->n_chains > 0x7fffffff) return fail(HYPIC_E_INVALID, "n_items * n_chains too large");
    // (the kernel moves four channels per vector load and store)
    const int es = esize(L->in_dtype);
    if (((raw->tok_stride * es) & 15) || ((raw->chain_stride * es) & 15))
        return fail(HYPIC_E_INVALID, "raw q/k/v strides must be multiples of 16 bytes");
    if (!aligned16(raw->q) || !aligned16(raw->k) || !aligned16(raw->v) || !aligned16(d_q_out) ||
        !aligned16(d_k_out) || !aligned16(d_v_out))
        return fail(HYPIC_E_INVALID, "raw q/k/v and the outputs must be 16-byte aligned");
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    if (validate_on()) {
        std::vector<int64_t> tb;
        if ((rc = read_back(tb, d_tok_begin, n_items, st, "d_tok_begin"))) return rc;
        for (int i = 0; i < n_items; ++i)
            if (tb[i] < 0)
                return fail(HYPIC_E_INVALID, "HYPIC_VALIDATE: item %d starts at token %lld", i, (long long)tb[i]);
    }
    if ((rc = injected("conv"))) return rc;
    hy::ConvArgs a{};
    a.x = to_tok(raw);
    a.n_chains = L->n_chains;
    a.n_items = n_items;
    a.dk = L->dk;
    a.w = w;
    a.K = conv_k;
    a.act = act;
    a.tok_begin = d_tok_begin;
    a.taps = d_taps;
    a.q_out = d_q_out;
    a.k_out = d_k_out;
    a.v_out = d_v_out;
    return launched(hy::conv_warmup(a, L->in_dtype == HYPIC_BF16, n_items, st), "conv warm-up launch", st);
}

int hypic_seam_advance(const hypic_layout *L, const hypic_tokens *x, int32_t n_items, const int64_t *d_tok_begin,
                       int32_t w, float *d_state, float *d_o, void *stream) {
    int rc = check_layout(L);
    if (rc) return rc;
    if ((rc = check_tokens(L, x, true))) return rc;
    if (n_items < 0) return fail(HYPIC_E_INVALID, "n_items < 0");
    if (w < 0) return fail(HYPIC_E_INVALID, "w < 0");
    if (n_items == 0 || w == 0) return ok();
    if (!d_tok_begin || !d_state || !d_o) return fail(HYPIC_E_INVALID, "NULL pointer");
    if ((int64_t)n_items * L->n_chains > 0x7fffffff) return fail(HYPIC_E_INVALID, "n_items * n_chains too large");
    if (validate_on()) {
        std::vector<int64_t> tb;
        if ((rc = read_back(tb, d_tok_begin, n_items, reinterpret_cast<hipStream_t>(stream), "d_tok_begin"))) return rc;
        for (int i = 0; i < n_items; ++i)
            if (tb[i] < 0)
                return fail(HYPIC_E_INVALID, "HYPIC_VALIDATE: item %d starts at token %lld", i, (long long)tb[i]);
    }
    if ((rc = injected("seam"))) return rc;
    hy::SeamArgs a;
    a.x = to_tok(x);
    a.n_chains = L->n_chains;
    a.dk = L->dk;
    a.w = w;
    a.tok_begin = d_tok_begin;
    a.state = d_state;
    a.o = d_o;
    return launched(hy::seam_advance(a, L->family, L->in_dtype == HYPIC_BF16, padded_d(L->dk), n_items,
                                     reinterpret_cast<hipStream_t>(stream)),
                    "seam advance launch", reinterpret_cast<hipStream_t>(stream));
}

const char *hypic_status_string(int status) {
    switch (status) {
    case HYPIC_OK: return "ok";
    case HYPIC_E_INVALID: return "invalid argument";
    case HYPIC_E_UNSUPPORTED: return "unsupported";
    case HYPIC_E_WORKSPACE: return "workspace too small";
    case HYPIC_E_DEVICE: return "device error";
    }
    return "unknown status";
}

const char *hypic_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
