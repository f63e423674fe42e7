// Composition of cached pairs and the seam advance, for gfx950.
//
// Composition law (HYPIC, codernav.top article, section on linear layers):
//     S(C1.C2) = T(C2) S(C1) + S(C2)
// Reuse left-multiplies the cached T_C and adds the cached S(C|0).  Before
// each internal segment's pair, the running state is advanced through the
// segment's seam window (its first w tokens, which were not cached) token by
// token, emitting o_t = S_t^T q_t for every seam token (same article, section
// on full-attention layers and seam windows).
//
// Mapping: one workgroup per (request, chain) with d/32 waves; wave w keeps
// columns 32w .. 32w+31 of the running state in MFMA accumulators for the
// whole list.  Dense T (DeltaNet, GDN, KDA): S <- T S + S_slot as a small
// GEMM on the matrix cores, T streamed from HBM straight into A operands and
// the state fed back as the B operand (three-pass bf16 split for bf16 inputs,
// fp32 matrix cores for fp32 inputs; fp32 state either way).
// Diagonal T: a row scale plus add on the vector ALUs.  The seam recurrence
// runs on the vector ALUs over the same accumulator registers; the one
// cross-lane reduction per token (k^T S and q^T S over the state rows) is
// two lane shuffles.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace hy {

constexpr int SEAM_STAGE = 8;  // seam tokens staged in LDS at a time

// LDS staging of up to SEAM_STAGE seam tokens of one chain, fp32.  Decays are
// staged already exponentiated.
template <int D>
struct SeamSmem {
    float q[SEAM_STAGE][D];
    float k[SEAM_STAGE][D];
    float v[SEAM_STAGE][D];
    float a[SEAM_STAGE][D];  // per-row decay exp(g) (GLA, KDA), or a[t][0] (scalar)
    float beta[SEAM_STAGE];
};

template <int D, int FAM, typename TIN>
__device__ void stage_seam(SeamSmem<D> &sm, const Tok &x, int chain, int dk, int64_t tok0, int nt) {
    const int tid = threadIdx.x, nthr = blockDim.x;
    const TIN *qp = reinterpret_cast<const TIN *>(x.q) + (int64_t)chain * x.cs;
    const TIN *kp = reinterpret_cast<const TIN *>(x.k) + (int64_t)chain * x.cs;
    const TIN *vp = reinterpret_cast<const TIN *>(x.v) + (int64_t)chain * x.cs;
    for (int item = tid; item < SEAM_STAGE * D; item += nthr) {
        const int t = item / D, i = item % D;
        float qv = 0.f, kv = 0.f, vv = 0.f, av = 1.f;
        if (t < nt && i < dk) {
            const int64_t off = (tok0 + t) * x.ts + i;
            qv = ldf(qp + off);
            kv = ldf(kp + off);
            vv = ldf(vp + off);
            if (fam_vgate(FAM))
                av = expf(ldf(reinterpret_cast<const TIN *>(x.g) + (int64_t)chain * x.gcs + (tok0 + t) * x.gts + i));
        }
        sm.q[t][i] = qv;
        sm.k[t][i] = kv;
        sm.v[t][i] = vv;
        if (fam_vgate(FAM)) sm.a[t][i] = av;
    }
    if (tid < SEAM_STAGE) {
        const int t = tid;
        float av = 1.f, bv = 1.f;
        if (t < nt) {
            if (fam_sgate(FAM))
                av = expf(ldf(reinterpret_cast<const TIN *>(x.g) + (int64_t)chain * x.gcs + (tok0 + t) * x.gts));
            if (FAM == RETNET) av = x.gamma[chain];
            if (fam_beta(FAM)) bv = ldf(reinterpret_cast<const TIN *>(x.beta) + (int64_t)chain * x.bcs + (tok0 + t) * x.bts);
        }
        if (!fam_vgate(FAM)) sm.a[t][0] = av;
        sm.beta[t] = bv;
    }
}

// Advance the accumulator-resident state columns through nt staged tokens.
// o_row(t) points at the output row (dv floats) of staged token t.
template <int D, int FAM>
__device__ void seam_tokens(f32x4 (&X)[D / 16][2], const SeamSmem<D> &sm, int nt, float *o_first,
                            int64_t o_tok_stride, int cbase, int dv) {
    constexpr int RT = D / 16;
    const int lane = lane_id(), r16 = lane & 15, grp = lane >> 4;
    for (int t = 0; t < nt; ++t) {
        // per-row decay first where the family applies it before the erase (KDA) or alone (GLA)
        if (fam_vgate(FAM)) {
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                const f32x4 a4 = *reinterpret_cast<const f32x4 *>(&sm.a[t][16 * rt + 4 * grp]);
#pragma unroll
                for (int nt2 = 0; nt2 < 2; ++nt2)
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) X[rt][nt2][jj] *= a4[jj];
            }
        }
        const float sa = fam_vgate(FAM) ? 1.f : sm.a[t][0];
        const float bt = sm.beta[t];
        float vcol[2];
#pragma unroll
        for (int nt2 = 0; nt2 < 2; ++nt2) vcol[nt2] = sm.v[t][cbase + 16 * nt2 + r16];
        if (fam_dense(FAM)) {
            // p = k^T S (per column), then S <- a (S - beta k p) + beta k v
            float p[2] = {0.f, 0.f};
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                const f32x4 k4 = *reinterpret_cast<const f32x4 *>(&sm.k[t][16 * rt + 4 * grp]);
#pragma unroll
                for (int nt2 = 0; nt2 < 2; ++nt2)
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) p[nt2] += k4[jj] * X[rt][nt2][jj];
            }
            float coef[2];
#pragma unroll
            for (int nt2 = 0; nt2 < 2; ++nt2) {
                p[nt2] = wave_sum16x(p[nt2]);
                coef[nt2] = bt * (vcol[nt2] - sa * p[nt2]);
            }
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                const f32x4 k4 = *reinterpret_cast<const f32x4 *>(&sm.k[t][16 * rt + 4 * grp]);
#pragma unroll
                for (int nt2 = 0; nt2 < 2; ++nt2)
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) X[rt][nt2][jj] = sa * X[rt][nt2][jj] + k4[jj] * coef[nt2];
            }
        } else {
            // S <- a S + k v^T
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                const f32x4 k4 = *reinterpret_cast<const f32x4 *>(&sm.k[t][16 * rt + 4 * grp]);
#pragma unroll
                for (int nt2 = 0; nt2 < 2; ++nt2)
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) X[rt][nt2][jj] = sa * X[rt][nt2][jj] + k4[jj] * vcol[nt2];
            }
        }
        // o = S^T q (post-update state)
        float o[2] = {0.f, 0.f};
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            const f32x4 q4 = *reinterpret_cast<const f32x4 *>(&sm.q[t][16 * rt + 4 * grp]);
#pragma unroll
            for (int nt2 = 0; nt2 < 2; ++nt2)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) o[nt2] += q4[jj] * X[rt][nt2][jj];
        }
#pragma unroll
        for (int nt2 = 0; nt2 < 2; ++nt2) {
            o[nt2] = wave_sum16x(o[nt2]);
            const int col = cbase + 16 * nt2 + r16;
            if (grp == 0 && col < dv) o_first[t * o_tok_stride + col] = o[nt2];
        }
    }
}

template <int D>
__device__ __forceinline__ void load_state(f32x4 (&X)[D / 16][2], const float *p, int dk, int cbase) {
    const int lane = lane_id(), r16 = lane & 15, grp = lane >> 4;
#pragma unroll
    for (int rt = 0; rt < D / 16; ++rt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int row = 16 * rt + 4 * grp + jj, col = cbase + 16 * nt + r16;
                X[rt][nt][jj] = (row < dk && col < dk) ? p[row * dk + col] : 0.f;
            }
}

template <int D>
__device__ __forceinline__ void store_state(const f32x4 (&X)[D / 16][2], float *p, int dk, int cbase) {
    const int lane = lane_id(), r16 = lane & 15, grp = lane >> 4;
#pragma unroll
    for (int rt = 0; rt < D / 16; ++rt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int row = 16 * rt + 4 * grp + jj, col = cbase + 16 * nt + r16;
                if (row < dk && col < dk) p[row * dk + col] = X[rt][nt][jj];
            }
}

// 8 fp32 of row `row` of a dk x dk row-major matrix at the permuted k subset of
// k block kb, zero outside dk.
__device__ __forceinline__ void glb_perm(const float *M, int dk, int row, int kb, int grp, float (&x)[8]) {
    const int c0 = 32 * kb + 4 * grp, c1 = c0 + 16;
    f32x4 a = {0.f, 0.f, 0.f, 0.f}, b = {0.f, 0.f, 0.f, 0.f};
    if (row < dk) {
        if (c0 < dk) a = *reinterpret_cast<const f32x4 *>(M + row * dk + c0);
        if (c1 < dk) b = *reinterpret_cast<const f32x4 *>(M + row * dk + c1);
    }
    x[0] = a[0]; x[1] = a[1]; x[2] = a[2]; x[3] = a[3];
    x[4] = b[0]; x[5] = b[1]; x[6] = b[2]; x[7] = b[3];
}

template <int D, int FAM, typename TIN>
__global__ void __launch_bounds__(D / 32 * 64)
k_compose_seq(ComposeArgs a) {
    constexpr int RT = D / 16, KB = D / 32;
    __shared__ SeamSmem<D> sm;
    const int lane = lane_id(), wv = threadIdx.x >> 6;
    const int r16 = lane & 15, grp = lane >> 4;
    const int req = blockIdx.x / a.n_chains, chain = blockIdx.x % a.n_chains;
    const int dk = a.dk, cbase = wv * 32;
    float *st = a.state + ((int64_t)req * a.n_chains + chain) * dk * dk;
    f32x4 X[RT][2];
    load_state<D>(X, st, dk, cbase);

    const int e0 = a.list_off[req], e1 = a.list_off[req + 1];
    for (int e = e0; e < e1; ++e) {
        if (a.has_seam) {
            const int64_t sb = a.seam_begin[e];
            if (sb >= 0) {
                for (int s0 = 0; s0 < a.w; s0 += SEAM_STAGE) {
                    const int nt = a.w - s0 < SEAM_STAGE ? a.w - s0 : SEAM_STAGE;
                    __syncthreads();
                    stage_seam<D, FAM, TIN>(sm, a.x, chain, dk, sb + s0, nt);
                    __syncthreads();
                    float *o_first = a.o + (((int64_t)e * a.w + s0) * a.n_chains + chain) * dk;
                    seam_tokens<D, FAM>(X, sm, nt, o_first, (int64_t)a.n_chains * dk, cbase, dk);
                }
            }
        }
        const int64_t slot = a.pair_id[e];
        const float *Tp = a.T + (slot * a.n_chains + chain) * a.t_elems;
        const float *Sp = a.S + (slot * a.n_chains + chain) * dk * dk;
        if (fam_dense(FAM)) {
            // old state as B operands (fp32 fragments), then S <- S_slot + T S_old
            constexpr bool F32 = std::is_same<TIN, float>::value;
            float xv[KB][2][8];
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int nt = 0; nt < 2; ++nt) acc_to_perm(X[2 * kb][nt], X[2 * kb + 1][nt], xv[kb][nt]);
            load_state<D>(X, Sp, dk, cbase);
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int kb = 0; kb < KB; ++kb) {
                    float tv[8];
                    glb_perm(Tp, dk, 16 * rt + r16, kb, grp, tv);
#pragma unroll
                    for (int nt = 0; nt < 2; ++nt) X[rt][nt] = mma_split<F32>(tv, xv[kb][nt], X[rt][nt]);
                }
        } else {
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int nt = 0; nt < 2; ++nt)
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) {
                        const int row = 16 * rt + 4 * grp + jj, col = cbase + 16 * nt + r16;
                        if (row < dk && col < dk) {
                            const float tv = a.t_elems == 1 ? Tp[0] : Tp[row];
                            X[rt][nt][jj] = tv * X[rt][nt][jj] + Sp[row * dk + col];
                        }
                    }
        }
    }
    store_state<D>(X, st, dk, cbase);
}

template <int D, int FAM, typename TIN>
__global__ void __launch_bounds__(D / 32 * 64)
k_seam_advance(SeamArgs a) {
    constexpr int RT = D / 16;
    __shared__ SeamSmem<D> sm;
    const int wv = threadIdx.x >> 6;
    const int item = blockIdx.x / a.n_chains, chain = blockIdx.x % a.n_chains;
    const int dk = a.dk, cbase = wv * 32;
    float *st = a.state + ((int64_t)item * a.n_chains + chain) * dk * dk;
    f32x4 X[RT][2];
    load_state<D>(X, st, dk, cbase);
    const int64_t tb = a.tok_begin[item];
    for (int s0 = 0; s0 < a.w; s0 += SEAM_STAGE) {
        const int nt = a.w - s0 < SEAM_STAGE ? a.w - s0 : SEAM_STAGE;
        __syncthreads();
        stage_seam<D, FAM, TIN>(sm, a.x, chain, dk, tb + s0, nt);
        __syncthreads();
        float *o_first = a.o + (((int64_t)item * a.w + s0) * a.n_chains + chain) * dk;
        seam_tokens<D, FAM>(X, sm, nt, o_first, (int64_t)a.n_chains * dk, cbase, dk);
    }
    store_state<D>(X, st, dk, cbase);
}

template <int D, int FAM, typename TIN>
static hipError_t launch_compose(const ComposeArgs &a, int n_req, hipStream_t st) {
    hipLaunchKernelGGL((k_compose_seq<D, FAM, TIN>), dim3((unsigned)(n_req * (int64_t)a.n_chains)), dim3(D / 32 * 64), 0,
                       st, a);
    return hipGetLastError();
}

template <int D, int FAM, typename TIN>
static hipError_t launch_seam(const SeamArgs &a, int n_items, hipStream_t st) {
    hipLaunchKernelGGL((k_seam_advance<D, FAM, TIN>), dim3((unsigned)(n_items * (int64_t)a.n_chains)), dim3(D / 32 * 64),
                       0, st, a);
    return hipGetLastError();
}

#define HY_DISPATCH_FAMILY(FN, ARGS, D, TIN)                     \
    switch (family) {                                           \
    case LINEAR: return FN<D, LINEAR, TIN> ARGS;                \
    case RETNET: return FN<D, RETNET, TIN> ARGS;                \
    case MAMBA2: return FN<D, MAMBA2, TIN> ARGS;                \
    case GLA: return FN<D, GLA, TIN> ARGS;                      \
    case DELTANET: return FN<D, DELTANET, TIN> ARGS;            \
    case GDN: return FN<D, GDN, TIN> ARGS;                      \
    case KDA: return FN<D, KDA, TIN> ARGS;                      \
    }                                                           \
    return hipErrorInvalidValue;

template <int D, typename TIN>
static hipError_t compose_fam(const ComposeArgs &a, int family, int n_req, hipStream_t st) {
    HY_DISPATCH_FAMILY(launch_compose, (a, n_req, st), D, TIN)
}
template <int D, typename TIN>
static hipError_t seam_fam(const SeamArgs &a, int family, int n_items, hipStream_t st) {
    HY_DISPATCH_FAMILY(launch_seam, (a, n_items, st), D, TIN)
}

hipError_t compose_seq(const ComposeArgs &a, int family, bool bf16_in, int D, int n_req, hipStream_t st) {
    switch (D) {
    case 32: return bf16_in ? compose_fam<32, bf16>(a, family, n_req, st) : compose_fam<32, float>(a, family, n_req, st);
    case 64: return bf16_in ? compose_fam<64, bf16>(a, family, n_req, st) : compose_fam<64, float>(a, family, n_req, st);
    case 128: return bf16_in ? compose_fam<128, bf16>(a, family, n_req, st) : compose_fam<128, float>(a, family, n_req, st);
    }
    return hipErrorInvalidValue;
}

hipError_t seam_advance(const SeamArgs &a, int family, bool bf16_in, int D, int n_items, hipStream_t st) {
    switch (D) {
    case 32: return bf16_in ? seam_fam<32, bf16>(a, family, n_items, st) : seam_fam<32, float>(a, family, n_items, st);
    case 64: return bf16_in ? seam_fam<64, bf16>(a, family, n_items, st) : seam_fam<64, float>(a, family, n_items, st);
    case 128: return bf16_in ? seam_fam<128, bf16>(a, family, n_items, st) : seam_fam<128, float>(a, family, n_items, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace hy
