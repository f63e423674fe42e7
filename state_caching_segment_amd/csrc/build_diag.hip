// Scalar / diagonal-decay pair build (plain linear attention, RetNet, Mamba2,
// GLA) for gfx950.
//
// T stays diagonal: T = exp(sum_t g_t) (a scalar times I, or one value per
// key channel) and S(C|0) = sum_t (exp(Gamma_end - Gamma_t) * k_t) v_t^T
// (HYPIC, codernav.top article, section on linear layers: the segment's
// transition product and zero-initial state).  Tokens are streamed in chunks
// of 64; per chunk the state takes exp(Gamma_c) S + Kt^T V' on the matrix
// cores, where the chunk-local decay is folded into the values (scalar
// decays) or into the keys (per-channel decay, GLA).
//
// Mapping: one workgroup per (segment, chain), d/32 waves, wave w keeps
// columns 32w .. 32w+31 of S in MFMA accumulators across the segment.
#include <type_traits>

#include "common.h"
#include "kernels.h"
#include "compose_common.h"

namespace hy {

template <int D, int FAM, typename TIN>
struct DiagCfg {
    static constexpr bool F32 = std::is_same<TIN, float>::value;  // fp32 inputs: fp32 matrix cores
    // bf16 inputs: the operand that carries the chunk-local decay is not
    // bf16-exact and gets a lo part
    static constexpr bool KLO = !F32 && FAM == GLA;
    static constexpr bool VLO = !F32 && (FAM == RETNET || FAM == MAMBA2);
    static constexpr int ES = F32 ? 4 : 2;
    static constexpr int NW = D / 32;
    static constexpr int NT = NW * 64;
    static constexpr int RT = D / 16;
    static constexpr int LDT = F32 ? CH + 4 : CH + 8;
    static constexpr int offKT = 0;
    static constexpr int szKT = (KLO ? 2 : 1) * D * LDT * ES;
    static constexpr int offVT = offKT + szKT;
    static constexpr int szVT = (VLO ? 2 : 1) * D * LDT * ES;
    static constexpr int offG = offVT + szVT;  // chunk log-gates: [CH] or [CH][D] fp32
    static constexpr int szG = (FAM == GLA ? CH * D : CH) * 4;
    static constexpr int offLam = offG + szG;  // exp(Gamma_c): [1] or [D]
    static constexpr int szLam = D * 4;
    static constexpr int offTot = offLam + szLam;  // running segment log-decay (double)
    static constexpr int szTot = D * 8;
    static constexpr int total = offTot + szTot;
    static_assert(total <= 160 * 1024, "LDS budget");
};

template <int D, int FAM, typename TIN>
__global__ void __launch_bounds__(D / 32 * 64)
k_build_diag(BuildArgs a) {
    using Cfg = DiagCfg<D, FAM, TIN>;
    constexpr int NT = Cfg::NT, RT = Cfg::RT, LDT = Cfg::LDT;
    constexpr bool KLO = Cfg::KLO, VLO = Cfg::VLO, F32 = Cfg::F32;
    using OpT = typename std::conditional<F32, float, bf16>::type;
    __shared__ __attribute__((aligned(16))) char smem[Cfg::total];
    OpT *sKTh = reinterpret_cast<OpT *>(smem + Cfg::offKT);
    OpT *sKTl = sKTh + D * LDT;
    OpT *sVTh = reinterpret_cast<OpT *>(smem + Cfg::offVT);
    OpT *sVTl = sVTh + D * LDT;
    float *sG = reinterpret_cast<float *>(smem + Cfg::offG);
    float *sLam = reinterpret_cast<float *>(smem + Cfg::offLam);
    double *sTot = reinterpret_cast<double *>(smem + Cfg::offTot);

    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int r16 = lane & 15, grp = lane >> 4;
    const int seg = blockIdx.x / a.n_chains, chain = blockIdx.x % a.n_chains;
    const int dk = a.dk;
    const int64_t b0 = a.seg_begin[seg], n = a.seg_end[seg] - b0;
    const TIN *kp = reinterpret_cast<const TIN *>(a.x.k) + (int64_t)chain * a.x.cs;
    const TIN *vp = reinterpret_cast<const TIN *>(a.x.v) + (int64_t)chain * a.x.cs;
    const TIN *gp = (FAM == MAMBA2 || FAM == GLA) ? reinterpret_cast<const TIN *>(a.x.g) + (int64_t)chain * a.x.gcs
                                                  : nullptr;
    const float lgam = FAM == RETNET ? logf(a.x.gamma[chain]) : 0.f;
    const int cbase = wv * 32;

    f32x4 X[RT][2];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) X[rt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (tid < D) sTot[tid] = 0.0;

    for (int64_t c0 = 0; c0 < n; c0 += CH) {
        const int L = (int)(n - c0 < CH ? n - c0 : CH);
        const int64_t t0 = b0 + c0;
        // ---- chunk-local cumulative log-decay
        if (FAM == GLA) {
            for (int i = tid; i < D; i += NT) {
                float s = 0.f;
                for (int t = 0; t < CH; ++t) {
                    if (t < L && i < dk) s += ldf(gp + (t0 + t) * a.x.gts + i);
                    sG[t * D + i] = s;
                }
                sLam[i] = expf(s);
                sTot[i] += (double)s;
            }
        } else if (wv == 0) {
            float gt = 0.f;
            if (lane < L) gt = FAM == MAMBA2 ? ldf(gp + (t0 + lane) * a.x.gts) : (FAM == RETNET ? lgam : 0.f);
            float s = gt;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                float y = __shfl_up(s, off);
                if (lane >= off) s += y;
            }
            sG[lane] = s;
            const float gc = __shfl(s, 63);
            if (lane == 0) {
                sLam[0] = expf(gc);
                sTot[0] += (double)gc;
            }
        }
        __syncthreads();
        // ---- stage K^T and V^T with the decay exp(Gamma_c - Gamma_t) folded in
        for (int item = tid; item < CH * D / 8; item += NT) {
            const int t = item / (D / 8), i8 = (item % (D / 8)) * 8;
            float kv[8], vv[8];
            if (t < L && i8 < dk) {
                load8(kp + (t0 + t) * a.x.ts + i8, kv);
                load8(vp + (t0 + t) * a.x.ts + i8, vv);
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) kv[e] = vv[e] = 0.f;
            }
            if (FAM == GLA) {
#pragma unroll
                for (int e = 0; e < 8; ++e) kv[e] *= expf(sG[(CH - 1) * D + i8 + e] - sG[t * D + i8 + e]);
            } else if (FAM != LINEAR) {
                const float f = expf(sG[CH - 1] - sG[t]);
#pragma unroll
                for (int e = 0; e < 8; ++e) vv[e] *= f;
            }
            if constexpr (F32) {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    sKTh[(i8 + e) * LDT + t] = kv[e];
                    sVTh[(i8 + e) * LDT + t] = vv[e];
                }
            } else {
                bf16x8 h, l;
                split8(kv, h, l);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    sKTh[(i8 + e) * LDT + t] = h[e];
                    if (KLO) sKTl[(i8 + e) * LDT + t] = l[e];
                }
                split8(vv, h, l);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    sVTh[(i8 + e) * LDT + t] = h[e];
                    if (VLO) sVTl[(i8 + e) * LDT + t] = l[e];
                }
            }
        }
        __syncthreads();
        // ---- S <- exp(Gamma_c) S + Kt^T V'
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            f32x4 lam;
            if (FAM == GLA) {
                lam = *reinterpret_cast<const f32x4 *>(sLam + 16 * rt + 4 * grp);
            } else {
                const float l0 = FAM == LINEAR ? 1.f : sLam[0];
                lam = f32x4{l0, l0, l0, l0};
            }
#pragma unroll
            for (int nt = 0; nt < 2; ++nt)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) X[rt][nt][jj] *= lam[jj];
        }
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            if constexpr (F32) {
                float vf[2][8];
#pragma unroll
                for (int nt = 0; nt < 2; ++nt) lds_cont_f(sVTh, LDT, cbase + 16 * nt + r16, 32 * kb, grp, vf[nt]);
#pragma unroll
                for (int rt = 0; rt < RT; ++rt) {
                    float kf[8];
                    lds_cont_f(sKTh, LDT, 16 * rt + r16, 32 * kb, grp, kf);
#pragma unroll
                    for (int nt = 0; nt < 2; ++nt) X[rt][nt] = mma_f32(kf, vf[nt], X[rt][nt]);
                }
            } else {
                bf16x8 vh[2], vl[2];
#pragma unroll
                for (int nt = 0; nt < 2; ++nt) {
                    vh[nt] = lds_cont(sVTh, LDT, cbase + 16 * nt + r16, 32 * kb, grp);
                    if (VLO) vl[nt] = lds_cont(sVTl, LDT, cbase + 16 * nt + r16, 32 * kb, grp);
                }
#pragma unroll
                for (int rt = 0; rt < RT; ++rt) {
                    const bf16x8 kh = lds_cont(sKTh, LDT, 16 * rt + r16, 32 * kb, grp);
                    bf16x8 kl;
                    if (KLO) kl = lds_cont(sKTl, LDT, 16 * rt + r16, 32 * kb, grp);
#pragma unroll
                    for (int nt = 0; nt < 2; ++nt) {
                        X[rt][nt] = mfma(kh, vh[nt], X[rt][nt]);
                        if (VLO) X[rt][nt] = mfma(kh, vl[nt], X[rt][nt]);
                        if (KLO) X[rt][nt] = mfma(kl, vh[nt], X[rt][nt]);
                    }
                }
            }
        }
        __syncthreads();
    }

    float *So = a.S + ((int64_t)seg * a.n_chains + chain) * dk * dk;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int row = 16 * rt + 4 * grp + jj, col = cbase + 16 * nt + r16;
                if (row < dk && col < dk) So[row * dk + col] = X[rt][nt][jj];
            }
    if (FAM == GLA) {
        for (int i = tid; i < dk; i += NT) a.T[((int64_t)seg * a.n_chains + chain) * dk + i] = (float)exp(sTot[i]);
    } else if (tid == 0) {
        float tv = 1.f;
        if (FAM == RETNET) tv = (float)pow((double)a.x.gamma[chain], (double)n);
        if (FAM == MAMBA2) tv = (float)exp(sTot[0]);
        a.T[(int64_t)seg * a.n_chains + chain] = tv;
    }
}

// ---- bf16 inputs: three token slices of a segment in parallel ----------------
//
// The state of a diagonal-decay segment is a sum over its tokens,
//     S = sum_t diag(e^{Gamma_end - Gamma_t}) k_t v_t^T,
// so a segment splits into slices whose partial states combine in order,
//     S = L_2 (L_1 S_0 + S_1) + S_2,
// L_g the slice's decay product (one value per key channel).  One workgroup
// per (segment, chain) holds three slice groups of d/32 waves each (three
// rather than four: 12 waves leave each 168 registers, 16 would leave 128 and
// spill); group g streams its third of the segment's 32-token chunks, a
// contiguous run, last chunk first, so
// the decay from a token to the slice's end is a product of per-token gates
// that is known when the token is staged: within the chunk, a suffix product
// over the lane's 8 tokens and across the 4 lanes holding the chunk's quarters;
// beyond it, D, the running product over the chunks already done.  All these
// factors are at most 1.  The staging lanes (one channel pair and one quarter
// of the chunk's tokens each) write K~ = k * decay (hi and lo bf16) and V rows
// to LDS; each wave then adds K~^T V into its 32 columns of the slice state on
// the matrix cores, through transpose reads.  A group's staging area is
// double-buffered by chunk parity, so one barrier per chunk suffices and one
// wave's staging overlaps another's products.  The groups meet only at the
// end: each chunk's barrier is per group (an LDS arrival counter and a
// bounded wait), so the groups drift apart and one group's staging issues
// beside another's products.  At the end the slice states are combined
// through LDS; T = exp(sum of the segment's log-gates).
template <int D>
struct SliceCfg {
    static constexpr int NW = D / 32;  // waves per slice group (one per 32 columns / 32 channels)
    static constexpr int NG = 3;       // slice groups
    static constexpr int NT = NG * NW * 64;
    static constexpr int CS = 32;      // tokens per chunk
    static constexpr int LDK = D + 8;  // bf16 row stride of K~ and V rows
    static constexpr int al(int x) { return (x + 15) / 16 * 16; }
    static constexpr int gK = 0;
    static constexpr int gKl = gK + al(CS * LDK * 2);
    static constexpr int gV = gKl + al(CS * LDK * 2);
    static constexpr int GRP = al(gV + CS * LDK * 2);
    static constexpr int LDS_ = D + 4;  // fp32 row stride of the combine's S
    static constexpr int cS = 0, cTot = al(D * LDS_ * 4);
    static constexpr int main_ = (2 * NG * GRP > cTot + NG * D * 4) ? 2 * NG * GRP : cTot + NG * D * 4;
    static constexpr int offCnt = al(main_);  // one arrival counter per slice group
    static constexpr int total = offCnt + 16;
    static_assert(total <= 160 * 1024, "LDS budget");
};

template <int D, int FAM>
__global__ void __launch_bounds__(SliceCfg<D>::NT)
k_build_diag_slices(BuildArgs a) {
    using Cfg = SliceCfg<D>;
    constexpr int NW = Cfg::NW, NG = Cfg::NG, RT = D / 16, CS = Cfg::CS, LDK = Cfg::LDK;
    constexpr float L2E = 1.4426950408889634f;
    constexpr bool VG = FAM == GLA;                      // a log-gate per channel
    constexpr bool DEC = FAM != LINEAR;                  // any decay
    __shared__ __attribute__((aligned(16))) char smem[Cfg::total];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int gi = wv / NW, q = wv % NW;  // slice group; column block (carry) = channel block (staging)
    const int r16 = lane & 15, grp = lane >> 4;
    const int seg = blockIdx.x / a.n_chains, chain = blockIdx.x % a.n_chains;
    const int dk = a.dk;
    const int64_t b0 = a.seg_begin[seg], n = a.seg_end[seg] - b0;
    const int nch = (int)((n + CS - 1) / CS);
    // Chunks per slice group.  On each SIMD the three groups' waves compete and
    // the earlier groups' issue first (measured periods about 7.2k, 8.1k and
    // 9.3k cycles per chunk with equal shares), so the groups take about 37 %,
    // 33 % and 30 % of the chunks and finish together.
    static_assert(NG == 3, "chunk shares are set for three slice groups");
    const int n0 = (nch * 37 + 50) / 100, n1 = (nch * 33 + 50) / 100;
    const int per = gi == 0 ? n0 : gi == 1 ? n1 : nch - n0 - n1;
    const int start = gi == 0 ? 0 : gi == 1 ? n0 : n0 + n1;
    // each group's staging area is double-buffered by chunk parity
    char *gb0 = smem + 2 * gi * Cfg::GRP;

    // staging role: channels ch, ch + 1 and tokens 8 tq .. 8 tq + 7 of the chunk
    const int tq = lane >> 4, ch = 32 * q + 2 * (lane & 15);
    const bool ch_ok = ch < dk;
    const bf16 *kb = reinterpret_cast<const bf16 *>(a.x.k) + (int64_t)chain * a.x.cs;
    const bf16 *vb = reinterpret_cast<const bf16 *>(a.x.v) + (int64_t)chain * a.x.cs;
    const bf16 *gb = (VG || FAM == MAMBA2) ? reinterpret_cast<const bf16 *>(a.x.g) + (int64_t)chain * a.x.gcs : nullptr;
    const float lgam = FAM == RETNET ? logf(a.x.gamma[chain]) * L2E : 0.f;
    // Loads go through a buffer view of the chunk's valid tokens, so tokens
    // past the segment's end (and a chunk outside the segment) read as zeros:
    // zero k and v add nothing and a zero log-gate decays nothing.  The token
    // offsets sit in the per-lane offset, which the view's range check covers
    // (the scalar offset is not checked).  Lanes past dk read out of range.
    // Offsets stay below 2^31: token strides are at most 2^24 elements.
    const int ts2 = (int)a.x.ts * 2, gts2 = (int)a.x.gts * 2;
    constexpr int OOR = 0x40000000;  // beyond any chunk view (32 tokens x 2^25 bytes)
    const int voff = ch_ok ? 8 * tq * ts2 + 2 * ch : OOR;
    const int goff = VG ? (ch_ok ? 8 * tq * gts2 + 2 * ch : OOR) : 8 * tq * gts2;

    typedef bf16 bf16x2 __attribute__((ext_vector_type(2)));
    bf16x2 pk[8], pv[8], pg[8];
    bf16 pgs[8];
    int pvalid = 0;  // (RetNet) bit j: token 8 tq + j of the prefetched chunk exists
    // chunk gc of the segment into the prefetch registers
    auto fetch = [&](int gc) {
        const int64_t c0 = (int64_t)gc * CS;
        const int L = (gc >= 0 && gc < nch) ? (int)(n - c0 < CS ? n - c0 : CS) : 0;
        const int64_t tb = b0 + (L > 0 ? c0 : 0);
        const auto rk = buffer_view(kb + tb * a.x.ts, L * ts2);
        const auto rv = buffer_view(vb + tb * a.x.ts, L * ts2);
        if (FAM == RETNET) {
            pvalid = 0;
#pragma unroll
            for (int j = 0; j < 8; ++j)
                if (8 * tq + j < L && ch_ok) pvalid |= 1 << j;
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            pk[j] = __builtin_bit_cast(bf16x2, __builtin_amdgcn_raw_buffer_load_b32(rk, voff + j * ts2, 0, 0));
            pv[j] = __builtin_bit_cast(bf16x2, __builtin_amdgcn_raw_buffer_load_b32(rv, voff + j * ts2, 0, 0));
        }
        if constexpr (VG || FAM == MAMBA2) {
            const auto rg = buffer_view(gb + tb * a.x.gts, L * gts2);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                if (VG)
                    pg[j] = __builtin_bit_cast(bf16x2, __builtin_amdgcn_raw_buffer_load_b32(rg, goff + j * gts2, 0, 0));
                else
                    pgs[j] = __builtin_bit_cast(
                        bf16, (unsigned short)__builtin_amdgcn_raw_buffer_load_b16(rg, goff + j * gts2, 0, 0));
            }
        }
    };

    f32x4 X[RT][2];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) X[rt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    float Dd[2] = {1.f, 1.f};    // decay from the end of the chunk being staged to the slice's end
    float gsum[2] = {0.f, 0.f};  // summed log2-gates of this lane's tokens over the slice

    const int first = start + per - 1;  // chunks run last to first
    int *gcnt = reinterpret_cast<int *>(smem + Cfg::offCnt);
    if (tid < NG) gcnt[tid] = 0;
    __syncthreads();
    if (per > 0) fetch(first);
    for (int c = 0; c < per; ++c) {
        const int gc = first - c;
        char *gb = gb0 + (c & 1) * Cfg::GRP;
        bf16 *sK = reinterpret_cast<bf16 *>(gb + Cfg::gK);
        bf16 *sKl = reinterpret_cast<bf16 *>(gb + Cfg::gKl);
        bf16 *sV = reinterpret_cast<bf16 *>(gb + Cfg::gV);
        // ---- this lane's quarter: product of its 8 tokens' gates per channel
        auto gate = [&](int j, int e) -> float {
            if (FAM == RETNET) return (pvalid & (1 << j)) ? lgam : 0.f;
            return VG ? (float)pg[j][e] * L2E : (float)pgs[j] * L2E;
        };
        float P[2] = {1.f, 1.f};
        if (DEC) {
#pragma unroll
            for (int j = 0; j < 8; ++j)
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    const float g = gate(j, e);
                    gsum[e] += g;
                    P[e] *= __builtin_amdgcn_exp2f(g);
                }
        }
        // the later quarters' products (lanes + 16, + 32, + 48 hold them)
        float E[2] = {1.f, 1.f};
        if (DEC) {
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const float p1 = __shfl_down(P[e], 16), p2 = __shfl_down(P[e], 32), p3 = __shfl_down(P[e], 48);
                E[e] = (tq < 3 ? p1 : 1.f) * (tq < 2 ? p2 : 1.f) * (tq < 1 ? p3 : 1.f) * Dd[e];
            }
        }
        // ---- stage K~ = k * decay (hi, lo) and V rows, last token first:
        // the decay of token j is E times the gates of the tokens after it
        float W[2] = {E[0], E[1]};
#pragma unroll
        for (int j = 7; j >= 0; --j) {
            float kv[2];
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                kv[e] = (float)pk[j][e] * W[e];
                if (DEC) W[e] *= __builtin_amdgcn_exp2f(gate(j, e));
            }
            const bf16 h0 = (bf16)kv[0], h1 = (bf16)kv[1];
            const bf16x2 hh = {h0, h1};
            const bf16x2 ll = {(bf16)(kv[0] - (float)h0), (bf16)(kv[1] - (float)h1)};
            const bf16x2 vv = pv[j];
            const int o = (8 * tq + j) * LDK + ch;
            *reinterpret_cast<bf16x2 *>(sK + o) = hh;
            if (DEC) *reinterpret_cast<bf16x2 *>(sKl + o) = ll;
            *reinterpret_cast<bf16x2 *>(sV + o) = vv;
        }
        // the chunk's whole decay joins D for the chunks before it
        // (quarter 0's W now spans the whole chunk and the chunks after it)
        if (DEC) {
#pragma unroll
            for (int e = 0; e < 2; ++e) Dd[e] = __shfl(W[e], r16);
        }
        // the group's NW waves meet here (the other groups run on): every
        // wave's staging of this chunk is in LDS before any of them reads it
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
        if (lane == 0) atomicAdd(&gcnt[gi], 1);
        {
            const volatile int *vc = gcnt + gi;
            for (int it = 0; it < (1 << 14) && *vc < NW * (c + 1); ++it) __builtin_amdgcn_s_sleep(1);
        }
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
        fetch(gc - 1);
        // ---- carry: S_g += K~^T V for columns 32q .. 32q+31
        bf16x8 vb[2];
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
            const bf16x4 u = lds_tr4(sV, LDK, 4 * grp, 32 * q + 16 * nt, r16);
            const bf16x4 v = lds_tr4(sV, LDK, 16 + 4 * grp, 32 * q + 16 * nt, r16);
            vb[nt] = bf16x8{u[0], u[1], u[2], u[3], v[0], v[1], v[2], v[3]};
        }
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            const bf16x8 kh = lds_tr_perm(sK, LDK, 0, 16 * rt, r16, grp);
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) X[rt][nt] = mfma(kh, vb[nt], X[rt][nt]);
            if (DEC) {
                const bf16x8 kl = lds_tr_perm(sKl, LDK, 0, 16 * rt, r16, grp);
#pragma unroll
                for (int nt = 0; nt < 2; ++nt) X[rt][nt] = mfma(kl, vb[nt], X[rt][nt]);
            }
        }
        // (no barrier here: the next chunk stages into the other buffer, and a
        // wave reaches the next barrier only after this carry)
    }
    __syncthreads();  // every carry is done before the staging areas are reused

    // ---- combine the slice states in order through LDS
    float *cS = reinterpret_cast<float *>(smem + Cfg::cS);
    float *cTot = reinterpret_cast<float *>(smem + Cfg::cTot);  // [NG][D] summed log2-gates
    constexpr int LDS_ = Cfg::LDS_;
    // the slice's log2-gate sum per channel: over the 4 quarters of this channel pair
#pragma unroll
    for (int e = 0; e < 2; ++e) {
        gsum[e] += __shfl_xor(gsum[e], 16);
        gsum[e] += __shfl_xor(gsum[e], 32);
    }
    if (tq == 0) {
        if (VG) {
            cTot[gi * D + ch] = gsum[0];
            cTot[gi * D + ch + 1] = gsum[1];
        } else if (lane == 0 && q == 0) {
            cTot[gi * D] = gsum[0];
        }
    }
    __syncthreads();
    for (int g = 0; g < NG; ++g) {
        if (gi == g) {
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int nt = 0; nt < 2; ++nt)
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) {
                        const int row = 16 * rt + 4 * grp + jj, col = 32 * q + 16 * nt + r16;
                        float v = X[rt][nt][jj];
                        if (g > 0) v += __builtin_amdgcn_exp2f(cTot[g * D + (VG ? row : 0)]) * cS[row * LDS_ + col];
                        X[rt][nt][jj] = v;
                        if (g < NG - 1) cS[row * LDS_ + col] = v;
                    }
        }
        __syncthreads();
    }
    if (gi == NG - 1) {
        float *So = a.S + ((int64_t)seg * a.n_chains + chain) * dk * dk;
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int nt = 0; nt < 2; ++nt)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const int row = 16 * rt + 4 * grp + jj, col = 32 * q + 16 * nt + r16;
                    if (row < dk && col < dk) So[row * dk + col] = X[rt][nt][jj];
                }
    }
    if (gi == 0) {
        const int tq2 = q * 64 + lane;
        if (VG) {
            for (int i = tq2; i < dk; i += NW * 64) {
                float s2 = 0.f;
                for (int g = 0; g < NG; ++g) s2 += cTot[g * D + i];
                a.T[((int64_t)seg * a.n_chains + chain) * dk + i] = __builtin_amdgcn_exp2f(s2);
            }
        } else if (tq2 == 0) {
            float tv = 1.f;
            if (FAM == RETNET) tv = (float)pow((double)a.x.gamma[chain], (double)n);
            if (FAM == MAMBA2) {
                float s2 = 0.f;
                for (int g = 0; g < NG; ++g) s2 += cTot[g * D];
                tv = exp2f(s2);
            }
            a.T[(int64_t)seg * a.n_chains + chain] = tv;
        }
    }
}

template <int D, int FAM>
static hipError_t launch_slices(const BuildArgs &a, int n_seg, hipStream_t st) {
    const dim3 grid((unsigned)(n_seg * (int64_t)a.n_chains));
    hipLaunchKernelGGL((k_build_diag_slices<D, FAM>), grid, dim3(SliceCfg<D>::NT), 0, st, a);
    return hipGetLastError();
}

template <int FAM>
static hipError_t launch_slices_d(const BuildArgs &a, int D, int n_seg, hipStream_t st) {
    switch (D) {
    case 32: return launch_slices<32, FAM>(a, n_seg, st);
    case 64: return launch_slices<64, FAM>(a, n_seg, st);
    case 128: return launch_slices<128, FAM>(a, n_seg, st);
    }
    return hipErrorInvalidValue;
}

template <int D, int FAM, typename TIN>
static hipError_t launch_diag(const BuildArgs &a, int n_seg, hipStream_t st) {
    const dim3 grid((unsigned)(n_seg * (int64_t)a.n_chains));
    hipLaunchKernelGGL((k_build_diag<D, FAM, TIN>), grid, dim3(DiagCfg<D, FAM, TIN>::NT), 0, st, a);
    return hipGetLastError();
}

template <int FAM, typename TIN>
static hipError_t launch_diag_d(const BuildArgs &a, int D, int n_seg, hipStream_t st) {
    switch (D) {
    case 32: return launch_diag<32, FAM, TIN>(a, n_seg, st);
    case 64: return launch_diag<64, FAM, TIN>(a, n_seg, st);
    case 128: return launch_diag<128, FAM, TIN>(a, n_seg, st);
    }
    return hipErrorInvalidValue;
}

template <typename TIN>
static hipError_t diag_by_family(const BuildArgs &a, int family, int D, int n_seg, hipStream_t st) {
    switch (family) {
    case LINEAR: return launch_diag_d<LINEAR, TIN>(a, D, n_seg, st);
    case RETNET: return launch_diag_d<RETNET, TIN>(a, D, n_seg, st);
    case MAMBA2: return launch_diag_d<MAMBA2, TIN>(a, D, n_seg, st);
    case GLA: return launch_diag_d<GLA, TIN>(a, D, n_seg, st);
    }
    return hipErrorInvalidValue;
}

hipError_t build_diag(const BuildArgs &a, int family, bool bf16_in, int D, int n_seg, hipStream_t st) {
    if (!bf16_in) return diag_by_family<float>(a, family, D, n_seg, st);
    switch (family) {
    case LINEAR: return launch_slices_d<LINEAR>(a, D, n_seg, st);
    case RETNET: return launch_slices_d<RETNET>(a, D, n_seg, st);
    case MAMBA2: return launch_slices_d<MAMBA2>(a, D, n_seg, st);
    case GLA: return launch_slices_d<GLA>(a, D, n_seg, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace hy
