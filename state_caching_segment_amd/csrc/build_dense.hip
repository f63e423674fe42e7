// Dense-transition pair build (DeltaNet, Gated DeltaNet) for gfx950.
//
// For every (segment, chain) this computes T_C = A_n ... A_1 and S(C|0)
// (HYPIC, codernav.top article, section on linear layers: the pair cached at
// a segment's first prefill).  With A_t = a_t (I - beta_t k_t k_t^T), a_t =
// exp(g_t) (GDN) or 1 (DeltaNet), a chunk of c = 64 tokens is applied at once
// in the UT / WY form (Gamma_t = chunk-local cumulative log-decay):
//     G_ti = (k_t . k_i) exp(Gamma_t - Gamma_i)            for t > i
//     Inv  = (I + diag(beta) tril(G, -1))^-1                (unit lower)
//     X   <- exp(Gamma_c) X + K^T diag(exp(Gamma_c - Gamma)) R,
//     R    = [0 | Inv diag(beta) V] - Inv diag(beta exp(Gamma)) (K X)
// on X = [T | S] (d x 2d), starting from [I | 0].  (R is A([0|V] - K_L X)
// with A = Inv diag(beta) and K_L = diag(exp Gamma) K: the UT transform's W
// and U never need to be formed.)
//
// Mapping: one workgroup per (segment, chain), 2d/32 waves; wave w owns
// columns 32w .. 32w+31 of X for the whole segment and keeps them in MFMA
// accumulators; every product of the carry takes the wave's own columns
// straight from (and back to) its accumulators.  Per chunk the workgroup
// stages K, K^T and V^T in LDS (loaded one chunk ahead into registers),
// forms the Gram matrix on the matrix cores and inverts I + L in 16 x 16
// blocks: diagonal blocks by forward substitution, off-diagonal blocks
//     Inv_ij = -Inv_ii sum_{k=j}^{i-1} L_ik Inv_kj
// by distance from the diagonal on the fp32 matrix cores.
//
// Precision: bf16 inputs use bf16 matrix cores; keys and values are exact in
// bf16, every other operand is split into hi + lo (two or three passes, fp32
// accumulation, fp32 state).  fp32 inputs use the fp32 matrix cores for every
// contraction.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace hy {

template <int D, typename TIN>
struct DenseCfg {
    static constexpr bool F32 = std::is_same<TIN, float>::value;
    static constexpr int ES = F32 ? 4 : 2;  // bytes per LDS operand element
    static constexpr int NW = 2 * D / 32;
    static constexpr int NT = NW * 64;
    static constexpr int RT = D / 16;
    static constexpr int KB = D / 32;
    static constexpr int ITEMS = CH * D / 8 / NT;      // 8-element rows of K (and V) per thread per chunk
    static constexpr int LDK = F32 ? D + 4 : D + 8;    // row stride of [CH][D] operand arrays
    static constexpr int LDT = F32 ? CH + 4 : CH + 8;  // row stride of [D][CH] operand arrays
    static constexpr int LDL = CH + 1;                 // fp32 row stride of L
    static constexpr int LDI = CH + 4;                 // fp32 row stride of Inv
    static constexpr int al(int x) { return (x + 15) / 16 * 16; }
    static constexpr int offK = 0;
    static constexpr int offKT = offK + al(CH * LDK * ES);
    static constexpr int offVT = offKT + al(D * LDT * ES);
    // -Inv diag(beta exp Gamma) (Aw) and Inv diag(beta) (Au) as A operands: hi and lo
    // bf16, or fp32.  Aw reuses L's space: L is dead once the inverse is formed.
    static constexpr int LDA = F32 ? CH + 4 : CH + 8;
    static constexpr int szA = F32 ? CH * LDA * 4 : 2 * CH * LDA * 2;
    static constexpr int offL = offVT + al(D * LDT * ES);
    static constexpr int offAw = offL;
    static constexpr int offInv = offL + al(CH * LDL * 4 > szA ? CH * LDL * 4 : szA);
    static constexpr int offAu = offInv + al(CH * LDI * 4);
    static constexpr int offSc = offAu + al(szA);  // Gamma, beta, exp(Gc-Gamma), beta exp(Gamma), lam
    static constexpr int total = offSc + (4 * CH + 4) * 4;
    static_assert(total <= 160 * 1024, "LDS budget");
    static_assert(ITEMS * NT * 8 == CH * D, "staging split");
};

// Eight raw input elements held in registers between a prefetch and its use.
template <typename TIN>
struct Raw8;
template <>
struct Raw8<bf16> {
    bf16x8 v;
    __device__ void load(const bf16 *p) { v = *reinterpret_cast<const bf16x8 *>(p); }
    __device__ void zero() {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = (bf16)0.f;
    }
    __device__ float get(int e) const { return (float)v[e]; }
};
template <>
struct Raw8<float> {
    f32x4 a, b;
    __device__ void load(const float *p) {
        a = *reinterpret_cast<const f32x4 *>(p);
        b = *reinterpret_cast<const f32x4 *>(p + 4);
    }
    __device__ void zero() { a = b = f32x4{0.f, 0.f, 0.f, 0.f}; }
    __device__ float get(int e) const { return e < 4 ? a[e] : b[e - 4]; }
};

template <int D, int FAM, typename TIN>
__global__ void __launch_bounds__(2 * D / 32 * 64)
k_build_dense(BuildArgs a) {
    using Cfg = DenseCfg<D, TIN>;
    constexpr bool F32 = Cfg::F32;
    using OpT = typename std::conditional<F32, float, bf16>::type;
    constexpr int NW = Cfg::NW, NT = Cfg::NT, RT = Cfg::RT, KB = Cfg::KB, ITEMS = Cfg::ITEMS;
    constexpr int LDK = Cfg::LDK, LDT = Cfg::LDT, LDL = Cfg::LDL, LDI = Cfg::LDI, LDA = Cfg::LDA;
    __shared__ __attribute__((aligned(16))) char smem[Cfg::total];
    OpT *sK = reinterpret_cast<OpT *>(smem + Cfg::offK);
    OpT *sKT = reinterpret_cast<OpT *>(smem + Cfg::offKT);
    OpT *sVT = reinterpret_cast<OpT *>(smem + Cfg::offVT);
    float *sL = reinterpret_cast<float *>(smem + Cfg::offL);
    float *sInv = reinterpret_cast<float *>(smem + Cfg::offInv);
    bf16 *sAwh = reinterpret_cast<bf16 *>(smem + Cfg::offAw), *sAwl = sAwh + CH * LDA;
    bf16 *sAuh = reinterpret_cast<bf16 *>(smem + Cfg::offAu), *sAul = sAuh + CH * LDA;
    float *sAwf = reinterpret_cast<float *>(smem + Cfg::offAw);
    float *sAuf = reinterpret_cast<float *>(smem + Cfg::offAu);
    float *sGam = reinterpret_cast<float *>(smem + Cfg::offSc);
    float *sBeta = sGam + CH;
    float *sEc = sBeta + CH;
    float *sAwS = sEc + CH;
    float *sLam = sAwS + CH;

    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int r16 = lane & 15, grp = lane >> 4;
    const int seg = blockIdx.x / a.n_chains, chain = blockIdx.x % a.n_chains;
    const int dk = a.dk;
    const int64_t b0 = a.seg_begin[seg], n = a.seg_end[seg] - b0;
    const TIN *kp = reinterpret_cast<const TIN *>(a.x.k) + (int64_t)chain * a.x.cs;
    const TIN *vp = reinterpret_cast<const TIN *>(a.x.v) + (int64_t)chain * a.x.cs;
    const TIN *gp = FAM == GDN ? reinterpret_cast<const TIN *>(a.x.g) + (int64_t)chain * a.x.gcs : nullptr;
    const TIN *bp = reinterpret_cast<const TIN *>(a.x.beta) + (int64_t)chain * a.x.bcs;

    const int cbase = wv * 32;
    const bool isS = cbase >= D;
    f32x4 X[RT][2];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj)
                X[rt][nt][jj] = (16 * rt + 4 * grp + jj == cbase + 16 * nt + r16) ? 1.f : 0.f;

    // ---- inputs of the next chunk, prefetched into registers
    Raw8<TIN> kpre[ITEMS], vpre[ITEMS];
    TIN gpre = (TIN)0.f, bpre = (TIN)0.f;
    // per-lane element offsets within a chunk (32-bit; the chunk base is wave-uniform)
    int loff[ITEMS];
#pragma unroll
    for (int it = 0; it < ITEMS; ++it) {
        // a wave covers 64 consecutive tokens of one 8-feature group, so the
        // transposed LDS stores below are contiguous across lanes
        const int item = tid + it * NT;
        loff[it] = (item % CH) * (int)a.x.ts + (item / CH) * 8;
    }
    auto prefetch = [&](int64_t c0) {
        const int L = (int)(n - c0 < CH ? n - c0 : CH);
        const int64_t t0 = b0 + c0;
        const TIN *kc = kp + t0 * a.x.ts, *vc = vp + t0 * a.x.ts;
#pragma unroll
        for (int it = 0; it < ITEMS; ++it) {
            const int item = tid + it * NT;
            const int t = item % CH, i8 = (item / CH) * 8;
            if (t < L && i8 < dk) {
                kpre[it].load(kc + loff[it]);
                vpre[it].load(vc + loff[it]);
            } else {
                kpre[it].zero();
                vpre[it].zero();
            }
        }
        if (wv == 0) {
            gpre = bpre = (TIN)0.f;
            if (lane < L) {
                if (FAM == GDN) gpre = gp[(t0 + lane) * a.x.gts];
                bpre = bp[(t0 + lane) * a.x.bts];
            }
        }
    };
    if (n > 0) prefetch(0);

    for (int64_t c0 = 0; c0 < n; c0 += CH) {
        // ---- stage the chunk (K rows, K^T, V^T) from registers; gate prefix sums
#pragma unroll
        for (int it = 0; it < ITEMS; ++it) {
            const int item = tid + it * NT;
            const int t = item % CH, i8 = (item / CH) * 8;
            if constexpr (F32) {
                *reinterpret_cast<f32x4 *>(sK + t * LDK + i8) = kpre[it].a;
                *reinterpret_cast<f32x4 *>(sK + t * LDK + i8 + 4) = kpre[it].b;
            } else {
                *reinterpret_cast<bf16x8 *>(sK + t * LDK + i8) = kpre[it].v;
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                sKT[(i8 + e) * LDT + t] = (OpT)kpre[it].get(e);
                sVT[(i8 + e) * LDT + t] = (OpT)vpre[it].get(e);
            }
        }
        if (wv == 0) {
            float s = (float)gpre;
            const float bt = (float)bpre;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const float y = __shfl_up(s, off);
                if (lane >= off) s += y;
            }
            const float gc = __shfl(s, 63);
            sGam[lane] = s;
            sBeta[lane] = bt;
            sEc[lane] = expf(gc - s);
            sAwS[lane] = bt * expf(s);
            if (lane == 0) sLam[0] = expf(gc);
        }
        if (c0 + CH < n) prefetch(c0 + CH);
        __syncthreads();

        // ---- Gram of the chunk's keys, scaled into the strictly lower L
        for (int tile = wv; tile < 10; tile += NW) {
            int mt = 0, nt = tile;
            while (nt > mt) { nt -= mt + 1; ++mt; }  // lower-triangular tile (mt >= nt)
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                if constexpr (F32) {
                    float av[8], bv[8];
                    lds_cont_f(sK, LDK, 16 * mt + r16, 32 * kb, grp, av);
                    lds_cont_f(sK, LDK, 16 * nt + r16, 32 * kb, grp, bv);
                    acc = mma_f32(av, bv, acc);
                } else {
                    acc = mfma(lds_cont(sK, LDK, 16 * mt + r16, 32 * kb, grp),
                               lds_cont(sK, LDK, 16 * nt + r16, 32 * kb, grp), acc);
                }
            }
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int t = 16 * mt + 4 * grp + jj, i = 16 * nt + r16;
                float val = 0.f;
                if (t > i) {
                    val = sBeta[t] * acc[jj];
                    if (FAM == GDN) val *= expf(sGam[t] - sGam[i]);
                }
                sL[t * LDL + i] = val;
            }
        }
        __syncthreads();

        // ---- (I + L)^-1: diagonal 16 x 16 blocks by forward substitution
        if (wv == 0) {
            const int bk = grp, c = r16;
            float xr[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float s = (r == c) ? 1.f : 0.f;
#pragma unroll
                for (int j = 0; j < r; ++j) s -= sL[(16 * bk + r) * LDL + 16 * bk + j] * xr[j];
                xr[r] = s;
                __builtin_amdgcn_sched_barrier(0);  // keep each row's L loads next to their use
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) sInv[(16 * bk + r) * LDI + 16 * bk + c] = xr[r];
        } else {
            // blocks above the diagonal are zero
            for (int idx = tid - 64; idx < 6 * 256; idx += NT - 64) {
                const int blk = idx >> 8, e = idx & 255;
                const int bi = blk < 3 ? 0 : (blk < 5 ? 1 : 2);
                const int bj = blk < 3 ? blk + 1 : (blk < 5 ? blk - 1 : 3);
                sInv[(16 * bi + (e >> 4)) * LDI + 16 * bj + (e & 15)] = 0.f;
            }
        }
        __syncthreads();
        // off-diagonal blocks by distance d: P = sum_k L_ik Inv_kj, Inv_ij = -Inv_ii P,
        // each 16 x 16 x 16 product as four v_mfma_f32_16x16x4_f32 (k = 4*grp + s)
        for (int d = 1; d < 4; ++d) {
            for (int blk = wv; blk < 4 - d; blk += NW) {
                const int bi = blk + d, bj = blk;
                f32x4 P = {0.f, 0.f, 0.f, 0.f};
                for (int kb = bj; kb < bi; ++kb) {
#pragma unroll
                    for (int s = 0; s < 4; ++s)
                        P = __builtin_amdgcn_mfma_f32_16x16x4f32(sL[(16 * bi + r16) * LDL + 16 * kb + 4 * grp + s],
                                                                 sInv[(16 * kb + 4 * grp + s) * LDI + 16 * bj + r16],
                                                                 P, 0, 0, 0);
                }
                f32x4 O = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s = 0; s < 4; ++s)
                    O = __builtin_amdgcn_mfma_f32_16x16x4f32(sInv[(16 * bi + r16) * LDI + 16 * bi + 4 * grp + s], P[s],
                                                             O, 0, 0, 0);
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) sInv[(16 * bi + 4 * grp + jj) * LDI + 16 * bj + r16] = -O[jj];
            }
            __syncthreads();
        }
        // A operands of the carry: Aw = -Inv diag(beta exp Gamma), Au = Inv diag(beta)
        for (int idx = tid; idx < CH * CH / 4; idx += NT) {
            const int t = idx / (CH / 4), i4 = (idx % (CH / 4)) * 4;
            const f32x4 iv = *reinterpret_cast<const f32x4 *>(sInv + t * LDI + i4);
            const f32x4 sw = *reinterpret_cast<const f32x4 *>(sAwS + i4);
            const f32x4 su = *reinterpret_cast<const f32x4 *>(sBeta + i4);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float w = -iv[e] * sw[e], u = iv[e] * su[e];
                if constexpr (F32) {
                    sAwf[t * LDA + i4 + e] = w;
                    sAuf[t * LDA + i4 + e] = u;
                } else {
                    bf16 h, l;
                    split1(w, h, l);
                    sAwh[t * LDA + i4 + e] = h;
                    sAwl[t * LDA + i4 + e] = l;
                    split1(u, h, l);
                    sAuh[t * LDA + i4 + e] = h;
                    sAul[t * LDA + i4 + e] = l;
                }
            }
        }
        __syncthreads();

        // ---- carry this wave's 32 columns of X = [T | S] through the chunk
        {
            // Z = K X
            f32x4 Z[4][2];
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                for (int nt = 0; nt < 2; ++nt) Z[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                float xv[2][8];
#pragma unroll
                for (int nt = 0; nt < 2; ++nt) acc_to_perm(X[2 * kb][nt], X[2 * kb + 1][nt], xv[nt]);
                if constexpr (F32) {
#pragma unroll
                    for (int mt = 0; mt < 4; ++mt) {
                        float kf[8];
                        lds_perm_f(sK, LDK, 16 * mt + r16, 32 * kb, grp, kf);
#pragma unroll
                        for (int nt = 0; nt < 2; ++nt) Z[mt][nt] = mma_f32(kf, xv[nt], Z[mt][nt]);
                    }
                } else {
                    bf16x8 xh[2], xl[2];
#pragma unroll
                    for (int nt = 0; nt < 2; ++nt) split8(xv[nt], xh[nt], xl[nt]);
#pragma unroll
                    for (int mt = 0; mt < 4; ++mt) {
                        const bf16x8 kh = lds_perm(sK, LDK, 16 * mt + r16, 32 * kb, grp);
#pragma unroll
                        for (int nt = 0; nt < 2; ++nt) {
                            Z[mt][nt] = mfma(kh, xh[nt], Z[mt][nt]);
                            Z[mt][nt] = mfma(kh, xl[nt], Z[mt][nt]);
                        }
                    }
                }
            }
            // X <- exp(Gamma_c) X + K^T R',  R' = diag(exp(Gamma_c - Gamma)) R,
            // R = [0 | Au V] + Aw Z  (Au = Inv diag(beta), Aw = -Inv diag(beta exp Gamma)),
            // in two halves of 32 token rows so only half of R is live at a time
            const float lam = sLam[0];
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int nt = 0; nt < 2; ++nt) X[rt][nt] *= lam;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                f32x4 R[2][2];
#pragma unroll
                for (int m2 = 0; m2 < 2; ++m2)
#pragma unroll
                    for (int nt = 0; nt < 2; ++nt) R[m2][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    float zv[2][8];
#pragma unroll
                    for (int nt = 0; nt < 2; ++nt) acc_to_perm(Z[2 * kb][nt], Z[2 * kb + 1][nt], zv[nt]);
                    if constexpr (F32) {
#pragma unroll
                        for (int m2 = 0; m2 < 2; ++m2) {
                            const int mt = 2 * h + m2;
                            float aw[8];
                            lds_perm_f(sAwf, LDA, 16 * mt + r16, 32 * kb, grp, aw);
#pragma unroll
                            for (int nt = 0; nt < 2; ++nt) R[m2][nt] = mma_f32(aw, zv[nt], R[m2][nt]);
                            if (isS) {
                                float au[8];
                                lds_perm_f(sAuf, LDA, 16 * mt + r16, 32 * kb, grp, au);
#pragma unroll
                                for (int nt = 0; nt < 2; ++nt) {
                                    float vf[8];
                                    lds_perm_f(sVT, LDT, cbase - D + 16 * nt + r16, 32 * kb, grp, vf);
                                    R[m2][nt] = mma_f32(au, vf, R[m2][nt]);
                                }
                            }
                        }
                    } else {
                        bf16x8 zh[2], zl[2];
#pragma unroll
                        for (int nt = 0; nt < 2; ++nt) split8(zv[nt], zh[nt], zl[nt]);
#pragma unroll
                        for (int m2 = 0; m2 < 2; ++m2) {
                            const int mt = 2 * h + m2;
                            const bf16x8 awh = lds_perm(sAwh, LDA, 16 * mt + r16, 32 * kb, grp);
                            const bf16x8 awl = lds_perm(sAwl, LDA, 16 * mt + r16, 32 * kb, grp);
#pragma unroll
                            for (int nt = 0; nt < 2; ++nt) {
                                R[m2][nt] = mfma(awh, zh[nt], R[m2][nt]);
                                R[m2][nt] = mfma(awh, zl[nt], R[m2][nt]);
                                R[m2][nt] = mfma(awl, zh[nt], R[m2][nt]);
                            }
                            if (isS) {
                                const bf16x8 auh = lds_perm(sAuh, LDA, 16 * mt + r16, 32 * kb, grp);
                                const bf16x8 aul = lds_perm(sAul, LDA, 16 * mt + r16, 32 * kb, grp);
#pragma unroll
                                for (int nt = 0; nt < 2; ++nt) {
                                    const bf16x8 vb = lds_perm(sVT, LDT, cbase - D + 16 * nt + r16, 32 * kb, grp);
                                    R[m2][nt] = mfma(auh, vb, R[m2][nt]);
                                    R[m2][nt] = mfma(aul, vb, R[m2][nt]);
                                }
                            }
                        }
                    }
                }
                float rv[2][8];
#pragma unroll
                for (int m2 = 0; m2 < 2; ++m2) {
                    const f32x4 ec = *reinterpret_cast<const f32x4 *>(sEc + 16 * (2 * h + m2) + 4 * grp);
#pragma unroll
                    for (int nt = 0; nt < 2; ++nt) R[m2][nt] *= ec;
                }
#pragma unroll
                for (int nt = 0; nt < 2; ++nt) acc_to_perm(R[0][nt], R[1][nt], rv[nt]);
                if constexpr (F32) {
#pragma unroll
                    for (int rt = 0; rt < RT; ++rt) {
                        float kf[8];
                        lds_perm_f(sKT, LDT, 16 * rt + r16, 32 * h, grp, kf);
#pragma unroll
                        for (int nt = 0; nt < 2; ++nt) X[rt][nt] = mma_f32(kf, rv[nt], X[rt][nt]);
                    }
                } else {
                    bf16x8 rh[2], rl[2];
#pragma unroll
                    for (int nt = 0; nt < 2; ++nt) split8(rv[nt], rh[nt], rl[nt]);
#pragma unroll
                    for (int rt = 0; rt < RT; ++rt) {
                        const bf16x8 kh = lds_perm(sKT, LDT, 16 * rt + r16, 32 * h, grp);
#pragma unroll
                        for (int nt = 0; nt < 2; ++nt) {
                            X[rt][nt] = mfma(kh, rh[nt], X[rt][nt]);
                            X[rt][nt] = mfma(kh, rl[nt], X[rt][nt]);
                        }
                    }
                }
            }
        }
        __syncthreads();
    }

    // ---- write the pair: T = X[:, :d], S = X[:, d:]
    float *To = a.T + ((int64_t)seg * a.n_chains + chain) * dk * dk;
    float *So = a.S + ((int64_t)seg * a.n_chains + chain) * dk * dk;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int row = 16 * rt + 4 * grp + jj;
                const int col = cbase + 16 * nt + r16 - (isS ? D : 0);
                if (row < dk && col < dk) (isS ? So : To)[row * dk + col] = X[rt][nt][jj];
            }
}

template <int D, int FAM, typename TIN>
static hipError_t launch_dense(const BuildArgs &a, int n_seg, hipStream_t st) {
    const dim3 grid((unsigned)(n_seg * (int64_t)a.n_chains));
    hipLaunchKernelGGL((k_build_dense<D, FAM, TIN>), grid, dim3(DenseCfg<D, TIN>::NT), 0, st, a);
    return hipGetLastError();
}

template <int FAM, typename TIN>
static hipError_t launch_dense_d(const BuildArgs &a, int D, int n_seg, hipStream_t st) {
    switch (D) {
    case 32: return launch_dense<32, FAM, TIN>(a, n_seg, st);
    case 64: return launch_dense<64, FAM, TIN>(a, n_seg, st);
    case 128: return launch_dense<128, FAM, TIN>(a, n_seg, st);
    }
    return hipErrorInvalidValue;
}

hipError_t build_dense(const BuildArgs &a, int family, bool bf16_in, int D, int n_seg, hipStream_t st) {
    if (family == GDN)
        return bf16_in ? launch_dense_d<GDN, bf16>(a, D, n_seg, st) : launch_dense_d<GDN, float>(a, D, n_seg, st);
    if (family == DELTANET)
        return bf16_in ? launch_dense_d<DELTANET, bf16>(a, D, n_seg, st)
                       : launch_dense_d<DELTANET, float>(a, D, n_seg, st);
    return hipErrorInvalidValue;
}

}  // namespace hy
