// Pair build for per-channel decay with delta erasure (KDA), bf16 inputs, on
// gfx950, with the chunk factors formed ahead of the carry.
//
// A_t = (I - beta_t k_t k_t^T) diag(exp(g_t)), g_t in R^dk; the cached pair
// (T_C, S(C|0)) is the one the HYPIC pages cache per segment (codernav.top
// article, section on linear layers).  Chunks of c = 32 tokens in the UT / WY
// form with per-channel cumulative log-decays Gamma_t (chunk local).  With
// K_L rows exp(Gamma_t) * k_t and K_i rows exp(-Gamma_t) * k_t:
//     G   = tril(K_L K_i^T, -1)            (G_ti = sum k_t k_i exp(Gamma_t - Gamma_i))
//     A   = (I + diag(beta) G)^-1 diag(beta)
//     R   = A ([0 | V] - K_L X)
//     X  <- diag(exp(Gamma_c)) (X + K_i^T R)
// on X = [T | S] from [I | 0].  (The last line is the usual
// diag(exp Gamma_c) X + Kt^T R with Kt rows exp(Gamma_c - Gamma_t) * k_t.)
// Every factor except exp(-Gamma_t) is at most 1; that one is bounded by the
// chunk's total decay, whence the range: per-channel log-decay over a chunk
// of 32 tokens above about -80.
//
// Workgroup: 2d/32 carry waves and one solver wave per (segment, chain).
//   carry waves: wave w keeps columns 32w .. 32w+31 of X in MFMA accumulators
//     and carries chunk j; then, one 8-element item per thread, forms chunk
//     j+2's factors from registers (the log-gates scanned across the 32 lanes
//     of a half-wave with DPP, the exponentials, K_L and K_i split hi + lo, V^T,
//     exp(Gamma_c)) and requests chunk j+3's inputs.
//   solver wave: chunk j+1's Gram on the matrix cores, the 32 x 32 unit lower
//     triangular inverse, and A = Inv diag(beta) written pre-split.
// Staged chunk arrays are three buffers deep, A two; one barrier per chunk.
#include "common.h"
#include "kernels.h"

namespace hy {

constexpr int KPC = 32;  // tokens per chunk
constexpr float KP_L2E = 1.4426950408889634f;

template <int D>
struct KpCfg {
    static constexpr int NC = 2 * D / 32;  // carry waves
    static constexpr int NT = (NC + 1) * 64;
    static constexpr int RT = D / 16;
    static constexpr int KB = D / 32;
    static constexpr int LDK = D + 8;    // bf16 row stride of [KPC][D] arrays
    static constexpr int LDV = KPC + 8;  // bf16 row stride of V^T [D][KPC]
    static constexpr int LDA = KPC + 8;  // bf16 row stride of A [KPC][KPC]
    static constexpr int al(int x) { return (x + 15) / 16 * 16; }
    // one stage: K_L hi, lo; K_i hi, lo; V^T; exp(Gamma_c); beta
    static constexpr int sKLh = 0;
    static constexpr int sKLl = sKLh + al(KPC * LDK * 2);
    static constexpr int sKih = sKLl + al(KPC * LDK * 2);
    static constexpr int sKil = sKih + al(KPC * LDK * 2);
    static constexpr int sVT = sKil + al(KPC * LDK * 2);
    static constexpr int sLam = sVT + al(D * LDV * 2);
    static constexpr int sBeta = sLam + al(D * 4);
    static constexpr int STAGE = al(sBeta + KPC * 4);
    // A (hi, lo), two buffers
    static constexpr int offA = 3 * STAGE;
    static constexpr int ABUF = al(2 * KPC * LDA * 2);
    // solver scratch
    static constexpr int LDL = KPC + 4, LDI = KPC + 4;  // 16-byte aligned rows
    static constexpr int offL = offA + 2 * ABUF;
    static constexpr int offInv = offL + al(KPC * LDL * 4);
    static constexpr int total = offInv + al(KPC * LDI * 4);
    static_assert(total <= 160 * 1024, "LDS budget");
    static_assert(KPC * D / 8 == NC * 64, "one 8-element item per carry thread");
};

typedef short s4k __attribute__((ext_vector_type(4)));

// inclusive prefix sum over the 32 lanes of each half-wave: shifts within
// rows of 16, then row 0's total into row 1 and row 2's into row 3
template <int CTRL, int ROWS, bool ZERO>
__device__ __forceinline__ float kp_dpp(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, ROWS, 0xf, ZERO));
}
__device__ __forceinline__ float half_incl_scan(float v) {
    v += kp_dpp<0x111, 0xf, true>(v);   // row_shr:1
    v += kp_dpp<0x112, 0xf, true>(v);   // row_shr:2
    v += kp_dpp<0x114, 0xf, true>(v);   // row_shr:4
    v += kp_dpp<0x118, 0xf, true>(v);   // row_shr:8
    v += kp_dpp<0x142, 0xa, false>(v);  // row_bcast:15 into rows 1, 3
    return v;
}

// keep the compiler from moving LDS accesses across a point where another
// lane of the same wave reads what this one wrote
__device__ __forceinline__ void kp_wave_fence() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <int D>
__global__ void __launch_bounds__((2 * D / 32 + 1) * 64)
k_build_kda_pipe(BuildArgs a) {
    using Cfg = KpCfg<D>;
    constexpr int NC = Cfg::NC, RT = Cfg::RT, KB = Cfg::KB;
    constexpr int LDK = Cfg::LDK, LDV = Cfg::LDV, LDA = Cfg::LDA, LDL = Cfg::LDL, LDI = Cfg::LDI;
    __shared__ __attribute__((aligned(16))) char smem[Cfg::total];
    const int tid = threadIdx.x;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int seg = blockIdx.x / a.n_chains, chain = blockIdx.x % a.n_chains;
    const int dk = a.dk;
    const int64_t b0 = a.seg_begin[seg], n = a.seg_end[seg] - b0;
    const int nch = (int)((n + KPC - 1) / KPC);
    auto stage = [&](int c) -> char * { return smem + (c % 3) * Cfg::STAGE; };
    auto abuf = [&](int c) -> char * { return smem + Cfg::offA + (c & 1) * Cfg::ABUF; };

    // Both roles meet at the same barriers: one after the first chunk is
    // staged (nch > 0), then one per window c = -1 .. nch - 1.
    if (wv == NC) {
        // ---- solver wave: A of chunk c + 1 in window c
        const int lane = tid & 63, r16 = lane & 15, grp = lane >> 4;
        float *sL = reinterpret_cast<float *>(smem + Cfg::offL);
        float *sInv = reinterpret_cast<float *>(smem + Cfg::offInv);
        auto solve = [&](int c) {
            const char *st = stage(c);
            const bf16 *KLh = reinterpret_cast<const bf16 *>(st + Cfg::sKLh);
            const bf16 *KLl = reinterpret_cast<const bf16 *>(st + Cfg::sKLl);
            const bf16 *Kih = reinterpret_cast<const bf16 *>(st + Cfg::sKih);
            const bf16 *Kil = reinterpret_cast<const bf16 *>(st + Cfg::sKil);
            const float *sBeta = reinterpret_cast<const float *>(st + Cfg::sBeta);
            // Gram blocks (0,0), (1,0), (1,1), scaled by beta_t, strictly lower
#pragma unroll
            for (int tile = 0; tile < 3; ++tile) {
                const int mt = tile == 0 ? 0 : 1, nt = tile == 2 ? 1 : 0;
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kb = 0; kb < KB; ++kb) {
                    const bf16x8 ah = lds_cont(KLh, LDK, 16 * mt + r16, 32 * kb, grp);
                    const bf16x8 al = lds_cont(KLl, LDK, 16 * mt + r16, 32 * kb, grp);
                    const bf16x8 bh = lds_cont(Kih, LDK, 16 * nt + r16, 32 * kb, grp);
                    const bf16x8 bl = lds_cont(Kil, LDK, 16 * nt + r16, 32 * kb, grp);
                    acc = mfma(ah, bh, acc);
                    acc = mfma(ah, bl, acc);
                    acc = mfma(al, bh, acc);
                }
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const int t = 16 * mt + 4 * grp + jj, i = 16 * nt + r16;
                    sL[t * LDL + i] = t > i ? sBeta[t] * acc[jj] : 0.f;
                }
            }
            kp_wave_fence();
            // (I + L)^-1: the two diagonal 16 x 16 blocks, one row r16 per lane
            // (block grp): y (I + L_bb) = e_r, swept from the last row up; once
            // y_i is final its multiple of row i of L_bb leaves every y_j,
            // j < i, so the dependent chain is 16 steps, each row read as four
            // vectors one step ahead.  Zeros in the upper right.
            if (grp < 2) {
                const float *Lb = sL + 16 * grp * LDL + 16 * grp;
                float y[16];
#pragma unroll
                for (int j = 0; j < 16; ++j) y[j] = (j == r16) ? 1.f : 0.f;
                f32x4 cur[4], nxt[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) cur[q] = *reinterpret_cast<const f32x4 *>(Lb + 15 * LDL + 4 * q);
#pragma unroll
                for (int i = 15; i > 0; --i) {
#pragma unroll
                    for (int q = 0; 4 * q < i - 1; ++q)
                        nxt[q] = *reinterpret_cast<const f32x4 *>(Lb + (i - 1) * LDL + 4 * q);
#pragma unroll
                    for (int q = 0; 4 * q < i; ++q)
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            if (4 * q + e < i) y[4 * q + e] -= y[i] * cur[q][e];
#pragma unroll
                    for (int q = 0; q < 4; ++q) cur[q] = nxt[q];
                }
                float *Ib = sInv + (16 * grp + r16) * LDI + 16 * grp;
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    *reinterpret_cast<f32x4 *>(Ib + 4 * q) = f32x4{y[4 * q], y[4 * q + 1], y[4 * q + 2], y[4 * q + 3]};
            } else {
                for (int e = lane - 32; e < 256; e += 32) sInv[(e >> 4) * LDI + 16 + (e & 15)] = 0.f;
            }
            kp_wave_fence();
            // Inv_10 = -Inv_11 L_10 Inv_00 on the fp32 matrix cores
            {
                f32x4 P = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s = 0; s < 4; ++s)
                    P = __builtin_amdgcn_mfma_f32_16x16x4f32(sL[(16 + r16) * LDL + 4 * grp + s],
                                                             sInv[(4 * grp + s) * LDI + r16], P, 0, 0, 0);
                f32x4 O = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s = 0; s < 4; ++s)
                    O = __builtin_amdgcn_mfma_f32_16x16x4f32(sInv[(16 + r16) * LDI + 16 + 4 * grp + s], P[s], O, 0,
                                                             0, 0);
                kp_wave_fence();
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) sInv[(16 + 4 * grp + jj) * LDI + r16] = -O[jj];
            }
            kp_wave_fence();
            // A = Inv diag(beta), split, rows t (A operand of R = A B)
            bf16 *Ah = reinterpret_cast<bf16 *>(abuf(c));
            bf16 *Al = Ah + KPC * LDA;
#pragma unroll
            for (int it = 0; it < KPC * KPC / 64; ++it) {
                const int idx = it * 64 + lane, t = idx / KPC, i = idx % KPC;
                bf16 h, l;
                split1(sInv[t * LDI + i] * sBeta[i], h, l);
                Ah[t * LDA + i] = h;
                Al[t * LDA + i] = l;
            }
        };
        if (nch > 0) __syncthreads();
        for (int c = -1; c < nch; ++c) {
            if (c + 1 < nch) solve(c + 1);
            __syncthreads();
        }
        return;
    }

    // ---- carry waves
    const int lane = tid & 63, r16 = lane & 15, grp = lane >> 4;
    const int cbase = wv * 32;
    const bool isS = cbase >= D;
    // this thread's staging item of every chunk: token it_t, features it_i8 .. +7
    const int it_t = tid % KPC, it_i8 = (tid / KPC) * 8;
    const bf16 *kp = reinterpret_cast<const bf16 *>(a.x.k) + (int64_t)chain * a.x.cs;
    const bf16 *vp = reinterpret_cast<const bf16 *>(a.x.v) + (int64_t)chain * a.x.cs;
    const bf16 *gp = reinterpret_cast<const bf16 *>(a.x.g) + (int64_t)chain * a.x.gcs;
    const bf16 *bp = reinterpret_cast<const bf16 *>(a.x.beta) + (int64_t)chain * a.x.bcs;
    bf16x8 kpre, vpre, gpre;
    bf16 bpre = (bf16)0.f;
    auto prefetch = [&](int c) {
        const int64_t c0 = (int64_t)c * KPC;
        const int L = (int)(n - c0 < KPC ? n - c0 : KPC);
        const bool on = it_t < L && it_i8 < dk;
        const int64_t t = b0 + c0 + (on ? it_t : 0);
        const int i8 = on ? it_i8 : 0;
        const bf16x8 k8 = *reinterpret_cast<const bf16x8 *>(kp + t * a.x.ts + i8);
        const bf16x8 v8 = *reinterpret_cast<const bf16x8 *>(vp + t * a.x.ts + i8);
        const bf16x8 g8 = *reinterpret_cast<const bf16x8 *>(gp + t * a.x.gts + i8);
        kpre = on ? k8 : bf16x8{};
        vpre = on ? v8 : bf16x8{};
        gpre = on ? g8 : bf16x8{};
        bpre = (bf16)0.f;
        if (tid < KPC && tid < L) bpre = bp[(b0 + c0 + tid) * a.x.bts];
    };
    // form chunk c's staged arrays from the prefetched registers
    auto stage_chunk = [&](int c) {
        char *st = stage(c);
        bf16 *KLh = reinterpret_cast<bf16 *>(st + Cfg::sKLh);
        bf16 *KLl = reinterpret_cast<bf16 *>(st + Cfg::sKLl);
        bf16 *Kih = reinterpret_cast<bf16 *>(st + Cfg::sKih);
        bf16 *Kil = reinterpret_cast<bf16 *>(st + Cfg::sKil);
        bf16 *VT = reinterpret_cast<bf16 *>(st + Cfg::sVT);
        float *lam = reinterpret_cast<float *>(st + Cfg::sLam);
        float *sBeta = reinterpret_cast<float *>(st + Cfg::sBeta);
        const int ln = lane_fresh();
        const int t = ln & (KPC - 1), i8 = it_i8;  // (it_t == lane % 32)
        float kl[8], ki[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float G = half_incl_scan((float)gpre[e] * KP_L2E);  // log2 units, tokens 0 .. t
            const float kv = (float)kpre[e];
            const float eg = __builtin_amdgcn_exp2f(G);
            kl[e] = kv * eg;
            ki[e] = kv * __builtin_amdgcn_exp2f(-G);
            // the chunk's total decay is the last token's (tokens past a
            // ragged end carry zero log-gates)
            if (t == KPC - 1) lam[i8 + e] = eg;
            VT[(i8 + e) * LDV + t] = vpre[e];
        }
        bf16x8 h, l;
        split8(kl, h, l);
        *reinterpret_cast<bf16x8 *>(KLh + t * LDK + i8) = h;
        *reinterpret_cast<bf16x8 *>(KLl + t * LDK + i8) = l;
        split8(ki, h, l);
        *reinterpret_cast<bf16x8 *>(Kih + t * LDK + i8) = h;
        *reinterpret_cast<bf16x8 *>(Kil + t * LDK + i8) = l;
        if (tid < KPC) sBeta[tid] = (float)bpre;
    };

    f32x4 X[RT][2];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) X[rt][nt][jj] = (16 * rt + 4 * grp + jj == cbase + 16 * nt + r16) ? 1.f : 0.f;

    if (nch > 0) {
        prefetch(0);
        stage_chunk(0);
        if (nch > 1) prefetch(1);
        __syncthreads();
    }
    // The two carry waves of a SIMD take the window's two jobs in opposite
    // orders (T waves carry then stage, S waves stage then carry), so that
    // one wave's staging arithmetic issues beside the other's matrix work.
    // The staging of chunk c + 2 does not depend on the carry of chunk c.
    for (int c = -1; c < nch; ++c) {
        if (isS && c + 2 < nch) {
            __builtin_amdgcn_s_setprio(0);
            stage_chunk(c + 2);
            if (c + 3 < nch) prefetch(c + 3);
        }
        __builtin_amdgcn_sched_barrier(0);
        if (c >= 0) {
            // the carry goes first at issue, the other wave's staging fills
            // in beside it: 3.23 against 3.32 ms for one 512-chain KDA layer
            // in the same calls (the solver wave above the carry: 3.39)
            __builtin_amdgcn_s_setprio(1);
            const char *st = stage(c);
            const bf16 *KLh = reinterpret_cast<const bf16 *>(st + Cfg::sKLh);
            const bf16 *KLl = reinterpret_cast<const bf16 *>(st + Cfg::sKLl);
            const bf16 *Kih = reinterpret_cast<const bf16 *>(st + Cfg::sKih);
            const bf16 *Kil = reinterpret_cast<const bf16 *>(st + Cfg::sKil);
            const bf16 *VT = reinterpret_cast<const bf16 *>(st + Cfg::sVT);
            const float *lam = reinterpret_cast<const float *>(st + Cfg::sLam);
            const bf16 *Ah = reinterpret_cast<const bf16 *>(abuf(c));
            const bf16 *Al = Ah + KPC * LDA;
            // Z = K_L X
            f32x4 Z[2][2];
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                for (int nt = 0; nt < 2; ++nt) Z[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                bf16x8 xh[2], xl[2];
#pragma unroll
                for (int nt = 0; nt < 2; ++nt) {
                    float xv[8];
                    acc_to_perm(X[2 * kb][nt], X[2 * kb + 1][nt], xv);
                    split8(xv, xh[nt], xl[nt]);
                }
#pragma unroll
                for (int mt = 0; mt < 2; ++mt) {
                    const bf16x8 ah = lds_perm(KLh, LDK, 16 * mt + r16, 32 * kb, grp);
                    const bf16x8 al = lds_perm(KLl, LDK, 16 * mt + r16, 32 * kb, grp);
#pragma unroll
                    for (int nt = 0; nt < 2; ++nt) {
                        Z[mt][nt] = mfma(ah, xh[nt], Z[mt][nt]);
                        Z[mt][nt] = mfma(ah, xl[nt], Z[mt][nt]);
                        Z[mt][nt] = mfma(al, xh[nt], Z[mt][nt]);
                    }
                }
            }
            // R = A ([0 | V] - Z), B operand split
            f32x4 R[2][2];
            {
                bf16x8 bh[2], bl[2];
#pragma unroll
                for (int nt = 0; nt < 2; ++nt) {
                    float bv[8];
                    acc_to_perm(Z[0][nt], Z[1][nt], bv);
                    if (isS) {
                        const bf16x8 v8 = lds_perm(VT, LDV, cbase - D + 16 * nt + r16, 0, grp);
#pragma unroll
                        for (int e = 0; e < 8; ++e) bv[e] = (float)v8[e] - bv[e];
                    } else {
#pragma unroll
                        for (int e = 0; e < 8; ++e) bv[e] = -bv[e];
                    }
                    split8(bv, bh[nt], bl[nt]);
                }
#pragma unroll
                for (int mt = 0; mt < 2; ++mt) {
                    const bf16x8 ah = lds_perm(Ah, LDA, 16 * mt + r16, 0, grp);
                    const bf16x8 al = lds_perm(Al, LDA, 16 * mt + r16, 0, grp);
#pragma unroll
                    for (int nt = 0; nt < 2; ++nt) {
                        f32x4 r = mfma(ah, bh[nt], f32x4{0.f, 0.f, 0.f, 0.f});
                        r = mfma(ah, bl[nt], r);
                        R[mt][nt] = mfma(al, bh[nt], r);
                    }
                }
            }
            // X = diag(exp Gamma_c) (X + K_i^T R); K_i^T rows by transpose reads
            {
                bf16x8 rh[2], rl[2];
#pragma unroll
                for (int nt = 0; nt < 2; ++nt) {
                    float rv[8];
                    acc_to_perm(R[0][nt], R[1][nt], rv);
                    split8(rv, rh[nt], rl[nt]);
                }
#pragma unroll
                for (int rt = 0; rt < RT; ++rt) {
                    const bf16x8 kh = lds_tr_perm(Kih, LDK, 0, 16 * rt, r16, grp);
                    const bf16x8 kl = lds_tr_perm(Kil, LDK, 0, 16 * rt, r16, grp);
#pragma unroll
                    for (int nt = 0; nt < 2; ++nt) {
                        X[rt][nt] = mfma(kh, rh[nt], X[rt][nt]);
                        X[rt][nt] = mfma(kh, rl[nt], X[rt][nt]);
                        X[rt][nt] = mfma(kl, rh[nt], X[rt][nt]);
                    }
                    const f32x4 lm = *reinterpret_cast<const f32x4 *>(lam + 16 * rt + 4 * grp);
#pragma unroll
                    for (int nt = 0; nt < 2; ++nt) X[rt][nt] *= lm;
                }
            }
        }
        __builtin_amdgcn_sched_barrier(0);
        if (!isS && c + 2 < nch) {
            __builtin_amdgcn_s_setprio(0);
            stage_chunk(c + 2);
            if (c + 3 < nch) prefetch(c + 3);
        }
        __syncthreads();
    }

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

template <int D>
static hipError_t launch_kda_pipe(const BuildArgs &a, int n_seg, hipStream_t st) {
    hipLaunchKernelGGL((k_build_kda_pipe<D>), dim3((unsigned)(n_seg * (int64_t)a.n_chains)), dim3(KpCfg<D>::NT), 0, st,
                       a);
    return hipGetLastError();
}

hipError_t build_kda_pipe(const BuildArgs &a, int D, int n_seg, hipStream_t st) {
    switch (D) {
    case 32: return launch_kda_pipe<32>(a, n_seg, st);
    case 64: return launch_kda_pipe<64>(a, n_seg, st);
    case 128: return launch_kda_pipe<128>(a, n_seg, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace hy
