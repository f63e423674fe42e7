// Pair build for per-channel decay with delta erasure (KDA) on gfx950.
//
// A_t = (I - beta_t k_t k_t^T) diag(exp(g_t)), g_t in R^dk: the state decays
// channel by channel, then the delta rule erases and writes.  The pair
// (T_C, S(C|0)) is the one the HYPIC pages cache per segment (codernav.top
// article, section on linear layers).  Chunks of c = 32 tokens are applied
// in the UT / WY form with per-channel cumulative log-decays Gamma_t (chunk
// local):
//     G_ti = sum_ch k_t,ch k_i,ch exp(Gamma_t,ch - Gamma_i,ch)      (t > i)
//     A    = (I + diag(beta) tril(G, -1))^-1 diag(beta)
//     X   <- diag(exp(Gamma_c)) X + Kt^T (A ([0 | V] - K_L X))
// with K_L rows exp(Gamma_t) * k_t and Kt rows exp(Gamma_c - Gamma_t) * k_t,
// on X = [T | S] from [I | 0].  The per-channel decay cannot be folded into a
// row scale, so K_L and Kt are formed per chunk (hi + lo bf16, or fp32).  The
// Gram uses a reference token r per 16-token row block (the block's first
// token): its operands are k_t exp(Gamma_t - Gamma_r) and k_i exp(Gamma_r -
// Gamma_i), every exponent at most 0 except within a diagonal 16 x 16 block,
// where it is bounded by the decay over at most 15 tokens.
//
// Mapping as in the DeltaNet / GDN build: one workgroup per (segment, chain),
// 2d/32 waves, wave w keeps columns 32w .. 32w+31 of X in MFMA accumulators.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace hy {

constexpr int KC = 32;  // tokens per chunk
constexpr float L2E = 1.4426950408889634f;  // log2(e): gates are kept in log2 units, exponentials are exp2

template <int D, typename TIN>
struct KdaCfg {
    static constexpr bool F32 = std::is_same<TIN, float>::value;
    static constexpr int ES = F32 ? 4 : 2;
    static constexpr int NS = F32 ? 1 : 2;  // copies of a split operand (hi, lo)
    static constexpr int NW = 2 * D / 32;
    static constexpr int NT = NW * 64;
    static constexpr int RT = D / 16;
    static constexpr int KB = D / 32;
    static constexpr int LDK = F32 ? D + 4 : D + 8;    // [KC][D] operand arrays
    static constexpr int LDT = F32 ? KC + 4 : KC + 8;  // [D][KC] operand arrays
    static constexpr int LDG = D + 4;                  // fp32 [KC][D] log-decays
    static constexpr int LDL = KC + 1;
    static constexpr int LDI = KC + 4;
    static constexpr int LDA = F32 ? KC + 4 : KC + 8;
    static constexpr int al(int x) { return (x + 15) / 16 * 16; }
    static constexpr int offK = 0;                                   // raw keys, rows
    static constexpr int offKL = offK + al(KC * LDK * ES);           // K_L rows (split)
    static constexpr int offVT = offKL + al(NS * KC * LDK * ES);     // V^T, two buffers by chunk parity
    static constexpr int offKtT = offVT + 2 * al(D * LDT * ES);      // Kt^T (split)
    static constexpr int offG = offKtT + al(NS * D * LDT * ES);      // Gamma [t][i]
    static constexpr int offL = offG + al(KC * LDG * 4);
    static constexpr int offInv = offL + al(KC * LDL * 4);
    static constexpr int offA = offInv + al(KC * LDI * 4);           // Inv diag(beta) (split)
    static constexpr int offLam = offA + al(NS * KC * LDA * ES);     // exp(Gamma_c) [D]
    static constexpr int offBeta = offLam + al(D * 4);
    static constexpr int total = offBeta + KC * 4;
    static_assert(total <= 160 * 1024, "LDS budget");
    static_assert(KC * D / 8 == NT, "one 8-element item per thread");
};

template <typename TIN>
struct Raw8k;
template <>
struct Raw8k<bf16> {
    bf16x8 v;
    __device__ void load(const bf16 *p) { v = *reinterpret_cast<const bf16x8 *>(p); }
    __device__ void zero() {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = (bf16)0.f;
    }
    __device__ float get(int e) const { return (float)v[e]; }
};
template <>
struct Raw8k<float> {
    f32x4 a, b;
    __device__ void load(const float *p) {
        a = *reinterpret_cast<const f32x4 *>(p);
        b = *reinterpret_cast<const f32x4 *>(p + 4);
    }
    __device__ void zero() { a = b = f32x4{0.f, 0.f, 0.f, 0.f}; }
    __device__ float get(int e) const { return e < 4 ? a[e] : b[e - 4]; }
};

// store x as an A/B operand element: fp32, or bf16 hi at p and lo at p + lo_off
template <bool F32, typename OpT>
__device__ __forceinline__ void put_split(OpT *p, int lo_off, float x) {
    if constexpr (F32) {
        *p = x;
    } else {
        bf16 h, l;
        split1(x, h, l);
        *p = h;
        p[lo_off] = l;
    }
}

// D += A B where A comes as a split operand from LDS (perm k subset) and B is
// an fp32 fragment: three bf16 passes, or the fp32 matrix cores.
template <bool F32, typename OpT>
__device__ __forceinline__ f32x4 mma_lds_perm(const OpT *M, int lo_off, int ld, int row, int kbase, int grp,
                                              const float (&b)[8], f32x4 c, float sign = 1.f) {
    if constexpr (F32) {
        float a[8];
        lds_perm_f(M, ld, row, kbase, grp, a);
        if (sign < 0.f) {
#pragma unroll
            for (int e = 0; e < 8; ++e) a[e] = -a[e];
        }
        return mma_f32(a, b, c);
    } else {
        bf16x8 ah = lds_perm(M, ld, row, kbase, grp), al = lds_perm(M + lo_off, ld, row, kbase, grp);
        if (sign < 0.f) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                ah[e] = -ah[e];
                al[e] = -al[e];
            }
        }
        bf16x8 bh, bl;
        split8(b, bh, bl);
        c = mfma(ah, bh, c);
        c = mfma(ah, bl, c);
        c = mfma(al, bh, c);
        return c;
    }
}

template <int D, typename TIN>
__global__ void __launch_bounds__(2 * D / 32 * 64)
k_build_kda(BuildArgs a) {
    using Cfg = KdaCfg<D, TIN>;
    constexpr bool F32 = Cfg::F32;
    using OpT = typename std::conditional<F32, float, bf16>::type;
    constexpr int NW = Cfg::NW, NT = Cfg::NT, RT = Cfg::RT, KB = Cfg::KB;
    constexpr int LDK = Cfg::LDK, LDT = Cfg::LDT, LDG = Cfg::LDG, LDL = Cfg::LDL, LDI = Cfg::LDI, LDA = Cfg::LDA;
    constexpr int LOK = KC * LDK, LOT = D * LDT, LOA = KC * LDA;  // offsets of lo copies
    __shared__ __attribute__((aligned(16))) char smem[Cfg::total];
    OpT *sK = reinterpret_cast<OpT *>(smem + Cfg::offK);
    OpT *sKL = reinterpret_cast<OpT *>(smem + Cfg::offKL);
    OpT *const sVT0 = reinterpret_cast<OpT *>(smem + Cfg::offVT);
    OpT *sKtT = reinterpret_cast<OpT *>(smem + Cfg::offKtT);
    float *sG = reinterpret_cast<float *>(smem + Cfg::offG);
    float *sL = reinterpret_cast<float *>(smem + Cfg::offL);
    float *sInv = reinterpret_cast<float *>(smem + Cfg::offInv);
    OpT *sA = reinterpret_cast<OpT *>(smem + Cfg::offA);
    float *sLam = reinterpret_cast<float *>(smem + Cfg::offLam);
    float *sBeta = reinterpret_cast<float *>(smem + Cfg::offBeta);

    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int r16 = lane & 15, grp = lane >> 4;
    const int seg = blockIdx.x / a.n_chains, chain = blockIdx.x % a.n_chains;
    const int dk = a.dk;
    const int64_t b0 = a.seg_begin[seg], n = a.seg_end[seg] - b0;
    const TIN *kp = reinterpret_cast<const TIN *>(a.x.k) + (int64_t)chain * a.x.cs;
    const TIN *vp = reinterpret_cast<const TIN *>(a.x.v) + (int64_t)chain * a.x.cs;
    const TIN *gp = reinterpret_cast<const TIN *>(a.x.g) + (int64_t)chain * a.x.gcs;
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

    // this thread's item of every chunk: token t, features i8 .. i8+7
    const int it_t = tid % KC, it_i8 = (tid / KC) * 8;
    const int koff = it_t * (int)a.x.ts + it_i8, goff = it_t * (int)a.x.gts + it_i8;
    Raw8k<TIN> kpre, vpre, gpre;
    TIN bpre = (TIN)0.f;
    auto prefetch = [&](int64_t c0) {
        const int L = (int)(n - c0 < KC ? n - c0 : KC);
        const int64_t t0 = b0 + c0;
        if (it_t < L && it_i8 < dk) {
            kpre.load(kp + t0 * a.x.ts + koff);
            vpre.load(vp + t0 * a.x.ts + koff);
            gpre.load(gp + t0 * a.x.gts + goff);
        } else {
            kpre.zero();
            vpre.zero();
            gpre.zero();
        }
        bpre = (TIN)0.f;
        if (wv == 0 && lane < L) bpre = bp[(t0 + lane) * a.x.bts];
    };
    if (n > 0) prefetch(0);

    for (int64_t c0 = 0; c0 < n; c0 += KC) {
        OpT *const sVT = sVT0 + (int)((c0 / KC) & 1) * (Cfg::al(D * LDT * Cfg::ES) / Cfg::ES);
        // ---- stage raw keys, V^T and log-gates
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            sK[it_t * LDK + it_i8 + e] = (OpT)kpre.get(e);
            sVT[(it_i8 + e) * LDT + it_t] = (OpT)vpre.get(e);
            sG[it_t * LDG + it_i8 + e] = gpre.get(e) * L2E;  // log2 units
        }
        if (wv == 0 && lane < KC) sBeta[lane] = (float)bpre;
        if (c0 + KC < n) prefetch(c0 + KC);
        __syncthreads();
        // ---- per-channel cumulative log-decay within the chunk
        for (int i = tid; i < D; i += NT) {
            float s = 0.f;
            for (int t = 0; t < KC; ++t) {
                s += sG[t * LDG + i];
                sG[t * LDG + i] = s;
            }
            sLam[i] = __builtin_amdgcn_exp2f(s);
        }
        __syncthreads();
        // ---- K_L = exp(Gamma) * K (rows) and Kt^T = (exp(Gamma_c - Gamma) * K)^T
        {
            const int t = it_t, i8 = it_i8;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int i = i8 + e;
                const float kv = (float)sK[t * LDK + i];
                const float gm = sG[t * LDG + i];
                put_split<F32>(sKL + t * LDK + i, LOK, kv * __builtin_amdgcn_exp2f(gm));
                put_split<F32>(sKtT + i * LDT + t, LOT, kv * __builtin_amdgcn_exp2f(sG[(KC - 1) * LDG + i] - gm));
            }
        }
        // ---- Gram with per-block reference tokens, scaled into the strictly lower L
        for (int tile = wv; tile < 3; tile += NW) {
            const int mt = tile == 0 ? 0 : 1, nt = tile == 2 ? 1 : 0;
            const int r = 16 * mt, ta = 16 * mt + r16, tb = 16 * nt + r16;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                const int i0 = 32 * kb + 8 * grp;
                float av[8], bv[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float gr = sG[r * LDG + i0 + e];
                    av[e] = (float)sK[ta * LDK + i0 + e] * __builtin_amdgcn_exp2f(sG[ta * LDG + i0 + e] - gr);
                    bv[e] = (float)sK[tb * LDK + i0 + e] * __builtin_amdgcn_exp2f(gr - sG[tb * LDG + i0 + e]);
                }
                acc = mma_split<F32>(av, bv, acc);
            }
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int t = 16 * mt + 4 * grp + jj, i = 16 * nt + r16;
                sL[t * LDL + i] = t > i ? sBeta[t] * acc[jj] : 0.f;
            }
        }
        __syncthreads();
        // ---- (I + L)^-1: two diagonal 16 x 16 blocks by forward substitution, then
        //      Inv_10 = -Inv_11 L_10 Inv_00 on the fp32 matrix cores
        if (wv == 0 && grp < 2) {
            const int bk = grp, c = r16;
            float xr[16];
#pragma unroll
            for (int rr = 0; rr < 16; ++rr) {
                float s = (rr == c) ? 1.f : 0.f;
#pragma unroll
                for (int j = 0; j < rr; ++j) s -= sL[(16 * bk + rr) * LDL + 16 * bk + j] * xr[j];
                xr[rr] = s;
            }
#pragma unroll
            for (int rr = 0; rr < 16; ++rr) sInv[(16 * bk + rr) * LDI + 16 * bk + c] = xr[rr];
        } else if (wv == 1) {
            for (int e = lane; e < 256; e += 64) sInv[(e >> 4) * LDI + 16 + (e & 15)] = 0.f;
        }
        __syncthreads();
        if (wv == 0) {
            f32x4 P = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < 4; ++s)
                P = __builtin_amdgcn_mfma_f32_16x16x4f32(sL[(16 + r16) * LDL + 4 * grp + s],
                                                         sInv[(4 * grp + s) * LDI + r16], P, 0, 0, 0);
            f32x4 O = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < 4; ++s)
                O = __builtin_amdgcn_mfma_f32_16x16x4f32(sInv[(16 + r16) * LDI + 16 + 4 * grp + s], P[s], O, 0, 0, 0);
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) sInv[(16 + 4 * grp + jj) * LDI + r16] = -O[jj];
        }
        __syncthreads();
        // ---- A = Inv diag(beta) as an A operand
        for (int idx = tid; idx < KC * KC; idx += NT) {
            const int t = idx / KC, i = idx % KC;
            put_split<F32>(sA + t * LDA + i, LOA, sInv[t * LDI + i] * sBeta[i]);
        }
        __syncthreads();

        // ---- carry this wave's 32 columns of X = [T | S] through the chunk
        {
            // Z = K_L X
            f32x4 Z[2][2];
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                for (int nt = 0; nt < 2; ++nt) Z[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                float xv[2][8];
#pragma unroll
                for (int nt = 0; nt < 2; ++nt) acc_to_perm(X[2 * kb][nt], X[2 * kb + 1][nt], xv[nt]);
#pragma unroll
                for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                    for (int nt = 0; nt < 2; ++nt)
                        Z[mt][nt] = mma_lds_perm<F32>(sKL, LOK, LDK, 16 * mt + r16, 32 * kb, grp, xv[nt], Z[mt][nt]);
            }
            // R = A ([0 | V] - Z)
            f32x4 R[2][2];
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                for (int nt = 0; nt < 2; ++nt) R[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
            float zv[2][8];
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) acc_to_perm(Z[0][nt], Z[1][nt], zv[nt]);
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                for (int nt = 0; nt < 2; ++nt) {
                    R[mt][nt] = mma_lds_perm<F32>(sA, LOA, LDA, 16 * mt + r16, 0, grp, zv[nt], R[mt][nt], -1.f);
                    if (isS) {
                        float vv[8];
                        const int col = cbase - D + 16 * nt + r16;
                        if constexpr (F32) {
                            lds_perm_f(sVT, LDT, col, 0, grp, vv);
                        } else {
                            const bf16x8 vb = lds_perm(sVT, LDT, col, 0, grp);
#pragma unroll
                            for (int e = 0; e < 8; ++e) vv[e] = (float)vb[e];
                        }
                        R[mt][nt] = mma_lds_perm<F32>(sA, LOA, LDA, 16 * mt + r16, 0, grp, vv, R[mt][nt]);
                    }
                }
            // X = diag(exp Gamma_c) X + Kt^T R
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                const f32x4 lam = *reinterpret_cast<const f32x4 *>(sLam + 16 * rt + 4 * grp);
#pragma unroll
                for (int nt = 0; nt < 2; ++nt) X[rt][nt] *= lam;
            }
            float rv[2][8];
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) acc_to_perm(R[0][nt], R[1][nt], rv[nt]);
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int nt = 0; nt < 2; ++nt)
                    X[rt][nt] = mma_lds_perm<F32>(sKtT, LOT, LDT, 16 * rt + r16, 0, grp, rv[nt], X[rt][nt]);
        }
        // (no barrier here: of what the next chunk's staging writes only V^T is
        // read by the carry, and it alternates between two buffers; the rest is
        // rewritten after the next chunk's first barrier, which every wave
        // reaches only after this carry)
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

template <int D, typename TIN>
static hipError_t launch_kda(const BuildArgs &a, int n_seg, hipStream_t st) {
    const dim3 grid((unsigned)(n_seg * (int64_t)a.n_chains));
    hipLaunchKernelGGL((k_build_kda<D, TIN>), grid, dim3(KdaCfg<D, TIN>::NT), 0, st, a);
    return hipGetLastError();
}

hipError_t build_kda(const BuildArgs &a, bool bf16_in, int D, int n_seg, hipStream_t st) {
    switch (D) {
    case 32: return bf16_in ? launch_kda<32, bf16>(a, n_seg, st) : launch_kda<32, float>(a, n_seg, st);
    case 64: return bf16_in ? launch_kda<64, bf16>(a, n_seg, st) : launch_kda<64, float>(a, n_seg, st);
    case 128: return bf16_in ? launch_kda<128, bf16>(a, n_seg, st) : launch_kda<128, float>(a, n_seg, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace hy
