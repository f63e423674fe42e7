// Dense-transition pair build (DeltaNet, Gated DeltaNet), bf16 inputs, for
// gfx950: the chunk factors of chunk j+1 are formed while chunk j is carried.
//
// Method: HYPIC (codernav.top article, section on linear layers: the cached
// pair (T_C, S(C|0))), advanced in chunks of c = 64 tokens on X = [T | S] from
// [I | 0].  With chunk-local cumulative log-gates Gamma_t, lambda = e^{Gamma_c},
// E = diag(e^{Gamma_c - Gamma_t}) and the undecayed strictly lower
// N0 = diag(beta) tril(K K^T, -1), the decayed chunk system is the similarity
// transform E^-1 (I + N0) E of the undecayed one, so per chunk
//     Y  = [0 | E V] - lambda K X
//     R' = (I + N0)^-1 diag(beta) Y          (R' = E R of the decayed form)
//     X <- lambda X + K^T R'
// and no exponent appears inside the chunk system.  R' is found by blocked
// forward substitution in 16-row blocks,
//     R'_b = A_b Y_b - sum_{c<b} M_bc R'_c,   A_b = (I + N0_bb)^-1 diag(beta_b),
//                                             M_bc = (I + N0_bb)^-1 N0_bc.
//
// Workgroup = 2d/32 carry waves + 2 factor waves, one (segment, chain) each.
//   carry wave w: columns 32w .. 32w+31 of X, resident in MFMA accumulators;
//     per chunk Z = K X, Y, the block solve (16x16x16 MFMAs whose B operand is
//     an accumulator tile as it stands) and the X update.  K^T comes from
//     transpose reads of the row-major K rows in LDS.
//   factor wave 0: stages K of the next chunk, forms the Gram tiles on the
//     matrix cores, inverts the four diagonal blocks (one row per lane, one
//     block per lane group) and forms A_b and M_bc, written pre-split into
//     hi + lo bf16 in the layout the carry waves read as MFMA A operands.
//   factor wave 1: scans the gates (DPP) and stages E V of the next chunk in
//     fp32, transposed, so an S wave reads its Y tile in one 16-byte load
//     (prefill: then forms the lower blocks of tril(Q K^T) once factor wave
//     0 has flagged the chunk's K and Q rows in LDS).
// Each factor wave works alone, so its steps need no workgroup barrier.
// Chunk inputs are prefetched two chunks ahead into the factor waves'
// registers; the factors live in a double-buffered LDS area; the workgroup
// meets at one barrier per chunk.
//
// Precision: keys and values are exact in bf16; every other operand is split
// into hi + lo bf16 (two or three passes, fp32 accumulation, fp32 state).
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace hy {

typedef short s4 __attribute__((ext_vector_type(4)));

// PF (prefill): the chunk's Q rows and the lower blocks of tril(Q K^T) are
// staged too, and V is staged as bf16 V^T with the per-token decays apart
// (ev = e^{Gamma_c - Gamma_t}, eo = e^{Gamma_t}, ei = e^{Gamma_t - Gamma_c}),
// which makes room for them.
template <int D, bool PF = false>
struct PipeCfg {
    static constexpr int NC = 2 * D / 32;  // carry waves
    static constexpr int NT = (NC + 2) * 64;
    static constexpr int RT = D / 16;
    static constexpr int KB = D / 32;
    static constexpr int LDK = D + 8;   // bf16 row stride of K (and Q) rows
    static constexpr int LDV = CH + 4;  // fp32 row stride of (E V)^T
    static constexpr int LDVB = CH + 8; // bf16 row stride of V^T (PF)
    static constexpr int LDT = 20;      // fp32 row stride of a diagonal block of N0
    static constexpr int TILE = 512;    // bf16 per pre-split 16 x 16 tile: [row][4 col groups][hi 4 | lo 4]
    static constexpr int al(int x) { return (x + 15) / 16 * 16; }
    // one buffer: K rows, [Q rows], (E V)^T or V^T and the decays, A_b, -M_bc, lambda
    static constexpr int bK = 0;
    static constexpr int bQ = bK + al(CH * LDK * 2);
    static constexpr int bV = PF ? bQ + al(CH * LDK * 2) : bQ;
    static constexpr int bE = bV + (PF ? al(D * LDVB * 2) : al(D * LDV * 4));
    static constexpr int bA = bE + (PF ? 3 * CH * 4 : 0);
    static constexpr int bQK = bA + 4 * TILE * 2;  // (PF) the ten lower 16 x 16 blocks of tril(Q K^T), pre-split
    static constexpr int bM = bQK + (PF ? 10 * TILE * 2 : 0);
    static constexpr int bLam = bM + 6 * TILE * 2;
    static constexpr int BUF = al(bLam + 16);
    // factor-wave scratch: beta, diagonal blocks of N0, their inverses (pre-split)
    static constexpr int offB = 2 * BUF;
    static constexpr int offN = offB + CH * 4;
    static constexpr int offI = offN + 4 * 16 * LDT * 4;
    // (PF) the chunk whose K and Q rows the factor wave has stored: the gate
    // wave forms tril(Q K^T) from them
    static constexpr int offFlag = offI + 4 * TILE * 2;
    static constexpr int total = offFlag + 16;
    static_assert(total <= 160 * 1024, "LDS budget");
};

typedef short s8v __attribute__((ext_vector_type(8)));

__device__ __forceinline__ void split4(const f32x4 &x, s4 &h, s4 &l) {
    u32x2 hu, lu;
    uint32_t a, b;
    split2(x[0], x[1], a, b);
    hu[0] = a;
    lu[0] = b;
    split2(x[2], x[3], a, b);
    hu[1] = a;
    lu[1] = b;
    h = __builtin_bit_cast(s4, hu);
    l = __builtin_bit_cast(s4, lu);
}

// C += A B on v_mfma_f32_16x16x16_bf16, operands split hi + lo (hi.hi + hi.lo +
// lo.hi).  A: lane holds A[r16][4grp + e]; B: B[4grp + e][r16], which is how a
// 16 x 16 accumulator tile sits in the lanes.
__device__ __forceinline__ f32x4 mma16(const s4 &ah, const s4 &al, const s4 &bh, const s4 &bl, f32x4 c) {
    c = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ah, bh, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ah, bl, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(al, bh, c, 0, 0, 0);
    return c;
}

// A fragment of a pre-split tile: 16 bytes per lane, [hi 4 | lo 4]
__device__ __forceinline__ void tile_frag(const bf16 *t, int r16, int grp, s4 &h, s4 &l) {
    const s8v v = *reinterpret_cast<const s8v *>(t + (r16 * 4 + grp) * 8);
    h = __builtin_shufflevector(v, v, 0, 1, 2, 3);
    l = __builtin_shufflevector(v, v, 4, 5, 6, 7);
}

__device__ __forceinline__ void tile_put(bf16 *t, int row, int q, const f32x4 &x) {
    s4 h, l;
    split4(x, h, l);
    *reinterpret_cast<s8v *>(t + (row * 4 + q) * 8) = __builtin_shufflevector(h, l, 0, 1, 2, 3, 4, 5, 6, 7);
}

template <int CTRL, int ROWS, bool ZERO>
__device__ __forceinline__ float dpp_take(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, ROWS, 0xf, ZERO));
}

// inclusive prefix sum over the 64 lanes: shifts within rows of 16, then the
// row totals carried forward by the row broadcasts of lanes 15 and 31
__device__ __forceinline__ float wave_incl_scan(float v) {
    v += dpp_take<0x111, 0xf, true>(v);  // row_shr:1
    v += dpp_take<0x112, 0xf, true>(v);  // row_shr:2
    v += dpp_take<0x114, 0xf, true>(v);  // row_shr:4
    v += dpp_take<0x118, 0xf, true>(v);  // row_shr:8
    v += dpp_take<0x142, 0xa, false>(v); // row_bcast:15 into rows 1, 3
    v += dpp_take<0x143, 0xc, false>(v); // row_bcast:31 into rows 2, 3
    return v;
}

// keep the compiler from moving LDS accesses across a point where another lane
// of the same wave reads what this one wrote (the wave's LDS ops run in order)
__device__ __forceinline__ void wave_lds_fence() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// PF: fused cold prefill.  Besides the pair, every token's output of the
// segment read from a zero state, o_t = S_t^T q_t, written in bf16 to a.o.
// Within a chunk that starts from S0, with u_i the i-th row of the decayed
// solve (R'_i = e^{Gamma_c - Gamma_i} u_i),
//     S_t = e^{Gamma_t} S0 + sum_{i<=t} e^{Gamma_t - Gamma_i} k_i u_i^T,
// so  O = diag(e^{Gamma_t}) Q S0 + diag(e^{Gamma_t - Gamma_c}) tril(Q K^T) R'
// (tril inclusive): each S wave forms its 32 columns of O on the matrix cores
// after its block solve, before the carry update.
// One carry wave's 16 output columns (c0 + 16 .. c0 + 31 of o) for the chunk
// of tokens t0 .. t0 + min(L, 64) - 1, from P = Q S0 on those columns (formed
// beside Z = K X from the same split state), the solved R' (split, C layout
// per 16-row block, tile 1) and the staged blocks of tril(Q K^T).  The bf16
// outputs are staged transposed in this wave's own 16 rows of the chunk's V^T
// (read only by this wave, in its Y step) and leave as 8-byte row pieces:
// four stores per lane instead of sixteen 2-byte ones.
template <int D, typename Cfg>
__device__ __forceinline__ void prefill_out(const f32x4 (&P)[4], const s4 (&Rh)[4][2], const s4 (&Rl)[4][2],
                                            const char *buf, const BuildArgs &a, int64_t t0, int L, int chain, int c0) {
    constexpr int TILE = Cfg::TILE, LDVB = Cfg::LDVB;
    constexpr int nt = 1;
    const int lane = lane_fresh(), r16 = lane & 15, grp = lane >> 4;
    const bf16 *bQK = reinterpret_cast<const bf16 *>(buf + Cfg::bQK);
    const float *bE = reinterpret_cast<const float *>(buf + Cfg::bE);
    bf16 *stg = const_cast<bf16 *>(reinterpret_cast<const bf16 *>(buf + Cfg::bV)) + (c0 + 16) * LDVB;
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
        f32x4 oi = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ib = 0; ib <= tb; ++ib) {
            s4 ch, cl;
            tile_frag(bQK + (tb * (tb + 1) / 2 + ib) * TILE, r16, grp, ch, cl);
            oi = mma16(ch, cl, Rh[ib][nt], Rl[ib][nt], oi);
        }
        const f32x4 eo = *reinterpret_cast<const f32x4 *>(bE + CH + 16 * tb + 4 * grp);
        const f32x4 ei = *reinterpret_cast<const f32x4 *>(bE + 2 * CH + 16 * tb + 4 * grp);
        bf16x4 ov;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) ov[jj] = (bf16)(eo[jj] * P[tb][jj] + ei[jj] * oi[jj]);
        // column r16, tokens 16 tb + 4 grp .. + 3
        *reinterpret_cast<bf16x4 *>(stg + r16 * LDVB + 16 * tb + 4 * grp) = ov;
        __builtin_amdgcn_sched_barrier(0);
    }
    wave_lds_fence();
    // lane group g takes columns 4 g .. 4 g + 3 of token 16 blk + r16
    bf16 *o = reinterpret_cast<bf16 *>(a.o) + (int64_t)chain * a.ocs + c0 + 16 + 4 * grp;
    const bool col_ok = c0 + 16 + 4 * grp < a.dk;
#pragma unroll
    for (int blk = 0; blk < 4; ++blk) {
        const bf16x4 w = lds_tr4(stg, LDVB, 4 * grp, 16 * blk, r16);
        const int t = 16 * blk + r16;
        if (t < L && col_ok) *reinterpret_cast<bf16x4 *>(o + (t0 + t) * a.ots) = w;
    }
}

template <int D, int FAM, bool PF = false>
__global__ void __launch_bounds__((2 * D / 32 + 2) * 64)
k_build_dense_pipe(BuildArgs a) {
    using Cfg = PipeCfg<D, PF>;
    constexpr int NC = Cfg::NC, RT = Cfg::RT, KB = Cfg::KB;
    constexpr int LDK = Cfg::LDK, LDV = Cfg::LDV, LDVB = Cfg::LDVB, LDT = Cfg::LDT, TILE = Cfg::TILE;
    constexpr float L2E = 1.4426950408889634f;
    __shared__ __attribute__((aligned(16))) char smem[Cfg::total];

    const int tid = threadIdx.x;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform role
    const int seg = blockIdx.x / a.n_chains, chain = blockIdx.x % a.n_chains;
    const int dk = a.dk;
    const int64_t b0 = a.seg_begin[seg], n = a.seg_end[seg] - b0;
    const int nch = (int)((n + CH - 1) / CH);

    if constexpr (PF) {
        if (tid == 0) *reinterpret_cast<int *>(smem + Cfg::offFlag) = -1;
        __syncthreads();
    }
    // Carry waves and factor waves run separate loops that meet at the same
    // number of barriers: (nch > 0) + nch.
    if (wv >= NC) {
        // the factor waves go first at issue on the SIMDs they share with
        // carry waves: their chains of short dependent steps set the period
        __builtin_amdgcn_s_setprio(3);
        // each role is its own instantiation, so that neither holds the
        // other's prefetch registers
        auto role = [&](auto KWC) {
        constexpr bool kw = decltype(KWC)::value;  // K / factor wave, else V / gate wave
        const int lane = tid & 63;
        const bf16 *src = reinterpret_cast<const bf16 *>(kw ? a.x.k : a.x.v) + (int64_t)chain * a.x.cs;
        const bf16 *gp = FAM == GDN ? reinterpret_cast<const bf16 *>(a.x.g) + (int64_t)chain * a.x.gcs : nullptr;
        const bf16 *bp = reinterpret_cast<const bf16 *>(a.x.beta) + (int64_t)chain * a.x.bcs;
        // token row `lane` of a chunk (D bf16 = D/8 16-byte pieces) and its
        // beta (K wave) or gate (V wave), two chunks ahead of the carry
        constexpr int RV = D / 8;
        bf16x8 pre[RV];
        bf16 spre = (bf16)0.f;
        const bf16 *qsrc = PF ? reinterpret_cast<const bf16 *>(a.x.q) + (int64_t)chain * a.x.cs : nullptr;
        auto prefetch = [&](int c) {
            const int64_t c0 = (int64_t)c * CH;
            const int L = (int)(n - c0 < CH ? n - c0 : CH);
            const int64_t t = b0 + c0 + lane;
            const bf16 *row = src + t * a.x.ts;
#pragma unroll
            for (int p = 0; p < RV; ++p) {
                if (lane < L && 8 * p < dk) {
                    pre[p] = *reinterpret_cast<const bf16x8 *>(row + 8 * p);
                } else {
#pragma unroll
                    for (int e = 0; e < 8; ++e) pre[p][e] = (bf16)0.f;
                }
            }
            spre = (bf16)0.f;
            if (lane < L) {
                if (kw) spre = bp[t * a.x.bts];
                else if (FAM == GDN) spre = gp[t * a.x.gts];
            }
        };
        auto factors = [&](int c) {
            // lane-derived addresses are rebuilt here from an opaque copy of
            // the lane id rather than held in registers across the chunk loop
            int lane = tid & 63;
            asm volatile("" : "+v"(lane));
            const int r16 = lane & 15, grp = lane >> 4;
            char *buf = smem + (c & 1) * Cfg::BUF;
            if (!kw) {
                // gate scan (lane = token, Gamma in log2 units), lambda, (E V)^T
                float s = 0.f, gc = 0.f;
                if (FAM == GDN) {
                    s = wave_incl_scan((float)spre * L2E);
                    gc = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, s), 63));
                }
                const float ec = __builtin_amdgcn_exp2f(gc - s);
                if constexpr (PF) {
                    bf16 *bV = reinterpret_cast<bf16 *>(buf + Cfg::bV);
#pragma unroll
                    for (int p = 0; p < RV; ++p)
#pragma unroll
                        for (int e = 0; e < 8; ++e) bV[(8 * p + e) * LDVB + lane] = pre[p][e];
                    float *bE = reinterpret_cast<float *>(buf + Cfg::bE);
                    bE[lane] = ec;
                    bE[CH + lane] = __builtin_amdgcn_exp2f(s);
                    bE[2 * CH + lane] = __builtin_amdgcn_exp2f(s - gc);
                } else {
                    float *bV = reinterpret_cast<float *>(buf + Cfg::bV);
#pragma unroll
                    for (int p = 0; p < RV; ++p)
#pragma unroll
                        for (int e = 0; e < 8; ++e) bV[(8 * p + e) * LDV + lane] = ec * (float)pre[p][e];
                }
                if (lane == 0) *reinterpret_cast<float *>(buf + Cfg::bLam) = __builtin_amdgcn_exp2f(gc);
                if constexpr (PF) {
                    // the lower blocks of tril(Q K^T), once the factor wave
                    // has stored this chunk's K and Q rows (a bounded wait:
                    // the factor wave sets the flag early in its step).  On
                    // the factor wave they set the prefill's period: 19.6
                    // against 16.7 ms without them.
                    const volatile int *vf = reinterpret_cast<const volatile int *>(smem + Cfg::offFlag);
                    for (int it = 0; it < (1 << 20) && *vf != c; ++it) __builtin_amdgcn_s_sleep(1);
                    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
                    const bf16 *bK = reinterpret_cast<const bf16 *>(buf + Cfg::bK);
                    // block (tb, ib <= tb) of tril(Q K^T) as the A operand: the lane
                    // needs (Q K^T)[16 tb + r16][16 ib + 4 grp + e], which is where
                    // the C layout of K_ib Q_tb^T puts it (exact: bf16 products
                    // summed in fp32), split hi + lo
                    const bf16 *bQ = reinterpret_cast<const bf16 *>(buf + Cfg::bQ);
                    bf16 *bQK = reinterpret_cast<bf16 *>(buf + Cfg::bQK);
#pragma unroll
                    for (int tb = 0; tb < 4; ++tb) {
#pragma unroll
                        for (int ib = 0; ib <= tb; ++ib) {
                            f32x4 cq = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                            for (int kb = 0; kb < KB; ++kb)
                                cq = mfma(lds_cont(bK, LDK, 16 * ib + r16, 32 * kb, grp),
                                          lds_cont(bQ, LDK, 16 * tb + r16, 32 * kb, grp), cq);
                            if (ib == tb) {
#pragma unroll
                                for (int e = 0; e < 4; ++e) cq[e] = (4 * grp + e <= r16) ? cq[e] : 0.f;
                            }
                            tile_put(bQK + (tb * (tb + 1) / 2 + ib) * TILE, r16, grp, cq);
                        }
                        __builtin_amdgcn_sched_barrier(0);
                    }
                }
                return;
            }
            bf16 *bK = reinterpret_cast<bf16 *>(buf + Cfg::bK);
            bf16 *bA = reinterpret_cast<bf16 *>(buf + Cfg::bA);
            bf16 *bM = reinterpret_cast<bf16 *>(buf + Cfg::bM);
            float *sB = reinterpret_cast<float *>(smem + Cfg::offB);
            float *sN = reinterpret_cast<float *>(smem + Cfg::offN);
            bf16 *sI = reinterpret_cast<bf16 *>(smem + Cfg::offI);
#pragma unroll
            for (int p = 0; p < RV; ++p) *reinterpret_cast<bf16x8 *>(bK + lane * LDK + 8 * p) = pre[p];
            sB[lane] = (float)spre;
            // (PF) this chunk's q rows, not fetched ahead: they are requested
            // once the K rows are stored (the factor wave has slack in
            // the chunk period; holding them two chunks ahead next to the K
            // rows would not fit its registers)
            bf16x8 preq[PF ? RV : 1];
            if constexpr (PF) {
                const int64_t c0 = (int64_t)c * CH;
                const int L = (int)(n - c0 < CH ? n - c0 : CH);
                const bool on = lane < L;
                const bf16 *qrow = qsrc + (on ? b0 + c0 + lane : b0) * a.x.ts;
#pragma unroll
                for (int p = 0; p < RV; ++p) {
                    const bf16x8 v = *reinterpret_cast<const bf16x8 *>(qrow + 8 * (8 * p < dk ? p : 0));
                    preq[p] = (on && 8 * p < dk) ? v : bf16x8{};
                }
            }
            if constexpr (PF) {
                bf16 *bQ = reinterpret_cast<bf16 *>(buf + Cfg::bQ);
#pragma unroll
                for (int p = 0; p < RV; ++p) *reinterpret_cast<bf16x8 *>(bQ + lane * LDK + 8 * p) = preq[p];
            }
            wave_lds_fence();
            if constexpr (PF) {
                // K and Q rows of chunk c are in place: the gate wave takes
                // tril(Q K^T) from here
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
                if (lane == 0) *reinterpret_cast<volatile int *>(smem + Cfg::offFlag) = c;
            }
            // Gram tiles, one block row b at a time, in C layout: the lane holds
            // rows t = 16b + 4grp + e, column i = 16c + r16 of N0 = beta_t G_ti.
            // Diagonal blocks go to LDS row-major for the inverse; the six
            // off-diagonal ones stay in registers for the M products.
            f32x4 noff[6];
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                f32x4 acc[4];
#pragma unroll
                for (int nt = 0; nt <= mt; ++nt) acc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kb = 0; kb < KB; ++kb) {
                    const bf16x8 km = lds_cont(bK, LDK, 16 * mt + r16, 32 * kb, grp);
#pragma unroll
                    for (int nt = 0; nt < mt; ++nt)
                        acc[nt] = mfma(km, lds_cont(bK, LDK, 16 * nt + r16, 32 * kb, grp), acc[nt]);
                    acc[mt] = mfma(km, km, acc[mt]);
                }
                const f32x4 b4 = *reinterpret_cast<const f32x4 *>(sB + 16 * mt + 4 * grp);
#pragma unroll
                for (int nt = 0; nt < mt; ++nt) noff[mt * (mt - 1) / 2 + nt] = acc[nt] * b4;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    sN[(16 * mt + 4 * grp + e) * LDT + r16] = (4 * grp + e > r16) ? b4[e] * acc[mt][e] : 0.f;
                __builtin_amdgcn_sched_barrier(0);
            }
            wave_lds_fence();
            // row r16 of (I + N0_bb)^-1 for block b = grp: y (I + N0_bb) = e_r.
            // Swept from the last row up: once y_i is final its multiple of row
            // i of N0_bb leaves every y_j, j < i, so the dependent chain is 16
            // steps long.  Stored pre-split as is (for M) and times diag(beta_b)
            // (A_b).
            {
                float y[16];
#pragma unroll
                for (int j = 0; j < 16; ++j) y[j] = (j == r16) ? 1.f : 0.f;
                f32x4 cur[4], nxt[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) cur[q] = *reinterpret_cast<const f32x4 *>(sN + (16 * grp + 15) * LDT + 4 * q);
#pragma unroll
                for (int i = 15; i > 0; --i) {
#pragma unroll
                    for (int q = 0; 4 * q < i - 1; ++q)
                        nxt[q] = *reinterpret_cast<const f32x4 *>(sN + (16 * grp + i - 1) * LDT + 4 * q);
#pragma unroll
                    for (int q = 0; 4 * q < i; ++q)
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            if (4 * q + e < i) y[4 * q + e] -= y[i] * cur[q][e];
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int q = 0; q < 4; ++q) cur[q] = nxt[q];
                }
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const f32x4 yq = {y[4 * q], y[4 * q + 1], y[4 * q + 2], y[4 * q + 3]};
                    const f32x4 bq = *reinterpret_cast<const f32x4 *>(sB + 16 * grp + 4 * q);
                    tile_put(sI + grp * TILE, r16, q, yq);
                    tile_put(bA + grp * TILE, r16, q, yq * bq);
                }
            }
            wave_lds_fence();
            // -M_bc: C = N0_bc^T Inv_b^T = M_bc^T in C layout, i.e. the lane
            // holds M_bc[r16][4grp + e], the A-operand layout
#pragma unroll
            for (int mt = 1; mt < 4; ++mt) {
                s4 ih, il;
                tile_frag(sI + mt * TILE, r16, grp, ih, il);
#pragma unroll
                for (int nt = 0; nt < mt; ++nt) {
                    s4 nh, nl;
                    split4(noff[mt * (mt - 1) / 2 + nt], nh, nl);
                    const f32x4 m = mma16(nh, nl, ih, il, f32x4{0.f, 0.f, 0.f, 0.f});
                    tile_put(bM + (mt * (mt - 1) / 2 + nt) * TILE, r16, grp, -m);
                }
            }
        };
        if (nch > 0) {
            prefetch(0);
            factors(0);
            if (nch > 1) prefetch(1);
            __syncthreads();
        }
        for (int c = 0; c < nch; ++c) {
            if (c + 1 < nch) {
                factors(c + 1);
                if (c + 2 < nch) prefetch(c + 2);
            }
            __syncthreads();
        }
        };
        if (wv == NC)
            role(std::true_type{});
        else
            role(std::false_type{});
        return;
    }

    const int lane = tid & 63, r16 = lane & 15, grp = lane >> 4;
    // Columns of [T | S] per wave.  Plain build: carry slot p holds columns
    // 32 p .. 32 p + 31 (T: p < d/32).  Wave i of the workgroup runs on SIMD
    // i % 4, so the factor waves (NC, NC + 1) share SIMDs 0 and 1 with carry
    // waves; at d = 128 those are given T slots, whose waves finish their
    // chunk earlier than the S waves (E V), and the S waves take SIMDs 2 and
    // 3: 12.72 against 12.85 ms for 960 GDN chains of a 32k-token request in
    // the same calls (S waves beside the factor waves instead, 12.84).  At
    // d <= 64 the T waves are on SIMDs 0 and 1 as they stand.  Prefill: tile
    // 0 holds T columns 16 wv .. 16 wv + 15
    // and tile 1 the same columns of S, so that every carry wave writes the
    // outputs of 16 columns (the outputs cost as much as the carry of S).
    const int slot = PF || NC != 8 ? wv : (wv & 1) + 2 * (wv >> 2) + 4 * ((wv >> 1) & 1);
    const int cbase = slot * 32;
    const bool isS = cbase >= D;
    auto col0 = [&](int nt) { return PF ? (nt ? D : 0) + 16 * wv : cbase + 16 * nt; };
    f32x4 X[RT][2];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) X[rt][nt][jj] = (16 * rt + 4 * grp + jj == col0(nt) + r16) ? 1.f : 0.f;
    if (nch > 0) __syncthreads();
    for (int c = 0; c < nch; ++c) {
        const char *buf = smem + (c & 1) * Cfg::BUF;
        const bf16 *bK = reinterpret_cast<const bf16 *>(buf + Cfg::bK);
        const float *bV = reinterpret_cast<const float *>(buf + Cfg::bV);
        const bf16 *bA = reinterpret_cast<const bf16 *>(buf + Cfg::bA);
        const bf16 *bM = reinterpret_cast<const bf16 *>(buf + Cfg::bM);
        const float lam = FAM == GDN ? *reinterpret_cast<const float *>(buf + Cfg::bLam) : 1.f;
        // Z = K X (and, for the prefill, QS = Q S0 on the S tile)
        const bf16 *bQ = reinterpret_cast<const bf16 *>(buf + Cfg::bQ);
        f32x4 QS[PF ? 4 : 1];
#pragma unroll
        for (int mt = 0; mt < (PF ? 4 : 1); ++mt) QS[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
        f32x4 Z[4][2];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
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
            for (int mt = 0; mt < 4; ++mt) {
                const bf16x8 kh = lds_perm(bK, LDK, 16 * mt + r16, 32 * kb, grp);
#pragma unroll
                for (int nt = 0; nt < 2; ++nt) {
                    Z[mt][nt] = mfma(kh, xh[nt], Z[mt][nt]);
                    Z[mt][nt] = mfma(kh, xl[nt], Z[mt][nt]);
                }
                if constexpr (PF) {
                    // Q S0 on the S tile, from the same split state
                    const bf16x8 qh = lds_perm(bQ, LDK, 16 * mt + r16, 32 * kb, grp);
                    QS[mt] = mfma(qh, xh[1], QS[mt]);
                    QS[mt] = mfma(qh, xl[1], QS[mt]);
                }
            }
        }
        // Y = [0 | E V] - lambda Z, split.  Y and the block solve are a
        // dependent chain: a carry wave in them goes first at issue on its
        // SIMD (11.63-11.83 against 11.69-11.90 ms for 960 GDN chains of a
        // 32k-token request, six same-call comparisons; the prefill 19.50-19.53
        // against 19.61-19.66 ms).
        __builtin_amdgcn_s_setprio(1);
        s4 Yh[4][2], Yl[4][2];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
                f32x4 y = -lam * Z[mt][nt];
                if constexpr (PF) {
                    if (nt == 1) {
                        const bf16x4 v4 = *reinterpret_cast<const bf16x4 *>(
                            reinterpret_cast<const bf16 *>(buf + Cfg::bV) + (16 * wv + r16) * LDVB + 16 * mt +
                            4 * grp);
                        const f32x4 e4 = *reinterpret_cast<const f32x4 *>(
                            reinterpret_cast<const float *>(buf + Cfg::bE) + 16 * mt + 4 * grp);
#pragma unroll
                        for (int e = 0; e < 4; ++e) y[e] += e4[e] * (float)v4[e];
                    }
                } else {
                    if (isS)
                        y += *reinterpret_cast<const f32x4 *>(bV + (cbase - D + 16 * nt + r16) * LDV + 16 * mt + 4 * grp);
                }
                split4(y, Yh[mt][nt], Yl[mt][nt]);
            }
        // R'_b = A_b Y_b - sum_{c<b} M_bc R'_c, kept split
        s4 Rh[4][2], Rl[4][2];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            f32x4 r[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
            s4 ah, al;
            tile_frag(bA + b * TILE, r16, grp, ah, al);
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) r[nt] = mma16(ah, al, Yh[b][nt], Yl[b][nt], r[nt]);
#pragma unroll
            for (int c2 = 0; c2 < b; ++c2) {
                s4 mh, ml;
                tile_frag(bM + (b * (b - 1) / 2 + c2) * TILE, r16, grp, mh, ml);
#pragma unroll
                for (int nt = 0; nt < 2; ++nt) r[nt] = mma16(mh, ml, Rh[c2][nt], Rl[c2][nt], r[nt]);
            }
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) split4(r[nt], Rh[b][nt], Rl[b][nt]);
        }
        if constexpr (PF) {
            prefill_out<D, Cfg>(QS, Rh, Rl, buf, a, b0 + (int64_t)c * CH, (int)(n - (int64_t)c * CH), chain,
                                   16 * wv - 16);
        }
        __builtin_amdgcn_s_setprio(0);
        // X = lambda X + K^T R'
        if (FAM == GDN) {
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int nt = 0; nt < 2; ++nt) X[rt][nt] *= lam;
        }
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            bf16x8 rh[2], rl[2];
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
                rh[nt] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(Rh[2 * h][nt], Rh[2 * h + 1][nt], 0, 1, 2, 3, 4, 5, 6, 7));
                rl[nt] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(Rl[2 * h][nt], Rl[2 * h + 1][nt], 0, 1, 2, 3, 4, 5, 6, 7));
            }
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                const bf16x8 kt = lds_tr_perm(bK, LDK, 32 * h, 16 * rt, r16, grp);
#pragma unroll
                for (int nt = 0; nt < 2; ++nt) {
                    X[rt][nt] = mfma(kt, rh[nt], X[rt][nt]);
                    X[rt][nt] = mfma(kt, rl[nt], X[rt][nt]);
                }
            }
        }
        __syncthreads();
    }

    float *To = a.T + ((int64_t)seg * a.n_chains + chain) * dk * dk;
    float *So = a.S + ((int64_t)seg * a.n_chains + chain) * dk * dk;
    // (row and column indices from a fresh lane index: shared with the
    // identity start above, the compiler kept them across the chunk loop and
    // spilled them in the prefill instantiation)
    const int lf = lane_fresh(), fr16 = lf & 15, fgrp = lf >> 4;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int row = 16 * rt + 4 * fgrp + jj;
                const bool s_ = col0(nt) >= D;
                const int col = col0(nt) + fr16 - (s_ ? D : 0);
                if (row < dk && col < dk) (s_ ? So : To)[row * dk + col] = X[rt][nt][jj];
            }
}

template <int D, int FAM>
static hipError_t launch_pipe(const BuildArgs &a, int n_seg, hipStream_t st) {
    const dim3 grid((unsigned)(n_seg * (int64_t)a.n_chains));
    if (a.o)
        hipLaunchKernelGGL((k_build_dense_pipe<D, FAM, true>), grid, dim3(PipeCfg<D, true>::NT), 0, st, a);
    else
        hipLaunchKernelGGL((k_build_dense_pipe<D, FAM, false>), grid, dim3(PipeCfg<D>::NT), 0, st, a);
    return hipGetLastError();
}

hipError_t build_dense_pipe(const BuildArgs &a, int family, int D, int n_seg, hipStream_t st) {
    if (family != GDN && family != DELTANET) return hipErrorInvalidValue;
    switch (D) {
    case 32: return family == GDN ? launch_pipe<32, GDN>(a, n_seg, st) : launch_pipe<32, DELTANET>(a, n_seg, st);
    case 64: return family == GDN ? launch_pipe<64, GDN>(a, n_seg, st) : launch_pipe<64, DELTANET>(a, n_seg, st);
    case 128: return family == GDN ? launch_pipe<128, GDN>(a, n_seg, st) : launch_pipe<128, DELTANET>(a, n_seg, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace hy
