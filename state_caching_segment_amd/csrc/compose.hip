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
// Sequential mode: one workgroup per (request, chain) with d/32 waves; wave w
// keeps columns 32w .. 32w+31 of the running state in MFMA accumulators for
// the whole list.  Dense T (k_compose_dense): S <- T S + S_slot as a small GEMM
// on the matrix cores, T staged once per workgroup through LDS one entry ahead
// and the state fed back as the B operand (three-pass bf16 split for bf16
// inputs, fp32 matrix cores for fp32 inputs; fp32 state either way).
// Diagonal T (k_compose_seq): a row scale plus add.
// The seam recurrence runs on the vector ALUs over the same registers.
//
// Tree mode, the associative form (T_b, S_b) o (T_a, S_a) = (T_b T_a,
// T_b S_a + S_b) over each request's entries in blocks of B:
//   1. per (request, block, chain): run the block's entries from (I, 0) on
//      [T_p | S_p]; a seam token updates both halves with its transition (the
//      T half takes v = 0), so the S half's read-out is the block-local output
//      o^_t and the T half's is the pulled-back query p_t = T_p^T q_t; each
//      pair gives (T T_p, T S_p + S).  Writes the block aggregate.
//   2. per (request, chain): scan the block aggregates in order, keeping each
//      block's incoming state S_in and the final state.
//   3. per (request, block, chain): o_t = o^_t + S_in^T p_t.
// Every pair is read once; the price is the T T_p product (about twice the
// sequential flops).
#include <mutex>

#include "compose_common.h"
#include "kernels.h"

namespace hy {

template <int D, int FAM, typename TIN>
__global__ void __launch_bounds__(D / 32 * 64)
k_compose_seq(ComposeArgs a) {
    constexpr bool F32 = std::is_same<TIN, float>::value;
    __shared__ SeamSmem<D, FAM> sm;
    const int wv = threadIdx.x >> 6;
    const int req = blockIdx.x / a.n_chains, chain = blockIdx.x % a.n_chains;
    const int dk = a.dk, c0 = wv * 32;
    float *st = a.state + ((int64_t)req * a.n_chains + chain) * dk * dk;
    f32x4 X[D / 16][2];
    if constexpr (fam_dense(FAM))
        load_tile<D>(X, st, dk, dk, c0, dk);
    else
        load_tile_buf<D>(X, st, dk, c0);

    const int e0 = a.list_off[req], e1 = a.list_off[req + 1];
    // a window that fits one stage is fetched one entry ahead into registers
    // (not for a per-channel gate: measured slower here, 0.49 ms against 0.44
    // on a 16-chain GLA request, while the tree's block phase gains)
    SeamPrefetch<D, TIN> pf;
    const bool one = !fam_vgate(FAM) && a.has_seam && a.w <= SEAM_STAGE;
    // (the seam tokens, gamma included, exist only when the call has seams)
    const float rg = (FAM == RETNET && one) ? a.x.gamma[chain] : 1.f;
    if (one && e0 < e1) seam_fetch<D, FAM, TIN>(pf, a.x, chain, dk, a.seam_begin[e0], a.w);
    for (int e = e0; e < e1; ++e) {
        if (a.has_seam) {
            const int64_t sb = a.seam_begin[e];
            if (one) {
                if (sb >= 0) {
                    __syncthreads();
                    seam_put<D, FAM, TIN>(sm, pf, dk, a.w, rg);
                    __syncthreads();
                }
                seam_fetch<D, FAM, TIN>(pf, a.x, chain, dk, e + 1 < e1 ? a.seam_begin[e + 1] : -1, a.w);
                if (sb >= 0)
                    seam_tokens<D, FAM>(X, sm, a.w, a.o + ((int64_t)e * a.w * a.n_chains + chain) * dk,
                                        (int64_t)a.n_chains * dk, c0, c0, false, dk);
            } else if (sb >= 0) {
                for (int s0 = 0; s0 < a.w; s0 += SEAM_STAGE) {
                    const int nt = a.w - s0 < SEAM_STAGE ? a.w - s0 : SEAM_STAGE;
                    __syncthreads();
                    stage_seam<D, FAM, TIN>(sm, a.x, chain, dk, sb + s0, nt);
                    __syncthreads();
                    float *o_first = a.o + (((int64_t)e * a.w + s0) * a.n_chains + chain) * dk;
                    seam_tokens<D, FAM>(X, sm, nt, o_first, (int64_t)a.n_chains * dk, c0, c0, false, dk);
                }
            }
        }
        const int64_t slot = a.pair_id[e];
        const float *Tp = a.T + (slot * a.n_chains + chain) * a.t_elems;
        const float *Sp = a.S + (slot * a.n_chains + chain) * dk * dk;
        if constexpr (fam_dense(FAM))
            apply_dense_T<D, F32>(X, Tp, dk, Sp, c0);
        else
            apply_diag_T_buf<D>(X, Tp, a.t_elems, dk, Sp, c0);
        if (a.prefix) store_tile_buf<D>(X, a.prefix + ((int64_t)e * a.n_chains + chain) * dk * dk, dk, c0);
    }
    if constexpr (fam_dense(FAM))
        store_tile<D>(X, st, dk, dk, c0, dk);
    else
        store_tile_buf<D>(X, st, dk, c0);
}

template <int D, int FAM, typename TIN>
__global__ void __launch_bounds__(D / 32 * 64)
k_seam_advance(SeamArgs a) {
    __shared__ SeamSmem<D, FAM> sm;
    const int wv = threadIdx.x >> 6;
    const int item = blockIdx.x / a.n_chains, chain = blockIdx.x % a.n_chains;
    const int dk = a.dk, c0 = wv * 32;
    float *st = a.state + ((int64_t)item * a.n_chains + chain) * dk * dk;
    f32x4 X[D / 16][2];
    load_tile<D>(X, st, dk, dk, c0, dk);
    const int64_t tb = a.tok_begin[item];
    for (int s0 = 0; s0 < a.w; s0 += SEAM_STAGE) {
        const int nt = a.w - s0 < SEAM_STAGE ? a.w - s0 : SEAM_STAGE;
        __syncthreads();
        stage_seam<D, FAM, TIN>(sm, a.x, chain, dk, tb + s0, nt);
        __syncthreads();
        float *o_first = a.o + (((int64_t)item * a.w + s0) * a.n_chains + chain) * dk;
        seam_tokens<D, FAM>(X, sm, nt, o_first, (int64_t)a.n_chains * dk, c0, c0, false, dk);
    }
    store_tile<D>(X, st, dk, dk, c0, dk);
}

// Sequential compose for dense T (DeltaNet, GDN, KDA).  The workgroup owns one
// (request, chain); wave w keeps columns 32w .. 32w+31 of the running state in
// MFMA accumulators.  Each entry's T is read from HBM once per workgroup: every
// wave loads its share of T's rows one entry ahead into registers and, once
// the previous product is done, writes them into the LDS copy of T -- split
// into hi and lo bf16 halves of each row for bf16 inputs (fp32 rows for fp32
// inputs) -- from which all waves take their A operands.  The LDS copy is
// double-buffered, so T_{j+1} is written while T_j is in use and T_{j+2} is
// in flight.  The entry's S columns of each wave are requested as soon as the
// previous ones have seeded the accumulators of S <- T S + S_j, so their loads
// overlap the product.
template <int D, bool F32>
struct DenseTLds {
    static constexpr int LDT = F32 ? D + 4 : 2 * D + 8;  // elements per T row: fp32, or [hi | lo] bf16
    static constexpr int BYTES = D * LDT * (F32 ? 4 : 2);
};

// TREE: the first phase of the tree compose on the same machinery.  The
// workgroup owns one (request, block of entries, chain) and runs the block's
// entries from (I, 0) on [T_p | S_p] with 2d/32 waves: the T half takes no
// S_j and, at seams, zero values, so its seam read-out is the pulled-back
// query T_p^T q_t; the block aggregate is written at the end.
// Output rows of seam tokens s0 .. of list entry e: the S half writes o_t,
// the T half of a tree block writes the pulled-back queries.
__device__ __forceinline__ float *seam_out(const TreeArgs &t, bool isS, int e, int req, int jl, int chain, int s0,
                                           int dk) {
    const ComposeArgs &a = t.c;
    return isS ? a.o + (((int64_t)e * a.w + s0) * a.n_chains + chain) * dk
               : t.pvec + ((((int64_t)req * t.max_list + jl) * a.w + s0) * a.n_chains + chain) * dk;
}

// One staged stage of nt seam tokens on the wave's columns.
template <int D, int FAM, bool CHUNK, typename SM, bool UPDATE_FIRST = false>
__device__ __forceinline__ void seam_stage_run(f32x4 (&X)[D / 16][2], const SM &sm, int nt,
                                               float *o_first, const ComposeArgs &a, int c0, int dk,
                                               float (*nm)[SEAM_STAGE][9], bool v_zero) {
    if constexpr (CHUNK && FAM == KDA)
        seam_chunk_kda<D>(X, sm, nt, o_first, (int64_t)a.n_chains * dk, c0, dk, nm[0], nm[1], v_zero);
    else if constexpr (CHUNK)
        seam_chunk_bf16<D, FAM, SM, UPDATE_FIRST>(X, sm, nt, o_first, (int64_t)a.n_chains * dk, c0, dk, nm[0],
                                                  nm[1], v_zero);
    else
        seam_tokens<D, FAM>(X, sm, nt, o_first, (int64_t)a.n_chains * dk, c0, c0, v_zero, dk);
}

template <int D, int FAM, typename TIN, bool TREE>
__global__ void __launch_bounds__((TREE ? 2 : 1) * D / 32 * 64)
k_compose_dense(TreeArgs t) {
    const ComposeArgs &a = t.c;
    constexpr bool F32 = std::is_same<TIN, float>::value;
    constexpr int NW = D / 32, RT = D / 16, KB = D / 32;
    constexpr int NWT = (TREE ? 2 : 1) * NW;  // waves in the workgroup
    using TL = DenseTLds<D, F32>;
    constexpr int LDT = TL::LDT;
    constexpr int NV = D * D / 4 / 64 / NWT;  // 16-byte pieces of T per lane
    constexpr int RPW = D / NWT;              // T rows staged by one wave
    __shared__ __attribute__((aligned(16))) char tsm[2][TL::BYTES];
    constexpr bool CHUNK_SEAM = !F32 && fam_dense(FAM);
    // (KDA's chunk seam takes its window pre-decayed)
    __shared__ typename std::conditional<CHUNK_SEAM && FAM == KDA, SeamSmemKda<D>, SeamSmem<D, FAM>>::type sm;
    __shared__ float seam_nm[CHUNK_SEAM ? NWT : 1][2][SEAM_STAGE][9];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int r16 = lane & 15, grp = lane >> 4;
    const int chain = blockIdx.x % a.n_chains;
    int req, j0 = 0, blk = 0;
    if (TREE) {
        const int rb = blockIdx.x / a.n_chains;
        req = rb / t.NB;
        blk = rb % t.NB;
        j0 = blk * t.B;
    } else {
        req = blockIdx.x / a.n_chains;
    }
    const bool isS = !TREE || wv >= NW;  // owns S columns (else T columns)
    // d = 64 and d = 128 run unpadded (dk == D), which makes every offset below
    // a compile-time constant off one per-lane base
    const int dk = D >= 64 ? D : a.dk, c0 = (wv % NW) * 32;
    float *st = a.state + ((int64_t)req * a.n_chains + chain) * dk * dk;
    const int len = a.list_off[req + 1] - a.list_off[req];
    if (TREE && j0 >= len) return;  // uniform over the workgroup
    // this workgroup's entries: e0 .. e0 + m - 1 (list positions j0 ..)
    const int e0 = a.list_off[req] + j0;
    const int m = TREE ? (len - j0 < t.B ? len - j0 : t.B) : len;

    // pair ids and seam starts of 64 entries at a time: lane l holds entry
    // base + l, read back with readlane (no dependent scalar loads per entry)
    int win_base = 0, win_pid = 0;
    int64_t win_sb = -1;
    auto win_load = [&](int b) {
        win_base = b;
        const int idx = b + lane < m ? b + lane : m - 1;
        win_pid = a.pair_id[e0 + idx];
        win_sb = a.has_seam ? a.seam_begin[e0 + idx] : -1;
        __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): settled here, not at every later use
    };
    auto pid_at = [&](int j) -> int64_t { return __builtin_amdgcn_readlane(win_pid, j - win_base); };
    auto sb_at = [&](int j) -> int64_t {
        const uint64_t u = (uint64_t)win_sb;
        const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)u, j - win_base);
        const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(u >> 32), j - win_base);
        return (int64_t)(((uint64_t)hi << 32) | lo);
    };

    f32x4 tpre[NV];
    f32x4 spre[RT][2];  // S_j rows: lane (4q + i, grp) holds row 4 grp + i, columns 4q .. 4q+3 of each tile
    // (the loads, stores and products below take per-lane offsets from a
    // fresh copy of the lane index, not from values held across the loop)
    auto t_load = [&](int j) {
        const float *Tp = a.T + (pid_at(j) * a.n_chains + chain) * a.t_elems;
        const int lf = lane_fresh();
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int item = i * 64 + lf, row = wv * RPW + item / (D / 4), c4 = item % (D / 4);
            if (D >= 64) {
                tpre[i] = *reinterpret_cast<const f32x4 *>(Tp + row * D + 4 * c4);
            } else {
                const f32x4 v = *reinterpret_cast<const f32x4 *>(Tp + (row < dk ? row : dk - 1) * dk +
                                                                 (4 * c4 < dk ? 4 * c4 : dk - 4));
                tpre[i] = (row < dk && 4 * c4 < dk) ? v : f32x4{0.f, 0.f, 0.f, 0.f};
            }
        }
    };
    auto t_put = [&](int buf) {
        const int lf = lane_fresh();
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int item = i * 64 + lf, row = wv * RPW + item / (D / 4), c4 = item % (D / 4);
            if (F32) {
                *reinterpret_cast<f32x4 *>(reinterpret_cast<float *>(tsm[buf]) + row * LDT + 4 * c4) = tpre[i];
            } else {
                // columns permuted within each 32-block so that a lane's A
                // fragment (k = 4grp.., 16+4grp..) is 8 consecutive bf16
                const int sub = c4 % 8, pos = 32 * (c4 / 8) + 8 * (sub % 4) + 4 * (sub / 4);
                bf16x4 h, l;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    h[e] = (bf16)tpre[i][e];
                    l[e] = (bf16)(tpre[i][e] - (float)h[e]);
                }
                bf16 *tr = reinterpret_cast<bf16 *>(tsm[buf]) + row * LDT;
                *reinterpret_cast<bf16x4 *>(tr + pos) = h;
                *reinterpret_cast<bf16x4 *>(tr + D + pos) = l;
            }
        }
    };
    auto s_load = [&](int j) {
        const float *Sp = a.S + (pid_at(j) * a.n_chains + chain) * dk * dk;
        const int lf = lane_fresh(), fr16 = lf & 15, fgrp = lf >> 4;
        const int rw = 4 * fgrp + (fr16 & 3), cl = c0 + 4 * (fr16 >> 2);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
                const int row = 16 * rt + rw, col = cl + 16 * nt;
                if (D >= 64) {
                    spre[rt][nt] = *reinterpret_cast<const f32x4 *>(Sp + row * D + col);
                } else {
                    const f32x4 v = *reinterpret_cast<const f32x4 *>(Sp + (row < dk ? row : dk - 1) * dk +
                                                                     (col < dk ? col : dk - 4));
                    spre[rt][nt] = (row < dk && col < dk) ? v : f32x4{0.f, 0.f, 0.f, 0.f};
                }
            }
    };
    // seam tokens of the next entry, fetched ahead when the whole window fits
    // one staging stage and the gate is a scalar per token
    SeamPrefetch<D, TIN> seam_pf;
    const bool seam_one_stage = !fam_vgate(FAM) && a.has_seam && a.w <= SEAM_STAGE;
    // KDA (bf16 inputs), sequential mode: the next window is fetched ahead
    // too, one channel per thread, and staged in its decayed forms at the
    // seam (in tree mode, eight waves at 256 registers, it would spill)
    constexpr bool KDA_PF = CHUNK_SEAM && FAM == KDA && !TREE;
    // (a prefetched window is staged by KNG threads per channel: every
    // thread of the workgroup)
    constexpr int KNG = NWT * 64 / D;
    KdaSeamPrefetch<D, TIN, KNG> kda_pf;
    const bool kda_one_stage = KDA_PF && a.has_seam && a.w <= SEAM_STAGE;

    f32x4 X[RT][2];
    if (TREE) {
        if (isS) {
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int nt = 0; nt < 2; ++nt) X[rt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
        } else {
            identity_tile<D>(X, c0);
        }
    } else {
        load_tile_buf<D>(X, st, dk, c0);
    }
    if (m > 0) {
        win_load(0);
        t_load(0);
        if (!TREE || F32) s_load(0);
        t_put(0);
        t_load(m > 1 ? 1 : 0);
        if (seam_one_stage) seam_fetch<D, FAM, TIN>(seam_pf, a.x, chain, dk, sb_at(0), a.w);
        if constexpr (KDA_PF)
            if (kda_one_stage) seam_fetch_kda<D, TIN, KNG>(kda_pf, a.x, chain, dk, sb_at(0), a.w);
        __syncthreads();
    }
    for (int j = 0; j < m; ++j) {
        const int e = e0 + j;
        if (j + 2 >= win_base + 64) win_load(j);
        if (a.has_seam) {
            const int64_t sb = sb_at(j);
            if (sb >= 0 && seam_one_stage) {
                // the whole window was fetched ahead: no loop around it, so the
                // compiler's wait counts stay exact through this block
                if constexpr (!fam_vgate(FAM)) {
                    __syncthreads();
                    seam_put<D, FAM, TIN>(sm, seam_pf, dk, a.w);
                    __syncthreads();
                    seam_stage_run<D, FAM, CHUNK_SEAM, decltype(sm), TREE && FAM == GDN>(X, sm, a.w, seam_out(t, isS, e, req, j0 + j, chain, 0, dk), a,
                                                       c0, dk, seam_nm[wv], !isS);
                }
            } else if (sb >= 0 && kda_one_stage) {
                if constexpr (KDA_PF) {
                    __syncthreads();
                    seam_put_kda<D, TIN, KNG>(sm, kda_pf, dk, a.w);
                    __syncthreads();
                    seam_stage_run<D, FAM, CHUNK_SEAM, decltype(sm), TREE && FAM == GDN>(X, sm, a.w, seam_out(t, isS, e, req, j0 + j, chain, 0, dk), a,
                                                       c0, dk, seam_nm[wv], !isS);
                }
            } else if (sb >= 0) {
                for (int s0 = 0; s0 < a.w; s0 += SEAM_STAGE) {
                    const int nt = a.w - s0 < SEAM_STAGE ? a.w - s0 : SEAM_STAGE;
                    __syncthreads();
                    if constexpr (CHUNK_SEAM && FAM == KDA)
                        stage_seam_kda<D, TIN>(sm, a.x, chain, dk, sb + s0, nt);
                    else
                        stage_seam<D, FAM, TIN>(sm, a.x, chain, dk, sb + s0, nt);
                    __syncthreads();
                    seam_stage_run<D, FAM, CHUNK_SEAM, decltype(sm), TREE && FAM == GDN>(X, sm, nt, seam_out(t, isS, e, req, j0 + j, chain, s0, dk), a,
                                                       c0, dk, seam_nm[wv], !isS);
                }
            }
        }
        // S <- T_j S + S_j; the next S_j is requested as soon as this one is in
        // the accumulators.  Tree mode (bf16) instead loads S_j in the S half
        // only, just before the product, and adds it after the product: no
        // S_j registers are held across the seam window, where its eight
        // waves run out of registers
        if (F32) {
            float xv[KB][2][8];
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int nt = 0; nt < 2; ++nt) acc_to_perm(X[2 * kb][nt], X[2 * kb + 1][nt], xv[kb][nt]);
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int nt = 0; nt < 2; ++nt) {
                    const f32x4 sj = quad_transpose(spre[rt][nt], lane);
                    X[rt][nt] = isS ? sj : f32x4{0.f, 0.f, 0.f, 0.f};
                }
            // (past the last entry these re-read the last one: the same loads on
            // every path keep the compiler's wait counts exact)
            const int jn = j + 1 < m ? j + 1 : j;
            s_load(jn);
            if (seam_one_stage) seam_fetch<D, FAM, TIN>(seam_pf, a.x, chain, dk, sb_at(jn), a.w);
            if constexpr (KDA_PF)
                if (kda_one_stage) seam_fetch_kda<D, TIN, KNG>(kda_pf, a.x, chain, dk, sb_at(jn), a.w);
            const float *tf = reinterpret_cast<const float *>(tsm[j & 1]);
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int kb = 0; kb < KB; ++kb) {
                    float tv[8];
                    lds_perm_f(tf, LDT, 16 * rt + r16, 32 * kb, grp, tv);
#pragma unroll
                    for (int nt = 0; nt < 2; ++nt) X[rt][nt] = mma_f32(tv, xv[kb][nt], X[rt][nt]);
                }
        } else {
            bf16x8 xh[KB][2], xl[KB][2];
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int nt = 0; nt < 2; ++nt) {
                    float xv[8];
                    acc_to_perm(X[2 * kb][nt], X[2 * kb + 1][nt], xv);
                    split8(xv, xh[kb][nt], xl[kb][nt]);
                }
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int nt = 0; nt < 2; ++nt)
                    X[rt][nt] = (!TREE && isS) ? quad_transpose(spre[rt][nt], lane) : f32x4{0.f, 0.f, 0.f, 0.f};
            const int jn = j + 1 < m ? j + 1 : j;
            if (!TREE) s_load(jn);
            else if (isS) s_load(j);
            if (seam_one_stage) seam_fetch<D, FAM, TIN>(seam_pf, a.x, chain, dk, sb_at(jn), a.w);
            if constexpr (KDA_PF)
                if (kda_one_stage) seam_fetch_kda<D, TIN, KNG>(kda_pf, a.x, chain, dk, sb_at(jn), a.w);
            const bf16 *th = reinterpret_cast<const bf16 *>(tsm[j & 1]);
            const int lp = lane_fresh(), pr16 = lp & 15, pgrp = lp >> 4;
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int kb = 0; kb < KB; ++kb) {
                    const int off = (16 * rt + pr16) * LDT + 32 * kb + 8 * pgrp;
                    const bf16x8 ah = *reinterpret_cast<const bf16x8 *>(th + off);
                    const bf16x8 al = *reinterpret_cast<const bf16x8 *>(th + D + off);
#pragma unroll
                    for (int nt = 0; nt < 2; ++nt) {
                        X[rt][nt] = mfma(ah, xh[kb][nt], X[rt][nt]);
                        X[rt][nt] = mfma(ah, xl[kb][nt], X[rt][nt]);
                        X[rt][nt] = mfma(al, xh[kb][nt], X[rt][nt]);
                    }
                }
            if (TREE && isS) {
#pragma unroll
                for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                    for (int nt = 0; nt < 2; ++nt) X[rt][nt] += quad_transpose(spre[rt][nt], lane);
            }
        }
        if (!TREE && a.prefix) store_tile_buf<D>(X, a.prefix + ((int64_t)e * a.n_chains + chain) * dk * dk, dk, c0);
        if (j + 1 < m) t_put((j + 1) & 1);  // that buffer's last readers finished entry j - 1
        t_load(j + 2 < m ? j + 2 : m - 1);
        __syncthreads();
    }
    if (TREE) {
        const int64_t agg = (((int64_t)req * t.NB + blk) * a.n_chains + chain) * dk * dk;
        // (fp32 inputs keep the plain stores here: in that instantiation the
        // buffer form spills more, not less)
        if constexpr (F32)
            store_tile<D>(X, (isS ? t.aggS : t.aggT) + agg, dk, dk, c0, dk);
        else
            store_tile_buf<D>(X, (isS ? t.aggS : t.aggT) + agg, dk, c0);
    } else {
        store_tile_buf<D>(X, st, dk, c0);
    }
}

// Sequential compose, lean form, for bf16 inputs of the scalar-gate erasing
// families (DeltaNet, GDN) at d >= 64: the same product and seam chunk as
// k_compose_dense, laid out so that two workgroups share a compute unit and
// hide each other's waits.  One LDS copy of T (hi | lo bf16 rows) and bf16
// seam staging keep a workgroup's LDS under half of the compute unit's; at most
// 256 registers per lane, no spills.  Per entry j:
//   seam:    the state is advanced through entry j's window, staged in LDS
//            during the previous staging phase (chunk form on the matrix
//            cores);
//   product: the state becomes the split B operand, S_j is requested, the
//            accumulators run T_j S from the LDS copy and then take + S_j
//            (the compiler issues the S_j loads at the end of the product,
//            which keeps the product within 256 registers; they arrive with
//            T_{j+1}'s, and the add is folded into the next entry's start);
//   staging: once every wave is past the product, the next window and
//            T_{j+1} are requested and written into LDS (the wait for them is
//            the other workgroup's time on the compute unit).
// Nothing prefetched is held in registers across a phase, which is what keeps
// the register count at 256.
//
// SCAN: the tree compose's second phase on the same machinery.  The entries
// are the request's block aggregates (slot req * NB + b of aggT / aggS, no
// seams), and the state entering each block is stored to sin before its
// product.
// PREFIX: also store the state after every entry to a.prefix (a separate
// instantiation, so that the plain form carries no trace of it).
// TC: compact pairs: T is stored as bf16 T^ with a power-of-two scale per
// (slot, chain), T = sigma T^ (a.T points at the bf16 values, a.t_scale at
// the scales).  T^ is staged as it stands (no split) and the product takes
// two passes, T^ S_hi + T^ S_lo; the scale joins the add of S_j.
template <int D, int FAM, bool SCAN = false, bool PREFIX = false, bool TC = false>
__global__ void __launch_bounds__(D / 32 * 64, 2)
k_compose_lean(TreeArgs targ) {
    static_assert(D >= 64 && (FAM == DELTANET || FAM == GDN), "lean compose: d >= 64, scalar-gate erasing families");
    const ComposeArgs a = targ.c;
    constexpr int NW = D / 32, RT = D / 16, KB = D / 32;
    using TL = DenseTLds<D, false>;
    constexpr int LDT = TL::LDT;
    constexpr int NV = D * D / (TC ? 8 : 4) / 64 / NW;  // 16-byte pieces of T per lane
    constexpr int RPW = D / NW;                         // T rows staged by one wave
    constexpr int dk = D;
    __shared__ __attribute__((aligned(16))) bf16 tsm[D * LDT];
    __shared__ SeamSmemB<D> sm;
    __shared__ float seam_nm[NW][2][SEAM_STAGE][9];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int r16 = lane & 15, grp = lane >> 4;
    const int req = blockIdx.x / a.n_chains, chain = blockIdx.x % a.n_chains;
    const int c0 = wv * 32;
    float *st = a.state + ((int64_t)req * a.n_chains + chain) * dk * dk;
    const int e0 = a.list_off[req];
    const int len = a.list_off[req + 1] - e0;
    const int m = SCAN ? (len + targ.B - 1) / targ.B : len;

    // pair ids and seam starts of 64 entries at a time, read back with readlane
    int win_base = 0, win_pid = 0;
    int64_t win_sb = -1;
    auto win_load = [&](int b) {
        win_base = b;
        const int idx = b + lane < m ? b + lane : m - 1;
        win_pid = SCAN ? req * targ.NB + idx : a.pair_id[e0 + idx];
        win_sb = (a.has_seam && !SCAN) ? a.seam_begin[e0 + idx] : -1;
        __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): settled here, not at every later use
    };
    auto pid_at = [&](int j) -> int64_t { return __builtin_amdgcn_readlane(win_pid, j - win_base); };
    auto sb_at = [&](int j) -> int64_t {
        const uint64_t u = (uint64_t)win_sb;
        const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)u, j - win_base);
        const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(u >> 32), j - win_base);
        return (int64_t)(((uint64_t)hi << 32) | lo);
    };

    // Loads go through buffer views of the slot's T and S: one per-lane
    // offset, the rest compile-time immediates (no per-load address math).
    // T: lane ln of wave wv stages rows wv*RPW + i*(256/D) + ln/(D/4), columns
    // 4 (ln % (D/4)) .. +3, for i < NV.
    constexpr int TROWS = (TC ? 512 : 256) / D;  // rows of T per 64-lane piece
    f32x4 tpre[NV];  // (TC: eight bf16 as raw bits)
    auto t_load = [&](int j, int ln) {
        if constexpr (TC) {
            const auto r = buffer_view(reinterpret_cast<const bf16 *>(a.T) + (pid_at(j) * a.n_chains + chain) * D * D,
                                       D * D * 2);
            const int voff = ((wv * RPW + (int)((unsigned)ln / (D / 8))) * D + 8 * (int)((unsigned)ln % (D / 8))) * 2;
#pragma unroll
            for (int i = 0; i < NV; ++i)
                tpre[i] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, i * TROWS * D * 2, 0));
            return;
        }
        const auto r = buffer_view(a.T + (pid_at(j) * a.n_chains + chain) * a.t_elems, D * D * 4);
        const int voff = ((wv * RPW + (int)((unsigned)ln / (D / 4))) * D + 4 * (int)((unsigned)ln % (D / 4))) * 4;
#pragma unroll
        for (int i = 0; i < NV; ++i)
            tpre[i] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, i * TROWS * D * 4, 0));
    };
    auto t_put = [&](int ln) {
        if constexpr (TC) {
            // columns 8 c8 .. 8 c8 + 7 are the 4-column groups 2 c8 and 2 c8 + 1,
            // placed as the fp32 path places them (hi half of the row only)
            const int c8 = (int)((unsigned)ln % (D / 8));
            auto pos = [](int c4) { const int sub = c4 % 8; return 32 * (c4 / 8) + 8 * (sub % 4) + 4 * (sub / 4); };
            bf16 *tr = tsm + (wv * RPW + (int)((unsigned)ln / (D / 8))) * LDT;
#pragma unroll
            for (int i = 0; i < NV; ++i) {
                const u32x4 u = __builtin_bit_cast(u32x4, tpre[i]);
                *reinterpret_cast<u32x2 *>(tr + i * TROWS * LDT + pos(2 * c8)) = u32x2{u[0], u[1]};
                *reinterpret_cast<u32x2 *>(tr + i * TROWS * LDT + pos(2 * c8 + 1)) = u32x2{u[2], u[3]};
            }
            return;
        }
        // columns permuted within each 32-block so that a lane's A fragment
        // (k = 4grp.., 16+4grp..) is 8 consecutive bf16
        const int c4 = (int)((unsigned)ln % (D / 4)), sub = c4 % 8;
        const int pos = 32 * (c4 / 8) + 8 * (sub % 4) + 4 * (sub / 4);
        bf16 *tr = tsm + (wv * RPW + (int)((unsigned)ln / (D / 4))) * LDT + pos;
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            uint32_t h0, l0, h1, l1;
            split2(tpre[i][0], tpre[i][1], h0, l0);
            split2(tpre[i][2], tpre[i][3], h1, l1);
            *reinterpret_cast<u32x2 *>(tr + i * TROWS * LDT) = u32x2{h0, h1};
            *reinterpret_cast<u32x2 *>(tr + i * TROWS * LDT + D) = u32x2{l0, l1};
        }
    };
    // S_j straight into the C layout: spre[rt][nt][jj] = S_j[16 rt + 4 grp + jj][c0 + 16 nt + r16]
    float spre[RT][2][4];
    auto s_load = [&](int j, int ln) {
        const auto r = buffer_view(a.S + (pid_at(j) * a.n_chains + chain) * dk * dk, D * D * 4);
        const int voff = ((int)((unsigned)ln >> 4) * 4 * D + c0 + (int)((unsigned)ln & 15)) * 4;
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int nt = 0; nt < 2; ++nt)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj)
                    spre[rt][nt][jj] = __builtin_bit_cast(
                        float, __builtin_amdgcn_raw_buffer_load_b32(r, voff, ((16 * rt + jj) * D + 16 * nt) * 4, 0));
    };
    SeamPrefetch<D, bf16> seam_pf;
    const bool seam_one_stage = a.has_seam && a.w <= SEAM_STAGE;

    f32x4 X[RT][2];
    {
        const auto r = buffer_view(st, D * D * 4);
        const int voff = (grp * 4 * D + c0 + r16) * 4;
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int nt = 0; nt < 2; ++nt)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj)
                    X[rt][nt][jj] = __builtin_bit_cast(
                        float, __builtin_amdgcn_raw_buffer_load_b32(r, voff, ((16 * rt + jj) * D + 16 * nt) * 4, 0));
    }
    if (m > 0) {
        win_load(0);
        if (seam_one_stage) seam_fetch<D, FAM, bf16>(seam_pf, a.x, chain, dk, sb_at(0), a.w);
        t_load(0, lane);
        if (seam_one_stage) seam_put_b<D, FAM>(sm, seam_pf, a.w);
        t_put(lane);
        __syncthreads();
    }
    for (int j = 0; j < m; ++j) {
        const int e = e0 + j;
        if (j + 2 >= win_base + 64) win_load(j);
        const int ln = lane_fresh(), lr16 = ln & 15, lgrp = ln >> 4;
        if constexpr (SCAN) {
            // the state entering block j
            const auto r = buffer_view(targ.sin + (((int64_t)req * targ.NB + j) * a.n_chains + chain) * dk * dk,
                                       D * D * 4);
            const int voff = ((int)((unsigned)ln >> 4) * 4 * D + c0 + (int)((unsigned)ln & 15)) * 4;
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int nt = 0; nt < 2; ++nt)
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) {
                        const float v = X[rt][nt][jj];
                        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), r, voff,
                                                              ((16 * rt + jj) * D + 16 * nt) * 4, 0);
                    }
        }
        if (a.has_seam && !SCAN) {
            const int64_t sb = sb_at(j);
            float *o_first = a.o + ((int64_t)e * a.w * a.n_chains + chain) * dk;
            if (sb >= 0 && seam_one_stage) {
                // (staged during the previous staging phase)  The window is a
                // dependent chain; the other workgroup's waves on the SIMD are
                // mostly in their product or staging, so the window goes first
                // at issue: 1.281-1.289 against 1.298-1.308 ms on 960 GDN
                // chains (d = 128, 48 entries) in the same calls.
                __builtin_amdgcn_s_setprio(1);
                seam_chunk_bf16<D, FAM>(X, sm, a.w, o_first, (int64_t)a.n_chains * dk, c0, dk, seam_nm[wv][0],
                                        seam_nm[wv][1]);
                __builtin_amdgcn_s_setprio(0);
                // the window's output stores complete before S_j is requested
                // (the memory counter is counted in issue order): 1.321-1.323
                // against 1.338-1.343 ms on 960 GDN chains (d = 128, 48
                // entries) in the same call
                __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
            } else if (sb >= 0) {
                for (int s0 = 0; s0 < a.w; s0 += SEAM_STAGE) {
                    const int nt = a.w - s0 < SEAM_STAGE ? a.w - s0 : SEAM_STAGE;
                    __syncthreads();
                    stage_seam_b<D, FAM>(sm, a.x, chain, sb + s0, nt);
                    __syncthreads();
                    seam_chunk_bf16<D, FAM>(X, sm, nt, o_first + (int64_t)s0 * a.n_chains * dk,
                                            (int64_t)a.n_chains * dk, c0, dk, seam_nm[wv][0], seam_nm[wv][1]);
                }
            }
        }
        // S <- T_j S + S_j
        bf16x8 xh[KB][2], xl[KB][2];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
                float xv[8];
                acc_to_perm(X[2 * kb][nt], X[2 * kb + 1][nt], xv);
                split8(xv, xh[kb][nt], xl[kb][nt]);
            }
        s_load(j, ln);
        const float sig = TC ? a.t_scale[pid_at(j) * a.n_chains + chain] : 1.f;
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) X[rt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
        // (past the last entry these re-read the last one: the same loads on
        // every path keep the compiler's wait counts exact)
        const int jn = j + 1 < m ? j + 1 : j;
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                const int off = (16 * rt + lr16) * LDT + 32 * kb + 8 * lgrp;
                const bf16x8 ah = *reinterpret_cast<const bf16x8 *>(tsm + off);
                if constexpr (TC) {
#pragma unroll
                    for (int nt = 0; nt < 2; ++nt) {
                        X[rt][nt] = mfma(ah, xh[kb][nt], X[rt][nt]);
                        X[rt][nt] = mfma(ah, xl[kb][nt], X[rt][nt]);
                    }
                } else {
                    const bf16x8 al = *reinterpret_cast<const bf16x8 *>(tsm + D + off);
#pragma unroll
                    for (int nt = 0; nt < 2; ++nt) {
                        X[rt][nt] = mfma(ah, xh[kb][nt], X[rt][nt]);
                        X[rt][nt] = mfma(ah, xl[kb][nt], X[rt][nt]);
                        X[rt][nt] = mfma(al, xh[kb][nt], X[rt][nt]);
                    }
                }
            }
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int nt = 0; nt < 2; ++nt)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    if constexpr (TC)
                        X[rt][nt][jj] = sig * X[rt][nt][jj] + spre[rt][nt][jj];
                    else
                        X[rt][nt][jj] += spre[rt][nt][jj];
                }
        if constexpr (PREFIX && !SCAN) {
            // the state after entry e
            const auto r = buffer_view(a.prefix + ((int64_t)e * a.n_chains + chain) * dk * dk, D * D * 4);
            const int voff = ((int)((unsigned)ln >> 4) * 4 * D + c0 + (int)((unsigned)ln & 15)) * 4;
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int nt = 0; nt < 2; ++nt)
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) {
                        const float v = X[rt][nt][jj];
                        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), r, voff,
                                                              ((16 * rt + jj) * D + 16 * nt) * 4, 0);
                    }
        }
        // (every product is issued before the barrier, so that the B operands
        // are dead in the staging phase)
        __builtin_amdgcn_sched_barrier(0);
        __syncthreads();  // every wave is past T_j and the seam staging
        __builtin_amdgcn_sched_barrier(0);
        // Staging.  The next window goes straight to LDS: its loads are in
        // flight together with T's, and nothing holds them across a barrier.
        const int ln2 = lane_fresh();
        if (seam_one_stage) seam_fetch<D, FAM, bf16>(seam_pf, a.x, chain, dk, sb_at(jn), a.w);
        t_load(jn, ln2);
        if (seam_one_stage) seam_put_b<D, FAM>(sm, seam_pf, a.w);
        __builtin_amdgcn_sched_barrier(0);
        t_put(ln2);
        __syncthreads();  // T_{j+1} in place
    }
    {
        const int ln = lane_fresh();
        const auto r = buffer_view(st, D * D * 4);
        const int voff = ((int)((unsigned)ln >> 4) * 4 * D + c0 + (int)((unsigned)ln & 15)) * 4;
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int nt = 0; nt < 2; ++nt)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    // (the element is copied out first: this compiler's
                    // __builtin_bit_cast of a vector element reads element 0)
                    const float v = X[rt][nt][jj];
                    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), r, voff,
                                                          ((16 * rt + jj) * D + 16 * nt) * 4, 0);
                }
    }
}

// ---- tree mode --------------------------------------------------------------

// phase 1: block aggregates, block-local seam outputs and pulled-back queries
template <int D, int FAM, typename TIN>
__global__ void __launch_bounds__(2 * D / 32 * 64)
k_tree_block(TreeArgs t) {
    constexpr bool F32 = std::is_same<TIN, float>::value;
    const ComposeArgs &a = t.c;
    __shared__ SeamSmem<D, FAM> sm;
    const int wv = threadIdx.x >> 6;
    const int chain = blockIdx.x % a.n_chains;
    const int rb = blockIdx.x / a.n_chains, req = rb / t.NB, blk = rb % t.NB;
    const int dk = a.dk;
    const int e0 = a.list_off[req], len = a.list_off[req + 1] - e0;
    const int j0 = blk * t.B;
    if (j0 >= len) return;  // uniform over the workgroup
    const int j1 = j0 + t.B < len ? j0 + t.B : len;
    const bool isS = wv >= D / 32;
    const int c0 = (isS ? wv - D / 32 : wv) * 32;
    f32x4 X[D / 16][2];
    if (isS) {
#pragma unroll
        for (int rt = 0; rt < D / 16; ++rt)
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) X[rt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    } else {
        identity_tile<D>(X, c0);
    }
    // a window that fits one stage is fetched one entry ahead into registers
    SeamPrefetch<D, TIN> pf;
    const bool one = a.has_seam && a.w <= SEAM_STAGE;
    // (the seam tokens, gamma included, exist only when the call has seams)
    const float rg = (FAM == RETNET && one) ? a.x.gamma[chain] : 1.f;
    if (one) seam_fetch<D, FAM, TIN>(pf, a.x, chain, dk, a.seam_begin[e0 + j0], a.w);
    for (int j = j0; j < j1; ++j) {
        const int e = e0 + j;
        if (a.has_seam && one) {
            const int64_t sb = a.seam_begin[e];
            if (sb >= 0) {
                __syncthreads();
                seam_put<D, FAM, TIN>(sm, pf, dk, a.w, rg);
                __syncthreads();
            }
            seam_fetch<D, FAM, TIN>(pf, a.x, chain, dk, j + 1 < j1 ? a.seam_begin[e + 1] : -1, a.w);
            if (sb >= 0) {
                float *o_first = isS ? a.o + ((int64_t)e * a.w * a.n_chains + chain) * dk
                                     : t.pvec + (((int64_t)req * t.max_list + j) * a.w * a.n_chains + chain) * dk;
                seam_tokens<D, FAM>(X, sm, a.w, o_first, (int64_t)a.n_chains * dk, c0, c0, !isS, dk);
            }
        } else if (a.has_seam) {
            const int64_t sb = a.seam_begin[e];
            if (sb >= 0) {
                for (int s0 = 0; s0 < a.w; s0 += SEAM_STAGE) {
                    const int nt = a.w - s0 < SEAM_STAGE ? a.w - s0 : SEAM_STAGE;
                    __syncthreads();
                    stage_seam<D, FAM, TIN>(sm, a.x, chain, dk, sb + s0, nt);
                    __syncthreads();
                    float *o_first =
                        isS ? a.o + (((int64_t)e * a.w + s0) * a.n_chains + chain) * dk
                            : t.pvec + ((((int64_t)req * t.max_list + j) * a.w + s0) * a.n_chains + chain) * dk;
                    seam_tokens<D, FAM>(X, sm, nt, o_first, (int64_t)a.n_chains * dk, c0, c0, !isS, dk);
                }
            }
        }
        const int64_t slot = a.pair_id[e];
        const float *Tp = a.T + (slot * a.n_chains + chain) * a.t_elems;
        const float *Sp = isS ? a.S + (slot * a.n_chains + chain) * dk * dk : nullptr;
        if constexpr (fam_dense(FAM))
            apply_dense_T<D, F32>(X, Tp, dk, Sp, c0);
        else
            apply_diag_T_buf<D>(X, Tp, a.t_elems, dk, Sp, c0);
    }
    const int64_t agg = (((int64_t)req * t.NB + blk) * a.n_chains + chain) * dk * dk;
    store_tile_buf<D>(X, (isS ? t.aggS : t.aggT) + agg, dk, c0);
}

// phase 2: sequential scan over the block aggregates.  DIAG: the family's T
// is diagonal, so is every block aggregate's, and its diagonal (stride dk + 1
// in the dense aggregate) scales the rows.
template <int D, typename TIN, bool DIAG>
__global__ void __launch_bounds__(D / 32 * 64)
k_tree_scan(TreeArgs t) {
    constexpr bool F32 = std::is_same<TIN, float>::value;
    const ComposeArgs &a = t.c;
    const int wv = threadIdx.x >> 6;
    const int req = blockIdx.x / a.n_chains, chain = blockIdx.x % a.n_chains;
    const int dk = a.dk, c0 = wv * 32;
    float *st = a.state + ((int64_t)req * a.n_chains + chain) * dk * dk;
    f32x4 X[D / 16][2];
    const int len = a.list_off[req + 1] - a.list_off[req];
    const int nb = (len + t.B - 1) / t.B;
    if constexpr (DIAG) {
        load_tile_buf<D>(X, st, dk, c0);
        for (int b = 0; b < nb; ++b) {
            const int64_t agg = (((int64_t)req * t.NB + b) * a.n_chains + chain) * dk * dk;
            store_tile_buf<D>(X, t.sin + agg, dk, c0);
            apply_diag_agg<D>(X, t.aggT + agg, t.aggS + agg, dk, c0);
        }
        store_tile_buf<D>(X, st, dk, c0);
    } else {
        load_tile<D>(X, st, dk, dk, c0, dk);
        for (int b = 0; b < nb; ++b) {
            const int64_t agg = (((int64_t)req * t.NB + b) * a.n_chains + chain) * dk * dk;
            store_tile<D>(X, t.sin + agg, dk, dk, c0, dk);
            apply_dense_T<D, F32>(X, t.aggT + agg, dk, t.aggS + agg, c0);
        }
        store_tile<D>(X, st, dk, dk, c0, dk);
    }
}

// phase 3: o_t += S_in^T p_t for the block's seam tokens
template <int D>
__global__ void __launch_bounds__(D / 32 * 64)
k_tree_fix(TreeArgs t) {
    constexpr int RT = D / 16;
    const ComposeArgs &a = t.c;
    __shared__ float sp[SEAM_STAGE][D];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int r16 = lane & 15, grp = lane >> 4;
    const int chain = blockIdx.x % a.n_chains;
    const int rb = blockIdx.x / a.n_chains, req = rb / t.NB, blk = rb % t.NB;
    const int dk = a.dk, c0 = wv * 32;
    const int e0 = a.list_off[req], len = a.list_off[req + 1] - e0;
    const int j0 = blk * t.B;
    if (j0 >= len) return;
    const int j1 = j0 + t.B < len ? j0 + t.B : len;
    f32x4 X[RT][2];
    load_tile<D>(X, t.sin + (((int64_t)req * t.NB + blk) * a.n_chains + chain) * dk * dk, dk, dk, c0, dk);
    for (int j = j0; j < j1; ++j) {
        const int e = e0 + j;
        if (a.seam_begin[e] < 0) continue;
        for (int s0 = 0; s0 < a.w; s0 += SEAM_STAGE) {
            const int nt = a.w - s0 < SEAM_STAGE ? a.w - s0 : SEAM_STAGE;
            __syncthreads();
            for (int item = tid; item < SEAM_STAGE * D; item += blockDim.x) {
                const int ts = item / D, i = item % D;
                sp[ts][i] = (ts < nt && i < dk)
                                ? t.pvec[((((int64_t)req * t.max_list + j) * a.w + s0 + ts) * a.n_chains + chain) * dk + i]
                                : 0.f;
            }
            __syncthreads();
            float *o_first = a.o + (((int64_t)e * a.w + s0) * a.n_chains + chain) * dk;
            for (int ts = 0; ts < nt; ++ts) {
                float o[2] = {0.f, 0.f};
#pragma unroll
                for (int rt = 0; rt < RT; ++rt) {
                    const f32x4 p4 = *reinterpret_cast<const f32x4 *>(&sp[ts][16 * rt + 4 * grp]);
#pragma unroll
                    for (int nt2 = 0; nt2 < 2; ++nt2)
#pragma unroll
                        for (int jj = 0; jj < 4; ++jj) o[nt2] += p4[jj] * X[rt][nt2][jj];
                }
#pragma unroll
                for (int nt2 = 0; nt2 < 2; ++nt2) {
                    const float ov = wave_sum16x(o[nt2]);
                    const int col = c0 + 16 * nt2 + r16;
                    if (grp == 0 && col < dk) o_first[(int64_t)ts * a.n_chains * dk + col] += ov;
                }
            }
        }
    }
}

// phase 3 on the matrix cores (bf16 inputs, d >= 64): the block's seam
// tokens, 64 at a time, as rows of P (their pulled-back queries), so that
// O = P S_in is one product per wave on its 32 columns; o += O.  P is staged
// once per workgroup through LDS as hi | lo bf16 rows (the layout the lean
// compose uses for T); S_in is the split B operand.
template <int D>
__global__ void __launch_bounds__(D / 32 * 64)
k_tree_fix_mma(TreeArgs t) {
    constexpr int RT = D / 16, KB = D / 32, NW = D / 32;
    constexpr int PR = 64;               // token rows per pass
    constexpr int LDP = 2 * D + 8;       // bf16 per staged row: [hi | lo] + pad
    constexpr int NV = PR * D / 4 / 64 / NW;  // 16-byte pieces of P per lane
    __shared__ __attribute__((aligned(16))) bf16 psm[PR * LDP];
    const ComposeArgs &a = t.c;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int r16 = lane & 15, grp = lane >> 4;
    const int chain = blockIdx.x % a.n_chains;
    const int rb = blockIdx.x / a.n_chains, req = rb / t.NB, blk = rb % t.NB;
    constexpr int dk = D;
    const int c0 = wv * 32;
    const int e0 = a.list_off[req], len = a.list_off[req + 1] - e0;
    const int j0 = blk * t.B;
    if (j0 >= len) return;  // uniform over the workgroup
    const int j1 = j0 + t.B < len ? j0 + t.B : len;
    const int nrows = (j1 - j0) * a.w;
    // S_in columns c0 .. c0+31 in the C layout, split as the B operand
    bf16x8 xh[KB][2], xl[KB][2];
    {
        const auto r = buffer_view(t.sin + (((int64_t)req * t.NB + blk) * a.n_chains + chain) * dk * dk, D * D * 4);
        const int voff = (grp * 4 * D + c0 + r16) * 4;
        f32x4 X[RT][2];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int nt = 0; nt < 2; ++nt)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj)
                    X[rt][nt][jj] = __builtin_bit_cast(
                        float, __builtin_amdgcn_raw_buffer_load_b32(r, voff, ((16 * rt + jj) * D + 16 * nt) * 4, 0));
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
                float xv[8];
                acc_to_perm(X[2 * kb][nt], X[2 * kb + 1][nt], xv);
                split8(xv, xh[kb][nt], xl[kb][nt]);
            }
    }
    for (int r0 = 0; r0 < nrows; r0 += PR) {
        // stage P rows r0 .. r0 + 63 (token s of entry j0 + r / w); rows past
        // the block or of entries without a seam are zero
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int item = (i * NW + wv) * 64 + lane, row = item / (D / 4), c4 = item % (D / 4);
            const int r = r0 + row, j = j0 + r / a.w, sidx = r % a.w;
            const bool ok = r < nrows && a.seam_begin[e0 + (j < j1 ? j : j1 - 1)] >= 0;
            const int jc = ok ? j : j0, sc = ok ? sidx : 0;
            const f32x4 v = *reinterpret_cast<const f32x4 *>(
                t.pvec + ((((int64_t)req * t.max_list + jc) * a.w + sc) * a.n_chains + chain) * dk + 4 * c4);
            const int sub = c4 % 8, pos = 32 * (c4 / 8) + 8 * (sub % 4) + 4 * (sub / 4);
            uint32_t h0, l0, h1, l1;
            split2(ok ? v[0] : 0.f, ok ? v[1] : 0.f, h0, l0);
            split2(ok ? v[2] : 0.f, ok ? v[3] : 0.f, h1, l1);
            *reinterpret_cast<u32x2 *>(psm + row * LDP + pos) = u32x2{h0, h1};
            *reinterpret_cast<u32x2 *>(psm + row * LDP + D + pos) = u32x2{l0, l1};
        }
        __syncthreads();
        // O = P S_in for this wave's columns, then o += O
#pragma unroll
        for (int rt = 0; rt < PR / 16; ++rt) {
            f32x4 O[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                const int off = (16 * rt + r16) * LDP + 32 * kb + 8 * grp;
                const bf16x8 ah = *reinterpret_cast<const bf16x8 *>(psm + off);
                const bf16x8 al = *reinterpret_cast<const bf16x8 *>(psm + D + off);
#pragma unroll
                for (int nt = 0; nt < 2; ++nt) {
                    O[nt] = mfma(ah, xh[kb][nt], O[nt]);
                    O[nt] = mfma(ah, xl[kb][nt], O[nt]);
                    O[nt] = mfma(al, xh[kb][nt], O[nt]);
                }
            }
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int r = r0 + 16 * rt + 4 * grp + jj, j = j0 + r / a.w, sidx = r % a.w;
                if (r < nrows && a.seam_begin[e0 + (j < j1 ? j : j1 - 1)] >= 0) {
                    float *op = a.o + (((int64_t)(e0 + j) * a.w + sidx) * a.n_chains + chain) * dk + c0 + r16;
#pragma unroll
                    for (int nt = 0; nt < 2; ++nt) op[16 * nt] += O[nt][jj];
                }
            }
        }
        __syncthreads();
    }
}

// Entry offsets of every (request, block) as its own list: block b of request
// r holds entries list_off[r] + b B .. list_off[r] + min((b + 1) B, len) - 1,
// so consecutive blocks share their bounds and blocks past a request's end
// are empty.  A sequential compose over these lists, started from the states
// entering each block, re-walks the blocks in parallel.
__global__ void k_block_offsets(const int32_t *list_off, int n_req, int B, int NB, int32_t *blk_off) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n_req * NB) {
        const int r = i / NB, b = i % NB;
        const int len = list_off[r + 1] - list_off[r];
        blk_off[i] = list_off[r] + (b * B < len ? b * B : len);
    }
    if (i == 0) blk_off[n_req * NB] = list_off[n_req];
}

// ---- the library's own tree workspace ------------------------------------------
// For callers that cannot allocate device memory: a fixed-size workspace in
// the code object, one copy per GPU, held until the process ends.  Host code
// never passes the array's name to a kernel (on the host that name is only a
// stand-in); the device address comes from hipGetSymbolAddress, once per
// device, and is kept per device.
static __device__ __align__(256) char scratch[kStaticWorkspaceBytes];

hipError_t static_workspace(void **ptr) {
    static std::mutex mu;
    static void *addr[kMaxDevices] = {};
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        addr[dev] = p;
    }
    *ptr = addr[dev];
    return hipSuccess;
}

// ---- launchers ----------------------------------------------------------------

#define HY_DISPATCH_FAMILY(FN, ARGS, D, TIN)          \
    switch (family) {                                \
    case LINEAR: return FN<D, LINEAR, TIN> ARGS;     \
    case RETNET: return FN<D, RETNET, TIN> ARGS;     \
    case MAMBA2: return FN<D, MAMBA2, TIN> ARGS;     \
    case GLA: return FN<D, GLA, TIN> ARGS;           \
    case DELTANET: return FN<D, DELTANET, TIN> ARGS; \
    case GDN: return FN<D, GDN, TIN> ARGS;           \
    case KDA: return FN<D, KDA, TIN> ARGS;           \
    }                                                \
    return hipErrorInvalidValue;

template <int D, int FAM, typename TIN>
static hipError_t launch_compose(const ComposeArgs &a, int n_req, hipStream_t st) {
    const dim3 grid((unsigned)(n_req * (int64_t)a.n_chains)), block(D / 32 * 64);
    if constexpr (std::is_same<TIN, bf16>::value && D >= 64 && (FAM == DELTANET || FAM == GDN)) {
        TreeArgs t{};
        t.c = a;
        if (a.prefix)
            hipLaunchKernelGGL((k_compose_lean<D, FAM, false, true>), grid, block, 0, st, t);
        else
            hipLaunchKernelGGL((k_compose_lean<D, FAM, false, false>), grid, block, 0, st, t);
    } else if constexpr (fam_dense(FAM)) {
        TreeArgs t{};
        t.c = a;
        hipLaunchKernelGGL((k_compose_dense<D, FAM, TIN, false>), grid, block, 0, st, t);
    } else
        hipLaunchKernelGGL((k_compose_seq<D, FAM, TIN>), grid, block, 0, st, a);
    return hipGetLastError();
}

hipError_t compose_seq_compact(const ComposeArgs &a, int family, int D, int n_req, hipStream_t st) {
    const dim3 grid((unsigned)(n_req * (int64_t)a.n_chains)), block(D / 32 * 64);
    TreeArgs t{};
    t.c = a;
#define HY_COMPACT(DD, FF)                                                                                   \
    if (a.prefix)                                                                                          \
        hipLaunchKernelGGL((k_compose_lean<DD, FF, false, true, true>), grid, block, 0, st, t);            \
    else                                                                                                   \
        hipLaunchKernelGGL((k_compose_lean<DD, FF, false, false, true>), grid, block, 0, st, t);           \
    return hipGetLastError();
    if (D == 128 && family == GDN) { HY_COMPACT(128, GDN) }
    if (D == 128 && family == DELTANET) { HY_COMPACT(128, DELTANET) }
    if (D == 64 && family == GDN) { HY_COMPACT(64, GDN) }
    if (D == 64 && family == DELTANET) { HY_COMPACT(64, DELTANET) }
#undef HY_COMPACT
    return hipErrorInvalidValue;
}

template <int D, int FAM, typename TIN>
static hipError_t launch_seam(const SeamArgs &a, int n_items, hipStream_t st) {
    hipLaunchKernelGGL((k_seam_advance<D, FAM, TIN>), dim3((unsigned)(n_items * (int64_t)a.n_chains)), dim3(D / 32 * 64),
                       0, st, a);
    return hipGetLastError();
}

template <int D, int FAM, typename TIN>
static hipError_t launch_tree(const TreeArgs &t, int n_req, hipStream_t st) {
    const unsigned blocks = (unsigned)((int64_t)n_req * t.NB * t.c.n_chains);
    if constexpr (fam_dense(FAM))
        hipLaunchKernelGGL((k_compose_dense<D, FAM, TIN, true>), dim3(blocks), dim3(2 * D / 32 * 64), 0, st, t);
    else
        hipLaunchKernelGGL((k_tree_block<D, FAM, TIN>), dim3(blocks), dim3(2 * D / 32 * 64), 0, st, t);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    if constexpr (std::is_same<TIN, bf16>::value && D >= 64 && fam_dense(FAM)) {
        // the scan over dense block aggregates is a seam-free sequential
        // compose of them (any dense family: no family-specific step remains)
        TreeArgs ts = t;
        ts.c.T = t.aggT;
        ts.c.S = t.aggS;
        ts.c.t_elems = (int64_t)t.c.dk * t.c.dk;
        ts.c.has_seam = 0;
        hipLaunchKernelGGL((k_compose_lean<D, GDN, true>), dim3((unsigned)(n_req * (int64_t)t.c.n_chains)),
                           dim3(D / 32 * 64), 0, st, ts);
    } else {
        hipLaunchKernelGGL((k_tree_scan<D, TIN, !fam_dense(FAM)>), dim3((unsigned)(n_req * (int64_t)t.c.n_chains)),
                           dim3(D / 32 * 64), 0, st, t);
    }
    if ((err = hipGetLastError()) != hipSuccess) return err;
    if (t.c.prefix) {
        // The states after every entry: each block is re-walked from the state
        // entering it by the sequential compose, which also writes its seam
        // outputs whole (so the fix-up is not needed).
        const int nblk = n_req * t.NB;
        hipLaunchKernelGGL(k_block_offsets, dim3((unsigned)((nblk + 256) / 256)), dim3(256), 0, st, t.c.list_off, n_req,
                           t.B, t.NB, t.blk_off);
        if ((err = hipGetLastError()) != hipSuccess) return err;
        ComposeArgs rw = t.c;
        rw.list_off = t.blk_off;
        rw.state = t.sin;
        return launch_compose<D, FAM, TIN>(rw, nblk, st);
    }
    if (t.c.has_seam) {
        if constexpr (std::is_same<TIN, bf16>::value && D >= 64)
            hipLaunchKernelGGL((k_tree_fix_mma<D>), dim3(blocks), dim3(D / 32 * 64), 0, st, t);
        else
            hipLaunchKernelGGL((k_tree_fix<D>), dim3(blocks), dim3(D / 32 * 64), 0, st, t);
        err = hipGetLastError();
    }
    return err;
}

template <int D, typename TIN>
static hipError_t compose_fam(const ComposeArgs &a, int family, int n_req, hipStream_t st) {
    HY_DISPATCH_FAMILY(launch_compose, (a, n_req, st), D, TIN)
}
template <int D, typename TIN>
static hipError_t seam_fam(const SeamArgs &a, int family, int n_items, hipStream_t st) {
    HY_DISPATCH_FAMILY(launch_seam, (a, n_items, st), D, TIN)
}
template <int D, typename TIN>
static hipError_t tree_fam(const TreeArgs &t, int family, int n_req, hipStream_t st) {
    HY_DISPATCH_FAMILY(launch_tree, (t, n_req, st), D, TIN)
}

#define HY_DISPATCH_D(FN, ...)                                                               \
    switch (D) {                                                                             \
    case 32: return bf16_in ? FN<32, bf16>(__VA_ARGS__) : FN<32, float>(__VA_ARGS__);        \
    case 64: return bf16_in ? FN<64, bf16>(__VA_ARGS__) : FN<64, float>(__VA_ARGS__);        \
    case 128: return bf16_in ? FN<128, bf16>(__VA_ARGS__) : FN<128, float>(__VA_ARGS__);     \
    }                                                                                        \
    return hipErrorInvalidValue;

hipError_t compose_seq(const ComposeArgs &a, int family, bool bf16_in, int D, int n_req, hipStream_t st) {
    HY_DISPATCH_D(compose_fam, a, family, n_req, st)
}

hipError_t seam_advance(const SeamArgs &a, int family, bool bf16_in, int D, int n_items, hipStream_t st) {
    HY_DISPATCH_D(seam_fam, a, family, n_items, st)
}

hipError_t compose_tree(const TreeArgs &t, int family, bool bf16_in, int D, int n_req, hipStream_t st) {
    HY_DISPATCH_D(tree_fam, t, family, n_req, st)
}

}  // namespace hy
