// bwd_dq.hpp -- query-outer pass of the FA2 backward on gfx950 matrix cores:
// dQ (unscaled, fp32) for bf16 and fp16, head dims 64 and 128.
//
// FA2 chapter 16 sec 16.3 weighs adding dQ partials with global atomics
// against a second pass.  On MI355X the fp32 atomics run at about 340 G/s
// (all of them execute beyond the L2), so one partial per (key block, query
// tile) caps the whole backward far below the matrix-core rate.  This pass
// instead gives each work item 256 query rows and loops over all key blocks,
// recomputing S = scale Q K^T, P = exp(S - L) (sec 16.4), dP = dO V^T and
// dS = P (dP - D) (sec 16.1), and accumulating dQ = dS K in registers; each
// dq_accum row is written once, with plain stores.  Under the causal mask the
// key loop stops at the diagonal (sec 16.8 item 2).
//
// gfx950 mapping: a persistent grid (one workgroup per CU, each running a
// fixed list of work items with their key blocks back to back, see dq_run);
// 8 waves, two per SIMD, in two roles that overlap on each SIMD:
//   * score waves 0..3 own queries [64 s, 64 s + 64) of the block as two
//     groups of 32; their Q^T and dO^T B-operand fragments (d / 16 of each
//     per group), L and D stay in registers.  Per key block of 32 they form S^T = K Q^T and
//     dP^T = V dO^T for both groups (key on rows, query on lanes; each K or V
//     fragment read from LDS feeds two products), take the exponentials of S
//     while the dP products issue, then dS = P (dP - D), and store dS (16-bit)
//     to LDS in their own register order, one 1 KiB slab per (16-key step,
//     query group);
//   * gradient wave 4 + g owns 64 columns of d of dQ for 128 queries
//     (d = 128: queries [128 (g / 2), +128), columns [64 (g % 2), +64)) or
//     64 queries (d = 64: queries [64 g, +64), all columns); accumulators
//     in registers.  One key block behind, it reads the K operand of that
//     block (key on the contraction index) with ds_read_b64_tr_b16 -- each
//     fragment feeds one product per query group of the wave -- and dS
//     straight from the slabs, each slab feeding two products;
//   * K blocks rotate through four LDS buffers (score waves read block p,
//     gradient waves block p - 1, the copies of block p + 1, issued one
//     phase earlier, complete before the phase's barrier, and direct-to-LDS
//     copies of block p + 2 go out spread over the gradient steps), V blocks
//     through three, dS through two (88 KiB at d = 128, 60 KiB at d = 64).
//     One barrier per block;
//   * rows at or beyond N are staged as copies of row N - 1; in the last key
//     block their P is forced to 0, and query rows at or beyond N are not
//     stored.
#pragma once

#include <type_traits>

#include "mfma_common.hpp"

namespace fa {
namespace dqp {

using namespace mf;

constexpr int BQ = 256;                  // queries per workgroup
constexpr int BK = 32;                   // keys per block
constexpr int NWAVE = 8;
constexpr int QG = BQ / 32;              // 32-query groups of a workgroup
constexpr int SLAB = 1024;               // one 32-query x 16-key 16-bit operand, lane order
constexpr int DSB = 2 * QG * SLAB;       // dS of one block: 16 KiB
constexpr int NKB = 4;                   // K buffers: blocks p - 1 .. p + 2
constexpr int NVB = 3;                   // V buffers: blocks p .. p + 2

// LDS plan for head dim DH
template <int DH>
struct Plan {
    static constexpr int ROWB = 2 * DH;           // bytes per 16-bit row
    static constexpr int NI = DH / 16;            // d-chunks of a product's contraction
    static constexpr int TILE = BK * ROWB;        // one K or V block
    static constexpr int OFF_K = 0;
    static constexpr int OFF_V = NKB * TILE;
    static constexpr int OFF_DS = OFF_V + NVB * TILE;  // 2 buffers
    static constexpr int LDS_BYTES = OFF_DS + 2 * DSB;
    static_assert(LDS_BYTES <= 88 * 1024, "LDS plan");
};

// Score role: dS of key block k0 for this wave's two groups of 32 queries
// (lane queries qa and qa + 32), stored as slabs (16-key step t, query group
// 2 s + g), lane-ordered 16 bytes.
template <typename E, int DH, bool MASK, bool CAUSAL>
__device__ __forceinline__ void score_step(unsigned char* smem, int kbuf, int vbuf, int dbuf,
                                           int k0, int qa, int N, float sc,
                                           const float (&Lq)[2], const float (&Dq)[2],
                                           const v16x8_t (&qt)[2][DH / 16],
                                           const v16x8_t (&gt)[2][DH / 16],
                                           const int (&so)[DH / 16], const v16x8_t (&bD)[2],
                                           const v16x8_t& ones, int s, int l) {
    using PL = Plan<DH>;
    constexpr int NI = PL::NI;
    const int h = l >> 5;
    const unsigned char* sK = smem + PL::OFF_K + kbuf * PL::TILE;
    const unsigned char* sV = smem + PL::OFF_V + vbuf * PL::TILE;
    unsigned char* sS = smem + PL::OFF_DS + dbuf * DSB;
    // dS = P (dP - D), packed, into the group's two slabs; grouped by
    // operation so that dependent instructions stand sixteen apart
    auto finish = [&](f32x16_t& P, const f32x16_t& dP, int g) {
#pragma unroll
        for (int e = 0; e < 16; ++e) P[e] *= dP[e];
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int t = 0; t < 2; ++t)
            *reinterpret_cast<uint4*>(sS + (t * QG + 2 * s + g) * SLAB + l * 16) =
                make_uint4(E::pack2(P[8 * t], P[8 * t + 1]), E::pack2(P[8 * t + 2], P[8 * t + 3]),
                           E::pack2(P[8 * t + 4], P[8 * t + 5]),
                           E::pack2(P[8 * t + 6], P[8 * t + 7]));
    };
    f32x16_t S0 = f32x16_t{}, S1 = f32x16_t{}, dP0, dP1;
    if (MASK) {
        dP0 = mfma(ones, bD[0], f32x16_t{});
        dP1 = mfma(ones, bD[1], f32x16_t{});
#pragma unroll
        for (int dk = 0; dk < NI; ++dk) {
            const v16x8_t a = lds_b128(sK + so[dk]);
            const v16x8_t b = lds_b128(sV + so[dk]);
            S0 = E::mma(a, qt[0][dk], S0);
            S1 = E::mma(a, qt[1][dk], S1);
            dP0 = E::mma(b, gt[0][dk], dP0);
            dP1 = E::mma(b, gt[1][dk], dP1);
        }
        // P, masked, grouped by operation eight elements at a time
        auto expm = [&](f32x16_t& S, int qq, float Lg) {
            const int krow = k0 + 4 * h;
#pragma unroll
            for (int c = 0; c < 2; ++c) {
#pragma unroll
                for (int e = 8 * c; e < 8 * c + 8; ++e) {
                    float x = __builtin_fmaf(S[e], sc, -Lg);
                    const int key = krow + 8 * (e >> 2) + (e & 3);
                    if (key >= N || (CAUSAL && key > qq)) x = -INFINITY;
                    S[e] = x;
                }
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int e = 8 * c; e < 8 * c + 8; ++e) S[e] = __builtin_amdgcn_exp2f(S[e]);
                __builtin_amdgcn_sched_barrier(0);
            }
        };
        expm(S0, qa, Lq[0]);
        expm(S1, qa + 32, Lq[1]);
        finish(S0, dP0, 0);
        finish(S1, dP1, 1);
        return;
    }
    // Operand u = 0..2 NI - 1 (K fragment u, then V fragment u - NI) sits in
    // slot u % 3, read two steps ahead.
    v16x8_t op[3];
    op[0] = lds_b128(sK + so[0]);
    op[1] = lds_b128(sK + so[1]);
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        op[(i + 2) % 3] = i + 2 < NI ? lds_b128(sK + so[i + 2]) : lds_b128(sV + so[i + 2 - NI]);
        S0 = E::mma(op[i % 3], qt[0][i], S0);
        S1 = E::mma(op[i % 3], qt[1][i], S1);
        __builtin_amdgcn_sched_barrier(0);
    }
    // Exponentials of S under the dP products.  A wave's next product waits
    // for the matrix pipe, and its vector work behind that product waits too,
    // so the arithmetic sits between the two products of a step (about 27
    // cycles of it under each 32-cycle product at d = 128): half-step k of the
    // 2 NI exponentiates elements EPH k .. EPH k + EPH - 1 of the 32 (scaled
    // one step earlier) and scales those of half-step k + 2.  Elements 0..15
    // are S0's, 16..31 S1's.
    constexpr int EPH = 16 / NI;
    auto scale2 = [&](int k) {
#pragma unroll
        for (int e = EPH * k; e < EPH * k + EPH; ++e) {
            if (e < 16) {
                float t = __builtin_fmaf(S0[e], sc, -Lq[0]);
                pin(t);
                S0[e] = t;
            } else {
                float t = __builtin_fmaf(S1[e - 16], sc, -Lq[1]);
                pin(t);
                S1[e - 16] = t;
            }
        }
    };
    auto exp2 = [&](int k) {
#pragma unroll
        for (int e = EPH * k; e < EPH * k + EPH; ++e) {
            if (e < 16) {
                float t = __builtin_amdgcn_exp2f(S0[e]);
                pin(t);
                S0[e] = t;
            } else {
                float t = __builtin_amdgcn_exp2f(S1[e - 16]);
                pin(t);
                S1[e - 16] = t;
            }
        }
    };
    // dP starts at -D: one product per group broadcasts the lane's value
    dP0 = mfma(ones, bD[0], f32x16_t{});
    dP1 = mfma(ones, bD[1], f32x16_t{});
    scale2(0);
    scale2(1);
#pragma unroll
    for (int j = 0; j < NI; ++j) {
        const int u = NI + j;
        if (u + 2 < 2 * NI) op[(u + 2) % 3] = lds_b128(sV + so[j + 2]);
        dP0 = E::mma(op[u % 3], gt[0][j], dP0);
        __builtin_amdgcn_sched_barrier(0);
        exp2(2 * j);
        if (2 * j + 2 < 2 * NI) scale2(2 * j + 2);
        __builtin_amdgcn_sched_barrier(0);
        dP1 = E::mma(op[u % 3], gt[1][j], dP1);
        __builtin_amdgcn_sched_barrier(0);
        exp2(2 * j + 1);
        if (2 * j + 3 < 2 * NI) scale2(2 * j + 3);
        __builtin_amdgcn_sched_barrier(0);
    }
    finish(S0, dP0, 0);
    finish(S1, dP1, 1);
}

// Score role, a key block wholly above this wave's queries (causal): dS = 0.
template <int DH>
__device__ __forceinline__ void zero_step(unsigned char* smem, int dbuf, int s, int l) {
    unsigned char* sS = smem + Plan<DH>::OFF_DS + dbuf * DSB;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int g = 0; g < 2; ++g)
            *reinterpret_cast<uint4*>(sS + (t * QG + 2 * s + g) * SLAB + l * 16) =
                make_uint4(0u, 0u, 0u, 0u);
}

// Gradient role: for the QGW query groups qg0 .. qg0 + QGW - 1 of the wave
// (d = 128: four, d = 64: two) and d columns [32 dt0, 32 dt0 + 64) (d tiles
// dt0, dt0 + 1), dQ += dS K for the block's 32 keys: per 16-key step two K
// operands (transposing reads; ob0 / ob1: the lane's offsets for rows
// 4 h + (l % 16) / 4 and that + 8, rows 16 t + ... sharing their swizzle) and
// QGW dS slabs, 2 QGW products.  Both steps' operands are read before the
// first step's products.  stage(t) issues part of a later block's copies
// after step t's products, so that the copies never pile up in the memory
// pipeline in front of this wave's work.
template <typename E, int DH, typename Stage>
__device__ __forceinline__ void grad_step(const unsigned char* smem, int kbuf, int dbuf,
                                          f32x16_t (&acc)[DH / 32][2], const int (&ob0)[2],
                                          const int (&ob1)[2], int qg0, int l, Stage&& stage) {
    using PL = Plan<DH>;
    constexpr int QGW = DH / 32;
    const unsigned char* sK = smem + PL::OFF_K + kbuf * PL::TILE;
    const unsigned char* sl = smem + PL::OFF_DS + dbuf * DSB + l * 16;
    v16x8_t bK[2][2], aS[2][QGW];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
        for (int dt = 0; dt < 2; ++dt)
            bK[t][dt] = tr16_pair(sK + ob0[dt] + 16 * PL::ROWB * t,
                                  sK + ob1[dt] + 16 * PL::ROWB * t);
#pragma unroll
        for (int qg = 0; qg < QGW; ++qg) aS[t][qg] = lds_b128(sl + (t * QG + qg0 + qg) * SLAB);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
        for (int qg = 0; qg < QGW; ++qg)
#pragma unroll
            for (int dt = 0; dt < 2; ++dt) acc[qg][dt] = E::mma(aS[t][qg], bK[t][dt], acc[qg][dt]);
        stage(t);
        __builtin_amdgcn_sched_barrier(0);
    }
}

// Work item of the pass: query block q0 of head `head` (batch and head
// folded) and its number of key blocks.
template <int DH, bool CAUSAL>
struct QueryItem {
    int head, q0, nblk;
    __device__ __forceinline__ QueryItem(int work, int nwork, int nqb, int N) {
        int qblk = work % nqb;
        head = work / nqb;
        if (CAUSAL) {  // heaviest (last) query blocks first
            heavy_first_work(work, nwork, nqb, head, qblk);
            qblk = nqb - 1 - qblk;
        }
        q0 = qblk * BQ;
        const int kend = CAUSAL ? min(N, q0 + BQ) : N;  // causal: the loop stops at the diagonal
        nblk = (kend + BK - 1) / BK;
    }
    __device__ __forceinline__ long long hoff(int N) const { return (long long)head * N * DH; }
};

// A position in a workgroup's run of key blocks: block p of the item of round m.
template <int DH, bool CAUSAL>
struct QueryCursor {
    int m, p;
    QueryItem<DH, CAUSAL> it;
    __device__ __forceinline__ bool valid(const Run& r) const { return m < r.m1; }
    __device__ __forceinline__ void advance(const Schedule& s, const Run& r, int nwork, int nqb,
                                            int N) {
        if (++p == it.nblk) {
            p = 0;
            if (++m < r.m1) it = QueryItem<DH, CAUSAL>(r.item(s, m), nwork, nqb, N);
        }
    }
};

// The workgroup's run of work items (rounds [run.m0, run.m1) of the
// schedule), their key blocks back to back: block g of the run is staged
// during phase g - 2, scored in phase g and reduced into dQ in phase g + 1,
// whether or not it starts a new item, so that an item's first blocks overlap
// the previous item's last ones.  At an item boundary the score waves load the
// next item's Q^T and dO^T fragments, L and D right after their last product
// with the old ones, and the gradient waves store the finished dQ rows just
// before the first products of the next item.
// DIRECT: instead of the unscaled fp32 dq_accum, write dQ = scale * acc in the
// element type (round to nearest even), exactly what the convert step makes of
// dq_accum; out is then the dQ tensor.  A DIRECT run holds one work item (the
// launcher gives it one workgroup per item).
template <typename E, int DH, bool CAUSAL, bool DIRECT>
__device__ __forceinline__ void dq_run(
    const e16_t* __restrict__ Q, const e16_t* __restrict__ K, const e16_t* __restrict__ V,
    const e16_t* __restrict__ dO, const float* __restrict__ Lg, const float* __restrict__ Dg,
    void* __restrict__ dq_out, int N, int nqb, float scale, const Schedule& sch, const Run& run,
    int nwork, unsigned char* smem) {
    using PL = Plan<DH>;
    using Item = QueryItem<DH, CAUSAL>;
    using Cursor = QueryCursor<DH, CAUSAL>;
    constexpr int NI = PL::NI;
    constexpr int QGW = DH / 32;  // query groups per gradient wave
    if (run.m0 >= run.m1) return;

    const int wave = threadIdx.x >> 6, l = threadIdx.x & 63, h = l >> 5, n = l & 31;
    const bool score = wave < 4;
    const int r4 = wave & 3;  // query pair of groups (score) or d block (gradient)
    const float sc = scale * kLog2e;
    const Item first(run.item(sch, run.m0), nwork, nqb, N);

    // blocks 0 and 1 of the run up front (one 1 KiB slice per wave: all eight
    // waves at d = 128, four at d = 64); block g + 2 is copied during phase g
    Cursor stg{run.m0, 0, first};  // the block staged last
    constexpr int SW = PL::TILE / 1024 < NWAVE ? PL::TILE / 1024 : NWAVE;
    if (SW == NWAVE || wave < SW) {
        stage_rows<BK, SW, DH>(smem + PL::OFF_K, K + first.hoff(N), 0, N, wave, l);
        stage_rows<BK, SW, DH>(smem + PL::OFF_V, V + first.hoff(N), 0, N, wave, l);
    }
    stg.advance(sch, run, nwork, nqb, N);
    if (stg.valid(run) && (SW == NWAVE || wave < SW)) {
        const long long hoff = stg.it.hoff(N);
        stage_rows<BK, SW, DH>(smem + PL::OFF_K + PL::TILE, K + hoff, stg.p * BK, N, wave, l);
        stage_rows<BK, SW, DH>(smem + PL::OFF_V + PL::TILE, V + hoff, stg.p * BK, N, wave, l);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    // Phase g (one barrier each, one more than the run has blocks): score
    // waves work on block g; gradient waves copy block g + 2 and work on
    // block g - 1 (the score waves' MFMA work is twice theirs).  Each role has
    // its own loop so their registers never coexist.  Block g uses K buffer
    // g % NKB, V buffer g % NVB and dS buffer g % 2.
    if (score) {
        int so[NI];
#pragma unroll
        for (int i = 0; i < NI; ++i) so[i] = tile_off<PL::ROWB>(n, 32 * i + 16 * h);
        // Starting value -D of the dP accumulators, made by one product per
        // group: A is 1 on k-slots 0..2 (lanes of half 0), B holds -D of the
        // lane's query split into three bf16 terms on those k-slots (about
        // 2^-26 relative), so the product broadcasts -D down the key rows.
        const v16x8_t ones = as_v16x8(h ? make_uint4(0, 0, 0, 0) : make_uint4(0x3F803F80u, 0x00003F80u, 0, 0));
        v16x8_t qt[2][NI], gt[2][NI];
        float Lraw[2], Draw[2];
        // the item's fragments, L and D (used only from its first block on,
        // so that the loads overlap the previous item's last block)
        auto load_q = [&](const Item& it) {
            const long long hoff = it.hoff(N);
            const int qa = it.q0 + 64 * r4 + n;
#pragma unroll
            for (int g = 0; g < 2; ++g) {
                const int qc = qa + 32 * g < N ? qa + 32 * g : N - 1;  // clamped: finite, not stored
#pragma unroll
                for (int dk = 0; dk < NI; ++dk) {
                    qt[g][dk] = as_v16x8(*reinterpret_cast<const uint4*>(Q + hoff + (long long)qc * DH + 16 * dk + 8 * h));
                    gt[g][dk] = as_v16x8(*reinterpret_cast<const uint4*>(dO + hoff + (long long)qc * DH + 16 * dk + 8 * h));
                }
                Lraw[g] = Lg[(long long)it.head * N + qc];
                Draw[g] = Dg[(long long)it.head * N + qc];
            }
        };
        Item it = first;
        load_q(it);
        int gb = 0;  // the run's block index g
        for (int m = run.m0; m < run.m1; ++m) {
            const bool more = m + 1 < run.m1;
            const int qw = it.q0 + 64 * r4;  // this wave's first query
            const int qa = qw + n;           // this lane's query in group 0 (group 1: + 32)
            float Lq[2], Dq[2];
            v16x8_t bD[2];
#pragma unroll
            for (int g = 0; g < 2; ++g) {
                Lq[g] = Lraw[g] * kLog2e;
                Dq[g] = Draw[g];
                const float u = -Dq[g];
                const float hi = (float)(__bf16)u;
                const float r1 = u - hi;
                const float mid = (float)(__bf16)r1;
                bD[g] = as_v16x8(h ? make_uint4(0, 0, 0, 0)
                                   : make_uint4(pack_bf16x2(hi, mid), pack_bf16x2(r1 - mid, 0.f), 0, 0));
            }
            // blocks needing no mask for any of this wave's queries
            const int full = CAUSAL ? min(qw / BK, N / BK) : N / BK;
            for (int p = 0; p < it.nblk; ++p, ++gb) {
                const int k0 = p * BK;
                if (CAUSAL && k0 >= qw + 64)
                    zero_step<DH>(smem, gb & 1, r4, l);
                else if (p < full)
                    score_step<E, DH, false, CAUSAL>(smem, gb % NKB, gb % NVB, gb & 1, k0, qa, N, sc,
                                                     Lq, Dq, qt, gt, so, bD, ones, r4, l);
                else
                    score_step<E, DH, true, CAUSAL>(smem, gb % NKB, gb % NVB, gb & 1, k0, qa, N, sc,
                                                    Lq, Dq, qt, gt, so, bD, ones, r4, l);
                if (p + 1 == it.nblk && more) load_q(Item(run.item(sch, m + 1), nwork, nqb, N));
                // LDS traffic only: the next item's loads stay in flight
                __builtin_amdgcn_s_waitcnt(kLgkmOnly);
                __syncthreads();
            }
            if (more) it = Item(run.item(sch, m + 1), nwork, nqb, N);
        }
        __builtin_amdgcn_s_waitcnt(kLgkmOnly);
        __syncthreads();  // the gradient waves' last block
        __builtin_amdgcn_s_waitcnt(0);
        return;
    }

    // gradient wave r4: d = 128: query half r4 / 2 (groups 4 (r4 / 2) ..),
    // d half r4 % 2 (d tiles 2 (r4 % 2), + 1); d = 64: query quarter r4
    // (groups 2 r4, 2 r4 + 1), both d tiles
    const int qg0 = DH == 128 ? 4 * (r4 >> 1) : 2 * r4;
    const int dt0 = DH == 128 ? 2 * (r4 & 1) : 0;
    f32x16_t acc[QGW][2];
    auto zero = [](f32x16_t(&a)[QGW][2]) {
#pragma unroll
        for (int i = 0; i < QGW; ++i) a[i][0] = a[i][1] = f32x16_t{};
    };
    zero(acc);
    using Copier = TileCopier<BK, NWAVE / 2, DH>;
    const Copier cp(r4, l);
    const uint32_t lds0 = lds_addr(smem);
    int ob0[2], ob1[2];
    {
        const int g2 = (l >> 4) & 1, x = 4 * h + ((l & 15) >> 2);
#pragma unroll
        for (int dt = 0; dt < 2; ++dt) {
            const int colb = 64 * (dt0 + dt) + 32 * g2 + 8 * (l & 3);
            ob0[dt] = tile_off<PL::ROWB>(x, colb);
            ob1[dt] = tile_off<PL::ROWB>(x + 8, colb);
        }
    }
    // acc[qg][dt] holds dQ for queries q0 + 32 (qg0 + qg) + 8 (r / 4) + 4 h +
    // r % 4, column 32 (dt0 + dt) + n
    // a block wholly inside N (every block but a ragged last one) stores
    // without a per-row test
    auto store_rows = [&](const Item& it, auto ragged_tag) {
        constexpr bool RAGGED = decltype(ragged_tag)::value;
        const long long hoff = it.hoff(N);
        if constexpr (DIRECT) {
            e16_t* out = reinterpret_cast<e16_t*>(dq_out) + hoff;
#pragma unroll
            for (int qg = 0; qg < QGW; ++qg)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int qq = it.q0 + 32 * (qg0 + qg) + 8 * (r >> 2) + 4 * h + (r & 3);
                    e16_t* orow = out + (long long)qq * DH + 32 * dt0 + n;
                    if (!RAGGED || qq < N)
#pragma unroll
                        for (int dt = 0; dt < 2; ++dt) {
                            // the fp32 product first, as the convert step
                            // forms it (not fused into one mixed-precision
                            // rounding)
                            float x = acc[qg][dt][r] * scale;
                            pin(x);
                            orow[32 * dt] = (e16_t)(E::pack2(x, 0.f) & 0xffffu);
                        }
                }
        } else {
            float* out = reinterpret_cast<float*>(dq_out) + hoff;
#pragma unroll
            for (int qg = 0; qg < QGW; ++qg)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int qq = it.q0 + 32 * (qg0 + qg) + 8 * (r >> 2) + 4 * h + (r & 3);
                    float* orow = out + (long long)qq * DH + 32 * dt0 + n;
                    if (!RAGGED || qq < N)
#pragma unroll
                        for (int dt = 0; dt < 2; ++dt) orow[32 * dt] = acc[qg][dt][r];
                }
        }
    };
    auto epilogue = [&](const Item& it) {
        if (it.q0 + BQ <= N)
            store_rows(it, std::false_type{});
        else
            store_rows(it, std::true_type{});
    };
    Cursor grd{run.m0, 0, first};  // the next block to reduce
    Item acc_it = first;           // the item the accumulators belong to
    for (int g = 0;; ++g) {
        // copies of block g + 2, spread over the gradient steps; past the
        // run's last block they are issued all the same (rows clamped into
        // the last item's head) into buffers no one reads, so that no branch
        // splits the products they are spread over
        stg.advance(sch, run, nwork, nqb, N);
        const long long shoff = stg.it.hoff(N);
        const int kn = stg.valid(run) ? stg.p * BK : N;
        const uint32_t lk = lds0 + PL::OFF_K + ((g + 2) % NKB) * PL::TILE;
        const uint32_t lv = lds0 + PL::OFF_V + ((g + 2) % NVB) * PL::TILE;
        // step t issues slice t (d = 128: two slices per block, d = 64: one)
        auto stage = [&](int j) {
            if (j < Copier::SLICES) {
                cp.copy(j, K + shoff, kn, N, lk);
                cp.copy(j, V + shoff, kn, N, lv);
            }
        };
        static_assert(Copier::SLICES >= 1 && Copier::SLICES <= 2, "at most one slice per 16-key step");
        if (g >= 1) {
            // DIRECT runs one item per workgroup: its 16-bit epilogue inside
            // the loop would not fit the registers
            if (!DIRECT && grd.p == 0 && grd.m > run.m0) {
                // the block starts a new item: the previous item's sums are
                // complete; store them, then start from zero
                epilogue(acc_it);
                zero(acc);
            }
            if (grd.p == 0) acc_it = grd.it;
            grad_step<E, DH>(smem, (g - 1) % NKB, (g - 1) & 1, acc, ob0, ob1, qg0, l, stage);
            grd.advance(sch, run, nwork, nqb, N);
        } else {
#pragma unroll
            for (int j = 0; j < 2; ++j) stage(j);
        }
        // block g + 1's copies (issued one phase ago) must have landed; this
        // phase's 2 SLICES may stay in flight, except in the last phase
        if (grd.valid(run))
            __builtin_amdgcn_s_waitcnt(vmcnt_lgkm0(2 * Copier::SLICES));
        else
            __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (!grd.valid(run)) break;
    }
    epilogue(acc_it);
}

}  // namespace dqp
}  // namespace fa
