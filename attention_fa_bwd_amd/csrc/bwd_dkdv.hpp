// bwd_dkdv.hpp -- key-outer pass of the FA2 backward on gfx950 matrix cores:
// dK and dV for bf16 and fp16, head dims 64 and 128.
//
// Method (FA2 chapter 16): one work item per (key block of 128 keys, head,
// batch), key blocks outer and query tiles inner (sec 16.2); per query tile
// S = scale Q K^T and P = exp(S - L) are recomputed (sec 16.4), dP = dO V^T,
// dS = P (dP - D) with D from the preprocess (sec 16.1, sec 16.8 item 1), and
// dV += P^T dO, dK += dS^T Q accumulate in registers for the whole loop and are
// written once, dK scaled by the softmax scale (sec 16.6).  Under the causal
// mask the query loop starts at the key block's first key, so tiles wholly
// above the diagonal are never visited (sec 16.8 item 2).  dQ is produced by
// the query-outer pass in bwd_dq.hip.
//
// gfx950 mapping: a persistent grid (one workgroup per CU, each running a
// fixed list of work items with their query tiles back to back, see
// dkdv_run); 8 waves, two per SIMD, in two roles that overlap on each
// SIMD (one wave's matrix-core work runs while the other computes or waits on
// LDS):
//   * score wave s owns key groups 2 (s % 2) and 2 (s % 2) + 1 (64 keys; K^T
//     and V^T B-operand fragments, d / 16 of each per key group, in
//     registers) for query rows
//     [32 (s / 2), +32) of every tile, so that each Q or dO fragment read
//     from LDS feeds two products; per tile it forms S = Q K^T and
//     dP = dO V^T (query on rows, key on lanes), P = exp2(S scale log2(e) -
//     L log2(e)) and dS = P (dP - D), and stores P and dS (16-bit) to LDS in
//     its own register order, one 1 KiB slab per (16-query step, key group);
//   * gradient waves 4..7 own one output each, dV^T (waves 4, 5) or dK^T
//     (waves 6, 7), for 64 rows of d and 64 (d = 64) or 128 (d = 128) keys:
//     with d = 128 the two waves of an output split d, with d = 64 they
//     split the keys (accumulators in registers).  One tile behind the score
//     waves, they read dO^T or Q^T fragments of that tile with
//     ds_read_b64_tr_b16 -- each fragment feeds one product per key group of
//     the wave -- and P or dS straight from the slabs, each slab feeding two
//     products;
//   * Q and dO tiles (64 rows, swizzled rows of 2 d bytes) rotate through
//     three LDS buffers (score waves read tile p, gradient waves tile p - 1,
//     loads fill tile p + 1 with direct-to-LDS copies); P and dS through two.
//     One barrier per tile.  LDS: 96 + 64 = 160 KiB (d = 128), 48 + 64 KiB
//     (d = 64);
//   * rows at or beyond N are staged as copies of row N - 1 and get P = 0;
//     keys at or beyond N only reach their own dV / dK rows, which are not
//     stored.
#pragma once

#include <type_traits>

#include "mfma_common.hpp"

namespace fa {
namespace dkvp {

using namespace mf;

constexpr int BC = 128;                  // keys per workgroup
constexpr int BR = 64;                   // queries per tile
constexpr int NWAVE = 8;
constexpr int SLAB = 1024;               // one 16-query x 32-key 16-bit operand, lane order
constexpr int PDS = 4 * 4 * SLAB;        // P (or dS) of one tile: 16 KiB

// LDS plan for head dim DH
template <int DH>
struct Plan {
    static constexpr int ROWB = 2 * DH;           // bytes per 16-bit row
    static constexpr int NI = DH / 16;            // d-chunks of a product's contraction
    static constexpr int TILE = BR * ROWB;        // one Q or dO tile
    static constexpr int OFF_Q = 0;               // 3 buffers
    static constexpr int OFF_DO = 3 * TILE;       // 3 buffers
    static constexpr int OFF_P = 6 * TILE;        // 2 buffers
    static constexpr int OFF_DS = OFF_P + 2 * PDS;  // 2 buffers
    static constexpr int LDS_BYTES = OFF_DS + 2 * PDS;
    static_assert(LDS_BYTES <= 160 * 1024, "LDS plan");
};

// Row statistics enter the score products as the accumulators' starting
// values: S starts at -L / scale and dP at -D, so that P = exp2(S scale log2 e)
// and dS = P dP need no per-element correction.  Those starting values are
// made by one matrix-core product per accumulator: the A operand holds, on
// row n, the value split into three bf16 terms (k-slots 0..2 on lanes of
// half 0 for S, k-slots 8..10 on lanes of half 1 for dP), the B operand is 1
// on those k-slots for every column, so the product broadcasts the row's value
// across the 32 key columns in accumulator layout.  The three terms carry the
// value to about 2^-26 relative.  Each lane fetches a single float per
// 32-row block (L of row n on half 0, D of row n on half 1), one tile ahead.

// float of a 32-row block for this lane: L (half 0) or D (half 1) of row q,
// clamped into [0, N).
__device__ __forceinline__ float fetch_stat(const float* src, int q, int N) {
    return src[q < N ? q : N - 1];
}

// bias operands of one 32-row block from the fetched float; fac is -1/scale
// on half 0 and -1 on half 1.  RAGGED: row q >= N gets S = -1e30 (P = 0) and
// dP = 0.
template <bool RAGGED>
__device__ __forceinline__ void bias_operands(float raw, int q, int N, int h, float fac,
                                              v16x8_t& aS, v16x8_t& aD) {
    float u = raw * fac;
    if (RAGGED && q >= N) u = h ? 0.f : -1e30f;
    const float hi = (float)(__bf16)u;
    const float r1 = u - hi;
    const float mid = (float)(__bf16)r1;
    const uint32_t w0 = pack_bf16x2(hi, mid), w1 = pack_bf16x2(r1 - mid, 0.f);
    aS = as_v16x8(h ? make_uint4(0, 0, 0, 0) : make_uint4(w0, w1, 0, 0));
    aD = as_v16x8(h ? make_uint4(w0, w1, 0, 0) : make_uint4(0, 0, 0, 0));
}

// 1.0 on k-slots 0..2 of every lane: B operand of the bias products
__device__ __forceinline__ v16x8_t bias_ones() {
    return as_v16x8(make_uint4(0x3F803F80u, 0x00003F80u, 0, 0));
}

// dS of elements r, r + 1 from P (already exponentiated, in S) and dP, and
// both pairs packed.
template <typename E>
__device__ __forceinline__ void ds_finish(const f32x16_t& P, const f32x16_t& dP, int r,
                                          uint32_t& pp, uint32_t& pd) {
    pp = E::pack2(P[r], P[r + 1]);
    pd = E::pack2(P[r] * dP[r], P[r + 1] * dP[r + 1]);
}

// Score role, wave w: key groups 2 kp and 2 kp + 1 (kp = w % 2; 64 keys, K^T
// and V^T fragments in registers) for query rows [32 qh, 32 qh + 32) of the
// tile (qh = w / 2), so that every Q or dO fragment read from LDS feeds two
// products.  S and dP of both key groups start from the row statistics
// (bias products), P = exp2(S scale log2 e), dS = P dP; P and dS go to the
// slabs (16-query step t = 2 qh + hh, key group 2 kp + c), lane-ordered.
// RAGGED: the tile runs past row N.  DIAG: the tile crosses the causal
// diagonal and the mask is applied element by element.  Operand reads run
// two products ahead, and the exponentials sit between the dP products,
// each pinned to its place.
template <typename E, int DH, bool RAGGED, bool DIAG>
__device__ __forceinline__ void score_step(unsigned char* smem, int qbuf, int pbuf, int q0, int N,
                                           int k0, float sc, float fac, float st,
                                           const v16x8_t (&kt)[2][DH / 16],
                                           const v16x8_t (&vt)[2][DH / 16],
                                           const int (&so)[DH / 16], int kp, int qh, int l) {
    using PL = Plan<DH>;
    constexpr int NI = PL::NI;
    // elements exponentiated per dP product: the 32 of the two key groups
    // spread over the 2 NI products
    constexpr int EPP = 16 / NI;
    const int h = l >> 5, n = l & 31;
    // rows 32 qh + n share row n's swizzle
    const unsigned char* sQ = smem + PL::OFF_Q + qbuf * PL::TILE + 32 * PL::ROWB * qh;
    const unsigned char* sdO = sQ + (PL::OFF_DO - PL::OFF_Q);
    unsigned char* sP = smem + PL::OFF_P + pbuf * PDS;
    unsigned char* sS = smem + PL::OFF_DS + pbuf * PDS;
    const v16x8_t ones = bias_ones();
    v16x8_t bS, bD;
    bias_operands<RAGGED>(st, q0 + 32 * qh + n, N, h, fac, bS, bD);
    const f32x16_t zS = mfma(bS, ones, f32x16_t{});
    __builtin_amdgcn_sched_barrier(0);

    v16x8_t aq[3], ag[3];
    aq[0] = lds_b128(sQ + so[0]);
    aq[1] = lds_b128(sQ + so[1]);
    f32x16_t S0 = zS, S1 = zS;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        if (i + 2 < NI) aq[(i + 2) % 3] = lds_b128(sQ + so[i + 2]);
        else ag[i + 2 - NI] = lds_b128(sdO + so[i + 2 - NI]);
        S0 = E::mma(aq[i % 3], kt[0][i], S0);
        S1 = E::mma(aq[i % 3], kt[1][i], S1);
        __builtin_amdgcn_sched_barrier(0);
    }
    // elements e = 0..31: S0's, then S1's.  DIAG: elements above the
    // diagonal (key past the query) get -inf, so P = 0 there.
    // element e: key key0 + 32 (e / 16), row qrow + 8 ((e % 16) / 4) + e % 4;
    // masked when (key0 - qrow) exceeds a constant of e
    const int kmq = (k0 + 64 * kp + n) - (q0 + 32 * qh + 4 * h);
    auto scl = [&](int e) {
        f32x16_t& S = e < 16 ? S0 : S1;
        float t = S[e & 15] * sc;
        if (DIAG && kmq > 8 * ((e & 15) >> 2) + (e & 3) - 32 * (e >> 4)) t = -INFINITY;
        pin(t);
        S[e & 15] = t;
    };
    auto ex = [&](int e) {
        f32x16_t& S = e < 16 ? S0 : S1;
        float t = __builtin_amdgcn_exp2f(S[e & 15]);
        pin(t);
        S[e & 15] = t;
    };
    // dP (its bias product only now, so that its accumulator is not live
    // through the S products); after product m (m = 0..2 NI - 1) the
    // exponentials of elements EPP m .. EPP m + EPP - 1, scaled (and masked)
    // one product earlier
    const f32x16_t zD = mfma(bD, ones, f32x16_t{});
    f32x16_t dP0 = zD, dP1 = zD;
#pragma unroll
    for (int e = 0; e < EPP; ++e) scl(e);
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        if (i + 2 < NI) ag[(i + 2) % 3] = lds_b128(sdO + so[i + 2]);
        dP0 = E::mma(ag[i % 3], vt[0][i], dP0);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int e = 0; e < EPP; ++e) ex(2 * EPP * i + e);
#pragma unroll
        for (int e = 0; e < EPP; ++e) scl(2 * EPP * i + EPP + e);
        __builtin_amdgcn_sched_barrier(0);
        dP1 = E::mma(ag[i % 3], vt[1][i], dP1);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int e = 0; e < EPP; ++e) ex(2 * EPP * i + EPP + e);
        if (i + 1 < NI)
#pragma unroll
            for (int e = 0; e < EPP; ++e) scl(2 * EPP * (i + 1) + e);
        __builtin_amdgcn_sched_barrier(0);
    }
    // dS = P dP and the packing, grouped by operation, then the slabs
#pragma unroll
    for (int c = 0; c < 2; ++c) {
        const f32x16_t& P = c ? S1 : S0;
        const f32x16_t& dP = c ? dP1 : dP0;
        uint32_t pk[8], dk[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) ds_finish<E>(P, dP, 2 * j, pk[j], dk[j]);
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            const int slab = ((2 * qh + hh) * 4 + 2 * kp + c) * SLAB + l * 16;
            *reinterpret_cast<uint4*>(sP + slab) = make_uint4(pk[4 * hh], pk[4 * hh + 1], pk[4 * hh + 2], pk[4 * hh + 3]);
            *reinterpret_cast<uint4*>(sS + slab) = make_uint4(dk[4 * hh], dk[4 * hh + 1], dk[4 * hh + 2], dk[4 * hh + 3]);
        }
    }
}

// Gradient role: one output per wave -- dV^T += dO^T P (DK = false) or
// dK^T += Q^T dS (DK = true) -- for 64 rows of d (two 32-row blocks) and KG
// key groups starting at kg0 (d = 128: all four, d = 64: two), so each P or
// dS slab is read by two waves.  Operands of a 16-query step: two
// transposing-read pairs (one per d block, each feeding KG products) and KG
// slabs (one per key group, each feeding two), read two steps ahead.
// ob0 / ob1: the lane's transposing-read offsets of rows 4 h + (l % 16) / 4
// and that + 8 in each d block (rows 16 t + ... share their swizzle).
template <typename E, int DH>
__device__ __forceinline__ void grad_step(const unsigned char* smem, int qbuf, int pbuf, bool dk,
                                          f32x16_t (&acc)[2][DH / 32], const int (&ob0)[2],
                                          const int (&ob1)[2], int kg0, int l) {
    using PL = Plan<DH>;
    constexpr int KG = DH / 32;
    const unsigned char* sA = smem + (dk ? PL::OFF_Q : PL::OFF_DO) + qbuf * PL::TILE;
    const unsigned char* sl = smem + (dk ? PL::OFF_DS : PL::OFF_P) + pbuf * PDS + l * 16;
    v16x8_t a[3][2], b[3][KG];
    auto fetch = [&](int t, int slot) {
#pragma unroll
        for (int db = 0; db < 2; ++db)
            a[slot][db] = tr16_pair(sA + ob0[db] + 16 * PL::ROWB * t,
                                    sA + ob1[db] + 16 * PL::ROWB * t);
#pragma unroll
        for (int kg = 0; kg < KG; ++kg) b[slot][kg] = lds_b128(sl + (t * 4 + kg0 + kg) * SLAB);
    };
    fetch(0, 0);
    fetch(1, 1);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        if (t + 2 < 4) fetch(t + 2, (t + 2) % 3);
        // the reads ahead go out before this step's products, which then run
        // back to back (left to itself the compiler threads the reads through
        // the products with a wait before nearly every one)
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int kg = 0; kg < KG; ++kg)
#pragma unroll
            for (int db = 0; db < 2; ++db)
                acc[db][kg] = E::mma(a[t % 3][db], b[t % 3][kg], acc[db][kg]);
        __builtin_amdgcn_sched_barrier(0);
    }
}


// Work item of the pass: key block k0 of head `head` (batch and head folded),
// its first query tile and its number of query tiles.
template <int DH, bool CAUSAL>
struct KeyItem {
    int head, k0, q_begin, ntiles;
    __device__ __forceinline__ KeyItem(int work, int nwork, int nkb, int N) {
        int kblk = work % nkb;
        head = work / nkb;
        if (CAUSAL) heavy_first_work(work, nwork, nkb, head, kblk);  // heaviest (first) key blocks first
        k0 = kblk * BC;
        q_begin = CAUSAL ? k0 : 0;  // causal: tiles wholly above the diagonal are skipped
        ntiles = (N - q_begin + BR - 1) / BR;
    }
    __device__ __forceinline__ long long hoff(int N) const { return (long long)head * N * DH; }
};

// A position in a workgroup's run of tiles: tile p of the item of round m.
template <int DH, bool CAUSAL>
struct KeyCursor {
    int m, p;
    KeyItem<DH, CAUSAL> it;
    __device__ __forceinline__ bool valid(const Run& r) const { return m < r.m1; }
    __device__ __forceinline__ void advance(const Schedule& s, const Run& r, int nwork, int nkb,
                                            int N) {
        if (++p == it.ntiles) {
            p = 0;
            if (++m < r.m1) it = KeyItem<DH, CAUSAL>(r.item(s, m), nwork, nkb, N);
        }
    }
};

// The workgroup's run of work items (rounds [run.m0, run.m1) of the
// schedule), their query tiles back to back: tile g of the run is scored in
// phase g, staged in phase g - 1 and reduced into dK / dV in phase g + 1,
// whether or not it starts a new item, so that an item's first tiles overlap
// the previous item's last ones.  At an item boundary the score waves load the
// next item's K^T and V^T fragments right after their last product with the
// old ones, and the gradient waves store the finished dK / dV rows just
// before the first products of the next item.
template <typename E, int DH, bool CAUSAL>
__device__ __forceinline__ void dkdv_run(
    const e16_t* __restrict__ Q, const e16_t* __restrict__ K, const e16_t* __restrict__ V,
    const e16_t* __restrict__ dO, const float* __restrict__ Lg, const float* __restrict__ Dg,
    e16_t* __restrict__ dK, e16_t* __restrict__ dV, int N, int nkb, float scale,
    const Schedule& sch, const Run& run, int nwork, unsigned char* smem) {
    using PL = Plan<DH>;
    using Item = KeyItem<DH, CAUSAL>;
    constexpr int NI = PL::NI;
    constexpr int KG = DH / 32;  // key groups per gradient wave
    if (run.m0 >= run.m1) return;

    const int wave = threadIdx.x >> 6, l = threadIdx.x & 63, h = l >> 5, n = l & 31;
    const bool score = wave < 4;
    const int r4 = wave & 3;  // key group (score) or d block (gradient)
    const float sc = scale * kLog2e;
    const Item first(run.item(sch, run.m0), nwork, nkb, N);

    // tile 0 of the run, by all waves
    stage_rows<BR, NWAVE, DH>(smem + PL::OFF_Q, Q + first.hoff(N), first.q_begin, N, wave, l);
    stage_rows<BR, NWAVE, DH>(smem + PL::OFF_DO, dO + first.hoff(N), first.q_begin, N, wave, l);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    // Phase g (one barrier each, one more than the run has tiles): score
    // waves work on tile g; gradient waves stage tile g + 1 (the score waves'
    // only memory traffic is L, D and, at item boundaries, K and V, so their
    // waits never cover the staging copies) and work on tile g - 1.  Each role
    // has its own loop so that its registers never coexist with the other
    // role's.  Tile g uses Q / dO buffer g % 3 and P / dS buffer g % 2.
    if (score) {
        const int kp = r4 & 1, qh = r4 >> 1;  // key pair, query half of each tile
        const float fac = h ? -1.f : -1.f / scale;
        int so[NI];
#pragma unroll
        for (int i = 0; i < NI; ++i) so[i] = tile_off<PL::ROWB>(n, 32 * i + 16 * h);
        v16x8_t kt[2][NI], vt[2][NI];
        auto load_kv = [&](const Item& it) {
            const long long hoff = it.hoff(N);
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                const int kk = it.k0 + 64 * kp + 32 * c + n;
                const int keyc = kk < N ? kk : N - 1;  // clamped: finite data, outputs not stored
#pragma unroll
                for (int dk = 0; dk < NI; ++dk) {
                    kt[c][dk] = as_v16x8(*reinterpret_cast<const uint4*>(K + hoff + (long long)keyc * DH + 16 * dk + 8 * h));
                    vt[c][dk] = as_v16x8(*reinterpret_cast<const uint4*>(V + hoff + (long long)keyc * DH + 16 * dk + 8 * h));
                }
            }
        };
        // row statistic of this wave's rows (L on lane half 0, D on half 1),
        // that of the next tile (possibly the next item's first) fetched
        // during each step
        auto stat_of = [&](const Item& it) {
            return (h ? Dg : Lg) + (long long)it.head * N + 32 * qh;
        };
        Item it = first;
        load_kv(it);
        const float* stat = stat_of(it);
        float st = fetch_stat(stat, it.q_begin + n, N - 32 * qh);
        int qb = 0, pb = 0;
        for (int m = run.m0; m < run.m1; ++m) {
            const bool more = m + 1 < run.m1;
            const Item nxt = more ? Item(run.item(sch, m + 1), nwork, nkb, N) : it;
            const float* nstat = stat_of(nxt);
            // tiles crossing the diagonal (causal only) first, then the rest;
            // the waits before each barrier cover only LDS traffic, so the
            // next statistic (and the next item's K and V) stay in flight
            // across it
            const int nmask = CAUSAL ? BC / BR : 0;
            for (int p = 0; p < it.ntiles; ++p) {
                const int q0 = it.q_begin + p * BR;
                const bool last = p + 1 == it.ntiles;
                const float nx = fetch_stat(last ? nstat : stat, (last ? nxt.q_begin : q0 + BR) + n,
                                            N - 32 * qh);
                const bool ragged = q0 + BR > N;
                if (CAUSAL && p < nmask) {
                    if (ragged)
                        score_step<E, DH, true, true>(smem, qb, pb, q0, N, it.k0, sc, fac, st, kt, vt, so, kp, qh, l);
                    else
                        score_step<E, DH, false, true>(smem, qb, pb, q0, N, it.k0, sc, fac, st, kt, vt, so, kp, qh, l);
                } else {
                    if (ragged)
                        score_step<E, DH, true, false>(smem, qb, pb, q0, N, it.k0, sc, fac, st, kt, vt, so, kp, qh, l);
                    else
                        score_step<E, DH, false, false>(smem, qb, pb, q0, N, it.k0, sc, fac, st, kt, vt, so, kp, qh, l);
                }
                st = nx;
                if (last && more) load_kv(nxt);
                qb = qb == 2 ? 0 : qb + 1;
                pb ^= 1;
                __builtin_amdgcn_s_waitcnt(kLgkmOnly);
                __syncthreads();
            }
            it = nxt;
            stat = nstat;
        }
        __builtin_amdgcn_s_waitcnt(kLgkmOnly);
        __syncthreads();  // the gradient waves' last tile
        __builtin_amdgcn_s_waitcnt(0);
        return;
    }

    // gradient wave r4: dV (r4 < 2) or dK (r4 >= 2); d = 128: rows
    // [64 (r4 & 1), +64) of d for all four key groups; d = 64: all 64 rows of
    // d for key groups 2 (r4 & 1), 2 (r4 & 1) + 1
    const bool is_dk = r4 >= 2;
    const int db0 = DH == 128 ? 2 * (r4 & 1) : 0;  // first 32-row block of d
    const int kg0 = DH == 128 ? 0 : 2 * (r4 & 1);  // first key group
    f32x16_t acc[2][KG];
    auto zero = [](f32x16_t(&a)[2][KG]) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < KG; ++j) a[i][j] = f32x16_t{};
    };
    zero(acc);
    const TileCopier<BR, NWAVE / 2, DH> cp(r4, l);
    const uint32_t lds0 = lds_addr(smem);
    int ob0[2], ob1[2];
    {
        const int g2 = (l >> 4) & 1, x = 4 * h + ((l & 15) >> 2);
#pragma unroll
        for (int db = 0; db < 2; ++db) {
            const int colb = 64 * (db0 + db) + 32 * g2 + 8 * (l & 3);
            ob0[db] = tile_off<PL::ROWB>(x, colb);
            ob1[db] = tile_off<PL::ROWB>(x + 8, colb);
        }
    }
    // acc[db][kg] holds dV^T or dK^T for keys k0 + 32 (kg0 + kg) + n, rows of
    // d 32 (db0 + db) + 8 (r / 4) + 4 h + r % 4
    e16_t* const out = is_dk ? dK : dV;
    const float osc = is_dk ? scale : 1.f;
    auto store_rows = [&](const Item& it, auto ragged_tag) {
        constexpr bool RAGGED = decltype(ragged_tag)::value;
        const long long hoff = it.hoff(N);
#pragma unroll
        for (int kg = 0; kg < KG; ++kg) {
            const int kk = it.k0 + 32 * (kg0 + kg) + n;
            if (RAGGED && kk >= N) continue;
            e16_t* row = out + hoff + (long long)kk * DH;
#pragma unroll
            for (int db = 0; db < 2; ++db)
#pragma unroll
                for (int a4 = 0; a4 < 4; ++a4) {
                    const int d0 = 32 * (db0 + db) + 8 * a4 + 4 * h;
                    const int r = 4 * a4;
                    uint2 v;
                    v.x = E::pack2(acc[db][kg][r] * osc, acc[db][kg][r + 1] * osc);
                    v.y = E::pack2(acc[db][kg][r + 2] * osc, acc[db][kg][r + 3] * osc);
                    *reinterpret_cast<uint2*>(row + d0) = v;
                }
        }
    };
    // a block wholly inside N (every block but a ragged last one) stores
    // without a per-row test
    auto epilogue = [&](const Item& it) {
        if (it.k0 + BC <= N)
            store_rows(it, std::false_type{});
        else
            store_rows(it, std::true_type{});
    };
    KeyCursor<DH, CAUSAL> stg{run.m0, 0, first};  // the tile staged last
    KeyCursor<DH, CAUSAL> grd{run.m0, 0, first};  // the next tile to reduce
    Item acc_it = first;                          // the item the accumulators belong to
    int qb = 0, pb = 0;                           // buffers of tile g
    for (int g = 0;; ++g) {
        // copies of tile g + 1 first: they need the whole phase to land
        stg.advance(sch, run, nwork, nkb, N);
        const int qbn = qb == 2 ? 0 : qb + 1;
        if (stg.valid(run)) {
            const long long hoff = stg.it.hoff(N);
            const int qn = stg.it.q_begin + stg.p * BR;
            const uint32_t lq = lds0 + PL::OFF_Q + qbn * PL::TILE;
#pragma unroll
            for (int j = 0; j < cp.SLICES; ++j) {
                cp.copy(j, Q + hoff, qn, N, lq);
                cp.copy(j, dO + hoff, qn, N, lq + (PL::OFF_DO - PL::OFF_Q));
            }
        }
        if (g >= 1) {
            const int qbp = qb == 0 ? 2 : qb - 1;
            if (grd.p == 0 && grd.m > run.m0) {
                // the tile starts a new item: the previous item's sums are
                // complete; store them, then start from zero
                epilogue(acc_it);
                zero(acc);
            }
            if (grd.p == 0) acc_it = grd.it;
            grad_step<E, DH>(smem, qbp, pb ^ 1, is_dk, acc, ob0, ob1, kg0, l);
            grd.advance(sch, run, nwork, nkb, N);
        }
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (!grd.valid(run)) break;
        qb = qbn;
        pb ^= 1;
    }
    epilogue(acc_it);
}

}  // namespace dkvp
}  // namespace fa
