// bwd_dkdv.hpp -- key-outer pass of the FA2 backward on gfx950 matrix cores:
// dK and dV for bf16 and fp16, head dims 64 and 128.
//
// Method (FA2 chapter 16): one workgroup per (key block of 128 keys, head,
// batch), key blocks outer and query tiles inner (sec 16.2); per query tile
// S = scale Q K^T and P = exp(S - L) are recomputed (sec 16.4), dP = dO V^T,
// dS = P (dP - D) with D from the preprocess (sec 16.1, sec 16.8 item 1), and
// dV += P^T dO, dK += dS^T Q accumulate in registers for the whole loop and are
// written once, dK scaled by the softmax scale (sec 16.6).  Under the causal
// mask the query loop starts at the key block's first key, so tiles wholly
// above the diagonal are never visited (sec 16.8 item 2).  dQ is produced by
// the query-outer pass in bwd_dq.hip.
//
// gfx950 mapping: 8 waves, two per SIMD, in two roles that overlap on each
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

template <typename E, int DH, bool CAUSAL>
__device__ __forceinline__ void dkdv_work(
    const e16_t* __restrict__ Q, const e16_t* __restrict__ K, const e16_t* __restrict__ V,
    const e16_t* __restrict__ dO, const float* __restrict__ Lg, const float* __restrict__ Dg,
    e16_t* __restrict__ dK, e16_t* __restrict__ dV, int N, int nkb, float scale, int bid, int nwork,
    unsigned char* smem) {
    using PL = Plan<DH>;
    constexpr int NI = PL::NI;
    constexpr int KG = DH / 32;  // key groups per gradient wave

    const int work = xcd_work_item(bid, nwork);
    int head = work / nkb, kblk = work % nkb;
    if (CAUSAL) heavy_first_work(work, nwork, nkb, head, kblk);  // heaviest (first) key blocks first
    const int k0 = kblk * BC;
    const long long hoff = (long long)head * N * DH;
    const e16_t* Qh = Q + hoff;
    const e16_t* dOh = dO + hoff;
    const float* Lh = Lg + (long long)head * N;
    const float* Dh = Dg + (long long)head * N;

    const int wave = threadIdx.x >> 6, l = threadIdx.x & 63, h = l >> 5, n = l & 31;
    const bool score = wave < 4;
    const int r4 = wave & 3;  // key group (score) or d block (gradient)

    const int q_begin = CAUSAL ? k0 : 0;
    const int ntiles = (N - q_begin + BR - 1) / BR;
    const int nmask = CAUSAL ? BC / BR : 0;  // tiles that cross the diagonal
    const float sc = scale * kLog2e;

    stage_rows<BR, NWAVE, DH>(smem + PL::OFF_Q, Qh, q_begin, N, wave, l);
    stage_rows<BR, NWAVE, DH>(smem + PL::OFF_DO, dOh, q_begin, N, wave, l);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    // Phase p (one barrier each, ntiles + 1 phases): score waves work on tile p;
    // gradient waves stage tile p + 1 (the score waves' only memory traffic is
    // L and D, so their waits never cover the staging copies) and work on
    // tile p - 1.  Each role has its own loop so that its registers never
    // coexist with the other role's.
    if (score) {
        const int kp = r4 & 1, qh = r4 >> 1;  // key pair, query half of each tile
        v16x8_t kt[2][NI], vt[2][NI];
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            const int kk = k0 + 64 * kp + 32 * c + n;
            const int keyc = kk < N ? kk : N - 1;  // clamped: finite data, outputs not stored
#pragma unroll
            for (int dk = 0; dk < NI; ++dk) {
                kt[c][dk] = as_v16x8(*reinterpret_cast<const uint4*>(K + hoff + (long long)keyc * DH + 16 * dk + 8 * h));
                vt[c][dk] = as_v16x8(*reinterpret_cast<const uint4*>(V + hoff + (long long)keyc * DH + 16 * dk + 8 * h));
            }
        }
        // row statistic of this wave's rows in tile p in st (L on lane half
        // 0, D on half 1), that of tile p + 1 fetched during step p
        const float* stat = (h ? Dh : Lh) + 32 * qh;
        const float fac = h ? -1.f : -1.f / scale;
        auto fetch1 = [&](int qn) { return fetch_stat(stat, qn + n, N - 32 * qh); };
        int so[NI];
#pragma unroll
        for (int i = 0; i < NI; ++i) so[i] = tile_off<PL::ROWB>(n, 32 * i + 16 * h);
        float st = fetch1(q_begin);
        // diagonal tiles (causal only) first, then the rest; the waits before
        // each barrier cover only LDS traffic, so the next tile's statistic
        // stays in flight across it
        int p = 0;
        for (; p < min(nmask, ntiles); ++p) {
            const int q0 = q_begin + p * BR;
            const float nx = fetch1(q0 + BR);
            if (q0 + BR > N)
                score_step<E, DH, true, true>(smem, p % 3, p & 1, q0, N, k0, sc, fac, st, kt, vt, so, kp, qh, l);
            else
                score_step<E, DH, false, true>(smem, p % 3, p & 1, q0, N, k0, sc, fac, st, kt, vt, so, kp, qh, l);
            st = nx;
            __builtin_amdgcn_s_waitcnt(kLgkmOnly);
            __syncthreads();
        }
        for (; p <= ntiles; ++p) {
            if (p < ntiles) {
                const int q0 = q_begin + p * BR;
                const float nx = fetch1(q0 + BR);
                if (q0 + BR > N)
                    score_step<E, DH, true, false>(smem, p % 3, p & 1, q0, N, k0, sc, fac, st, kt, vt, so, kp, qh, l);
                else
                    score_step<E, DH, false, false>(smem, p % 3, p & 1, q0, N, k0, sc, fac, st, kt, vt, so, kp, qh, l);
                st = nx;
            }
            __builtin_amdgcn_s_waitcnt(kLgkmOnly);
            __syncthreads();
        }
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
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < KG; ++j) acc[i][j] = f32x16_t{};
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
    for (int p = 0; p <= ntiles; ++p) {
        // copies of tile p + 1 first: they need the whole phase to land.  In
        // the last two phases the buffer they fill is read by no one; they
        // are issued all the same (rows clamped into range) rather than
        // behind a branch.
        const int qn = q_begin + (p + 1) * BR;
        const uint32_t lq = lds0 + PL::OFF_Q + ((p + 1) % 3) * PL::TILE;
#pragma unroll
        for (int j = 0; j < cp.SLICES; ++j) {
            cp.copy(j, Qh, qn, N, lq);
            cp.copy(j, dOh, qn, N, lq + (PL::OFF_DO - PL::OFF_Q));
        }
        if (p >= 1) grad_step<E, DH>(smem, (p - 1) % 3, (p - 1) & 1, is_dk, acc, ob0, ob1, kg0, l);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    }

    // epilogue: acc[db][kg] holds dV^T or dK^T for keys k0 + 32 (kg0 + kg) + n,
    // rows of d 32 (db0 + db) + 8 (r / 4) + 4 h + r % 4
    e16_t* out = is_dk ? dK : dV;
    const float osc = is_dk ? scale : 1.f;
#pragma unroll
    for (int kg = 0; kg < KG; ++kg) {
        const int kk = k0 + 32 * (kg0 + kg) + n;
        if (kk >= N) continue;
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
}

}  // namespace dkvp
}  // namespace fa
