// bwd_dq.hip -- query-outer pass of the FA2 backward on gfx950 matrix cores:
// dQ (unscaled, fp32) for bf16 and fp16, head dim 128.
//
// FA2 chapter 16 sec 16.3 weighs adding dQ partials with global atomics
// against a second pass.  On MI355X the fp32 atomics run at about 340 G/s
// (all of them execute beyond the L2), so one partial per (key block, query
// tile) caps the whole backward far below the matrix-core rate.  This pass
// instead gives each workgroup 128 query rows and loops over all key blocks,
// recomputing S = scale Q K^T, P = exp(S - L) (sec 16.4), dP = dO V^T and
// dS = P (dP - D) (sec 16.1), and accumulating dQ = dS K in registers; each
// dq_accum row is written once, with plain stores.  Under the causal mask the
// key loop stops at the diagonal (sec 16.8 item 2).
//
// gfx950 mapping: 8 waves, two per SIMD, in two roles that overlap on each
// SIMD:
//   * score waves 0..3 own queries [32 s, 32 s + 32) of the block; their Q^T
//     and dO^T B-operand fragments, L and D stay in registers.  Per key block
//     of 64 they form S^T = K Q^T and dP^T = V dO^T (key on rows, query on
//     lanes) and dS = P (dP - D), and store dS (16-bit) to LDS in their own
//     register order, one 1 KiB slab per (16-key step, query group);
//   * gradient waves 4..7 own columns [32 g, 32 g + 32) of d of dQ for all
//     128 queries (accumulators in registers).  One key block behind, they
//     read the K operand of that block (key on the contraction index) with
//     ds_read_b64_tr_b16 -- each fragment feeds four products, one per query
//     group -- and dS straight from the slabs;
//   * K blocks rotate through four LDS buffers (score waves read block p,
//     gradient waves block p - 1, block p + 1 has landed, direct-to-LDS
//     copies fill block p + 2, spread over the gradient steps), V blocks
//     through three, dS through two (144 KiB).  One barrier per block;
//   * rows at or beyond N are staged as copies of row N - 1; in the last key
//     block their P is forced to 0, and query rows at or beyond N are not
//     stored.
#include "launch.hpp"
#include "mfma_common.hpp"

namespace fa {
namespace {

using namespace mf;

constexpr int BQ = 128;                  // queries per workgroup
constexpr int BK = 64;                   // keys per block
constexpr int NWAVE = 8;
constexpr int TILE = BK * ROWB;          // 16 KiB
constexpr int SLAB = 1024;               // one 32-query x 16-key 16-bit operand, lane order
constexpr int DSB = 4 * 4 * SLAB;        // dS of one block: 16 KiB
constexpr int NKB = 4;                   // K buffers: blocks p - 1 .. p + 2
constexpr int NVB = 3;                   // V buffers: blocks p .. p + 2
constexpr int OFF_K = 0;
constexpr int OFF_V = NKB * TILE;
constexpr int OFF_DS = OFF_V + NVB * TILE;  // 2 buffers
constexpr int LDS_BYTES = OFF_DS + 2 * DSB;
static_assert(LDS_BYTES == 144 * 1024, "LDS plan");

// dS of elements r, r + 1 from P (already exponentiated, in S) and dP,
// packed.
template <typename E>
__device__ __forceinline__ uint32_t ds_finish(const f32x16_t& P, const f32x16_t& dP, int r,
                                              float Dq) {
    return E::pack2(P[r] * (dP[r] - Dq), P[r + 1] * (dP[r + 1] - Dq));
}

// Score role: dS of key block k0 for this wave's 32 queries, stored as slabs
// (t = 2 mb + hh, query group s), lane-ordered 16 bytes.  Operand reads run
// two MFMA pairs ahead; outside masked blocks the S^T/dP^T products of key
// half 1 are interleaved with the dS arithmetic of half 0 (order pinned with
// sched_barrier).  Masked blocks (at most two per workgroup) keep the plain
// order, which needs fewer registers.
template <typename E, bool MASK, bool CAUSAL>
__device__ __forceinline__ void score_step(unsigned char* smem, int kbuf, int vbuf, int dbuf,
                                           int k0, int q, int N, float sc, float Lq, float Dq,
                                           const v16x8_t (&qt)[8], const v16x8_t (&gt)[8],
                                           const int (&so)[8], int s, int l) {
    const int h = l >> 5, n = l & 31;
    const unsigned char* sK = smem + OFF_K + kbuf * TILE;
    const unsigned char* sV = smem + OFF_V + vbuf * TILE;
    unsigned char* sS = smem + OFF_DS + dbuf * DSB;
    auto store = [&](int mb, const uint32_t (&pk)[8]) {
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
            *reinterpret_cast<uint4*>(sS + ((2 * mb + hh) * 4 + s) * SLAB + l * 16) =
                make_uint4(pk[4 * hh], pk[4 * hh + 1], pk[4 * hh + 2], pk[4 * hh + 3]);
    };
    if (MASK) {
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
            f32x16_t S = f32x16_t{}, dP = f32x16_t{};
            const int row = 32 * mb + n;
#pragma unroll
            for (int dk = 0; dk < 8; ++dk) {
                const int off = tile_off(row, 32 * dk + 16 * h);
                S = E::mma(lds_b128(sK + off), qt[dk], S);
                dP = E::mma(lds_b128(sV + off), gt[dk], dP);
            }
            // dS, masked, grouped by operation eight elements at a time, so
            // that dependent instructions stand eight apart
            const int krow = k0 + 32 * mb + 4 * h;
            uint32_t pk[8];
#pragma unroll
            for (int g = 0; g < 2; ++g) {
#pragma unroll
                for (int e = 8 * g; e < 8 * g + 8; ++e) {
                    float x = __builtin_fmaf(S[e], sc, -Lq);
                    const int key = krow + 8 * (e >> 2) + (e & 3);
                    if (key >= N || (CAUSAL && key > q)) x = -INFINITY;
                    S[e] = x;
                }
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int e = 8 * g; e < 8 * g + 8; ++e) S[e] = __builtin_amdgcn_exp2f(S[e]);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int j = 4 * g; j < 4 * g + 4; ++j) pk[j] = ds_finish<E>(S, dP, 2 * j, Dq);
            }
            store(mb, pk);
        }
        return;
    }
    // operand of step i (i = 0..15: key half i / 8, d-chunk i % 8); rows
    // 32 + n share row n's swizzle
    auto opoff = [&](int i) { return so[i & 7] + 32 * ROWB * (i >> 3); };
    v16x8_t ak[3], av[3];
    ak[0] = lds_b128(sK + opoff(0));
    av[0] = lds_b128(sV + opoff(0));
    ak[1] = lds_b128(sK + opoff(1));
    av[1] = lds_b128(sV + opoff(1));
    f32x16_t S0 = f32x16_t{}, dP0 = f32x16_t{}, S1 = f32x16_t{}, dP1 = f32x16_t{};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        ak[(i + 2) % 3] = lds_b128(sK + opoff(i + 2));
        av[(i + 2) % 3] = lds_b128(sV + opoff(i + 2));
        S0 = E::mma(ak[i % 3], qt[i], S0);
        dP0 = E::mma(av[i % 3], gt[i], dP0);
        __builtin_amdgcn_sched_barrier(0);
    }
    // Half 0's dS under half 1's products, software-pipelined so that no
    // result is used by the very next instruction: after the first pair of
    // products all sixteen scores go to exp2 units; step k then takes the
    // exponentials of pair k and finishes pair k - 1.
    uint32_t pk[8];
#pragma unroll
    for (int i = 8; i < 16; ++i) {
        const int k = i - 8;
        if (i + 2 < 16) {
            ak[(i + 2) % 3] = lds_b128(sK + opoff(i + 2));
            av[(i + 2) % 3] = lds_b128(sV + opoff(i + 2));
        }
        S1 = E::mma(ak[i % 3], qt[i - 8], S1);
        dP1 = E::mma(av[i % 3], gt[i - 8], dP1);
        if (k == 0)
#pragma unroll
            for (int e = 0; e < 16; ++e) S0[e] = __builtin_fmaf(S0[e], sc, -Lq);
        S0[2 * k] = __builtin_amdgcn_exp2f(S0[2 * k]);
        S0[2 * k + 1] = __builtin_amdgcn_exp2f(S0[2 * k + 1]);
        if (k >= 1) pk[k - 1] = ds_finish<E>(S0, dP0, 2 * k - 2, Dq);
        __builtin_amdgcn_sched_barrier(0);
    }
    pk[7] = ds_finish<E>(S0, dP0, 14, Dq);
    store(0, pk);
    // half 1's dS with nothing else to overlap: grouped by operation so that
    // dependent instructions stand sixteen apart
#pragma unroll
    for (int e = 0; e < 16; ++e) S1[e] = __builtin_fmaf(S1[e], sc, -Lq);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int e = 0; e < 16; ++e) S1[e] = __builtin_amdgcn_exp2f(S1[e]);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < 8; ++j) pk[j] = ds_finish<E>(S1, dP1, 2 * j, Dq);
    store(1, pk);
}

// Gradient role: dQ[:, 32 g .. 32 g + 31] += dS K for the block's 64 keys;
// the next step's operands are read while the current step's products issue.
// ob0 / ob1: the lane's transposing-read offsets for rows 4 h + (l % 16) / 4
// and that + 8 (rows 16 t + ... share their swizzle).  stage(t) issues part
// of a later block's copies after step t's products, so that the copies never
// pile up in the memory pipeline in front of this wave's work.
template <typename E, typename Stage>
__device__ __forceinline__ void grad_step(const unsigned char* smem, int kbuf, int dbuf,
                                          f32x16_t (&acc)[4], int ob0, int ob1, int l,
                                          Stage&& stage) {
    const unsigned char* sK = smem + OFF_K + kbuf * TILE;
    const unsigned char* k0p = sK + ob0;
    const unsigned char* k1p = sK + ob1;
    const unsigned char* sl = smem + OFF_DS + dbuf * DSB + l * 16;
    v16x8_t bK[2], aS[2][4];
    auto fetch = [&](int t, int slot) {
        bK[slot] = tr16_pair(k0p + 16 * ROWB * t, k1p + 16 * ROWB * t);
#pragma unroll
        for (int qg = 0; qg < 4; ++qg) aS[slot][qg] = lds_b128(sl + (t * 4 + qg) * SLAB);
    };
    fetch(0, 0);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        if (t + 1 < 4) fetch(t + 1, (t + 1) & 1);
        // the next step's reads go out before this step's products, which
        // then run back to back
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int qg = 0; qg < 4; ++qg) acc[qg] = E::mma(aS[t & 1][qg], bK[t & 1], acc[qg]);
        stage(t);
        __builtin_amdgcn_sched_barrier(0);
    }
}

template <typename E, bool CAUSAL>
__global__ __launch_bounds__(NWAVE * 64) void bwd_dq_kernel(
    const e16_t* __restrict__ Q, const e16_t* __restrict__ K, const e16_t* __restrict__ V,
    const e16_t* __restrict__ dO, const float* __restrict__ Lg, const float* __restrict__ Dg,
    float* __restrict__ dqa, int N, int nqb, float scale) {
    __shared__ __attribute__((aligned(1024))) unsigned char smem[LDS_BYTES];

    const int work = xcd_work_item(blockIdx.x, gridDim.x);
    const int head = work / nqb;
    const int qblk = CAUSAL ? nqb - 1 - work % nqb : work % nqb;  // heaviest first
    const int q0 = qblk * BQ;
    const long long hoff = (long long)head * N * D;
    const e16_t* Kh = K + hoff;
    const e16_t* Vh = V + hoff;

    const int wave = threadIdx.x >> 6, l = threadIdx.x & 63, h = l >> 5, n = l & 31;
    const bool score = wave < 4;
    const int r4 = wave & 3;             // query group (score) or d block (gradient)
    const int q = q0 + 32 * r4 + n;      // score waves: this lane's query in S^T / dP^T

    const int kend = CAUSAL ? min(N, q0 + BQ) : N;
    const int nblk = (kend + BK - 1) / BK;
    const int full = CAUSAL ? min(q0 / BK, N / BK) : N / BK;  // blocks needing no mask
    const float sc = scale * kLog2e;

    // blocks 0 and 1 up front; block p + 2 is copied during phase p
    stage_rows<BK, NWAVE>(smem + OFF_K, Kh, 0, N, wave, l);
    stage_rows<BK, NWAVE>(smem + OFF_V, Vh, 0, N, wave, l);
    if (nblk > 1) {
        stage_rows<BK, NWAVE>(smem + OFF_K + TILE, Kh, BK, N, wave, l);
        stage_rows<BK, NWAVE>(smem + OFF_V + TILE, Vh, BK, N, wave, l);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    // Phase p (one barrier each, nblk + 1 phases): score waves work on block p;
    // gradient waves copy block p + 2 and work on block p - 1 (the score
    // waves' MFMA work is twice theirs).  Each role has its own loop so their
    // registers never coexist.
    if (score) {
        const int qc = q < N ? q : N - 1;  // clamped: finite data, row not stored
        v16x8_t qt[8], gt[8];
#pragma unroll
        for (int dk = 0; dk < 8; ++dk) {
            qt[dk] = as_v16x8(*reinterpret_cast<const uint4*>(Q + hoff + (long long)qc * D + 16 * dk + 8 * h));
            gt[dk] = as_v16x8(*reinterpret_cast<const uint4*>(dO + hoff + (long long)qc * D + 16 * dk + 8 * h));
        }
        const float Lq = Lg[(long long)head * N + qc] * kLog2e;
        const float Dq = Dg[(long long)head * N + qc];
        int so[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) so[i] = tile_off(n, 32 * i + 16 * h);
        for (int p = 0; p <= nblk; ++p) {
            if (p < nblk) {
                if (p < full)
                    score_step<E, false, CAUSAL>(smem, p % NKB, p % NVB, p & 1, p * BK, q, N, sc, Lq,
                                              Dq, qt, gt, so, r4, l);
                else
                    score_step<E, true, CAUSAL>(smem, p % NKB, p % NVB, p & 1, p * BK, q, N, sc, Lq,
                                             Dq, qt, gt, so, r4, l);
            }
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
        }
        return;
    }

    f32x16_t acc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] = f32x16_t{};
    const TileCopier<BK, NWAVE / 2> cp(r4, l);
    const uint32_t lds0 = lds_addr(smem);
    const int g2 = (l >> 4) & 1, colb = 64 * r4 + 32 * g2 + 8 * (l & 3);
    const int x = 4 * h + ((l & 15) >> 2);
    const int ob0 = tile_off(x, colb), ob1 = tile_off(x + 8, colb);
    for (int p = 0; p <= nblk; ++p) {
        // copies of block p + 2 first; block p + 1's (issued one phase ago)
        // must have landed by the barrier, these may stay in flight.  Past
        // the last block the buffers they fill are read by no one; they are
        // issued all the same (rows clamped into range), so that no branch
        // splits the products they are spread over.
        const int kn = (p + 2) * BK;
        const uint32_t lk = lds0 + OFF_K + ((p + 2) % NKB) * TILE;
        const uint32_t lv = lds0 + OFF_V + ((p + 2) % NVB) * TILE;
        auto stage = [&](int j) {
            cp.copy(j, Kh, kn, N, lk);
            cp.copy(j, Vh, kn, N, lv);
        };
        static_assert(TileCopier<BK, NWAVE / 2>::SLICES == 4, "one slice per 16-key step");
        if (p >= 1) {
            grad_step<E>(smem, (p - 1) % NKB, (p - 1) & 1, acc, ob0, ob1, l, stage);
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) stage(j);
        }
        if (p < nblk)
            __builtin_amdgcn_s_waitcnt(kVmcnt8Lgkm0);
        else
            __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    }

    // epilogue: acc[qg] holds dQ for queries q0 + 32 qg + 8 (r / 4) + 4 h + r % 4,
    // column 32 g + n
    float* out = dqa + hoff;
#pragma unroll
    for (int qg = 0; qg < 4; ++qg)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int qq = q0 + 32 * qg + 8 * (r >> 2) + 4 * h + (r & 3);
            if (qq < N) out[(long long)qq * D + 32 * r4 + n] = acc[qg][r];
        }
}

template <typename E>
hipError_t launch_dq(const void* Q, const void* K, const void* V, const void* dO, const float* L,
                     const float* Dv, float* dqa, Shape s, float scale, bool causal,
                     hipStream_t st) {
    const int nqb = (s.N + BQ - 1) / BQ;
    const long long nwork = (long long)nqb * s.H * s.B;
    if (nwork > 0x7fffffffLL) return hipErrorInvalidValue;
    dim3 grid((unsigned)nwork);
    if (causal)
        hipLaunchKernelGGL((bwd_dq_kernel<E, true>), grid, dim3(NWAVE * 64), 0, st,
                           (const e16_t*)Q, (const e16_t*)K, (const e16_t*)V, (const e16_t*)dO, L,
                           Dv, dqa, s.N, nqb, scale);
    else
        hipLaunchKernelGGL((bwd_dq_kernel<E, false>), grid, dim3(NWAVE * 64), 0, st,
                           (const e16_t*)Q, (const e16_t*)K, (const e16_t*)V, (const e16_t*)dO, L,
                           Dv, dqa, s.N, nqb, scale);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_dq_d128(int dtype, const void* Q, const void* K, const void* V,
                              const void* dO, const float* L, const float* Dv, float* dqa,
                              Shape s, float scale, bool causal, hipStream_t st) {
    return dtype == DT_F16 ? launch_dq<F16E>(Q, K, V, dO, L, Dv, dqa, s, scale, causal, st)
                           : launch_dq<Bf16E>(Q, K, V, dO, L, Dv, dqa, s, scale, causal, st);
}

}  // namespace fa
