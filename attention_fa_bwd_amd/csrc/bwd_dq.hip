// bwd_dq.hip -- query-outer pass of the FA2 backward on gfx950 matrix cores:
// dQ (unscaled, fp32) for bf16, head dim 128.
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
// gfx950 mapping (4 waves, one per SIMD; wave w owns queries [32 w, 32 w + 32)):
//   * the Q^T and dO^T B-operand fragments of S^T = K Q^T and dP^T = V dO^T
//     stay in registers for the whole key loop, as do L * log2(e) and -D of the
//     lane's query row, and the dQ accumulator (32 queries x 128 d);
//   * key blocks of 64 rows of K and V are double-buffered in LDS (swizzled
//     256-byte rows), filled one block ahead with direct-to-LDS loads;
//   * S^T and dP^T leave the matrix core with the query on the lane, so dS is
//     the A operand of dQ = dS K straight from registers; the K operand with
//     the key on the contraction index comes from the same LDS tile through
//     ds_read_b64_tr_b16;
//   * rows at or beyond N are staged as copies of row N - 1; in the last key
//     block their P is forced to 0, and query rows at or beyond N are not
//     stored.
#include "launch.hpp"
#include "mfma_common.hpp"

namespace fa {
namespace {

using namespace mf;

constexpr int BQ = 128;                 // queries per workgroup
constexpr int BK = 64;                  // keys per block
constexpr int NW = 4;                   // waves
constexpr int TILE = BK * ROWB;         // 16 KiB
constexpr int OFF_K = 0;                // 2 buffers
constexpr int OFF_V = 2 * TILE;         // 2 buffers
constexpr int LDS_BYTES = 4 * TILE;

// MASK: apply key > query (causal) and key >= N (last block) element by element.
template <bool MASK, bool CAUSAL>
__device__ __forceinline__ void block_step(const unsigned char* smem, int buf, int k0, int q, int N,
                                           float sc, float Lq, const f32x16_t& negD,
                                           const bf16x8_t (&qt)[8], const bf16x8_t (&gt)[8],
                                           f32x16_t (&acc)[4], int l) {
    const int h = l >> 5, n = l & 31, g2 = (l >> 4) & 1;
    const unsigned char* sK = smem + OFF_K + buf * TILE;
    const unsigned char* sV = smem + OFF_V + buf * TILE;

    // S^T = K Q^T and dP^T - D = V dO^T - D; key on rows, query on lanes
    f32x16_t S[2], dP[2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
        S[mb] = f32x16_t{};
        dP[mb] = negD;
        const int row = 32 * mb + n;
#pragma unroll
        for (int dk = 0; dk < 8; ++dk) {
            const int off = tile_off(row, 32 * dk + 16 * h);
            S[mb] = mfma(lds_b128(sK + off), qt[dk], S[mb]);
            dP[mb] = mfma(lds_b128(sV + off), gt[dk], dP[mb]);
        }
    }

    // dS = P (dP - D) with P = exp2(S sc - L'), to bf16
    bf16x8_t dSb[2][2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
        float ds[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float x = __builtin_fmaf(S[mb][r], sc, -Lq);
            if (MASK) {
                const int key = k0 + 32 * mb + 8 * (r >> 2) + 4 * h + (r & 3);
                if (key >= N || (CAUSAL && key > q)) x = -INFINITY;
            }
            ds[r] = __builtin_amdgcn_exp2f(x) * dP[mb][r];
        }
        dSb[mb][0] = as_bf16x8(pack8(ds));
        dSb[mb][1] = as_bf16x8(pack8(ds + 8));
    }

    // dQ += dS K; query on rows, d on lanes
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const int r0 = 16 * t + 4 * h + ((l & 15) >> 2);
#pragma unroll
        for (int db = 0; db < 4; ++db) {
            const int colb = 64 * db + 32 * g2 + 8 * (l & 3);
            acc[db] = mfma(dSb[t >> 1][t & 1],
                           tr16_pair(sK + tile_off(r0, colb), sK + tile_off(r0 + 8, colb)), acc[db]);
        }
    }

}

template <bool CAUSAL>
__global__ __launch_bounds__(NW * 64) void bwd_dq_kernel(
    const bf16_t* __restrict__ Q, const bf16_t* __restrict__ K, const bf16_t* __restrict__ V,
    const bf16_t* __restrict__ dO, const float* __restrict__ Lg, const float* __restrict__ Dg,
    float* __restrict__ dqa, int N, int nqb, float scale) {
    __shared__ __attribute__((aligned(1024))) unsigned char smem[LDS_BYTES];

    const int work = xcd_work_item(blockIdx.x, gridDim.x);
    const int head = work / nqb;
    const int qblk = CAUSAL ? nqb - 1 - work % nqb : work % nqb;  // heaviest first
    const int q0 = qblk * BQ;
    const long long hoff = (long long)head * N * D;
    const bf16_t* Kh = K + hoff;
    const bf16_t* Vh = V + hoff;

    const int w = threadIdx.x >> 6, l = threadIdx.x & 63, h = l >> 5, n = l & 31;
    const int q = q0 + 32 * w + n;          // this lane's query in S^T / dP^T
    const int qc = q < N ? q : N - 1;       // clamped: finite data, row not stored

    bf16x8_t qt[8], gt[8];
#pragma unroll
    for (int dk = 0; dk < 8; ++dk) {
        qt[dk] = as_bf16x8(*reinterpret_cast<const uint4*>(Q + hoff + (long long)qc * D + 16 * dk + 8 * h));
        gt[dk] = as_bf16x8(*reinterpret_cast<const uint4*>(dO + hoff + (long long)qc * D + 16 * dk + 8 * h));
    }
    const float Lq = Lg[(long long)head * N + qc] * kLog2e;
    const float nD = -Dg[(long long)head * N + qc];
    f32x16_t negD;
#pragma unroll
    for (int r = 0; r < 16; ++r) negD[r] = nD;
    f32x16_t acc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] = f32x16_t{};

    const int kend = CAUSAL ? min(N, q0 + BQ) : N;
    const int nblk = (kend + BK - 1) / BK;
    const int full = CAUSAL ? min(q0 / BK, (N / BK)) : N / BK;  // blocks needing no mask
    const float sc = scale * kLog2e;

    stage_rows<BK, NW>(smem + OFF_K, Kh, 0, N, w, l);
    stage_rows<BK, NW>(smem + OFF_V, Vh, 0, N, w, l);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    for (int it = 0; it < nblk; ++it) {
        const int buf = it & 1;
        const int k0 = it * BK;
        if (it + 1 < nblk) {
            stage_rows<BK, NW>(smem + OFF_K + (buf ^ 1) * TILE, Kh, k0 + BK, N, w, l);
            stage_rows<BK, NW>(smem + OFF_V + (buf ^ 1) * TILE, Vh, k0 + BK, N, w, l);
        }
        if (it < full)
            block_step<false, CAUSAL>(smem, buf, k0, q, N, sc, Lq, negD, qt, gt, acc, l);
        else
            block_step<true, CAUSAL>(smem, buf, k0, q, N, sc, Lq, negD, qt, gt, acc, l);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    }

    // dq_accum[query][d] = acc: lane holds column 32 db + n, rows 8 (r / 4) + 4 h + r % 4
    float* out = dqa + hoff;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int qq = q0 + 32 * w + 8 * (r >> 2) + 4 * h + (r & 3);
            if (qq < N) out[(long long)qq * D + 32 * db + n] = acc[db][r];
        }
}

}  // namespace

hipError_t launch_bwd_dq_d128(const void* Q, const void* K, const void* V, const void* dO,
                              const float* L, const float* Dv, float* dqa, Shape s, float scale,
                              bool causal, hipStream_t st) {
    const int nqb = (s.N + BQ - 1) / BQ;
    const long long nwork = (long long)nqb * s.H * s.B;
    if (nwork > 0x7fffffffLL) return hipErrorInvalidValue;
    dim3 grid((unsigned)nwork);
    if (causal)
        hipLaunchKernelGGL((bwd_dq_kernel<true>), grid, dim3(NW * 64), 0, st, (const bf16_t*)Q,
                           (const bf16_t*)K, (const bf16_t*)V, (const bf16_t*)dO, L, Dv, dqa, s.N,
                           nqb, scale);
    else
        hipLaunchKernelGGL((bwd_dq_kernel<false>), grid, dim3(NW * 64), 0, st, (const bf16_t*)Q,
                           (const bf16_t*)K, (const bf16_t*)V, (const bf16_t*)dO, L, Dv, dqa, s.N,
                           nqb, scale);
    return hipGetLastError();
}

}  // namespace fa
