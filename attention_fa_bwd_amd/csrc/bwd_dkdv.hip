// bwd_dkdv.hip -- key-outer pass of the FA2 backward on gfx950 matrix cores:
// dK and dV for bf16, head dim 128.
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
// gfx950 mapping (4 waves, one per SIMD; wave w owns keys [32 w, 32 w + 32)):
//   * the K^T and V^T B-operand fragments of S = Q K^T and dP = dO V^T stay in
//     registers for the whole query loop, as do the dV^T and dK^T accumulators
//     (32 d x 32 keys x 4 d-blocks each);
//   * query tiles of 64 rows of Q and dO are double-buffered in LDS (swizzled
//     256-byte rows) and filled with direct-to-LDS loads one tile ahead;
//   * S and dP leave the matrix core with the key on the lane, so P and dS are
//     B operands of dV^T = dO^T P and dK^T = Q^T dS straight from registers;
//     the transposed A operands dO^T and Q^T come from the same LDS tiles
//     through ds_read_b64_tr_b16;
//   * the dP accumulator starts from -D, so it leaves the matrix core as
//     dP - D; P = exp2(S * scale * log2(e) - L * log2(e)) with L * log2(e)
//     staged once per tile; rows at or beyond N get L = +inf (P = 0, dS = 0);
//   * keys at or beyond N need no mask: their P and dS only reach their own
//     dV / dK rows, which are not stored.
#include "launch.hpp"
#include "mfma_common.hpp"

namespace fa {
namespace {

using namespace mf;

constexpr int BC = 128;                 // keys per workgroup
constexpr int BR = 64;                  // queries per tile
constexpr int NW = 4;                   // waves
constexpr int TILE = BR * ROWB;         // 16 KiB
constexpr int OFF_Q = 0;                // 2 buffers
constexpr int OFF_DO = 2 * TILE;        // 2 buffers
constexpr int OFF_L = 4 * TILE;         // 2 x BR floats: L * log2(e)
constexpr int OFF_ND = OFF_L + 2 * BR * 4;  // 2 x BR floats: -D
constexpr int LDS_BYTES = OFF_ND + 2 * BR * 4;

// Issue the loads of query tile q0 into buffer `buf` (Q, dO direct to LDS;
// L and D into registers of waves 0 and 1, written to LDS by put_rowstats).
__device__ __forceinline__ float stage_tile(unsigned char* smem, int buf, const bf16_t* Qh,
                                            const bf16_t* dOh, const float* Lh, const float* Dh,
                                            int q0, int N, int w, int l) {
    stage_rows<BR, NW>(smem + OFF_Q + buf * TILE, Qh, q0, N, w, l);
    stage_rows<BR, NW>(smem + OFF_DO + buf * TILE, dOh, q0, N, w, l);
    float v = 0.f;
    const int q = q0 + l;
    if (w == 0) v = q < N ? Lh[q] * kLog2e : INFINITY;
    if (w == 1) v = q < N ? -Dh[q] : 0.f;
    return v;
}

__device__ __forceinline__ void put_rowstats(unsigned char* smem, int buf, float v, int w, int l) {
    if (w == 0) reinterpret_cast<float*>(smem + OFF_L)[buf * BR + l] = v;
    if (w == 1) reinterpret_cast<float*>(smem + OFF_ND)[buf * BR + l] = v;
}

template <bool MASK>
__device__ __forceinline__ void tile_step(const unsigned char* smem, int buf, int q0, int key,
                                          float sc, const bf16x8_t (&kt)[8],
                                          const bf16x8_t (&vt)[8], f32x16_t (&accdV)[4],
                                          f32x16_t (&accdK)[4], int l) {
    const int h = l >> 5, n = l & 31, g2 = (l >> 4) & 1;
    const unsigned char* sQ = smem + OFF_Q + buf * TILE;
    const unsigned char* sdO = smem + OFF_DO + buf * TILE;
    const float* sL = reinterpret_cast<const float*>(smem + OFF_L) + buf * BR;
    const float* sND = reinterpret_cast<const float*>(smem + OFF_ND) + buf * BR;

    // S = Q K^T and dP - D = dO V^T - D; query on rows, key on lanes
    f32x16_t S[2], dP[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
        f32x4_t nd[4];
#pragma unroll
        for (int a4 = 0; a4 < 4; ++a4)
            nd[a4] = *reinterpret_cast<const f32x4_t*>(sND + 32 * qb + 8 * a4 + 4 * h);
        dP[qb] = __builtin_shufflevector(
            __builtin_shufflevector(nd[0], nd[1], 0, 1, 2, 3, 4, 5, 6, 7),
            __builtin_shufflevector(nd[2], nd[3], 0, 1, 2, 3, 4, 5, 6, 7), 0, 1, 2, 3, 4, 5, 6, 7,
            8, 9, 10, 11, 12, 13, 14, 15);
        S[qb] = f32x16_t{};
        const int row = 32 * qb + n;
#pragma unroll
        for (int dk = 0; dk < 8; ++dk) {
            const int off = tile_off(row, 32 * dk + 16 * h);
            S[qb] = mfma(lds_b128(sQ + off), kt[dk], S[qb]);
            dP[qb] = mfma(lds_b128(sdO + off), vt[dk], dP[qb]);
        }
    }

    // P = exp2(S sc - L'), dS = P (dP - D), both to bf16
    bf16x8_t Pb[2][2], dSb[2][2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
        float p[16], ds[16];
#pragma unroll
        for (int a4 = 0; a4 < 4; ++a4) {
            const int rq = 32 * qb + 8 * a4 + 4 * h;
            const f32x4_t Lv = *reinterpret_cast<const f32x4_t*>(sL + rq);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 4 * a4 + e;
                float x = __builtin_fmaf(S[qb][r], sc, -Lv[e]);
                if (MASK && key > q0 + rq + e) x = -INFINITY;
                const float pv = __builtin_amdgcn_exp2f(x);
                p[r] = pv;
                ds[r] = pv * dP[qb][r];
            }
        }
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            Pb[qb][hh] = as_bf16x8(pack8(p + 8 * hh));
            dSb[qb][hh] = as_bf16x8(pack8(ds + 8 * hh));
        }
    }

    // dV^T += dO^T P, dK^T += Q^T dS; d on rows, key on lanes
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const int r0 = 16 * t + 4 * h + ((l & 15) >> 2);
#pragma unroll
        for (int db = 0; db < 4; ++db) {
            const int colb = 64 * db + 32 * g2 + 8 * (l & 3);
            const int o0 = tile_off(r0, colb), o1 = tile_off(r0 + 8, colb);
            accdV[db] = mfma(tr16_pair(sdO + o0, sdO + o1), Pb[t >> 1][t & 1], accdV[db]);
            accdK[db] = mfma(tr16_pair(sQ + o0, sQ + o1), dSb[t >> 1][t & 1], accdK[db]);
        }
    }

}

template <bool CAUSAL>
__global__ __launch_bounds__(NW * 64) void bwd_dkdv_kernel(
    const bf16_t* __restrict__ Q, const bf16_t* __restrict__ K, const bf16_t* __restrict__ V,
    const bf16_t* __restrict__ dO, const float* __restrict__ Lg, const float* __restrict__ Dg,
    bf16_t* __restrict__ dK, bf16_t* __restrict__ dV, int N, int nkb, float scale) {
    __shared__ __attribute__((aligned(1024))) unsigned char smem[LDS_BYTES];

    const int work = xcd_work_item(blockIdx.x, gridDim.x);
    const int head = work / nkb;
    const int k0 = (work % nkb) * BC;  // heaviest key blocks first under the causal mask
    const long long hoff = (long long)head * N * D;
    const bf16_t* Qh = Q + hoff;
    const bf16_t* dOh = dO + hoff;
    const float* Lh = Lg + (long long)head * N;
    const float* Dh = Dg + (long long)head * N;

    const int w = threadIdx.x >> 6, l = threadIdx.x & 63, h = l >> 5, n = l & 31;
    const int key = k0 + 32 * w + n;
    const int keyc = key < N ? key : N - 1;  // clamped: finite data, outputs not stored

    bf16x8_t kt[8], vt[8];
#pragma unroll
    for (int dk = 0; dk < 8; ++dk) {
        kt[dk] = as_bf16x8(*reinterpret_cast<const uint4*>(K + hoff + (long long)keyc * D + 16 * dk + 8 * h));
        vt[dk] = as_bf16x8(*reinterpret_cast<const uint4*>(V + hoff + (long long)keyc * D + 16 * dk + 8 * h));
    }
    f32x16_t accdV[4], accdK[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) accdV[i] = accdK[i] = f32x16_t{};

    const int q_begin = CAUSAL ? k0 : 0;
    const int ntiles = (N - q_begin + BR - 1) / BR;
    const int nmask = CAUSAL ? BC / BR : 0;  // tiles that cross the diagonal
    const float sc = scale * kLog2e;

    float rs = stage_tile(smem, 0, Qh, dOh, Lh, Dh, q_begin, N, w, l);
    put_rowstats(smem, 0, rs, w, l);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    for (int it = 0; it < ntiles; ++it) {
        const int buf = it & 1;
        const int q0 = q_begin + it * BR;
        const bool more = it + 1 < ntiles;
        if (more) rs = stage_tile(smem, buf ^ 1, Qh, dOh, Lh, Dh, q0 + BR, N, w, l);
        if (it < nmask)
            tile_step<true>(smem, buf, q0, key, sc, kt, vt, accdV, accdK, l);
        else
            tile_step<false>(smem, buf, q0, key, sc, kt, vt, accdV, accdK, l);
        if (more) put_rowstats(smem, buf ^ 1, rs, w, l);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    }

    if (key < N) {
        bf16_t* dKr = dK + hoff + (long long)key * D;
        bf16_t* dVr = dV + hoff + (long long)key * D;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int a4 = 0; a4 < 4; ++a4) {
                const int d0 = 32 * db + 8 * a4 + 4 * h;
                const int r = 4 * a4;
                uint2 kv, vv;
                kv.x = pack_bf16x2(accdK[db][r] * scale, accdK[db][r + 1] * scale);
                kv.y = pack_bf16x2(accdK[db][r + 2] * scale, accdK[db][r + 3] * scale);
                vv.x = pack_bf16x2(accdV[db][r], accdV[db][r + 1]);
                vv.y = pack_bf16x2(accdV[db][r + 2], accdV[db][r + 3]);
                *reinterpret_cast<uint2*>(dKr + d0) = kv;
                *reinterpret_cast<uint2*>(dVr + d0) = vv;
            }
    }
}

}  // namespace

hipError_t launch_bwd_dkdv_d128(const void* Q, const void* K, const void* V, const void* dO,
                                const float* L, const float* Dv, void* dK, void* dV, Shape s,
                                float scale, bool causal, hipStream_t st) {
    const int nkb = (s.N + BC - 1) / BC;
    const long long nwork = (long long)nkb * s.H * s.B;
    if (nwork > 0x7fffffffLL) return hipErrorInvalidValue;
    dim3 grid((unsigned)nwork);
    if (causal)
        hipLaunchKernelGGL((bwd_dkdv_kernel<true>), grid, dim3(NW * 64), 0, st, (const bf16_t*)Q,
                           (const bf16_t*)K, (const bf16_t*)V, (const bf16_t*)dO, L, Dv,
                           (bf16_t*)dK, (bf16_t*)dV, s.N, nkb, scale);
    else
        hipLaunchKernelGGL((bwd_dkdv_kernel<false>), grid, dim3(NW * 64), 0, st, (const bf16_t*)Q,
                           (const bf16_t*)K, (const bf16_t*)V, (const bf16_t*)dO, L, Dv,
                           (bf16_t*)dK, (bf16_t*)dV, s.N, nkb, scale);
    return hipGetLastError();
}

}  // namespace fa
