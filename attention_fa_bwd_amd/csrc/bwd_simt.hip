// bwd_simt.hip -- FA2 backward on the vector ALUs (fp32 FMA): fp32 inputs (true
// fp32 end to end) and 16-bit inputs with head dims below 64.
//
// The same two passes as the matrix-core path, so that every dtype and head
// dim sums dQ the same way (FA2 chapter 16 sec 16.3 weighs fp32 atomics for
// dQ against a second, query-outer kernel; on MI355X the atomics measured far
// too slow, and without them every output is bitwise reproducible):
//   * dK/dV pass: key blocks outer, one workgroup per key block, head and
//     batch (sec 16.2, the sec 16.6 grid); per query tile S = scale Q K^T and
//     P = exp(S - L) are recomputed (sec 16.4), dP = dO V^T, dS = P (dP - D)
//     (sec 16.1), and dV += P^T dO, dK += dS^T Q accumulate in registers and
//     are written once, dK scaled at write-out (sec 16.6).  Under the causal
//     mask the query loop starts at the first tile that holds a row >= the
//     key block's first key (sec 16.8 item 2).
//   * dQ pass: query blocks outer, key blocks inner; the same recomputation
//     per tile, dQ += dS K in registers, each dq_accum row written once,
//     unscaled.  Under the causal mask the key loop stops after the block
//     that holds the last query's diagonal.
// Diagonal tiles are masked element by element.
//
// Tiles: BC keys x BR queries with 256 lanes.  K, V, Q, dO tiles live in LDS
// as fp32 with one word of padding per row so column walks hit distinct banks.
#include "launch.hpp"

namespace fa {

// Work split shared by both passes: a score row is handled by LPR lanes
// (score elements c = lane % LPR + LPR u), an output column of d by the lanes
// tid % D, each owning rows tid / D + CSTEP u.
template <int D, int BC, int BR>
struct SimtSplit {
    static constexpr int NT = 256;
    static constexpr int LPR = NT / BR;         // lanes per score row
    static constexpr int EA = BC / LPR;         // score elements per lane
    static constexpr int CSTEP = NT / D;        // lanes sharing one column of d
    static_assert(LPR >= 1 && EA >= 1 && LPR * EA == BC && CSTEP >= 1, "tile too small");
};

// S and dP of score row r against the BC staged keys, then P = exp(S - L) and
// dS = P (dP - D) into sP / sdS (P = 0 where the key is past N, past the
// query under the causal mask, or the row is past N).
template <int D, int BC, int BR, bool CAUSAL>
__device__ __forceinline__ void simt_scores(const float (&sQ)[BR][D + 1],
                                            const float (&sdO)[BR][D + 1],
                                            const float (&sK)[BC][D + 1],
                                            const float (&sV)[BC][D + 1], const float* sL,
                                            const float* sD, float (*sP)[BC + 1],
                                            float (&sdS)[BR][BC + 1], int q0, int k0, int N,
                                            float scale) {
    using W = SimtSplit<D, BC, BR>;
    const int tid = threadIdx.x;
    const int r = tid / W::LPR, i = q0 + r;
    float s[W::EA], dp[W::EA];
#pragma unroll
    for (int u = 0; u < W::EA; ++u) s[u] = dp[u] = 0.f;
#pragma unroll 4
    for (int k = 0; k < D; ++k) {
        const float qk = sQ[r][k], gk = sdO[r][k];
#pragma unroll
        for (int u = 0; u < W::EA; ++u) {
            const int c = tid % W::LPR + W::LPR * u;
            s[u] = fmaf(qk, sK[c][k], s[u]);
            dp[u] = fmaf(gk, sV[c][k], dp[u]);
        }
    }
#pragma unroll
    for (int u = 0; u < W::EA; ++u) {
        const int c = tid % W::LPR + W::LPR * u, j = k0 + c;
        const bool vis = i < N && j < N && (!CAUSAL || j <= i);
        const float p = vis ? expf(s[u] * scale - sL[r]) : 0.f;
        if (sP) sP[r][c] = p;
        sdS[r][c] = p * (dp[u] - sD[r]);
    }
}

// rows [r0, r0 + ROWS) of a [N, D] head into an LDS tile (zeros past N)
template <typename T, int D, int ROWS>
__device__ __forceinline__ void simt_stage(float (&dst)[ROWS][D + 1], const T* src, int r0, int N) {
    for (int e = threadIdx.x; e < ROWS * D; e += 256) {
        const int r = e / D, k = e % D, g = r0 + r;
        dst[r][k] = g < N ? to_f32(src[(long long)g * D + k]) : 0.f;
    }
}

// dK/dV pass, key block kb of head `head` (batch and head folded)
template <typename T, int D, int BC, int BR, bool CAUSAL>
__device__ __forceinline__ void simt_dkdv_block(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
    const T* __restrict__ dO, const float* __restrict__ L, const float* __restrict__ Dv,
    T* __restrict__ dK, T* __restrict__ dV, int N, float scale, int kb, long long head) {
    using W = SimtSplit<D, BC, BR>;
    constexpr int KV_OUT = BC * D / W::NT;  // dK / dV accumulators per lane
    static_assert(KV_OUT >= 1 && KV_OUT * W::NT == BC * D, "tile too small");

    __shared__ float sK[BC][D + 1], sV[BC][D + 1];
    __shared__ float sQ[BR][D + 1], sdO[BR][D + 1];
    __shared__ float sP[BR][BC + 1], sdS[BR][BC + 1];
    __shared__ float sL[BR], sD[BR];

    const long long hoff = head * N * D;
    const int k0 = kb * BC;
    const int tid = threadIdx.x;

    simt_stage<T, D, BC>(sK, K + hoff, k0, N);
    simt_stage<T, D, BC>(sV, V + hoff, k0, N);

    const int kcol = tid % D;       // column of d owned in the accumulation phase
    const int rbase = tid / D;      // first key row owned there
    float accK[KV_OUT], accV[KV_OUT];
#pragma unroll
    for (int u = 0; u < KV_OUT; ++u) accK[u] = accV[u] = 0.f;

    const int q_begin = CAUSAL ? (k0 / BR) * BR : 0;
    for (int q0 = q_begin; q0 < N; q0 += BR) {
        __syncthreads();  // previous tile fully consumed (and K/V staged on entry)
        simt_stage<T, D, BR>(sQ, Q + hoff, q0, N);
        simt_stage<T, D, BR>(sdO, dO + hoff, q0, N);
        for (int r = tid; r < BR; r += W::NT) {
            const int i = q0 + r;
            sL[r] = i < N ? L[head * N + i] : 0.f;
            sD[r] = i < N ? Dv[head * N + i] : 0.f;
        }
        __syncthreads();
        simt_scores<D, BC, BR, CAUSAL>(sQ, sdO, sK, sV, sL, sD, sP, sdS, q0, k0, N, scale);
        __syncthreads();
        // dV += P^T dO, dK += dS^T Q  (key rows rbase + CSTEP u, column kcol)
#pragma unroll 2
        for (int r = 0; r < BR; ++r) {
            const float g = sdO[r][kcol], qv = sQ[r][kcol];
#pragma unroll
            for (int u = 0; u < KV_OUT; ++u) {
                const int c = rbase + W::CSTEP * u;
                accV[u] = fmaf(sP[r][c], g, accV[u]);
                accK[u] = fmaf(sdS[r][c], qv, accK[u]);
            }
        }
    }

#pragma unroll
    for (int u = 0; u < KV_OUT; ++u) {
        const int j = k0 + rbase + W::CSTEP * u;
        if (j < N) {
            dK[hoff + (long long)j * D + kcol] = from_f32<T>(accK[u] * scale);
            dV[hoff + (long long)j * D + kcol] = from_f32<T>(accV[u]);
        }
    }
}

// DIRECT: instead of the unscaled fp32 dq_accum, write dQ = scale * acc in the
// element type (round to nearest even), exactly what the convert step makes of
// dq_accum; out is then the dQ tensor.
// dQ pass, query block qb of head `head`
template <typename T, int D, int BC, int BR, bool CAUSAL, bool DIRECT>
__device__ __forceinline__ void simt_dq_block(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
    const T* __restrict__ dO, const float* __restrict__ L, const float* __restrict__ Dv,
    void* __restrict__ out, int N, float scale, int qb, long long head) {
    using W = SimtSplit<D, BC, BR>;
    constexpr int DQ_OUT = BR * D / W::NT;  // dQ accumulators per lane
    static_assert(DQ_OUT >= 1 && DQ_OUT * W::NT == BR * D, "tile too small");

    __shared__ float sK[BC][D + 1], sV[BC][D + 1];
    __shared__ float sQ[BR][D + 1], sdO[BR][D + 1];
    __shared__ float sdS[BR][BC + 1];
    __shared__ float sL[BR], sD[BR];

    const long long hoff = head * N * D;
    const int q0 = qb * BR;
    const int tid = threadIdx.x;

    simt_stage<T, D, BR>(sQ, Q + hoff, q0, N);
    simt_stage<T, D, BR>(sdO, dO + hoff, q0, N);
    for (int r = tid; r < BR; r += W::NT) {
        const int i = q0 + r;
        sL[r] = i < N ? L[head * N + i] : 0.f;
        sD[r] = i < N ? Dv[head * N + i] : 0.f;
    }

    const int kcol = tid % D;       // column of d owned in the accumulation phase
    const int rbase = tid / D;      // first query row owned there
    float acc[DQ_OUT];
#pragma unroll
    for (int u = 0; u < DQ_OUT; ++u) acc[u] = 0.f;

    const int kend = CAUSAL ? min(N, q0 + BR) : N;
    for (int k0 = 0; k0 < kend; k0 += BC) {
        __syncthreads();  // previous block fully consumed (and Q/dO staged on entry)
        simt_stage<T, D, BC>(sK, K + hoff, k0, N);
        simt_stage<T, D, BC>(sV, V + hoff, k0, N);
        __syncthreads();
        simt_scores<D, BC, BR, CAUSAL>(sQ, sdO, sK, sV, sL, sD, nullptr, sdS, q0, k0, N, scale);
        __syncthreads();
        // dQ += dS K  (query rows rbase + CSTEP u, column kcol)
#pragma unroll 2
        for (int c = 0; c < BC; ++c) {
            const float kv = sK[c][kcol];
#pragma unroll
            for (int u = 0; u < DQ_OUT; ++u) acc[u] = fmaf(sdS[rbase + W::CSTEP * u][c], kv, acc[u]);
        }
    }

#pragma unroll
    for (int u = 0; u < DQ_OUT; ++u) {
        const int i = q0 + rbase + W::CSTEP * u;
        if (i >= N) continue;
        if constexpr (DIRECT) {
            // the fp32 product first, as the convert step forms it (not fused
            // into one mixed-precision rounding)
            float x = acc[u] * scale;
            asm volatile("" : "+v"(x));
            reinterpret_cast<T*>(out)[hoff + (long long)i * D + kcol] = from_f32<T>(x);
        } else
            reinterpret_cast<float*>(out)[hoff + (long long)i * D + kcol] = acc[u];
    }
}

template <typename T, int D, int BC, int BR, bool CAUSAL>
__global__ __launch_bounds__(256) void simt_dkdv_kernel(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
    const T* __restrict__ dO, const float* __restrict__ L, const float* __restrict__ Dv,
    T* __restrict__ dK, T* __restrict__ dV, int N, float scale) {
    simt_dkdv_block<T, D, BC, BR, CAUSAL>(Q, K, V, dO, L, Dv, dK, dV, N, scale, blockIdx.x,
                                          (long long)blockIdx.z * gridDim.y + blockIdx.y);
}

template <typename T, int D, int BC, int BR, bool CAUSAL, bool DIRECT>
__global__ __launch_bounds__(256) void simt_dq_kernel(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
    const T* __restrict__ dO, const float* __restrict__ L, const float* __restrict__ Dv,
    void* __restrict__ out, int N, float scale) {
    simt_dq_block<T, D, BC, BR, CAUSAL, DIRECT>(Q, K, V, dO, L, Dv, out, N, scale, blockIdx.x,
                                                (long long)blockIdx.z * gridDim.y + blockIdx.y);
}

// Both passes in one launch (fa_bwd): workgroups x < nqb run dQ-pass blocks,
// the others dK/dV-pass blocks; they read the same inputs and write disjoint
// outputs, so nothing orders them, and the results are bitwise those of the
// two kernels above.
template <typename T, int D, int BC, int BR, bool CAUSAL>
__global__ __launch_bounds__(256) void simt_fused_kernel(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
    const T* __restrict__ dO, const float* __restrict__ L, const float* __restrict__ Dv,
    float* __restrict__ dq_accum, T* __restrict__ dK, T* __restrict__ dV, int N, int nqb,
    float scale) {
    const long long head = (long long)blockIdx.z * gridDim.y + blockIdx.y;
    if ((int)blockIdx.x < nqb)
        simt_dq_block<T, D, BC, BR, CAUSAL, false>(Q, K, V, dO, L, Dv, dq_accum, N, scale,
                                                   blockIdx.x, head);
    else
        simt_dkdv_block<T, D, BC, BR, CAUSAL>(Q, K, V, dO, L, Dv, dK, dV, N, scale,
                                              blockIdx.x - nqb, head);
}

namespace {

// tiles of 16 (d = 128) or 32 rows keep the static LDS within 64 KiB
template <int D>
constexpr int simt_tile() { return D >= 128 ? 16 : 32; }

template <typename T, int D>
hipError_t dkdv_t(const void* Q, const void* K, const void* V, const void* dO, const float* L,
                  const float* Dv, void* dK, void* dV, Shape s, float scale, bool causal,
                  hipStream_t st) {
    constexpr int BT = simt_tile<D>();
    dim3 grid((s.N + BT - 1) / BT, s.H, s.B);
    if (causal)
        hipLaunchKernelGGL((simt_dkdv_kernel<T, D, BT, BT, true>), grid, dim3(256), 0, st,
                           (const T*)Q, (const T*)K, (const T*)V, (const T*)dO, L, Dv, (T*)dK,
                           (T*)dV, s.N, scale);
    else
        hipLaunchKernelGGL((simt_dkdv_kernel<T, D, BT, BT, false>), grid, dim3(256), 0, st,
                           (const T*)Q, (const T*)K, (const T*)V, (const T*)dO, L, Dv, (T*)dK,
                           (T*)dV, s.N, scale);
    return hipGetLastError();
}

template <typename T, int D, bool DIRECT>
hipError_t dq_t(const void* Q, const void* K, const void* V, const void* dO, const float* L,
                const float* Dv, void* out, Shape s, float scale, bool causal, hipStream_t st) {
    constexpr int BT = simt_tile<D>();
    dim3 grid((s.N + BT - 1) / BT, s.H, s.B);
    if (causal)
        hipLaunchKernelGGL((simt_dq_kernel<T, D, BT, BT, true, DIRECT>), grid, dim3(256), 0, st,
                           (const T*)Q, (const T*)K, (const T*)V, (const T*)dO, L, Dv, out, s.N,
                           scale);
    else
        hipLaunchKernelGGL((simt_dq_kernel<T, D, BT, BT, false, DIRECT>), grid, dim3(256), 0, st,
                           (const T*)Q, (const T*)K, (const T*)V, (const T*)dO, L, Dv, out, s.N,
                           scale);
    return hipGetLastError();
}

template <typename T, int D>
hipError_t fused_t(const void* Q, const void* K, const void* V, const void* dO, const float* L,
                   const float* Dv, float* dqa, void* dK, void* dV, Shape s, float scale,
                   bool causal, hipStream_t st) {
    constexpr int BT = simt_tile<D>();
    const int nb = (s.N + BT - 1) / BT;
    dim3 grid(2 * nb, s.H, s.B);
    if (causal)
        hipLaunchKernelGGL((simt_fused_kernel<T, D, BT, BT, true>), grid, dim3(256), 0, st,
                           (const T*)Q, (const T*)K, (const T*)V, (const T*)dO, L, Dv, dqa,
                           (T*)dK, (T*)dV, s.N, nb, scale);
    else
        hipLaunchKernelGGL((simt_fused_kernel<T, D, BT, BT, false>), grid, dim3(256), 0, st,
                           (const T*)Q, (const T*)K, (const T*)V, (const T*)dO, L, Dv, dqa,
                           (T*)dK, (T*)dV, s.N, nb, scale);
    return hipGetLastError();
}

template <typename T>
hipError_t fused_d(const void* Q, const void* K, const void* V, const void* dO, const float* L,
                   const float* Dv, float* dqa, void* dK, void* dV, Shape s, float scale,
                   bool causal, hipStream_t st) {
    switch (s.d) {
        case 16: return fused_t<T, 16>(Q, K, V, dO, L, Dv, dqa, dK, dV, s, scale, causal, st);
        case 32: return fused_t<T, 32>(Q, K, V, dO, L, Dv, dqa, dK, dV, s, scale, causal, st);
        case 64: return fused_t<T, 64>(Q, K, V, dO, L, Dv, dqa, dK, dV, s, scale, causal, st);
        case 128: return fused_t<T, 128>(Q, K, V, dO, L, Dv, dqa, dK, dV, s, scale, causal, st);
    }
    return hipErrorInvalidValue;
}

template <typename T>
hipError_t dkdv_d(const void* Q, const void* K, const void* V, const void* dO, const float* L,
                  const float* Dv, void* dK, void* dV, Shape s, float scale, bool causal,
                  hipStream_t st) {
    switch (s.d) {
        case 16: return dkdv_t<T, 16>(Q, K, V, dO, L, Dv, dK, dV, s, scale, causal, st);
        case 32: return dkdv_t<T, 32>(Q, K, V, dO, L, Dv, dK, dV, s, scale, causal, st);
        case 64: return dkdv_t<T, 64>(Q, K, V, dO, L, Dv, dK, dV, s, scale, causal, st);
        case 128: return dkdv_t<T, 128>(Q, K, V, dO, L, Dv, dK, dV, s, scale, causal, st);
    }
    return hipErrorInvalidValue;
}

template <typename T, bool DIRECT>
hipError_t dq_d(const void* Q, const void* K, const void* V, const void* dO, const float* L,
                const float* Dv, void* out, Shape s, float scale, bool causal, hipStream_t st) {
    switch (s.d) {
        case 16: return dq_t<T, 16, DIRECT>(Q, K, V, dO, L, Dv, out, s, scale, causal, st);
        case 32: return dq_t<T, 32, DIRECT>(Q, K, V, dO, L, Dv, out, s, scale, causal, st);
        case 64: return dq_t<T, 64, DIRECT>(Q, K, V, dO, L, Dv, out, s, scale, causal, st);
        case 128: return dq_t<T, 128, DIRECT>(Q, K, V, dO, L, Dv, out, s, scale, causal, st);
    }
    return hipErrorInvalidValue;
}

template <bool DIRECT>
hipError_t dq_any(int dtype, const void* Q, const void* K, const void* V, const void* dO,
                  const float* L, const float* D, void* out, Shape s, float scale, bool causal,
                  hipStream_t st) {
    return dtype == DT_BF16  ? dq_d<bf16_t, DIRECT>(Q, K, V, dO, L, D, out, s, scale, causal, st)
           : dtype == DT_F16 ? dq_d<f16_t, DIRECT>(Q, K, V, dO, L, D, out, s, scale, causal, st)
                             : dq_d<float, DIRECT>(Q, K, V, dO, L, D, out, s, scale, causal, st);
}

}  // namespace

hipError_t launch_bwd_dkdv_simt(int dtype, const void* Q, const void* K, const void* V,
                                const void* dO, const float* L, const float* D, void* dK,
                                void* dV, Shape s, float scale, bool causal, hipStream_t st) {
    return dtype == DT_BF16   ? dkdv_d<bf16_t>(Q, K, V, dO, L, D, dK, dV, s, scale, causal, st)
           : dtype == DT_F16  ? dkdv_d<f16_t>(Q, K, V, dO, L, D, dK, dV, s, scale, causal, st)
                              : dkdv_d<float>(Q, K, V, dO, L, D, dK, dV, s, scale, causal, st);
}

hipError_t launch_bwd_fused_simt(int dtype, const void* Q, const void* K, const void* V,
                                 const void* dO, const float* L, const float* D, float* dq_accum,
                                 void* dK, void* dV, Shape s, float scale, bool causal,
                                 hipStream_t st) {
    return dtype == DT_BF16  ? fused_d<bf16_t>(Q, K, V, dO, L, D, dq_accum, dK, dV, s, scale, causal, st)
           : dtype == DT_F16 ? fused_d<f16_t>(Q, K, V, dO, L, D, dq_accum, dK, dV, s, scale, causal, st)
                             : fused_d<float>(Q, K, V, dO, L, D, dq_accum, dK, dV, s, scale, causal, st);
}

hipError_t launch_bwd_dq_simt(int dtype, const void* Q, const void* K, const void* V,
                              const void* dO, const float* L, const float* D, float* dq_accum,
                              Shape s, float scale, bool causal, hipStream_t st) {
    return dq_any<false>(dtype, Q, K, V, dO, L, D, dq_accum, s, scale, causal, st);
}

hipError_t launch_bwd_dq_simt_direct(int dtype, const void* Q, const void* K, const void* V,
                                     const void* dO, const float* L, const float* D, void* dQ,
                                     Shape s, float scale, bool causal, hipStream_t st) {
    return dq_any<true>(dtype, Q, K, V, dO, L, D, dQ, s, scale, causal, st);
}

}  // namespace fa
