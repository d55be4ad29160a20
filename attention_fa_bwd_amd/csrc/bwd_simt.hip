// bwd_simt.hip -- FA2 backward main kernel on the vector ALUs (fp32 FMA).
//
// It is the fp32 path (true fp32 end to end) and the bring-up path for bf16.
// Loop order and arithmetic follow FA2 chapter 16: key blocks outer (one
// workgroup per key block, head and batch, sec 16.2 and the sec 16.6 grid),
// query blocks inner; per tile S = scale Q K^T and P = exp(S - L) are
// recomputed (sec 16.4), dP = dO V^T, dS = P (dP - D) (sec 16.1), dV += P^T dO
// and dK += dS^T Q accumulate in registers and are written once, dK scaled at
// write-out (sec 16.6), and the unscaled dS K is added into the fp32 dq_accum
// buffer with atomics (sec 16.3).  Under the causal mask the query loop starts
// at the first tile that holds a row >= the key block's first key, and
// diagonal tiles are masked element by element (sec 16.8 item 2).
//
// Tiles: BC keys x BR queries with 256 lanes.  K, V, Q, dO tiles live in LDS
// as fp32 with one word of padding per row so column walks hit distinct banks.
#include "launch.hpp"

namespace fa {

template <typename T, int D, int BC, int BR, bool CAUSAL>
__global__ __launch_bounds__(256) void bwd_simt_kernel(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
    const T* __restrict__ dO, const float* __restrict__ L, const float* __restrict__ Dv,
    float* __restrict__ dqa, T* __restrict__ dK, T* __restrict__ dV, int N, float scale) {
    constexpr int NT = 256;
    constexpr int LPR = NT / BR;         // lanes per score row
    constexpr int EA = BC / LPR;         // score elements per lane
    constexpr int KV_OUT = BC * D / NT;  // dK / dV accumulators per lane
    constexpr int DQ_OUT = BR * D / NT;  // dQ partials per lane
    constexpr int CSTEP = NT / D;        // lanes sharing one column of d
    static_assert(LPR >= 1 && EA >= 1 && LPR * EA == BC && KV_OUT >= 1 && DQ_OUT >= 1 && CSTEP >= 1, "tile too small");

    __shared__ float sK[BC][D + 1], sV[BC][D + 1];
    __shared__ float sQ[BR][D + 1], sdO[BR][D + 1];
    __shared__ float sP[BR][BC + 1], sdS[BR][BC + 1];
    __shared__ float sL[BR], sD[BR];

    const long long head = (long long)blockIdx.z * gridDim.y + blockIdx.y;
    const long long hoff = head * N * D;
    const int k0 = blockIdx.x * BC;
    const int tid = threadIdx.x;

    for (int e = tid; e < BC * D; e += NT) {
        const int c = e / D, k = e % D, j = k0 + c;
        sK[c][k] = j < N ? to_f32(K[hoff + (long long)j * D + k]) : 0.f;
        sV[c][k] = j < N ? to_f32(V[hoff + (long long)j * D + k]) : 0.f;
    }

    const int kcol = tid % D;     // column of d owned in the accumulation phases
    const int rbase = tid / D;    // first key / query row owned in those phases
    float accK[KV_OUT], accV[KV_OUT];
#pragma unroll
    for (int u = 0; u < KV_OUT; ++u) accK[u] = accV[u] = 0.f;

    const int q_begin = CAUSAL ? (k0 / BR) * BR : 0;
    for (int q0 = q_begin; q0 < N; q0 += BR) {
        __syncthreads();  // previous tile fully consumed (and K/V staged on entry)
        for (int e = tid; e < BR * D; e += NT) {
            const int r = e / D, k = e % D, i = q0 + r;
            sQ[r][k] = i < N ? to_f32(Q[hoff + (long long)i * D + k]) : 0.f;
            sdO[r][k] = i < N ? to_f32(dO[hoff + (long long)i * D + k]) : 0.f;
        }
        for (int r = tid; r < BR; r += NT) {
            const int i = q0 + r;
            sL[r] = i < N ? L[head * N + i] : 0.f;
            sD[r] = i < N ? Dv[head * N + i] : 0.f;
        }
        __syncthreads();

        // S, P, dP, dS for this tile: lane owns row r and columns c_u
        {
            const int r = tid / LPR, i = q0 + r;
            float s[EA], dp[EA];
#pragma unroll
            for (int u = 0; u < EA; ++u) s[u] = dp[u] = 0.f;
#pragma unroll 4
            for (int k = 0; k < D; ++k) {
                const float qk = sQ[r][k], gk = sdO[r][k];
#pragma unroll
                for (int u = 0; u < EA; ++u) {
                    const int c = tid % LPR + LPR * u;
                    s[u] = fmaf(qk, sK[c][k], s[u]);
                    dp[u] = fmaf(gk, sV[c][k], dp[u]);
                }
            }
#pragma unroll
            for (int u = 0; u < EA; ++u) {
                const int c = tid % LPR + LPR * u, j = k0 + c;
                const bool vis = i < N && j < N && (!CAUSAL || j <= i);
                const float p = vis ? expf(s[u] * scale - sL[r]) : 0.f;
                sP[r][c] = p;
                sdS[r][c] = p * (dp[u] - sD[r]);
            }
        }
        __syncthreads();

        // dV += P^T dO, dK += dS^T Q  (key rows rbase + CSTEP u, column kcol)
#pragma unroll 2
        for (int r = 0; r < BR; ++r) {
            const float g = sdO[r][kcol], qv = sQ[r][kcol];
#pragma unroll
            for (int u = 0; u < KV_OUT; ++u) {
                const int c = rbase + CSTEP * u;
                accV[u] = fmaf(sP[r][c], g, accV[u]);
                accK[u] = fmaf(sdS[r][c], qv, accK[u]);
            }
        }
        // dq_accum += dS K  (query rows rbase + CSTEP u, column kcol)
        {
            float a[DQ_OUT];
#pragma unroll
            for (int u = 0; u < DQ_OUT; ++u) a[u] = 0.f;
#pragma unroll 2
            for (int c = 0; c < BC; ++c) {
                const float kv = sK[c][kcol];
#pragma unroll
                for (int u = 0; u < DQ_OUT; ++u) a[u] = fmaf(sdS[rbase + CSTEP * u][c], kv, a[u]);
            }
#pragma unroll
            for (int u = 0; u < DQ_OUT; ++u) {
                const int i = q0 + rbase + CSTEP * u;
                if (i < N) atomicAdd(dqa + hoff + (long long)i * D + kcol, a[u]);
            }
        }
    }

#pragma unroll
    for (int u = 0; u < KV_OUT; ++u) {
        const int j = k0 + rbase + CSTEP * u;
        if (j < N) {
            dK[hoff + (long long)j * D + kcol] = from_f32<T>(accK[u] * scale);
            dV[hoff + (long long)j * D + kcol] = from_f32<T>(accV[u]);
        }
    }
}

template <typename T, int D>
static hipError_t bwd_t(const void* Q, const void* K, const void* V, const void* dO,
                        const float* L, const float* Dv, float* dqa, void* dK, void* dV,
                        Shape s, float scale, bool causal, hipStream_t st) {
    constexpr int BT = (D >= 128) ? 16 : 32;  // keep static LDS within 64 KiB
    dim3 grid((s.N + BT - 1) / BT, s.H, s.B);
    if (causal)
        hipLaunchKernelGGL((bwd_simt_kernel<T, D, BT, BT, true>), grid, dim3(256), 0, st,
                           (const T*)Q, (const T*)K, (const T*)V, (const T*)dO, L, Dv, dqa,
                           (T*)dK, (T*)dV, s.N, scale);
    else
        hipLaunchKernelGGL((bwd_simt_kernel<T, D, BT, BT, false>), grid, dim3(256), 0, st,
                           (const T*)Q, (const T*)K, (const T*)V, (const T*)dO, L, Dv, dqa,
                           (T*)dK, (T*)dV, s.N, scale);
    return hipGetLastError();
}

template <typename T>
static hipError_t bwd_d(const void* Q, const void* K, const void* V, const void* dO,
                        const float* L, const float* Dv, float* dqa, void* dK, void* dV,
                        Shape s, float scale, bool causal, hipStream_t st) {
    switch (s.d) {
        case 16: return bwd_t<T, 16>(Q, K, V, dO, L, Dv, dqa, dK, dV, s, scale, causal, st);
        case 32: return bwd_t<T, 32>(Q, K, V, dO, L, Dv, dqa, dK, dV, s, scale, causal, st);
        case 64: return bwd_t<T, 64>(Q, K, V, dO, L, Dv, dqa, dK, dV, s, scale, causal, st);
        case 128: return bwd_t<T, 128>(Q, K, V, dO, L, Dv, dqa, dK, dV, s, scale, causal, st);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_bwd_simt(int dtype, const void* Q, const void* K, const void* V, const void* dO,
                      const float* L, const float* D, float* dq_accum, void* dK, void* dV,
                      Shape s, float scale, bool causal, hipStream_t st) {
    return dtype == DT_BF16
               ? bwd_d<bf16_t>(Q, K, V, dO, L, D, dq_accum, dK, dV, s, scale, causal, st)
           : dtype == DT_F16
               ? bwd_d<f16_t>(Q, K, V, dO, L, D, dq_accum, dK, dV, s, scale, causal, st)
               : bwd_d<float>(Q, K, V, dO, L, D, dq_accum, dK, dV, s, scale, causal, st);
}

}  // namespace fa
