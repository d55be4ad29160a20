// fwd.hip -- attention forward producing O and the logsumexp L (supporting
// step: it feeds the backward with O and L) on the vector ALUs: fp32 inputs,
// and 16-bit inputs with head dims 16 and 32 (fwd_mfma.hip takes 16-bit
// inputs with head dims 64 and 128).
//
// Query blocks outer, key blocks inner, online softmax per row (1point3acres
// post "手扒了FlashAttention": running max m, denominator l and accumulator a
// start at (-inf, 0, 0); per key block m' = max(m, max s), alpha = exp(m - m'),
// l' = alpha l + sum p, a' = alpha a + p V; finally O = a / l and
// L = m + log l, which FA2 chapter 16 sec 16.4 stores for the backward).
//
// Work split: a 256-lane workgroup owns 64 query rows; each row is handled by
// a quad of lanes that own interleaved columns (k = lane + 4 i) of q and of the
// accumulator, so a K/V row read from LDS is a 4-address broadcast.  Key blocks
// of 32 rows are staged in LDS as fp32.  Under the causal mask the key loop
// stops after the block's last row (whole tiles above the diagonal are never
// visited, FA2 chapter 16 sec 16.8 item 2).  Without O (WITH_O false) the
// kernel only keeps m and l: the pass that recomputes L when the forward did
// not store it (FA2 chapter 16 sec 16.4).
#include "launch.hpp"

namespace fa {

template <typename T, int D, bool CAUSAL, bool WITH_O>
__global__ __launch_bounds__(256) void fwd_simt_kernel(const T* __restrict__ Q,
                                                       const T* __restrict__ K,
                                                       const T* __restrict__ V,
                                                       T* __restrict__ O,
                                                       float* __restrict__ L, int N,
                                                       float scale) {
    constexpr int BR = 64, BC = 32, CPT = D / 4;
    __shared__ float sK[BC][D];
    __shared__ float sV[BC][D];

    const long long head = (long long)blockIdx.z * gridDim.y + blockIdx.y;
    const T* Qh = Q + head * N * D;
    const T* Kh = K + head * N * D;
    const T* Vh = V + head * N * D;
    const int t = threadIdx.x & 3;
    const int r = blockIdx.x * BR + (threadIdx.x >> 2);

    float q[CPT], o[CPT];
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
        q[i] = r < N ? to_f32(Qh[(long long)r * D + t + 4 * i]) * scale : 0.f;
        o[i] = 0.f;
    }
    float m = -INFINITY, l = 0.f;

    const int kend = CAUSAL ? min(N, (int)(blockIdx.x * BR + BR)) : N;
    for (int k0 = 0; k0 < kend; k0 += BC) {
        __syncthreads();
        for (int e = threadIdx.x; e < BC * D; e += 256) {
            const int c = e / D, k = e % D, j = k0 + c;
            sK[c][k] = j < N ? to_f32(Kh[(long long)j * D + k]) : 0.f;
            if (WITH_O) sV[c][k] = j < N ? to_f32(Vh[(long long)j * D + k]) : 0.f;
        }
        __syncthreads();
        float s[BC];
        float mb = -INFINITY;
#pragma unroll
        for (int c = 0; c < BC; ++c) {
            float acc = 0.f;
#pragma unroll
            for (int i = 0; i < CPT; ++i) acc = fmaf(q[i], sK[c][t + 4 * i], acc);
            acc += __shfl_xor(acc, 1, 64);
            acc += __shfl_xor(acc, 2, 64);
            const int j = k0 + c;
            const bool vis = j < N && (!CAUSAL || j <= r);
            s[c] = vis ? acc : -INFINITY;
            mb = fmaxf(mb, s[c]);
        }
        const float mn = fmaxf(m, mb);
        if (mn == -INFINITY) continue;  // nothing visible yet for this row
        const float alpha = (m == -INFINITY) ? 0.f : expf(m - mn);
        l *= alpha;
        if (WITH_O)
#pragma unroll
            for (int i = 0; i < CPT; ++i) o[i] *= alpha;
#pragma unroll
        for (int c = 0; c < BC; ++c) {
            const float p = (s[c] == -INFINITY) ? 0.f : expf(s[c] - mn);
            l += p;
            if (WITH_O)
#pragma unroll
                for (int i = 0; i < CPT; ++i) o[i] = fmaf(p, sV[c][t + 4 * i], o[i]);
        }
        m = mn;
    }
    if (r < N) {
        if (WITH_O) {
            const float inv = 1.f / l;
#pragma unroll
            for (int i = 0; i < CPT; ++i)
                O[head * N * D + (long long)r * D + t + 4 * i] = from_f32<T>(o[i] * inv);
        }
        if (t == 0) L[head * N + r] = m + logf(l);
    }
}

template <typename T, int D, bool WITH_O>
static hipError_t fwd_t(const void* Q, const void* K, const void* V, void* O, float* L, Shape s,
                        float scale, bool causal, hipStream_t st) {
    dim3 grid((s.N + 63) / 64, s.H, s.B);
    if (causal)
        hipLaunchKernelGGL((fwd_simt_kernel<T, D, true, WITH_O>), grid, dim3(256), 0, st,
                           (const T*)Q, (const T*)K, (const T*)V, (T*)O, L, s.N, scale);
    else
        hipLaunchKernelGGL((fwd_simt_kernel<T, D, false, WITH_O>), grid, dim3(256), 0, st,
                           (const T*)Q, (const T*)K, (const T*)V, (T*)O, L, s.N, scale);
    return hipGetLastError();
}

template <typename T, bool WITH_O>
static hipError_t fwd_d(const void* Q, const void* K, const void* V, void* O, float* L, Shape s,
                        float scale, bool causal, hipStream_t st) {
    switch (s.d) {
        case 16: return fwd_t<T, 16, WITH_O>(Q, K, V, O, L, s, scale, causal, st);
        case 32: return fwd_t<T, 32, WITH_O>(Q, K, V, O, L, s, scale, causal, st);
        case 64: return fwd_t<T, 64, WITH_O>(Q, K, V, O, L, s, scale, causal, st);
        case 128: return fwd_t<T, 128, WITH_O>(Q, K, V, O, L, s, scale, causal, st);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_fwd(int dtype, const void* Q, const void* K, const void* V, void* O, float* L,
                      Shape s, float scale, bool causal, hipStream_t st) {
    return dtype == DT_BF16  ? fwd_d<bf16_t, true>(Q, K, V, O, L, s, scale, causal, st)
           : dtype == DT_F16 ? fwd_d<f16_t, true>(Q, K, V, O, L, s, scale, causal, st)
                             : fwd_d<float, true>(Q, K, V, O, L, s, scale, causal, st);
}

// L alone (no O); V is never read, K stands in for it.
hipError_t launch_lse(int dtype, const void* Q, const void* K, float* L, Shape s, float scale,
                      bool causal, hipStream_t st) {
    return dtype == DT_BF16  ? fwd_d<bf16_t, false>(Q, K, K, nullptr, L, s, scale, causal, st)
           : dtype == DT_F16 ? fwd_d<f16_t, false>(Q, K, K, nullptr, L, s, scale, causal, st)
                             : fwd_d<float, false>(Q, K, K, nullptr, L, s, scale, causal, st);
}

}  // namespace fa
