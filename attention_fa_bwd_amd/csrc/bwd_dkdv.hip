// bwd_dkdv.hip -- the key-outer dK/dV pass (bwd_dkdv.hpp) as a kernel of its own,
// and its launcher (fa_bwd_dkdv): a persistent grid, each workgroup running its
// scheduled work items back to back.
#include "launch.hpp"
#include "bwd_dkdv.hpp"

namespace fa {
namespace {

using namespace mf;
using namespace dkvp;

template <typename E, int DH, bool CAUSAL>
__global__ __launch_bounds__(dkvp::NWAVE * 64) void bwd_dkdv_kernel(
    const e16_t* __restrict__ Q, const e16_t* __restrict__ K, const e16_t* __restrict__ V,
    const e16_t* __restrict__ dO, const float* __restrict__ Lg, const float* __restrict__ Dg,
    e16_t* __restrict__ dK, e16_t* __restrict__ dV, int N, int nkb, int nwork, float scale) {
    __shared__ __attribute__((aligned(1024))) unsigned char smem[dkvp::Plan<DH>::LDS_BYTES];
    const Schedule sch(nwork, 0, gridDim.x, blockIdx.x);
    dkvp::dkdv_run<E, DH, CAUSAL>(Q, K, V, dO, Lg, Dg, dK, dV, N, nkb, scale, sch, Run(sch, 0),
                                  nwork, smem);
}

template <typename E, int DH, bool CAUSAL>
hipError_t launch_dkdv_k(const void* Q, const void* K, const void* V, const void* dO,
                         const float* L, const float* Dv, void* dK, void* dV, Shape s,
                         float scale, int nkb, int nwork, hipStream_t st) {
    static const int per_cu = resident_per_cu(
        reinterpret_cast<const void*>(&bwd_dkdv_kernel<E, DH, CAUSAL>), NWAVE * 64);
    const int G = persistent_grid(nwork, per_cu);
    if (G <= 0) return hipErrorInvalidDevice;
    hipLaunchKernelGGL((bwd_dkdv_kernel<E, DH, CAUSAL>), dim3(G), dim3(NWAVE * 64), 0, st,
                       (const e16_t*)Q, (const e16_t*)K, (const e16_t*)V, (const e16_t*)dO, L, Dv,
                       (e16_t*)dK, (e16_t*)dV, s.N, nkb, nwork, scale);
    return hipGetLastError();
}

template <typename E, int DH>
hipError_t launch_dkdv(const void* Q, const void* K, const void* V, const void* dO,
                       const float* L, const float* Dv, void* dK, void* dV, Shape s, float scale,
                       bool causal, hipStream_t st) {
    const int nkb = (s.N + BC - 1) / BC;
    const long long nwork = (long long)nkb * s.H * s.B;
    if (nwork > 0x7fffffffLL) return hipErrorInvalidValue;
    return causal ? launch_dkdv_k<E, DH, true>(Q, K, V, dO, L, Dv, dK, dV, s, scale, nkb,
                                                (int)nwork, st)
                  : launch_dkdv_k<E, DH, false>(Q, K, V, dO, L, Dv, dK, dV, s, scale, nkb,
                                                 (int)nwork, st);
}

template <typename E>
hipError_t launch_dkdv_e(const void* Q, const void* K, const void* V, const void* dO,
                         const float* L, const float* Dv, void* dK, void* dV, Shape s,
                         float scale, bool causal, hipStream_t st) {
    return s.d == 64 ? launch_dkdv<E, 64>(Q, K, V, dO, L, Dv, dK, dV, s, scale, causal, st)
                     : launch_dkdv<E, 128>(Q, K, V, dO, L, Dv, dK, dV, s, scale, causal, st);
}

}  // namespace

hipError_t launch_bwd_dkdv_mfma(int dtype, const void* Q, const void* K, const void* V,
                                const void* dO, const float* L, const float* Dv, void* dK,
                                void* dV, Shape s, float scale, bool causal, hipStream_t st) {
    if (s.d != 64 && s.d != 128) return hipErrorInvalidValue;
    return dtype == DT_F16 ? launch_dkdv_e<F16E>(Q, K, V, dO, L, Dv, dK, dV, s, scale, causal, st)
                           : launch_dkdv_e<Bf16E>(Q, K, V, dO, L, Dv, dK, dV, s, scale, causal, st);
}

}  // namespace fa
