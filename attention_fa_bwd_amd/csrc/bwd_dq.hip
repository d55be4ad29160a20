// bwd_dq.hip -- the query-outer dQ pass (bwd_dq.hpp) as a kernel of its own, and
// its launchers (fa_bwd_dq, and the dQ-writing form of fa_bwd_noalloc): a
// persistent grid, each workgroup running its scheduled work items back to back.
#include "launch.hpp"
#include "bwd_dq.hpp"

namespace fa {
namespace {

using namespace mf;
using namespace dqp;

template <typename E, int DH, bool CAUSAL, bool DIRECT>
__global__ __launch_bounds__(dqp::NWAVE * 64) void bwd_dq_kernel(
    const e16_t* __restrict__ Q, const e16_t* __restrict__ K, const e16_t* __restrict__ V,
    const e16_t* __restrict__ dO, const float* __restrict__ Lg, const float* __restrict__ Dg,
    void* __restrict__ dq_out, int N, int nqb, int nwork, float scale) {
    __shared__ __attribute__((aligned(1024))) unsigned char smem[dqp::Plan<DH>::LDS_BYTES];
    const Schedule sch(nwork, 0, gridDim.x, blockIdx.x);
    dqp::dq_run<E, DH, CAUSAL, DIRECT>(Q, K, V, dO, Lg, Dg, dq_out, N, nqb, scale, sch,
                                       Run(sch, 0), nwork, smem);
}

template <typename E, int DH, bool CAUSAL, bool DIRECT>
hipError_t launch_dq_k(const void* Q, const void* K, const void* V, const void* dO,
                       const float* L, const float* Dv, void* out, Shape s, float scale, int nqb,
                       int nwork, hipStream_t st) {
    static const int per_cu = resident_per_cu(
        reinterpret_cast<const void*>(&bwd_dq_kernel<E, DH, CAUSAL, DIRECT>), NWAVE * 64);
    // DIRECT: one workgroup per work item (its epilogue cannot sit in the
    // item loop)
    const int G = DIRECT ? nwork : persistent_grid(nwork, per_cu);
    if (G <= 0) return hipErrorInvalidDevice;
    hipLaunchKernelGGL((bwd_dq_kernel<E, DH, CAUSAL, DIRECT>), dim3(G), dim3(NWAVE * 64), 0, st,
                       (const e16_t*)Q, (const e16_t*)K, (const e16_t*)V, (const e16_t*)dO, L, Dv,
                       out, s.N, nqb, nwork, scale);
    return hipGetLastError();
}

template <typename E, int DH, bool DIRECT>
hipError_t launch_dq(const void* Q, const void* K, const void* V, const void* dO, const float* L,
                     const float* Dv, void* out, Shape s, float scale, bool causal,
                     hipStream_t st) {
    const int nqb = (s.N + BQ - 1) / BQ;
    const long long nwork = (long long)nqb * s.H * s.B;
    if (nwork > 0x7fffffffLL) return hipErrorInvalidValue;
    return causal ? launch_dq_k<E, DH, true, DIRECT>(Q, K, V, dO, L, Dv, out, s, scale, nqb,
                                                      (int)nwork, st)
                  : launch_dq_k<E, DH, false, DIRECT>(Q, K, V, dO, L, Dv, out, s, scale, nqb,
                                                       (int)nwork, st);
}

template <typename E, bool DIRECT>
hipError_t launch_dq_e(const void* Q, const void* K, const void* V, const void* dO,
                       const float* L, const float* Dv, void* out, Shape s, float scale,
                       bool causal, hipStream_t st) {
    return s.d == 64 ? launch_dq<E, 64, DIRECT>(Q, K, V, dO, L, Dv, out, s, scale, causal, st)
                     : launch_dq<E, 128, DIRECT>(Q, K, V, dO, L, Dv, out, s, scale, causal, st);
}

template <bool DIRECT>
hipError_t launch_dq_any(int dtype, const void* Q, const void* K, const void* V, const void* dO,
                         const float* L, const float* Dv, void* out, Shape s, float scale,
                         bool causal, hipStream_t st) {
    if (s.d != 64 && s.d != 128) return hipErrorInvalidValue;
    return dtype == DT_F16
               ? launch_dq_e<F16E, DIRECT>(Q, K, V, dO, L, Dv, out, s, scale, causal, st)
               : launch_dq_e<Bf16E, DIRECT>(Q, K, V, dO, L, Dv, out, s, scale, causal, st);
}

}  // namespace

hipError_t launch_bwd_dq_mfma(int dtype, const void* Q, const void* K, const void* V,
                              const void* dO, const float* L, const float* Dv, float* dqa,
                              Shape s, float scale, bool causal, hipStream_t st) {
    return launch_dq_any<false>(dtype, Q, K, V, dO, L, Dv, dqa, s, scale, causal, st);
}

hipError_t launch_bwd_dq_mfma_direct(int dtype, const void* Q, const void* K, const void* V,
                                     const void* dO, const float* L, const float* Dv, void* dQ,
                                     Shape s, float scale, bool causal, hipStream_t st) {
    return launch_dq_any<true>(dtype, Q, K, V, dO, L, Dv, dQ, s, scale, causal, st);
}

}  // namespace fa
