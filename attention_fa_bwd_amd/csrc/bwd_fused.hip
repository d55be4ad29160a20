// bwd_fused.hip -- fa_bwd's two matrix-core passes in one launch.
//
// Given D, the query-outer dQ pass (bwd_dq.hpp) and the key-outer dK/dV pass
// (bwd_dkdv.hpp) read the same inputs and write disjoint outputs, so nothing
// orders them (FA2 chapter 16 sec 16.3: dQ by a separate kernel instead of
// atomics).  One grid holds the work items of both: workgroups [0, nq) run
// dQ-pass items, workgroups [nq, nq + nk) dK/dV-pass items, each exactly as
// in its own kernel (same code, same per-item order and XCD placement, so the
// results are bitwise those of fa_bwd_dq followed by fa_bwd_dkdv).  The
// dQ-pass items go first (each carries 1.5 times the work of a dK/dV item at
// the same N); the CUs that finish them start on dK/dV items while the last
// dQ items still run, so neither pass leaves a tail of idle CUs, a small
// problem runs both passes side by side instead of one after the other, and
// the second launch is saved.
#include "bwd_dkdv.hpp"
#include "bwd_dq.hpp"
#include "launch.hpp"

namespace fa {
namespace {

using namespace mf;

static_assert(dqp::NWAVE == dkvp::NWAVE, "one workgroup shape for both passes");

template <int DH>
constexpr int fused_lds() {
    return dqp::Plan<DH>::LDS_BYTES > dkvp::Plan<DH>::LDS_BYTES ? dqp::Plan<DH>::LDS_BYTES
                                                                 : dkvp::Plan<DH>::LDS_BYTES;
}

template <typename E, int DH, bool CAUSAL>
__global__ __launch_bounds__(dqp::NWAVE * 64) void bwd_fused_kernel(
    const e16_t* __restrict__ Q, const e16_t* __restrict__ K, const e16_t* __restrict__ V,
    const e16_t* __restrict__ dO, const float* __restrict__ Lg, const float* __restrict__ Dg,
    float* __restrict__ dqa, e16_t* __restrict__ dK, e16_t* __restrict__ dV, int N, int nqb,
    int nkb, int nq, int nk, float scale) {
    __shared__ __attribute__((aligned(1024))) unsigned char smem[fused_lds<DH>()];
    const int bid = blockIdx.x;
    if (bid < nq)
        dqp::dq_work<E, DH, CAUSAL, false>(Q, K, V, dO, Lg, Dg, dqa, N, nqb, scale, bid, nq, smem);
    else
        dkvp::dkdv_work<E, DH, CAUSAL>(Q, K, V, dO, Lg, Dg, dK, dV, N, nkb, scale, bid - nq, nk,
                                       smem);
}

template <typename E, int DH>
hipError_t launch_fused(const void* Q, const void* K, const void* V, const void* dO,
                        const float* L, const float* Dv, float* dqa, void* dK, void* dV, Shape s,
                        float scale, bool causal, hipStream_t st) {
    const int nqb = (s.N + dqp::BQ - 1) / dqp::BQ;
    const int nkb = (s.N + dkvp::BC - 1) / dkvp::BC;
    const long long nq = (long long)nqb * s.H * s.B, nk = (long long)nkb * s.H * s.B;
    if (nq + nk > 0x7fffffffLL) return hipErrorInvalidValue;
    dim3 grid((unsigned)(nq + nk));
    if (causal)
        hipLaunchKernelGGL((bwd_fused_kernel<E, DH, true>), grid, dim3(dqp::NWAVE * 64), 0, st,
                           (const e16_t*)Q, (const e16_t*)K, (const e16_t*)V, (const e16_t*)dO,
                           L, Dv, dqa, (e16_t*)dK, (e16_t*)dV, s.N, nqb, nkb, (int)nq, (int)nk,
                           scale);
    else
        hipLaunchKernelGGL((bwd_fused_kernel<E, DH, false>), grid, dim3(dqp::NWAVE * 64), 0, st,
                           (const e16_t*)Q, (const e16_t*)K, (const e16_t*)V, (const e16_t*)dO,
                           L, Dv, dqa, (e16_t*)dK, (e16_t*)dV, s.N, nqb, nkb, (int)nq, (int)nk,
                           scale);
    return hipGetLastError();
}

template <typename E>
hipError_t launch_fused_e(const void* Q, const void* K, const void* V, const void* dO,
                          const float* L, const float* Dv, float* dqa, void* dK, void* dV,
                          Shape s, float scale, bool causal, hipStream_t st) {
    return s.d == 64
               ? launch_fused<E, 64>(Q, K, V, dO, L, Dv, dqa, dK, dV, s, scale, causal, st)
               : launch_fused<E, 128>(Q, K, V, dO, L, Dv, dqa, dK, dV, s, scale, causal, st);
}

}  // namespace

hipError_t launch_bwd_fused_mfma(int dtype, const void* Q, const void* K, const void* V,
                                 const void* dO, const float* L, const float* Dv, float* dqa,
                                 void* dK, void* dV, Shape s, float scale, bool causal,
                                 hipStream_t st) {
    if (s.d != 64 && s.d != 128) return hipErrorInvalidValue;
    return dtype == DT_F16
               ? launch_fused_e<F16E>(Q, K, V, dO, L, Dv, dqa, dK, dV, s, scale, causal, st)
               : launch_fused_e<Bf16E>(Q, K, V, dO, L, Dv, dqa, dK, dV, s, scale, causal, st);
}

}  // namespace fa
