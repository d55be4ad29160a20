// api.hip -- the extern "C" entry points declared in include/fa_bwd.h:
// argument validation, then one launcher per call.  No allocation; the only
// global mutable state is the calling thread's last HIP error code, the CU
// count of each device (queried once) and, for fa_bwd_noalloc, the per-device
// address of its static scratch array.
#include <atomic>
#include <mutex>

#include "../../include/fa_bwd.h"
#include "launch.hpp"

// D (one fp32 per row) of fa_bwd_noalloc: a static device array of the
// library, one copy per GPU, held until the process ends.  In host code this
// name stands for the host-side shadow of the array, not a device address:
// kernels get the address hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) float scratch[FA_NOALLOC_MAX_ROWS];

namespace fa {

int resident_per_cu(const void* k, int threads) {
    int per = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, k, threads, 0) != hipSuccess || per < 1)
        return 1;
    return per;
}

int persistent_grid(long long items, int per_cu) {
    constexpr int kDevices = 64;
    static std::atomic<int> cus[kDevices];
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
    int c = dev < kDevices ? cus[dev].load(std::memory_order_relaxed) : 0;
    if (c <= 0) {
        if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            c <= 0)
            return 0;
        if (dev < kDevices) cus[dev].store(c, std::memory_order_relaxed);
    }
    const long long g = (long long)c * (per_cu < 1 ? 1 : per_cu);
    return (int)(items < g ? items : g);
}

}  // namespace fa

namespace {

thread_local int g_last_hip_error = 0;

int hip_status(hipError_t e) {
    if (e == hipSuccess) return FA_OK;
    g_last_hip_error = (int)e;
    return FA_EHIP;
}

bool dims_ok(int B, int H, int N, int d) {
    if (B < 1 || H < 1 || N < 1 || d < 1) return false;
    if (B >= 65536 || H >= 65536) return false;
    // row and tile indices (N plus a few tile sizes) are 32-bit in the kernels
    if (N > (1 << 30)) return false;
    const long long e = (long long)B * H * N * d;
    return e < (1LL << 40);
}

bool dtype_ok(int dtype) {
    return dtype == FA_DTYPE_F32 || dtype == FA_DTYPE_BF16 || dtype == FA_DTYPE_F16;
}

// The matrix-core kernels: 16-bit elements, head dims 64 and 128.
bool matrix_core(int dtype, int d) {
    return (dtype == FA_DTYPE_BF16 || dtype == FA_DTYPE_F16) && (d == 64 || d == 128);
}

bool head_dim_ok(int d) { return d == 16 || d == 32 || d == 64 || d == 128; }

// The softmax scale of the attention calls: finite and positive (the
// matrix-core backward feeds -L / scale into its score products).
bool scale_ok(float scale) { return scale > 0.f && scale <= 3.0e38f; }

// Common checks; returns FA_OK when the call may proceed.
int check(int dtype, int B, int H, int N, int d, std::initializer_list<const void*> ptrs) {
    if (!dtype_ok(dtype) || !dims_ok(B, H, N, d)) return FA_EINVAL;
    for (const void* p : ptrs)
        if (p == nullptr || (reinterpret_cast<uintptr_t>(p) & 15u) != 0) return FA_EINVAL;
    if (!head_dim_ok(d)) return FA_EUNSUPPORTED;
    return FA_OK;
}

// Fails with FA_EHIP when no device is usable, before any launch.
int device_ready() {
    int dev = -1;
    return hip_status(hipGetDevice(&dev));
}

// The two passes of the backward, on the matrix cores where they apply.
hipError_t launch_dkdv(int dtype, const void* Q, const void* K, const void* V, const void* dO,
                       const float* L, const float* D, void* dK, void* dV, fa::Shape s,
                       float scale, bool causal, hipStream_t st) {
    return matrix_core(dtype, s.d)
               ? fa::launch_bwd_dkdv_mfma(dtype, Q, K, V, dO, L, D, dK, dV, s, scale, causal, st)
               : fa::launch_bwd_dkdv_simt(dtype, Q, K, V, dO, L, D, dK, dV, s, scale, causal, st);
}

hipError_t launch_dq(int dtype, const void* Q, const void* K, const void* V, const void* dO,
                     const float* L, const float* D, float* dq_accum, fa::Shape s, float scale,
                     bool causal, hipStream_t st) {
    return matrix_core(dtype, s.d)
               ? fa::launch_bwd_dq_mfma(dtype, Q, K, V, dO, L, D, dq_accum, s, scale, causal, st)
               : fa::launch_bwd_dq_simt(dtype, Q, K, V, dO, L, D, dq_accum, s, scale, causal, st);
}

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
float* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch array, looked up once per
// device (with that device current) and kept.
hipError_t scratch_for_current_device(float** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        g_scratch_ptr[dev] = static_cast<float*>(p);
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

// The dQ pass writing the scaled dQ in the element type (no dq_accum).
hipError_t launch_dq_direct(int dtype, const void* Q, const void* K, const void* V,
                            const void* dO, const float* L, const float* D, void* dQ,
                            fa::Shape s, float scale, bool causal, hipStream_t st) {
    return matrix_core(dtype, s.d)
               ? fa::launch_bwd_dq_mfma_direct(dtype, Q, K, V, dO, L, D, dQ, s, scale, causal, st)
               : fa::launch_bwd_dq_simt_direct(dtype, Q, K, V, dO, L, D, dQ, s, scale, causal, st);
}

}  // namespace

extern "C" {

int fa_fwd_lse(int dtype, const void* Q, const void* K, const void* V, void* O, float* L,
               int B, int H, int N, int d, float scale, int causal, void* stream) {
    int rc = check(dtype, B, H, N, d, {Q, K, V, O, L});
    if (rc != FA_OK) return rc;
    if (!scale_ok(scale)) return FA_EINVAL;
    if ((rc = device_ready()) != FA_OK) return rc;
    const fa::Shape s{B, H, N, d};
    if (matrix_core(dtype, d))
        return hip_status(fa::launch_fwd_mfma(dtype, Q, K, V, O, L, s, scale, causal != 0,
                                              (hipStream_t)stream));
    return hip_status(fa::launch_fwd(dtype, Q, K, V, O, L, s, scale, causal != 0,
                                     (hipStream_t)stream));
}

int fa_lse(int dtype, const void* Q, const void* K, float* L, int B, int H, int N, int d,
           float scale, int causal, void* stream) {
    int rc = check(dtype, B, H, N, d, {Q, K, L});
    if (rc != FA_OK) return rc;
    if (!scale_ok(scale)) return FA_EINVAL;
    if ((rc = device_ready()) != FA_OK) return rc;
    const fa::Shape s{B, H, N, d};
    if (matrix_core(dtype, d))
        return hip_status(fa::launch_lse_mfma(dtype, Q, K, L, s, scale, causal != 0,
                                              (hipStream_t)stream));
    return hip_status(fa::launch_lse(dtype, Q, K, L, s, scale, causal != 0, (hipStream_t)stream));
}

int fa_bwd_preprocess(int dtype, const void* O, const void* dO, float* D, int B, int H, int N,
                      int d, void* stream) {
    int rc = check(dtype, B, H, N, d, {O, dO, D});
    if (rc != FA_OK) return rc;
    if ((rc = device_ready()) != FA_OK) return rc;
    return hip_status(
        fa::launch_preprocess(dtype, O, dO, D, fa::Shape{B, H, N, d}, (hipStream_t)stream));
}

int fa_bwd(int dtype, const void* Q, const void* K, const void* V, const void* dO,
           const float* L, const float* D, float* dq_accum, void* dK, void* dV, int B, int H,
           int N, int d, float scale, int causal, void* stream) {
    int rc = check(dtype, B, H, N, d, {Q, K, V, dO, L, D, dq_accum, dK, dV});
    if (rc != FA_OK) return rc;
    if (!scale_ok(scale)) return FA_EINVAL;
    if ((rc = device_ready()) != FA_OK) return rc;
    const fa::Shape s{B, H, N, d};
    const hipStream_t st = (hipStream_t)stream;
    // the two passes, dQ (query-outer) and dK/dV (key-outer), in one launch
    // whose grid holds the work items of both
    if (matrix_core(dtype, d))
        return hip_status(fa::launch_bwd_fused_mfma(dtype, Q, K, V, dO, L, D, dq_accum, dK, dV, s,
                                                    scale, causal != 0, st));
    return hip_status(fa::launch_bwd_fused_simt(dtype, Q, K, V, dO, L, D, dq_accum, dK, dV, s,
                                                scale, causal != 0, st));
}

int fa_bwd_dkdv(int dtype, const void* Q, const void* K, const void* V, const void* dO,
                const float* L, const float* D, void* dK, void* dV, int B, int H, int N, int d,
                float scale, int causal, void* stream) {
    int rc = check(dtype, B, H, N, d, {Q, K, V, dO, L, D, dK, dV});
    if (rc != FA_OK) return rc;
    if (!scale_ok(scale)) return FA_EINVAL;
    if ((rc = device_ready()) != FA_OK) return rc;
    return hip_status(launch_dkdv(dtype, Q, K, V, dO, L, D, dK, dV, fa::Shape{B, H, N, d}, scale,
                                  causal != 0, (hipStream_t)stream));
}

int fa_bwd_dq(int dtype, const void* Q, const void* K, const void* V, const void* dO,
              const float* L, const float* D, float* dq_accum, int B, int H, int N, int d,
              float scale, int causal, void* stream) {
    int rc = check(dtype, B, H, N, d, {Q, K, V, dO, L, D, dq_accum});
    if (rc != FA_OK) return rc;
    if (!scale_ok(scale)) return FA_EINVAL;
    if ((rc = device_ready()) != FA_OK) return rc;
    return hip_status(launch_dq(dtype, Q, K, V, dO, L, D, dq_accum, fa::Shape{B, H, N, d}, scale,
                                causal != 0, (hipStream_t)stream));
}

int fa_bwd_convert_dq(int dtype, const float* dq_accum, void* dQ, int B, int H, int N, int d,
                      float scale, void* stream) {
    int rc = check(dtype, B, H, N, d, {dq_accum, dQ});
    if (rc != FA_OK) return rc;
    if ((rc = device_ready()) != FA_OK) return rc;
    return hip_status(fa::launch_convert_dq(dtype, dq_accum, dQ, fa::Shape{B, H, N, d}, scale,
                                            (hipStream_t)stream));
}

int fa_bwd_noalloc(int dtype, const void* Q, const void* K, const void* V, const void* O,
                   const void* dO, const float* L, void* dQ, void* dK, void* dV, int B, int H,
                   int N, int d, float scale, int causal, void* stream) {
    int rc = check(dtype, B, H, N, d, {Q, K, V, O, dO, L, dQ, dK, dV});
    if (rc != FA_OK) return rc;
    if (!scale_ok(scale)) return FA_EINVAL;
    if ((long long)B * H * N > FA_NOALLOC_MAX_ROWS) return FA_ESCRATCH;
    if ((rc = device_ready()) != FA_OK) return rc;
    float* Dbuf = nullptr;
    if ((rc = hip_status(scratch_for_current_device(&Dbuf))) != FA_OK) return rc;
    const fa::Shape s{B, H, N, d};
    const hipStream_t st = (hipStream_t)stream;
    // D into the scratch array, then the dQ pass (dQ scaled and cast in its
    // epilogue) and the dK/dV pass, in order on the caller's stream
    if ((rc = hip_status(fa::launch_preprocess(dtype, O, dO, Dbuf, s, st))) != FA_OK) return rc;
    rc = hip_status(launch_dq_direct(dtype, Q, K, V, dO, L, Dbuf, dQ, s, scale, causal != 0, st));
    if (rc != FA_OK) return rc;
    return hip_status(
        launch_dkdv(dtype, Q, K, V, dO, L, Dbuf, dK, dV, s, scale, causal != 0, st));
}

const char* fa_strerror(int status) {
    switch (status) {
        case FA_OK: return "success";
        case FA_EINVAL: return "invalid argument (null or misaligned pointer, bad size or dtype)";
        case FA_EUNSUPPORTED: return "unsupported head dimension (supported: 16, 32, 64, 128)";
        case FA_EHIP: return "HIP runtime error (see fa_last_hip_error)";
        case FA_ESCRATCH:
            return "problem too large for fa_bwd_noalloc (B * H * N above FA_NOALLOC_MAX_ROWS)";
    }
    return "unknown status";
}

int fa_last_hip_error(void) { return g_last_hip_error; }

}  // extern "C"
