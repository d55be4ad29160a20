// api.hip -- the extern "C" entry points declared in include/fa_bwd.h:
// argument validation, then one launcher per call.  No allocation, no global
// mutable state other than the calling thread's last HIP error code.
#include "../../include/fa_bwd.h"
#include "launch.hpp"

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
    // the two passes: dQ (query-outer), then dK/dV (key-outer)
    rc = hip_status(launch_dq(dtype, Q, K, V, dO, L, D, dq_accum, s, scale, causal != 0, st));
    if (rc != FA_OK) return rc;
    return hip_status(launch_dkdv(dtype, Q, K, V, dO, L, D, dK, dV, s, scale, causal != 0, st));
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

const char* fa_strerror(int status) {
    switch (status) {
        case FA_OK: return "success";
        case FA_EINVAL: return "invalid argument (null or misaligned pointer, bad size or dtype)";
        case FA_EUNSUPPORTED: return "unsupported head dimension (supported: 16, 32, 64, 128)";
        case FA_EHIP: return "HIP runtime error (see fa_last_hip_error)";
    }
    return "unknown status";
}

int fa_last_hip_error(void) { return g_last_hip_error; }

}  // extern "C"
