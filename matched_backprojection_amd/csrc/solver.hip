// solver.hip -- the normal operator of the pair and CGLS on it, in the caller's layout.
//
// The normal operator A^T A applies mbp_project then mbp_backproject; volumes stay in the
// plan's layout, so a caller that keeps them z-fastest pays no layout copy per application
// ("diffct 2.2.1 -> 2.4.0", CHANGELOG 2.4.0: keeping the native layout saves two whole-volume
// copies per normal-operator application).
//
// CGLS (conjugate gradients on the normal equations A^T A x = A^T y, in the form that keeps
// the residual r = y - A x) minimises ||A x - y|| from a starting volume, one independent
// problem per batch member. Norms accumulate in fp64 blocks ("diffct 2.1.0 -> 2.2.1",
// CHANGELOG 2.2.0) and the step sizes are formed in fp64 on the device, so the whole solve is
// enqueued on one stream without host synchronisation. The solver reports a residual history
// and takes an optional start and a relative residual threshold ("diffct 2.2.1 -> 2.3.0",
// CHANGELOG 2.3.0, "Added"); a member that reaches the threshold is frozen on the device
// (its later steps have length 0) instead of stopping the stream.
//
// Reductions are deterministic: each block sums a fixed strided share of the vector in fp64,
// then one block per member adds the block sums in a fixed tree.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <vector>

#include "../../include/mbp.h"
#include "mbp_internal.h"

namespace {

constexpr int kDotBlocks = 512;     // partial sums per member and reduction
constexpr int kThreads = 256;

// Scalars of one member: slots of a double[kSlots] record.
enum Slot { kGamma = 0, kDelta, kAlpha, kBeta, kY2, kActive, kR2, kSlots = 8 };

__global__ void __launch_bounds__(kThreads) dot_partial_kernel(const float* __restrict__ a,
                                                               const float* __restrict__ b,
                                                               int64_t n, double* __restrict__ partial) {
    __shared__ double sh[kThreads];
    const int64_t m = blockIdx.y;
    const float* am = a + m * n;
    const float* bm = b + m * n;
    double acc = 0.0;
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += (int64_t)gridDim.x * kThreads)
        acc += (double)am[i] * (double)bm[i];
    sh[threadIdx.x] = acc;
    __syncthreads();
    for (int s = kThreads / 2; s > 0; s >>= 1) {
        if ((int)threadIdx.x < s) sh[threadIdx.x] += sh[threadIdx.x + s];
        __syncthreads();
    }
    if (threadIdx.x == 0) partial[m * gridDim.x + blockIdx.x] = sh[0];
}

// Sum of member m's kDotBlocks partials, in a fixed tree (all threads get the result).
__device__ double sum_partials(const double* __restrict__ partial, int m, double* sh) {
    double acc = 0.0;
    for (int i = threadIdx.x; i < kDotBlocks; i += kThreads) acc += partial[m * kDotBlocks + i];
    sh[threadIdx.x] = acc;
    __syncthreads();
    for (int s = kThreads / 2; s > 0; s >>= 1) {
        if ((int)threadIdx.x < s) sh[threadIdx.x] += sh[threadIdx.x + s];
        __syncthreads();
    }
    const double r = sh[0];
    __syncthreads();
    return r;
}

// What a finishing reduction does with its sum.
enum Finish {
    kStoreY2 = 0,     // ||y||^2
    kStart = 1,       // ||r0||^2 (needs kStoreY2 before): history[0], active flag
    kGamma0 = 2,      // ||s0||^2 -> gamma
    kAlphaFromQ = 3,  // ||q||^2 -> delta, alpha = gamma / delta (0 when frozen or delta == 0)
    kResidual = 4,    // ||r||^2 -> history[k + 1]; freezes the member below the threshold
    kBetaFromS = 5    // ||s||^2 -> beta = ||s||^2 / gamma (0 when frozen), gamma = ||s||^2
};

__global__ void __launch_bounds__(kThreads) dot_finish_kernel(const double* __restrict__ partial,
                                                              double* __restrict__ scal,
                                                              double* __restrict__ hist,
                                                              int32_t hist_len, int32_t k,
                                                              int32_t what, double rtol2) {
    __shared__ double sh[kThreads];
    const int m = blockIdx.x;
    const double v = sum_partials(partial, m, sh);
    if (threadIdx.x != 0) return;
    double* S = scal + m * kSlots;
    switch (what) {
        case kStoreY2:
            S[kY2] = v;
            break;
        case kStart:
            S[kR2] = v;
            hist[m * hist_len] = sqrt(v);
            S[kActive] = v > rtol2 * S[kY2] ? 1.0 : 0.0;
            break;
        case kGamma0:
            S[kGamma] = v;
            if (!(v > 0.0)) S[kActive] = 0.0;       // A^T r = 0: already a least-squares point
            break;
        case kAlphaFromQ:
            S[kDelta] = v;
            S[kAlpha] = (S[kActive] != 0.0 && v > 0.0) ? S[kGamma] / v : 0.0;
            break;
        case kResidual:
            if (S[kActive] != 0.0) S[kR2] = v;
            hist[m * hist_len + k + 1] = sqrt(S[kR2]);
            if (!(S[kR2] > rtol2 * S[kY2])) S[kActive] = 0.0;
            break;
        case kBetaFromS:
            if (S[kActive] != 0.0 && S[kGamma] > 0.0) {
                S[kBeta] = v / S[kGamma];
                S[kGamma] = v;
                if (!(v > 0.0)) S[kActive] = 0.0;
            } else {
                S[kBeta] = 0.0;
            }
            break;
    }
}

// out[m] = a[m] - b[m]  (r0 = y - A x0)
__global__ void __launch_bounds__(kThreads) sub_kernel(const float* __restrict__ a, const float* __restrict__ b,
                                                       int64_t n, float* __restrict__ out) {
    const int64_t m = blockIdx.y;
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += (int64_t)gridDim.x * kThreads)
        out[m * n + i] = a[m * n + i] - b[m * n + i];
}

// y[m] += sign * alpha_m * x[m], alpha from the member's scalars (skipped when 0).
__global__ void __launch_bounds__(kThreads) axpy_kernel(const double* __restrict__ scal, float sign,
                                                        const float* __restrict__ x, int64_t n,
                                                        float* __restrict__ y) {
    const int64_t m = blockIdx.y;
    const double alpha = scal[m * kSlots + kAlpha];
    if (alpha == 0.0) return;
    const float a = (float)(sign * alpha);
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += (int64_t)gridDim.x * kThreads)
        y[m * n + i] = fmaf(a, x[m * n + i], y[m * n + i]);
}

// p[m] = s[m] + beta_m * p[m] (beta = 0 copies s).
__global__ void __launch_bounds__(kThreads) direction_kernel(const double* __restrict__ scal,
                                                             const float* __restrict__ s, int64_t n,
                                                             float* __restrict__ p) {
    const int64_t m = blockIdx.y;
    const float beta = (float)scal[m * kSlots + kBeta];
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += (int64_t)gridDim.x * kThreads)
        p[m * n + i] = fmaf(beta, p[m * n + i], s[m * n + i]);
}

__global__ void init_scalars_kernel(double* scal, int32_t batch) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < batch * kSlots) scal[i] = 0.0;
}

dim3 vec_grid(int64_t n, int64_t batch) {
    const int64_t want = (n + kThreads - 1) / kThreads;
    return dim3((unsigned)(want < 2048 ? (want > 0 ? want : 1) : 2048), (unsigned)batch);
}

struct Work {
    float* r;      // [B][rays]
    float* q;      // [B][rays]
    float* s;      // [B][vox]
    float* p;      // [B][vox]
    double* scal;  // [B][kSlots]
    double* hist;  // [B][iters + 1]
    double* part;  // [B][kDotBlocks]
};

size_t align256(size_t b) { return (b + 255) / 256 * 256; }

size_t work_bytes(int64_t rays, int64_t vox, int64_t batch, int32_t iters, Work* w, char* base) {
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t at = off;
        off += align256(bytes);
        return base ? base + at : nullptr;
    };
    char* r = take((size_t)batch * rays * sizeof(float));
    char* q = take((size_t)batch * rays * sizeof(float));
    char* s = take((size_t)batch * vox * sizeof(float));
    char* p = take((size_t)batch * vox * sizeof(float));
    char* sc = take((size_t)batch * kSlots * sizeof(double));
    char* h = take((size_t)batch * (iters + 1) * sizeof(double));
    char* pa = take((size_t)batch * kDotBlocks * sizeof(double));
    if (w) {
        w->r = reinterpret_cast<float*>(r);
        w->q = reinterpret_cast<float*>(q);
        w->s = reinterpret_cast<float*>(s);
        w->p = reinterpret_cast<float*>(p);
        w->scal = reinterpret_cast<double*>(sc);
        w->hist = reinterpret_cast<double*>(h);
        w->part = reinterpret_cast<double*>(pa);
    }
    return off;
}

int hip_err(hipError_t e, const char* what) {
    return mbp::set_error(MBP_EHIP, "%s: %s", what, hipGetErrorString(e));
}

// ||a||^2-style reduction of member vectors a . b of length n, finished as `what`.
int dot(const Work& w, const float* a, const float* b, int64_t n, int64_t batch, int32_t what,
        int32_t k, int32_t hist_len, double rtol2, hipStream_t st) {
    mbp::trace_launch("dot_partial_kernel", dim3(kDotBlocks, (unsigned)batch), dim3(kThreads), 0, "members %lld", (long long)batch);
    dot_partial_kernel<<<dim3(kDotBlocks, (unsigned)batch), dim3(kThreads), 0, st>>>(a, b, n, w.part);
    mbp::trace_launch("dot_finish_kernel", dim3((unsigned)batch), dim3(kThreads), 0, "iteration %d", (int)k);
    dot_finish_kernel<<<dim3((unsigned)batch), dim3(kThreads), 0, st>>>(w.part, w.scal, w.hist, hist_len, k, what, rtol2);
    const hipError_t e = hipGetLastError();
    return e == hipSuccess ? MBP_OK : hip_err(e, "solver reduction launch");
}

int info_of(const mbp_plan* plan, mbp_plan_info* info) {
    return mbp_plan_get_info(plan, info);
}

}  // namespace

extern "C" {

int mbp_normal(mbp_plan* plan, const float* volume, int64_t batch, float* sinogram, float* out,
               void* stream) {
    if (!plan) return mbp::set_error(MBP_EINVAL, "plan is NULL");
    if (batch < 0) return mbp::set_error(MBP_EINVAL, "batch must be >= 0 (got %lld)", (long long)batch);
    if (batch == 0) return MBP_OK;
    if (!volume || !sinogram || !out)
        return mbp::set_error(MBP_EINVAL, "volume, sinogram and out must be non-NULL");
    if (out == volume) return mbp::set_error(MBP_EINVAL, "out must not alias volume");
    int rc = mbp_project(plan, volume, batch, sinogram, stream);
    if (rc != MBP_OK) return rc;
    return mbp_backproject(plan, sinogram, batch, out, 0, stream);
}

int mbp_cgls_workspace_size(const mbp_plan* plan, int64_t batch, int32_t iters, size_t* bytes) {
    if (!plan || !bytes) return mbp::set_error(MBP_EINVAL, "plan and bytes must be non-NULL");
    if (batch < 0) return mbp::set_error(MBP_EINVAL, "batch must be >= 0 (got %lld)", (long long)batch);
    if (iters < 0) return mbp::set_error(MBP_EINVAL, "iters must be >= 0 (got %d)", iters);
    mbp_plan_info info;
    const int rc = info_of(plan, &info);
    if (rc != MBP_OK) return rc;
    *bytes = batch == 0 ? 0 : work_bytes(info.rays, info.voxels, batch, iters, nullptr, nullptr);
    return MBP_OK;
}

int mbp_cgls(mbp_plan* plan, const float* sinogram, int64_t batch, float* volume, int32_t iters,
             double rtol, void* workspace, size_t workspace_bytes, double* residual_norms,
             void* stream) {
    if (!plan) return mbp::set_error(MBP_EINVAL, "plan is NULL");
    if (batch < 0) return mbp::set_error(MBP_EINVAL, "batch must be >= 0 (got %lld)", (long long)batch);
    if (iters < 0) return mbp::set_error(MBP_EINVAL, "iters must be >= 0 (got %d)", iters);
    if (!std::isfinite(rtol) || rtol < 0.0)
        return mbp::set_error(MBP_EINVAL, "rtol must be finite and >= 0");
    if (batch == 0) return MBP_OK;
    if (batch > 65535) return mbp::set_error(MBP_EINVAL, "batch above 65535 members");
    if (!sinogram || !volume || !workspace)
        return mbp::set_error(MBP_EINVAL, "sinogram, volume and workspace must be non-NULL");
    if (reinterpret_cast<uintptr_t>(workspace) & 255u)
        return mbp::set_error(MBP_EINVAL, "workspace must be 256-byte aligned");
    mbp_plan_info info;
    int rc = info_of(plan, &info);
    if (rc != MBP_OK) return rc;
    const int64_t rays = info.rays, vox = info.voxels;
    Work w{};
    const size_t need = work_bytes(rays, vox, batch, iters, &w, static_cast<char*>(workspace));
    if (workspace_bytes < need)
        return mbp::set_error(MBP_ENOMEM, "CGLS workspace of %zu bytes is below the %zu needed", workspace_bytes, need);
    hipStream_t st = static_cast<hipStream_t>(stream);
    const int32_t hl = iters + 1;
    const double rtol2 = rtol * rtol;
    const dim3 gv = vec_grid(vox, batch), gs = vec_grid(rays, batch);

    mbp::trace_launch("init_scalars_kernel", dim3((unsigned)((batch * kSlots + 255) / 256)), dim3(256), 0, "");
    init_scalars_kernel<<<dim3((unsigned)((batch * kSlots + 255) / 256)), dim3(256), 0, st>>>(w.scal, (int32_t)batch);
    // r0 = y - A x0, s0 = A^T r0, p0 = s0
    if ((rc = mbp_project(plan, volume, batch, w.q, stream)) != MBP_OK) return rc;
    mbp::trace_launch("sub_kernel", gs, dim3(kThreads), 0, "");
    sub_kernel<<<gs, dim3(kThreads), 0, st>>>(sinogram, w.q, rays, w.r);
    if ((rc = dot(w, sinogram, sinogram, rays, batch, kStoreY2, 0, hl, rtol2, st)) != MBP_OK) return rc;
    if ((rc = dot(w, w.r, w.r, rays, batch, kStart, 0, hl, rtol2, st)) != MBP_OK) return rc;
    if ((rc = mbp_backproject(plan, w.r, batch, w.s, 0, stream)) != MBP_OK) return rc;
    if ((rc = dot(w, w.s, w.s, vox, batch, kGamma0, 0, hl, rtol2, st)) != MBP_OK) return rc;
    hipError_t e = hipMemcpyAsync(w.p, w.s, (size_t)batch * vox * sizeof(float), hipMemcpyDeviceToDevice, st);
    if (e != hipSuccess) return hip_err(e, "hipMemcpyAsync");
    for (int32_t k = 0; k < iters; ++k) {
        // q = A p; alpha = gamma / ||q||^2; x += alpha p; r -= alpha q
        if ((rc = mbp_project(plan, w.p, batch, w.q, stream)) != MBP_OK) return rc;
        if ((rc = dot(w, w.q, w.q, rays, batch, kAlphaFromQ, k, hl, rtol2, st)) != MBP_OK) return rc;
        mbp::trace_launch("axpy_kernel", gv, dim3(kThreads), 0, "x += alpha p");
        axpy_kernel<<<gv, dim3(kThreads), 0, st>>>(w.scal, 1.0f, w.p, vox, volume);
        mbp::trace_launch("axpy_kernel", gs, dim3(kThreads), 0, "r -= alpha q");
        axpy_kernel<<<gs, dim3(kThreads), 0, st>>>(w.scal, -1.0f, w.q, rays, w.r);
        if ((rc = dot(w, w.r, w.r, rays, batch, kResidual, k, hl, rtol2, st)) != MBP_OK) return rc;
        // s = A^T r; beta = ||s||^2 / gamma; p = s + beta p
        if ((rc = mbp_backproject(plan, w.r, batch, w.s, 0, stream)) != MBP_OK) return rc;
        if ((rc = dot(w, w.s, w.s, vox, batch, kBetaFromS, k, hl, rtol2, st)) != MBP_OK) return rc;
        mbp::trace_launch("direction_kernel", gv, dim3(kThreads), 0, "");
        direction_kernel<<<gv, dim3(kThreads), 0, st>>>(w.scal, w.s, vox, w.p);
        if ((e = hipGetLastError()) != hipSuccess) return hip_err(e, "solver update launch");
    }
    if (residual_norms) {
        e = hipMemcpyAsync(residual_norms, w.hist, (size_t)batch * hl * sizeof(double), hipMemcpyDeviceToHost, st);
        if (e != hipSuccess) return hip_err(e, "hipMemcpyAsync(residual history)");
        e = hipStreamSynchronize(st);
        if (e != hipSuccess) return hip_err(e, "hipStreamSynchronize");
    }
    return MBP_OK;
}

}  // extern "C"
