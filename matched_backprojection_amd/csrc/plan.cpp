// plan.cpp -- host side of the C ABI: validation, plans, frame staging, launch scheduling.
//
// Validation follows the diffct pages' rules where they state them and our reading where they
// only name them: voxel pitch in [1e-6, 1e6] with max/min at most 1e4 ("diffct 2.4.3 ->
// 2.4.4", CHANGELOG 2.4.4); one work array below 2^31 elements (same page, CHANGELOG 2.4.4);
// finite geometry, source and detector that must differ, and "near"/"far" geometry limits
// (test names and messages on "diffct 2.4.1 -> 2.4.2", tests/test_surface_geometry_cudasim.py).
// Every check runs before any device work; a rejected request changes nothing.
//
// Scheduling: per-view frames are staged once per device; a launch covers as many views as
// index and grid limits allow, and backprojection accumulates over all view launches before
// any layout conversion ("diffct 2.1.0 -> 2.2.1", CHANGELOG 2.2.0: accumulators span all
// contributing view batches). The column walk needs a z-fastest volume; callers that hold
// (D, H, W) volumes get one conversion per call into a workspace, with up to four batch
// members interleaved so that one walk serves them all. The workspace obeys the memory rule
// of "diffct 2.4.3 -> 2.4.4", CHANGELOG 2.4.4 (one call uses at most a quarter of the free
// device memory); free memory is only queried when the workspace has to grow.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "../../include/mbp.h"
#include "mbp_internal.h"

using mbp::Box;
using mbp::Frame;

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return code;
}

int hip_fail(hipError_t e, const char* what) {
    return fail(MBP_EHIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr int64_t kMaxElems = (int64_t)1 << 31;   // per-member array limit (exclusive)
constexpr double kPitchMin = 1e-6, kPitchMax = 1e6, kPitchRatio = 1e4;
constexpr double kNear = 1e-6, kFar = 1e15;

struct DeviceState {
    int device = -1;
    Frame* frames = nullptr;
    float* ws = nullptr;              // library-owned workspace
    size_t ws_bytes = 0;
    unsigned long long* counter = nullptr;
    mbp::ColLine* lines = nullptr;    // gather constants per (view, column)
};

bool finite3(const double* p, int n) {
    for (int i = 0; i < n; ++i)
        if (!std::isfinite(p[i])) return false;
    return true;
}

}  // namespace

namespace mbp {
int set_error(int code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return code;
}
}  // namespace mbp

struct mbp_plan {
    mbp_geometry g{};
    int rank = 3;
    Box box{};
    std::vector<Frame> frames;
    bool column_capable = false;
    bool tilt_capable = false;        // cone geometry off the column walk: per-ray gather
    int32_t forced_path = MBP_PATH_AUTO;
    int32_t adjoint_kind = MBP_ADJOINT_AUTO;
    int64_t view_batch = 0;           // 0: automatic
    void* user_ws = nullptr;
    size_t user_ws_bytes = 0;
    std::vector<DeviceState> devs;
    // what the last backprojection ran (reported by mbp_plan_get_info)
    int32_t last_adjoint = MBP_ADJOINT_AUTO;
    int32_t last_walk = MBP_PATH_AUTO;
    int64_t last_views = 0;
    // and what the last forward projection ran
    int32_t last_fwd_walk = MBP_PATH_AUTO;
    int32_t last_fwd_members = 0;
    // turn symmetry of the views (find_orbit) and whether the gather may share items over it
    int32_t orbit = 1;
    int32_t orbit_dir = 0;
    bool orbit_enabled = true;
    int32_t last_orbit = 0;           // cells that shared each item in the last backprojection
    int32_t last_fwd_orbit = 0;       // rays that shared each walk in the last projection
    std::mutex mu;
};

namespace {

int32_t active_path(const mbp_plan* p) {
    if (p->forced_path == MBP_PATH_GENERIC) return MBP_PATH_GENERIC;
    if (p->forced_path == MBP_PATH_COLUMN) return MBP_PATH_COLUMN;
    return p->column_capable ? MBP_PATH_COLUMN : MBP_PATH_GENERIC;
}

int64_t views_per_launch(const mbp_plan* p) {
    const mbp_geometry& g = p->g;
    // 32-bit lane indices of one launch: rows are padded to whole waves in the column walk
    const int64_t per_view = g.cols * ((g.rows + 63) / 64) * 64;
    const int64_t cap = std::max<int64_t>(1, (kMaxElems - 1) / per_view);
    int64_t v = std::min<int64_t>(g.views, cap);
    if (p->view_batch > 0) v = std::min(v, p->view_batch);
    return std::max<int64_t>(v, 1);
}

// Geometry checks of one plan; `frames` already hold the 3-D frames.
int validate_frames(const mbp_plan& P) {
    const mbp_geometry& g = P.g;
    const bool three_d = g.beam == MBP_CONE || g.beam == MBP_PARALLEL3D;
    const bool cone = g.beam == MBP_CONE;
    double minp = std::min(g.spacing[1], g.spacing[2]);
    if (three_d) minp = std::min(minp, g.spacing[0]);
    const double ctr[3] = {g.center[0], g.center[1], three_d ? g.center[2] : 0.0};
    for (int64_t i = 0; i < g.views; ++i) {
        const Frame& F = P.frames[(size_t)i];
        double un = 0, vn = 0, sn = 0;
        for (int a = 0; a < 3; ++a) { un += F.u[a] * F.u[a]; vn += F.v[a] * F.v[a]; sn += F.s[a] * F.s[a]; }
        if (un == 0.0) return fail(MBP_ECOINCIDENT, "view %lld: detector u axis must be nonzero (axes must differ from zero)", (long long)i);
        if (three_d) {
            if (vn == 0.0) return fail(MBP_ECOINCIDENT, "view %lld: detector v axis must be nonzero", (long long)i);
            const double cx = F.u[1] * F.v[2] - F.u[2] * F.v[1];
            const double cy = F.u[2] * F.v[0] - F.u[0] * F.v[2];
            const double cz = F.u[0] * F.v[1] - F.u[1] * F.v[0];
            if (cx == 0.0 && cy == 0.0 && cz == 0.0)
                return fail(MBP_ECOINCIDENT, "view %lld: detector axes must differ in direction", (long long)i);
        }
        for (int a = 0; a < 3; ++a) {
            if (std::fabs(F.c[a] - ctr[a]) > kFar * minp)
                return fail(MBP_ERANGE, "view %lld: detector centre is farther than 1e15 voxel pitches (far geometry)", (long long)i);
        }
        if (g.beam == MBP_PARALLEL || g.beam == MBP_PARALLEL3D) {
            if (sn == 0.0) return fail(MBP_ECOINCIDENT, "view %lld: ray direction must differ from zero", (long long)i);
            continue;
        }
        for (int a = 0; a < 3; ++a) {
            if (std::fabs(F.s[a] - ctr[a]) > kFar * minp)
                return fail(MBP_ERANGE, "view %lld: source is farther than 1e15 voxel pitches (far geometry)", (long long)i);
        }
        // distance of the source to the detector plane (cone) or line (fan), and whether its
        // foot point lies on the pixel array (widened by half a pixel)
        double n[3];
        if (cone) {
            n[0] = F.u[1] * F.v[2] - F.u[2] * F.v[1];
            n[1] = F.u[2] * F.v[0] - F.u[0] * F.v[2];
            n[2] = F.u[0] * F.v[1] - F.u[1] * F.v[0];
        } else {
            n[0] = -F.u[1]; n[1] = F.u[0]; n[2] = 0.0;
        }
        const double nn = std::sqrt(n[0] * n[0] + n[1] * n[1] + n[2] * n[2]);
        double rel[3], dist = 0.0;
        for (int a = 0; a < 3; ++a) rel[a] = F.s[a] - F.c[a];
        for (int a = 0; a < 3; ++a) dist += rel[a] * n[a] / nn;
        dist = std::fabs(dist);
        if (dist < kNear * minp) {
            // detector coordinates of the source's foot point (least squares on u, v)
            double uu = 0, uv = 0, vv = 0, ru = 0, rv = 0;
            for (int a = 0; a < 3; ++a) {
                uu += F.u[a] * F.u[a]; uv += F.u[a] * F.v[a]; vv += F.v[a] * F.v[a];
                ru += rel[a] * F.u[a]; rv += rel[a] * F.v[a];
            }
            double u, v;
            if (cone) {
                const double det = uu * vv - uv * uv;
                u = (ru * vv - rv * uv) / det;
                v = (rv * uu - ru * uv) / det;
            } else {
                u = ru / uu;
                v = 0.0;
            }
            const double hu = 0.5 * (double)g.cols * g.du, hv = 0.5 * (double)g.rows * g.dv;
            if (std::fabs(u) <= hu && (!cone || std::fabs(v) <= hv)) {
                if (dist == 0.0)
                    return fail(MBP_ECOINCIDENT, "view %lld: source and detector pixel must differ", (long long)i);
                return fail(MBP_ERANGE, "view %lld: source lies within 1e-6 voxel pitch of the detector (near geometry; limit 1e6 times closer than a voxel)", (long long)i);
            }
        }
    }
    return MBP_OK;
}

bool column_ok(const mbp_plan& P) {
    const mbp_geometry& g = P.g;
    if (g.beam != MBP_CONE && g.beam != MBP_PARALLEL3D) return false;
    // a z column of up to four interleaved members must fit a 32-bit byte offset
    if (g.D >= ((int64_t)1 << 26)) return false;
    const double minp = std::min(g.spacing[0], std::min(g.spacing[1], g.spacing[2]));
    for (int64_t i = 0; i < g.views; ++i) {
        const Frame& F = P.frames[(size_t)i];
        if (F.v[0] != 0.0 || F.v[1] != 0.0) return false;
        if (g.beam == MBP_PARALLEL3D) {
            // the rays' common xy direction must not vanish against their length
            const double sxy = std::sqrt(F.s[0] * F.s[0] + F.s[1] * F.s[1]);
            const double sn = std::sqrt(sxy * sxy + F.s[2] * F.s[2]);
            if (!(sxy > 1e-6 * sn)) return false;
            continue;
        }
        for (int64_t j = 0; j < g.cols; ++j) {
            const double u = mbp::centred((int32_t)j, (int32_t)g.cols, g.du);
            const double px = F.c[0] + u * F.u[0], py = F.c[1] + u * F.u[1];
            const double dx = px - F.s[0], dy = py - F.s[1];
            if (!(std::sqrt(dx * dx + dy * dy) > kNear * minp)) return false;
        }
    }
    return true;
}

DeviceState* device_state(mbp_plan* p, int* rc) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) { *rc = hip_fail(e, "hipGetDevice"); return nullptr; }
    for (auto& d : p->devs)
        if (d.device == dev) { *rc = MBP_OK; return &d; }
    DeviceState d;
    d.device = dev;
    const size_t bytes = p->frames.size() * sizeof(Frame);
    e = hipMalloc(reinterpret_cast<void**>(&d.frames), bytes);
    if (e != hipSuccess) { *rc = hip_fail(e, "hipMalloc(frames)"); return nullptr; }
    e = hipMemcpy(d.frames, p->frames.data(), bytes, hipMemcpyHostToDevice);
    if (e != hipSuccess) { (void)hipFree(d.frames); *rc = hip_fail(e, "hipMemcpy(frames)"); return nullptr; }
    p->devs.push_back(d);
    *rc = MBP_OK;
    return &p->devs.back();
}

// Ray kind the kernels take: lines for both parallel beams, segments from the source for
// fan and cone.
int32_t kernel_beam(const mbp_geometry& g) {
    if (g.beam == MBP_PARALLEL || g.beam == MBP_PARALLEL3D) return mbp::BEAM_PARALLEL;
    return g.beam == MBP_FAN ? mbp::BEAM_FAN : mbp::BEAM_CONE;
}

mbp::GenericLaunch generic_args(const mbp_plan* p, const DeviceState* d, int32_t whd) {
    const mbp_geometry& g = p->g;
    mbp::GenericLaunch a{};
    a.frames = d->frames;
    a.rows = (int32_t)g.rows;
    a.cols = (int32_t)g.cols;
    a.du = g.du;
    a.dv = g.dv;
    a.beam = kernel_beam(g);
    a.box = p->box;
    const int32_t D = (int32_t)g.D, H = (int32_t)g.H, W = (int32_t)g.W;
    if (whd) { a.sz = 1; a.sy = D; a.sx = D * H; }
    else     { a.sx = 1; a.sy = W; a.sz = W * H; }
    // in a z-fastest volume, rays of neighbouring detector rows read neighbouring voxels
    a.rows_fast = whd && g.rows > 1;
    return a;
}

mbp::ColumnLaunch column_args(const mbp_plan* p, const DeviceState* d) {
    const mbp_geometry& g = p->g;
    mbp::ColumnLaunch a{};
    a.frames = d->frames;
    a.rows = (int32_t)g.rows;
    a.cols = (int32_t)g.cols;
    a.row_blocks = (int32_t)((g.rows + 63) / 64);
    a.beam = kernel_beam(g);
    a.du = g.du;
    a.dv = g.dv;
    a.box = p->box;
    a.H = (int32_t)g.H;
    a.D = (int32_t)g.D;
    return a;
}

// Members one column walk serves (1, 2 or 4), limited by the batch and by 32-bit indexing of
// the interleaved volume.
int interleave_for(const mbp_plan* p, int64_t remaining) {
    const int64_t vox = p->g.D * p->g.H * p->g.W;
    int nb = remaining >= 4 ? 4 : (remaining >= 2 ? 2 : 1);
    while (nb > 1 && (int64_t)nb * vox >= kMaxElems) nb /= 2;
    return nb;
}

// A workspace of at least `least` bytes, as close to `want` as the memory rule allows; its size
// in *got. A caller workspace is used whole when it holds `least` (else MBP_ENOMEM). The
// library's own grows on demand: free device memory is queried only then, and one call uses at
// most a quarter of it ("diffct 2.4.3 -> 2.4.4", CHANGELOG 2.4.4). Returns nullptr with rc
// MBP_OK when not even `least` bytes fit that rule.
float* get_workspace(mbp_plan* p, DeviceState* d, size_t want, size_t least, size_t* got, int* rc) {
    *rc = MBP_OK;
    *got = 0;
    if (p->user_ws) {
        if (p->user_ws_bytes < least) {
            *rc = fail(MBP_ENOMEM, "caller workspace holds %zu bytes, the call needs at least %zu", p->user_ws_bytes, least);
            return nullptr;
        }
        *got = p->user_ws_bytes;
        return static_cast<float*>(p->user_ws);
    }
    if (d->ws_bytes >= want) {
        *got = d->ws_bytes;
        return d->ws;
    }
    size_t free_b = 0, total_b = 0;
    hipError_t e = hipMemGetInfo(&free_b, &total_b);
    if (e != hipSuccess) { *rc = hip_fail(e, "hipMemGetInfo"); return nullptr; }
    const size_t target = std::min(want, (free_b + d->ws_bytes) / 4);
    if (target < least) return nullptr;
    if (d->ws_bytes >= target) {
        *got = d->ws_bytes;
        return d->ws;
    }
    if (d->ws) {
        e = hipDeviceSynchronize();
        if (e != hipSuccess) { *rc = hip_fail(e, "hipDeviceSynchronize"); return nullptr; }
        (void)hipFree(d->ws);
        d->ws = nullptr;
        d->ws_bytes = 0;
    }
    e = hipMalloc(reinterpret_cast<void**>(&d->ws), target);
    if (e != hipSuccess) { *rc = hip_fail(e, "hipMalloc(workspace)"); return nullptr; }
    d->ws_bytes = target;
    *got = target;
    return d->ws;
}

// Adjoint kernel of the column walk: the atomic-free gather unless the scatter is forced.
int32_t adjoint_kind(const mbp_plan* p) {
    return p->adjoint_kind == MBP_ADJOINT_SCATTER ? MBP_ADJOINT_SCATTER : MBP_ADJOINT_GATHER;
}

// Whether the adjoint takes the per-ray gather (cone geometry off the column walk, walk chosen
// automatically, gather adjoint).
bool tilt_gather(const mbp_plan* p) {
    return p->tilt_capable && p->forced_path == MBP_PATH_AUTO && adjoint_kind(p) == MBP_ADJOINT_GATHER;
}

// Turn symmetry of the views about the vertical axis through the grid's xy centre (orbit_cell),
// a property of the geometry that every operator with a shared form takes: 4 when view
// v + V/4 is view v turned a quarter turn for every v (square grid of equal x and y pitch),
// else 2 when view v + V/2 is view v turned a half turn, else 1; the grid's W must be even (no
// cell is its own image). *dir: the quarter turn's sense (+1 anticlockwise seen from +z).
// Turned frames are formed exactly (the turns only swap and negate coordinates relative to the
// axis) and must match the stored ones within 1e-12 of the frame's extent, far below fp32
// rounding, so the shared forms give the sums of the unshared ones to rounding.
int32_t find_orbit(const mbp_plan& P, int32_t* dir) {
    *dir = 0;
    const mbp_geometry& g = P.g;
    if (g.W % 2 != 0) return 1;
    const double ax = 0.5 * (P.box.lo[0] + P.box.hi[0]), ay = 0.5 * (P.box.lo[1] + P.box.hi[1]);
    const bool line = g.beam == MBP_PARALLEL3D || g.beam == MBP_PARALLEL;   // s: a direction
    // whether frame B is frame A turned k quarter turns (k = 1 or -1) or a half turn (k = 2)
    auto turned = [&](const Frame& A, const Frame& B, int k) {
        auto turn = [&](const double* p, bool point, double* out) {
            const double x = point ? p[0] - ax : p[0], y = point ? p[1] - ay : p[1];
            double tx, ty;
            if (k == 2) { tx = -x; ty = -y; }
            else if (k == 1) { tx = -y; ty = x; }
            else { tx = y; ty = -x; }
            out[0] = point ? tx + ax : tx;
            out[1] = point ? ty + ay : ty;
            out[2] = p[2];
        };
        auto close = [](const double* a, const double* b, double scale) {
            double d = 0.0;
            for (int i = 0; i < 3; ++i) d = std::max(d, std::fabs(a[i] - b[i]));
            return d <= 1e-12 * scale;
        };
        auto norm = [&](const double* p, bool point) {
            const double x = point ? p[0] - ax : p[0], y = point ? p[1] - ay : p[1];
            return std::sqrt(x * x + y * y + p[2] * p[2]);
        };
        const double pos = std::max(norm(A.c, true), line ? 0.0 : norm(A.s, true));
        double t[3];
        turn(A.s, !line, t);
        if (!close(t, B.s, line ? norm(A.s, false) : pos)) return false;
        turn(A.c, true, t);
        if (!close(t, B.c, pos)) return false;
        turn(A.u, false, t);
        if (!close(t, B.u, norm(A.u, false))) return false;
        turn(A.v, false, t);
        return close(t, B.v, norm(A.v, false));
    };
    auto all_turned = [&](int64_t q, int k) {
        for (int64_t v = 0; v + q < g.views; ++v)
            if (!turned(P.frames[(size_t)v], P.frames[(size_t)(v + q)], k)) return false;
        return true;
    };
    if (g.views % 4 == 0 && g.W == g.H && g.spacing[1] == g.spacing[2]) {
        for (int k : {1, -1}) {
            if (all_turned(g.views / 4, k)) {
                *dir = k;
                return 4;
            }
        }
    }
    if (g.views % 2 == 0 && all_turned(g.views / 2, 2)) return 2;
    return 1;
}

// Workspace of one column-walk pass over nb members: the interleaved z-fastest volume (not
// needed when the caller's own z-fastest buffer is used directly) and, for the gather adjoint,
// the reordered sinogram of one launch of `views` views.
size_t column_ws_bytes(const mbp_plan* p, int nb, bool direct, bool gather, int64_t views) {
    const mbp_geometry& g = p->g;
    size_t n = 0;
    if (!direct) n += (size_t)nb * (size_t)(g.D * g.H * g.W);
    if (gather) n += (size_t)mbp::gather_sino_floats((int32_t)views, (int32_t)g.cols, (int32_t)g.rows, nb);
    return n * sizeof(float);
}

// Views per gather launch whose reordered sinogram (plus `extra` bytes per view) fits `bytes`
// of workspace next to the volume part (at most vmax; 0 when not even one view fits).
int64_t gather_views_fit(const mbp_plan* p, int nb, bool direct, size_t bytes, int64_t vmax,
                         size_t extra = 0) {
    const size_t fixed = column_ws_bytes(p, nb, direct, true, 0);
    const size_t per_view = column_ws_bytes(p, nb, direct, true, 1) - fixed + extra;
    if (bytes < fixed + per_view) return 0;
    return std::min<int64_t>(vmax, (int64_t)((bytes - fixed) / per_view));
}

int check_call(const mbp_plan* p, const void* a, const void* b, int64_t batch) {
    if (!p) return fail(MBP_EINVAL, "plan is NULL");
    if (batch < 0) return fail(MBP_EINVAL, "batch must be >= 0 (got %lld)", (long long)batch);
    if (batch == 0) return MBP_OK;
    if (!a || !b) return fail(MBP_EINVAL, "volume and sinogram pointers must be non-NULL");
    if ((reinterpret_cast<uintptr_t>(a) & 3u) || (reinterpret_cast<uintptr_t>(b) & 3u))
        return fail(MBP_EINVAL, "volume and sinogram pointers must be 4-byte aligned");
    return MBP_OK;
}

// Run the generic walk over all views for members [m0, m0 + nb) in the caller's layout.
int run_generic(mbp_plan* p, DeviceState* d, bool adjoint, const float* in, float* out,
                int64_t m0, int nb, hipStream_t s) {
    const mbp_geometry& g = p->g;
    const int64_t vox = g.D * g.H * g.W, rays = g.views * g.rows * g.cols;
    mbp::GenericLaunch a = generic_args(p, d, g.layout == MBP_LAYOUT_WHD);
    a.nb = nb;
    const float* src[4] = {nullptr, nullptr, nullptr, nullptr};
    float* dst[4] = {nullptr, nullptr, nullptr, nullptr};
    for (int m = 0; m < nb; ++m) {
        src[m] = in + (m0 + m) * (adjoint ? rays : vox);
        dst[m] = out + (m0 + m) * (adjoint ? vox : rays);
    }
    const int64_t vb = views_per_launch(p);
    // the forward of one member shares each walk over the views' turn symmetry (as run_column)
    const int32_t orbit = !adjoint && nb == 1 && p->orbit_enabled ? p->orbit : 1;
    const int64_t views = g.views / orbit;
    if (!adjoint) p->last_fwd_orbit = p->last_fwd_orbit ? std::min(p->last_fwd_orbit, orbit) : orbit;
    for (int64_t v0 = 0; v0 < views; v0 += vb) {
        a.view0 = (int32_t)v0;
        a.nviews = (int32_t)std::min(vb, views - v0);
        hipError_t e = adjoint ? mbp::launch_generic_adjoint(a, src, dst, s)
                               : mbp::launch_generic_forward(a, src, dst, s, orbit, p->orbit_dir,
                                                             views * g.rows * g.cols);
        if (e != hipSuccess) return hip_fail(e, adjoint ? "generic adjoint launch" : "generic forward launch");
    }
    return MBP_OK;
}

// Column walk over all views for `nb` interleaved members held in `native`.
int run_column(mbp_plan* p, DeviceState* d, bool adjoint, const float* native_in,
               float* native_out, const float* const* sino_in, float* const* sino_out, int nb,
               hipStream_t s) {
    const mbp_geometry& g = p->g;
    mbp::ColumnLaunch a = column_args(p, d);
    const int64_t vb = views_per_launch(p);
    // the forward of one member shares each walk over the views' turn symmetry: launches over
    // the first V / orbit views, each ray also giving the rays of the views V / orbit apart
    const int32_t orbit = !adjoint && nb == 1 && p->orbit_enabled ? p->orbit : 1;
    const int64_t views = g.views / orbit;
    if (!adjoint) p->last_fwd_orbit = p->last_fwd_orbit ? std::min(p->last_fwd_orbit, orbit) : orbit;
    for (int64_t v0 = 0; v0 < views; v0 += vb) {
        a.view0 = (int32_t)v0;
        a.nviews = (int32_t)std::min(vb, views - v0);
        a.tasks = (uint32_t)((int64_t)a.nviews * a.cols * a.row_blocks);
        hipError_t e = adjoint ? mbp::launch_column_adjoint(a, nb, sino_in, native_out, s)
                               : mbp::launch_column_forward(a, nb, native_in, sino_out, s, orbit, p->orbit_dir,
                                                            views * g.rows * g.cols);
        if (e != hipSuccess) return hip_fail(e, adjoint ? "column adjoint launch" : "column forward launch");
    }
    return MBP_OK;
}

}  // namespace

// ------------------------------------------------------------------------------------------
// C ABI

extern "C" {

int mbp_abi_version(void) { return MBP_ABI_VERSION; }

const char* mbp_last_error(void) { return g_last_error.c_str(); }

const char* mbp_status_string(int status) {
    switch (status) {
        case MBP_OK: return "ok";
        case MBP_EINVAL: return "invalid argument";
        case MBP_ENONFINITE: return "geometry must be finite";
        case MBP_ECOINCIDENT: return "source and detector must differ";
        case MBP_ERANGE: return "geometry out of range";
        case MBP_ETOOLARGE: return "array too large (2^31 elements per member)";
        case MBP_EHIP: return "HIP runtime error";
        case MBP_ENOMEM: return "out of memory";
        default: return "unknown status";
    }
}

int mbp_plan_create(const mbp_geometry* geometry, const double* src, const double* det,
                    const double* eu, const double* ev, mbp_plan** out) {
    g_last_error.clear();
    if (!out) return fail(MBP_EINVAL, "out must be non-NULL");
    *out = nullptr;
    if (!geometry) return fail(MBP_EINVAL, "geometry must be non-NULL");
    const mbp_geometry g = *geometry;
    if (g.beam != MBP_PARALLEL && g.beam != MBP_FAN && g.beam != MBP_CONE && g.beam != MBP_PARALLEL3D)
        return fail(MBP_EINVAL, "beam must be MBP_PARALLEL, MBP_FAN, MBP_CONE or MBP_PARALLEL3D (got %d)", g.beam);
    if (g.layout != MBP_LAYOUT_DHW && g.layout != MBP_LAYOUT_WHD)
        return fail(MBP_EINVAL, "layout must be MBP_LAYOUT_DHW or MBP_LAYOUT_WHD (got %d)", g.layout);
    const bool cone = g.beam == MBP_CONE || g.beam == MBP_PARALLEL3D;   // a 3-D beam
    if (!cone && (g.D != 1 || g.rows != 1))
        return fail(MBP_EINVAL, "2-D beams need D == 1 and rows == 1");
    if (!cone && g.layout != MBP_LAYOUT_DHW)
        return fail(MBP_EINVAL, "2-D beams take (H, W) volumes (layout DHW)");
    if (g.D < 1 || g.H < 1 || g.W < 1) return fail(MBP_EINVAL, "volume shape must be positive");
    if (g.views < 1 || g.rows < 1 || g.cols < 1) return fail(MBP_EINVAL, "views, rows and cols must be positive");
    if (!src || !det || !eu || (cone && !ev))
        return fail(MBP_EINVAL, "trajectory arrays src, det, eu%s must be non-NULL", cone ? ", ev" : "");
    const int npitch = cone ? 3 : 2;
    const double* pitch = cone ? g.spacing : g.spacing + 1;
    if (!finite3(pitch, npitch)) return fail(MBP_ENONFINITE, "voxel spacing must be finite");
    if (!finite3(g.center, cone ? 3 : 2)) return fail(MBP_ENONFINITE, "volume centre must be finite");
    if (!std::isfinite(g.du) || (cone && !std::isfinite(g.dv)))
        return fail(MBP_ENONFINITE, "detector pitch must be finite");
    if (!(g.du > 0.0) || (cone && !(g.dv > 0.0))) return fail(MBP_EINVAL, "detector pitch must be positive");
    double pmin = INFINITY, pmax = 0.0;
    for (int i = 0; i < npitch; ++i) {
        if (!(pitch[i] >= kPitchMin && pitch[i] <= kPitchMax))
            return fail(MBP_ERANGE, "voxel spacing %g must lie in [1e-6, 1e6]", pitch[i]);
        pmin = std::min(pmin, pitch[i]);
        pmax = std::max(pmax, pitch[i]);
    }
    if (pmax / pmin > kPitchRatio) return fail(MBP_ERANGE, "voxel spacing max/min ratio %g exceeds 1e4", pmax / pmin);
    if (g.D * g.H >= kMaxElems || g.D * g.H * g.W >= kMaxElems)
        return fail(MBP_ETOOLARGE, "volume has %lld elements; one work array must stay below 2^31", (long long)(g.D * g.H * g.W));
    if (g.views * g.rows >= kMaxElems || g.views * g.rows * g.cols >= kMaxElems)
        return fail(MBP_ETOOLARGE, "sinogram has %lld elements; one work array must stay below 2^31", (long long)(g.views * g.rows * g.cols));
    const int R = cone ? 3 : 2;
    for (int64_t i = 0; i < g.views * R; ++i) {
        if (!std::isfinite(src[i]) || !std::isfinite(det[i]) || !std::isfinite(eu[i]) || (cone && !std::isfinite(ev[i])))
            return fail(MBP_ENONFINITE, "trajectory (view %lld) must be finite", (long long)(i / R));
    }
    mbp_plan* p = new (std::nothrow) mbp_plan();
    if (!p) return fail(MBP_ENOMEM, "plan allocation failed");
    p->g = g;
    p->rank = R;
    try {
        p->frames.resize((size_t)g.views);
    } catch (...) {
        delete p;
        return fail(MBP_ENOMEM, "frame allocation failed");
    }
    const double cz = cone ? g.center[2] : 0.0;
    for (int64_t i = 0; i < g.views; ++i) {
        Frame& F = p->frames[(size_t)i];
        for (int a = 0; a < 3; ++a) {
            if (a < R) {
                F.s[a] = src[i * R + a];
                F.c[a] = det[i * R + a];
                F.u[a] = eu[i * R + a];
                F.v[a] = cone ? ev[i * R + a] : 0.0;
            } else {   // 2-D beams: rays in the plane z = centre z of a one-cell-thick slab
                F.s[a] = g.beam == MBP_PARALLEL ? 0.0 : cz;   // (2-D beams only reach here)
                F.c[a] = cz;
                F.u[a] = 0.0;
                F.v[a] = 0.0;
            }
        }
    }
    const int64_t n[3] = {g.W, g.H, g.D};
    const double pw[3] = {g.spacing[2], g.spacing[1], cone ? g.spacing[0] : 1.0};
    const double c3[3] = {g.center[0], g.center[1], cz};
    for (int a = 0; a < 3; ++a) {
        p->box.n[a] = (int32_t)n[a];
        p->box.pitch[a] = pw[a];
        p->box.lo[a] = c3[a] - 0.5 * (double)n[a] * pw[a];
        p->box.hi[a] = c3[a] + 0.5 * (double)n[a] * pw[a];
    }
    const int rc = validate_frames(*p);
    if (rc != MBP_OK) { delete p; return rc; }
    p->column_capable = column_ok(*p);
    p->tilt_capable = !p->column_capable && g.beam == MBP_CONE && g.D < ((int64_t)1 << 26);
    p->orbit = find_orbit(*p, &p->orbit_dir);
    *out = p;
    return MBP_OK;
}

void mbp_plan_destroy(mbp_plan* plan) {
    if (!plan) return;
    int cur = -1;
    const bool have_cur = hipGetDevice(&cur) == hipSuccess;
    for (auto& d : plan->devs) {
        if (hipSetDevice(d.device) != hipSuccess) continue;
        if (d.frames) (void)hipFree(d.frames);
        if (d.ws) (void)hipFree(d.ws);
        if (d.counter) (void)hipFree(d.counter);
        if (d.lines) (void)hipFree(d.lines);
    }
    if (have_cur && !plan->devs.empty()) (void)hipSetDevice(cur);
    delete plan;
}

int mbp_plan_get_info(const mbp_plan* plan, mbp_plan_info* info) {
    if (!plan || !info) return fail(MBP_EINVAL, "plan and info must be non-NULL");
    const mbp_geometry& g = plan->g;
    info->path = active_path(plan);
    info->column_capable = plan->column_capable ? 1 : 0;
    info->views_per_launch = views_per_launch(plan);
    info->launches = (g.views + info->views_per_launch - 1) / info->views_per_launch;
    info->rays = g.views * g.rows * g.cols;
    info->voxels = g.D * g.H * g.W;
    info->members_per_pass = 1;
    if (info->path == MBP_PATH_COLUMN) info->members_per_pass = interleave_for(plan, 4);
    else info->members_per_pass = 4;
    info->last_adjoint = plan->last_adjoint;
    info->last_adjoint_walk = plan->last_walk;
    info->last_adjoint_views_per_launch = plan->last_views;
    info->last_forward_walk = plan->last_fwd_walk;
    info->last_forward_members_per_pass = plan->last_fwd_members;
    info->orbit = plan->orbit;
    info->last_adjoint_orbit = plan->last_orbit;
    info->last_forward_orbit = plan->last_fwd_orbit;
    return MBP_OK;
}

int mbp_plan_set_path(mbp_plan* plan, int32_t path) {
    if (!plan) return fail(MBP_EINVAL, "plan is NULL");
    if (path != MBP_PATH_AUTO && path != MBP_PATH_GENERIC && path != MBP_PATH_COLUMN)
        return fail(MBP_EINVAL, "unknown path %d", path);
    if (path == MBP_PATH_COLUMN && !plan->column_capable)
        return fail(MBP_EINVAL, "the column walk needs a 3-D beam whose detector row axis is parallel to z");
    plan->forced_path = path;
    return MBP_OK;
}

int mbp_plan_set_orbit(mbp_plan* plan, int32_t enable) {
    if (!plan) return fail(MBP_EINVAL, "plan is NULL");
    if (enable != 0 && enable != 1) return fail(MBP_EINVAL, "enable must be 0 or 1 (got %d)", enable);
    plan->orbit_enabled = enable == 1;
    return MBP_OK;
}

int mbp_plan_set_view_batch(mbp_plan* plan, int64_t views) {
    if (!plan) return fail(MBP_EINVAL, "plan is NULL");
    if (views < 0) return fail(MBP_EINVAL, "views per launch must be >= 0");
    plan->view_batch = views;
    return MBP_OK;
}

int mbp_workspace_size(const mbp_plan* plan, int64_t batch, size_t* bytes) {
    if (!plan || !bytes) return fail(MBP_EINVAL, "plan and bytes must be non-NULL");
    if (batch < 0) return fail(MBP_EINVAL, "batch must be >= 0");
    *bytes = 0;
    const bool tilt = tilt_gather(plan);
    if (batch == 0 || (active_path(plan) != MBP_PATH_COLUMN && !tilt)) return MBP_OK;
    const bool direct = plan->g.layout == MBP_LAYOUT_WHD && batch == 1;
    const int nb = direct ? 1 : interleave_for(plan, batch);
    *bytes = column_ws_bytes(plan, nb, direct, tilt || adjoint_kind(plan) == MBP_ADJOINT_GATHER,
                             views_per_launch(plan));
    return MBP_OK;
}

int mbp_plan_set_adjoint(mbp_plan* plan, int32_t kind) {
    if (!plan) return fail(MBP_EINVAL, "plan is NULL");
    if (kind != MBP_ADJOINT_AUTO && kind != MBP_ADJOINT_GATHER && kind != MBP_ADJOINT_SCATTER)
        return fail(MBP_EINVAL, "unknown adjoint kernel %d", kind);
    plan->adjoint_kind = kind;
    return MBP_OK;
}

int mbp_set_workspace(mbp_plan* plan, void* ptr, size_t bytes) {
    if (!plan) return fail(MBP_EINVAL, "plan is NULL");
    if ((ptr == nullptr) != (bytes == 0)) return fail(MBP_EINVAL, "workspace pointer and size must both be set or both be empty");
    if (reinterpret_cast<uintptr_t>(ptr) & 15u) return fail(MBP_EINVAL, "workspace must be 16-byte aligned");
    plan->user_ws = ptr;
    plan->user_ws_bytes = bytes;
    return MBP_OK;
}

int mbp_project(mbp_plan* plan, const float* volume, int64_t batch, float* sinogram, void* stream) {
    int rc = check_call(plan, volume, sinogram, batch);
    if (rc != MBP_OK || batch == 0) return rc;
    std::lock_guard<std::mutex> lock(plan->mu);
    hipStream_t s = static_cast<hipStream_t>(stream);
    DeviceState* d = device_state(plan, &rc);
    if (!d) return rc;
    const mbp_geometry& g = plan->g;
    const int64_t vox = g.D * g.H * g.W, rays = g.views * g.rows * g.cols;
    int64_t m0 = 0;
    plan->last_fwd_walk = MBP_PATH_GENERIC;
    plan->last_fwd_members = 0;
    plan->last_fwd_orbit = 0;         // the fewest rays any column pass shared a walk over
    if (active_path(plan) == MBP_PATH_COLUMN) {
        const bool whd = g.layout == MBP_LAYOUT_WHD;
        plan->last_fwd_walk = MBP_PATH_COLUMN;
        plan->last_fwd_members = 4;
        while (m0 < batch) {
            if (whd && batch == 1) {
                float* so[4] = {sinogram, nullptr, nullptr, nullptr};
                rc = run_column(plan, d, false, volume, nullptr, nullptr, so, 1, s);
                if (rc != MBP_OK) return rc;
                plan->last_fwd_members = 1;
                m0 = 1;
                break;
            }
            int nb = interleave_for(plan, batch - m0);
            float* ws = nullptr;
            for (;;) {
                const size_t need = column_ws_bytes(plan, nb, false, false, 0);
                size_t got = 0;
                ws = get_workspace(plan, d, need, need, &got, &rc);
                if (rc != MBP_OK) return rc;
                if (ws || nb == 1) break;
                nb /= 2;
            }
            if (!ws) {
                // not even one member's copy fits the memory rule: the generic walk, which
                // reads the caller's layout in place, takes the rest (reported by
                // mbp_plan_get_info)
                plan->last_fwd_walk = MBP_PATH_GENERIC;
                plan->last_fwd_members = 0;
                break;
            }
            plan->last_fwd_members = std::min(plan->last_fwd_members, nb);
            hipError_t e = mbp::launch_to_native(volume + m0 * vox, vox, nb, (int32_t)g.D, (int32_t)g.H,
                                                 (int32_t)g.W, whd ? 1 : 0, ws, s);
            if (e != hipSuccess) return hip_fail(e, "layout conversion launch");
            float* so[4] = {nullptr, nullptr, nullptr, nullptr};
            for (int m = 0; m < nb; ++m) so[m] = sinogram + (m0 + m) * rays;
            rc = run_column(plan, d, false, ws, nullptr, nullptr, so, nb, s);
            if (rc != MBP_OK) return rc;
            m0 += nb;
        }
    }
    while (m0 < batch) {
        const int nb = (int)std::min<int64_t>(4, batch - m0);
        rc = run_generic(plan, d, false, volume, sinogram, m0, nb, s);
        if (rc != MBP_OK) return rc;
        m0 += nb;
    }
    return MBP_OK;
}

}  // extern "C"

namespace {

// A device region that one backprojection takes every buffer from, in place of the plan's own
// (the no-allocation entry point): the reordered sinogram, the interleaved volume and, per
// view batch, the gather's line table.
struct FixedRegion {
    char* ptr;
    size_t bytes;
};

constexpr size_t kRegionAlign = 256;

size_t align_up(size_t n) { return (n + kRegionAlign - 1) / kRegionAlign * kRegionAlign; }

// The backprojection on device state d (frames staged). With `fixed`, the workspace is that
// region, the line table is built per view batch inside it, and nothing is allocated; a call
// whose least need exceeds the region fails with MBP_ETOOLARGE.
int backproject_on(mbp_plan* plan, DeviceState* d, const float* sinogram, int64_t batch, float* volume,
                   int32_t accumulate, hipStream_t s, const FixedRegion* fixed) {
    int rc = MBP_OK;
    const mbp_geometry& g = plan->g;
    const int64_t vox = g.D * g.H * g.W, rays = g.views * g.rows * g.cols;
    int64_t m0 = 0;
    const bool tilt = tilt_gather(plan);
    plan->last_adjoint = MBP_ADJOINT_SCATTER;
    plan->last_walk = MBP_PATH_GENERIC;
    plan->last_views = views_per_launch(plan);
    plan->last_orbit = 1;
    if (active_path(plan) == MBP_PATH_COLUMN || tilt) {
        const bool whd = g.layout == MBP_LAYOUT_WHD;
        const bool direct = whd && batch == 1;
        const bool gather = tilt || adjoint_kind(plan) == MBP_ADJOINT_GATHER;
        const int64_t vmax = views_per_launch(plan);
        // in a fixed region the column gather's line table covers one view batch
        const size_t lines_per_view = fixed && gather && !tilt ? (size_t)g.cols * sizeof(mbp::ColLine) : 0;
        const size_t lines_pad = lines_per_view ? kRegionAlign : 0;
        while (m0 < batch) {
            int nb = direct ? 1 : interleave_for(plan, batch - m0);
            float* ws = nullptr;
            size_t got = 0;
            for (;;) {
                // all views in one gather launch if the memory rule allows, else as many as fit
                const size_t want = column_ws_bytes(plan, nb, direct, gather, vmax) + lines_pad + lines_per_view * vmax;
                const size_t least = column_ws_bytes(plan, nb, direct, gather, 1) + lines_pad + lines_per_view;
                if (fixed) {
                    if (fixed->bytes >= least) {
                        ws = reinterpret_cast<float*>(fixed->ptr);
                        got = fixed->bytes;
                    } else if (nb == 1) {
                        return fail(MBP_ETOOLARGE, "the no-allocation backprojection's scratch holds %zu bytes for this plan; "
                                    "the call needs at least %zu (%s one view's reordered sinogram)", fixed->bytes, least,
                                    direct ? "" : "one member's z-fastest volume and");
                    }
                } else {
                    ws = get_workspace(plan, d, want, least, &got, &rc);
                    if (rc != MBP_OK) return rc;
                }
                if (ws || nb == 1) break;
                nb /= 2;
            }
            if (!ws) break;   // not even one member and one view fit: generic walk for the rest
            const int64_t vb = gather ? gather_views_fit(plan, nb, direct, got - lines_pad, vmax, lines_per_view) : vmax;
            plan->last_adjoint = gather ? MBP_ADJOINT_GATHER : MBP_ADJOINT_SCATTER;
            plan->last_walk = tilt ? MBP_PATH_GENERIC : MBP_PATH_COLUMN;
            plan->last_views = vb;
            float* target = direct ? volume : ws;
            float* ysc = direct ? ws : ws + (size_t)nb * (size_t)vox;
            mbp::ColLine* batch_lines = lines_per_view
                ? reinterpret_cast<mbp::ColLine*>(reinterpret_cast<char*>(ws) +
                                                  align_up(column_ws_bytes(plan, nb, direct, gather, vb)))
                : nullptr;
            const int acc_target = direct ? accumulate : 0;
            hipError_t e;
            if (!gather && !acc_target) {
                e = mbp::launch_fill_zero(target, (int64_t)nb * vox, s);
                if (e != hipSuccess) return hip_fail(e, "zero fill launch");
            }
            const float* si[4] = {nullptr, nullptr, nullptr, nullptr};
            for (int m = 0; m < nb; ++m) si[m] = sinogram + (m0 + m) * rays;
            if (gather && !tilt && !fixed && !d->lines) {
                const size_t bytes = (size_t)g.views * (size_t)g.cols * sizeof(mbp::ColLine);
                e = hipMalloc(reinterpret_cast<void**>(&d->lines), bytes);
                if (e != hipSuccess) { d->lines = nullptr; return hip_fail(e, "hipMalloc(column lines)"); }
                mbp::ColumnLaunch a = column_args(plan, d);
                a.view0 = 0;
                e = mbp::launch_column_lines(a, (int32_t)g.views, d->lines, s);
                if (e != hipSuccess) return hip_fail(e, "column line launch");
            }
            // the turn symmetry's shared items: one member, all views in one launch
            const int32_t orbit = gather && nb == 1 && vb == g.views && plan->orbit_enabled
                                      ? plan->orbit : 1;
            if (orbit > 1) {
                // pre-pass over the first q = V / orbit views with member m the view v + m q;
                // one gather over all views writes every voxel
                mbp::ColumnLaunch a = column_args(plan, d);
                const int64_t q = g.views / orbit;
                a.view0 = 0;
                a.nviews = (int32_t)q;
                const float* so[4] = {nullptr, nullptr, nullptr, nullptr};
                for (int m = 0; m < orbit; ++m) so[m] = si[0] + m * q * g.rows * g.cols;
                e = mbp::launch_sino_prepass(a, orbit, so, ysc, s, (int32_t)q);
                if (e != hipSuccess) return hip_fail(e, "sinogram pre-pass launch");
                a.nviews = (int32_t)g.views;
                const mbp::ColLine* lines = d->lines;
                if (batch_lines) {
                    e = mbp::launch_column_lines(a, (int32_t)q, batch_lines, s);
                    if (e != hipSuccess) return hip_fail(e, "column line launch");
                    lines = batch_lines;
                }
                e = tilt ? mbp::launch_tilt_gather(a, 1, ysc, target, acc_target, s, orbit, plan->orbit_dir)
                         : mbp::launch_column_gather(a, 1, lines, ysc, target, acc_target, s, orbit, plan->orbit_dir);
                if (e != hipSuccess) return hip_fail(e, tilt ? "tilt gather launch" : "column gather launch");
                plan->last_orbit = orbit;
            } else if (gather) {
                // one pre-pass and one gather per view batch; every launch after the first adds
                // into the volume (accumulators span all view batches)
                mbp::ColumnLaunch a = column_args(plan, d);
                for (int64_t v0 = 0; v0 < g.views; v0 += vb) {
                    a.view0 = (int32_t)v0;
                    a.nviews = (int32_t)std::min(vb, g.views - v0);
                    e = mbp::launch_sino_prepass(a, nb, si, ysc, s);
                    if (e != hipSuccess) return hip_fail(e, "sinogram pre-pass launch");
                    const mbp::ColLine* lines = d->lines ? d->lines + (size_t)v0 * (size_t)g.cols : batch_lines;
                    if (batch_lines) {
                        e = mbp::launch_column_lines(a, a.nviews, batch_lines, s);
                        if (e != hipSuccess) return hip_fail(e, "column line launch");
                        lines = batch_lines;
                    }
                    const int acc = v0 == 0 ? acc_target : 1;
                    e = tilt ? mbp::launch_tilt_gather(a, nb, ysc, target, acc, s)
                             : mbp::launch_column_gather(a, nb, lines, ysc, target, acc, s);
                    if (e != hipSuccess) return hip_fail(e, tilt ? "tilt gather launch" : "column gather launch");
                }
            } else {
                rc = run_column(plan, d, true, nullptr, target, si, nullptr, nb, s);
                if (rc != MBP_OK) return rc;
            }
            if (!direct) {
                e = mbp::launch_from_native(ws, nb, (int32_t)g.D, (int32_t)g.H, (int32_t)g.W, whd ? 1 : 0,
                                            volume + m0 * vox, vox, accumulate, s);
                if (e != hipSuccess) return hip_fail(e, "layout conversion launch");
            }
            m0 += nb;
        }
    }
    if (m0 < batch) {
        plan->last_adjoint = MBP_ADJOINT_SCATTER;
        plan->last_walk = MBP_PATH_GENERIC;
        plan->last_views = views_per_launch(plan);
    }
    if (m0 < batch && !accumulate) {
        hipError_t e = mbp::launch_fill_zero(volume + m0 * vox, (batch - m0) * vox, s);
        if (e != hipSuccess) return hip_fail(e, "zero fill launch");
    }
    while (m0 < batch) {
        const int nb = (int)std::min<int64_t>(4, batch - m0);
        rc = run_generic(plan, d, true, sinogram, volume, m0, nb, s);
        if (rc != MBP_OK) return rc;
        m0 += nb;
    }
    return MBP_OK;
}

// Scratch of the no-allocation backprojection: one array per device, resolved to its device
// address once per device (the array's name in host code is only a stand-in for it).
constexpr size_t kScratchBytes = (size_t)128 << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
std::vector<std::pair<int, char*>> g_scratch;   // (device, device address of `scratch`)

char* scratch_on(int dev, int* rc) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    for (const auto& e : g_scratch)
        if (e.first == dev) return e.second;
    void* ptr = nullptr;
    hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) {
        *rc = hip_fail(e != hipSuccess ? e : hipErrorInvalidSymbol, "hipGetSymbolAddress(scratch)");
        return nullptr;
    }
    g_scratch.emplace_back(dev, static_cast<char*>(ptr));
    return static_cast<char*>(ptr);
}

}  // namespace

extern "C" {

int mbp_backproject(mbp_plan* plan, const float* sinogram, int64_t batch, float* volume,
                    int32_t accumulate, void* stream) {
    int rc = check_call(plan, sinogram, volume, batch);
    if (rc != MBP_OK || batch == 0) return rc;
    if (accumulate != 0 && accumulate != 1) return fail(MBP_EINVAL, "accumulate must be 0 or 1");
    std::lock_guard<std::mutex> lock(plan->mu);
    DeviceState* d = device_state(plan, &rc);
    if (!d) return rc;
    return backproject_on(plan, d, sinogram, batch, volume, accumulate, static_cast<hipStream_t>(stream), nullptr);
}

int mbp_backproject_noalloc(mbp_plan* plan, const float* sinogram, int64_t batch, float* volume,
                            int32_t accumulate, void* stream) {
    int rc = check_call(plan, sinogram, volume, batch);
    if (rc != MBP_OK || batch == 0) return rc;
    if (accumulate != 0 && accumulate != 1) return fail(MBP_EINVAL, "accumulate must be 0 or 1");
    const size_t frame_bytes = align_up(plan->frames.size() * sizeof(Frame));
    if (frame_bytes >= kScratchBytes)
        return fail(MBP_ETOOLARGE, "the no-allocation backprojection's scratch (%zu bytes) cannot hold the %zu views' frames",
                    kScratchBytes, plan->frames.size());
    // the least the column and per-row gathers need (one member, one view), checked before
    // any device work
    const bool tilt = tilt_gather(plan);
    if (active_path(plan) == MBP_PATH_COLUMN || tilt) {
        const bool direct = plan->g.layout == MBP_LAYOUT_WHD && batch == 1;
        const bool gather = tilt || adjoint_kind(plan) == MBP_ADJOINT_GATHER;
        const size_t lines = gather && !tilt ? kRegionAlign + (size_t)plan->g.cols * sizeof(mbp::ColLine) : 0;
        const size_t least = frame_bytes + column_ws_bytes(plan, 1, direct, gather, 1) + lines;
        if (least > kScratchBytes)
            return fail(MBP_ETOOLARGE, "the no-allocation backprojection's scratch holds %zu bytes; this call needs at "
                        "least %zu (frames,%s one view's reordered sinogram)", kScratchBytes, least,
                        direct ? "" : " one member's z-fastest volume,");
    }
    std::lock_guard<std::mutex> lock(plan->mu);
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    char* base = scratch_on(dev, &rc);
    if (!base) return rc;
    hipStream_t s = static_cast<hipStream_t>(stream);
    // the frames go to the start of the scratch, the rest is the call's workspace
    e = hipMemcpyAsync(base, plan->frames.data(), plan->frames.size() * sizeof(Frame), hipMemcpyHostToDevice, s);
    if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync(frames)");
    DeviceState d;
    d.device = dev;
    d.frames = reinterpret_cast<Frame*>(base);
    const FixedRegion region{base + frame_bytes, kScratchBytes - frame_bytes};
    return backproject_on(plan, &d, sinogram, batch, volume, accumulate, s, &region);
}

int mbp_segment_count(mbp_plan* plan, int64_t* count, void* stream) {
    if (!plan || !count) return fail(MBP_EINVAL, "plan and count must be non-NULL");
    std::lock_guard<std::mutex> lock(plan->mu);
    int rc = MBP_OK;
    DeviceState* d = device_state(plan, &rc);
    if (!d) return rc;
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e;
    if (!d->counter) {
        e = hipMalloc(reinterpret_cast<void**>(&d->counter), sizeof(unsigned long long));
        if (e != hipSuccess) return hip_fail(e, "hipMalloc(counter)");
    }
    e = hipMemsetAsync(d->counter, 0, sizeof(unsigned long long), s);
    if (e != hipSuccess) return hip_fail(e, "hipMemsetAsync(counter)");
    const int64_t vb = views_per_launch(plan);
    const bool column = active_path(plan) == MBP_PATH_COLUMN;
    mbp::GenericLaunch a = generic_args(plan, d, 0);
    mbp::ColumnLaunch ca = column_args(plan, d);
    for (int64_t v0 = 0; v0 < plan->g.views; v0 += vb) {
        const int32_t nv = (int32_t)std::min(vb, plan->g.views - v0);
        if (column) {
            ca.view0 = (int32_t)v0;
            ca.nviews = nv;
            ca.tasks = (uint32_t)((int64_t)nv * ca.cols * ca.row_blocks);
            e = mbp::launch_column_count(ca, d->counter, s);
        } else {
            a.view0 = (int32_t)v0;
            a.nviews = nv;
            e = mbp::launch_count(a, d->counter, s);
        }
        if (e != hipSuccess) return hip_fail(e, "count launch");
    }
    unsigned long long host = 0;
    e = hipMemcpyAsync(&host, d->counter, sizeof(host), hipMemcpyDeviceToHost, s);
    if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync(counter)");
    e = hipStreamSynchronize(s);
    if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
    *count = (int64_t)host;
    return MBP_OK;
}

int mbp_stream_copy(const float* in, float* out, int64_t n, void* stream) {
    if (n < 0) return fail(MBP_EINVAL, "n must be >= 0");
    if (n == 0) return MBP_OK;
    if (!in || !out) return fail(MBP_EINVAL, "in and out must be non-NULL");
    if ((reinterpret_cast<uintptr_t>(in) & 15u) || (reinterpret_cast<uintptr_t>(out) & 15u))
        return fail(MBP_EINVAL, "in and out must be 16-byte aligned");
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(in), a1 = a0 + (uintptr_t)n * 4;
    const uintptr_t b0 = reinterpret_cast<uintptr_t>(out), b1 = b0 + (uintptr_t)n * 4;
    if (a0 < b1 && b0 < a1) return fail(MBP_EINVAL, "in and out must not overlap");
    hipError_t e = mbp::launch_stream_copy(in, out, n, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "stream copy launch");
    return MBP_OK;
}

int mbp_convert_layout(const float* in, int64_t batch, int64_t D, int64_t H, int64_t W,
                       int32_t to_whd, float* out, void* stream) {
    if (batch < 0) return fail(MBP_EINVAL, "batch must be >= 0");
    if (D < 1 || H < 1 || W < 1) return fail(MBP_EINVAL, "volume shape must be positive");
    if (D * H * W >= kMaxElems) return fail(MBP_ETOOLARGE, "one work array must stay below 2^31 elements");
    if (to_whd != 0 && to_whd != 1) return fail(MBP_EINVAL, "to_whd must be 0 or 1");
    if (batch == 0) return MBP_OK;
    if (!in || !out) return fail(MBP_EINVAL, "in and out must be non-NULL");
    const int64_t vox = D * H * W;
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(in), a1 = a0 + (uintptr_t)(batch * vox * 4);
    const uintptr_t b0 = reinterpret_cast<uintptr_t>(out), b1 = b0 + (uintptr_t)(batch * vox * 4);
    if (a0 < b1 && b0 < a1) return fail(MBP_EINVAL, "in and out must not overlap");
    hipStream_t s = static_cast<hipStream_t>(stream);
    for (int64_t m = 0; m < batch; ++m) {
        hipError_t e = mbp::launch_convert(in + m * vox, (int32_t)D, (int32_t)H, (int32_t)W, to_whd,
                                           out + m * vox, s);
        if (e != hipSuccess) return hip_fail(e, "layout conversion launch");
    }
    return MBP_OK;
}

}  // extern "C"
