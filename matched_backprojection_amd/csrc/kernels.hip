// kernels.hip -- gfx950 kernels of the ray-driven X-ray transform pair.
//
// Forward (diffct pages, "diffct 2.1.0 -> 2.2.1", README "Why diffct", bullet "Matched
// operators"): each detector pixel's value is the line integral of the cell-constant volume
// along its ray. Adjoint: each ray's value is scattered back along exactly the same segments,
// weighted by length, with global float atomics.
//
// Kernels:
//  * generic_*: one lane per ray, full 3-D walk from an fp64 entry (any flat detector, and
//    2-D beams with a single z cell); lanes of a wave are adjacent detector columns.
//  * column_*: for cone beams whose detector row axis is parallel to z. A wave takes 64
//    adjacent rows of one detector column of one view. Their rays share the xy line, so the
//    xy walk is wave-uniform, and every lane steps its own z crossings inside each xy cell
//    (diffct pages, "diffct 2.2.1 -> 2.4.0", CHANGELOG 2.4.0, "Changed": z crossings of each
//    xy cell stepped in an inner loop, adjacent detector rows grouped in a warp so that the
//    atomic additions hit neighbouring voxels of one column). On a z-fastest volume the 64
//    lanes then load from, or add into, a few consecutive cache lines.
//  * layout conversion between the caller's (D, H, W) order and the z-fastest order with up
//    to four batch members interleaved innermost, so one walk serves four volumes.
//
// Block-to-work mapping is XCD-aware: consecutive block ids are dealt round-robin to the
// eight XCDs, so the mapping hands each XCD one contiguous range of work (neighbouring
// columns of the same view share most voxels, and so each XCD's L2).
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <type_traits>

#include "mbp_internal.h"

namespace mbp {

namespace {

constexpr uint32_t kXcds = 8;

struct Ptrs4 { const float* p[4]; };
struct MPtrs4 { float* p[4]; };

__device__ __forceinline__ uint32_t xcd_remap(uint32_t b, uint32_t n) {
    const uint32_t xcd = b % kXcds, idx = b / kXcds;
    const uint32_t base = n / kXcds, rem = n % kXcds;
    return xcd * base + (xcd < rem ? xcd : rem) + idx;
}

__device__ __forceinline__ void atomic_add_f32(float* p, float v) {
    __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint32_t uniform(uint32_t v) {
    return __builtin_amdgcn_readfirstlane(v);
}

// ------------------------------------------------------------------------------------------
// Generic walk

// Pixel (row k, column j) of thread index `rem` within a view: columns fastest, or rows
// fastest for z-fastest volumes (A.rows_fast); `rem` becomes the pixel's sinogram offset
// k * cols + j.
__device__ __forceinline__ void generic_pixel(const GenericLaunch& A, uint32_t& rem, int32_t& k,
                                              int32_t& j) {
    if (A.rows_fast) {
        j = (int32_t)(rem / (uint32_t)A.rows);
        k = (int32_t)(rem - (uint32_t)j * (uint32_t)A.rows);
        rem = (uint32_t)k * (uint32_t)A.cols + (uint32_t)j;
    } else {
        k = (int32_t)(rem / (uint32_t)A.cols);
        j = (int32_t)(rem - (uint32_t)k * (uint32_t)A.cols);
    }
}

// P > 1 (one member): the walk shared over a turn symmetry of the views (orbit_cell). The
// launch's views are among the first q = V / P; each ray's walk also sums the turned cells
// (walk_ray_orbit) into the rays of the views q m later, stored slot_stride m elements after it.
template <int P>
__global__ void __launch_bounds__(256) generic_forward_kernel(const GenericLaunch A,
                                                              const Ptrs4 vol, const MPtrs4 sino,
                                                              int64_t slot_stride, int32_t dir) {
    const uint32_t per_view = (uint32_t)A.rows * (uint32_t)A.cols;
    uint32_t vl, rem;
    int32_t k, j;
    if (A.rows_fast) {
        // z-fastest volume: a block takes 4 adjacent columns of one 64-row block (wave =
        // column, lane = row), so that its waves cross neighbouring voxel columns at the same
        // heights; views are the fastest block index, then row blocks, then column
        // quadruples, dealt round-robin to the XCDs, as in the column forward (against 256
        // consecutive rows per block: the tilted 256^3 cone's forward 15.4 -> 13.5 ms; with
        // quadruples fastest and a contiguous range per XCD, 14.3)
        const uint32_t blk = blockIdx.x;
        const uint32_t rbs = ((uint32_t)A.rows + 63u) / 64u;
        vl = blk % (uint32_t)A.nviews;
        const uint32_t rest = blk / (uint32_t)A.nviews;
        const uint32_t rb = rest % rbs, cq = rest / rbs;
        j = (int32_t)(cq * 4u + (threadIdx.x >> 6));
        k = (int32_t)(rb * 64u + (threadIdx.x & 63u));
        if (vl >= (uint32_t)A.nviews || j >= A.cols || k >= A.rows) return;
        rem = (uint32_t)k * (uint32_t)A.cols + (uint32_t)j;
    } else {
        const uint32_t rid = blockIdx.x * 256u + threadIdx.x;
        if (rid >= (uint32_t)A.nviews * per_view) return;
        vl = rid / per_view;
        rem = rid - vl * per_view;
        generic_pixel(A, rem, k, j);
    }
    const int32_t view = A.view0 + (int32_t)vl;
    const Frame F = A.frames[view];
    RayWalk r;
    ray_setup(F, A.box, A.beam, centred(j, A.cols, A.du), centred(k, A.rows, A.dv), r);
    float acc0 = 0.0f, acc1 = 0.0f, acc2 = 0.0f, acc3 = 0.0f;
    const int nb = A.nb;
    // the voxel's element offset is kept by the walk (one add per crossing) rather than formed
    // from the cell indices and strides (three 32-bit multiplies per segment): -7% on the
    // tilted 256^3 cone
    const int64_t ray = (int64_t)view * per_view + rem;
    if constexpr (P == 1) {
        auto visit = [&](int32_t idx, float len) {
            acc0 = fmaf(len, vol.p[0][idx], acc0);
            if (nb > 1) acc1 = fmaf(len, vol.p[1][idx], acc1);
            if (nb > 2) acc2 = fmaf(len, vol.p[2][idx], acc2);
            if (nb > 3) acc3 = fmaf(len, vol.p[3][idx], acc3);
        };
        walk_ray_offsets(r, A.sx, A.sy, A.sz, visit);
        sino.p[0][ray] = acc0;
        if (nb > 1) sino.p[1][ray] = acc1;
        if (nb > 2) sino.p[2][ray] = acc2;
        if (nb > 3) sino.p[3][ray] = acc3;
    } else {
        int32_t base[P], tx[P], ty[P];
#pragma unroll
        for (int m = 0; m < P; ++m)
            orbit_strides(P, dir, A.box.n[0], A.box.n[1], A.sx, A.sy, m, base[m], tx[m], ty[m]);
        float acc[P];
#pragma unroll
        for (int m = 0; m < P; ++m) acc[m] = 0.0f;
        auto visit = [&](const int32_t (&idx)[P], float len) {
#pragma unroll
            for (int m = 0; m < P; ++m) acc[m] = fmaf(len, vol.p[0][idx[m]], acc[m]);
        };
        walk_ray_orbit<P>(r, base, tx, ty, A.sz, visit);
#pragma unroll
        for (int m = 0; m < P; ++m) sino.p[0][ray + m * slot_stride] = acc[m];
    }
}

__global__ void __launch_bounds__(256) generic_adjoint_kernel(const GenericLaunch A,
                                                              const Ptrs4 sino, const MPtrs4 vol) {
    const uint32_t per_view = (uint32_t)A.rows * (uint32_t)A.cols;
    const uint32_t rid = blockIdx.x * 256u + threadIdx.x;
    if (rid >= (uint32_t)A.nviews * per_view) return;
    const uint32_t vl = rid / per_view;
    uint32_t rem = rid - vl * per_view;
    int32_t k, j;
    generic_pixel(A, rem, k, j);
    const int32_t view = A.view0 + (int32_t)vl;
    const int64_t ray = (int64_t)view * per_view + rem;
    const int nb = A.nb;
    const float w0 = sino.p[0][ray];
    const float w1 = nb > 1 ? sino.p[1][ray] : 0.0f;
    const float w2 = nb > 2 ? sino.p[2][ray] : 0.0f;
    const float w3 = nb > 3 ? sino.p[3][ray] : 0.0f;
    if (w0 == 0.0f && w1 == 0.0f && w2 == 0.0f && w3 == 0.0f) return;
    const Frame F = A.frames[view];
    RayWalk r;
    ray_setup(F, A.box, A.beam, centred(j, A.cols, A.du), centred(k, A.rows, A.dv), r);
    auto visit = [&](int32_t idx, float len) {
        if (!(len > 0.0f)) return;
        atomic_add_f32(vol.p[0] + idx, len * w0);
        if (nb > 1) atomic_add_f32(vol.p[1] + idx, len * w1);
        if (nb > 2) atomic_add_f32(vol.p[2] + idx, len * w2);
        if (nb > 3) atomic_add_f32(vol.p[3] + idx, len * w3);
    };
    walk_ray_offsets(r, A.sx, A.sy, A.sz, visit);
}

// Segment counts: segments of the generic walk longer than 1e-6 of the smallest voxel pitch
// (shorter ones are the rounding residue of planes crossed at one point), grid-stride over
// rays, one 64-bit atomic per block.
__device__ __forceinline__ float count_eps(const Box& b) {
    return (float)(1e-6 * fmin(b.pitch[0], fmin(b.pitch[1], b.pitch[2])));
}

__device__ __forceinline__ void block_count_add(unsigned long long local, unsigned long long* count) {
    __shared__ unsigned long long part[256];
    part[threadIdx.x] = local;
    __syncthreads();
    for (uint32_t s = 128; s > 0; s >>= 1) {
        if (threadIdx.x < s) part[threadIdx.x] += part[threadIdx.x + s];
        __syncthreads();
    }
    if (threadIdx.x == 0 && part[0]) atomicAdd(count, part[0]);
}

__global__ void __launch_bounds__(256) generic_count_kernel(const GenericLaunch A,
                                                            unsigned long long* count) {
    const uint32_t per_view = (uint32_t)A.rows * (uint32_t)A.cols;
    const uint32_t n = (uint32_t)A.nviews * per_view;
    unsigned long long local = 0;
    for (uint32_t rid = blockIdx.x * 256u + threadIdx.x; rid < n; rid += gridDim.x * 256u) {
        const uint32_t vl = rid / per_view;
        const uint32_t rem = rid - vl * per_view;
        const int32_t k = (int32_t)(rem / (uint32_t)A.cols);
        const int32_t j = (int32_t)(rem - (uint32_t)k * (uint32_t)A.cols);
        const Frame F = A.frames[A.view0 + (int32_t)vl];
        RayWalk r;
        ray_setup(F, A.box, A.beam, centred(j, A.cols, A.du), centred(k, A.rows, A.dv), r);
        uint32_t c = 0;
        const float eps = count_eps(A.box);
        auto visit = [&](int32_t, int32_t, int32_t, float len) { c += len > eps ? 1u : 0u; };
        walk_ray(r, visit);
        local += c;
    }
    block_count_add(local, count);
}

// ------------------------------------------------------------------------------------------
// Column walk

template <int NB> struct VecOf;
template <> struct VecOf<1> { using T = float; };
template <> struct VecOf<2> { using T = float2; };
template <> struct VecOf<4> { using T = float4; };

template <int NB>
__device__ __forceinline__ void load_acc(const float* __restrict__ p, float len, float* acc) {
    if constexpr (NB == 1) {
        acc[0] = fmaf(len, p[0], acc[0]);
    } else if constexpr (NB == 2) {
        const float2 v = *reinterpret_cast<const float2*>(p);
        acc[0] = fmaf(len, v.x, acc[0]);
        acc[1] = fmaf(len, v.y, acc[1]);
    } else {
        const float4 v = *reinterpret_cast<const float4*>(p);
        acc[0] = fmaf(len, v.x, acc[0]);
        acc[1] = fmaf(len, v.y, acc[1]);
        acc[2] = fmaf(len, v.z, acc[2]);
        acc[3] = fmaf(len, v.w, acc[3]);
    }
}

template <int NB>
__device__ __forceinline__ void load_vals(const float* __restrict__ p, float* v) {
    if constexpr (NB == 1) {
        v[0] = p[0];
    } else if constexpr (NB == 2) {
        const float2 t = *reinterpret_cast<const float2*>(p);
        v[0] = t.x; v[1] = t.y;
    } else {
        const float4 t = *reinterpret_cast<const float4*>(p);
        v[0] = t.x; v[1] = t.y; v[2] = t.z; v[3] = t.w;
    }
}

// a * b with 0 * anything = 0 (also 0 * inf): one v_mul_legacy_f32.
__device__ __forceinline__ float mul_legacy(float a, float b) {
    float r;
    asm("v_mul_legacy_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
    return r;
}

// Third dword of a raw buffer resource (32-bit elements, unformatted access).
constexpr int kBufferFlags = 0x00020000;

template <int NB>
__device__ __forceinline__ void buffer_vals(__amdgpu_buffer_rsrc_t r, uint32_t off, float* v,
                                            uint32_t soff = 0) {
    if constexpr (NB == 1) {
        v[0] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, (int)off, (int)soff, 0));
    } else if constexpr (NB == 2) {
        const auto t = __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, (int)soff, 0);
        v[0] = __uint_as_float(t[0]); v[1] = __uint_as_float(t[1]);
    } else {
        const auto t = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, (int)soff, 0);
        v[0] = __uint_as_float(t[0]); v[1] = __uint_as_float(t[1]);
        v[2] = __uint_as_float(t[2]); v[3] = __uint_as_float(t[3]);
    }
}

struct ColumnTask {
    int32_t view, col, row;
    bool valid;
    bool live;
};

__device__ __forceinline__ ColumnTask column_task(const ColumnLaunch& A) {
    ColumnTask t;
    const uint32_t wave = uniform(threadIdx.x >> 6);
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t blk = uniform(xcd_remap(blockIdx.x, gridDim.x));
    const uint32_t task = blk * 4u + wave;
    t.live = task < A.tasks;
    const uint32_t rb = task % (uint32_t)A.row_blocks;
    const uint32_t vc = task / (uint32_t)A.row_blocks;
    t.col = (int32_t)(vc % (uint32_t)A.cols);
    t.view = A.view0 + (int32_t)(vc / (uint32_t)A.cols);
    t.row = (int32_t)(rb * 64u + lane);
    t.valid = t.live && t.row < A.rows;
    return t;
}

// The forward's waves: a block takes 4 adjacent detector columns of one 64-row block and view
// (one wave per column), so the waves on one compute unit cross the same voxel columns at the
// same heights and share their cache lines (against 4 row blocks of one column: c3 -5%, the
// 360-view 512^3 cone -3%). The views are taken in groups of kForwardViewGroup (the last
// group holding the rest); inside a group the views are the fastest block index, then row
// blocks, then column quadruples, and the blocks are dealt round-robin to the XCDs as the
// hardware deals them. The blocks running at one time on all XCDs then take a few column
// quadruples over the group's consecutive views, which cross the same voxels from nearby
// angles (and, on a helix, at nearby heights), so the XCDs share those voxels' lines in the
// memory-side cache. Measured (the 720-view 512^3 cone, c3, the 360-view 512^3 cone, the
// helical batch, ms): row blocks fastest, then quadruples, then views, each XCD a contiguous
// range 71.3 / 6.22 / 50.9 / 46.5; all views fastest, round-robin 65.5 / 5.95 / 50.5 / 43.8;
// groups of 16 views 65.6 / 5.96 / 47.6 / 32.0 (kept, with the XCD pairing of view_group_block:
// 65.0 / 5.92 / 47.3 / 30.8); the same with quadruples before row
// blocks 65.3 / 6.26 / 52.5 / 32.1; groups of 8 views 65.3 / 6.17 / 53.8 / 33.4; of 32 views
// 66.0 / 6.34 / 53.0 / 33.6 (both with quadruples before row blocks).
constexpr uint32_t kForwardViewGroup = 16;

// Block blk's (view, row block, column quadruple) in that order: groups of kForwardViewGroup
// views (the last group holding the rest), inside a group views fastest, then row blocks,
// then quadruples. A bijection of [0, nv * rbs * quads).
static_assert(kForwardViewGroup == 16, "the view pairing below deals 16 views to 8 XCDs");
__device__ __forceinline__ void view_group_block(uint32_t blk, uint32_t nv, uint32_t rbs, uint32_t quads,
                                                 uint32_t& vl, uint32_t& rb, uint32_t& cq) {
    const uint32_t per_view = quads * rbs;                            // blocks per view
    const uint32_t nfull = nv / kForwardViewGroup, full = nfull * kForwardViewGroup * per_view;
    const uint32_t grp = blk < full ? blk / (kForwardViewGroup * per_view) : nfull;
    const uint32_t r = blk < full ? blk % (kForwardViewGroup * per_view) : blk - full;
    const uint32_t gs = blk < full ? kForwardViewGroup : nv - nfull * kForwardViewGroup;
    // in a full group, block r mod 8 runs on XCD r mod 8 (the hardware deals blocks
    // round-robin to the 8 XCDs and a group starts at a multiple of 8): XCD x takes the
    // adjacent views 2x and 2x + 1, which share more of their lines in its L2 (against views
    // x and x + 8: the 720-view 512^3 cone 65.4 -> 65.0 ms, c3 5.97 -> 5.92, the 360-view
    // 512^3 cone 48.0 -> 47.3, the helical batch 31.9 -> 30.8)
    uint32_t g = r % gs;
    if (gs == kForwardViewGroup) g = (g % 8u) * 2u + g / 8u;
    vl = grp * kForwardViewGroup + g;
    const uint32_t rest = r / gs;
    rb = rest % rbs;
    cq = rest / rbs;
}
__device__ __forceinline__ ColumnTask forward_task(const ColumnLaunch& A) {
    ColumnTask t;
    const uint32_t wave = uniform(threadIdx.x >> 6);
    const uint32_t lane = threadIdx.x & 63u;
    uint32_t vl, rb, cq;
    view_group_block(blockIdx.x, (uint32_t)A.nviews, (uint32_t)A.row_blocks,
                     ((uint32_t)A.cols + 3u) / 4u, vl, rb, cq);
    t.col = (int32_t)(cq * 4u + wave);
    t.view = A.view0 + (int32_t)vl;
    t.row = (int32_t)(rb * 64u + lane);
    t.live = vl < (uint32_t)A.nviews && t.col < A.cols;
    t.valid = t.live && t.row < A.rows;
    return t;
}

// Sum over the wave of a lane value in {0, 1, 2}.
__device__ __forceinline__ int32_t wave_sum012(int32_t v) {
    return (int32_t)(__popcll(__ballot(v & 1)) + 2 * __popcll(__ballot((v >> 1) & 1)));
}

// Makes one lane's LDS writes visible to the other lanes of its wave (and keeps the compiler
// from moving LDS accesses across this point).
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

typedef __attribute__((address_space(3))) XYEvent lds_event;

// The LDS address of a wave's run of events (a uniform address), copied once into a vector
// register: the reads of a group of cells then take it with immediate offsets, where the
// compiler would otherwise copy the scalar address into a vector register before each read.
__device__ __forceinline__ const lds_event* events_in_vgpr(const XYEvent* e) {
    const int32_t a = (int32_t)(uintptr_t)(const lds_event*)e;
    int32_t r;
    asm volatile("v_mov_b32 %0, %1" : "=v"(r) : "s"(a));
    return (const lds_event*)(uintptr_t)(uint32_t)r;
}

// FLAT: the volume's bytes fit a 31-bit offset, so one buffer resource spans it and each
// cell's column is reached through the load's scalar offset (one scalar multiply per cell);
// otherwise each cell gets a resource based at its column.
//
// P > 1 (one member): the projection shared over a turn symmetry of the views (orbit_cell).
// The launch's views are among the first q = V / P; a ray (v, column, row) crosses the cells
// R^m C with the chords it has through C, and so gives ray (v + m q, column, row), which is
// stored slot_stride elements after it: one walk serves P rays, each summing its own cells.
template <int NB, bool FLAT, int P>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(NB == 1 && P == 1 ? 8 : P == 1 ? 1 : 4)))
column_forward_kernel(const ColumnLaunch A, const float* __restrict__ vol, const MPtrs4 sino,
                      int64_t slot_stride, int32_t dir) {
    static_assert(P == 1 || NB == 1, "a turn symmetry is taken for one member");
    constexpr int NA = NB * P;          // sums per lane: the members, or the orbit's rays
    __shared__ XYEvent events[4][kXYChunk];
    __shared__ int32_t turned[P == 4 ? 4 : 1][P == 4 ? kXYChunk : 1];
    const ColumnTask t = forward_task(A);
    if (!t.live) return;
    const uint32_t wave = uniform(threadIdx.x >> 6);
    const int32_t lane = (int32_t)(threadIdx.x & 63u);
    XYEvent* E = events[wave];
    int32_t* const C1 = P == 4 ? turned[wave] : nullptr;
    const uint32_t WH1 = (uint32_t)A.box.n[0] * (uint32_t)A.H - 1u;
    // the wave's first ray (uniform, held in scalar registers through the walk); a lane's ray
    // adds its row
    const int64_t ray0 = ((int64_t)t.view * A.rows + (t.row - lane)) * A.cols + t.col;
    const uint32_t ray_lo = uniform((uint32_t)ray0), ray_hi = uniform((uint32_t)((uint64_t)ray0 >> 32));
    const Frame F = A.frames[t.view];
    ColumnWalk c;
    column_setup(F, A.box, A.beam, centred(t.col, A.cols, A.du), c);
    RowWalk r;
    row_setup(c, A.box, centred(t.row, A.rows, A.dv), F.v[2], r);
    if (!t.valid) { r.t_lo = 0.0; r.t_hi = 0.0; }
    float acc[NA];
#pragma unroll
    for (int m = 0; m < NA; ++m) acc[m] = 0.0f;
    if (c.hit) {
        const uint32_t D = (uint32_t)A.D;
        uint32_t c1 = 0;        // quarter turn: the turned column of the cell visited next
        auto visit = [&](int32_t cxy, int32_t cz, float len) {
            if constexpr (P == 1) {
                load_acc<NB>(vol + ((uint32_t)cxy * D + (uint32_t)cz) * NB, len, acc);
            } else {
                uint32_t cell[P];
                orbit_columns<P>((uint32_t)cxy, c1, WH1, cell);
#pragma unroll
                for (int m = 0; m < P; ++m) load_acc<1>(vol + (cell[m] * D + (uint32_t)cz), len, acc + m);
            }
        };
        int32_t cz = r.z.c0, kz = 0;
        double nz = r.z.steps > 0 ? r.z.t_first : INFINITY;
        const int32_t total = c.x.steps + c.y.steps;
        int32_t done = 0, kx0 = 0, ky0 = 0;
        double ta = 0.0;
        // when every lane meets at most one z plane per xy cell, cells are handled in fixed
        // groups with all their loads issued before the sums
        const bool two_pieces = __all(row_single_crossing(r, A.box));
        for (;;) {
            const int32_t count = total - done < kXYChunk ? total - done : kXYChunk;
            int32_t a = 0;
            if (count > 0) {
                a = wave_sum012(xy_chunk_fill(c, A.H, kx0, ky0, count, lane, E, C1, A.box.n[0], dir));
                wave_lds_sync();
            }
            int32_t p = 0;
            if (two_pieces) {
                // groups of kCellGroup cells: every lane's pieces (at most two per cell: before and
                // after its single z crossing) first, then all their loads, then the sums. When
                // the chunk lies inside every lane's slab, the pieces need no clip.
                const double t_end = count > 0 ? E[count - 1].tb : ta;
                const bool inside = __all(r.t_lo <= ta && r.t_hi >= t_end &&
                                          stepped_walk_ok(r, kz, count, t_end));
                auto groups = [&](auto pieces) {
                    for (; p + kCellGroup <= count; p += kCellGroup) {
                        uint32_t off[2 * kCellGroup];
                        float len[2 * kCellGroup];
                        uint32_t cell[kCellGroup][P];
#pragma unroll
                        for (int q = 0; q < kCellGroup; ++q) {
                            const double tb = E[p + q].tb;
                            orbit_columns<P>(uniform((uint32_t)E[p + q].cxy),
                                             P == 4 ? uniform((uint32_t)C1[p + q]) : 0u, WH1, cell[q]);
                            int32_t z0, z1;
                            pieces(tb, z0, len[2 * q], z1, len[2 * q + 1]);
                            off[2 * q] = (uint32_t)z0 * NB;
                            off[2 * q + 1] = (uint32_t)z1 * NB;
                            ta = tb;
                        }
                        float val[2 * kCellGroup][NA];
#pragma unroll
                        for (int q = 0; q < 2 * kCellGroup; ++q) {
#pragma unroll
                            for (int m = 0; m < P; ++m) {
                                if (len[q] != 0.0f) {
                                    load_vals<NB>(vol + cell[q / 2][m] * D * NB + off[q], val[q] + m * NB);
                                } else {
#pragma unroll
                                    for (int b = 0; b < NB; ++b) val[q][m * NB + b] = 0.0f;
                                }
                            }
                        }
#pragma unroll
                        for (int q = 0; q < 2 * kCellGroup; ++q)
#pragma unroll
                            for (int m = 0; m < NA; ++m) acc[m] = fmaf(len[q], val[q][m], acc[m]);
                    }
                };
                if (inside) {
                    // the clip-free counted form: the cells' chords computed once for all
                    // rows, then per cell the crossing count, the next crossing and the z
                    // offsets (in bytes) without branches. Voxels are read through a buffer
                    // resource (per cell, based at the cell's z column, unless the volume fits
                    // one 31-bit resource), so each load takes a 32-bit offset.
                    // a row with no crossing left keeps nz = +inf (crossing() is not asked for
                    // its planes again)
                    if (kz >= r.z.steps) { r.z.t_first = INFINITY; r.z.t_step = 0.0; }
                    nz = crossing(r.z, kz);
                    xy_chunk_chords(E, count, ta, lane);
                    wave_lds_sync();
                    const int32_t colbytes = (int32_t)(D * NB * sizeof(float));
                    const __amdgpu_buffer_rsrc_t rs_all = __builtin_amdgcn_make_buffer_rsrc(
                        const_cast<float*>(vol), (short)0, 0x7FFFFFFF, kBufferFlags);
                    const int32_t zbytes = NB * sizeof(float);
                    const int32_t zstep = r.z.step * zbytes;
                    const int32_t zbase = r.z.c0 * zbytes;
                    int32_t k = kz;
                    for (; p + kCellGroup <= count; p += kCellGroup) {
                        uint32_t zoff[2 * kCellGroup];
                        float len[2 * kCellGroup];
                        uint32_t cell[kCellGroup][P];
                        bool cross[kCellGroup];
                        const lds_event* const Eg = events_in_vgpr(E + p);
#pragma unroll
                        for (int q = 0; q < kCellGroup; ++q) {
                            orbit_columns<P>(uniform((uint32_t)Eg[q].cxy),
                                             P == 4 ? uniform((uint32_t)C1[p + q]) : 0u, WH1, cell[q]);
                            zoff[2 * q] = (uint32_t)(zbase + __mul24(k, zstep));
                            cross[q] = row_cell_two_counted(r.z.t_first, r.z.t_step, Eg[q].tb, Eg[q].chord, k, nz,
                                                 len[2 * q], len[2 * q + 1]);
                            zoff[2 * q + 1] = (uint32_t)(zbase + __mul24(k, zstep));
                        }
                        float val[2 * kCellGroup][NA];
#pragma unroll
                        for (int q = 0; q < kCellGroup; ++q) {
#pragma unroll
                            for (int o = 0; o < P; ++o) {
                                const __amdgpu_buffer_rsrc_t rs = FLAT ? rs_all
                                    : __builtin_amdgcn_make_buffer_rsrc(
                                          const_cast<float*>(vol + (size_t)cell[q][o] * D * NB), (short)0,
                                          colbytes, kBufferFlags);
                                const uint32_t soff = FLAT ? cell[q][o] * (uint32_t)colbytes : 0u;
#pragma unroll
                                for (int h = 0; h < 2; ++h) {
                                    // one member: the first piece (empty only when the row meets
                                    // a z plane exactly at the cell's entry) is loaded
                                    // unconditionally and multiplied with 0 * anything = 0, so an
                                    // empty piece adds nothing even next to a non-finite voxel;
                                    // the second piece is loaded by the lanes that cross a z plane
                                    // in the cell (its length tb - nz > 0 then rounds to a nonzero
                                    // fp32 unless it is below 2^-150), the others add 0
                                    if (NB == 1 ? (h == 0 || cross[q]) : len[2 * q + h] != 0.0f) {
                                        buffer_vals<NB>(rs, zoff[2 * q + h], val[2 * q + h] + o * NB, soff);
                                    } else {
#pragma unroll
                                        for (int m = 0; m < NB; ++m) val[2 * q + h][o * NB + m] = 0.0f;
                                    }
                                }
                            }
                        }
#pragma unroll
                        for (int q = 0; q < 2 * kCellGroup; ++q) {
                            if constexpr (NB == 1) {
#pragma unroll
                                for (int o = 0; o < P; ++o) {
                                    if (q % 2 == 0)
                                        acc[o] += mul_legacy(len[q], val[q][o]);
                                    else
                                        acc[o] = fmaf(len[q], val[q][o], acc[o]);
                                }
                            } else {
#pragma unroll
                                for (int m = 0; m < NB; ++m) acc[m] = fmaf(len[q], val[q][m], acc[m]);
                            }
                        }
                    }
                    // the state the remaining cells continue from
                    if (p > 0) ta = E[p - 1].tb;
                    cz = r.z.c0 + r.z.step * k;
                    kz = k;
                    nz = kz < r.z.steps ? crossing(r.z, kz) : INFINITY;
                } else {
                    groups([&](double tb, int32_t& z0, float& l0, int32_t& z1, float& l1) {
                        row_cell_two(r, ta, tb, cz, kz, nz, z0, l0, z1, l1);
                    });
                }
            }
            for (; p < count; ++p) {
                const double tb = E[p].tb;
                if constexpr (P == 4) c1 = (uint32_t)C1[p];
                row_cell(r, ta, tb, E[p].cxy, cz, kz, nz, visit);
                ta = tb;
            }
            kx0 += a;
            ky0 += count - a;
            done += count;
            if (done >= total) {
                const int32_t ix = c.x.c0 + c.x.step * c.x.steps, iy = c.y.c0 + c.y.step * c.y.steps;
                if constexpr (P == 4) {
                    int32_t ox, oy;
                    orbit_cell(4, dir, A.box.n[0], A.H, ix, iy, 1, ox, oy);
                    c1 = (uint32_t)(ox * A.H + oy);
                }
                row_cell(r, ta, c.T, ix * A.H + iy, cz, kz, nz, visit);
                break;
            }
            wave_lds_sync();
        }
    }
    if (t.valid) {
        const int64_t ray = (int64_t)(((uint64_t)ray_hi << 32) | ray_lo) + (int64_t)lane * A.cols;
        if constexpr (P == 1) {
#pragma unroll
            for (int m = 0; m < NB; ++m) sino.p[m][ray] = acc[m] * r.kappa;
        } else {
#pragma unroll
            for (int m = 0; m < P; ++m) sino.p[0][ray + m * slot_stride] = acc[m] * r.kappa;
        }
    }
}

template <int NB>
__global__ void __launch_bounds__(256) column_adjoint_kernel(const ColumnLaunch A,
                                                             const Ptrs4 sino,
                                                             float* __restrict__ vol) {
    const ColumnTask t = column_task(A);
    if (!t.live) return;
    const Frame F = A.frames[t.view];
    ColumnWalk c;
    column_setup(F, A.box, A.beam, centred(t.col, A.cols, A.du), c);
    RowWalk r;
    row_setup(c, A.box, centred(t.row, A.rows, A.dv), F.v[2], r);
    float w[NB];
    bool any = false;
    const int64_t ray = ((int64_t)t.view * A.rows + t.row) * A.cols + t.col;
#pragma unroll
    for (int m = 0; m < NB; ++m) {
        w[m] = t.valid ? sino.p[m][ray] * r.kappa : 0.0f;
        any = any || w[m] != 0.0f;
    }
    if (!any) { r.t_lo = 0.0f; r.t_hi = 0.0f; }
    const uint32_t H = (uint32_t)A.H, D = (uint32_t)A.D;
    auto visit = [&](int32_t cx, int32_t cy, int32_t cz, float len) {
        const uint32_t base = (((uint32_t)cx * H + (uint32_t)cy) * D + (uint32_t)cz) * NB;
#pragma unroll
        for (int m = 0; m < NB; ++m) atomic_add_f32(vol + base + m, len * w[m]);
    };
    walk_column_row(c, r, visit);
}

__global__ void __launch_bounds__(256) column_count_kernel(const ColumnLaunch A,
                                                           unsigned long long* count) {
    const ColumnTask t = column_task(A);
    uint32_t c = 0;
    if (t.live) {
        const Frame F = A.frames[t.view];
        ColumnWalk cw;
        column_setup(F, A.box, A.beam, centred(t.col, A.cols, A.du), cw);
        RowWalk r;
        row_setup(cw, A.box, centred(t.row, A.rows, A.dv), F.v[2], r);
        if (!t.valid) { r.t_lo = 0.0f; r.t_hi = 0.0f; }
        const float eps = count_eps(A.box);
        auto visit = [&](int32_t, int32_t, int32_t, float len) { c += len > eps ? 1u : 0u; };
        walk_column_row(cw, r, visit);
    }
    block_count_add(c, count);
}

// ------------------------------------------------------------------------------------------
// Column gather: the matched adjoint without global atomics.
//
// The adjoint value of voxel v is the sum over rays of len(ray, v) * y[ray]. For the column
// geometry the rays of detector column j (all rows) share one line in the xy plane, and a ray
// parameter alpha (0 at the source, 1 at the pixel) is the same for all of them at a given xy
// point. So for one xy cell and one view:
//  * the columns whose xy line crosses the cell are the pixels whose centre lies inside the
//    detector interval that the cell's four corners project to;
//  * for such a column the xy cell is crossed for alpha in [a0, a1] (fp64 slab clip), by
//    every row alike;
//  * along that piece row k's z runs linearly from z_k(a0) to z_k(a1); the part inside z cell
//    iz has length (a1 - a0) * |d_k| * (z overlap / z extent), which is exactly the chord of
//    the ray through the voxel.
// A wave owns one xy cell (all of its z cells, held in LDS) and loops over every view, every
// crossing column and all rows (lanes = 64 adjacent rows), adding each piece into LDS; the
// column is written once at the end. The sinogram is read through a pre-pass copy in
// [view][col][row] order (rows contiguous, so a wave's 64 lanes load 256 contiguous bytes),
// already multiplied by |d_k|, the ray's length per unit of alpha.

// mview: views between consecutive members (0: the members are volumes of a batch and share
// the view; q: member m is view view + m q of one sinogram, for the gather shared over a turn
// symmetry), which also fixes each member's ray lengths.
template <int NB>
__global__ void __launch_bounds__(256) sino_prepass_kernel(const ColumnLaunch A, const Ptrs4 sino,
                                                           int32_t rows_pad, int32_t mview,
                                                           float* __restrict__ ysc) {
    __shared__ float tile[NB][32][33];
    const int32_t j0 = blockIdx.x * 32, k0 = blockIdx.y * 32;
    const int32_t view = A.view0 + (int32_t)blockIdx.z;
    const int32_t tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
    const int64_t vbase = (int64_t)view * A.rows * A.cols;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int32_t k = k0 + ty + 8 * i, j = j0 + tx;
#pragma unroll
        for (int m = 0; m < NB; ++m)
            tile[m][ty + 8 * i][tx] = (k < A.rows && j < A.cols)
                                          ? sino.p[m][vbase + (int64_t)k * A.cols + j] : 0.0f;
    }
    __syncthreads();
    auto ray_len = [&](const Frame& F, int32_t j, int32_t k) {
        if (A.beam == BEAM_PARALLEL) return sqrt(F.s[0] * F.s[0] + F.s[1] * F.s[1] + F.s[2] * F.s[2]);
        double p[3];
        pixel_point(F, centred(j, A.cols, A.du), centred(k, A.rows, A.dv), p);
        const double dx = p[0] - F.s[0], dy = p[1] - F.s[1], dz = p[2] - F.s[2];
        return sqrt(dx * dx + dy * dy + dz * dz);
    };
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int32_t j = j0 + ty + 8 * i, k = k0 + tx;
        if (k < rows_pad && j < A.cols) {
            const int64_t o = (((int64_t)blockIdx.z * A.cols + j) * rows_pad + k) * NB;
            float scale = (float)ray_len(A.frames[view], j, k);
#pragma unroll
            for (int m = 0; m < NB; ++m) {
                if (m > 0 && mview != 0) scale = (float)ray_len(A.frames[view + m * mview], j, k);
                ysc[o + m] = tile[m][tx][ty + 8 * i] * scale;
            }
        }
    }
}

__global__ void __launch_bounds__(256) column_line_kernel(const ColumnLaunch A, int32_t views,
                                                          ColLine* __restrict__ out) {
    const int64_t n = (int64_t)views * A.cols;
    for (int64_t i = blockIdx.x * 256ll + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
        const int32_t view = A.view0 + (int32_t)(i / A.cols), j = (int32_t)(i % A.cols);
        column_line(A.frames[view], A.box, A.beam, j, A.cols, A.rows, A.du, A.dv, out[i]);
    }
}

// Rows are taken in groups of S * 64 (S = min(kGroup, ceil(rows / 64))): lane l holds rows
// g0 + S l .. g0 + S l + S - 1 of a group, and one instruction handles row g0 + S l + c of every
// lane. A lane's neighbours in an instruction are S rows away, which on these geometries is
// more than one z cell, so the 64 LDS additions of one instruction go to different addresses.
constexpr int kGroup = kGatherGroup;
// Items a wave queues before it processes them (the queue is drained once it holds more
// than kQueue - 64, so one more round of 64 always fits). 80 items are 5 KiB per wave: with a
// column of at most 5 KiB (about 1280 cells of one member, 640 of two, 320 of four) a block
// of four waves takes at most 40 KiB, so four blocks share a CU's 160 KiB and the register
// budget, not LDS, sets the occupancy.
constexpr int kQueue = 80;
// The tilted gather's queue: 64 items of 88 bytes (5.5 KiB), drained after every round that
// adds to it; with a column of up to about 4 KiB a block of four waves then takes at most
// 40 KiB, and four blocks fit a CU.
constexpr int kTiltQueue = 64;
// Lanes per view when items are built.
constexpr int kViewLanes = 4;

// The column of one wave in LDS, indexed from its guard cell below: index i holds z cell
// z0 - 1 + i for i in [0, n + 1] (n = z1 - z0; indices 0 and n + 1 are guard cells just
// outside the chunk, never written out); indices -2, -1 and n + 2 take pieces that fall
// outside the chunk, so a clamp of the pair index to [-2, n + 1] keeps every pair that
// touches a chunk cell and parks the rest on cells that are never written out.
__host__ __device__ constexpr int32_t gather_column_floats(int32_t zchunk, int nb) {
    return (zchunk + 5) * nb;
}

// Cells are dealt in tiles of tx x ty (y fastest inside a tile): the tasks that run at the
// same time on one XCD then cover a compact patch of the grid, whose shadow on the detector
// is a few dozen columns in every view, so its waves share sinogram lines in L2 (a line of
// cells along y would cover the whole detector width in views along x). Each launcher takes
// the first of its tile shapes that the grid holds a whole number of, else 1 x H (plain
// y-fastest order).
__device__ __forceinline__ void gather_tile_cell(uint32_t xy, int32_t H, int32_t tx, int32_t ty,
                                                 int32_t& ix, int32_t& iy) {
    const uint32_t per = (uint32_t)(tx * ty);
    const uint32_t tile = xy / per, within = xy % per;
    const uint32_t tiles_y = (uint32_t)(H / ty);
    ix = (int32_t)((tile / tiles_y) * (uint32_t)tx + within / (uint32_t)ty);
    iy = (int32_t)((tile % tiles_y) * (uint32_t)ty + within % (uint32_t)ty);
}

// A lane's KR consecutive rows starting at row k0 of one sinogram line, KR being S rounded up
// (gather_rows_loaded; rows past the lane's S are loaded and ignored: a fixed count keeps the
// loads unconditional, so the next unit's loads can be in flight while the current one is
// summed).
template <int NB, int KR>
__device__ __forceinline__ void gather_load_rows(const float* __restrict__ p, float (&w)[KR][NB]) {
#pragma unroll
    for (int c = 0; c < KR; ++c) load_vals<NB>(p + c * NB, w[c]);
}

// Rows a lane loads per unit for S rows per lane: S rounded up to 1, 2, 4, 6 or 8.
__host__ __device__ constexpr int32_t gather_rows_loaded(int32_t S) {
    return S <= 1 ? 1 : S <= 2 ? 2 : S <= 4 ? 4 : S <= 6 ? 6 : kGroup;
}

// Pair index clamped to [-2, hi]: one v_med3_i32 (the compiler emits a max and a min).
__device__ __forceinline__ int32_t clamp_pair(int32_t i, int32_t hi) {
    int32_t r;
    asm("v_med3_i32 %0, %1, -2, %2" : "=v"(r) : "v"(i), "s"(hi));
    return r;
}

// i clamped to [lo, hi] (lo in a vector register, hi uniform): one v_med3_i32.
__device__ __forceinline__ int32_t clamp_range(int32_t i, int32_t lo, int32_t hi) {
    int32_t r;
    asm("v_med3_i32 %0, %1, %2, %3" : "=v"(r) : "v"(i), "v"(lo), "s"(hi));
    return r;
}

// (i << SH) + b: one v_lshl_add_u32, kept as written (the compiler would otherwise fold the
// per-lane base back into each row's index).
template <int SH>
__device__ __forceinline__ int32_t shl_add(int32_t i, int32_t b) {
    int32_t r;
    asm("v_lshl_add_u32 %0, %1, %2, %3" : "=v"(r) : "v"(i), "i"(SH), "v"(b));
    return r;
}

// A uniform value held in a vector register (one v_mov_b32, made once).
__device__ __forceinline__ int32_t in_vgpr(int32_t v) {
    int32_t r;
    asm volatile("v_mov_b32 %0, %1" : "=v"(r) : "s"(v));
    return r;
}

typedef __attribute__((address_space(3))) float lds_float;

// The LDS byte address of a pointer into the kernel's shared memory, and back.
__device__ __forceinline__ int32_t lds_addr(float* p) {
    return (int32_t)(uintptr_t)(lds_float*)p;
}
__device__ __forceinline__ lds_float* lds_ptr(int32_t a) {
    return (lds_float*)(uintptr_t)(uint32_t)a;
}

// Values of the neighbouring lane one step along the wave (DPP wave_shl:1 takes lane l + 1's
// value, wave_shr:1 lane l - 1's; both cross the 16-lane rows). UP: the neighbour "forward"
// is lane l + 1. Floats read 0 past the wave's ends; keys read -1 there.
constexpr int kDppWaveShl1 = 0x130;
constexpr int kDppWaveShr1 = 0x138;
template <bool UP>
__device__ __forceinline__ float from_fwd(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v),
                                                      UP ? kDppWaveShl1 : kDppWaveShr1, 0xF, 0xF, true));
}
template <bool UP>
__device__ __forceinline__ float from_bwd(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v),
                                                      UP ? kDppWaveShr1 : kDppWaveShl1, 0xF, 0xF, true));
}
template <bool UP>
__device__ __forceinline__ int32_t key_fwd(int32_t k) {
    return __builtin_amdgcn_update_dpp(-1, k, UP ? kDppWaveShl1 : kDppWaveShr1, 0xF, 0xF, false);
}
template <bool UP>
__device__ __forceinline__ int32_t key_bwd(int32_t k) {
    return __builtin_amdgcn_update_dpp(-1, k, UP ? kDppWaveShr1 : kDppWaveShl1, 0xF, 0xF, false);
}

// The adds of one instruction of a kFastRuns item: lane l adds qa to the cell pair's lower
// cell and qb to its upper cell (pair address dst, monotone along the wave: rising with the
// lane when UP). Lanes with the same pair form runs of at most G consecutive lanes. Each run's
// lower-cell shares are summed into its first lane (towards lower cells) and its upper-cell
// shares into its last lane, by G - 1 steps of a one-lane shift; the first lane also takes
// the upper-cell sum of the run just below when that run's upper cell is its lower cell.
// Then the first lane of every run writes its lower cell, and the last lane of a run whose
// upper cell no other run holds writes that one: the cells written by one instruction are
// distinct. Lanes with nothing to write add into the parked pair at index -2 (park). Needs
// all 64 lanes active.
template <int NB, bool UP>
__device__ __forceinline__ void gather_runs_add(lds_float* dst, lds_float* park, const float (&qa)[NB],
                                                const float (&qb)[NB], int32_t G) {
    typedef __attribute__((address_space(3))) float __attribute__((ext_vector_type(NB))) cell_t;
    const int32_t key = (int32_t)(uintptr_t)dst;
    const int32_t kb = key_bwd<UP>(key), kf = key_fwd<UP>(key);
    const bool first = kb != key, last = kf != key;
    const bool adj = kf == key + 4 * NB;             // the next run's lower cell is our upper cell
    // the first shift step for any G (with G == 1 every lane is a run of its own and the step
    // adds zeros), the rest in a loop
    float T[NB], U[NB];
#pragma unroll
    for (int m = 0; m < NB; ++m) {
        T[m] = qa[m] + from_fwd<UP>(first ? 0.0f : qa[m]);
        U[m] = qb[m] + from_bwd<UP>(last ? 0.0f : qb[m]);
    }
    for (int32_t k = 2; k < G; ++k) {
#pragma unroll
        for (int m = 0; m < NB; ++m) {
            T[m] = qa[m] + from_fwd<UP>(first ? 0.0f : T[m]);
            U[m] = qb[m] + from_bwd<UP>(last ? 0.0f : U[m]);
        }
    }
#pragma unroll
    for (int m = 0; m < NB; ++m) T[m] += from_bwd<UP>(adj ? U[m] : 0.0f);
    cell_t* const p0 = (cell_t*)(first ? dst : park);
    cell_t* const p1 = (cell_t*)(last && !adj ? dst : park);
    cell_t lo = p0[0], hi = p1[1];
#pragma unroll
    for (int m = 0; m < NB; ++m) {
        lo[m] += T[m];
        hi[m] += U[m];
    }
    p0[0] = lo;
    p1[1] = hi;
}

// Fast form of one item for one group of rows (see gather_fast): every row adds its two
// pieces to the cell pair {fa, fa + 1}. The lane's rows are placed relative to its origin row
// c0 (fast_origin_row): row c lies (c - c0) per-row advances a1, b1 from it, an exact integer
// step. Not RUNS (kFastPairs): all lanes update their pairs at once with one paired read and
// write. RUNS (kFastRuns): lanes that share a pair are combined first (gather_runs_add); lanes
// S * G rows apart never share one. FULL: the lane takes all KR loaded rows (S == KR), so the
// unrolled rows need no guard. CLAMP: some row may leave the chunk's pair indices (the item is
// not kFastInside), so every pair index is clamped. SH: the cell slots take the loaded members
// turned by SH places (slot m adds member (m - SH) mod NB: the gather shared over a turn
// symmetry, where the members are the lines of the views the turn relates).
template <int NB, int KR, bool FULL, bool RUNS, bool CLAMP, int SH = 0>
__device__ __forceinline__ void gather_fast_group(const GatherItem& it, int32_t a1, int32_t b1,
                                                  float dt, const float (&w)[KR][NB],
                                                  int32_t k0, int32_t S, int32_t z0, int32_t n,
                                                  float* col, int32_t G) {
    // the origin row of fast_origin_row(S): the middle one when S == kGroup
    constexpr int c0 = FULL && KR == kGroup ? kGroup / 2 : 0;
    uint32_t la, lb;
    int32_t base;
    fast_origin(it, k0 + c0, z0 - 1, la, lb, base);
    // A row's pair index is base + fb (fb in [0, 15]); with CLAMP it is clamped to [-2, n + 1].
    // One member: the index is a byte address, and the clamp works on it. The base is first
    // clamped to [-24, n + 8], which leaves every clamped index unchanged and keeps the address
    // far from overflow, so each row forms its address with one shift-add and one clamp (two
    // and four members keep the index form, which needs fewer registers).
    const int32_t a0 = lds_addr(col);
    int32_t abase = 0, alo = 0, ahi = 0;
    if constexpr (NB == 1) {
        if constexpr (CLAMP) {
            abase = (clamp_range(base, -24, n + 8) << 2) + a0;
            alo = in_vgpr(a0 - 8);
            ahi = a0 + ((n + 1) << 2);
        } else {
            abase = (base << 2) + a0;
        }
    }
    uint32_t za[KR], zb[KR];
    za[c0] = la;
    zb[c0] = lb;
#pragma unroll
    for (int c = c0 + 1; c < KR; ++c) {
        za[c] = za[c - 1] + (uint32_t)a1;
        zb[c] = zb[c - 1] + (uint32_t)b1;
    }
#pragma unroll
    for (int c = c0 - 1; c >= 0; --c) {
        za[c] = za[c + 1] - (uint32_t)a1;
        zb[c] = zb[c + 1] - (uint32_t)b1;
    }
#pragma unroll
    for (int c = 0; c < KR; ++c) {
        if (!FULL && c >= S) continue;
        int32_t fb;
        uint32_t num, ext;
        fast_row(za[c], zb[c], fb, num, ext);
        // the shares of the lower and upper cells, num / ext and (ext - num) / ext, when the
        // row crosses the plane above fa, else 1 and 0: num >= ext exactly when it does not,
        // so a min with 1 and a saturating difference select both cases; a row of zero extent
        // has an infinite reciprocal, which the min turns into 1 (num >= 1) and the legacy
        // multiply (0 times anything is 0) into 0. Each share comes from its own integer, so
        // a thin piece keeps its relative precision.
        const float r = __builtin_amdgcn_rcpf((float)ext);
        const float f = fminf((float)num * r, 1.0f);
        const float g = mul_legacy((float)__builtin_elementwise_sub_sat(ext, num), r);
        const float fd = f * dt, gd = g * dt;
        lds_float* dst;
        if constexpr (NB == 1) {
            const int32_t ad = shl_add<2>(fb, abase);
            dst = lds_ptr(CLAMP ? clamp_range(ad, alo, ahi) : ad);
        } else {
            const int32_t pi = base + fb;
            dst = lds_ptr(a0 + (CLAMP ? clamp_pair(pi, n + 1) : pi) * (4 * NB));
        }
        float qa[NB], qb[NB];
#pragma unroll
        for (int m = 0; m < NB; ++m) {
            qa[m] = fd * w[c][(m + NB - SH) % NB];
            qb[m] = gd * w[c][(m + NB - SH) % NB];
        }
        // cells are moved through their own vector type, so that the compiler knows their
        // alignment (4 * NB bytes) and moves each with one access
        typedef __attribute__((address_space(3))) float __attribute__((ext_vector_type(NB))) cell_t;
        if constexpr (RUNS) {
            lds_float* const park = lds_ptr(a0 - 8 * NB);
            if (a1 > 0)
                gather_runs_add<NB, true>(dst, park, qa, qb, G);
            else
                gather_runs_add<NB, false>(dst, park, qa, qb, G);
        } else if constexpr (NB == 1) {
            const float lo = dst[0], hi = dst[1];
            dst[0] = lo + qa[0];
            dst[1] = hi + qb[0];
        } else {
            cell_t* cp = (cell_t*)dst;
            cell_t lo = cp[0], hi = cp[1];
#pragma unroll
            for (int m = 0; m < NB; ++m) {
                lo[m] += qa[m];
                hi[m] += qb[m];
            }
            cp[0] = lo;
            cp[1] = hi;
        }
    }
}

// General form of one item for one group of rows: rows of any z extent, pieces walked in
// fp64; plain LDS read-add-write when the item's lanes add exclusively, else LDS atomics.
template <int NB, int KR, int SH = 0>
__device__ __forceinline__ void gather_general_group(const GatherItem& it, bool exclusive,
                                                     const float (&w)[KR][NB], int32_t k0,
                                                     int32_t S, int32_t z0, int32_t z1,
                                                     float* col) {
    const double dt = (double)it.dt;
    const float fdt = it.dt;
    auto add = [&](int32_t iz, float f, const float* wv) {
        float* dst = col + (iz - z0 + 1) * NB;
        if (exclusive) {
#pragma unroll
            for (int m = 0; m < NB; ++m) dst[m] += f * wv[m];
        } else {
#pragma unroll
            for (int m = 0; m < NB; ++m) atomicAdd(dst + m, f * wv[m]);
        }
    };
#pragma unroll
    for (int c = 0; c < KR; ++c) {
        if (c >= S) continue;
        float wr[NB];      // the members in slot order (turned by SH, as in gather_fast_group)
#pragma unroll
        for (int m = 0; m < NB; ++m) wr[m] = w[c][(m + NB - SH) % NB];
        const double kd = (double)(k0 + c);
        const double za = fma(kd, it.za1, it.za0);
        const double zb = fma(kd, it.zb1, it.zb0);
        const double zmin = fmin(za, zb), zmax = fmax(za, zb);
        const double ext = zmax - zmin;
        if (ext < 1.0) {
            // at most two z cells: fa gets the share f of dt, fb the rest
            const double fa = floor(zmin), fb = floor(zmax);
            const float f = fa == fb ? 1.0f
                : (float)(fa + 1.0 - zmin) * __builtin_amdgcn_rcpf((float)ext);
            const float p1 = f * fdt, p2 = fdt - p1;
            if (fa >= (double)z0 && fa < (double)z1) add((int32_t)fa, p1, wr);
            if (fb != fa && fb >= (double)z0 && fb < (double)z1) add((int32_t)fb, p2, wr);
        } else {
            auto piece = [&](int32_t iz, double share) { add(iz, (float)share, wr); };
            row_pieces_split(za, zb, dt, z0, z1, exclusive, piece);
        }
    }
}

// Occupancy: four waves per SIMD (at most 128 vector registers) for one member, three (168)
// for two and four.
//
// P > 1: the gather shared over a turn symmetry of the views (orbit_cell). The launch's views
// are the first q = nviews / P; NB == P and member m of the reordered sinogram is the line of
// view v + m q. A wave owns the P cells of one orbit, held as the NB slots of its column (slot
// a: cell R^a of the orbit's cell in the grid orbit_grid gives), and the item of slot a's cell
// adds member m to slot (a + m) mod P; the volume written has one member.
template <int NB, int KR, int P>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(NB == 1 ? 4 : 3)))
column_gather_kernel(const ColumnLaunch A, const ColLine* __restrict__ lines,
                     const float* __restrict__ ysc, float* __restrict__ vol, int32_t zchunk,
                     int32_t nchunks, int32_t tx, int32_t ty, int32_t accumulate, int32_t dir) {
    static_assert(P == 1 || P == NB, "an orbit takes one member per slot");
    extern __shared__ __align__(16) unsigned char lds_raw[];
    const uint32_t wave = uniform(threadIdx.x >> 6);
    const int32_t lane = (int32_t)(threadIdx.x & 63u);
    // blocks dealt round-robin to the XCDs, as the hardware deals them: the XCDs work on
    // neighbouring cells of one tile at a time and share its sinogram lines in the
    // memory-side cache
    const uint32_t blk = blockIdx.x;
    const uint32_t task = blk * 4u + wave;
    const int32_t W = A.box.n[0], H = A.box.n[1], D = A.box.n[2];
    int32_t Wr, Hr;
    orbit_grid(P, W, H, Wr, Hr);
    const int32_t zc = (int32_t)(task % (uint32_t)nchunks);
    const bool live = task < (uint32_t)Wr * (uint32_t)Hr * (uint32_t)nchunks;
    int32_t ix, iy;
    gather_tile_cell(task / (uint32_t)nchunks, Hr, tx, ty, ix, iy);
    const int32_t z0 = zc * zchunk;
    const int32_t z1 = live ? (z0 + zchunk < D ? z0 + zchunk : D) : z0;
    const int32_t n = z1 - z0;
    const int32_t colf = gather_column_floats(zchunk, NB);
    float* const cols = reinterpret_cast<float*>(lds_raw) + wave * colf;
    float* const col = cols + 2 * NB;                   // the guard cell below the chunk
    GatherItem* Q = reinterpret_cast<GatherItem*>(lds_raw + 4 * (size_t)colf * sizeof(float)) + wave * kQueue;
    for (int32_t i = lane; i < colf; i += 64) cols[i] = 0.0f;
    __syncthreads();
    // lanes per view when items are built: one for one slot (the helical batch: 123.5 ms,
    // against 125.8 with two and 129.1 with four), four for an orbit (the 512^3 cone: 87.8
    // against 90.9 with two)
    constexpr int VL = P == 1 ? 1 : kViewLanes;
    if (live) {
        const bool line = A.beam == BEAM_PARALLEL;
        const int32_t S = gather_stride(A.rows);
        const int32_t rows_pad = gather_rows_padded(A.rows);
        const int32_t vend = A.view0 + A.nviews / P;

        // Units of work: (item, row group) in queue order, counted without divisions. The rows
        // of the next unit are loaded while the current one is summed.
        const int32_t ngroups = rows_pad / (64 * S);
        // Fast items that keep to the chunk skip the clamp when a lane holds several rows. With
        // one row per lane a unit is short, and the unclamped variants' extra code costs more
        // than the clamp (measured on the helical batch), so those items keep it and skip the
        // range test.
        constexpr bool kUnclamped = KR > 1;
        const float in_lo = kUnclamped ? fast_inside_lo(z0, n) : INFINITY;
        const float in_hi = kUnclamped ? fast_inside_hi(z0, n) : -INFINITY;
        int32_t lane_row = S * lane;
        asm volatile("" : "+v"(lane_row));    // kept as one value: a unit's first row is one add
        auto unit_rows = [&](int32_t i, int32_t gi) {
            const int32_t yoff = (int32_t)uniform((uint32_t)Q[i].yoff);
            return ysc + ((int64_t)yoff * rows_pad + gi * 64 * S + lane_row) * NB;
        };
        // The queue's items all belong to one cell of the orbit (slot SH = decltype(shift)):
        // their rows go to the slots turned by SH places.
        auto drain = [&](auto shift, int32_t count) __attribute__((always_inline)) {
            constexpr int SH = decltype(shift)::value;
            if (count == 0) return;
            float wa[KR][NB], wb[KR][NB];
            gather_load_rows<NB, KR>(unit_rows(0, 0), wa);
            int32_t i = 0, gi = 0;
            // One unit: the next unit's rows are loaded into nxt while cur is summed; false
            // after the last unit.
            auto unit = [&](const float (&cur)[KR][NB], float (&nxt)[KR][NB]) {
                int32_t ni = i, ngi = gi + 1;
                if (ngi == ngroups) {
                    ngi = 0;
                    ++ni;
                }
                const bool more = ni < count;
                gather_load_rows<NB, KR>(unit_rows(more ? ni : i, more ? ngi : gi), nxt);
                const int32_t k0 = gi * 64 * S + lane_row;
                const GatherItem it = Q[i];
                const int32_t form = (int32_t)uniform((uint32_t)it.form);
                {
                    if (form > 0) {
                        const float dt = __uint_as_float(uniform(__float_as_uint(it.dt)));
                        const int32_t a1 = (int32_t)uniform((uint32_t)it.a1fx);
                        const int32_t b1 = (int32_t)uniform((uint32_t)it.b1fx);
                        // items whose rows all stay inside the chunk skip the clamp (full groups
                        // of several rows per lane only)
                        const bool inside = kUnclamped && (form & kFastInside) != 0;
                        if ((form & ~kFastInside) == kFastPairs) {
                            if (S == KR && inside)
                                gather_fast_group<NB, KR, true, false, false, SH>(it, a1, b1, dt, cur, k0, S, z0, n, col, 1);
                            else if (S == KR)
                                gather_fast_group<NB, KR, true, false, true, SH>(it, a1, b1, dt, cur, k0, S, z0, n, col, 1);
                            else
                                gather_fast_group<NB, KR, false, false, true, SH>(it, a1, b1, dt, cur, k0, S, z0, n, col, 1);
                        } else {
                            const int32_t G = (int32_t)uniform((uint32_t)it.run);
                            if (S == KR && inside)
                                gather_fast_group<NB, KR, true, true, false, SH>(it, a1, b1, dt, cur, k0, S, z0, n, col, G);
                            else if (S == KR)
                                gather_fast_group<NB, KR, true, true, true, SH>(it, a1, b1, dt, cur, k0, S, z0, n, col, G);
                            else
                                gather_fast_group<NB, KR, false, true, true, SH>(it, a1, b1, dt, cur, k0, S, z0, n, col, G);
                        }
                    } else {
                        gather_general_group<NB, KR, SH>(it, form == kGeneralExclusive, cur, k0, S, z0, z1, col);
                    }
                }
                i = ni;
                gi = ngi;
                return more;
            };
            if constexpr (NB == 1 && KR > 1) {
                // the buffers swap roles from unit to unit, so no rows are copied
                while (unit(wa, wb) && unit(wb, wa)) {
                }
            } else {
                // one copy of the unit's code and the prefetched rows moved over: with one row
                // per lane the short units are sensitive to code size, and with several members
                // two copies would not stay inlined
                while (unit(wa, wb)) {
#pragma unroll
                    for (int c = 0; c < KR; ++c)
#pragma unroll
                        for (int m = 0; m < NB; ++m) wa[c][m] = wb[c][m];
                }
            }
        };

        // Items: VL lanes take one view of a round of 64 / VL and walk its
        // candidate columns, lane r of a view taking candidates j0 + r, j0 + r + VL, ...;
        // the crossings found are appended to the queue in lane order. A round spans few
        // views, so the sinogram lines the concurrently running waves of a tile read stay few
        // enough to share L2. With an orbit, the slots' cells take their turns, each over the
        // launch's views, and the queue is drained at the end of each turn, so that one drain
        // sees items of one slot only.
        int32_t count = 0;
        auto flush = [&](int32_t a) __attribute__((always_inline)) {
            if constexpr (P == 1) {
                drain(std::integral_constant<int, 0>{}, count);
            } else {
                if (a == 0) drain(std::integral_constant<int, 0>{}, count);
                else if (a == 1) drain(std::integral_constant<int, 1>{}, count);
                else if constexpr (P == 4) {
                    if (a == 2) drain(std::integral_constant<int, 2>{}, count);
                    else drain(std::integral_constant<int, 3>{}, count);
                }
            }
            count = 0;
        };
        for (int32_t a = 0; a < P; ++a) {
            int32_t cx, cy;
            orbit_cell(P, dir, W, H, ix, iy, a, cx, cy);
            const double x0 = A.box.lo[0] + cx * A.box.pitch[0], x1 = x0 + A.box.pitch[0];
            const double y0 = A.box.lo[1] + cy * A.box.pitch[1], y1 = y0 + A.box.pitch[1];
            for (int32_t vb = A.view0; vb < vend; vb += 64 / VL) {
                const int32_t view = vb + lane / VL;
                int32_t jn = 0, j1 = -1;
                if (view < vend &&
                    !cell_column_range(A.frames[view], A.beam, A.cols, A.du, x0, x1, y0, y1, jn, j1)) {
                    jn = 0;
                    j1 = -1;
                }
                if (view >= vend) j1 = -1;
                jn += lane % VL;
                while (__ballot(jn <= j1) != 0) {
                    GatherItem it;
                    bool hit = false;
                    if (jn <= j1) {
                        const int32_t yoff = (view - A.view0) * A.cols + jn;
                        hit = gather_item(lines[yoff], line, x0, x1, y0, y1, S, A.rows, rows_pad, yoff,
                                          it, in_lo, in_hi);
                        jn += VL;
                    }
                    const uint64_t m = __ballot(hit);
                    if (hit) {
                        const uint32_t below = __builtin_amdgcn_mbcnt_hi(
                            (uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
                        Q[count + (int32_t)below] = it;
                    }
                    count += (int32_t)__popcll(m);
                    if (count > kQueue - 64) {
                        wave_lds_sync();
                        flush(a);
                        wave_lds_sync();
                    }
                }
            }
            wave_lds_sync();
            flush(a);
            wave_lds_sync();
        }
    }
    __syncthreads();
    if (live) {
        if constexpr (P == 1) {
            const int64_t base = (((int64_t)ix * H + iy) * D + z0) * NB;
            for (int32_t i = lane; i < n * NB; i += 64)
                vol[base + i] = accumulate ? vol[base + i] + col[NB + i] : col[NB + i];
        } else {
            // slot a of z cell i is col[NB (i + 1) + a]; each slot's cell gets its own column
#pragma unroll
            for (int32_t a = 0; a < P; ++a) {
                int32_t cx, cy;
                orbit_cell(P, dir, W, H, ix, iy, a, cx, cy);
                const int64_t base = ((int64_t)cx * H + cy) * D + z0;
                for (int32_t i = lane; i < n; i += 64) {
                    const float v = col[NB * (i + 1) + a];
                    vol[base + i] = accumulate ? vol[base + i] + v : v;
                }
            }
        }
    }
}

// ------------------------------------------------------------------------------------------
// Gather for cone geometries whose detector rows do not run along z (tilted detectors, any
// frame): a wave owns one xy cell's z column in LDS as in column_gather_kernel, but each lane
// takes one row of an item (view, column, up to 64 rows) and clips that row's own ray
// against the cell in fp64.

// The adds of one instruction when the lanes' pair addresses are monotone along the wave
// (rising with the lane when UP): as gather_runs_add, with as many shift steps as the longest
// run of equal addresses strictly between the parked pairs (park, at index -2, and top, at
// the column's upper end) needs, found by comparing each lane's address with the one t lanes
// ahead. Runs on the parked pairs hold only shares that are never written out and are left
// unmerged. Needs all 64 lanes active.
template <int NB, bool UP>
__device__ __forceinline__ void gather_runs_add_any(lds_float* dst, lds_float* park, lds_float* top,
                                                    const float (&qa)[NB], const float (&qb)[NB]) {
    typedef __attribute__((address_space(3))) float __attribute__((ext_vector_type(NB))) cell_t;
    const int32_t key = (int32_t)(uintptr_t)dst;
    const int32_t kb = key_bwd<UP>(key), kf = key_fwd<UP>(key);
    const bool first = kb != key, last = kf != key;
    const bool adj = kf == key + 4 * NB;
    float T[NB], U[NB];
#pragma unroll
    for (int m = 0; m < NB; ++m) {
        T[m] = qa[m];
        U[m] = qb[m];
    }
    const bool inner = key > (int32_t)(uintptr_t)park && key < (int32_t)(uintptr_t)top;
    int32_t ahead = kf;                              // the address t lanes ahead (t = 1, 2, ...)
    while (__ballot(inner && ahead == key) != 0) {
#pragma unroll
        for (int m = 0; m < NB; ++m) {
            T[m] = qa[m] + from_fwd<UP>(first ? 0.0f : T[m]);
            U[m] = qb[m] + from_bwd<UP>(last ? 0.0f : U[m]);
        }
        ahead = key_fwd<UP>(ahead);
    }
#pragma unroll
    for (int m = 0; m < NB; ++m) T[m] += from_bwd<UP>(adj ? U[m] : 0.0f);
    cell_t* const p0 = (cell_t*)(first ? dst : park);
    cell_t* const p1 = (cell_t*)(last && !adj ? dst : park);
    cell_t lo = p0[0], hi = p1[1];
#pragma unroll
    for (int m = 0; m < NB; ++m) {
        lo[m] += T[m];
        hi[m] += U[m];
    }
    p0[0] = lo;
    p1[1] = hi;
}

// 1 / x in fp64 for x != 0: the hardware reciprocal refined by one Newton step, which squares
// its relative error. Measured on MI355X over a million inputs with |x| in [1e-3, 1e4]: the
// bare reciprocal within 4.6e-8, one step within 2.3e-15 of 1 / x (a parameter error of that
// size moves a row's ends by less than 1e-12 cell).
__device__ __forceinline__ double rcp_f64(double x) {
    const double r = __builtin_amdgcn_rcp(x);
    return fma(fma(-x, r, 1.0), r, r);
}

// The clip of tilt_clip from the walls' offsets from the source (wl = lo - s, wh = hi - s per
// axis), with rcp_f64 in place of the divisions: [t0, t1], empty unless t1 > t0.
__device__ __forceinline__ void tilt_clip_walls(const double (&d)[2], const double (&wl)[2],
                                                const double (&wh)[2], double& t0, double& t1) {
    double a = 0.0, b = 1.0;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        if (d[k] != 0.0) {
            const double r = rcp_f64(d[k]);
            const double p = wl[k] * r, q = wh[k] * r;
            a = fmax(a, fmin(p, q));
            b = fmin(b, fmax(p, q));
        } else if (wl[k] > 0.0 || wh[k] <= 0.0) {      // the source outside [lo, hi)
            b = -1.0;
        }
    }
    t0 = a;
    t1 = b;
}

// P > 1: shared over a turn symmetry of the views as column_gather_kernel is (orbit_cell): the
// launch's views are the first q = nviews / P, member m of the reordered sinogram is the line
// of view v + m q, and a wave owns the P cells of an orbit as the NB == P slots of its column.
// Occupancy: four waves per SIMD (at most 128 vector registers; the LDS of a four-wave block,
// its columns and 64-item queues, stays within a quarter of the compute unit's for columns
// of up to 4 KiB). The wave takes one item at a time: preparing two at once, for their fp64
// chains to interleave, needed 168 registers and held the kernel to three waves per SIMD,
// which ran slower.
template <int NB, int P>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4)))
tilt_gather_kernel(const ColumnLaunch A, const float* __restrict__ ysc, float* __restrict__ vol,
                   int32_t zchunk, int32_t nchunks, int32_t tx, int32_t ty, int32_t accumulate,
                   int32_t dir) {
    static_assert(P == 1 || P == NB, "an orbit takes one member per slot");
    extern __shared__ __align__(16) unsigned char lds_raw[];
    const uint32_t wave = uniform(threadIdx.x >> 6);
    const int32_t lane = (int32_t)(threadIdx.x & 63u);
    // blocks dealt round-robin to the XCDs (against one contiguous range of tiles per XCD: the
    // tilted 256^3 cone 32.9 -> 32.2 ms)
    const uint32_t blk = blockIdx.x;
    const uint32_t task = blk * 4u + wave;
    const int32_t W = A.box.n[0], H = A.box.n[1], D = A.box.n[2];
    int32_t Wr, Hr;
    orbit_grid(P, W, H, Wr, Hr);
    const int32_t zc = (int32_t)(task % (uint32_t)nchunks);
    const bool live = task < (uint32_t)Wr * (uint32_t)Hr * (uint32_t)nchunks;
    int32_t ix, iy;
    gather_tile_cell(task / (uint32_t)nchunks, Hr, tx, ty, ix, iy);
    const int32_t z0 = zc * zchunk;
    const int32_t z1 = live ? (z0 + zchunk < D ? z0 + zchunk : D) : z0;
    const int32_t n = z1 - z0;
    const int32_t colf = gather_column_floats(zchunk, NB);
    float* const cols = reinterpret_cast<float*>(lds_raw) + wave * colf;
    float* const col = cols + 2 * NB;                   // the guard cell below the chunk
    TiltItem* Q = reinterpret_cast<TiltItem*>(lds_raw + 4 * (size_t)colf * sizeof(float)) + wave * kTiltQueue;
    for (int32_t i = lane; i < colf; i += 64) cols[i] = 0.0f;
    __syncthreads();
    if (live) {
        const int32_t rows_pad = gather_rows_padded(A.rows);
        const int32_t vend = A.view0 + A.nviews / P;
        const double ipz = 1.0 / A.box.pitch[2];
        const int32_t a0 = lds_addr(col);
        lds_float* const park = lds_ptr(a0 - 8 * NB);
        lds_float* const top = lds_ptr(a0 + 4 * NB * (n + 1));

        // one lane's row values of item i (zero past the item's rows)
        auto load_rows = [&](int32_t i, float (&w)[NB]) {
            const int32_t view = (int32_t)uniform((uint32_t)Q[i].view);
            const int32_t j = (int32_t)uniform((uint32_t)Q[i].j);
            const int32_t k0 = (int32_t)uniform((uint32_t)Q[i].k0);
            const int32_t nrows = (int32_t)uniform((uint32_t)Q[i].nrows);
            // lanes past the item's rows read its last row (always in the line) and take 0, so
            // the load needs no branch
            const bool in = lane < nrows;
            const int32_t k = k0 + (in ? lane : nrows - 1);
            const float* yp = ysc + (((int64_t)(view - A.view0) * A.cols + j) * rows_pad + k) * NB;
#pragma unroll
            for (int m = 0; m < NB; ++m) w[m] = in ? yp[m] : 0.0f;
        };
        const double lane_dv = (double)lane * A.dv;
        // One lane's row of one item: its clip against the cell, z at both ends and the two-cell
        // shares (prep, arithmetic only), then its adds into the column (commit). The drain preps
        // two items before committing either, so that their independent fp64 chains interleave.
        struct Row {
            float qa[NB], qb[NB];
            double za, zb, dtd;
            int32_t i0;
            bool active, two, lng, up;
        };
        // SH: the slots take the members turned by SH places (slot m adds member (m - SH) mod NB)
        auto prep = [&](auto shift, const TiltItem& it, const float (&w)[NB], Row& R) __attribute__((always_inline)) {
            constexpr int SH = decltype(shift)::value;
            const int32_t nrows = (int32_t)uniform((uint32_t)it.nrows);
            // the row's ray direction: xy in world units, z in cells per unit parameter
            const double v = centred((int32_t)uniform((uint32_t)it.k0), A.rows, A.dv) + lane_dv;
            const double d[2] = {fma(v, it.evx, it.bx), fma(v, it.evy, it.by)};
            const double dzc = fma(v, it.evzc, it.bzc);
            const double wl[2] = {it.wx0, it.wy0};
            const double wh[2] = {it.wx0 + A.box.pitch[0], it.wy0 + A.box.pitch[1]};
            double t0, t1;
            if (__ballot(d[0] == 0.0 || d[1] == 0.0) == 0) {
                // no row of the item runs parallel to a wall (the rule): no per-lane branch
                const double rx = rcp_f64(d[0]), ry = rcp_f64(d[1]);
                const double px = wl[0] * rx, qx = wh[0] * rx, py = wl[1] * ry, qy = wh[1] * ry;
                t0 = fmax(fmax(fmin(px, qx), fmin(py, qy)), 0.0);
                t1 = fmin(fmin(fmax(px, qx), fmax(py, qy)), 1.0);
            } else {
                tilt_clip_walls(d, wl, wh, t0, t1);
            }
            R.active = lane < nrows && t1 > t0;
            const double szc = it.szc;
            R.za = fma(t0, dzc, szc);
            R.zb = fma(t1, dzc, szc);
            R.dtd = t1 - t0;
            const double zmin = fmin(R.za, R.zb), zmax = fmax(R.za, R.zb);
            const double fa = floor(zmin);
            R.lng = R.active && !(zmax < fa + 2.0);                // spans more than two cells
            // the shares of cells fa and fa + 1: (fa + 1 - zmin) / ext and (zmax - fa - 1) / ext,
            // the second 0 when the row stays in cell fa
            const float dt = (float)R.dtd;
            const float r = __builtin_amdgcn_rcpf((float)(zmax - zmin));
            const float f = fminf((float)(fa + 1.0 - zmin) * r, 1.0f);
            const float g = mul_legacy(fmaxf((float)(zmax - (fa + 1.0)), 0.0f), r);
            R.two = R.active && !R.lng;
#pragma unroll
            for (int m = 0; m < NB; ++m) {
                const float q = R.two ? dt * w[(m + NB - SH) % NB] : 0.0f;
                R.qa[m] = f * q;
                R.qb[m] = g * q;
            }
            R.i0 = (int32_t)fmax(fmin(fa - (double)(z0 - 1), (double)(n + 1)), -2.0);
            R.up = it.evzc >= 0.0;
        };
        auto commit = [&](auto shift, const Row& R, const float (&w)[NB]) __attribute__((always_inline)) {
            constexpr int SH = decltype(shift)::value;
            // pair address, clamped to the parked pairs below and above the chunk; lanes past
            // the item's crossing rows take the parked pair at their end of the column, so the
            // addresses stay monotone when the rows' cells are
            const bool up = R.up;
            const uint64_t act = __ballot(R.active);
            int32_t key = a0 + R.i0 * 4 * NB;
            const int32_t kpark = lds_addr((float*)park), ktop = lds_addr((float*)top);
            if (act != 0) {
                const int32_t lo_lane = (int32_t)__builtin_ctzll(act), hi_lane = 63 - (int32_t)__builtin_clzll(act);
                if (lane < lo_lane) key = up ? kpark : ktop;
                if (lane > hi_lane) key = up ? ktop : kpark;
            } else {
                key = kpark;
            }
            lds_float* const dst = lds_ptr(key);
            // addresses monotone along the wave in the rows' direction: combine runs; else LDS
            // atomics
            const int32_t kf = up ? key_fwd<true>(key) : key_fwd<false>(key);
            if (__ballot(kf != -1 && kf < key) == 0) {
                if (up)
                    gather_runs_add_any<NB, true>(dst, park, top, R.qa, R.qb);
                else
                    gather_runs_add_any<NB, false>(dst, park, top, R.qa, R.qb);
            } else if (R.two) {
                float* const c0 = col + R.i0 * NB;
#pragma unroll
                for (int m = 0; m < NB; ++m) {
                    atomicAdd(c0 + m, R.qa[m]);
                    atomicAdd(c0 + NB + m, R.qb[m]);
                }
            }
            if (R.lng) {
                auto piece = [&](int32_t iz, double share) {
                    float* const c = col + (iz - z0 + 1) * NB;
#pragma unroll
                    for (int m = 0; m < NB; ++m) atomicAdd(c + m, (float)share * w[(m + NB - SH) % NB]);
                };
                row_pieces_split(R.za, R.zb, R.dtd, z0, z1, false, piece);
            }
        };
        auto any_nonzero = [&](const float (&w)[NB]) {
            bool nz = false;
#pragma unroll
            for (int m = 0; m < NB; ++m) nz |= w[m] != 0.0f;
            return __ballot(nz) != 0;
        };
        // Items in queue order, one at a time; the next item's row values are loaded while the
        // current one is summed (the buffers swap roles from step to step). An item whose rows
        // are all zero adds nothing.
        // The queue's items all belong to one cell of the orbit (slot SH = decltype(shift)).
        auto drain = [&](auto shift, int32_t count) __attribute__((always_inline)) {
            if (count == 0) return;
            float wa[NB], wb[NB];
            load_rows(0, wa);
            int32_t i = 0;
            auto step = [&](const float (&cur)[NB], float (&nxt)[NB]) {
                if (i + 1 < count) load_rows(i + 1, nxt);
                if (any_nonzero(cur)) {
                    Row r;
                    prep(shift, Q[i], cur, r);
                    commit(shift, r, cur);
                }
                ++i;
                return i < count;
            };
            while (step(wa, wb) && step(wb, wa)) {
            }
        };

        // Items: kViewLanes lanes take one view of a round; lane r of a view walks its
        // candidate columns j0 + r, j0 + r + kViewLanes, ... and emits the column's rows that
        // can cross the cell in pieces of at most 64.
        int32_t count = 0;
        auto flush = [&](int32_t a) __attribute__((always_inline)) {
            if constexpr (P == 1) {
                drain(std::integral_constant<int, 0>{}, count);
            } else {
                if (a == 0) drain(std::integral_constant<int, 0>{}, count);
                else if (a == 1) drain(std::integral_constant<int, 1>{}, count);
                else if constexpr (P == 4) {
                    if (a == 2) drain(std::integral_constant<int, 2>{}, count);
                    else drain(std::integral_constant<int, 3>{}, count);
                }
            }
            count = 0;
        };
        for (int32_t a = 0; a < P; ++a) {
            if (a > 0) {
                // the previous slot's last items
                wave_lds_sync();
                flush(a - 1);
                wave_lds_sync();
            }
            int32_t cx, cy;
            orbit_cell(P, dir, W, H, ix, iy, a, cx, cy);
            const double x0 = A.box.lo[0] + cx * A.box.pitch[0], x1 = x0 + A.box.pitch[0];
            const double y0 = A.box.lo[1] + cy * A.box.pitch[1], y1 = y0 + A.box.pitch[1];
            for (int32_t vb = A.view0; vb < vend; vb += 64 / kViewLanes) {
                const int32_t view = vb + lane / kViewLanes;
                TiltCorners T;
                int32_t jn = 0, j1 = -1;
                if (view < vend) {
                    tilt_corners(A.frames[view], x0, x1, y0, y1, T);
                    if (!tilt_column_range(T, A.rows, A.cols, A.du, A.dv, jn, j1)) j1 = -1;
                }
                jn += lane % kViewLanes;
                int32_t jc = 0, kk = 0, kl = -1;
                for (;;) {
                    if (kk > kl && jn <= j1) {
                        jc = jn;
                        jn += kViewLanes;
                        if (!tilt_row_range(T, jc, A.rows, A.cols, A.du, A.dv, kk, kl)) {
                            kk = 0;
                            kl = -1;
                        }
                    }
                    const bool emit = kk <= kl;
                    if (__ballot(emit || jn <= j1) == 0) break;
                    const uint64_t m = __ballot(emit);
                    if (emit) {
                        const uint32_t below = __builtin_amdgcn_mbcnt_hi(
                            (uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
                        const Frame& F = A.frames[view];
                        const double u = centred(jc, A.cols, A.du);
                        TiltItem t;
                        t.bx = (F.c[0] - F.s[0]) + u * F.u[0];
                        t.by = (F.c[1] - F.s[1]) + u * F.u[1];
                        t.bzc = ((F.c[2] - F.s[2]) + u * F.u[2]) * ipz;
                        t.evx = F.v[0];
                        t.evy = F.v[1];
                        t.evzc = F.v[2] * ipz;
                        t.wx0 = x0 - F.s[0];
                        t.wy0 = y0 - F.s[1];
                        t.szc = (F.s[2] - A.box.lo[2]) * ipz;
                        t.view = view;
                        t.j = jc;
                        t.k0 = kk;
                        t.nrows = kl - kk + 1 < 64 ? kl - kk + 1 : 64;
                        Q[count + (int32_t)below] = t;
                        kk += 64;
                    }
                    count += (int32_t)__popcll(m);
                    if (count > kTiltQueue - 64) {
                        wave_lds_sync();
                        flush(a);
                        wave_lds_sync();
                    }
                }
            }
        }
        wave_lds_sync();
        flush(P - 1);
    }
    __syncthreads();
    if (live) {
        if constexpr (P == 1) {
            const int64_t base = (((int64_t)ix * H + iy) * D + z0) * NB;
            for (int32_t i = lane; i < n * NB; i += 64)
                vol[base + i] = accumulate ? vol[base + i] + col[NB + i] : col[NB + i];
        } else {
            // slot a of z cell i is col[NB (i + 1) + a]; each slot's cell gets its own column
#pragma unroll
            for (int32_t a = 0; a < P; ++a) {
                int32_t cx, cy;
                orbit_cell(P, dir, W, H, ix, iy, a, cx, cy);
                const int64_t base = ((int64_t)cx * H + cy) * D + z0;
                for (int32_t i = lane; i < n; i += 64) {
                    const float v = col[NB * (i + 1) + a];
                    vol[base + i] = accumulate ? vol[base + i] + v : v;
                }
            }
        }
    }
}

// ------------------------------------------------------------------------------------------
// Layout conversion. DHW member m: element (z, y, x) at m*ms + (z*H + y)*W + x.
// Native: element (x, y, z, m) at ((x*H + y)*D + z)*NB + m.

template <int NB>
__global__ void __launch_bounds__(256) dhw_to_native_kernel(const float* __restrict__ in,
                                                            int64_t ms, int32_t D, int32_t H,
                                                            int32_t W, int32_t y0,
                                                            float* __restrict__ out) {
    __shared__ float tile[NB][32][33];
    const int32_t x0 = blockIdx.x * 32, z0 = blockIdx.y * 32, y = y0 + (int32_t)blockIdx.z;
    const int32_t tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
#pragma unroll
    for (int m = 0; m < NB; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int32_t z = z0 + ty + 8 * i, x = x0 + tx;
            if (z < D && x < W) tile[m][ty + 8 * i][tx] = in[m * ms + ((int64_t)z * H + y) * W + x];
        }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int32_t x = x0 + ty + 8 * i, z = z0 + tx;
        if (x < W && z < D) {
            const int64_t o = (((int64_t)x * H + y) * D + z) * NB;
#pragma unroll
            for (int m = 0; m < NB; ++m) out[o + m] = tile[m][tx][ty + 8 * i];
        }
    }
}

template <int NB>
__global__ void __launch_bounds__(256) native_to_dhw_kernel(const float* __restrict__ in,
                                                            int32_t D, int32_t H, int32_t W,
                                                            int32_t y0, float* __restrict__ out,
                                                            int64_t ms, int32_t accumulate) {
    __shared__ float tile[NB][32][33];
    const int32_t x0 = blockIdx.x * 32, z0 = blockIdx.y * 32, y = y0 + (int32_t)blockIdx.z;
    const int32_t tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int32_t x = x0 + ty + 8 * i, z = z0 + tx;
        if (x < W && z < D) {
            const int64_t o = (((int64_t)x * H + y) * D + z) * NB;
#pragma unroll
            for (int m = 0; m < NB; ++m) tile[m][tx][ty + 8 * i] = in[o + m];
        }
    }
    __syncthreads();
#pragma unroll
    for (int m = 0; m < NB; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int32_t z = z0 + ty + 8 * i, x = x0 + tx;
            if (z < D && x < W) {
                float* q = out + m * ms + ((int64_t)z * H + y) * W + x;
                const float v = tile[m][ty + 8 * i][tx];
                *q = accumulate ? *q + v : v;
            }
        }
}

// z-fastest member volumes <-> interleaved: element i of member m <-> native i*NB + m.
template <int NB>
__global__ void __launch_bounds__(256) interleave_kernel(const float* __restrict__ in, int64_t ms,
                                                         int64_t n, float* __restrict__ out) {
    for (int64_t i = blockIdx.x * 256ll + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
#pragma unroll
        for (int m = 0; m < NB; ++m) out[i * NB + m] = in[m * ms + i];
    }
}

template <int NB>
__global__ void __launch_bounds__(256) deinterleave_kernel(const float* __restrict__ in, int64_t n,
                                                           float* __restrict__ out, int64_t ms,
                                                           int32_t accumulate) {
    for (int64_t i = blockIdx.x * 256ll + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
#pragma unroll
        for (int m = 0; m < NB; ++m) {
            const float v = in[i * NB + m];
            float* q = out + m * ms + i;
            *q = accumulate ? *q + v : v;
        }
    }
}

__global__ void __launch_bounds__(256) fill_zero_kernel(float* __restrict__ p, int64_t n) {
    for (int64_t i = blockIdx.x * 256ll + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
        p[i] = 0.0f;
}

// Streaming copy, the bandwidth reference of the measurements and the kernel of known traffic
// that the byte counters are calibrated with: plain 16-byte loads and stores, the same kind of
// access as the walks' loads (nontemporal ones were no faster), grid-stride over a fixed grid
// (1024 blocks of 256 threads was the fastest of the grids tried on MI355X, 2 GiB copies),
// then the tail of fewer than 4 floats.
__global__ void __launch_bounds__(256) stream_copy_kernel(const float* __restrict__ in,
                                                          float* __restrict__ out, int64_t n) {
    const int64_t n4 = n >> 2;
    const float4* const in4 = reinterpret_cast<const float4*>(in);
    float4* const out4 = reinterpret_cast<float4*>(out);
    const int64_t stride = (int64_t)gridDim.x * 256;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += stride) out4[i] = in4[i];
    if (blockIdx.x == 0 && threadIdx.x < (n & 3)) out[4 * n4 + threadIdx.x] = in[4 * n4 + threadIdx.x];
}

constexpr int32_t kMaxGridYZ = 65535;

template <int NB>
hipError_t to_native_nb(const float* in, int64_t ms, int32_t D, int32_t H, int32_t W, int whd_in,
                        float* ws, hipStream_t s) {
    if (whd_in) {
        const int64_t n = (int64_t)D * H * W;
        const int64_t blocks = (n + 255) / 256 < 65536 ? (n + 255) / 256 : 65536;
        trace_launch("interleave_kernel", dim3((unsigned)blocks), dim3(256), 0, "members %d", NB);
        interleave_kernel<NB><<<dim3((unsigned)blocks), dim3(256), 0, s>>>(in, ms, n, ws);
        return hipGetLastError();
    }
    for (int32_t y0 = 0; y0 < H; y0 += kMaxGridYZ) {
        const int32_t ny = H - y0 < kMaxGridYZ ? H - y0 : kMaxGridYZ;
        dim3 grid((W + 31) / 32, (D + 31) / 32, ny);
        trace_launch("dhw_to_native_kernel", grid, dim3(256), 0, "members %d rows y %d..", NB, y0);
        dhw_to_native_kernel<NB><<<grid, dim3(256), 0, s>>>(in, ms, D, H, W, y0, ws);
    }
    return hipGetLastError();
}

template <int NB>
hipError_t from_native_nb(const float* ws, int32_t D, int32_t H, int32_t W, int whd_out, float* out,
                          int64_t ms, int accumulate, hipStream_t s) {
    if (whd_out) {
        const int64_t n = (int64_t)D * H * W;
        const int64_t blocks = (n + 255) / 256 < 65536 ? (n + 255) / 256 : 65536;
        trace_launch("deinterleave_kernel", dim3((unsigned)blocks), dim3(256), 0, "members %d", NB);
        deinterleave_kernel<NB><<<dim3((unsigned)blocks), dim3(256), 0, s>>>(ws, n, out, ms, accumulate);
        return hipGetLastError();
    }
    for (int32_t y0 = 0; y0 < H; y0 += kMaxGridYZ) {
        const int32_t ny = H - y0 < kMaxGridYZ ? H - y0 : kMaxGridYZ;
        dim3 grid((W + 31) / 32, (D + 31) / 32, ny);
        trace_launch("native_to_dhw_kernel", grid, dim3(256), 0, "members %d rows y %d..", NB, y0);
        native_to_dhw_kernel<NB><<<grid, dim3(256), 0, s>>>(ws, D, H, W, y0, out, ms, accumulate);
    }
    return hipGetLastError();
}

}  // namespace

// ------------------------------------------------------------------------------------------
// Launchers

// MBP_TRACE set (and not "0") in the environment: each launch prints its kernel, grid, block,
// dynamic LDS bytes and work range to stderr. Read at every launch, so it can be switched on
// while a process runs.
bool trace_on() {
    const char* e = std::getenv("MBP_TRACE");
    return e && e[0] && !(e[0] == '0' && e[1] == 0);
}

void trace_launch(const char* kernel, dim3 grid, dim3 block, size_t lds, const char* fmt, ...) {
    if (!trace_on()) return;
    char extra[256] = "";
    if (fmt && fmt[0]) {
        va_list ap;
        va_start(ap, fmt);
        vsnprintf(extra, sizeof(extra), fmt, ap);
        va_end(ap);
    }
    std::fprintf(stderr, "mbp-trace %s grid %u x %u x %u block %u lds %zu %s\n", kernel, grid.x, grid.y,
                 grid.z, block.x * block.y * block.z, lds, extra);
}

hipError_t launch_generic_forward(const GenericLaunch& a, const float* const* vol,
                                  float* const* sino, hipStream_t s, int orbit, int dir,
                                  int64_t slot_stride) {
    const int64_t n = (int64_t)a.nviews * a.rows * a.cols;
    if (n == 0) return hipSuccess;
    if (orbit != 1 && (a.nb != 1 || (orbit != 2 && orbit != 4) || a.box.n[0] % 2 != 0 ||
                       (orbit == 4 && a.box.n[0] != a.box.n[1])))
        return hipErrorInvalidValue;
    Ptrs4 v{};
    MPtrs4 o{};
    for (int m = 0; m < a.nb; ++m) { v.p[m] = vol[m]; o.p[m] = sino[m]; }
    // rows-fastest launches: one block per (view, 64-row block, 4 adjacent columns)
    const dim3 grid(a.rows_fast ? (unsigned)((int64_t)a.nviews * ((a.cols + 3) / 4) * ((a.rows + 63) / 64))
                                : (unsigned)((n + 255) / 256));
    trace_launch("generic_forward_kernel", grid, dim3(256), 0, "views %d..%d members %d orbit %d (turn %d)",
                 a.view0, a.view0 + a.nviews - 1, a.nb, orbit, dir);
    switch (orbit) {
        case 1: generic_forward_kernel<1><<<grid, dim3(256), 0, s>>>(a, v, o, slot_stride, dir); break;
        case 2: generic_forward_kernel<2><<<grid, dim3(256), 0, s>>>(a, v, o, slot_stride, dir); break;
        case 4: generic_forward_kernel<4><<<grid, dim3(256), 0, s>>>(a, v, o, slot_stride, dir); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_generic_adjoint(const GenericLaunch& a, const float* const* sino,
                                  float* const* vol, hipStream_t s) {
    const int64_t n = (int64_t)a.nviews * a.rows * a.cols;
    if (n == 0) return hipSuccess;
    Ptrs4 y{};
    MPtrs4 o{};
    for (int m = 0; m < a.nb; ++m) { y.p[m] = sino[m]; o.p[m] = vol[m]; }
    trace_launch("generic_adjoint_kernel", dim3((unsigned)((n + 255) / 256)), dim3(256), 0,
                 "views %d..%d members %d", a.view0, a.view0 + a.nviews - 1, a.nb);
    generic_adjoint_kernel<<<dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s>>>(a, y, o);
    return hipGetLastError();
}

hipError_t launch_column_forward(const ColumnLaunch& a, int nb, const float* vol,
                                 float* const* sino, hipStream_t s, int orbit, int dir,
                                 int64_t slot_stride) {
    if (a.tasks == 0) return hipSuccess;
    if (orbit != 1 && (nb != 1 || (orbit != 2 && orbit != 4) || a.box.n[0] % 2 != 0 ||
                       (orbit == 4 && a.box.n[0] != a.H)))
        return hipErrorInvalidValue;
    MPtrs4 o{};
    for (int m = 0; m < nb; ++m) o.p[m] = sino[m];
    const dim3 grid((unsigned)((int64_t)a.nviews * ((a.cols + 3) / 4) * a.row_blocks));
    const bool flat = (uint64_t)a.box.n[0] * (uint64_t)a.box.n[1] * (uint64_t)a.box.n[2] * (uint64_t)nb *
                          sizeof(float) < (1ull << 31);
    trace_launch(flat ? "column_forward_kernel<flat>" : "column_forward_kernel<resource per cell>", grid,
                 dim3(256), 0, "views %d..%d members %d orbit %d (turn %d)", a.view0, a.view0 + a.nviews - 1,
                 nb, orbit, dir);
#define MBP_FORWARD(NB_, FLAT_, P_) \
    if (nb == NB_ && flat == FLAT_ && orbit == P_) \
        column_forward_kernel<NB_, FLAT_, P_><<<grid, dim3(256), 0, s>>>(a, vol, o, slot_stride, dir)
    MBP_FORWARD(1, true, 1); else MBP_FORWARD(1, false, 1); else MBP_FORWARD(2, true, 1);
    else MBP_FORWARD(2, false, 1); else MBP_FORWARD(4, true, 1); else MBP_FORWARD(4, false, 1);
    else MBP_FORWARD(1, true, 2); else MBP_FORWARD(1, false, 2);
    else MBP_FORWARD(1, true, 4); else MBP_FORWARD(1, false, 4);
    else return hipErrorInvalidValue;
#undef MBP_FORWARD
    return hipGetLastError();
}

hipError_t launch_column_adjoint(const ColumnLaunch& a, int nb, const float* const* sino,
                                 float* vol, hipStream_t s) {
    if (a.tasks == 0) return hipSuccess;
    Ptrs4 y{};
    for (int m = 0; m < nb; ++m) y.p[m] = sino[m];
    const dim3 grid((a.tasks + 3) / 4);
    trace_launch("column_adjoint_kernel", grid, dim3(256), 0, "views %d..%d members %d", a.view0,
                 a.view0 + a.nviews - 1, nb);
    switch (nb) {
        case 1: column_adjoint_kernel<1><<<grid, dim3(256), 0, s>>>(a, y, vol); break;
        case 2: column_adjoint_kernel<2><<<grid, dim3(256), 0, s>>>(a, y, vol); break;
        case 4: column_adjoint_kernel<4><<<grid, dim3(256), 0, s>>>(a, y, vol); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_count(const GenericLaunch& a, unsigned long long* count, hipStream_t s) {
    const int64_t n = (int64_t)a.nviews * a.rows * a.cols;
    if (n == 0) return hipSuccess;
    const int64_t want = (n + 255) / 256;
    trace_launch("generic_count_kernel", dim3((unsigned)(want < 8192 ? want : 8192)), dim3(256), 0,
                 "views %d..%d", a.view0, a.view0 + a.nviews - 1);
    generic_count_kernel<<<dim3((unsigned)(want < 8192 ? want : 8192)), dim3(256), 0, s>>>(a, count);
    return hipGetLastError();
}

hipError_t launch_column_count(const ColumnLaunch& a, unsigned long long* count, hipStream_t s) {
    if (a.tasks == 0) return hipSuccess;
    trace_launch("column_count_kernel", dim3((a.tasks + 3) / 4), dim3(256), 0, "views %d..%d", a.view0,
                 a.view0 + a.nviews - 1);
    column_count_kernel<<<dim3((a.tasks + 3) / 4), dim3(256), 0, s>>>(a, count);
    return hipGetLastError();
}

hipError_t launch_sino_prepass(const ColumnLaunch& a, int nb, const float* const* sino, float* ysc,
                               hipStream_t s, int32_t mview) {
    if (a.nviews == 0) return hipSuccess;
    Ptrs4 y{};
    for (int m = 0; m < nb; ++m) y.p[m] = sino[m];
    const int32_t rows_pad = gather_rows_padded(a.rows);
    for (int32_t v0 = 0; v0 < a.nviews; v0 += 65535) {
        ColumnLaunch b = a;
        b.view0 = a.view0 + v0;
        b.nviews = a.nviews - v0 < 65535 ? a.nviews - v0 : 65535;
        const dim3 grid((a.cols + 31) / 32, (rows_pad + 31) / 32, b.nviews);
        float* const out = ysc + (int64_t)v0 * a.cols * rows_pad * nb;
        trace_launch("sino_prepass_kernel", grid, dim3(256), 0,
                     "views %d..%d members %d rows padded %d member views apart %d",
                     b.view0, b.view0 + b.nviews - 1, nb, rows_pad, mview);
        switch (nb) {
            case 1: sino_prepass_kernel<1><<<grid, dim3(256), 0, s>>>(b, y, rows_pad, mview, out); break;
            case 2: sino_prepass_kernel<2><<<grid, dim3(256), 0, s>>>(b, y, rows_pad, mview, out); break;
            case 4: sino_prepass_kernel<4><<<grid, dim3(256), 0, s>>>(b, y, rows_pad, mview, out); break;
            default: return hipErrorInvalidValue;
        }
    }
    return hipGetLastError();
}

int32_t gather_zchunk(int32_t D, int nb) {
    const int32_t cap = 2048 / nb;           // floats of LDS per wave: at most 8 KiB
    return D < cap ? D : cap;
}

hipError_t launch_column_lines(const ColumnLaunch& a, int32_t views, ColLine* lines, hipStream_t s) {
    const int64_t n = (int64_t)views * a.cols;
    if (n == 0) return hipSuccess;
    const int64_t want = (n + 255) / 256;
    trace_launch("column_line_kernel", dim3((unsigned)(want < 65536 ? want : 65536)), dim3(256), 0,
                 "views %d..%d", a.view0, a.view0 + views - 1);
    column_line_kernel<<<dim3((unsigned)(want < 65536 ? want : 65536)), dim3(256), 0, s>>>(a, views, lines);
    return hipGetLastError();
}

hipError_t launch_column_gather(const ColumnLaunch& a, int nb, const ColLine* lines, const float* ysc,
                                float* vol, int accumulate, hipStream_t s, int orbit, int dir) {
    const int32_t W = a.box.n[0], H = a.box.n[1], D = a.box.n[2];
    // an orbit's slots take the place of members: one member, orbit slots per cell
    if (orbit != 1 && (nb != 1 || (orbit != 2 && orbit != 4) || W % 2 != 0 ||
                       (orbit == 4 && H != W) || a.nviews % orbit != 0))
        return hipErrorInvalidValue;
    const int slots = orbit > 1 ? orbit : nb;
    const int32_t zchunk = gather_zchunk(D, slots);
    const int32_t nchunks = (D + zchunk - 1) / zchunk;
    int32_t Wr, Hr;
    orbit_grid(orbit, W, H, Wr, Hr);
    const uint64_t tasks = (uint64_t)Wr * (uint64_t)Hr * (uint64_t)nchunks;
    // tiles of 32 x 32 cells (of the orbits' grid for an orbit), else 16 x 32, else plain
    // y-fastest order; the kernel deals its blocks round-robin to the XCDs, so that all XCDs
    // work on one tile at a time and share its sinogram lines in the memory-side cache.
    // Measured against the earlier 8 x 8 orbit tiles (64 x 8 for one slot) with a contiguous
    // range of tiles per XCD: the 720-view 512^3 cone 90.0 -> 86.6 ms (64 x 64: 85.3), the
    // 360-view one 69.8 -> 68.1 (64 x 64: 68.6), the 256^3 cone 8.58 -> 7.85 (16 x 16: 7.90),
    // the helical batch 157.9 -> 130.1 ms (64 x 8: 132.0, 16 x 16: 130.9, 8 x 8: 133.7).
    const bool big = Wr % 32 == 0 && Hr % 32 == 0;
    const bool tiled = big || (Wr % 16 == 0 && Hr % 32 == 0);
    const int32_t tx = big ? 32 : tiled ? 16 : 1, ty = tiled ? 32 : Hr;
    if (tasks == 0) return hipSuccess;
    const dim3 grid((unsigned)((tasks + 3) / 4));
    const size_t lds = (size_t)4 * (kQueue * sizeof(GatherItem) +
                                    (size_t)gather_column_floats(zchunk, slots) * sizeof(float));
    const int32_t kr = gather_rows_loaded(gather_stride(a.rows));
    trace_launch("column_gather_kernel", grid, dim3(256), lds,
                 "views %d..%d members %d orbit %d (turn %d) rows per lane %d z chunk %d tiles %d x %d",
                 a.view0, a.view0 + a.nviews - 1, nb, orbit, dir, kr, zchunk, tx, ty);
#define MBP_GATHER(NB_, KR_, P_) \
    if (slots == NB_ && kr == KR_ && orbit == P_) \
        column_gather_kernel<NB_, KR_, P_><<<grid, dim3(256), lds, s>>>(a, lines, ysc, vol, zchunk, nchunks, tx, ty, accumulate, dir)
    MBP_GATHER(1, 1, 1); else MBP_GATHER(1, 2, 1); else MBP_GATHER(1, 4, 1); else MBP_GATHER(1, 6, 1); else MBP_GATHER(1, 8, 1);
    else MBP_GATHER(2, 1, 1); else MBP_GATHER(2, 2, 1); else MBP_GATHER(2, 4, 1); else MBP_GATHER(2, 6, 1); else MBP_GATHER(2, 8, 1);
    else MBP_GATHER(4, 1, 1); else MBP_GATHER(4, 2, 1); else MBP_GATHER(4, 4, 1); else MBP_GATHER(4, 6, 1); else MBP_GATHER(4, 8, 1);
    else MBP_GATHER(2, 1, 2); else MBP_GATHER(2, 2, 2); else MBP_GATHER(2, 4, 2); else MBP_GATHER(2, 6, 2); else MBP_GATHER(2, 8, 2);
    else MBP_GATHER(4, 1, 4); else MBP_GATHER(4, 2, 4); else MBP_GATHER(4, 4, 4); else MBP_GATHER(4, 6, 4); else MBP_GATHER(4, 8, 4);
    else return hipErrorInvalidValue;
#undef MBP_GATHER
    return hipGetLastError();
}

hipError_t launch_tilt_gather(const ColumnLaunch& a, int nb, const float* ysc, float* vol, int accumulate,
                              hipStream_t s, int orbit, int dir) {
    const int32_t W = a.box.n[0], H = a.box.n[1], D = a.box.n[2];
    if (orbit != 1 && (nb != 1 || (orbit != 2 && orbit != 4) || W % 2 != 0 ||
                       (orbit == 4 && H != W) || a.nviews % orbit != 0))
        return hipErrorInvalidValue;
    const int slots = orbit > 1 ? orbit : nb;
    const int32_t zchunk = gather_zchunk(D, slots);
    const int32_t nchunks = (D + zchunk - 1) / zchunk;
    int32_t Wr, Hr;
    orbit_grid(orbit, W, H, Wr, Hr);
    const uint64_t tasks = (uint64_t)Wr * (uint64_t)Hr * (uint64_t)nchunks;
    // tiles of 32 x 32 cells, as in the column gather (the tilted 256^3 cone: 31.9 ms, against
    // 32.2 with 8 x 8 and 33.5 with 16 x 32), else 16 x 32, else plain y-fastest order
    const bool big = Wr % 32 == 0 && Hr % 32 == 0;
    const bool tiled = big || (Wr % 16 == 0 && Hr % 32 == 0);
    const int32_t tx = big ? 32 : tiled ? 16 : 1, ty = tiled ? 32 : Hr;
    if (tasks == 0) return hipSuccess;
    const dim3 grid((unsigned)((tasks + 3) / 4));
    const size_t lds = (size_t)4 * (kTiltQueue * sizeof(TiltItem) +
                                    (size_t)gather_column_floats(zchunk, slots) * sizeof(float));
    trace_launch("tilt_gather_kernel", grid, dim3(256), lds,
                 "views %d..%d members %d orbit %d (turn %d) z chunk %d tiles %d x %d",
                 a.view0, a.view0 + a.nviews - 1, nb, orbit, dir, zchunk, tx, ty);
#define MBP_TILT(NB_, P_) \
    if (slots == NB_ && orbit == P_) \
        tilt_gather_kernel<NB_, P_><<<grid, dim3(256), lds, s>>>(a, ysc, vol, zchunk, nchunks, tx, ty, accumulate, dir)
    MBP_TILT(1, 1); else MBP_TILT(2, 1); else MBP_TILT(4, 1); else MBP_TILT(2, 2); else MBP_TILT(4, 4);
    else return hipErrorInvalidValue;
#undef MBP_TILT
    return hipGetLastError();
}

hipError_t launch_to_native(const float* in, int64_t ms, int nb, int32_t D, int32_t H, int32_t W,
                            int whd_in, float* ws, hipStream_t s) {
    switch (nb) {
        case 1: return to_native_nb<1>(in, ms, D, H, W, whd_in, ws, s);
        case 2: return to_native_nb<2>(in, ms, D, H, W, whd_in, ws, s);
        case 4: return to_native_nb<4>(in, ms, D, H, W, whd_in, ws, s);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_from_native(const float* ws, int nb, int32_t D, int32_t H, int32_t W, int whd_out,
                              float* out, int64_t ms, int accumulate, hipStream_t s) {
    switch (nb) {
        case 1: return from_native_nb<1>(ws, D, H, W, whd_out, out, ms, accumulate, s);
        case 2: return from_native_nb<2>(ws, D, H, W, whd_out, out, ms, accumulate, s);
        case 4: return from_native_nb<4>(ws, D, H, W, whd_out, out, ms, accumulate, s);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_convert(const float* in, int32_t D, int32_t H, int32_t W, int to_whd, float* out,
                          hipStream_t s) {
    if (to_whd) return to_native_nb<1>(in, 0, D, H, W, 0, out, s);
    return from_native_nb<1>(in, D, H, W, 0, out, 0, 0, s);
}

hipError_t launch_stream_copy(const float* in, float* out, int64_t n, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    const int64_t want = (n / 4 + 255) / 256;
    trace_launch("stream_copy_kernel", dim3((unsigned)(want < 1024 ? (want > 0 ? want : 1) : 1024)), dim3(256), 0,
                 "floats %lld", (long long)n);
    stream_copy_kernel<<<dim3((unsigned)(want < 1024 ? (want > 0 ? want : 1) : 1024)), dim3(256), 0, s>>>(in, out, n);
    return hipGetLastError();
}

hipError_t launch_fill_zero(float* p, int64_t n, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    const int64_t want = (n + 255) / 256;
    trace_launch("fill_zero_kernel", dim3((unsigned)(want < 65536 ? want : 65536)), dim3(256), 0, "floats %lld",
                 (long long)n);
    fill_zero_kernel<<<dim3((unsigned)(want < 65536 ? want : 65536)), dim3(256), 0, s>>>(p, n);
    return hipGetLastError();
}

}  // namespace mbp
