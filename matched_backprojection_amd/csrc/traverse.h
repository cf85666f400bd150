// traverse.h -- ray setup and cell traversal for the ray-driven X-ray transform pair.
//
// Model (diffct pages, "diffct 2.1.0 -> 2.2.1", README "Why diffct", bullet "Matched
// operators"): the forward value of a ray is the line integral of the cell-constant volume,
// sum over voxels of (physical length inside the voxel) x (voxel value); the backprojector is
// its exact transpose and so walks exactly the same segments.
//
// Precision scheme (diffct pages, "diffct 2.2.1 -> 2.3.0", CHANGELOG 2.3.0, "Added": rays are
// clipped and their entries located in FP64, and the FP32 traversal measures distances from
// each entry): everything up to the entry point, the entry cell and the per-axis crossing
// counts is fp64; the walk itself is fp32, with every crossing distance taken as
// first + k * step by one fma from fp64-rounded constants (never a running sum), measured
// from the fp64 entry point, so distant endpoints keep voxel-sized resolution.
//
// Two walks share the per-axis setup:
//  * the generic walk, one ray at a time, in 3-D (2-D beams run with a single z cell);
//  * the column walk, for flat detectors whose row axis is parallel to z: every row of one
//    detector column then projects to the same line in the xy plane, so the xy cell sequence
//    is shared by the whole column and each ray only adds its own z crossings inside each xy
//    cell (the z-inner stepping of "diffct 2.2.1 -> 2.4.0", CHANGELOG 2.4.0, "Changed").
//
// The header compiles for the GPU (hipcc) and for the host (g++); the host build is used by
// a CPU harness that replays the walks with bounds checks.
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#include <hip/hip_runtime.h>
#define MBP_HD __host__ __device__
#define MBP_INLINE __forceinline__
#else
#include <math.h>
#define MBP_HD
#define MBP_INLINE inline
#endif

namespace mbp {

enum { BEAM_PARALLEL = 0, BEAM_FAN = 1, BEAM_CONE = 2 };

// Per-view frame, staged once per plan (fp64). For 2-D beams z components are fixed:
// src.z = det.z = centre z, eu.z = 0, ev = 0.
struct Frame {
    double s[3];   // source (fan/cone) or ray direction (parallel)
    double c[3];   // detector centre
    double u[3];   // detector axis along columns (one pixel = du * u)
    double v[3];   // detector axis along rows    (one pixel = dv * v)
};

// Volume box in world axis order (x <-> W, y <-> H, z <-> D).
struct Box {
    double lo[3];
    double hi[3];
    double pitch[3];
    int32_t n[3];
};

// One axis of a walk: cells are entered at c0, then `steps` crossings follow, each moving
// one cell in direction `step`; the k-th crossing (k = 0..steps-1) lies at distance
// t_first + k * t_step from the entry point.
struct AxisWalk {
    int32_t c0;
    int32_t step;
    int32_t steps;
    float t_first;
    float t_step;
};

MBP_HD MBP_INLINE int32_t clamp_cell(double s, int32_t n) {
    if (!(s >= 0.0)) return 0;           // also catches NaN
    if (s >= (double)(n - 1)) return n - 1;
    return (int32_t)s;
}

// The cell a ray occupies just after position `s` (in units of pitch from the box low face)
// when moving in direction `w`: on a plane, a decreasing ray is already in the cell below;
// otherwise (and for w == 0, half-open cells) the cell is floor(s).
MBP_HD MBP_INLINE int32_t cell_after(double s, double w, int32_t n) {
    double f = floor(s);
    if (w < 0.0 && f == s) f -= 1.0;
    return clamp_cell(f, n);
}

// The cell a ray occupies just before position `s` when moving in direction `w`.
MBP_HD MBP_INLINE int32_t cell_before(double s, double w, int32_t n) {
    double f = floor(s);
    if (w > 0.0 && f == s) f -= 1.0;
    return clamp_cell(f, n);
}

// Walk of one axis from world coordinate `e` (the entry point) to `x` (the exit point);
// `w` is the world displacement along this axis per unit of walk distance; `t0` is the walk
// distance of `e` (added to every crossing distance).
// Crossing constants are kept finite (|value| <= 1e28, so first + k * step with k < 2^31
// cannot overflow): an axis with crossings left then always has a finite next distance and is
// chosen before any exhausted axis (whose next distance is +inf). That is what keeps every
// visited cell between the clamped entry and exit cells, whatever the rounding.
MBP_HD MBP_INLINE float finite_distance(double t) {
    return (float)(t > 1e28 ? 1e28 : (t < -1e28 ? -1e28 : t));
}

MBP_HD MBP_INLINE AxisWalk axis_walk(double e, double x, double w, double t0, double lo,
                                     double pitch, int32_t n) {
    AxisWalk a;
    const double se = (e - lo) / pitch;
    const double sx = (x - lo) / pitch;
    a.c0 = cell_after(se, w, n);
    if (w > 0.0) {
        const int32_t c1 = cell_before(sx, w, n);
        a.step = 1;
        a.steps = c1 > a.c0 ? c1 - a.c0 : 0;
        const double plane = lo + (double)(a.c0 + 1) * pitch;
        a.t_first = finite_distance(t0 + (plane - e) / w);
        a.t_step = finite_distance(pitch / w);
    } else if (w < 0.0) {
        const int32_t c1 = cell_before(sx, w, n);
        a.step = -1;
        a.steps = a.c0 > c1 ? a.c0 - c1 : 0;
        const double plane = lo + (double)a.c0 * pitch;
        a.t_first = finite_distance(t0 + (plane - e) / w);
        a.t_step = finite_distance(-pitch / w);
    } else {
        a.step = 0;
        a.steps = 0;
        a.t_first = INFINITY;
        a.t_step = 0.0f;
    }
    return a;
}

// Clip the parameter range [t0, t1] of the line a + t d to the half-open slab [lo, hi) on
// the axes 0..rank-1. Returns false when nothing of positive length remains.
MBP_HD MBP_INLINE bool clip_slab(const double* a, const double* d, const double* lo,
                                 const double* hi, int rank, double& t0, double& t1) {
    for (int k = 0; k < rank; ++k) {
        if (d[k] != 0.0) {
            const double s1 = (lo[k] - a[k]) / d[k];
            const double s2 = (hi[k] - a[k]) / d[k];
            const double smin = s1 < s2 ? s1 : s2;
            const double smax = s1 < s2 ? s2 : s1;
            if (smin > t0) t0 = smin;
            if (smax < t1) t1 = smax;
        } else if (a[k] < lo[k] || a[k] >= hi[k]) {
            return false;
        }
    }
    return t1 > t0;
}

// Pixel (row k, col j) world position: det + u_j eu + v_k ev with centred u_j, v_k.
MBP_HD MBP_INLINE void pixel_point(const Frame& F, double u, double v, double* p) {
    for (int a = 0; a < 3; ++a) p[a] = F.c[a] + u * F.u[a] + v * F.v[a];
}

MBP_HD MBP_INLINE double centred(int32_t i, int32_t n, double pitch) {
    return ((double)i - 0.5 * (double)(n - 1)) * pitch;
}

// ------------------------------------------------------------------------------------------
// Generic walk: one ray in 3-D.

struct RayWalk {
    AxisWalk ax[3];
    float T;        // physical length inside the box
    int32_t hit;
};

MBP_HD MBP_INLINE void ray_setup(const Frame& F, const Box& B, int beam, double u, double v,
                                 RayWalk& r) {
    double p[3];
    pixel_point(F, u, v, p);
    double a[3], d[3];
    double t0, t1;
    if (beam == BEAM_PARALLEL) {
        for (int k = 0; k < 3; ++k) { a[k] = p[k]; d[k] = F.s[k]; }
        t0 = -INFINITY; t1 = INFINITY;
    } else {
        for (int k = 0; k < 3; ++k) { a[k] = F.s[k]; d[k] = p[k] - F.s[k]; }
        t0 = 0.0; t1 = 1.0;
    }
    r.hit = clip_slab(a, d, B.lo, B.hi, 3, t0, t1) ? 1 : 0;
    if (!r.hit) {
        r.T = 0.0f;
        for (int k = 0; k < 3; ++k) { r.ax[k].c0 = 0; r.ax[k].step = 0; r.ax[k].steps = 0;
                                      r.ax[k].t_first = INFINITY; r.ax[k].t_step = 0.0f; }
        return;
    }
    const double dn = sqrt(d[0] * d[0] + d[1] * d[1] + d[2] * d[2]);
    for (int k = 0; k < 3; ++k) {
        const double e = a[k] + t0 * d[k];
        const double x = a[k] + t1 * d[k];
        r.ax[k] = axis_walk(e, x, d[k] / dn, 0.0, B.lo[k], B.pitch[k], B.n[k]);
    }
    r.T = (float)((t1 - t0) * dn);
}

// Visit the segments of a generic walk. `visit(cx, cy, cz, length)` once per segment, in
// order along the ray; lengths are physical.
template <class Visit>
MBP_HD MBP_INLINE void walk_ray(const RayWalk& r, Visit& visit) {
    if (!r.hit) return;
    int32_t cx = r.ax[0].c0, cy = r.ax[1].c0, cz = r.ax[2].c0;
    int32_t kx = 0, ky = 0, kz = 0;
    float nx = r.ax[0].steps > 0 ? r.ax[0].t_first : INFINITY;
    float ny = r.ax[1].steps > 0 ? r.ax[1].t_first : INFINITY;
    float nz = r.ax[2].steps > 0 ? r.ax[2].t_first : INFINITY;
    const int32_t total = r.ax[0].steps + r.ax[1].steps + r.ax[2].steps;
    float t = 0.0f;
    for (int32_t m = 0; m < total; ++m) {
        const bool bx = nx <= ny && nx <= nz;
        const bool by = !bx && ny <= nz;
        const float tb = bx ? nx : (by ? ny : nz);
        visit(cx, cy, cz, fmaxf(tb - t, 0.0f));
        t = fmaxf(t, tb);
        if (bx) {
            cx += r.ax[0].step; ++kx;
            nx = kx < r.ax[0].steps ? fmaf((float)kx, r.ax[0].t_step, r.ax[0].t_first) : INFINITY;
        } else if (by) {
            cy += r.ax[1].step; ++ky;
            ny = ky < r.ax[1].steps ? fmaf((float)ky, r.ax[1].t_step, r.ax[1].t_first) : INFINITY;
        } else {
            cz += r.ax[2].step; ++kz;
            nz = kz < r.ax[2].steps ? fmaf((float)kz, r.ax[2].t_step, r.ax[2].t_first) : INFINITY;
        }
    }
    visit(cx, cy, cz, fmaxf(r.T - t, 0.0f));
}

// ------------------------------------------------------------------------------------------
// Column walk: the rows of one column share their xy line.
//
// Walk distance `tau` is the arc length along the xy projection, measured from the fp64 xy
// entry point of the column's line into the box. A ray of the column then sits at
// z(tau) = z_entry + tau * (dz / |d_xy|), and a piece [tau_a, tau_b] of it is
// (tau_b - tau_a) * kappa long in 3-D, kappa = |d| / |d_xy|.

struct ColumnWalk {                  // shared by all rows of a column
    AxisWalk x, y;
    float T;                         // xy length inside the box's xy rectangle
    int32_t hit;
    double Txy;                      // the same length in fp64
    // kept for the row setup (fp64)
    double t_in;                     // ray parameter of the xy entry
    double dxy;                      // |d_xy|
    double sz, dz_col;               // source z (or pixel z for lines) and column z offset
    int32_t line;                    // 1: infinite line (parallel), 0: segment
    double t_lo, t_hi;               // parameter limits of the ray (segment: [0, 1])
};

struct RowWalk {                     // one row of the column
    AxisWalk z;
    float t_lo, t_hi;                // active tau range of this row (empty if t_hi <= t_lo)
    float kappa;
};

// Setup shared by a column. Returns hit = 0 when the column's xy line misses the box, and
// also when the line is degenerate (|d_xy| == 0: the plan rejects such geometry for this
// walk).
MBP_HD MBP_INLINE void column_setup(const Frame& F, const Box& B, int beam, double u,
                                    ColumnWalk& c) {
    double p[3];
    pixel_point(F, u, 0.0, p);           // v-independent part (ev has no xy component)
    double a[2], d[2];
    double t0, t1;
    if (beam == BEAM_PARALLEL) {
        a[0] = p[0]; a[1] = p[1]; d[0] = F.s[0]; d[1] = F.s[1];
        t0 = -INFINITY; t1 = INFINITY;
        c.line = 1;
        c.sz = p[2];
        c.dz_col = F.s[2];
    } else {
        a[0] = F.s[0]; a[1] = F.s[1]; d[0] = p[0] - F.s[0]; d[1] = p[1] - F.s[1];
        t0 = 0.0; t1 = 1.0;
        c.line = 0;
        c.sz = F.s[2];
        c.dz_col = p[2] - F.s[2];
    }
    c.t_lo = t0; c.t_hi = t1;
    c.dxy = sqrt(d[0] * d[0] + d[1] * d[1]);
    c.hit = (c.dxy > 0.0 && clip_slab(a, d, B.lo, B.hi, 2, t0, t1)) ? 1 : 0;
    c.t_in = t0;
    if (!c.hit) {
        c.T = 0.0f;
        c.Txy = 0.0;
        c.x.c0 = c.y.c0 = 0; c.x.step = c.y.step = 0; c.x.steps = c.y.steps = 0;
        c.x.t_first = c.y.t_first = INFINITY; c.x.t_step = c.y.t_step = 0.0f;
        return;
    }
    const double ex = a[0] + t0 * d[0], ey = a[1] + t0 * d[1];
    const double xx = a[0] + t1 * d[0], xy = a[1] + t1 * d[1];
    c.x = axis_walk(ex, xx, d[0] / c.dxy, 0.0, B.lo[0], B.pitch[0], B.n[0]);
    c.y = axis_walk(ey, xy, d[1] / c.dxy, 0.0, B.lo[1], B.pitch[1], B.n[1]);
    c.Txy = (t1 - t0) * c.dxy;
    c.T = (float)c.Txy;
}

// Row setup: `v` is the row's detector coordinate, `evz` the z component of the row axis.
MBP_HD MBP_INLINE void row_setup(const ColumnWalk& c, const Box& B, double v, double evz,
                                 RowWalk& r) {
    r.t_lo = 0.0f; r.t_hi = 0.0f; r.kappa = 0.0f;
    r.z.c0 = 0; r.z.step = 0; r.z.steps = 0; r.z.t_first = INFINITY; r.z.t_step = 0.0f;
    if (!c.hit) return;
    const double dz = c.line ? c.dz_col : c.dz_col + v * evz;   // z change per unit parameter
    const double z0 = c.line ? c.sz + v * evz : c.sz;           // z at parameter 0
    const double wz = dz / c.dxy;                                // z change per unit tau
    const double z_in = z0 + c.t_in * dz;                        // z at tau = 0
    // tau range where lo_z <= z < hi_z, intersected with the column's xy range [0, Txy]
    double tlo = 0.0, thi = c.Txy;
    if (wz != 0.0) {
        const double s1 = (B.lo[2] - z_in) / wz;
        const double s2 = (B.hi[2] - z_in) / wz;
        const double smin = s1 < s2 ? s1 : s2, smax = s1 < s2 ? s2 : s1;
        if (smin > tlo) tlo = smin;
        if (smax < thi) thi = smax;
    } else if (z_in < B.lo[2] || z_in >= B.hi[2]) {
        return;
    }
    if (!(thi > tlo)) return;
    r.z = axis_walk(z_in + tlo * wz, z_in + thi * wz, wz, tlo, B.lo[2], B.pitch[2], B.n[2]);
    r.t_lo = (float)tlo;
    r.t_hi = (float)thi;
    r.kappa = (float)(sqrt(c.dxy * c.dxy + dz * dz) / c.dxy);
}

// Visit the segments of one row of a column walk, in order: `visit(cx, cy, cz, length)`,
// lengths in units of tau (multiply by kappa for physical length). The xy loop is the same
// for every row of the column; each row adds its own z crossings inside each xy cell.
template <class Visit>
MBP_HD MBP_INLINE void walk_column_row(const ColumnWalk& c, const RowWalk& r, Visit& visit) {
    if (!c.hit) return;
    int32_t cx = c.x.c0, cy = c.y.c0;
    int32_t kx = 0, ky = 0;
    float nx = c.x.steps > 0 ? c.x.t_first : INFINITY;
    float ny = c.y.steps > 0 ? c.y.t_first : INFINITY;
    const int32_t total = c.x.steps + c.y.steps;
    int32_t cz = r.z.c0, kz = 0;
    float nz = r.z.steps > 0 ? r.z.t_first : INFINITY;
    float ta = 0.0f;
    for (int32_t m = 0; m <= total; ++m) {
        const bool last = m == total;
        const bool bx = !last && nx <= ny;
        const float tb = last ? c.T : (bx ? nx : ny);
        float lo = fmaxf(ta, r.t_lo);
        const float hi = fminf(tb, r.t_hi);
        if (lo < hi) {
            while (nz < hi) {
                visit(cx, cy, cz, fmaxf(nz - lo, 0.0f));
                lo = fmaxf(lo, nz);
                cz += r.z.step; ++kz;
                nz = kz < r.z.steps ? fmaf((float)kz, r.z.t_step, r.z.t_first) : INFINITY;
            }
            visit(cx, cy, cz, hi - lo);
        }
        ta = fmaxf(ta, tb);
        if (last) break;
        if (bx) {
            cx += c.x.step; ++kx;
            nx = kx < c.x.steps ? fmaf((float)kx, c.x.t_step, c.x.t_first) : INFINITY;
        } else {
            cy += c.y.step; ++ky;
            ny = ky < c.y.steps ? fmaf((float)ky, c.y.t_step, c.y.t_first) : INFINITY;
        }
    }
}

}  // namespace mbp
