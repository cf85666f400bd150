// traverse.h -- ray setup and cell traversal for the ray-driven X-ray transform pair.
//
// Model (diffct pages, "diffct 2.1.0 -> 2.2.1", README "Why diffct", bullet "Matched
// operators"): the forward value of a ray is the line integral of the cell-constant volume,
// sum over voxels of (physical length inside the voxel) x (voxel value); the backprojector is
// its exact transpose and so walks exactly the same segments.
//
// Precision scheme. The diffct pages ("diffct 2.2.1 -> 2.3.0", CHANGELOG 2.3.0, "Added") clip
// rays and locate their entries in FP64 and let an FP32 walk measure distances from each
// entry. Here the entry point, entry cell and per-axis crossing counts are fp64 as there, and
// every crossing distance is first + k * step (one fma from the fp64 constants, never a
// running sum) measured from the fp64 entry point; the distances themselves are also kept in
// fp64, because an fp32 distance carries an absolute error of about ulp(box chord), which is
// large against the short chords of grazing rays (it broke the 1e-4 per-ray bound). On
// gfx950 an fp64 fma issues at the same rate as an unpacked fp32 one, so this costs
// registers, not throughput. Voxel values, sinogram values and sums stay fp32.
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
    int32_t pad_;
    double t_first;
    double t_step;
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
// Crossing constants are kept finite (|value| <= 1e280, so first + k * step with k < 2^31
// cannot overflow): an axis with crossings left then always has a finite next distance and is
// chosen before any exhausted axis (whose next distance is +inf). That is what keeps every
// visited cell between the clamped entry and exit cells, whatever the rounding.
MBP_HD MBP_INLINE double finite_distance(double t) {
    return t > 1e280 ? 1e280 : (t < -1e280 ? -1e280 : t);
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
        a.t_step = 0.0;
    }
    a.pad_ = 0;
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
    double T;       // physical length inside the box
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
    // both outcomes fill locals that are stored once (see column_setup)
    AxisWalk w[3];
    double T = 0.0;
#pragma unroll
    for (int k = 0; k < 3; ++k) w[k] = AxisWalk{0, 0, 0, 0, INFINITY, 0.0};
    if (r.hit) {
        const double dn = sqrt(d[0] * d[0] + d[1] * d[1] + d[2] * d[2]);
#pragma unroll
        for (int k = 0; k < 3; ++k) {
            const double e = a[k] + t0 * d[k];
            const double x = a[k] + t1 * d[k];
            w[k] = axis_walk(e, x, d[k] / dn, 0.0, B.lo[k], B.pitch[k], B.n[k]);
        }
        T = (t1 - t0) * dn;
    }
#pragma unroll
    for (int k = 0; k < 3; ++k) r.ax[k] = w[k];
    r.T = T;
}

// Visit the segments of a generic walk. `visit(cx, cy, cz, length)` once per segment, in
// order along the ray; lengths are physical.
template <class Visit>
MBP_HD MBP_INLINE void walk_ray(const RayWalk& r, Visit& visit) {
    if (!r.hit) return;
    int32_t cx = r.ax[0].c0, cy = r.ax[1].c0, cz = r.ax[2].c0;
    int32_t kx = 0, ky = 0, kz = 0;
    double nx = r.ax[0].steps > 0 ? r.ax[0].t_first : INFINITY;
    double ny = r.ax[1].steps > 0 ? r.ax[1].t_first : INFINITY;
    double nz = r.ax[2].steps > 0 ? r.ax[2].t_first : INFINITY;
    const int32_t total = r.ax[0].steps + r.ax[1].steps + r.ax[2].steps;
    double t = 0.0;
    for (int32_t m = 0; m < total; ++m) {
        const bool bx = nx <= ny && nx <= nz;
        const bool by = !bx && ny <= nz;
        const double tb = bx ? nx : (by ? ny : nz);
        visit(cx, cy, cz, (float)fmax(tb - t, 0.0));
        t = fmax(t, tb);
        if (bx) {
            cx += r.ax[0].step; ++kx;
            nx = kx < r.ax[0].steps ? fma((double)kx, r.ax[0].t_step, r.ax[0].t_first) : INFINITY;
        } else if (by) {
            cy += r.ax[1].step; ++ky;
            ny = ky < r.ax[1].steps ? fma((double)ky, r.ax[1].t_step, r.ax[1].t_first) : INFINITY;
        } else {
            cz += r.ax[2].step; ++kz;
            nz = kz < r.ax[2].steps ? fma((double)kz, r.ax[2].t_step, r.ax[2].t_first) : INFINITY;
        }
    }
    visit(cx, cy, cz, (float)fmax(r.T - t, 0.0));
}

// walk_ray with the cell given as its element offset cx * sx + cy * sy + cz * sz, kept by one
// add per crossing (the offset of every visited cell fits 32 bits: the volume has fewer than
// 2^31 elements): `visit(offset, length)` once per segment, in order along the ray.
template <class Visit>
MBP_HD MBP_INLINE void walk_ray_offsets(const RayWalk& r, int32_t sx, int32_t sy, int32_t sz, Visit& visit) {
    if (!r.hit) return;
    int32_t off = r.ax[0].c0 * sx + r.ax[1].c0 * sy + r.ax[2].c0 * sz;
    const int32_t dx = r.ax[0].step * sx, dy = r.ax[1].step * sy, dz = r.ax[2].step * sz;
    int32_t kx = 0, ky = 0, kz = 0;
    double nx = r.ax[0].steps > 0 ? r.ax[0].t_first : INFINITY;
    double ny = r.ax[1].steps > 0 ? r.ax[1].t_first : INFINITY;
    double nz = r.ax[2].steps > 0 ? r.ax[2].t_first : INFINITY;
    const int32_t total = r.ax[0].steps + r.ax[1].steps + r.ax[2].steps;
    double t = 0.0;
    for (int32_t m = 0; m < total; ++m) {
        const bool bx = nx <= ny && nx <= nz;
        const bool by = !bx && ny <= nz;
        const double tb = bx ? nx : (by ? ny : nz);
        visit(off, (float)fmax(tb - t, 0.0));
        t = fmax(t, tb);
        off += bx ? dx : (by ? dy : dz);
        if (bx) {
            ++kx;
            nx = kx < r.ax[0].steps ? fma((double)kx, r.ax[0].t_step, r.ax[0].t_first) : INFINITY;
        } else if (by) {
            ++ky;
            ny = ky < r.ax[1].steps ? fma((double)ky, r.ax[1].t_step, r.ax[1].t_first) : INFINITY;
        } else {
            ++kz;
            nz = kz < r.ax[2].steps ? fma((double)kz, r.ax[2].t_step, r.ax[2].t_first) : INFINITY;
        }
    }
    visit(off, (float)fmax(r.T - t, 0.0));
}

// walk_ray_offsets for the rays a turn symmetry of the views relates (orbit_cell): the cell
// (cx, cy, cz) of the walked ray stands for cell R^m (cx, cy) at the same cz for the ray m steps
// of the turn later, whose element offset is base[m] + cx * tx[m] + cy * ty[m] + cz * sz
// (orbit_strides). `visit(offsets, length)` gets the P offsets of each segment.
template <int P, class Visit>
MBP_HD MBP_INLINE void walk_ray_orbit(const RayWalk& r, const int32_t (&base)[P], const int32_t (&tx)[P],
                                      const int32_t (&ty)[P], int32_t sz, Visit& visit) {
    if (!r.hit) return;
    int32_t off[P], dx[P], dy[P];
    for (int m = 0; m < P; ++m) {
        off[m] = base[m] + r.ax[0].c0 * tx[m] + r.ax[1].c0 * ty[m] + r.ax[2].c0 * sz;
        dx[m] = r.ax[0].step * tx[m];
        dy[m] = r.ax[1].step * ty[m];
    }
    const int32_t dz = r.ax[2].step * sz;
    int32_t kx = 0, ky = 0, kz = 0;
    double nx = r.ax[0].steps > 0 ? r.ax[0].t_first : INFINITY;
    double ny = r.ax[1].steps > 0 ? r.ax[1].t_first : INFINITY;
    double nz = r.ax[2].steps > 0 ? r.ax[2].t_first : INFINITY;
    const int32_t total = r.ax[0].steps + r.ax[1].steps + r.ax[2].steps;
    double t = 0.0;
    for (int32_t i = 0; i < total; ++i) {
        const bool bx = nx <= ny && nx <= nz;
        const bool by = !bx && ny <= nz;
        const double tb = bx ? nx : (by ? ny : nz);
        visit(off, (float)fmax(tb - t, 0.0));
        t = fmax(t, tb);
        for (int m = 0; m < P; ++m) off[m] += bx ? dx[m] : (by ? dy[m] : dz);
        if (bx) {
            ++kx;
            nx = kx < r.ax[0].steps ? fma((double)kx, r.ax[0].t_step, r.ax[0].t_first) : INFINITY;
        } else if (by) {
            ++ky;
            ny = ky < r.ax[1].steps ? fma((double)ky, r.ax[1].t_step, r.ax[1].t_first) : INFINITY;
        } else {
            ++kz;
            nz = kz < r.ax[2].steps ? fma((double)kz, r.ax[2].t_step, r.ax[2].t_first) : INFINITY;
        }
    }
    visit(off, (float)fmax(r.T - t, 0.0));
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
    double T;                        // xy length inside the box's xy rectangle
    int32_t hit;
    // kept for the row setup (fp64)
    double t_in;                     // ray parameter of the xy entry
    double dxy;                      // |d_xy|
    double sz, dz_col;               // source z (or pixel z for lines) and column z offset
    int32_t line;                    // 1: infinite line (parallel), 0: segment
    double t_lo, t_hi;               // parameter limits of the ray (segment: [0, 1])
};

struct RowWalk {                     // one row of the column
    AxisWalk z;
    double t_lo, t_hi;               // active tau range of this row (empty if t_hi <= t_lo)
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
    // both outcomes fill locals that are stored once (stores to the struct's fields in two
    // branches were merged by the device compiler into one store through a chosen pointer,
    // which kept the struct in scratch memory)
    AxisWalk wx = {0, 0, 0, 0, INFINITY, 0.0}, wy = wx;
    double T = 0.0;
    if (c.hit) {
        const double ex = a[0] + t0 * d[0], ey = a[1] + t0 * d[1];
        const double xx = a[0] + t1 * d[0], xy = a[1] + t1 * d[1];
        wx = axis_walk(ex, xx, d[0] / c.dxy, 0.0, B.lo[0], B.pitch[0], B.n[0]);
        wy = axis_walk(ey, xy, d[1] / c.dxy, 0.0, B.lo[1], B.pitch[1], B.n[1]);
        T = (t1 - t0) * c.dxy;
    }
    c.x = wx;
    c.y = wy;
    c.T = T;
}

// Row setup: `v` is the row's detector coordinate, `evz` the z component of the row axis.
MBP_HD MBP_INLINE void row_setup(const ColumnWalk& c, const Box& B, double v, double evz,
                                 RowWalk& r) {
    r.t_lo = 0.0; r.t_hi = 0.0; r.kappa = 0.0f;
    r.z.c0 = 0; r.z.step = 0; r.z.steps = 0; r.z.pad_ = 0; r.z.t_first = INFINITY;
    r.z.t_step = 0.0;
    if (!c.hit) return;
    const double dz = c.line ? c.dz_col : c.dz_col + v * evz;   // z change per unit parameter
    const double z0 = c.line ? c.sz + v * evz : c.sz;           // z at parameter 0
    const double wz = dz / c.dxy;                                // z change per unit tau
    const double z_in = z0 + c.t_in * dz;                        // z at tau = 0
    // tau range where lo_z <= z < hi_z, intersected with the column's xy range [0, Txy]
    double tlo = 0.0, thi = c.T;
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
    r.t_lo = tlo;
    r.t_hi = thi;
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
    double nx = c.x.steps > 0 ? c.x.t_first : INFINITY;
    double ny = c.y.steps > 0 ? c.y.t_first : INFINITY;
    const int32_t total = c.x.steps + c.y.steps;
    int32_t cz = r.z.c0, kz = 0;
    double nz = r.z.steps > 0 ? r.z.t_first : INFINITY;
    double ta = 0.0;
    for (int32_t m = 0; m <= total; ++m) {
        const bool last = m == total;
        const bool bx = !last && nx <= ny;
        const double tb = last ? c.T : (bx ? nx : ny);
        double lo = fmax(ta, r.t_lo);
        const double hi = fmin(tb, r.t_hi);
        if (lo < hi) {
            while (nz < hi) {
                visit(cx, cy, cz, (float)fmax(nz - lo, 0.0));
                lo = fmax(lo, nz);
                cz += r.z.step; ++kz;
                nz = kz < r.z.steps ? fma((double)kz, r.z.t_step, r.z.t_first) : INFINITY;
            }
            visit(cx, cy, cz, (float)(hi - lo));
        }
        ta = fmax(ta, tb);
        if (last) break;
        if (bx) {
            cx += c.x.step; ++kx;
            nx = kx < c.x.steps ? fma((double)kx, c.x.t_step, c.x.t_first) : INFINITY;
        } else {
            cy += c.y.step; ++ky;
            ny = ky < c.y.steps ? fma((double)ky, c.y.t_step, c.y.t_first) : INFINITY;
        }
    }
}

// ------------------------------------------------------------------------------------------
// Cell gather (matched adjoint of the column geometry, voxel side).
//
// All rows of detector column j share the column's line in the xy plane, and the ray
// parameter t (0 at the source, 1 at the pixel; any real for parallel lines) is the same for
// all of them at a given xy point. For one xy cell and one view:
//  * the columns whose xy line can cross the cell are found from the detector interval that
//    the cell's corners project to (fp32, widened by a pixel; the fp64 clip decides);
//  * the crossing is t in [t0, t1], a slab clip of the column's line against the cell;
//  * row k is at z cell coordinate zeta(t) = c0 + t c1 + k (c2 + t c3) (the z cell index is
//    floor(zeta)); along the crossing it runs from zeta_a to zeta_b, and its chord through z
//    cell iz is (t1 - t0) * |d_k| * (overlap of [zeta_a, zeta_b] with [iz, iz + 1]) / |zeta_b -
//    zeta_a|, or (t1 - t0) * |d_k| when the piece lies in one z cell.
// |d_k| (the ray's length per unit t) is folded into the sinogram by a pre-pass, so the
// gather adds share * y'.

// Per (view, column) constants of the column's line: t(x) = x * ax + bx when ax != 0, else
// the line keeps x == bx (likewise for y); zeta coefficients c0..c3 as above.
struct ColLine {
    double ax, bx, ay, by;
    double c0, c1, c2, c3;
};

MBP_HD MBP_INLINE void column_line(const Frame& F, const Box& B, int beam, int32_t j, int32_t cols,
                                   int32_t rows, double du, double dv, ColLine& L) {
    const double u = centred(j, cols, du);
    const double px = F.c[0] + u * F.u[0], py = F.c[1] + u * F.u[1], pz = F.c[2] + u * F.u[2];
    double ax, ay, dx, dy, zs, dz0;
    if (beam == BEAM_PARALLEL) {
        ax = px; ay = py; dx = F.s[0]; dy = F.s[1]; zs = pz; dz0 = F.s[2];
    } else {
        ax = F.s[0]; ay = F.s[1]; dx = px - F.s[0]; dy = py - F.s[1]; zs = F.s[2]; dz0 = pz - F.s[2];
    }
    if (dx != 0.0) { L.ax = 1.0 / dx; L.bx = -ax / dx; } else { L.ax = 0.0; L.bx = ax; }
    if (dy != 0.0) { L.ay = 1.0 / dy; L.by = -ay / dy; } else { L.ay = 0.0; L.by = ay; }
    const double inv = 1.0 / B.pitch[2];
    const double roff = 0.5 * (double)(rows - 1);
    const double evz = F.v[2] * dv;                 // z change per row at unit parameter
    if (beam == BEAM_PARALLEL) {                    // z = zs + v_k evz + t dz0
        L.c0 = (zs - roff * evz - B.lo[2]) * inv;
        L.c1 = dz0 * inv;
        L.c2 = evz * inv;
        L.c3 = 0.0;
    } else {                                        // z = zs + t (dz0 + v_k evz)
        L.c0 = (zs - B.lo[2]) * inv;
        L.c1 = (dz0 - roff * evz) * inv;
        L.c2 = 0.0;
        L.c3 = evz * inv;
    }
}

// Detector columns whose xy line can cross the cell [x0,x1) x [y0,y1): corner projections in
// fp32, widened by one pixel on each side (the fp64 clip of each column decides).
MBP_HD MBP_INLINE bool cell_column_range(const Frame& F, int beam, int32_t cols, double du,
                                         double x0, double x1, double y0, double y1,
                                         int32_t& j0, int32_t& j1) {
    float umin = INFINITY, umax = -INFINITY;
    bool bounded = true, neg = false;
    const float sx = (float)F.s[0], sy = (float)F.s[1];
    const float bx = (float)(F.c[0] - F.s[0]), by = (float)(F.c[1] - F.s[1]);
    const float ex = (float)F.u[0], ey = (float)F.u[1];
    const float cx = (float)F.c[0], cy = (float)F.c[1];
    for (int c = 0; c < 4; ++c) {
        const float qx = (float)((c & 1) ? x1 : x0), qy = (float)((c & 2) ? y1 : y0);
        float num, den;
        if (beam == BEAM_PARALLEL) {    // q + l r = det + u e: u = cross(q - det, r) / cross(e, r)
            num = (qx - cx) * sy - (qy - cy) * sx;
            den = ex * sy - ey * sx;
        } else {                        // s + l (q - s) = det + u e: u = cross(det - s, a) / cross(a, e)
            const float ax = qx - sx, ay = qy - sy;
            num = bx * ay - by * ax;
            den = ax * ey - ay * ex;
        }
        if (den == 0.0f || (c > 0 && (den < 0.0f) != neg)) bounded = false;
        neg = den < 0.0f;
        const float u = num / den;
        umin = fminf(umin, u);
        umax = fmaxf(umax, u);
    }
    j0 = 0;
    j1 = cols - 1;
    if (!bounded || !(umin == umin) || !(umax == umax)) return true;
    const float coff = 0.5f * (float)(cols - 1);
    const float inv = (float)(1.0 / du);
    const float f0 = ceilf(umin * inv + coff) - 1.0f, f1 = floorf(umax * inv + coff) + 1.0f;
    if (!(f1 >= 0.0f) || !(f0 <= (float)(cols - 1))) return false;
    j0 = f0 < 0.0f ? 0 : (int32_t)f0;
    j1 = f1 > (float)(cols - 1) ? cols - 1 : (int32_t)f1;
    return j0 <= j1;
}

// ------------------------------------------------------------------------------------------
// Gather for detectors whose rows do not run along z (cone beam, any frame).
//
// Pixel (u, v) lies at c + u eu + v ev; its ray's xy line runs from the source through
// c_xy + u eu_xy + v ev_xy. For a corner q of an xy cell, F_q(u, v) = cross(p_xy - s_xy,
// q - s_xy) = A_q + u Bu_q + v Bv_q is affine in u and v, and the pixel's xy line meets the
// cell exactly when the four F_q do not all have one strict sign. The bands below are
// supersets (widened by a pixel or a row) of the pixels whose rays can cross the cell; each
// ray's own clip decides.

struct TiltCorners {
    double A[4], Bu[4], Bv[4];
};

MBP_HD MBP_INLINE void tilt_corners(const Frame& F, double x0, double x1, double y0, double y1,
                                    TiltCorners& T) {
    const double bx = F.c[0] - F.s[0], by = F.c[1] - F.s[1];
    for (int c = 0; c < 4; ++c) {
        const double ax = ((c & 1) ? x1 : x0) - F.s[0], ay = ((c & 2) ? y1 : y0) - F.s[1];
        T.A[c] = bx * ay - by * ax;
        T.Bu[c] = F.u[0] * ay - F.u[1] * ax;
        T.Bv[c] = F.v[0] * ay - F.v[1] * ax;
    }
}

// Columns j0 .. j1 whose pixels, in some row, can have rays crossing the cell: at each row
// the crossing pixels lie between the corners' projections u_q(v) = -(A_q + v Bv_q) / Bu_q,
// affine in v, so the extremes over all rows are taken at the first and last rows. All
// columns when the corners' Bu_q do not share a sign. False when no column can.
MBP_HD MBP_INLINE bool tilt_column_range(const TiltCorners& T, int32_t rows, int32_t cols, double du,
                                         double dv, int32_t& j0, int32_t& j1) {
    j0 = 0;
    j1 = cols - 1;
    const double va = centred(0, rows, dv), vb = centred(rows - 1, rows, dv);
    double umin = INFINITY, umax = -INFINITY;
    for (int c = 0; c < 4; ++c) {
        if (!(T.Bu[c] != 0.0) || (T.Bu[c] < 0.0) != (T.Bu[0] < 0.0)) return true;
        const double ua = -(T.A[c] + va * T.Bv[c]) / T.Bu[c];
        const double ub = -(T.A[c] + vb * T.Bv[c]) / T.Bu[c];
        umin = fmin(umin, fmin(ua, ub));
        umax = fmax(umax, fmax(ua, ub));
    }
    if (!(umin == umin) || !(umax == umax)) return true;
    const double coff = 0.5 * (double)(cols - 1);
    const double f0 = ceil(umin / du + coff) - 1.0, f1 = floor(umax / du + coff) + 1.0;
    if (!(f1 >= 0.0) || !(f0 <= (double)(cols - 1))) return false;
    j0 = f0 < 0.0 ? 0 : (int32_t)f0;
    j1 = f1 > (double)(cols - 1) ? cols - 1 : (int32_t)f1;
    return j0 <= j1;
}

// Whether the xy line of pixel (u, v) meets the cell (the corners' F_q do not share a strict
// sign).
MBP_HD MBP_INLINE bool tilt_hits(const TiltCorners& T, double u, double v) {
    double lo = INFINITY, hi = -INFINITY;
    for (int c = 0; c < 4; ++c) {
        const double f = T.A[c] + u * T.Bu[c] + v * T.Bv[c];
        lo = fmin(lo, f);
        hi = fmax(hi, f);
    }
    return lo <= 0.0 && hi >= 0.0;
}

// Rows k0 .. k1 of column j whose rays can cross the cell. Along the column each F_q is
// affine in v, so the rows that cross form a set whose ends are roots of some F_q or ends of
// the column: its hull is the span of the roots inside the column and of the column's ends
// that cross, widened by a row. False when no row can.
MBP_HD MBP_INLINE bool tilt_row_range(const TiltCorners& T, int32_t j, int32_t rows, int32_t cols,
                                      double du, double dv, int32_t& k0, int32_t& k1) {
    const double u = centred(j, cols, du);
    const double va = centred(0, rows, dv), vb = centred(rows - 1, rows, dv);
    const double vlo = fmin(va, vb), vhi = fmax(va, vb);
    double lo = INFINITY, hi = -INFINITY;
    if (tilt_hits(T, u, va)) { lo = fmin(lo, va); hi = fmax(hi, va); }
    if (tilt_hits(T, u, vb)) { lo = fmin(lo, vb); hi = fmax(hi, vb); }
    for (int c = 0; c < 4; ++c) {
        if (T.Bv[c] == 0.0) continue;
        const double r = -(T.A[c] + u * T.Bu[c]) / T.Bv[c];
        if (r >= vlo && r <= vhi) { lo = fmin(lo, r); hi = fmax(hi, r); }
    }
    if (!(lo <= hi)) return false;
    const double coff = 0.5 * (double)(rows - 1);
    const double ka = lo / dv + coff, kb = hi / dv + coff;
    const double f0 = floor(fmin(ka, kb)) - 1.0, f1 = ceil(fmax(ka, kb)) + 1.0;
    k0 = f0 < 0.0 ? 0 : (int32_t)f0;
    k1 = f1 > (double)(rows - 1) ? rows - 1 : (int32_t)f1;
    return k0 <= k1;
}

// One item of the tilted gather: rows k0 .. k0 + nrows - 1 (at most 64) of column j in view
// `view`, with everything its rows share, computed once when the item is built: the column's
// ray direction at v = 0, b = c - s + u eu (xy components, and z in cells per unit parameter),
// the view's row axis ev (likewise), the offsets of the cell's lower walls from the source
// (x0 - sx, y0 - sy; the upper walls lie one pitch further) and the source's z in cells above
// the box (88 bytes). Row k's ray direction is b + v_k ev, v_k the row's centred coordinate.
struct TiltItem {
    double bx, by, bzc;
    double evx, evy, evzc;
    double wx0, wy0;
    double szc;
    int32_t view, j, k0, nrows;
};

// The clip of ray s + t d (t in [0, 1]) against the xy cell [x0, x1) x [y0, y1) with one
// reciprocal per axis: [t0, t1], empty unless t1 > t0.
MBP_HD MBP_INLINE void tilt_clip(const double* s, const double* d, double x0, double x1, double y0,
                                 double y1, double& t0, double& t1) {
    double a = 0.0, b = 1.0;
    const double lo[2] = {x0, y0}, hi[2] = {x1, y1};
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        if (d[k] != 0.0) {
            const double r = 1.0 / d[k];
            const double p = (lo[k] - s[k]) * r, q = (hi[k] - s[k]) * r;
            a = fmax(a, fmin(p, q));
            b = fmin(b, fmax(p, q));
        } else if (s[k] < lo[k] || s[k] >= hi[k]) {
            b = -1.0;
        }
    }
    t0 = a;
    t1 = b;
}

// Clip column line L to the cell: t in [t0, t1] (segments start from [0, 1]).
MBP_HD MBP_INLINE bool cell_clip(const ColLine& L, bool line, double x0, double x1, double y0,
                                 double y1, double& t0, double& t1) {
    t0 = line ? -INFINITY : 0.0;
    t1 = line ? INFINITY : 1.0;
    if (L.ax != 0.0) {
        const double p = x0 * L.ax + L.bx, q = x1 * L.ax + L.bx;
        t0 = fmax(t0, fmin(p, q));
        t1 = fmin(t1, fmax(p, q));
    } else if (!(L.bx >= x0 && L.bx < x1)) {
        return false;
    }
    if (L.ay != 0.0) {
        const double p = y0 * L.ay + L.by, q = y1 * L.ay + L.by;
        t0 = fmax(t0, fmin(p, q));
        t1 = fmin(t1, fmax(p, q));
    } else if (!(L.by >= y0 && L.by < y1)) {
        return false;
    }
    return t1 > t0;
}

// Pieces of the row whose z cell coordinate runs from za to zb, restricted to z cells
// [z0, z1), when they are not a single piece in one cell: piece(iz, share of (t1 - t0)).
// With `aligned`, the walk starts at floor(min(za, zb)) even below z0 (cells outside
// [z0, z1) are stepped over, not visited), so step i of every row is cell floor(zmin) + i:
// rows whose zmin differ by more than one cell then never meet in the same cell at the same
// step. The caller only asks for it when min(za, zb) lies at most a few cells below z0.
template <class Piece>
MBP_HD MBP_INLINE void row_pieces_split(double za, double zb, double dt, int32_t z0, int32_t z1,
                                        bool aligned, Piece& piece) {
    const double zmin = fmin(za, zb), zmax = fmax(za, zb);
    const double ext = zmax - zmin;
    if (!(ext > 0.0)) return;              // a point piece outside [z0, z1)
    if (!(zmax > (double)z0) || !(zmin < (double)z1)) return;
    const double scale = dt / ext;
    const int32_t ia = (int32_t)floor(aligned ? zmin : fmax(zmin, (double)z0));
    const int32_t ib = (int32_t)fmin(floor(zmax), (double)(z1 - 1));
    for (int32_t iz = ia; iz <= ib; ++iz) {
        if (iz < z0) continue;
        const double ov = fmin(zmax, (double)(iz + 1)) - fmax(zmin, (double)iz);
        if (ov > 0.0) piece(iz, ov * scale);
    }
}

// Row grouping of the gather: groups of S * 64 rows (S = min(kGatherGroup, ceil(rows / 64)))
// in which chunk c (one instruction's 64 lanes) holds rows c, c + S, c + 2S, ...
constexpr int32_t kGatherGroup = 8;

MBP_HD MBP_INLINE int32_t gather_stride(int32_t rows) {
    const int32_t s = (rows + 63) / 64;
    return s < kGatherGroup ? s : kGatherGroup;
}

// Rows of the reordered sinogram, padded with zeros to whole groups of S * 64.
MBP_HD MBP_INLINE int32_t gather_rows_padded(int32_t rows) {
    const int32_t g = 64 * gather_stride(rows);
    return (rows + g - 1) / g * g;
}

// Floats of the reordered sinogram of nb members: [view][column][padded row][member], plus a
// tail of kGatherGroup rows that a lane's fixed-width row loads may reach past the last line.
MBP_HD MBP_INLINE int64_t gather_sino_floats(int32_t views, int32_t cols, int32_t rows, int nb) {
    return (int64_t)nb * ((int64_t)views * cols * gather_rows_padded(rows) + kGatherGroup);
}

// Turn symmetry of a circular scan. When the V views fall into P groups of q = V / P such that
// view v + m q is view v turned by m P-ths of a full turn about the vertical axis through the
// grid's xy centre, and that turn maps the grid's cells onto cells, then line (view v + m q,
// column j) crosses cell C exactly as line (v, j) crosses the cell turned back by m steps: the
// intersection lengths are a property of the pair, and turning both leaves them unchanged. The
// forward then walks the rays of views v < q only: the walk of ray (v, j, row) through cells C
// gives ray (v + m q, j, row) from the cells R^m C (R: one step of the turn). The gather gives
// one wave the P cells of an orbit c, R c, ..., R^(P-1) c and forms items for views v < q
// only: the item of line (v, j) with cell R^a c carries the rows of line (v + m q, j) into
// cell R^(a+m) c, for every m.
//
// orbit_cell: cell (ox, oy) = R^a (ix, iy) on a W x H grid. P = 2: the half turn,
// (ix, iy) -> (W-1-ix, H-1-iy). P = 4 (square grid, W == H): a quarter turn, anticlockwise seen
// from +z for dir > 0 ((x, y) -> (-y, x), so (ix, iy) -> (W-1-iy, ix)), clockwise otherwise
// ((x, y) -> (y, -x), so (ix, iy) -> (iy, W-1-ix)). P = 1: the cell itself.
MBP_HD MBP_INLINE void orbit_cell(int32_t P, int32_t dir, int32_t W, int32_t H, int32_t ix,
                                  int32_t iy, int32_t a, int32_t& ox, int32_t& oy) {
    ox = ix;
    oy = iy;
    for (int32_t k = 0; k < a; ++k) {
        const int32_t x = ox, y = oy;
        if (P == 2) {
            ox = W - 1 - x;
            oy = H - 1 - y;
        } else if (P == 4 && dir > 0) {
            ox = W - 1 - y;
            oy = x;
        } else if (P == 4) {
            ox = y;
            oy = W - 1 - x;
        }
    }
}

// The column indices (ix * H + iy) of the cells of an orbit, slot m holding the cell turned m
// steps (orbit_cell): the half turn of a cell is W H - 1 - cxy; for a quarter turn (W == H)
// slot 1 is c1, the cell's quarter turn (from its ix and iy), slot 2 its half turn and slot 3
// the half turn of c1. WH1 = W H - 1.
template <int P>
MBP_HD MBP_INLINE void orbit_columns(uint32_t cxy, uint32_t c1, uint32_t WH1, uint32_t (&cell)[P]) {
    cell[0] = cxy;
    if (P == 2) cell[1 % P] = WH1 - cxy;
    if (P == 4) {
        cell[1 % P] = c1;
        cell[2 % P] = WH1 - cxy;
        cell[3 % P] = WH1 - c1;
    }
}

// Element offsets of the turned cells on a volume with element (x, y, z) at x sx + y sy + z sz:
// cell R^a (cx, cy) lies at base + cx tx + cy ty (+ cz sz), the map being affine in (cx, cy).
MBP_HD MBP_INLINE void orbit_strides(int32_t P, int32_t dir, int32_t W, int32_t H, int32_t sx,
                                     int32_t sy, int32_t a, int32_t& base, int32_t& tx, int32_t& ty) {
    int32_t x0, y0, x1, y1, x2, y2;
    orbit_cell(P, dir, W, H, 0, 0, a, x0, y0);
    orbit_cell(P, dir, W, H, 1, 0, a, x1, y1);
    orbit_cell(P, dir, W, H, 0, 1, a, x2, y2);
    base = x0 * sx + y0 * sy;
    tx = (x1 - x0) * sx + (y1 - y0) * sy;
    ty = (x2 - x0) * sx + (y2 - y0) * sy;
}

// The cells that stand for the orbits (one per orbit): ix < W / 2 for P = 2 (W even), ix and
// iy < W / 2 for P = 4 (W == H even); the whole grid for P = 1.
MBP_HD MBP_INLINE void orbit_grid(int32_t P, int32_t W, int32_t H, int32_t& Wr, int32_t& Hr) {
    Wr = P == 1 ? W : W / 2;
    Hr = P == 4 ? H / 2 : H;
}

// Whether the lanes of one gather instruction (rows S apart, z cell coordinate at row k
// za0 + k za1 at the crossing's start and zb0 + k zb1 at its end) always add into different
// z cells when pieces are walked aligned: S rows move z by more than one cell at both ends,
// and no row spans more than 64 z cells inside the xy cell.
MBP_HD MBP_INLINE bool gather_exclusive(int32_t S, int32_t rows, double za0, double za1, double zb0,
                                        double zb1) {
    const double span0 = fabs(zb0 - za0);
    const double span1 = fabs(zb0 - za0 + (double)(rows - 1) * (zb1 - za1));
    return (double)S * fmin(fabs(za1), fabs(zb1)) > 1.0 + 1e-6 && fmax(span0, span1) <= 64.0;
}

// ------------------------------------------------------------------------------------------
// Gather work items and the fixed-point row form.
//
// One item is one detector column crossing one xy cell in one view: row k's z cell
// coordinate is za0 + k za1 where it enters the cell and zb0 + k zb1 where it leaves, over a
// parameter length dt. Items are built by all lanes at once (one view per lane) and then
// processed one at a time by the whole wave (lanes = rows).
//
// The fast form applies when each row's z extent inside the cell is below one cell, so a
// row has at most two pieces (cells fa and fa + 1). When lanes that write together are more
// than two cells apart their cell pairs {fa, fa + 1} are disjoint; otherwise lanes that share
// a pair are consecutive, and their shares are combined across lanes first. A lane takes S
// consecutive rows. Its origin row (the middle one when the lane holds kGatherGroup rows,
// else the first) is placed from the item's 64-bit fixed-point positions: the integer cell I
// of that row's entry end, and the row's two ends relative to I in signed fixed point with
// kZFrac fraction bits, rounded to nearest. The other rows move from it by whole multiples of
// the per-row advance (rounded to the same resolution), which keeps every row of the lane
// within kFastSpan cells of it and so inside the fixed point's range. Differences of positions are exact integers: the share of
// each cell, (distance to the plane between them) / extent, keeps full relative precision
// however flat the row is.

constexpr int kZFrac = 28;
constexpr int32_t kZOne = 1 << kZFrac;
constexpr double kZScale = 268435456.0;            // 2^kZFrac
// Most cells a lane's rows move from its origin row: positions (the origin's ends within
// (-1, 2) cells of its integer cell) stay below 2 + kFastSpan cells in magnitude, inside the
// 8 cells of the fixed point.
constexpr double kFastSpan = 5.5;
// GatherItem::form. Fast form: all lanes update their cell pairs at once (kFastPairs), or
// lanes that share a pair, in runs of at most GatherItem::run consecutive lanes, combine
// their shares before the run's ends write (kFastRuns). General form: lanes add exclusively,
// or need atomics.
constexpr int32_t kFastPairs = 1;
constexpr int32_t kFastRuns = 2;
// Added to a fast form when every row's cell pair lies inside the column chunk's range of pair
// indices (gather_item with fast_inside_lo and fast_inside_hi), so that the kernel needs no
// clamp.
constexpr int32_t kFastInside = 4;
constexpr int32_t kGeneralExclusive = 0;
constexpr int32_t kGeneralAtomic = -1;

// Fast items hold their positions as signed fixed point with kPosFrac fraction bits instead
// of fp64, so that a lane's origin needs only integer multiply-adds. The start positions carry
// half a unit of 2^-kZFrac, so that truncating to kZFrac bits rounds to nearest.
constexpr int kPosFrac = 40;
constexpr double kPosScale = 1099511627776.0;      // 2^kPosFrac
// Fast items keep |z| below this many cells at every row, so positions fit in 64 bits.
constexpr double kPosLimit = 4194304.0;            // 2^22

struct GatherItem {
    // z cell coordinate where row k enters the cell, za0 + k za1, and where it leaves,
    // zb0 + k zb1; fast items: the same four values in fixed point (fa0 ... fb1)
    union { double za0; int64_t fa0; };
    union { double za1; int64_t fa1; };
    union { double zb0; int64_t fb0; };
    union { double zb1; int64_t fb1; };
    float dt;           // parameter length of the crossing
    int32_t yoff;       // (view - first view of the launch) * cols + column: the line of the
                        // reordered sinogram and of the line table
    int32_t a1fx;       // fast form: za1 in fixed point
    int32_t b1fx;       // fast form: zb1 in fixed point
    int32_t form;       // kFastPairs, kFastRuns, kGeneralExclusive or kGeneralAtomic
    int32_t run;        // kFastRuns: most consecutive lanes with one lower cell (fast_run)
    int32_t pad_[2];    // 64 bytes: the wave reads an item with four aligned 16-byte loads
};

// The row of a lane (0 .. S - 1) that holds the lane's origin, and the most rows any other row
// of the lane lies from it.
MBP_HD MBP_INLINE int32_t fast_origin_row(int32_t S) {
    return S == kGatherGroup ? kGatherGroup / 2 : 0;
}
MBP_HD MBP_INLINE int32_t fast_span_rows(int32_t S) {
    return S == kGatherGroup ? kGatherGroup / 2 : S - 1;
}

// Longest run of lanes that the fast form combines.
constexpr int32_t kMaxRun = 16;

// For a fast item whose rows advance by a1 and b1 per row (fixed point): the least G such
// that lanes G apart (S * G rows) are more than `cells` cells apart (plus a margin of 2^-10
// cell, far above the fixed point's rounding). With cells = 2, G = 1 means that the lanes'
// cell pairs are disjoint; with cells = 1, lanes sharing a lower cell come in runs of at most
// G consecutive lanes. G = floor(need / step) + 1 from an fp64 quotient of integers below
// 2^53: should the quotient round up to an integer, G comes out one larger, which is still a
// bound. 0 when more than kMaxRun would be needed.
MBP_HD MBP_INLINE int32_t fast_run(int32_t S, int32_t a1, int32_t b1, int32_t cells = 2) {
    const uint64_t a = (uint64_t)(a1 < 0 ? -(int64_t)a1 : (int64_t)a1);
    const uint64_t b = (uint64_t)(b1 < 0 ? -(int64_t)b1 : (int64_t)b1);
    const uint64_t step = (uint64_t)S * (a < b ? a : b);
    const uint64_t need = (uint64_t)cells * (uint64_t)kZOne + ((uint64_t)kZOne >> 10);
    if (step > need) return 1;
    if ((uint64_t)kMaxRun * step <= need) return 0;           // also step == 0
    return (int32_t)floor((double)need / (double)step) + 1;
}

// Whether an item takes the fast form (rows 0 .. rows_pad - 1): both ends move the same way,
// every row spans less than one cell, a lane's rows stay within kFastSpan cells of its
// origin row, and runs of lanes sharing a lower cell are at most kMaxRun long. a1, b1: the
// per-row advances in fixed point.
MBP_HD MBP_INLINE bool gather_fast(int32_t S, int32_t rows_pad, double za0, double za1,
                                   double zb0, double zb1, int32_t a1, int32_t b1) {
    const double e0 = fabs(zb0 - za0), e1 = fabs(zb0 - za0 + (double)(rows_pad - 1) * (zb1 - za1));
    return za1 * zb1 > 0.0 && (double)fast_span_rows(S) * fmax(fabs(za1), fabs(zb1)) <= kFastSpan &&
           fmax(e0, e1) < 1.0 - 1e-6 && fast_run(S, a1, b1, 1) > 0;
}

// Whether both ends of every row of an item lie in [lo, hi), from the ends of its first and
// last rows (positions are linear in the row, so the extremes are there), tested on the ends
// rounded to fp32.
MBP_HD MBP_INLINE bool rows_inside(double za_first, double zb_first, double za_last, double zb_last,
                                   float lo, float hi) {
    const float a0 = (float)za_first, b0 = (float)zb_first, a1 = (float)za_last, b1 = (float)zb_last;
    return fminf(fminf(a0, a1), fminf(b0, b1)) >= lo && fmaxf(fmaxf(a0, a1), fmaxf(b0, b1)) < hi;
}

// The z range, in cells, that a fast item's rows must keep to for the gather to write their
// cell pairs unclamped in the column chunk of n cells from z0 >= 0: the lower end's cell then
// lies in [z0 - 3, z0 + n] (pair indices [-2, n + 1] from the guard cell z0 - 1). The quarter
// cell of margin covers the fixed point's rounding (a few units of 2^-28) and the fp32
// rounding of rows_inside, which is below 2^-5 cell for ends that pass when z0 + n <= 2^19;
// deeper chunks accept nothing.
MBP_HD MBP_INLINE float fast_inside_lo(int32_t z0, int32_t n) {
    return z0 + n <= (1 << 19) ? (float)z0 - 2.75f : INFINITY;
}
MBP_HD MBP_INLINE float fast_inside_hi(int32_t z0, int32_t n) { return (float)(z0 + n) + 0.75f; }

// The item of column line L crossing the cell, or false when it misses. A fast item whose
// rows (padded ones too) keep both ends in [in_lo, in_hi) gets kFastInside (never with an
// empty range, such as the default, which skips the test).
MBP_HD MBP_INLINE bool gather_item(const ColLine& L, bool line, double x0, double x1, double y0,
                                   double y1, int32_t S, int32_t rows, int32_t rows_pad,
                                   int32_t yoff, GatherItem& it, float in_lo = INFINITY,
                                   float in_hi = -INFINITY) {
    double t0, t1;
    if (!cell_clip(L, line, x0, x1, y0, y1, t0, t1)) return false;
    it.za0 = L.c0 + t0 * L.c1;
    it.za1 = L.c2 + t0 * L.c3;
    it.zb0 = L.c0 + t1 * L.c1;
    it.zb1 = L.c2 + t1 * L.c3;
    it.dt = (float)(t1 - t0);
    it.yoff = yoff;
    // the per-row advances in fixed point (only meaningful when they fit; checked below), the
    // row count (row_times) and the positions' range at the first and last padded rows
    const double kl = (double)(rows_pad - 1);
    const double za_last = fma(kl, it.za1, it.za0), zb_last = fma(kl, it.zb1, it.zb0);
    const bool fits = rows_pad <= (1 << 20) && fabs(it.za1) < kFastSpan && fabs(it.zb1) < kFastSpan &&
                      fmax(fmax(fabs(it.za0), fabs(it.zb0)), fmax(fabs(za_last), fabs(zb_last))) < kPosLimit;
    const bool inside = in_lo < in_hi && rows_inside(it.za0, it.zb0, za_last, zb_last, in_lo, in_hi);
    it.a1fx = fits ? (int32_t)rint(it.za1 * kZScale) : 0;
    it.b1fx = fits ? (int32_t)rint(it.zb1 * kZScale) : 0;
    it.run = 0;
    if (fits && gather_fast(S, rows_pad, it.za0, it.za1, it.zb0, it.zb1, it.a1fx, it.b1fx)) {
        if (fast_run(S, it.a1fx, it.b1fx) == 1) {
            it.form = kFastPairs;
        } else {
            it.form = kFastRuns;
            it.run = fast_run(S, it.a1fx, it.b1fx, 1);
        }
        if (inside) it.form |= kFastInside;
        const double half = 0.5 / kZScale;
        const int64_t a0 = (int64_t)rint((it.za0 + half) * kPosScale);
        const int64_t a1 = (int64_t)rint(it.za1 * kPosScale);
        const int64_t b0 = (int64_t)rint((it.zb0 + half) * kPosScale);
        const int64_t b1 = (int64_t)rint(it.zb1 * kPosScale);
        it.fa0 = a0;
        it.fa1 = a1;
        it.fb0 = b0;
        it.fb1 = b1;
    } else {
        it.form = gather_exclusive(S, rows, it.za0, it.za1, it.zb0, it.zb1) ? kGeneralExclusive
                                                                          : kGeneralAtomic;
    }
    it.pad_[0] = it.pad_[1] = 0;
    return true;
}

// k * f for a row index 0 <= k < 2^20 and |f| < 2^43: the low word's 32 x 32 -> 64 product
// plus the high word's product (below 2^31 in magnitude) shifted up, modulo 2^64.
MBP_HD MBP_INLINE int64_t row_times(int32_t k, int64_t f) {
    const uint32_t lo = (uint32_t)f;
    const int32_t hi = (int32_t)(f >> 32);
    return (int64_t)((uint64_t)(uint32_t)k * lo + ((uint64_t)(uint32_t)(k * hi) << 32));
}

// Row ends are held unsigned, offset by kZBias (8 cells): a signed position p in (-8, 8) cells
// becomes p + 2^31, so that order, floor and differences are those of unsigned integers, and
// the cell of an end is its top four bits minus kZBiasCells.
constexpr uint32_t kZBias = 0x80000000u;
constexpr int32_t kZBiasCells = 8;
static_assert(kZBias == (uint32_t)kZBiasCells << kZFrac, "the offset is kZBiasCells cells");

// A lane's origin for the fast form from its origin row k: the integer cell I of that row's
// entry end and the row's ends relative to I in fixed point (the entry end in [0, 1) cell, the
// exit end in (-1, 2)), rounded to nearest, offset by kZBias: they are taken relative to the
// cell I - kZBiasCells. `base` is I - kZBiasCells - cell0 (cell0: the cell held at index 0),
// so that a row's pair index, its lower end's cell minus cell0, is base + fb (fast_row);
// |I| < 2^22 (kPosLimit).
MBP_HD MBP_INLINE void fast_origin(const GatherItem& it, int32_t k, int32_t cell0, uint32_t& la,
                                   uint32_t& lb, int32_t& base) {
    const int64_t pa = it.fa0 + row_times(k, it.fa1);
    const int64_t pb = it.fb0 + row_times(k, it.fb1);
    const int32_t Ib = (int32_t)(pa >> kPosFrac) - kZBiasCells;    // arithmetic shift: floor
    const int64_t ref = (int64_t)Ib * ((int64_t)1 << kPosFrac);
    la = (uint32_t)((pa - ref) >> (kPosFrac - kZFrac));
    lb = (uint32_t)((pb - ref) >> (kPosFrac - kZFrac));
    base = Ib - cell0;
}

// |a - b| (one v_sad_u32 on the device).
MBP_HD MBP_INLINE uint32_t abs_diff(uint32_t a, uint32_t b) {
#if defined(__HIP_DEVICE_COMPILE__)
    uint32_t r;
    asm("v_sad_u32 %0, %1, %2, 0" : "=v"(r) : "v"(a), "v"(b));
    return r;
#else
    return a > b ? a - b : b - a;
#endif
}

// One row of the fast form with ends za, zb (offset fixed point, relative to the lane
// origin): the lower end's cell relative to the origin's cell, plus kZBiasCells, fb; the
// distance num from the lower end to the plane above that cell; and the extent ext. The row crosses that plane exactly when num < ext; then the lower cell's share
// is num / ext and the upper one's (ext - num) / ext.
MBP_HD MBP_INLINE void fast_row(uint32_t za, uint32_t zb, int32_t& fb, uint32_t& num, uint32_t& ext) {
    const uint32_t lo = za < zb ? za : zb;
    fb = (int32_t)(lo >> kZFrac);
    num = kZOne - (lo & (kZOne - 1));
    ext = abs_diff(za, zb);
}

// ------------------------------------------------------------------------------------------
// Column walk in chunks: the xy crossings of a column, merged in order, built in parallel.
//
// The xy cells a column's line visits do not depend on the row, so a wave can lay them out
// once for all of its rows: the crossings are the x sequence x_i = first_x + i step_x and the
// y sequence y_j = first_y + j step_y (one fma each, as in walk_column_row), and their merged
// order, x first on ties, gives the cells. For a chunk of up to kXYChunk crossings that start
// after kx0 x and ky0 y crossings, x_i lands at position i + #{y in the chunk's y window
// strictly before x_i} and y_j at j + #{x in the x window at or before y_j}; the counts come
// from branch-free binary searches over the same fma'd values (both sequences are
// non-decreasing), so every position of the chunk is filled exactly once. Each entry holds
// the distance at which a cell ends and the cell's xy index, the cell before that crossing.

constexpr int32_t kXYChunk = 128;
// xy_chunk_fill gives each of a wave's 64 lanes two window indices of each axis.
static_assert(kXYChunk == 2 * 64, "xy_chunk_fill covers two crossings per lane");
// Cells per group when a row's pieces are computed ahead of their loads.
constexpr int32_t kCellGroup = 4;

struct XYEvent {
    double tb;          // distance at which the cell ends
    int32_t cxy;        // cx * H + cy
    float chord;        // tb minus the previous cell's tb, rounded to fp32 (xy_chunk_chords)
};

MBP_HD MBP_INLINE double crossing(const AxisWalk& a, int32_t k) {
    return fma((double)k, a.t_step, a.t_first);
}

// Number of crossings of `a` with index in [k0, k0 + n) at or before `t` (strict = false) or
// strictly before it (strict = true); n <= 255.
MBP_HD MBP_INLINE int32_t count_before(const AxisWalk& a, int32_t k0, int32_t n, double t, bool strict) {
    int32_t lo = 0;
    for (int32_t step = 128; step > 0; step >>= 1) {
        if (lo + step <= n) {
            const double v = crossing(a, k0 + lo + step - 1);
            if (strict ? v < t : v <= t) lo += step;
        }
    }
    return lo;
}

// Fill the entries of one lane's candidates (window indices lane and lane + 64 of each axis)
// for the chunk of `count` crossings after kx0 x and ky0 y crossings. Returns how many of
// this lane's x candidates fall inside the chunk (their sum over lanes is the number of x
// crossings the chunk consumes). With C1, C1[pos] also receives the column index of the
// event's cell turned a quarter turn of sense dir on the square W x H grid (orbit_cell).
MBP_HD MBP_INLINE int32_t xy_chunk_fill(const ColumnWalk& c, int32_t H, int32_t kx0, int32_t ky0,
                                        int32_t count, int32_t lane, XYEvent* E,
                                        int32_t* C1 = nullptr, int32_t W = 0, int32_t dir = 0) {
    auto turned = [&](int32_t pos, int32_t ix, int32_t iy) {
        if (!C1) return;
        int32_t ox, oy;
        orbit_cell(4, dir, W, H, ix, iy, 1, ox, oy);
        C1[pos] = ox * H + oy;
    };
    const int32_t nxw = c.x.steps - kx0 < kXYChunk ? c.x.steps - kx0 : kXYChunk;
    const int32_t nyw = c.y.steps - ky0 < kXYChunk ? c.y.steps - ky0 : kXYChunk;
    int32_t xin = 0;
    for (int32_t q = 0; q < 2; ++q) {
        const int32_t i = lane + 64 * q;
        if (i < nxw) {
            const double tx = crossing(c.x, kx0 + i);
            const int32_t jy = count_before(c.y, ky0, nyw, tx, true);
            const int32_t pos = i + jy;
            if (pos < count) {
                const int32_t ix = c.x.c0 + c.x.step * (kx0 + i), iy = c.y.c0 + c.y.step * (ky0 + jy);
                E[pos].tb = tx;
                E[pos].cxy = ix * H + iy;
                turned(pos, ix, iy);
                ++xin;
            }
        }
        if (i < nyw) {
            const double ty = crossing(c.y, ky0 + i);
            const int32_t ix = count_before(c.x, kx0, nxw, ty, false);
            const int32_t pos = i + ix;
            if (pos < count) {
                const int32_t cx = c.x.c0 + c.x.step * (kx0 + ix), cy = c.y.c0 + c.y.step * (ky0 + i);
                E[pos].tb = ty;
                E[pos].cxy = cx * H + cy;
                turned(pos, cx, cy);
            }
        }
    }
    return xin;
}

// One row's share of one xy cell [ta, tb] with column-base index `cxy`: visit(cxy, cz, len)
// for the row's pieces inside the cell (lengths in units of tau). The row's z state (cz, kz,
// nz) carries over from cell to cell.
template <class Visit>
MBP_HD MBP_INLINE void row_cell(const RowWalk& r, double ta, double tb, int32_t cxy, int32_t& cz,
                                int32_t& kz, double& nz, Visit& visit) {
    double lo = fmax(ta, r.t_lo);
    const double hi = fmin(tb, r.t_hi);
    if (!(lo < hi)) return;
    while (nz < hi) {
        visit(cxy, cz, (float)fmax(nz - lo, 0.0));
        lo = fmax(lo, nz);
        cz += r.z.step; ++kz;
        nz = kz < r.z.steps ? crossing(r.z, kz) : INFINITY;
    }
    visit(cxy, cz, (float)(hi - lo));
}

// A row meets at most one z plane inside any xy cell when its z crossings lie farther apart
// than the longest chord of an xy cell (the cell's diagonal); the margin is far above the
// rounding of the crossing distances.
MBP_HD MBP_INLINE bool row_single_crossing(const RowWalk& r, const Box& B) {
    const double diag = sqrt(B.pitch[0] * B.pitch[0] + B.pitch[1] * B.pitch[1]);
    return r.z.steps == 0 || r.z.t_step > 1.001 * diag;
}

// row_cell for a row with row_single_crossing(): the piece before the cell's z crossing
// (z cell cz0, length len0) and the piece after it (cz1, len1; len1 = 0 when the row meets
// no z plane in the cell). Lengths are 0 where the row is outside the slab.
MBP_HD MBP_INLINE void row_cell_two(const RowWalk& r, double ta, double tb, int32_t& cz,
                                    int32_t& kz, double& nz, int32_t& cz0, float& len0,
                                    int32_t& cz1, float& len1) {
    const double lo = fmax(ta, r.t_lo), hi = fmin(tb, r.t_hi);
    const bool in = lo < hi;
    const bool cross = in && nz < hi;
    cz0 = cz;
    len0 = in ? (float)(cross ? fmax(nz - lo, 0.0) : hi - lo) : 0.0f;
    len1 = 0.0f;
    if (cross) {
        len1 = (float)(hi - fmax(lo, nz));
        cz += r.z.step;
        ++kz;
        nz = kz < r.z.steps ? crossing(r.z, kz) : INFINITY;
    }
    cz1 = cz;
}

// The chords of a filled chunk whose first cell starts at ta, for the entries at positions
// lane and lane + 64 (every entry must be filled and visible to the lane first).
MBP_HD MBP_INLINE void xy_chunk_chords(XYEvent* E, int32_t count, double ta, int32_t lane) {
    for (int32_t q = 0; q < 2; ++q) {
        const int32_t i = lane + 64 * q;
        if (i < count) E[i].chord = (float)(E[i].tb - (i > 0 ? E[i - 1].tb : ta));
    }
}

// row_cell_two for a cell inside the row's slab (t_lo <= ta and tb <= t_hi) of a row with
// row_single_crossing(): no clip is needed, and the row's next z crossing nz is not before ta
// (the previous one lies inside an earlier cell, more than a cell diagonal back). The row
// crosses a z plane in the cell when nz < tb; the piece after it is tb - nz and the piece
// before it the rest of the cell's chord (so the two add up to the chord, and the first is 0
// exactly when nz == ta). k counts the row's crossings; a crossing recomputes nz from it with
// the same fma as crossing() (t_first = +inf for a row with no crossing left, so nz stays
// +inf). The caller checks with stepped_walk_ok() that the count cannot pass the row's last
// z plane inside the chunk.
MBP_HD MBP_INLINE bool row_cell_two_counted(double t_first, double t_step, double tb, float chord,
                                            int32_t& k, double& nz, float& len0, float& len1) {
    const bool cross = nz < tb;
    len1 = cross ? (float)(tb - nz) : 0.0f;
    len0 = chord - len1;
    k += cross ? 1 : 0;
    nz = fma((double)k, t_step, t_first);
    return cross;
}

// Whether a row that has made kz of its z crossings may take row_cell_two_counted over the
// cells of a chunk ending at t_end (count cells): with fewer crossings left than cells it
// could count past its last plane, which is harmless only if the plane after that one (where
// nz then lands) lies clearly after t_end.
MBP_HD MBP_INLINE bool stepped_walk_ok(const RowWalk& r, int32_t kz, int32_t count, double t_end) {
    if (kz >= r.z.steps || r.z.steps - kz >= count) return true;
    const double beyond = crossing(r.z, r.z.steps);
    return beyond > t_end + 1e-9 * (fabs(t_end) + r.z.t_step);
}

}  // namespace mbp
