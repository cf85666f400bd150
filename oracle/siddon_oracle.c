/*
 * siddon_oracle.c -- fp64 CPU oracle for the ray-driven X-ray transform pair.
 *
 * TEST INFRASTRUCTURE ONLY. This file is the slow, plain reference that the HIP path is
 * checked against. Only the tests, the smoke check and the benchmark's CPU-baseline leg may
 * load it. It shares no code, header, table or constant with the HIP library.
 *
 * What it computes (diffct pages, "diffct 2.1.0 -> 2.2.1", README "Why diffct", bullet
 * "Matched operators": project() and backproject() are an exact adjoint pair for the
 * cell-constant Siddon model; repeated on "diffct 2.2.1 -> 2.4.0", README):
 *
 *   forward   P[r]  = sum_v  len(r, v) * vol[v]      (line integral of the cell-constant
 *                                                    volume along ray r, physical length)
 *   adjoint   Bp[v] = sum_r  len(r, v) * y[r]        (its exact transpose)
 *
 * where len(r, v) is the physical length of ray r inside voxel v. No normalisation, no other
 * weighting.
 *
 * Method: Siddon's parametric formulation (R. L. Siddon, "Fast calculation of the exact
 * radiological path for a three-dimensional CT array", Med. Phys. 12(2), 1985): clip the ray
 * to the volume box, list the parameter values at which it crosses each family of grid
 * planes, merge the sorted lists, and give every consecutive pair of parameters the cell that
 * contains the midpoint. Everything is fp64; float inputs are widened on read.
 *
 * Geometry readings (the pages leave these open; the plainest reading is taken):
 *  - world x <-> W (fastest tensor axis), y <-> H, z <-> D; voxel pitch (dz, dy, dx) in tensor
 *    order (page "diffct 2.4.3 -> 2.4.4", README "Per-axis voxel spacing");
 *  - the volume box is centred on `center`: lo = center - N*pitch/2 per axis;
 *  - pixel (row k, col j) of view i sits at det + u_j*eu + v_k*ev with
 *    u_j = (j - (cols-1)/2)*du and v_k = (k - (rows-1)/2)*dv (centred detector; the per-view
 *    tuples are on page "diffct 2.1.0 -> 2.2.1", diffct/analytical.py);
 *  - fan/cone rays are the segments source -> pixel (parameter in [0, 1]); parallel rays are
 *    infinite lines through the pixel along the per-view ray direction (page
 *    "diffct 2.2.1 -> 2.4.0", CHANGELOG 2.4.0: infinite parallel rays; the same page adds a
 *    3-D parallel beam, "parallel3d", whose rays are such lines through the pixels of a flat
 *    2-D detector);
 *  - cells are half-open [lo, hi): a ray lying exactly in a grid plane belongs to the cell
 *    above it; a ray with a zero direction component outside [lo, hi) on that axis misses.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORC_PARALLEL = 0, ORC_FAN = 1, ORC_CONE = 2, ORC_PARALLEL3D = 3 };
enum { ORC_OK = 0, ORC_EINVAL = -1, ORC_ENOMEM = -2, ORC_ECAP = -3 };

/* Geometry, in tensor order as the caller holds it. Mirrored by oracle/oracle.py. */
typedef struct {
    int32_t beam;          /* ORC_PARALLEL, ORC_FAN (2-D), ORC_CONE, ORC_PARALLEL3D (3-D) */
    int32_t pad_;
    int64_t D, H, W;       /* volume shape; 2-D beams: D == 1                     */
    double dz, dy, dx;     /* voxel pitch; 2-D beams ignore dz                    */
    double cx, cy, cz;     /* world position of the volume centre                */
    int64_t views, rows, cols;
    double du, dv;         /* detector pitch along eu (cols) and ev (rows)       */
} orc_geom;

typedef struct {
    const double *src, *det, *eu, *ev;   /* [views][rank]; ev NULL for 2-D beams */
} orc_traj;

/* ---------------------------------------------------------------------------------------- */
/* Box and ray                                                                               */

typedef struct {
    int rank;
    int64_t n[3];          /* cells per world axis (x, y, z) */
    double pitch[3];
    double lo[3], hi[3];
} box_t;

typedef struct {
    double a[3];           /* start point (fan/cone: source; parallel: pixel)         */
    double d[3];           /* direction   (fan/cone: pixel - source; parallel: r)      */
    double tmin, tmax;     /* parameter range before clipping                         */
} ray_t;

static int rank_of(const orc_geom *g) {
    return g->beam == ORC_CONE || g->beam == ORC_PARALLEL3D ? 3 : 2;
}

/* Parallel beams (2-D and 3-D) have infinite lines for rays; fan and cone have segments. */
static int is_line(const orc_geom *g) {
    return g->beam == ORC_PARALLEL || g->beam == ORC_PARALLEL3D;
}

static void make_box(const orc_geom *g, box_t *b) {
    b->rank = rank_of(g);
    b->n[0] = g->W; b->n[1] = g->H; b->n[2] = g->D;
    b->pitch[0] = g->dx; b->pitch[1] = g->dy; b->pitch[2] = g->dz;
    const double c[3] = { g->cx, g->cy, g->cz };
    for (int a = 0; a < 3; ++a) {
        b->lo[a] = c[a] - 0.5 * (double)b->n[a] * b->pitch[a];
        b->hi[a] = c[a] + 0.5 * (double)b->n[a] * b->pitch[a];
    }
}

static void make_ray(const orc_geom *g, const orc_traj *t, int64_t view, int64_t row,
                     int64_t col, ray_t *r) {
    const int R = rank_of(g);
    const double u = ((double)col - 0.5 * (double)(g->cols - 1)) * g->du;
    const double v = ((double)row - 0.5 * (double)(g->rows - 1)) * g->dv;
    double p[3] = { 0, 0, 0 };
    for (int a = 0; a < R; ++a) {
        p[a] = t->det[view * R + a] + u * t->eu[view * R + a];
        if (R == 3) p[a] += v * t->ev[view * R + a];
    }
    for (int a = 0; a < 3; ++a) { r->a[a] = 0.0; r->d[a] = 0.0; }
    if (is_line(g)) {
        for (int a = 0; a < R; ++a) { r->a[a] = p[a]; r->d[a] = t->src[view * R + a]; }
        r->tmin = -INFINITY; r->tmax = INFINITY;
    } else {
        for (int a = 0; a < R; ++a) {
            r->a[a] = t->src[view * R + a];
            r->d[a] = p[a] - t->src[view * R + a];
        }
        r->tmin = 0.0; r->tmax = 1.0;
    }
}

static double norm_of(const double *d, int R) {
    double s = 0.0;
    for (int a = 0; a < R; ++a) s += d[a] * d[a];
    return sqrt(s);
}

/* Clip a ray's parameter range to the axis-aligned box [lo, hi) (slab intersection).
   Returns 0 when the ray misses or only touches the box. */
static int clip(const ray_t *r, int R, const double *lo, const double *hi,
                double *t0, double *t1) {
    double amin = r->tmin, amax = r->tmax;
    for (int a = 0; a < R; ++a) {
        if (r->d[a] != 0.0) {
            double s1 = (lo[a] - r->a[a]) / r->d[a];
            double s2 = (hi[a] - r->a[a]) / r->d[a];
            double smin = s1 < s2 ? s1 : s2, smax = s1 < s2 ? s2 : s1;
            if (smin > amin) amin = smin;
            if (smax < amax) amax = smax;
        } else if (r->a[a] < lo[a] || r->a[a] >= hi[a]) {
            return 0;
        }
    }
    if (!(amax > amin)) return 0;
    *t0 = amin; *t1 = amax;
    return 1;
}

/* ---------------------------------------------------------------------------------------- */
/* Siddon: sorted plane-crossing parameters per axis, merged, midpoint cells.               */

typedef struct {
    int64_t m, m_end, step;    /* next plane index, one past the last, +1 / -1 */
    double next;               /* parameter of plane m (INFINITY when exhausted) */
} plane_list;

static double plane_param(const ray_t *r, const box_t *b, int a, int64_t m) {
    return (b->lo[a] + (double)m * b->pitch[a] - r->a[a]) / r->d[a];
}

/* Advance list `L` of axis `a` to its first plane with parameter strictly inside (t0, t1). */
static void list_seek(plane_list *L, const ray_t *r, const box_t *b, int a, double t0, double t1) {
    for (;;) {
        if (L->m == L->m_end) { L->next = INFINITY; return; }
        double t = plane_param(r, b, a, L->m);
        if (t > t0 && t < t1) { L->next = t; return; }
        if (t >= t1) { L->next = INFINITY; L->m = L->m_end; return; }
        L->m += L->step;
    }
}

static void list_init(plane_list *L, const ray_t *r, const box_t *b, int a, double t0, double t1) {
    if (a >= b->rank || r->d[a] == 0.0) { L->m = L->m_end = 0; L->step = 1; L->next = INFINITY; return; }
    /* plane coordinates (in units of pitch) of the clipped endpoints, widened by one plane
       so rounding cannot drop a crossing; list_seek filters by the strict parameter test. */
    double s0 = (r->a[a] + t0 * r->d[a] - b->lo[a]) / b->pitch[a];
    double s1 = (r->a[a] + t1 * r->d[a] - b->lo[a]) / b->pitch[a];
    double smin = s0 < s1 ? s0 : s1, smax = s0 < s1 ? s1 : s0;
    int64_t mlo = (int64_t)floor(smin) - 1, mhi = (int64_t)ceil(smax) + 1;
    if (mlo < 0) mlo = 0;
    if (mhi > b->n[a]) mhi = b->n[a];
    if (r->d[a] > 0) { L->m = mlo; L->m_end = mhi + 1; L->step = 1; }
    else             { L->m = mhi; L->m_end = mlo - 1; L->step = -1; }
    list_seek(L, r, b, a, t0, t1);
}

static void list_pop(plane_list *L, const ray_t *r, const box_t *b, int a, double t0, double t1) {
    L->m += L->step;
    list_seek(L, r, b, a, t0, t1);
}

static int64_t flat_index(const box_t *b, const int64_t *c) {
    return (c[2] * b->n[1] + c[1]) * b->n[0] + c[0];   /* tensor (D, H, W), C order */
}

/* Enumerate the positive-length segments of a ray. For each, `visit(ctx, cell, len)`.
   Returns the number of segments. */
typedef void (*seg_visit)(void *ctx, int64_t cell, double len);

static int64_t siddon(const box_t *b, const ray_t *r, seg_visit visit, void *ctx) {
    const int R = b->rank;
    double t0, t1;
    if (!clip(r, R, b->lo, b->hi, &t0, &t1)) return 0;
    const double dn = norm_of(r->d, R);
    plane_list L[3];
    for (int a = 0; a < 3; ++a) list_init(&L[a], r, b, a, t0, t1);
    int64_t count = 0;
    double prev = t0;
    for (;;) {
        /* merge step: smallest head of the three sorted lists, or the exit parameter */
        int amin = -1;
        double cur = t1;
        for (int a = 0; a < R; ++a)
            if (L[a].next < cur) { cur = L[a].next; amin = a; }
        if (cur > prev) {
            double mid = 0.5 * (prev + cur);
            int64_t c[3] = { 0, 0, 0 };
            for (int a = 0; a < R; ++a) {
                double q = r->a[a] + mid * r->d[a];
                int64_t k = (int64_t)floor((q - b->lo[a]) / b->pitch[a]);
                if (k < 0) k = 0;
                if (k > b->n[a] - 1) k = b->n[a] - 1;
                c[a] = k;
            }
            visit(ctx, flat_index(b, c), (cur - prev) * dn);
            ++count;
        }
        if (amin < 0) break;
        prev = cur;
        list_pop(&L[amin], r, b, amin, t0, t1);
    }
    return count;
}

/* ---------------------------------------------------------------------------------------- */
/* Validation (argument shape only; geometry checks live in the library under test).        */

static int check(const orc_geom *g, const orc_traj *t) {
    if (!g || !t || !t->src || !t->det || !t->eu) return ORC_EINVAL;
    if (g->beam != ORC_PARALLEL && g->beam != ORC_FAN && g->beam != ORC_CONE &&
        g->beam != ORC_PARALLEL3D)
        return ORC_EINVAL;
    if (rank_of(g) == 3 && !t->ev) return ORC_EINVAL;
    if (rank_of(g) == 2 && (g->D != 1 || g->rows != 1)) return ORC_EINVAL;
    if (g->D < 1 || g->H < 1 || g->W < 1 || g->views < 0 || g->rows < 1 || g->cols < 1)
        return ORC_EINVAL;
    if (!(g->dx > 0) || !(g->dy > 0) || !(g->dz > 0)) return ORC_EINVAL;
    return ORC_OK;
}

static int threads_or_default(int n) {
#ifdef _OPENMP
    return n > 0 ? n : omp_get_max_threads();
#else
    (void)n;
    return 1;
#endif
}

/* ---------------------------------------------------------------------------------------- */
/* Forward                                                                                   */

typedef struct {
    const float *vol;      /* [B][D][H][W] */
    int64_t nvox, batch;
    double *acc;           /* [B] */
} fwd_ctx;

static void fwd_visit(void *p, int64_t cell, double len) {
    fwd_ctx *c = (fwd_ctx *)p;
    for (int64_t b = 0; b < c->batch; ++b)
        c->acc[b] += len * (double)c->vol[b * c->nvox + cell];
}

/* Rays given by flat id  view*rows*cols + row*cols + col.  out[B][n], counts[n] (or NULL). */
int orc_project_rays(const orc_geom *g, const double *src, const double *det, const double *eu,
                     const double *ev, const float *vol, int64_t batch, const int64_t *ray_ids,
                     int64_t n, double *out, int64_t *counts, int nthreads) {
    orc_traj t = { src, det, eu, ev };
    int rc = check(g, &t);
    if (rc) return rc;
    if (batch < 0 || (n > 0 && (!ray_ids || !out)) || (batch > 0 && !vol)) return ORC_EINVAL;
    box_t b;
    make_box(g, &b);
    const int64_t nvox = g->D * g->H * g->W;
    const int64_t per_view = g->rows * g->cols;
    const int64_t nrays = g->views * per_view;
    for (int64_t i = 0; i < n; ++i)
        if (ray_ids[i] < 0 || ray_ids[i] >= nrays) return ORC_EINVAL;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 64) num_threads(threads_or_default(nthreads))
    for (int64_t i = 0; i < n; ++i) {
        int64_t id = ray_ids[i];
        ray_t r;
        make_ray(g, &t, id / per_view, (id % per_view) / g->cols, id % g->cols, &r);
        double accbuf[64];
        double *acc = batch <= 64 ? accbuf : (double *)calloc((size_t)batch, sizeof(double));
        if (!acc) { bad = 1; continue; }
        for (int64_t k = 0; k < batch; ++k) acc[k] = 0.0;
        fwd_ctx c = { vol, nvox, batch, acc };
        int64_t cnt = siddon(&b, &r, fwd_visit, &c);
        for (int64_t k = 0; k < batch; ++k) out[k * n + i] = acc[k];
        if (counts) counts[i] = cnt;
        if (acc != accbuf) free(acc);
    }
    return bad ? ORC_ENOMEM : ORC_OK;
}

/* Full forward: sino[B][views][rows][cols] (fp64), counts[views*rows*cols] (or NULL). */
int orc_project(const orc_geom *g, const double *src, const double *det, const double *eu,
                const double *ev, const float *vol, int64_t batch, double *sino,
                int64_t *counts, int nthreads) {
    orc_traj t = { src, det, eu, ev };
    int rc = check(g, &t);
    if (rc) return rc;
    if (batch < 0 || (batch > 0 && (!vol || !sino))) return ORC_EINVAL;
    box_t b;
    make_box(g, &b);
    const int64_t nvox = g->D * g->H * g->W;
    const int64_t nrays = g->views * g->rows * g->cols;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 256) num_threads(threads_or_default(nthreads))
    for (int64_t id = 0; id < nrays; ++id) {
        ray_t r;
        const int64_t per_view = g->rows * g->cols;
        make_ray(g, &t, id / per_view, (id % per_view) / g->cols, id % g->cols, &r);
        double accbuf[64];
        double *acc = batch <= 64 ? accbuf : (double *)calloc((size_t)batch, sizeof(double));
        if (!acc) { bad = 1; continue; }
        for (int64_t k = 0; k < batch; ++k) acc[k] = 0.0;
        fwd_ctx c = { vol, nvox, batch, acc };
        int64_t cnt = siddon(&b, &r, fwd_visit, &c);
        for (int64_t k = 0; k < batch; ++k) sino[k * nrays + id] = acc[k];
        if (counts) counts[id] = cnt;
        if (acc != accbuf) free(acc);
    }
    return bad ? ORC_ENOMEM : ORC_OK;
}

/* ---------------------------------------------------------------------------------------- */
/* Adjoint by scattering along the same segments                                             */

typedef struct {
    double *vol;           /* private [B][nvox] */
    int64_t nvox, batch;
    const double *w;       /* [B] ray values */
} bwd_ctx;

static void bwd_visit(void *p, int64_t cell, double len) {
    bwd_ctx *c = (bwd_ctx *)p;
    for (int64_t b = 0; b < c->batch; ++b)
        c->vol[b * c->nvox + cell] += len * c->w[b];
}

/* Full adjoint: vol_out[B][D][H][W] (fp64) = sum over rays. Deterministic for a given
   thread count: views are split statically, each thread scatters into a private volume, and
   the private volumes are summed in thread order. */
int orc_backproject(const orc_geom *g, const double *src, const double *det, const double *eu,
                    const double *ev, const float *sino, int64_t batch, double *vol_out,
                    int nthreads) {
    orc_traj t = { src, det, eu, ev };
    int rc = check(g, &t);
    if (rc) return rc;
    if (batch < 0 || (batch > 0 && (!sino || !vol_out))) return ORC_EINVAL;
    box_t b;
    make_box(g, &b);
    const int64_t nvox = g->D * g->H * g->W;
    const int64_t per_view = g->rows * g->cols;
    const int64_t nrays = g->views * per_view;
    const int T = threads_or_default(nthreads);
    double **priv = (double **)calloc((size_t)T, sizeof(double *));
    if (!priv) return ORC_ENOMEM;
    int bad = 0;
    for (int i = 0; i < T; ++i) {
        priv[i] = (double *)calloc((size_t)(batch * nvox > 0 ? batch * nvox : 1), sizeof(double));
        if (!priv[i]) bad = 1;
    }
    if (!bad) {
#pragma omp parallel num_threads(T)
        {
#ifdef _OPENMP
            int me = omp_get_thread_num();
#else
            int me = 0;
#endif
            double wbuf[64];
            double *w = batch <= 64 ? wbuf : (double *)calloc((size_t)batch, sizeof(double));
#pragma omp for schedule(static)
            for (int64_t view = 0; view < g->views; ++view) {
                if (!w) continue;
                for (int64_t k = 0; k < per_view; ++k) {
                    int64_t id = view * per_view + k;
                    ray_t r;
                    make_ray(g, &t, view, k / g->cols, k % g->cols, &r);
                    for (int64_t bb = 0; bb < batch; ++bb) w[bb] = (double)sino[bb * nrays + id];
                    bwd_ctx c = { priv[me], nvox, batch, w };
                    siddon(&b, &r, bwd_visit, &c);
                }
            }
            if (!w) bad = 1;
            if (w && w != wbuf) free(w);
        }
        if (!bad) {
            for (int64_t i = 0; i < batch * nvox; ++i) {
                double s = 0.0;
                for (int k = 0; k < T; ++k) s += priv[k][i];
                vol_out[i] = s;
            }
        }
    }
    for (int i = 0; i < T; ++i) free(priv[i]);
    free(priv);
    return bad ? ORC_ENOMEM : ORC_OK;
}

/* ---------------------------------------------------------------------------------------- */
/* Adjoint at chosen voxels, straight from the definition                                    */
/*                                                                                           */
/* Bp[v] = sum_r len(r, v) * y[r], with len(r, v) the chord of ray r through voxel v's own  */
/* box. Candidate rays per view are the pixels inside the detector bounding box of the      */
/* voxel's corners (central projection for fan/cone, projection along the ray direction for  */
/* parallel beams), widened by one pixel. When a corner does not project in front of the    */
/* source, every pixel of that view is tried.                                                */

static int solve3(const double A[3][3], const double rhs[3], double x[3]) {
    double det = A[0][0] * (A[1][1] * A[2][2] - A[1][2] * A[2][1])
               - A[0][1] * (A[1][0] * A[2][2] - A[1][2] * A[2][0])
               + A[0][2] * (A[1][0] * A[2][1] - A[1][1] * A[2][0]);
    if (det == 0.0 || !isfinite(det)) return 0;
    for (int c = 0; c < 3; ++c) {
        double M[3][3];
        memcpy(M, A, sizeof(M));
        for (int r = 0; r < 3; ++r) M[r][c] = rhs[r];
        x[c] = (M[0][0] * (M[1][1] * M[2][2] - M[1][2] * M[2][1])
              - M[0][1] * (M[1][0] * M[2][2] - M[1][2] * M[2][0])
              + M[0][2] * (M[1][0] * M[2][1] - M[1][1] * M[2][0])) / det;
    }
    return 1;
}

/* Detector coordinates (u, v) where the ray through world point c meets the detector, and
   the ray parameter ratio (must be > 0 for fan/cone). Returns 0 if degenerate. */
static int project_point(const orc_geom *g, const orc_traj *t, int64_t view, const double *c,
                         double *u, double *v, double *s) {
    const int R = rank_of(g);
    const double *src = t->src + view * R, *det = t->det + view * R, *eu = t->eu + view * R;
    if (R == 2) {
        /* det + u*eu - s*w = base, with (w, base) = (r, c) parallel or (c - src, src) fan */
        double w[2], base[2];
        for (int a = 0; a < 2; ++a) {
            w[a] = g->beam == ORC_PARALLEL ? src[a] : c[a] - src[a];
            base[a] = g->beam == ORC_PARALLEL ? c[a] : src[a];
        }
        double A00 = eu[0], A01 = -w[0], A10 = eu[1], A11 = -w[1];
        double r0 = base[0] - det[0], r1 = base[1] - det[1];
        double dd = A00 * A11 - A01 * A10;
        if (dd == 0.0) return 0;
        *u = (r0 * A11 - A01 * r1) / dd;
        *s = (A00 * r1 - r0 * A10) / dd;
        *v = 0.0;
        return 1;
    }
    /* det + u*eu + v*ev = base + s*w, with (w, base) = (r, c) for a parallel beam (the line
       through c along the ray direction r) or (c - src, src) for a cone (the ray from the
       source through c) */
    const double *ev = t->ev + view * 3;
    double A[3][3], rhs[3], x[3];
    for (int a = 0; a < 3; ++a) {
        const double w = is_line(g) ? src[a] : c[a] - src[a];
        const double base = is_line(g) ? c[a] : src[a];
        A[a][0] = eu[a]; A[a][1] = ev[a]; A[a][2] = -w;
        rhs[a] = base - det[a];
    }
    if (!solve3(A, rhs, x)) return 0;
    *u = x[0]; *v = x[1]; *s = x[2];
    return 1;
}

int orc_backproject_voxels(const orc_geom *g, const double *src, const double *det,
                           const double *eu, const double *ev, const float *sino,
                           int64_t batch, const int64_t *vox_ids, int64_t n, double *out,
                           int nthreads) {
    orc_traj t = { src, det, eu, ev };
    int rc = check(g, &t);
    if (rc) return rc;
    if (batch < 0 || (n > 0 && (!vox_ids || !out)) || (batch > 0 && !sino)) return ORC_EINVAL;
    box_t b;
    make_box(g, &b);
    const int R = b.rank;
    const int64_t nvox = g->D * g->H * g->W;
    const int64_t per_view = g->rows * g->cols;
    const int64_t nrays = g->views * per_view;
    for (int64_t i = 0; i < n; ++i)
        if (vox_ids[i] < 0 || vox_ids[i] >= nvox) return ORC_EINVAL;
#pragma omp parallel for schedule(dynamic, 4) num_threads(threads_or_default(nthreads))
    for (int64_t i = 0; i < n; ++i) {
        const int64_t id = vox_ids[i];
        const int64_t c3[3] = { id % g->W, (id / g->W) % g->H, id / (g->W * g->H) };
        double vlo[3] = { 0, 0, 0 }, vhi[3] = { 0, 0, 0 };
        for (int a = 0; a < 3; ++a) {
            vlo[a] = b.lo[a] + (double)c3[a] * b.pitch[a];
            vhi[a] = b.lo[a] + (double)(c3[a] + 1) * b.pitch[a];
        }
        for (int64_t k = 0; k < batch; ++k) out[k * n + i] = 0.0;
        for (int64_t view = 0; view < g->views; ++view) {
            /* bounding box of corner projections in fractional pixel indices */
            double jlo = INFINITY, jhi = -INFINITY, klo = INFINITY, khi = -INFINITY;
            int ok = 1;
            const int ncorner = R == 3 ? 8 : 4;
            for (int m = 0; m < ncorner && ok; ++m) {
                double c[3] = { (m & 1) ? vhi[0] : vlo[0], (m & 2) ? vhi[1] : vlo[1],
                                (m & 4) ? vhi[2] : vlo[2] };
                double u, v, s;
                if (!project_point(g, &t, view, c, &u, &v, &s)) { ok = 0; break; }
                if (!is_line(g) && !(s > 0.0)) { ok = 0; break; }
                double jj = u / g->du + 0.5 * (double)(g->cols - 1);
                double kk = R == 3 ? v / g->dv + 0.5 * (double)(g->rows - 1) : 0.0;
                if (jj < jlo) jlo = jj;
                if (jj > jhi) jhi = jj;
                if (kk < klo) klo = kk;
                if (kk > khi) khi = kk;
            }
            int64_t j0 = 0, j1 = g->cols - 1, k0 = 0, k1 = g->rows - 1;
            if (ok) {
                double fj0 = floor(jlo) - 1, fj1 = ceil(jhi) + 1;
                double fk0 = floor(klo) - 1, fk1 = ceil(khi) + 1;
                if (fj1 < 0 || fj0 > (double)(g->cols - 1) || fk1 < 0 || fk0 > (double)(g->rows - 1))
                    continue;
                j0 = fj0 < 0 ? 0 : (int64_t)fj0;
                j1 = fj1 > (double)(g->cols - 1) ? g->cols - 1 : (int64_t)fj1;
                k0 = fk0 < 0 ? 0 : (int64_t)fk0;
                k1 = fk1 > (double)(g->rows - 1) ? g->rows - 1 : (int64_t)fk1;
            }
            for (int64_t k = k0; k <= k1; ++k) {
                for (int64_t j = j0; j <= j1; ++j) {
                    ray_t r;
                    make_ray(g, &t, view, k, j, &r);
                    double t0, t1;
                    if (!clip(&r, R, vlo, vhi, &t0, &t1)) continue;
                    double len = (t1 - t0) * norm_of(r.d, R);
                    int64_t ray = view * per_view + k * g->cols + j;
                    for (int64_t bb = 0; bb < batch; ++bb)
                        out[bb * n + i] += len * (double)sino[bb * nrays + ray];
                }
            }
        }
    }
    return ORC_OK;
}

/* ---------------------------------------------------------------------------------------- */
/* One ray's segment list (tests build small dense system matrices from it).                */

typedef struct {
    int64_t *cells;
    double *lens;
    int64_t cap, n;
} list_ctx;

static void list_visit(void *p, int64_t cell, double len) {
    list_ctx *c = (list_ctx *)p;
    if (c->n < c->cap) { c->cells[c->n] = cell; c->lens[c->n] = len; }
    c->n++;
}

/* Returns the number of segments (which may exceed `cap`; only `cap` are stored). */
int64_t orc_ray_segments(const orc_geom *g, const double *src, const double *det,
                         const double *eu, const double *ev, int64_t view, int64_t row,
                         int64_t col, int64_t *cells, double *lens, int64_t cap) {
    orc_traj t = { src, det, eu, ev };
    if (check(g, &t)) return ORC_EINVAL;
    if (view < 0 || view >= g->views || row < 0 || row >= g->rows || col < 0 || col >= g->cols)
        return ORC_EINVAL;
    box_t b;
    make_box(g, &b);
    ray_t r;
    make_ray(g, &t, view, row, col, &r);
    list_ctx c = { cells, lens, cap, 0 };
    siddon(&b, &r, list_visit, &c);
    return c.n;
}

int orc_max_threads(void) { return threads_or_default(0); }
