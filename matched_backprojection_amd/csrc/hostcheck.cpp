// hostcheck.cpp -- CPU replay of the GPU walks (test harness, not part of the library).
//
// Compiles traverse.h for the host and runs the generic and the column walk over every ray
// of a geometry, checking each visited cell index against the volume bounds and each length
// for sign. Tests use it to show that a launch configuration stays in bounds before it runs
// on a GPU, and to check the walk logic against the fp64 oracle on the CPU. It shares the
// traversal code with the HIP kernels, so agreement here is a logic check, not parity.
#include <stdint.h>

#include <algorithm>
#include <climits>
#include <cmath>
#include <utility>
#include <vector>

#include "traverse.h"

using namespace mbp;

namespace {

struct Checked {
    const Box* B;
    long long* violations;
    bool ok(int32_t cx, int32_t cy, int32_t cz, float len) const {
        const bool in = cx >= 0 && cx < B->n[0] && cy >= 0 && cy < B->n[1] && cz >= 0 && cz < B->n[2];
        if (!in || !(len >= 0.0f) || !std::isfinite(len)) {
            ++*violations;
            return false;
        }
        return true;
    }
};

void frames_from(const double* f, int views, std::vector<Frame>& out) {
    out.resize((size_t)views);
    for (int i = 0; i < views; ++i)
        for (int a = 0; a < 3; ++a) {
            out[i].s[a] = f[i * 12 + a];
            out[i].c[a] = f[i * 12 + 3 + a];
            out[i].u[a] = f[i * 12 + 6 + a];
            out[i].v[a] = f[i * 12 + 9 + a];
        }
}

Box box_from(const double* lo, const double* pitch, const int32_t* n) {
    Box B;
    for (int a = 0; a < 3; ++a) {
        B.lo[a] = lo[a];
        B.pitch[a] = pitch[a];
        B.n[a] = n[a];
        B.hi[a] = lo[a] + (double)n[a] * pitch[a];
    }
    return B;
}

}  // namespace

extern "C" {

// Forward projection with the generic (path 1) or column (path 2) walk. frames: views x 12
// doubles (s, c, u, v); volume element (x, y, z) at x*sx + y*sy + z*sz. Outputs the fp32
// sinogram [views][rows][cols], per-ray counts of segments longer than 1e-6 min pitch, and the number of bound violations.
// With orbit 2 or 4 (the generic walk; dir: the quarter turn's sense), the rays of the first
// views / orbit views are walked as the kernel shares them over a turn symmetry of the views
// (walk_ray_orbit), each also giving the rays of the views views / orbit apart.
int mbph_project(int path, const double* frames, int beam, const double* lo, const double* hi,
                 const double* pitch, const int32_t* n, int views, int rows, int cols,
                 double du, double dv, const float* vol, int64_t sx, int64_t sy, int64_t sz,
                 float* sino, int64_t* counts, long long* violations, int orbit, int dir) {
    (void)hi;
    std::vector<Frame> F;
    frames_from(frames, views, F);
    const Box B = box_from(lo, pitch, n);
    *violations = 0;
    Checked chk{&B, violations};
    const float eps = (float)(1e-6 * std::fmin(B.pitch[0], std::fmin(B.pitch[1], B.pitch[2])));
    if (orbit > 1) {
        if (path != 1) return -1;
        const int q = views / orbit;
        const int64_t vox = (int64_t)n[0] * n[1] * n[2];
        int32_t base[4] = {0, 0, 0, 0}, tx[4] = {0, 0, 0, 0}, ty[4] = {0, 0, 0, 0};
        for (int m = 0; m < orbit; ++m)
            orbit_strides(orbit, dir, n[0], n[1], (int32_t)sx, (int32_t)sy, m, base[m], tx[m], ty[m]);
        for (int i = 0; i < q; ++i)
            for (int j = 0; j < cols; ++j)
                for (int k = 0; k < rows; ++k) {
                    RayWalk r;
                    ray_setup(F[i], B, beam, centred(j, cols, du), centred(k, rows, dv), r);
                    float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
                    int64_t cnt = 0;
                    auto visit = [&](const int32_t* off, float len) {
                        if (len > eps) ++cnt;
                        for (int m = 0; m < orbit; ++m) {
                            if (off[m] < 0 || off[m] >= vox || !(len >= 0.0f)) { ++*violations; continue; }
                            acc[m] = fmaf(len, vol[off[m]], acc[m]);
                        }
                    };
                    if (orbit == 2) {
                        auto v2 = [&](const int32_t (&off)[2], float len) { visit(off, len); };
                        const int32_t b2[2] = {base[0], base[1]}, x2[2] = {tx[0], tx[1]}, y2[2] = {ty[0], ty[1]};
                        walk_ray_orbit<2>(r, b2, x2, y2, (int32_t)sz, v2);
                    } else {
                        auto v4 = [&](const int32_t (&off)[4], float len) { visit(off, len); };
                        walk_ray_orbit<4>(r, base, tx, ty, (int32_t)sz, v4);
                    }
                    for (int m = 0; m < orbit; ++m) {
                        const int64_t ray = ((int64_t)(i + m * q) * rows + k) * cols + j;
                        sino[ray] = acc[m];
                        if (counts) counts[ray] = cnt;
                    }
                }
        return 0;
    }
    for (int i = 0; i < views; ++i) {
        for (int j = 0; j < cols; ++j) {
            ColumnWalk c;
            if (path == 2) column_setup(F[i], B, beam, centred(j, cols, du), c);
            for (int k = 0; k < rows; ++k) {
                float acc = 0.0f;
                int64_t cnt = 0;
                auto visit = [&](int32_t cx, int32_t cy, int32_t cz, float len) {
                    if (len > eps) ++cnt;
                    if (!chk.ok(cx, cy, cz, len)) return;
                    acc = fmaf(len, vol[cx * sx + cy * sy + cz * sz], acc);
                };
                float scale = 1.0f;
                if (path == 2) {
                    RowWalk r;
                    row_setup(c, B, centred(k, rows, dv), F[i].v[2], r);
                    walk_column_row(c, r, visit);
                    scale = r.kappa;
                } else {
                    RayWalk r;
                    ray_setup(F[i], B, beam, centred(j, cols, du), centred(k, rows, dv), r);
                    // the forward kernel's walk keeps the element offset instead of the cell:
                    // it must name the same cells with the same lengths, in the same order
                    std::vector<std::pair<int64_t, float>> cells;
                    auto record = [&](int32_t cx, int32_t cy, int32_t cz, float len) {
                        cells.emplace_back(cx * sx + cy * sy + cz * sz, len);
                        visit(cx, cy, cz, len);
                    };
                    walk_ray(r, record);
                    size_t q = 0;
                    auto same = [&](int32_t off, float len) {
                        if (q >= cells.size() || cells[q].first != off || cells[q].second != len) ++*violations;
                        ++q;
                    };
                    walk_ray_offsets(r, (int32_t)sx, (int32_t)sy, (int32_t)sz, same);
                    if (q != cells.size()) ++*violations;
                }
                const int64_t ray = ((int64_t)i * rows + k) * cols + j;
                sino[ray] = acc * scale;
                if (counts) counts[ray] = cnt;
            }
        }
    }
    return 0;
}

// Forward projection with the chunked column walk of the forward kernel: per column, the
// 64 lanes' entries of each chunk of merged xy crossings are filled one lane after another,
// then every row consumes them (the kernel does the same with one wave per 64 rows). orbit > 1
// (2 or 4, with the quarter turn's sense dir): the walks of the first views / orbit views
// also give the rays of the views views / orbit apart from the turned cells (orbit_columns),
// as the kernel shares them over a turn symmetry of the views.
int mbph_project_chunked(const double* frames, int beam, const double* lo, const double* pitch,
                         const int32_t* n, int views, int rows, int cols, double du, double dv,
                         const float* vol, float* sino, long long* violations, int orbit, int dir) {
    std::vector<Frame> F;
    frames_from(frames, views, F);
    const Box B = box_from(lo, pitch, n);
    *violations = 0;
    const int32_t H = n[1], D = n[2];
    const uint32_t WH1 = (uint32_t)n[0] * (uint32_t)H - 1u;
    const int q = views / orbit;
    std::vector<XYEvent> E(kXYChunk);
    std::vector<int32_t> T(kXYChunk);
    std::vector<std::vector<XYEvent>> chunks;
    std::vector<std::vector<int32_t>> turns;     // quarter turn: each event's turned column
    for (int i = 0; i < q; ++i) {
        for (int j = 0; j < cols; ++j) {
            ColumnWalk c;
            column_setup(F[i], B, beam, centred(j, cols, du), c);
            // the column's chunks, as one wave builds them
            chunks.clear();
            turns.clear();
            std::vector<int32_t> counts;
            int32_t final_cxy = 0, final_c1 = 0;
            if (c.hit) {
                const int32_t total = c.x.steps + c.y.steps;
                int32_t done = 0, kx0 = 0, ky0 = 0;
                while (done < total) {
                    const int32_t count = total - done < kXYChunk ? total - done : kXYChunk;
                    for (auto& e : E) { e.tb = NAN; e.cxy = -1; }
                    for (auto& t : T) t = -1;
                    int32_t a = 0;
                    for (int lane = 0; lane < 64; ++lane)
                        a += xy_chunk_fill(c, H, kx0, ky0, count, lane, E.data(), orbit == 4 ? T.data() : nullptr,
                                           n[0], dir);
                    for (int32_t p = 0; p < count; ++p) {  // every position filled exactly once
                        if (E[p].cxy < 0 || E[p].cxy >= n[0] * H || !(E[p].tb == E[p].tb)) ++*violations;
                        if (orbit == 4 && (T[p] < 0 || T[p] >= n[0] * H)) ++*violations;
                    }
                    chunks.push_back(std::vector<XYEvent>(E.begin(), E.begin() + count));
                    turns.push_back(std::vector<int32_t>(T.begin(), T.begin() + count));
                    kx0 += a; ky0 += count - a; done += count;
                }
                if (kx0 != c.x.steps || ky0 != c.y.steps) ++*violations;
                const int32_t fx = c.x.c0 + c.x.step * c.x.steps, fy = c.y.c0 + c.y.step * c.y.steps;
                final_cxy = fx * H + fy;
                int32_t ox, oy;
                orbit_cell(4, dir, n[0], H, fx, fy, 1, ox, oy);
                final_c1 = ox * H + oy;
            }
            for (int k = 0; k < rows; ++k) {
                RowWalk r;
                row_setup(c, B, centred(k, rows, dv), F[i].v[2], r);
                float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
                int32_t c1 = 0;       // the turned column of the cell visited next
                auto visit = [&](int32_t cxy, int32_t cz, float len) {
                    if (cxy < 0 || cxy >= n[0] * H || cz < 0 || cz >= D || !(len >= 0.0f)) { ++*violations; return; }
                    uint32_t cell[4] = {(uint32_t)cxy, 0u, 0u, 0u};
                    if (orbit == 2) {
                        uint32_t o2[2];
                        orbit_columns<2>((uint32_t)cxy, 0u, WH1, o2);
                        cell[1] = o2[1];
                    } else if (orbit == 4) {
                        orbit_columns<4>((uint32_t)cxy, (uint32_t)c1, WH1, cell);
                    }
                    for (int m = 0; m < orbit; ++m) {
                        if (cell[m] >= (uint32_t)(n[0] * H)) { ++*violations; continue; }
                        const int32_t cx = (int32_t)cell[m] / H, cy = (int32_t)cell[m] % H;
                        acc[m] = fmaf(len, vol[((int64_t)cz * H + cy) * n[0] + cx], acc[m]);
                    }
                };
                if (c.hit) {
                    int32_t cz = r.z.c0, kz = 0;
                    double nz = r.z.steps > 0 ? r.z.t_first : INFINITY;
                    double ta = 0.0;
                    // rows meeting at most one z plane per xy cell take the grouped two-piece
                    // form for whole groups of a chunk, the general one for the rest
                    const bool two = row_single_crossing(r, B);
                    for (size_t ci = 0; ci < chunks.size(); ++ci) {
                        const auto& ch = chunks[ci];
                        const auto& tu = turns[ci];
                        const size_t grouped = two ? ch.size() / kCellGroup * kCellGroup : 0;
                        // chunks inside the row's slab (for this row; the kernel requires it of
                        // all 64 rows of a wave) take the clip-free form, with the next z
                        // crossing re-anchored at the chunk start and then stepped
                        const bool inside = !ch.empty() && r.t_lo <= ta && r.t_hi >= ch.back().tb &&
                                            stepped_walk_ok(r, kz, (int32_t)ch.size(), ch.back().tb);
                        std::vector<XYEvent> ce(ch);
                        const bool more = kz < r.z.steps;
                        const double t_first = more ? r.z.t_first : INFINITY;
                        const double t_step = more ? r.z.t_step : 0.0;
                        if (inside && grouped > 0) {
                            nz = more ? crossing(r.z, kz) : INFINITY;
                            for (int lane = 0; lane < 64; ++lane) xy_chunk_chords(ce.data(), (int32_t)ce.size(), ta, lane);
                        }
                        size_t p = 0;
                        for (; p < grouped; ++p) {
                            const double hi = fmin(ch[p].tb, r.t_hi);
                            int32_t z0, z1;
                            float l0, l1;
                            if (inside) {
                                if (nz < ta && kz < r.z.steps) ++*violations;   // a crossing left behind
                                z0 = cz;
                                const double nz_was = nz;
                                if (row_cell_two_counted(t_first, t_step, ce[p].tb, ce[p].chord, kz, nz, l0, l1))
                                    cz += r.z.step;
                                z1 = cz;
                                if (kz > r.z.steps) ++*violations;   // counted past the last plane
                                if (kz < r.z.steps && nz != crossing(r.z, kz)) ++*violations;
                                if (kz == r.z.steps && nz_was < ce[p].tb && !(nz > ch.back().tb)) ++*violations;
                                if (!(l0 >= 0.0f) || !(l1 >= 0.0f)) ++*violations;
                            } else {
                                row_cell_two(r, ta, ch[p].tb, cz, kz, nz, z0, l0, z1, l1);
                            }
                            if (nz < hi && fmax(ta, r.t_lo) < hi) ++*violations;   // a second crossing
                            c1 = tu[p];
                            if (l0 != 0.0f) visit(ch[p].cxy, z0, l0);
                            if (l1 != 0.0f) visit(ch[p].cxy, z1, l1);
                            ta = ch[p].tb;
                        }
                        if (inside && grouped > 0) nz = kz < r.z.steps ? crossing(r.z, kz) : INFINITY;
                        for (; p < ch.size(); ++p) {
                            c1 = tu[p];
                            row_cell(r, ta, ch[p].tb, ch[p].cxy, cz, kz, nz, visit);
                            ta = ch[p].tb;
                        }
                    }
                    c1 = final_c1;
                    row_cell(r, ta, c.T, final_cxy, cz, kz, nz, visit);
                }
                for (int m = 0; m < orbit; ++m)
                    sino[((int64_t)(i + m * q) * rows + k) * cols + j] = acc[m] * r.kappa;
            }
        }
    }
    return 0;
}

// Adjoint with the same walks, accumulated in fp64 on the host (order is deterministic).
int mbph_backproject(int path, const double* frames, int beam, const double* lo,
                     const double* hi, const double* pitch, const int32_t* n, int views,
                     int rows, int cols, double du, double dv, const float* sino, double* vol,
                     int64_t sx, int64_t sy, int64_t sz, long long* violations) {
    (void)hi;
    std::vector<Frame> F;
    frames_from(frames, views, F);
    const Box B = box_from(lo, pitch, n);
    *violations = 0;
    Checked chk{&B, violations};
    for (int i = 0; i < views; ++i) {
        for (int j = 0; j < cols; ++j) {
            ColumnWalk c;
            if (path == 2) column_setup(F[i], B, beam, centred(j, cols, du), c);
            for (int k = 0; k < rows; ++k) {
                const int64_t ray = ((int64_t)i * rows + k) * cols + j;
                double w = sino[ray];
                auto visit = [&](int32_t cx, int32_t cy, int32_t cz, float len) {
                    if (!chk.ok(cx, cy, cz, len)) return;
                    vol[cx * sx + cy * sy + cz * sz] += (double)len * w;
                };
                if (path == 2) {
                    RowWalk r;
                    row_setup(c, B, centred(k, rows, dv), F[i].v[2], r);
                    w *= (double)r.kappa;
                    walk_column_row(c, r, visit);
                } else {
                    RayWalk r;
                    ray_setup(F[i], B, beam, centred(j, cols, du), centred(k, rows, dv), r);
                    walk_ray(r, visit);
                }
            }
        }
    }
    return 0;
}

// Replays the gather adjoint item by item as the kernel forms items: per cell, view and
// crossing column one item, taken in the fast fixed-point form where the kernel takes it
// (rows of a lane relative to the lane's origin cell, shares in fp32 when `kernel_shares`,
// else in fp64 from the same integers) and in the fp64 general form otherwise; `general_only`
// takes every item in the general form. Sums in fp64. *violations counts pieces out of range
// and fast-form positions outside the fixed point's range; *fast counts fast items. orbit > 1
// (2 or 4, with the quarter turn's sense dir): items are formed as the kernel shares them over
// a turn symmetry of the views (orbit_cell), for the first views / orbit views only, each
// carrying the rows of the views q apart into the orbit's other cells.
int mbph_gather(const double* frames, int beam, const double* lo, const double* pitch,
                const int32_t* n, int views, int rows, int cols, double du, double dv,
                const float* sino, int kernel_shares, int general_only, double* vol,
                long long* violations, long long* fast, int orbit, int dir) {
    std::vector<Frame> F;
    frames_from(frames, views, F);
    const Box B = box_from(lo, pitch, n);
    *violations = 0;
    *fast = 0;
    std::vector<ColLine> lines((size_t)views * cols);
    for (int v = 0; v < views; ++v)
        for (int j = 0; j < cols; ++j) column_line(F[v], B, beam, j, cols, rows, du, dv, lines[(size_t)v * cols + j]);
    const bool line = beam == BEAM_PARALLEL;
    const int32_t S = gather_stride(rows), rows_pad = gather_rows_padded(rows), D = n[2];
    std::vector<double> w(rows_pad);
    // with an orbit (orbit_cell), the cells that stand for the orbits, each slot's cell in
    // turn, over the first q views; line (v + m q, j) then goes to slot (a + m) mod orbit
    int32_t Wr, Hr;
    orbit_grid(orbit, n[0], n[1], Wr, Hr);
    const int q = views / orbit;
    for (int ix = 0; ix < Wr; ++ix) {
        for (int iy = 0; iy < Hr; ++iy) {
          for (int a = 0; a < orbit; ++a) {
            int32_t cx, cy;
            orbit_cell(orbit, dir, n[0], n[1], ix, iy, a, cx, cy);
            const double x0 = B.lo[0] + cx * B.pitch[0], x1 = x0 + B.pitch[0];
            const double y0 = B.lo[1] + cy * B.pitch[1], y1 = y0 + B.pitch[1];
            int32_t tx = cx, ty = cy;     // the cell the current line's rows go to
            auto add = [&](int32_t iz, double share, double wk) {
                if (iz < 0 || iz >= D || !(share >= 0.0)) { ++*violations; return; }
                vol[((int64_t)iz * n[1] + ty) * n[0] + tx] += share * wk;
            };
            for (int v = 0; v < q; ++v) {
                int32_t j0, j1;
                if (!cell_column_range(F[v], beam, cols, du, x0, x1, y0, y1, j0, j1)) continue;
                if (j0 < 0 || j1 >= cols) ++*violations;
                for (int32_t j = j0; j <= j1; ++j) {
                    GatherItem it;
                    if (!gather_item(lines[(size_t)v * cols + j], line, x0, x1, y0, y1, S, rows,
                                     rows_pad, v * cols + j, it))
                        continue;
                    for (int m = 0; m < orbit; ++m) {
                        const int vw = v + m * q;
                        orbit_cell(orbit, dir, n[0], n[1], ix, iy, (a + m) % orbit, tx, ty);
                        // the reordered sinogram line: values times the ray length, zero padded
                        for (int k = 0; k < rows_pad; ++k) {
                            if (k >= rows) { w[k] = 0.0; continue; }
                            double len;
                            if (line) {
                                len = std::sqrt(F[vw].s[0] * F[vw].s[0] + F[vw].s[1] * F[vw].s[1] + F[vw].s[2] * F[vw].s[2]);
                            } else {
                                double p[3];
                                pixel_point(F[vw], centred(j, cols, du), centred(k, rows, dv), p);
                                const double ex = p[0] - F[vw].s[0], ey = p[1] - F[vw].s[1], ez = p[2] - F[vw].s[2];
                                len = std::sqrt(ex * ex + ey * ey + ez * ez);
                            }
                            w[k] = (double)sino[((int64_t)vw * rows + k) * cols + j] * len;
                        }
                        // the kernel carries the crossing length in fp32; the fp64 replay takes it
                        // from the clip again, and so the general form's positions (a fast item
                        // holds them in fixed point)
                        const ColLine& L = lines[(size_t)v * cols + j];
                        double t0, t1;
                        cell_clip(L, line, x0, x1, y0, y1, t0, t1);
                        const double dt = kernel_shares ? (double)it.dt : t1 - t0;
                        const double za0 = L.c0 + t0 * L.c1, za1 = L.c2 + t0 * L.c3;
                        const double zb0 = L.c0 + t1 * L.c1, zb1 = L.c2 + t1 * L.c3;
                        if (it.form > 0 && !general_only) {
                            if (m == 0) ++*fast;
                            for (int32_t g0 = 0; g0 < rows_pad; g0 += 64 * S)
                                for (int lane = 0; lane < 64; ++lane) {
                                    const int32_t k0 = g0 + S * lane;
                                    const int32_t c0 = fast_origin_row(S);
                                    uint32_t la, lb;
                                    int32_t base;
                                    fast_origin(it, k0 + c0, -1, la, lb, base);
                                    for (int32_t c = 0; c < S; ++c) {
                                        // the row's ends must stay inside the fixed point's range
                                        const int64_t pa = (int64_t)la + (int64_t)(c - c0) * it.a1fx;
                                        const int64_t pb = (int64_t)lb + (int64_t)(c - c0) * it.b1fx;
                                        if (pa < 0 || pa > (int64_t)UINT32_MAX || pb < 0 || pb > (int64_t)UINT32_MAX)
                                            ++*violations;
                                        int32_t fb;
                                        uint32_t num, ext;
                                        fast_row((uint32_t)pa, (uint32_t)pb, fb, num, ext);
                                        // both shares from integers: the lower cell's num / ext and
                                        // the upper one's (ext - num) / ext
                                        double f = 1.0, g = 0.0;
                                        if (num < ext) {
                                            if (kernel_shares) {
                                                const float r = 1.0f / (float)ext;
                                                f = (double)((float)num * r);
                                                g = (double)((float)(ext - num) * r);
                                            } else {
                                                f = (double)num / (double)ext;
                                                g = (double)(ext - num) / (double)ext;
                                            }
                                        }
                                        const int32_t i0 = base + fb;
                                        if ((uint32_t)i0 > (uint32_t)D) continue;     // outside: discarded
                                        const int32_t z = i0 - 1;                      // cell of index i0
                                        const double wk = w[k0 + c];
                                        if (z >= 0) add(z, f * dt, wk);
                                        if (z + 1 < D) add(z + 1, g * dt, wk);
                                    }
                                }
                            continue;
                        }
                        for (int k = 0; k < rows; ++k) {
                            auto piece = [&](int32_t iz, double share) { add(iz, share, w[k]); };
                            const double za = std::fma((double)k, za1, za0);
                            const double zb = std::fma((double)k, zb1, zb0);
                            const double fa = std::floor(std::fmin(za, zb)), fb = std::floor(std::fmax(za, zb));
                            if (fa == fb && fa >= 0.0 && fa < (double)D) piece((int32_t)fa, dt);
                            else row_pieces_split(za, zb, dt, 0, D, false, piece);
                        }
                    }
                }
            }
          }
        }
    }
    return 0;
}

// Checks that the tilted gather's bands (tilt_column_range, tilt_row_range) hold every pixel
// whose cone ray crosses an xy cell with positive length (fp64 slab clip, t in [0, 1]), over
// the cells (ix, iy) with ix, iy = stride / 2 + i * stride. Returns the crossings found;
// *misses counts crossings outside the bands, *candidates the pixels inside them.
int64_t mbph_tilt_band(const double* frames, const double* lo, const double* pitch, const int32_t* n,
                       int views, int rows, int cols, double du, double dv, int stride,
                       long long* misses, long long* candidates) {
    std::vector<Frame> F;
    frames_from(frames, views, F);
    const Box B = box_from(lo, pitch, n);
    *misses = 0;
    *candidates = 0;
    int64_t hits = 0;
    std::vector<int32_t> k0(cols), k1(cols);
    for (int ix = stride / 2; ix < n[0]; ix += stride) {
        for (int iy = stride / 2; iy < n[1]; iy += stride) {
            const double x0 = B.lo[0] + ix * B.pitch[0], x1 = x0 + B.pitch[0];
            const double y0 = B.lo[1] + iy * B.pitch[1], y1 = y0 + B.pitch[1];
            const double clo[2] = {x0, y0}, chi[2] = {x1, y1};
            for (int v = 0; v < views; ++v) {
                TiltCorners T;
                tilt_corners(F[v], x0, x1, y0, y1, T);
                int32_t j0 = 0, j1 = -1;
                if (!tilt_column_range(T, rows, cols, du, dv, j0, j1)) j1 = -1;
                for (int j = 0; j < cols; ++j) {
                    k0[j] = 0;
                    k1[j] = -1;
                    if (j >= j0 && j <= j1 && tilt_row_range(T, j, rows, cols, du, dv, k0[j], k1[j]))
                        *candidates += k1[j] - k0[j] + 1;
                }
                for (int j = 0; j < cols; ++j) {
                    for (int k = 0; k < rows; ++k) {
                        double p[3];
                        pixel_point(F[v], centred(j, cols, du), centred(k, rows, dv), p);
                        const double d[2] = {p[0] - F[v].s[0], p[1] - F[v].s[1]};
                        double t0 = 0.0, t1 = 1.0;
                        if (!clip_slab(F[v].s, d, clo, chi, 2, t0, t1)) continue;
                        ++hits;
                        if (k < k0[j] || k > k1[j]) ++*misses;
                    }
                }
            }
        }
    }
    return hits;
}

namespace {

// One instruction of a kFastRuns itemnamespace {

// One instruction of a kFastRuns item as the kernel performs it, on sets of lanes in place of
// values: lane l starts with its own lower-cell share {l} and upper-cell share {l}; `steps`
// one-lane shifts sum each run's lower-cell shares into its first lane and its upper-cell
// shares into its last lane; the first lane takes the upper-cell sum of the run before it when
// that run's upper cell is its lower cell. key: the lanes' clamped pair indices, monotone
// along the wave (rising with the lane when up); cells 1 .. D are the column's own. Returns
// whether a share bound for one of those cells is lost, taken twice or sent to another cell,
// or two lanes write one such cell in one store.
bool runs_fail(const int32_t* key, bool up, int32_t D, int32_t steps) {
    auto at = [&](int l, int d) {                       // lane d steps forward of l, or -1
        const int s = up ? l + d : l - d;
        return s >= 0 && s < 64 ? s : -1;
    };
    auto real = [&](int32_t cell) { return cell >= 1 && cell <= D; };
    bool first[64], last[64], adj[64];
    uint64_t T[64], U[64], T2[64], U2[64];
    for (int l = 0; l < 64; ++l) {
        const int f = at(l, 1), b = at(l, -1);
        first[l] = b < 0 || key[b] != key[l];
        last[l] = f < 0 || key[f] != key[l];
        adj[l] = f >= 0 && key[f] == key[l] + 1;
        T[l] = U[l] = 1ull << l;
    }
    for (int32_t k = 0; k < steps; ++k) {
        for (int l = 0; l < 64; ++l) {
            const int f = at(l, 1), b = at(l, -1);
            T2[l] = (1ull << l) | (f >= 0 && !first[f] ? T[f] : 0);
            U2[l] = (1ull << l) | (b >= 0 && !last[b] ? U[b] : 0);
        }
        std::copy(T2, T2 + 64, T);
        std::copy(U2, U2 + 64, U);
    }
    bool bad = false;
    int ca[64] = {}, cb[64] = {};
    std::vector<int32_t> w1, w2;
    for (int l = 0; l < 64; ++l) {
        if (first[l]) {
            const int b = at(l, -1);
            const uint64_t h = b >= 0 && adj[b] ? U[b] : 0;
            if (real(key[l])) w1.push_back(key[l]);
            for (int j = 0; j < 64; ++j) {
                if (T[l] >> j & 1) { bad |= key[j] != key[l]; ++ca[j]; }
                if (h >> j & 1) { bad |= key[j] + 1 != key[l]; ++cb[j]; }
            }
        }
        if (last[l] && !adj[l]) {
            if (real(key[l] + 1)) w2.push_back(key[l] + 1);
            for (int j = 0; j < 64; ++j)
                if (U[l] >> j & 1) { bad |= key[j] != key[l]; ++cb[j]; }
        }
    }
    for (int j = 0; j < 64; ++j) {
        if (real(key[j]) && ca[j] != 1) bad = true;
        if (real(key[j] + 1) && cb[j] != 1) bad = true;
    }
    for (auto* w : {&w1, &w2}) {
        std::sort(w->begin(), w->end());
        if (std::adjacent_find(w->begin(), w->end()) != w->end()) bad = true;
    }
    return bad;
}

// The tilted gather's combine of one unit (gather_runs_add_any): keys are column indices,
// monotone along the wave; the run length is found as the kernel finds it (shift steps while
// some lane strictly between the parked pairs, index -2 and D + 1, has its key t lanes
// ahead), then the combine is checked as in runs_fail.
bool runs_fail_any(const int32_t* key, bool up, int32_t D, int32_t short_by) {
    auto ahead = [&](int l, int t) {
        const int s = up ? l + t : l - t;
        return s >= 0 && s < 64 ? key[s] : INT32_MIN;
    };
    int32_t steps = 0;
    for (int t = 1; t < 64; ++t) {
        bool any = false;
        for (int l = 0; l < 64; ++l)
            any |= key[l] > -2 && key[l] < D + 1 && ahead(l, t) == key[l];
        if (!any) break;
        ++steps;
    }
    return runs_fail(key, up, D, steps > short_by ? steps - short_by : 0);
}

}  // namespace

// Replays the gather for cone geometries off the column walk (tilt_gather_kernel) on the CPU,
// item by item, with one column per xy cell (no z chunks): the bands, each row's fp64 clip
// (with divisions where the kernel refines a reciprocal), the two-cell shares in fp64 (pieces
// of rows spanning more cells from row_pieces_split), the row values of the pre-pass (value
// times ray length), and the pair keys of every unit as the kernel forms them (parked pairs
// for rows outside the crossing rows). Adds every share times its row's value into vol (fp64,
// element (x, y, z) at (z * H + y) * W + x). Units whose keys are monotone along the wave are
// replayed through the run combine on lane sets: *conflicts counts those that would lose,
// repeat or misdirect a share or write a cell twice; *atomic counts units that take the LDS
// atomics instead. Returns the units replayed. mode 1 plants a mistake: the run combine takes
// one shift step fewer than the kernel.
int64_t mbph_tilt_gather(const double* frames, const double* lo, const double* pitch, const int32_t* n,
                         int views, int rows, int cols, double du, double dv, const float* sino,
                         int mode, double* vol, long long* conflicts, long long* atomic) {
    std::vector<Frame> F;
    frames_from(frames, views, F);
    const Box B = box_from(lo, pitch, n);
    const int32_t D = n[2];
    *conflicts = 0;
    *atomic = 0;
    int64_t units = 0;
    for (int ix = 0; ix < n[0]; ++ix) {
        for (int iy = 0; iy < n[1]; ++iy) {
            const double x0 = B.lo[0] + ix * B.pitch[0], x1 = x0 + B.pitch[0];
            const double y0 = B.lo[1] + iy * B.pitch[1], y1 = y0 + B.pitch[1];
            auto add = [&](int32_t iz, double value) {
                if (iz >= 0 && iz < D) vol[((int64_t)iz * n[1] + iy) * n[0] + ix] += value;
            };
            for (int v = 0; v < views; ++v) {
                TiltCorners T;
                tilt_corners(F[v], x0, x1, y0, y1, T);
                int32_t j0, j1;
                if (!tilt_column_range(T, rows, cols, du, dv, j0, j1)) continue;
                for (int32_t j = j0; j <= j1; ++j) {
                    int32_t ka, kb;
                    if (!tilt_row_range(T, j, rows, cols, du, dv, ka, kb)) continue;
                    for (int32_t k0 = ka; k0 <= kb; k0 += 64) {
                        const int32_t nrows = std::min(64, kb - k0 + 1);
                        ++units;
                        int32_t key[64];
                        bool active[64];
                        const double u = centred(j, cols, du);
                        for (int l = 0; l < 64; ++l) {
                            const int32_t k = k0 + l;
                            double p[3], d[3];
                            pixel_point(F[v], u, centred(k, rows, dv), p);
                            for (int a = 0; a < 3; ++a) d[a] = p[a] - F[v].s[a];
                            double t0, t1;
                            tilt_clip(F[v].s, d, x0, x1, y0, y1, t0, t1);
                            active[l] = l < nrows && t1 > t0;
                            const double za = (F[v].s[2] + t0 * d[2] - B.lo[2]) / B.pitch[2];
                            const double zb = (F[v].s[2] + t1 * d[2] - B.lo[2]) / B.pitch[2];
                            const double zmin = std::fmin(za, zb), zmax = std::fmax(za, zb);
                            const double fa = std::floor(zmin);
                            key[l] = (int32_t)std::fmax(std::fmin(fa + 1.0, (double)(D + 1)), -2.0);
                            if (!active[l]) continue;
                            const double len = std::sqrt(d[0] * d[0] + d[1] * d[1] + d[2] * d[2]);
                            const double w = (double)sino[((int64_t)v * rows + k) * cols + j] * len;
                            const double dt = t1 - t0;
                            if (zmax < fa + 2.0) {
                                const double ext = zmax - zmin;
                                const double f = ext > 0.0 ? std::fmin((fa + 1.0 - zmin) / ext, 1.0) : 1.0;
                                const double g = ext > 0.0 ? std::fmax(zmax - (fa + 1.0), 0.0) / ext : 0.0;
                                add((int32_t)fa, f * dt * w);
                                add((int32_t)fa + 1, g * dt * w);
                            } else {
                                auto piece = [&](int32_t iz, double share) { add(iz, share * w); };
                                row_pieces_split(za, zb, dt, 0, D, false, piece);
                            }
                        }
                        // the kernel's keys: rows before and after the crossing rows take the
                        // parked pair at their end of the column
                        const bool up = F[v].v[2] >= 0.0;
                        int lo_lane = 64, hi_lane = -1;
                        for (int l = 0; l < 64; ++l)
                            if (active[l]) { lo_lane = std::min(lo_lane, l); hi_lane = l; }
                        for (int l = 0; l < 64; ++l) {
                            if (hi_lane < 0) key[l] = -2;
                            else if (l < lo_lane) key[l] = up ? -2 : D + 1;
                            else if (l > hi_lane) key[l] = up ? D + 1 : -2;
                        }
                        bool monotone = true;
                        for (int l = 0; l + 1 < 64; ++l) {
                            const int32_t a = key[up ? l : l + 1], b = key[up ? l + 1 : l];
                            if (b < a) monotone = false;
                        }
                        if (!monotone) ++*atomic;
                        else if (runs_fail_any(key, up, D, mode == 1 ? 1 : 0)) ++*conflicts;
                    }
                }
            }
        }
    }
    return units;
}

// Emulates the gather's instruction grouping and checks its race-freedom claims. Fast items:
// for every instruction (row c of each lane), the cell pairs {fa, fa + 1} that in-range lanes
// read and write must be disjoint (kFastPairs), or the combine of runs of lanes sharing a
// pair must deliver every share to its cell once, with distinct cells per store (kFastRuns,
// runs_fail). General items that the kernel treats as exclusive: for every instruction and
// every step (the single-piece add, then step i of the aligned piece walk), the z cells the
// active lanes add into must be distinct. Returns the number of items checked; *conflicts
// counts instructions or steps that fail, *fast the fast items. mode 0 replays the kernel;
// planted mistakes show the check can fail: mode 1 starts the walk of rows that span several
// cells at the first in-range cell (rows entering from below the box then meet in its bottom
// cell), mode 2 deals adjacent rows to the lanes of one instruction, mode 3 writes the cell
// pairs of kFastRuns items at once without combining, mode 4 shifts their runs one step
// fewer than the kernel.
int64_t mbph_gather_conflicts(const double* frames, int beam, const double* lo, const double* pitch,
                              const int32_t* n, int views, int rows, int cols, double du, double dv,
                              int mode, long long* conflicts, long long* fast) {
    const bool aligned = mode != 1;
    std::vector<Frame> F;
    frames_from(frames, views, F);
    const Box B = box_from(lo, pitch, n);
    *conflicts = 0;
    *fast = 0;
    const bool line = beam == BEAM_PARALLEL;
    const int32_t S = gather_stride(rows), rows_pad = gather_rows_padded(rows), D = n[2];
    int64_t checked = 0;
    std::vector<int32_t> seen;
    for (int ix = 0; ix < n[0]; ++ix) {
        for (int iy = 0; iy < n[1]; ++iy) {
            const double x0 = B.lo[0] + ix * B.pitch[0], x1 = x0 + B.pitch[0];
            const double y0 = B.lo[1] + iy * B.pitch[1], y1 = y0 + B.pitch[1];
            for (int v = 0; v < views; ++v) {
                int32_t j0, j1;
                if (!cell_column_range(F[v], beam, cols, du, x0, x1, y0, y1, j0, j1)) continue;
                for (int32_t j = j0; j <= j1; ++j) {
                    ColLine L;
                    column_line(F[v], B, beam, j, cols, rows, du, dv, L);
                    GatherItem it;
                    if (!gather_item(L, line, x0, x1, y0, y1, S, rows, rows_pad, v * cols + j, it)) continue;
                    const bool is_fast = it.form > 0;
                    if (it.form == kGeneralAtomic) continue;      // LDS atomics: nothing to check
                    ++checked;
                    if (is_fast) ++*fast;
                    for (int32_t g0 = 0; g0 < rows_pad; g0 += 64 * S) {
                        for (int32_t c = 0; c < S; ++c) {
                            if (is_fast) {
                                // the lanes' pair indices; mode 2: adjacent rows in one instruction
                                int32_t key[64];
                                for (int lane = 0; lane < 64; ++lane) {
                                    const int32_t k0 = mode == 2 ? g0 + 64 * c + lane - c : g0 + S * lane;
                                    const int32_t c0 = fast_origin_row(S);
                                    uint32_t la, lb, num, ext;
                                    int32_t base, fb;
                                    fast_origin(it, k0 + c0, -1, la, lb, base);
                                    fast_row(la + (uint32_t)((c - c0) * it.a1fx), lb + (uint32_t)((c - c0) * it.b1fx),
                                             fb, num, ext);
                                    key[lane] = base + fb;
                                }
                                if (it.form == kFastRuns && mode != 3) {
                                    // the kernel's clamp of the pair index to [-2, D + 1]
                                    int32_t kc[64];
                                    for (int lane = 0; lane < 64; ++lane)
                                        kc[lane] = std::min(std::max(key[lane], -2), D + 1);
                                    const int32_t steps = it.run - (mode == 4 ? 2 : 1);
                                    if (it.run < 1 || runs_fail(kc, it.a1fx > 0, D, steps)) ++*conflicts;
                                    continue;
                                }
                                // every lane's pair at once
                                seen.clear();
                                for (int lane = 0; lane < 64; ++lane) {
                                    if ((uint32_t)key[lane] > (uint32_t)D) continue;   // discard pair
                                    seen.push_back(key[lane]);
                                    seen.push_back(key[lane] + 1);
                                }
                                std::sort(seen.begin(), seen.end());
                                if (std::adjacent_find(seen.begin(), seen.end()) != seen.end()) ++*conflicts;
                                continue;
                            }
                            // steps: the two-piece adds (cell fa, then cell fb), then the
                            // steps of the aligned walk of rows spanning a cell or more
                            std::vector<std::vector<int32_t>> steps(2);
                            for (int lane = 0; lane < 64; ++lane) {
                                // padded rows too; mode 2 puts adjacent rows in one instruction
                                const int32_t k = mode == 2 ? g0 + 64 * c + lane : g0 + c + S * lane;
                                const double za = std::fma((double)k, it.za1, it.za0);
                                const double zb = std::fma((double)k, it.zb1, it.zb0);
                                const double zmin = std::fmin(za, zb), zmax = std::fmax(za, zb);
                                if (zmax - zmin < 1.0) {
                                    const double fa = std::floor(zmin), fb = std::floor(zmax);
                                    if (fa >= 0.0 && fa < (double)D) steps[0].push_back((int32_t)fa);
                                    if (fb != fa && fb >= 0.0 && fb < (double)D) steps[1].push_back((int32_t)fb);
                                    continue;
                                }
                                // step index of each piece: its position in this row's walk
                                const int32_t start = aligned ? (int32_t)std::floor(zmin)
                                                              : (int32_t)std::floor(std::fmax(zmin, 0.0));
                                auto piece = [&](int32_t iz, double) {
                                    const int step = iz - start + 2;
                                    if ((int)steps.size() <= step) steps.resize(step + 1);
                                    steps[step].push_back(iz);
                                };
                                row_pieces_split(za, zb, (double)it.dt, 0, D, aligned, piece);
                            }
                            for (auto& st : steps) {
                                seen = st;
                                std::sort(seen.begin(), seen.end());
                                if (std::adjacent_find(seen.begin(), seen.end()) != seen.end()) ++*conflicts;
                            }
                        }
                    }
                }
            }
        }
    }
    return checked;
}

// Checks kFastInside, under which the gather writes a fast item's cell pairs without clamping
// their indices: for every fast item and every z chunk of `zchunk` cells (the last one ragged)
// for which gather_item sets it, every row of every lane (padded rows too) must have its pair
// index, replayed in the kernel's fixed point, in [-2, n + 1]. Returns the fast items met;
// *inside counts the (item, chunk) pairs accepted, *violations the rows outside. mode 1
// plants a mistake: the range test looks at the first row only.
int64_t mbph_fast_inside(const double* frames, int beam, const double* lo, const double* pitch,
                         const int32_t* n, int views, int rows, int cols, double du, double dv,
                         int zchunk, int mode, long long* inside, long long* violations) {
    std::vector<Frame> F;
    frames_from(frames, views, F);
    const Box B = box_from(lo, pitch, n);
    *inside = 0;
    *violations = 0;
    const bool line = beam == BEAM_PARALLEL;
    const int32_t S = gather_stride(rows), rows_pad = gather_rows_padded(rows), D = n[2];
    int64_t fast = 0;
    for (int ix = 0; ix < n[0]; ++ix) {
        for (int iy = 0; iy < n[1]; ++iy) {
            const double x0 = B.lo[0] + ix * B.pitch[0], x1 = x0 + B.pitch[0];
            const double y0 = B.lo[1] + iy * B.pitch[1], y1 = y0 + B.pitch[1];
            for (int v = 0; v < views; ++v) {
                int32_t j0, j1;
                if (!cell_column_range(F[v], beam, cols, du, x0, x1, y0, y1, j0, j1)) continue;
                for (int32_t j = j0; j <= j1; ++j) {
                    ColLine L;
                    column_line(F[v], B, beam, j, cols, rows, du, dv, L);
                    GatherItem it;
                    if (!gather_item(L, line, x0, x1, y0, y1, S, rows, rows_pad, v * cols + j, it)) continue;
                    if (it.form <= 0) continue;
                    ++fast;
                    for (int32_t z0 = 0; z0 < D; z0 += zchunk) {
                        const int32_t nz = std::min(zchunk, D - z0);
                        const float in_lo = fast_inside_lo(z0, nz), in_hi = fast_inside_hi(z0, nz);
                        GatherItem ci;
                        gather_item(L, line, x0, x1, y0, y1, S, rows, rows_pad, v * cols + j, ci, in_lo, in_hi);
                        bool accepted = (ci.form & kFastInside) != 0;
                        if (mode == 1) {
                            double t0, t1;
                            cell_clip(L, line, x0, x1, y0, y1, t0, t1);
                            const double za0 = L.c0 + t0 * L.c1, zb0 = L.c0 + t1 * L.c1;
                            accepted = rows_inside(za0, zb0, za0, zb0, in_lo, in_hi);
                        }
                        if (!accepted) continue;
                        ++*inside;
                        const int32_t c0 = fast_origin_row(S);
                        for (int32_t k0 = 0; k0 < rows_pad; k0 += S) {
                            uint32_t la, lb, num, ext;
                            int32_t base, fb;
                            fast_origin(it, k0 + c0, z0 - 1, la, lb, base);
                            for (int32_t c = 0; c < S; ++c) {
                                fast_row(la + (uint32_t)((c - c0) * it.a1fx), lb + (uint32_t)((c - c0) * it.b1fx),
                                         fb, num, ext);
                                const int32_t pi = base + fb;
                                if (pi < -2 || pi > nz + 1) ++*violations;
                            }
                        }
                    }
                }
            }
        }
    }
    return fast;
}

// Bounds-only sweep of selected rays (flat ids) with either walk; returns visits.
int64_t mbph_check_rays(int path, const double* frames, int beam, const double* lo,
                        const double* pitch, const int32_t* n, int views, int rows, int cols,
                        double du, double dv, const int64_t* ray_ids, int64_t nrays,
                        long long* violations) {
    std::vector<Frame> F;
    frames_from(frames, views, F);
    const Box B = box_from(lo, pitch, n);
    *violations = 0;
    Checked chk{&B, violations};
    int64_t visits = 0;
    for (int64_t q = 0; q < nrays; ++q) {
        const int64_t id = ray_ids[q];
        const int i = (int)(id / ((int64_t)rows * cols));
        const int k = (int)((id / cols) % rows);
        const int j = (int)(id % cols);
        if (i < 0 || i >= views) { ++*violations; continue; }
        auto visit = [&](int32_t cx, int32_t cy, int32_t cz, float len) {
            ++visits;
            chk.ok(cx, cy, cz, len);
        };
        if (path == 2) {
            ColumnWalk c;
            column_setup(F[i], B, beam, centred(j, cols, du), c);
            RowWalk r;
            row_setup(c, B, centred(k, rows, dv), F[i].v[2], r);
            walk_column_row(c, r, visit);
        } else {
            RayWalk r;
            ray_setup(F[i], B, beam, centred(j, cols, du), centred(k, rows, dv), r);
            walk_ray(r, visit);
        }
    }
    return visits;
}

}  // extern "C"
