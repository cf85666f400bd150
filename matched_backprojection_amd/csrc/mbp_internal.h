// mbp_internal.h -- launch interface between the host plan (plan.cpp) and the kernels
// (kernels.hip). Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "traverse.h"

namespace mbp {

// Arguments of one generic-walk launch: rays [view0, view0 + nviews) x rows x cols, for `nb`
// batch members (1..4) whose volumes and sinograms start at vol[m] and sino[m].
struct GenericLaunch {
    const Frame* frames;      // device, all views of the plan
    int32_t view0, nviews;
    int32_t rows, cols;
    double du, dv;
    int32_t beam;
    int32_t nb;
    Box box;
    int32_t sx, sy, sz;       // volume element strides along world x, y, z
    int32_t rows_fast;        // consecutive threads take consecutive rows (z-fastest volumes)
};

// Arguments of one column-walk launch: waves over (view, column, block of 64 rows). The
// volume is z-fastest with `NB` members interleaved innermost: element (x, y, z, m) at
// ((x*H + y)*D + z)*NB + m.
struct ColumnLaunch {
    const Frame* frames;
    int32_t view0, nviews;
    int32_t rows, cols;
    int32_t row_blocks;       // ceil(rows / 64)
    int32_t beam;
    double du, dv;
    Box box;
    int32_t H, D;
    uint32_t tasks;           // nviews * cols * row_blocks
    uint32_t pad_;
};

// Forward: sino[m][ray] for rays of the launch; adjoint: atomically adds into vol. Forward with
// orbit 2 or 4 (nb = 1): the launch's views lie among the first q = V / orbit, and each ray's
// walk also gives the rays of the views q m apart (orbit_cell), stored slot_stride * m
// elements after it; dir: the quarter turn's sense.
hipError_t launch_generic_forward(const GenericLaunch& a, const float* const* vol,
                                  float* const* sino, hipStream_t s, int orbit = 1, int dir = 0,
                                  int64_t slot_stride = 0);
hipError_t launch_generic_adjoint(const GenericLaunch& a, const float* const* sino,
                                  float* const* vol, hipStream_t s);
// orbit 2 or 4 (nb = 1): the launch's views lie among the first q = V / orbit, and each ray's
// walk also gives the rays of the views q m apart (orbit_cell), stored slot_stride * m
// elements after it (slot_stride = q rows cols); dir: the quarter turn's sense.
hipError_t launch_column_forward(const ColumnLaunch& a, int nb, const float* vol,
                                 float* const* sino, hipStream_t s, int orbit = 1, int dir = 0,
                                 int64_t slot_stride = 0);
hipError_t launch_column_adjoint(const ColumnLaunch& a, int nb, const float* const* sino,
                                 float* vol, hipStream_t s);

// Matched adjoint of the column geometry without global atomics: a pre-pass copies the
// sinogram of the launch's views [view0, view0 + nviews) to [view - view0][col][row] order
// (nb members interleaved innermost) scaled by each ray's length per unit of its parameter,
// rows zero-padded to gather_rows_padded(rows), into ysc (gather_sino_floats(nviews, ...)
// floats); the gather then writes every voxel of the z-fastest interleaved volume once
// (optionally adding into it), reading the line constants of view view0 + i at lines[i * cols
// + column].
//
// Turn symmetry (orbit = 2 or 4, nb = 1; see orbit_cell): the pre-pass runs over the first
// q = V / orbit views with `orbit` members, member m being sino + m q rows cols (the views
// q m apart, mview = q); the gather then takes a launch over all V views (nviews = V, view0 = 0)
// and writes every voxel of the one-member volume once. dir: the turn's sense for orbit 4.
hipError_t launch_sino_prepass(const ColumnLaunch& a, int nb, const float* const* sino, float* ysc,
                               hipStream_t s, int32_t mview = 0);
hipError_t launch_column_gather(const ColumnLaunch& a, int nb, const ColLine* lines, const float* ysc,
                                float* vol, int accumulate, hipStream_t s, int orbit = 1, int dir = 0);
// The gather for cone geometries whose detector rows do not run along z: the same pre-pass
// sinogram (ysc) and output as launch_column_gather, each ray clipped against each cell on
// its own; orbit and dir as for launch_column_gather.
hipError_t launch_tilt_gather(const ColumnLaunch& a, int nb, const float* ysc, float* vol, int accumulate,
                              hipStream_t s, int orbit = 1, int dir = 0);
// Per-(view, column) line constants of the gather, for views [a.view0, a.view0 + views)
// (lines holds views * cols entries).
hipError_t launch_column_lines(const ColumnLaunch& a, int32_t views, ColLine* lines, hipStream_t s);

// Positive-length segments walked by the launch's rays; adds into *count (device, zeroed by
// the caller).
hipError_t launch_count(const GenericLaunch& a, unsigned long long* count, hipStream_t s);
hipError_t launch_column_count(const ColumnLaunch& a, unsigned long long* count, hipStream_t s);

// Layout conversion for the column walk. to_native: nb members of a DHW volume (member
// stride vox) -> interleaved z-fastest ws. from_native: the reverse, optionally adding into
// the destination.
hipError_t launch_to_native(const float* in, int64_t member_stride, int nb, int32_t D,
                            int32_t H, int32_t W, int whd_in, float* ws, hipStream_t s);
hipError_t launch_from_native(const float* ws, int nb, int32_t D, int32_t H, int32_t W,
                              int whd_out, float* out, int64_t member_stride, int accumulate,
                              hipStream_t s);
// Plain DHW <-> WHD conversion of one member.
hipError_t launch_convert(const float* in, int32_t D, int32_t H, int32_t W, int to_whd,
                          float* out, hipStream_t s);
hipError_t launch_fill_zero(float* p, int64_t n, hipStream_t s);
hipError_t launch_stream_copy(const float* in, float* out, int64_t n, hipStream_t s);

// With MBP_TRACE set in the environment, print one launch's kernel, grid, block, dynamic LDS
// bytes and work range (printf-style `fmt`) to stderr.
void trace_launch(const char* kernel, dim3 grid, dim3 block, size_t lds, const char* fmt, ...);

// Record the calling thread's error message (mbp_last_error) and return `code`.
int set_error(int code, const char* fmt, ...);

}  // namespace mbp
