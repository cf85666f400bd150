/*
 * mbp.h -- C ABI of the MI355X ray-driven X-ray transform pair.
 *
 * The pair (diffct pages, "diffct 2.1.0 -> 2.2.1", README "Why diffct", bullet "Matched
 * operators"): project() and backproject() form an exact adjoint pair for the cell-constant
 * Siddon model.
 *
 *   project      P[b, view, row, col] = sum_v len(ray, v) * volume[b, v]
 *   backproject  volume[b, v]        (+)= sum_rays len(ray, v) * sinogram[b, ray]
 *
 * len(ray, v) is the physical length of the ray inside voxel v. Each view has its own source
 * (or ray direction), detector centre and detector axes (page "diffct 2.2.1 -> 2.4.0",
 * README "Why diffct", bullet "Arbitrary trajectories"; the per-view tuples are on page
 * "diffct 2.1.0 -> 2.2.1", diffct/analytical.py). Geometry readings taken where the pages
 * are silent: the volume box is centred on `center`; world x <-> W, y <-> H, z <-> D; pixel
 * (row k, col j) sits at det + ((j - (cols-1)/2) du) eu + ((k - (rows-1)/2) dv) ev; fan and
 * cone rays are the segments source -> pixel; parallel rays are infinite lines through the
 * pixel along the view's ray direction; cells are half-open.
 *
 * Memory and ownership. Volume and sinogram pointers are HIP device pointers on the current
 * device, owned by the caller; the library never frees or reallocates them. Trajectory
 * arrays are host pointers, copied at plan creation. Calls that take a `stream` enqueue work
 * on that HIP stream (NULL = the default stream) and return without synchronising, except
 * mbp_segment_count, which waits for its own result. A plan may be used from one host
 * thread and one stream at a time; plans are independent of each other.
 *
 * Layouts. Volumes of one batch member are dense and either MBP_LAYOUT_DHW (C order of the
 * tensor shape (D, H, W), W fastest) or MBP_LAYOUT_WHD (the same (D, H, W) tensor with
 * z-fastest strides: element (z, y, x) at (x*H + y)*D + z; page "diffct 2.2.1 -> 2.4.0",
 * CHANGELOG 2.4.0, native_volume_layout). Sinograms are dense [views][rows][cols]. A leading
 * batch of B members is dense too: member b starts at b * D*H*W (volumes) and at
 * b * views*rows*cols (sinograms). B may be 0 (page "diffct 2.2.1 -> 2.3.0", CHANGELOG
 * 2.3.0, "Added": leading batch dimensions including empty batches).
 *
 * Errors. Every function validates all of its arguments before any device work and returns
 * MBP_OK (0) or a negative mbp_status; mbp_last_error() then holds a message for the calling
 * thread. A geometry that fails validation never produces a plan.
 */
#ifndef MBP_H
#define MBP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MBP_ABI_VERSION 4

typedef enum mbp_status {
    MBP_OK = 0,
    MBP_EINVAL = -1,       /* bad enum, shape, pointer, batch, or 2-D with D != 1 / rows != 1 */
    MBP_ENONFINITE = -2,   /* NaN or Inf in spacing, centre, pitch or trajectory ("must be finite") */
    MBP_ECOINCIDENT = -3,  /* source on a pixel, zero ray direction or detector axis, parallel
                              detector axes ("must differ") */
    MBP_ERANGE = -4,       /* voxel pitch outside [1e-6, 1e6] or max/min pitch > 1e4; source
                              nearer than 1e-6 min pitch to the detector ("near"); a coordinate
                              farther than 1e15 min pitch from the volume centre ("far") */
    MBP_ETOOLARGE = -5,    /* one batch member's volume or sinogram has >= 2^31 elements */
    MBP_EHIP = -6,         /* a HIP runtime call failed; mbp_last_error() has its message */
    MBP_ENOMEM = -7        /* host or device allocation failed, or a workspace is too small */
} mbp_status;

typedef enum mbp_beam {
    MBP_PARALLEL = 0,      /* 2-D parallel beam: volume (H, W), D = 1, rows = 1             */
    MBP_FAN = 1,           /* 2-D fan beam, flat (line) detector: D = 1, rows = 1           */
    MBP_CONE = 2,          /* 3-D cone beam, flat detector                                   */
    MBP_PARALLEL3D = 3     /* 3-D parallel beam, flat detector: infinite parallel rays, one
                              direction per view (page "diffct 2.2.1 -> 2.4.0", CHANGELOG
                              2.4.0, "Added")                                                */
} mbp_beam;

typedef enum mbp_layout {
    MBP_LAYOUT_DHW = 0,    /* W fastest (C order of (D, H, W))                               */
    MBP_LAYOUT_WHD = 1     /* D fastest; 3-D beams only                                      */
} mbp_layout;

typedef enum mbp_path {
    MBP_PATH_AUTO = 0,     /* pick the column walk when the geometry allows it               */
    MBP_PATH_GENERIC = 1,  /* one lane per ray, full 3-D walk, any flat-detector geometry    */
    MBP_PATH_COLUMN = 2    /* 3-D beam whose detector row axis is parallel to z: the rows of
                              a detector column share their xy walk                          */
} mbp_path;

typedef enum mbp_adjoint {
    MBP_ADJOINT_AUTO = 0,     /* the gather                                                   */
    MBP_ADJOINT_GATHER = 1,   /* each wave owns one xy cell's z column in LDS and sums, over
                                 views, crossing columns and rows, the exact chord of every
                                 ray through each of its voxels; no global atomics. Column
                                 walk: rows share their column's xy line. Cone geometries off
                                 the column walk (detector rows not along z), with the walk
                                 chosen automatically: each row's ray is clipped on its own  */
    MBP_ADJOINT_SCATTER = 2   /* each ray scatters its value along its segments with global
                                 float atomics: column walk with 64 adjacent rows per wave and
                                 z-inner stepping, or the generic walk (also always used when
                                 MBP_PATH_GENERIC is forced)                                   */
} mbp_adjoint;

typedef struct mbp_geometry {
    int32_t beam;          /* mbp_beam                                                       */
    int32_t layout;        /* mbp_layout of the caller's volumes                            */
    int64_t D, H, W;       /* volume shape in tensor order; 2-D beams: D = 1                */
    double spacing[3];     /* (dz, dy, dx): voxel pitch in tensor axis order, physical units
                              (page "diffct 2.4.3 -> 2.4.4", README "Per-axis voxel
                              spacing"); 2-D beams ignore dz                                 */
    double center[3];      /* world (x, y, z) of the volume centre; 2-D beams ignore z      */
    int64_t views, rows, cols;   /* sinogram [views][rows][cols]; 2-D beams: rows = 1       */
    double du, dv;         /* detector pitch along eu (columns) and ev (rows); > 0           */
} mbp_geometry;

typedef struct mbp_plan mbp_plan;

typedef struct mbp_plan_info {
    int32_t path;              /* MBP_PATH_GENERIC or MBP_PATH_COLUMN: the walk that runs
                                  (the forward's; the adjoint kernel follows mbp_adjoint)   */
    int32_t column_capable;    /* 1 if the geometry allows the column walk                  */
    int64_t views_per_launch;  /* view batch of one kernel launch                           */
    int64_t launches;          /* kernel launches per member group and operation            */
    int64_t rays;              /* views * rows * cols                                       */
    int64_t voxels;            /* D * H * W                                                 */
    int64_t members_per_pass;  /* batch members one walk serves (volume interleave)         */
    /* What the last mbp_backproject of this plan ran (all 0 before the first call with B > 0): */
    int32_t last_adjoint;      /* MBP_ADJOINT_GATHER or MBP_ADJOINT_SCATTER (global atomics)   */
    int32_t last_adjoint_walk; /* MBP_PATH_COLUMN (rows share their column's xy line) or
                                  MBP_PATH_GENERIC (each ray on its own: the per-row gather,
                                  or the generic walk's atomics)                              */
    int64_t last_adjoint_views_per_launch;  /* views per adjoint launch: below
                                  views_per_launch when the gather's workspace held fewer  */
    /* What the last mbp_project of this plan ran (0 before the first call with B > 0): */
    int32_t last_forward_walk; /* MBP_PATH_COLUMN, or MBP_PATH_GENERIC when the geometry needs
                                  it or when not even one member's z-fastest copy (needed for
                                  a (D,H,W) volume or a batch) fits the memory rule          */
    int32_t last_forward_members_per_pass;  /* fewest members one column walk served (1, 2
                                  or 4; below members_per_pass when the interleaved copy was
                                  halved to fit the memory rule); 0 on the generic walk     */
    int32_t orbit;             /* turn symmetry of the views found at plan creation (see
                                  mbp_plan_set_orbit): 4 (quarter turn), 2 (half turn) or 1   */
    int32_t last_adjoint_orbit; /* cells that shared each gather crossing in the last
                                  mbp_backproject: the orbit, or 1 (0 before the first call) */
    int32_t last_forward_orbit; /* rays that shared each column walk in the last mbp_project
                                  (the fewest over its passes): the orbit, or 1 (0 before the
                                  first call with B > 0)                                      */
} mbp_plan_info;

/* Validate the geometry and trajectory and build a plan. Trajectory arrays are host fp64,
   row-major [views][rank] with rank 3 for 3-D beams (cone, parallel3d) and 2 for 2-D beams:
   src = source position (fan/cone) or ray direction (parallel, parallel3d; any nonzero
   length); det = detector centre; eu, ev = detector axes (ev NULL for 2-D beams). The arrays
   are copied; no device call is made here (frames are staged to device memory on first use
   on each device). On success *out owns the plan. */
int mbp_plan_create(const mbp_geometry* geometry, const double* src, const double* det,
                    const double* eu, const double* ev, mbp_plan** out);

/* Free a plan and its device frames and library-owned workspace. NULL is a no-op. The
   caller must make sure no enqueued work still uses the plan. */
void mbp_plan_destroy(mbp_plan* plan);

/* Fill *info (host only, no device call). */
int mbp_plan_get_info(const mbp_plan* plan, mbp_plan_info* info);

/* Force a walk (MBP_PATH_AUTO restores the automatic choice). Forcing MBP_PATH_COLUMN on a
   geometry that cannot use it returns MBP_EINVAL. Both walks visit the same segments. */
int mbp_plan_set_path(mbp_plan* plan, int32_t path);

/* Choose the adjoint kernel (mbp_adjoint). All compute the same sums (the chord of every ray
   through every voxel times the ray's value); they differ in summation order. */
int mbp_plan_set_adjoint(mbp_plan* plan, int32_t kind);

/* Allow (1, the default) or forbid (0) the column walk and the gather adjoint to share their
   geometry over a turn symmetry of the views. Both operators are sums of chords, the length
   of a ray inside a voxel (the pair at the top of this header: page "diffct 2.1.0 -> 2.2.1",
   README "Why diffct", bullet "Matched operators"). When the views fall into P = 4 (or 2)
   groups of V / P such that view v + V / P is view v turned a quarter (half) turn about the
   vertical axis through the volume's xy centre, and the grid maps onto itself under that turn
   (W even; for a quarter turn also W == H and dx == dy), the chord of ray (v + m V / P,
   column, row) through a cell equals that of ray (v, column, row) through the cell turned
   back m steps. The forward then walks the rays of the first V / P views only, each walk
   summing the P turned cells into the P rays it stands for, and the gather forms its cell
   crossings for those views only, each serving the P cells of an orbit. Taken for single
   members (the forward: any pass of one member; the gather: batch 1 with every view in one
   launch). Frames are compared to 1e-12 of their extent, so the sums equal the unshared
   ones to fp32 rounding, and the forward and the gather still visit the same segments.
   Plan setting only: no device call. */
int mbp_plan_set_orbit(mbp_plan* plan, int32_t enable);

/* Limit the views of one kernel launch (0 = automatic: as many as index and grid limits
   allow). Results do not depend on it (page "diffct 2.1.0 -> 2.2.1", CHANGELOG 2.2.0,
   "Changed": backprojection accumulators span all contributing view batches). The gather
   adjoint's workspace holds the reordered sinogram of one launch, so a smaller batch also
   shrinks mbp_workspace_size. */
int mbp_plan_set_view_batch(mbp_plan* plan, int64_t views_per_launch);

/* Forward projection of `batch` volumes (caller's layout) into `sinogram` [batch][views]
   [rows][cols]. Every sinogram element is written; rays that miss the volume get 0. */
int mbp_project(mbp_plan* plan, const float* volume, int64_t batch, float* sinogram,
                void* stream);

/* Matched backprojection: volume = sum over rays of len * sinogram (accumulate = 0), or
   volume += that sum (accumulate = 1), in the caller's layout, for `batch` members. The
   segments are exactly those of mbp_project. The gather adjoint runs in view batches sized to
   its workspace (all views in one launch when the memory rule or the caller's workspace
   allows, else as many as fit, each launch adding into the previous ones); only when not even
   one view's share fits does the call take the generic walk's atomics, and mbp_plan_get_info
   then says so. The scatter adjoints' floating-point atomics make the summation order, and
   so the last bits, vary from run to run. */
int mbp_backproject(mbp_plan* plan, const float* sinogram, int64_t batch, float* volume,
                    int32_t accumulate, void* stream);

/* mbp_backproject for callers that cannot allocate device memory (code under HIP graph
   capture, tight serving loops, harnesses that forbid hipMalloc): the same arguments, result
   and error codes, and no hipMalloc, hipFree or other allocating call. Every device buffer of
   the call comes from a library array of 128 MiB per device (static device memory, held by
   each device the library runs on until the process ends): the plan's frames (copied in by
   each call), the gather's line table of one view batch, the reordered sinogram and, for
   batches or (D, H, W) volumes, the interleaved z-fastest volume. The gather takes as many
   views per launch as fit the array; a call that needs more than it holds even for one view
   (for example the z-fastest copy of a (D, H, W) volume above about 128 MiB) returns
   MBP_ETOOLARGE before any device work. All calls on one device share that device's array:
   calls that overlap in time on one device (other streams or host threads, any plan) race
   and give wrong results; calls in order on one stream are safe. */
int mbp_backproject_noalloc(mbp_plan* plan, const float* sinogram, int64_t batch, float* volume,
                            int32_t accumulate, void* stream);

/* Number of ray/voxel segments one projection of one member walks, counting those longer
   than 1e-6 of the smallest voxel pitch (shorter ones are rounding residue where a ray
   crosses several grid planes at one point). This is the work unit of the throughput
   metric. Runs a counting kernel on `stream`, then waits. */
int mbp_segment_count(mbp_plan* plan, int64_t* count, void* stream);

/* Device workspace the plan needs for `batch` members on the column walk, or for the gather:
   a z-fastest copy of up to four interleaved volumes (not needed for one z-fastest volume)
   plus, for the gather adjoint, a reordered copy of their sinograms over the views of one
   launch (views_per_launch; see mbp_plan_set_view_batch). 0 when none is needed. A smaller
   workspace serves the gather as long as it holds the volume part and one view's share: the
   gather then takes as many views per launch as fit. */
int mbp_workspace_size(const mbp_plan* plan, int64_t batch, size_t* bytes);

/* Hand the plan a caller-owned device workspace (NULL, 0 = let the library allocate its
   own on first use). The caller keeps ownership and must keep it alive while work that uses
   it is enqueued. A call whose least need (the volume part, plus one view's share for the
   gather) exceeds `bytes` returns MBP_ENOMEM. */
int mbp_set_workspace(mbp_plan* plan, void* device_ptr, size_t bytes);

/* Convert `batch` volumes between MBP_LAYOUT_DHW and MBP_LAYOUT_WHD (to_whd = 1: DHW ->
   WHD). `in` and `out` must not overlap. Lets a caller keep volumes in the z-fastest layout
   across repeated operator applications (page "diffct 2.2.1 -> 2.4.0", CHANGELOG 2.4.0:
   keeping the native layout saves two whole-volume copies per normal-operator
   application). */
int mbp_convert_layout(const float* in, int64_t batch, int64_t D, int64_t H, int64_t W,
                       int32_t to_whd, float* out, void* stream);

/* Normal operator of the pair: out = A^T (A volume) for `batch` members, in the plan's
   layout; `sinogram` ([batch][views][rows][cols], caller-owned) receives A volume on the way.
   `out` must not alias `volume`. A caller that keeps its volumes in MBP_LAYOUT_WHD pays no
   layout copy per application (page "diffct 2.2.1 -> 2.4.0", CHANGELOG 2.4.0,
   native_volume_layout). */
int mbp_normal(mbp_plan* plan, const float* volume, int64_t batch, float* sinogram, float* out,
               void* stream);

/* Device workspace bytes mbp_cgls needs for `batch` members and `iters` iterations: per
   member two sinograms (the residual r and q = A p) and two volumes (s = A^T r and the search
   direction p), plus fp64 scalars, the residual history and reduction partials. */
int mbp_cgls_workspace_size(const mbp_plan* plan, int64_t batch, int32_t iters, size_t* bytes);

/* CGLS (conjugate gradients on the normal equations, keeping the residual r = y - A x) for
   min_x ||A x - y||, one independent problem per batch member, started from the caller's
   `volume` (x0; zeros for a cold start), which holds the iterate after the call. `iters`
   iterations are enqueued; a member whose residual norm falls to rtol * ||y|| stays
   unchanged from then on (rtol = 0: never). Norms are accumulated in fp64 blocks and the
   step sizes formed in fp64 on the device (page "diffct 2.1.0 -> 2.2.1", CHANGELOG 2.2.0;
   solver with residual history, optional x0 and residual thresholds: page "diffct 2.2.1 ->
   2.3.0", CHANGELOG 2.3.0). `workspace` is caller-owned device memory of at least
   mbp_cgls_workspace_size bytes, 256-byte aligned, not overlapping `sinogram` or `volume`.
   residual_norms (host, may be NULL): [batch][iters + 1] values of ||r_k|| (the recursively
   updated residual), k = 0..iters; when it is non-NULL the call waits for `stream` to finish,
   otherwise nothing synchronises the host. */
int mbp_cgls(mbp_plan* plan, const float* sinogram, int64_t batch, float* volume, int32_t iters,
             double rtol, void* workspace, size_t workspace_bytes, double* residual_norms,
             void* stream);

/* Copy n floats from `in` to `out` (device pointers, 16-byte aligned, not overlapping) with a
   streaming kernel: 16-byte loads and stores over a fixed grid. It is the
   bandwidth reference of the measurements (the HBM rate a plain copy reaches on this GPU) and
   the kernel of known traffic that hardware byte counters are calibrated with. */
int mbp_stream_copy(const float* in, float* out, int64_t n, void* stream);

const char* mbp_status_string(int status);
const char* mbp_last_error(void);
int mbp_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MBP_H */
