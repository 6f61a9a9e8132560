/*
 * cgtp.h -- C ABI of libcgtp.so: the Clebsch-Gordan tensor-product (CGTP)
 * convolution, forward (fp32, and fp64 for l <= 4) and gradients (fp32, l <= 4), for
 * AMD Instinct MI355X (gfx950).
 *
 * What is computed (the pages print no formula; this is the textbook definition that
 * LunaTP's abstract says its kernels preserve):
 *   for every receiver i, every active edge e = (j -> i) of row i, every path
 *   p = (input irrep l1, edge-SH irrep l2 -> l3) and every channel u of the input irrep
 *     out[i, c_p(u), m3] += w[e, c_p(u)] * sum_{m1,m2} C_p[m1,m2,m3] x[j,u,m1] Y_{l2,m2}(r_e)
 *   with r_e = pos[j] - pos[i] + shift_e . cell.
 * Sources: LunaTP ("Enabling Efficient and Scalable Tensor Product for Equivariant
 * MLIPs"), Abstract and Figure 3(a) (node-centric accumulation, one store per node),
 * Table 1 (irreps cases; the uvu multiplicity and path rule are the readings that
 * reproduce its output irreps); BranchIP ("Learning Adaptive Equivariant Computation
 * for Interatomic Potentials"), Method: zero-gated edges are left out of the tensor
 * product and the sparse result equals the dense one; Allegro paragraph: neighbours
 * within a fixed cutoff.
 *
 * Conventions (the pages leave them open; fixed here):
 *   - irreps spec strings "128x0e+64x1o" (mul x l, parity e/o); l <= 6.
 *   - paths: for each input irrep (spec order), each SH irrep (spec order), each
 *     l3 in |l1-l2| .. min(l1+l2, l_out_max): p3 = p1*p2; CGTP_PATHS_PARITY keeps the
 *     path only if p3 == (-1)^l3, CGTP_PATHS_ALL keeps all.  Multiplicity = mul(l1).
 *   - output irreps sorted by (l3, e before o); within one output irrep the path blocks
 *     follow path order.
 *   - real CG: Racah (Condon-Shortley), mapped to real harmonics, real part for even
 *     l1+l2+l3, imaginary part for odd; no path normalisation.
 *   - real SH: component normalisation (Y_0 = 1, sum_m Y_lm^2 = 2l+1), l = 1 is
 *     sqrt(3) (y, z, x); a zero-length edge has Y_0 = 1 and Y_l = 0 for l >= 1.
 * Layouts (fp32 / int, row-major, device memory unless stated):
 *   x   [n_nodes, f_in]   irreps in spec order, each block [mul][2l+1]
 *   out [n_nodes, f_out]  output irreps in sorted order, each block [mul][2l+1]
 *   w   [n_edges, w_per_edge]  column = global output channel index (uvu weights)
 *   pos [n_nodes, 3]; row_ptr int32 [n_nodes+1]; col int32 [n_edges];
 *   shift int8 [n_edges, 3] in {-1,0,1}; mask uint8 [n_edges] (nonzero = active).
 *
 * Ownership: the caller allocates and owns every device buffer, including the
 * workspace; the library never allocates in cgtp_neighbors_build, cgtp_conv_prepare,
 * cgtp_conv_forward or cgtp_edge_sh and keeps no pointer after a call returns.  A plan
 * owns its small device tables and, when its forward takes several kernel launches (plans
 * with paths of l >= 4, or more path groups than one launch carries), up to three HIP
 * streams and four events of its own (all freed by cgtp_plan_destroy).  A plan's tables
 * are immutable after creation; it may be shared by threads and streams (forward calls
 * on one plan take a per-plan lock while they enqueue).
 * Asynchrony: device work is enqueued on `stream` (a hipStream_t; NULL = default
 * stream) and not waited for, except where stated.  Inputs must stay valid until the
 * stream reaches that point.
 * Errors: every int-returning call returns CGTP_OK (0) or a negative code; arguments
 * are validated on the host before any launch; cgtp_last_error() returns a
 * thread-local message for the last failing call.  Contents of device arrays are not
 * validated (a malformed CSR is undefined behaviour).
 */
#ifndef CGTP_H_
#define CGTP_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct cgtp_plan_s* cgtp_plan_t;

enum {
  CGTP_OK = 0,
  CGTP_ERR_INVALID_ARG = -1,  /* null/misaligned pointer, negative size, bad flag */
  CGTP_ERR_PARSE = -2,        /* malformed irreps spec */
  CGTP_ERR_UNSUPPORTED = -3,  /* l > 6, SH multiplicity != 1, no path, too many jobs */
  CGTP_ERR_CAPACITY = -4,     /* edge list longer than the caller's capacity */
  CGTP_ERR_WORKSPACE = -5,    /* workspace smaller than the size query returned */
  CGTP_ERR_HIP = -6,          /* a HIP runtime call failed */
  CGTP_ERR_NO_DEVICE = -7     /* no usable gfx950 device */
};

enum { CGTP_PATHS_ALL = 0, CGTP_PATHS_PARITY = 1 };

/* Plan flags.  CGTP_PLAN_HOST_ONLY: build host tables only (no device upload); such a
 * plan answers the query calls but cgtp_conv_* return CGTP_ERR_INVALID_ARG with it.
 * CGTP_PLAN_FP64: the plan's forward runs in fp64 (LunaTP reports its kernels in
 * double precision: Figure 8, Table 11); it is used with cgtp_conv_forward_f64 only,
 * supports l <= 4 (else CGTP_ERR_UNSUPPORTED), and its workspace holds fp64
 * harmonics.  The fp32 forward entry points return CGTP_ERR_INVALID_ARG with an fp64
 * plan and cgtp_conv_forward_f64 with an fp32 plan. */
enum { CGTP_PLAN_HOST_ONLY = 1u, CGTP_PLAN_FP64 = 2u };

/* Parse irreps, enumerate paths, build the real-CG tables and the wave-job schedule,
 * and (unless CGTP_PLAN_HOST_ONLY) upload the job table to the current device.
 * irreps_sh must hold multiplicity-1 irreps.  Source: LunaTP Table 1 (irreps cases)
 * and Figure 3(b) (paths grouped and mapped to SIMD lanes by channel block).
 * Returns CGTP_ERR_PARSE / CGTP_ERR_UNSUPPORTED / CGTP_ERR_NO_DEVICE / CGTP_ERR_HIP. */
int cgtp_plan_create(const char* irreps_in, const char* irreps_sh, int l_out_max,
                     int path_rule, unsigned flags, cgtp_plan_t* out);

/* Sizes of the plan.  Any output pointer may be NULL.  irreps_out receives the
 * output irreps string (NUL-terminated, truncated to irreps_out_cap); for the six
 * irreps cases of LunaTP Table 1 it is the output column of that table. */
int cgtp_plan_info(cgtp_plan_t plan, int64_t* f_in, int64_t* f_out, int64_t* w_per_edge,
                   int* n_paths, int* l_sh_max, char* irreps_out, size_t irreps_out_cap);

/* Host array rows[n_paths * 10]: l1, p1, l2, p2, l3, p3, mul, in_off, out_off, w_off
 * per path (offsets as in the layouts above): the uvu paths whose outputs make up the
 * output irreps of LunaTP Table 1. */
int cgtp_plan_paths(cgtp_plan_t plan, int32_t* rows);

/* Host array dense[(2l1+1)(2l2+1)(2l3+1)] = real CG of path `path`, fp32, index
 * ((m1+l1)(2l2+1) + (m2+l2))(2l3+1) + (m3+l3): the sparse coupling coefficients that
 * LunaTP Figure 3(c) treats as constants of the kernel. */
int cgtp_plan_cg(cgtp_plan_t plan, int path, float* dense);

/* Scheduler summary: number of wave jobs and of distinct kernel variants used. */
int cgtp_plan_schedule(cgtp_plan_t plan, int* n_jobs, int* n_variants);

/* Workspace bytes that cgtp_conv_forward needs for this graph size (alignment 256).
 * Interface bookkeeping: the pages define no such call; it exists because the library
 * allocates nothing. */
int cgtp_workspace_size(cgtp_plan_t plan, int64_t n_nodes, int64_t n_edges, int has_mask,
                        size_t* bytes);

/* Workspace bytes that cgtp_neighbors_build needs. */
int cgtp_neighbors_workspace_size(int64_t n_nodes, const float box[3], float cutoff,
                                  size_t* bytes);

/* Receiver-CSR neighbour list under the minimum image convention of an orthorhombic
 * periodic box (BranchIP, Allegro paragraph: neighbours within a fixed cutoff).
 * Predicate, evaluated in fp64 without contraction, identical bit for bit to any
 * implementation of it:
 *   d = (double)pos_j - (double)pos_i; if d > L/2: d -= L, s = -1; else if d < -L/2:
 *   d += L, s = +1; else s = 0;  r2 = (dx*dx + dy*dy) + dz*dz;
 *   edge iff r2 < (double)cutoff * (double)cutoff and i != j.
 * Rows are sorted by j.  Positions must lie in [0, box).  box (host) and cutoff > 0.
 * Writes row_ptr[n_nodes+1] always; writes col/shift only if the edge count fits
 * edge_capacity, else returns CGTP_ERR_CAPACITY.  *n_edges (host) receives the edge
 * count in both cases.  SYNCHRONISES `stream` (the count is returned to the host). */
int cgtp_neighbors_build(const float* pos, int64_t n_nodes, const float box[3], float cutoff,
                         int32_t* row_ptr, int32_t* col, int8_t* shift, int64_t edge_capacity,
                         int64_t* n_edges, void* workspace, size_t ws_bytes, void* stream);

/* Active-edge CSR and node order (BranchIP sparse evaluation; LunaTP Table 9: nodes in
 * descending degree order).  mask NULL = all edges active.  Outputs (device):
 * act_row_ptr[n_nodes+1]; act_eid[<= n_edges] = ids of active edges in CSR order;
 * order[n_nodes] = nodes by active degree descending, then id ascending.
 * workspace: at least cgtp_workspace_size(plan, n_nodes, n_edges, mask != NULL). */
int cgtp_conv_prepare(cgtp_plan_t plan, const int32_t* row_ptr, const uint8_t* mask,
                      int64_t n_nodes, int64_t n_edges, int32_t* act_row_ptr, int32_t* act_eid,
                      int32_t* order, void* workspace, size_t ws_bytes, void* stream);

/* Real SH of every edge: sh[n_edges, (l_sh_max+1)^2], block l at offset l*l, m = -l..l,
 * of r_e = pos[j] - pos[i] + shift_e . cell (cell host, row-major 3x3, rows are lattice
 * vectors; NULL = open boundaries, shift ignored; shift NULL = zero).  Geometry and
 * harmonics in fp64, stored fp32. */
int cgtp_edge_sh(cgtp_plan_t plan, const float* pos, int64_t n_nodes, const float cell[9],
                 const int32_t* row_ptr, const int32_t* col, const int8_t* shift,
                 int64_t n_edges, float* sh, void* stream);

/* The CGTP convolution forward.  out[n_nodes, f_out] is overwritten (not accumulated);
 * rows with no active edge get exactly 0; w and x_j of inactive edges are never read.
 * Arguments as above; x [n_nodes, f_in], w [n_edges, w_per_edge], mask NULL = all
 * active.  All device pointers 16-byte aligned; x must be smaller than 4 GiB (the
 * kernel addresses it with 32-bit byte offsets), else CGTP_ERR_UNSUPPORTED.
 * Asynchronous on `stream`.  The result is bitwise reproducible from run to run.
 * Launches of different kernel classes write disjoint output columns; when there are
 * several, the call forks the plan's own streams from `stream` after the per-row pass
 * and joins them back into `stream` (events), so work enqueued on `stream` after the
 * call sees the whole output, and the call may be captured into a HIP graph. */
int cgtp_conv_forward(cgtp_plan_t plan, const float* pos, int64_t n_nodes, const float cell[9],
                      const int32_t* row_ptr, const int32_t* col, const int8_t* shift,
                      int64_t n_edges, const float* x, const float* w, const uint8_t* mask,
                      float* out, void* workspace, size_t ws_bytes, void* stream);

/* The forward with BranchIP's continuation gate (BranchIP, Method: each feature is
 * multiplied by its gate f in [0, 1] before the next tensor product, and zero-gated
 * features are omitted — sparse evaluation).  gate: device fp32 [n_edges], 4-byte
 * aligned, NULL = 1.  An edge is active when mask (if any) keeps it and gate[e] != 0;
 * an active edge's message is scaled by gate[e] (the product is linear in the edge's
 * feature), so out[i] = sum over active e of gate[e] * message_e.  w and x_j of
 * inactive edges are never read.  Everything else as cgtp_conv_forward; the workspace
 * size is the same. */
int cgtp_conv_forward_gated(cgtp_plan_t plan, const float* pos, int64_t n_nodes, const float cell[9],
                            const int32_t* row_ptr, const int32_t* col, const int8_t* shift,
                            int64_t n_edges, const float* x, const float* w, const uint8_t* mask,
                            const float* gate, float* out, void* workspace, size_t ws_bytes,
                            void* stream);

/* cgtp_conv_forward_gated (gate may be NULL), and in addition has the caller's HIP events
 * (hipEvent_t) ev_conv_begin / ev_conv_end stamped by the dispatch of the fused
 * convolution kernel itself (at the start of its first launch and the end of its last),
 * so that the caller can time that kernel apart from the prepare and harmonics passes
 * and from launch gaps.  When the launches are spread over the plan's streams the two
 * events are recorded on `stream` just before the fork and just after the join instead.
 * Same kernels, same results. */
int cgtp_conv_forward_timed(cgtp_plan_t plan, const float* pos, int64_t n_nodes, const float cell[9],
                            const int32_t* row_ptr, const int32_t* col, const int8_t* shift,
                            int64_t n_edges, const float* x, const float* w, const uint8_t* mask,
                            const float* gate, float* out, void* workspace, size_t ws_bytes,
                            void* stream, void* ev_conv_begin, void* ev_conv_end);

/* The forward in double precision, for plans created with CGTP_PLAN_FP64 (LunaTP,
 * Figure 8 and Table 11: the kernels are measured in fp64).  Same definition,
 * semantics and integer arguments as cgtp_conv_forward_gated; pos [n_nodes, 3], cell
 * (host, may be NULL), x, w, gate (may be NULL) and out are fp64, x, w and out 16-byte
 * aligned, pos and gate 8-byte aligned; x must be smaller than 4 GiB.  Geometry,
 * harmonics, coefficients and accumulation are fp64.  ev_conv_begin / ev_conv_end
 * (hipEvent_t, may be NULL) are stamped as in cgtp_conv_forward_timed.  The workspace
 * size is cgtp_workspace_size of the same plan. */
int cgtp_conv_forward_f64(cgtp_plan_t plan, const double* pos, int64_t n_nodes, const double cell[9],
                          const int32_t* row_ptr, const int32_t* col, const int8_t* shift,
                          int64_t n_edges, const double* x, const double* w, const uint8_t* mask,
                          const double* gate, double* out, void* workspace, size_t ws_bytes,
                          void* stream, void* ev_conv_begin, void* ev_conv_end);

/* Size of the device scratch array that cgtp_conv_forward_noalloc uses in place of a
 * workspace: 64 MiB per GPU (for fp32 plans with edge harmonics up to l = 3, about
 * 900 000 edges). */
#define CGTP_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/* cgtp_conv_forward_gated without a workspace argument and without any allocation, for
 * callers that cannot allocate device memory: code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc.  The kernels' scratch (per-row active
 * degrees, node records, the compacted active edges and their harmonics) lives in a
 * device array of CGTP_NOALLOC_SCRATCH_BYTES that the library holds on each GPU it runs
 * on until the process ends; its address is looked up once per device, on the first
 * call.  Graphs whose scratch (cgtp_workspace_size of the same plan and sizes) exceeds
 * the array are refused with CGTP_ERR_WORKSPACE before any launch.  Every call on one
 * GPU shares that GPU's array, and no part of it needs to start at zero: every value a
 * call reads was written by the same call.  Calls that overlap on one GPU (on streams
 * that are not ordered with respect to each other) race on the array; calls in stream
 * order do not.  The caller still allocates x, w, out and the other arguments.  fp32
 * plans only (an fp64 plan gives CGTP_ERR_INVALID_ARG); results are bitwise those of
 * cgtp_conv_forward_gated on the same inputs. */
int cgtp_conv_forward_noalloc(cgtp_plan_t plan, const float* pos, int64_t n_nodes, const float cell[9],
                              const int32_t* row_ptr, const int32_t* col, const int8_t* shift,
                              int64_t n_edges, const float* x, const float* w, const uint8_t* mask,
                              const float* gate, float* out, void* stream);

/* Workspace bytes that cgtp_conv_backward needs for this graph size (alignment 256). */
int cgtp_backward_workspace_size(cgtp_plan_t plan, int64_t n_nodes, int64_t n_edges, size_t* bytes);

/* Gradients of the convolution (the backward pass; LunaTP, Abstract: the derivatives
 * that forces need are within its kernels' scope).  Given grad_out = dL/d out
 * [n_nodes, f_out] for a scalar L of the forward's output, writes (each may be NULL to
 * skip it; each is overwritten):
 *   grad_x [n_nodes, f_in]:   dL/dx;
 *   grad_w [n_edges, w_per_edge]: dL/dw, rows of inactive edges exactly 0;
 *   grad_pos [n_nodes, 3]:    dL/dpos through r_e = pos[j] - pos[i] + shift_e . cell and
 *                             dY/dr (forces are -grad_pos when L is an energy).
 * The mask, gate (BranchIP continuation gate; it scales the message and is not
 * differentiated), cell and shifts are constants; inactive edges contribute nothing
 * and their w and x_j are never read.  fp32 plans whose largest l is 4 or less (else
 * CGTP_ERR_UNSUPPORTED; an fp64 plan gives CGTP_ERR_INVALID_ARG).  Other arguments as
 * cgtp_conv_forward_gated; x, w, grad_out and grad_w 16-byte aligned (the edge pass
 * moves them in 16-byte vectors), the other pointers 4-byte aligned; x smaller than
 * 4 GiB; workspace at least cgtp_backward_workspace_size (256-byte aligned).
 * Asynchronous on `stream`; results are bitwise reproducible (no floating-point
 * atomics). */
int cgtp_conv_backward(cgtp_plan_t plan, const float* pos, int64_t n_nodes, const float cell[9],
                       const int32_t* row_ptr, const int32_t* col, const int8_t* shift,
                       int64_t n_edges, const float* x, const float* w, const uint8_t* mask,
                       const float* gate, const float* grad_out, float* grad_x, float* grad_w,
                       float* grad_pos, void* workspace, size_t ws_bytes, void* stream);

/* Frees the plan's device tables, streams and events (interface bookkeeping; the pages
 * define no such call).  NULL is ignored. */
void cgtp_plan_destroy(cgtp_plan_t plan);

/* Thread-local message of the last failing call ("" if none).  Interface bookkeeping;
 * the pages define no such call. */
const char* cgtp_last_error(void);

/* Library version string. */
const char* cgtp_version(void);

#ifdef __cplusplus
}
#endif

#endif /* CGTP_H_ */
