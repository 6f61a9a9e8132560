// Host-side launchers of the HIP kernels (implemented next to the kernels).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.hpp"

namespace cgtp {

struct NbrGrid {
  int nc[3];        // cells per dimension
  double box[3];    // box lengths (fp64 copies of the fp32 values)
  double rc2;       // cutoff^2 in fp64
  int n_cells() const { return nc[0] * nc[1] * nc[2]; }
};

// Workspace of the neighbour-list build, in int32 elements.
struct NbrWorkspace {
  int32_t* cell_count;   // [n_cells] (also the fill cursor)
  int32_t* cell_start;   // [n_cells + 1]
  int32_t* atom_cell;    // [n]
  int32_t* cell_atoms;   // [n]
  int32_t* row_count;    // [n]
};

NbrGrid make_nbr_grid(int64_t n, const float box[3], float cutoff);
size_t nbr_workspace_bytes(int64_t n, const NbrGrid& g);
NbrWorkspace carve_nbr_workspace(void* ws, int64_t n, const NbrGrid& g);

// Cell binning, per-row counts and their scan into row_ptr (device).
hipError_t launch_nbr_count(const float* pos, int n, const NbrGrid& g, const NbrWorkspace& w,
                            int32_t* row_ptr, hipStream_t s);
// Fill col/shift of every row and sort each row by j.
hipError_t launch_nbr_fill(const float* pos, int n, const NbrGrid& g, const NbrWorkspace& w,
                           const int32_t* row_ptr, int32_t* col, int8_t* shift, hipStream_t s);

// Per-row pass: active-edge count per row and, compacted within each row's CSR segment,
// the active edge ids, senders and harmonics (sh [n_edges, (l_sh_max+1)^2]).  Every
// output may be null.  Without a mask the slots are the edges themselves.  The fp64
// fields (pos64, gate64, sh64; l_sh_max <= 3) replace pos, gate and sh for an fp64
// forward; one pass uses one element type.
struct RowPass {
  const float* pos;
  const int32_t* row_ptr;
  const int32_t* col;
  const int8_t* shift;
  const uint8_t* mask;
  const float* gate;   // continuation gate per edge (may be null): 0 = inactive, else it
                       // scales the stored harmonics
  int32_t* deg;
  int32_t* act_e;  // active edge ids compacted within each row (at row_ptr[i] + q)
  int32_t* act_j;  // their senders
  float* sh;       // their harmonics, same slots
  const double* pos64;
  const double* gate64;
  double* sh64;
  int sh_stride;   // floats per SH row (0: (l_sh_max + 1)^2); entries past (l_sh_max + 1)^2 are zeroed
  int n_nodes;
  int n_edges;
  int has_cell;
  double cell[9];
};
hipError_t launch_rows(const RowPass& p, int l_sh_max, hipStream_t s);
// launch_rows and launch_degree_order in one launch, for a pass without mask and gate
// (the degrees are the row lengths); deg is still written when requested.
hipError_t launch_rows_order(const RowPass& p, int l_sh_max, int4* node_info, hipStream_t s);

// One workgroup: optional exclusive scan of deg into act_row_ptr and the node order by
// deg descending, ties by id ascending, into order (may be null).
// tmp_a, tmp_b: [n] int32 scratch.
hipError_t launch_order(const int32_t* deg, int n, int32_t* act_row_ptr, int32_t* order, int32_t* tmp_a,
                        int32_t* tmp_b, hipStream_t s);

// node_info[pos] = {node, row_ptr[node], deg[node], 0} by descending degree; nodes of
// equal degree in any order (one workgroup).
hipError_t launch_degree_order(const int32_t* deg, int n, const int32_t* row_ptr, int4* node_info, hipStream_t s);

// Ids of the active edges in CSR order, at act_row_ptr[i] + rank within row i.
hipError_t launch_compact(const int32_t* row_ptr, const uint8_t* mask, const int32_t* act_row_ptr, int n_nodes,
                          int n_edges, int32_t* act_eid, hipStream_t s);

// The fused conv kernel of one variant class over `args.total_wgs` workgroups (one per
// job group and node group; one explicit instantiation per class and element type,
// each class in its own translation unit; fp64 for the classes below kNumClassesF64).
// ev_start / ev_stop (may be null): HIP events stamped at this launch's start / end.
template <int C, typename T>
hipError_t launch_conv_class(const ConvArgsT<T>& args, hipStream_t s, hipEvent_t ev_start, hipEvent_t ev_stop);
hipError_t launch_conv(const ConvArgsT<float>& args, int cls, hipStream_t s, hipEvent_t ev_start, hipEvent_t ev_stop);
hipError_t launch_conv(const ConvArgsT<double>& args, int cls, hipStream_t s, hipEvent_t ev_start,
                       hipEvent_t ev_stop);

// Largest l of a plan that the backward supports.
constexpr int kBwdLmax = 4;

// Backward of the convolution (fp32, plans with l <= kBwdLmax).  bwd_edges: w-gradient of every
// edge (zero rows for inactive ones) and, when want_gy, the per-path dL/dY partial of
// every active slot; one wave per (receiver, path).  high: the plan has paths of
// l = kBwdLmax (they run in a second launch, built apart from the l <= 3 code).
hipError_t launch_bwd_edges(const BwdArgs& a, bool high, hipStream_t s);
// Active slots grouped by sender: t_row_ptr [n+1], t_slot / t_recv [active edges], each
// sender's entries in slot order.  t_cnt: [n] scratch.
hipError_t launch_bwd_transpose(const BwdArgs& a, int32_t* t_cnt, int32_t* t_row_ptr, int32_t* t_slot,
                                int32_t* t_recv, hipStream_t s);
// x-gradient: one wave per (sender, input irrep) when those waves fill the chip, else
// per-path partials (one wave per (sender, path)) and their sum per input irrep in path
// order; high as for the edge pass (the l = kBwdLmax paths run in a second launch).
hipError_t launch_bwd_x(const BwdArgs& a, bool high, hipStream_t s);
// dL/dr per active slot from the partials and dY/dr, then the position gradient.
hipError_t launch_bwd_pos(const BwdArgs& a, hipStream_t s);

}  // namespace cgtp
