// Host-side launchers of the HIP kernels (implemented next to the kernels).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.hpp"

namespace cgtp {

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
// The backward's edge pass over the same launch (args.grad_out, scratch_row, job_gy,
// job_xg and part_stride set; grad_w, gyp and xgp each null to skip): the w-gradient of
// every active edge and, per active slot, a row of partials holding each job's dL/dY and
// each job group's x-gradient of the edge.  Classes 0 .. kNumClassesBwd - 1.
template <int C>
hipError_t launch_conv_bwd_class(const ConvArgsT<float>& args, hipStream_t s);
hipError_t launch_conv_bwd(const ConvArgsT<float>& args, int cls, hipStream_t s);
constexpr int kNumClassesBwd = 7;
// Zeroes the w-gradient rows [n_edges, w_stride] of the inactive edges (mask == 0 or
// gate == 0; mask and gate may each be null).
hipError_t launch_zero_inactive(const int32_t* row_ptr, const uint8_t* mask, const float* gate, int n_nodes,
                                float* grad_w, int w_stride, hipStream_t s);
hipError_t launch_conv(const ConvArgsT<float>& args, int cls, hipStream_t s, hipEvent_t ev_start, hipEvent_t ev_stop);
hipError_t launch_conv(const ConvArgsT<double>& args, int cls, hipStream_t s, hipEvent_t ev_start,
                       hipEvent_t ev_stop);

// Largest l of a plan that the backward supports.
constexpr int kBwdLmax = 4;


// Active slots grouped by sender: t_row_ptr [n+1], t_slot / t_recv [active edges], each
// sender's entries in slot order.  t_cnt: [n] scratch.
hipError_t launch_bwd_transpose(const BwdArgs& a, int32_t* t_cnt, int32_t* t_row_ptr, int32_t* t_slot,
                                int32_t* t_recv, hipStream_t s);
// Per sender: dL/dx from the edge pass's x-gradient blocks of its slots.
hipError_t launch_bwd_gather_x(const BwdArgs& a, hipStream_t s);
// Per sender: dL/dr of its slots from their dL/dY partials and dY/dr.
hipError_t launch_bwd_force(const BwdArgs& a, hipStream_t s);
// The position gradient from dL/dr: + at each slot's sender, - at its receiver.
hipError_t launch_bwd_pos(const BwdArgs& a, hipStream_t s);

}  // namespace cgtp
