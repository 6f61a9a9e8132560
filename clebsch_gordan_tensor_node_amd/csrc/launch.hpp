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

// Mask prepare: per-row active counts -> act_row_ptr (scan) and node order.
// deg, tmp_a, tmp_b: [n] int32 scratch.
hipError_t launch_prepare_rows(const int32_t* row_ptr, const uint8_t* mask, int n, int32_t* deg,
                               int32_t* act_row_ptr, int32_t* order, int32_t* tmp_a,
                               int32_t* tmp_b, hipStream_t s);

// Per-edge pass: compacted active-edge arrays and/or edge harmonics.
// act_eid, act_col, sh may each be null.  cell null = open boundaries.
struct EdgeGeom {
  const float* pos;
  const int32_t* row_ptr;
  const int32_t* col;
  const int8_t* shift;
  const uint8_t* mask;
  const int32_t* act_row_ptr;
  int n_nodes;
  int n_edges;
  int has_cell;
  double cell[9];
};
hipError_t launch_edge_pass(const EdgeGeom& g, int32_t* act_eid, int32_t* act_col, float* sh,
                            int l_sh_max, hipStream_t s);

// The fused conv kernel of one variant class over `args.total_tasks` wave tasks
// (one explicit instantiation per class, each in its own translation unit).
template <int C>
hipError_t launch_conv_class(const ConvArgs& args, hipStream_t s);
hipError_t launch_conv(const ConvArgs& args, int variant_class, hipStream_t s);

// Wave-task prefix of the jobs of one launch, on the device:
// task_start[k] = sum_{q<k} ceil(n_nodes / (64 >> jobs[q].lanes_log2)).
hipError_t launch_task_prefix(const Job* jobs, int n_jobs, int n_nodes, int32_t* task_start, hipStream_t s);

}  // namespace cgtp
