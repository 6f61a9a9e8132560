// Host-side launchers of the receiver-CSR neighbour-list kernels (kernels_graph.hip).
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
  int32_t* stats;        // {edges, longest row}
};

NbrGrid make_nbr_grid(int64_t n, const float box[3], float cutoff);
size_t nbr_workspace_bytes(int64_t n, const NbrGrid& g);
NbrWorkspace carve_nbr_workspace(void* ws, int64_t n, const NbrGrid& g);

// Cell binning, per-row counts and their scan into row_ptr (device); w.stats receives
// {edge count, longest row}.
hipError_t launch_nbr_count(const float* pos, int n, const NbrGrid& g, const NbrWorkspace& w,
                            int32_t* row_ptr, hipStream_t s);
// Fill col/shift of every row, each row sorted by j (max_degree: the longest row).
hipError_t launch_nbr_fill(const float* pos, int n, const NbrGrid& g, const NbrWorkspace& w,
                           const int32_t* row_ptr, int32_t* col, int8_t* shift, int max_degree, hipStream_t s);

}  // namespace cgtp
