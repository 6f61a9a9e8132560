// Graph-side kernels: receiver-CSR neighbour list, mask prepare (active CSR and node
// order) and the per-edge pass that compacts active edges and evaluates the edge
// harmonics.  All integer outputs are deterministic: atomics are used only for
// counts, and every order-dependent result is sorted or scanned afterwards.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>

#include "launch.hpp"
#include "nbr.hpp"
#include "sh_eval.hpp"
#include "variants.hpp"

namespace cgtp {

namespace {

constexpr int kScanThreads = 1024;
constexpr int kDegCache = 8192;
constexpr int kScanWaves = kScanThreads / kWave;

__device__ inline int lane_id() { return __lane_id(); }

// Block-wide exclusive scan of one value per thread (1024 threads).  `wsum` holds
// kScanWaves ints of LDS.  Returns the exclusive prefix and sets `total`.
__device__ inline int block_exclusive_scan(int v, int* wsum, int& total) {
  const int lane = lane_id();
  const int wave = threadIdx.x / kWave;
  int inc = v;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    int t = __shfl_up(inc, d, kWave);
    if (lane >= d) inc += t;
  }
  if (lane == kWave - 1) wsum[wave] = inc;
  __syncthreads();
  if (threadIdx.x == 0) {
    int run = 0;
    for (int k = 0; k < kScanWaves; ++k) {
      int t = wsum[k];
      wsum[k] = run;
      run += t;
    }
    wsum[kScanWaves] = run;
  }
  __syncthreads();
  int excl = wsum[wave] + inc - v;
  total = wsum[kScanWaves];
  __syncthreads();
  return excl;
}

// out[k] = sum_{q<k} in[q] for k <= n (out has n+1 entries).  One workgroup.  stats
// (may be null) receives {sum, largest value}.
__global__ void __launch_bounds__(kScanThreads) scan_exclusive_kernel(const int32_t* in, int32_t* out, int n,
                                                                     int32_t* stats) {
  __shared__ int wsum[kScanWaves + 1];
  __shared__ int s_max;
  if (threadIdx.x == 0) s_max = 0;
  int carry = 0, vmax = 0;
  for (int base = 0; base < n; base += kScanThreads) {
    const int idx = base + threadIdx.x;
    const int v = idx < n ? in[idx] : 0;
    vmax = max(vmax, v);
    int total;
    const int ex = block_exclusive_scan(v, wsum, total);
    if (idx < n) out[idx] = carry + ex;
    carry += total;
  }
  if (stats) {
    atomicMax(&s_max, vmax);
    __syncthreads();
    if (threadIdx.x == 0) {
      stats[0] = carry;
      stats[1] = s_max;
    }
  }
  if (threadIdx.x == 0) out[n] = carry;
}

// ---------------------------------------------------------------------------------
// Neighbour list.  Predicate in fp64 with contraction disabled, so that the result is
// the same bit for bit as any implementation that follows the stated operation order.
// ---------------------------------------------------------------------------------

struct GridArgs {
  int nc[3];
  double box[3];
  double rc2;
};

__device__ inline bool pair_within(const float* __restrict__ pos, int i, int j, const GridArgs& g,
                                   int8_t* s) {
#pragma clang fp contract(off)
  double d[3];
#pragma unroll
  for (int k = 0; k < 3; ++k) {
    double dk = double(pos[3 * j + k]) - double(pos[3 * i + k]);
    const double half = 0.5 * g.box[k];
    int8_t sk = 0;
    if (dk > half) {
      dk = dk - g.box[k];
      sk = -1;
    } else if (dk < -half) {
      dk = dk + g.box[k];
      sk = 1;
    }
    d[k] = dk;
    s[k] = sk;
  }
  const double r2 = (d[0] * d[0] + d[1] * d[1]) + d[2] * d[2];
  return r2 < g.rc2;
}

__device__ inline int cell_coord(float x, double box, int nc) {
  int c = int(floor(double(x) * double(nc) / box));
  return c < 0 ? 0 : (c >= nc ? nc - 1 : c);
}

__global__ void fill_i32_kernel(int32_t* __restrict__ p, int n, int32_t v) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

__global__ void nbr_assign_kernel(const float* __restrict__ pos, int n, GridArgs g,
                                  int32_t* __restrict__ atom_cell, int32_t* __restrict__ cell_count) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const int cx = cell_coord(pos[3 * i + 0], g.box[0], g.nc[0]);
  const int cy = cell_coord(pos[3 * i + 1], g.box[1], g.nc[1]);
  const int cz = cell_coord(pos[3 * i + 2], g.box[2], g.nc[2]);
  const int c = (cz * g.nc[1] + cy) * g.nc[0] + cx;
  atom_cell[i] = c;
  atomicAdd(&cell_count[c], 1);
}

__global__ void nbr_bin_kernel(int n, const int32_t* __restrict__ atom_cell,
                               const int32_t* __restrict__ cell_start, int32_t* __restrict__ cursor,
                               int32_t* __restrict__ cell_atoms) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const int c = atom_cell[i];
  cell_atoms[cell_start[c] + atomicAdd(&cursor[c], 1)] = i;
}

// Visit every distinct stencil cell once (a dimension with 1 or 2 cells would
// otherwise be visited twice through the periodic wrap).
template <typename F>
__device__ inline void for_each_stencil_cell(int c, const GridArgs& g, F&& f) {
  const int cx = c % g.nc[0];
  const int cy = (c / g.nc[0]) % g.nc[1];
  const int cz = c / (g.nc[0] * g.nc[1]);
  const int lo[3] = {g.nc[0] >= 3 ? -1 : 0, g.nc[1] >= 3 ? -1 : 0, g.nc[2] >= 3 ? -1 : 0};
  const int hi[3] = {g.nc[0] >= 2 ? 1 : 0, g.nc[1] >= 2 ? 1 : 0, g.nc[2] >= 2 ? 1 : 0};
  for (int dz = lo[2]; dz <= hi[2]; ++dz) {
    const int z = (cz + dz + g.nc[2]) % g.nc[2];
    for (int dy = lo[1]; dy <= hi[1]; ++dy) {
      const int y = (cy + dy + g.nc[1]) % g.nc[1];
      for (int dx = lo[0]; dx <= hi[0]; ++dx) {
        const int x = (cx + dx + g.nc[0]) % g.nc[0];
        f((z * g.nc[1] + y) * g.nc[0] + x);
      }
    }
  }
}

// Wave-per-atom passes: the 64 lanes of a wave take atom i's candidates (the atoms of its
// distinct stencil cells, as one flattened list) 64 at a time, each testing one with the
// same predicate.  The stencil's cells and the running totals of their atom counts sit
// in a small per-wave LDS table that each lane searches for its candidate's cell.
constexpr int kNbrWaves = 4;         // waves (atoms) per workgroup
constexpr int kNbrRowCap = 1024;     // neighbours of one atom that the fill pass ranks in LDS

struct StencilTable {
  int pre[32];     // atoms in the stencil cells before cell s
  int start[32];   // cell s's first entry in cell_atoms
};

// Fills this wave's table for cell c; returns the stencil's atom count (every lane).
__device__ inline int stencil_table(int c, const GridArgs& g, const int32_t* __restrict__ cell_start,
                                    StencilTable& t) {
  const int lane = lane_id();
  const int cx = c % g.nc[0], cy = (c / g.nc[0]) % g.nc[1], cz = c / (g.nc[0] * g.nc[1]);
  int lo[3], cnt3[3];
#pragma unroll
  for (int k = 0; k < 3; ++k) {
    lo[k] = g.nc[k] >= 3 ? -1 : 0;
    cnt3[k] = (g.nc[k] >= 2 ? 1 : 0) - lo[k] + 1;   // distinct offsets along k
  }
  const int n_cells = cnt3[0] * cnt3[1] * cnt3[2];
  int cnt = 0, beg = 0;
  if (lane < n_cells) {
    const int ix = lane % cnt3[0], iy = (lane / cnt3[0]) % cnt3[1], iz = lane / (cnt3[0] * cnt3[1]);
    const int x = (cx + lo[0] + ix + g.nc[0]) % g.nc[0];
    const int y = (cy + lo[1] + iy + g.nc[1]) % g.nc[1];
    const int z = (cz + lo[2] + iz + g.nc[2]) % g.nc[2];
    const int cell = (z * g.nc[1] + y) * g.nc[0] + x;
    beg = cell_start[cell];
    cnt = cell_start[cell + 1] - beg;
  }
  int inc = cnt;
#pragma unroll
  for (int d = 1; d < 32; d <<= 1) {
    const int u = __shfl_up(inc, d, kWave);
    if (lane >= d) inc += u;
  }
  if (lane < 32) {
    t.pre[lane] = inc - cnt;
    t.start[lane] = beg;
  }
  return __shfl(inc, 31, kWave);
}

// Candidate q of the stencil (0 <= q < total): its atom id.
__device__ inline int stencil_atom(int q, const StencilTable& t, const int32_t* __restrict__ cell_atoms) {
  int s = 0;   // the last cell whose running total is at most q (binary search over 32)
#pragma unroll
  for (int b = 16; b > 0; b >>= 1)
    if (t.pre[s + b] <= q) s += b;
  return cell_atoms[t.start[s] + (q - t.pre[s])];
}

__global__ void __launch_bounds__(kNbrWaves * kWave) nbr_count_wave_kernel(
    const float* __restrict__ pos, int n, GridArgs g, const int32_t* __restrict__ atom_cell,
    const int32_t* __restrict__ cell_start, const int32_t* __restrict__ cell_atoms, int32_t* __restrict__ row_count) {
  __shared__ StencilTable tab[kNbrWaves];
  const int wave = threadIdx.x / kWave;
  const int i = __builtin_amdgcn_readfirstlane(int(blockIdx.x) * kNbrWaves + wave);
  if (i >= n) return;   // no barrier in this kernel: a wave may leave alone
  StencilTable& t = tab[wave];
  const int total = stencil_table(atom_cell[i], g, cell_start, t);
  __builtin_amdgcn_wave_barrier();
  int cnt = 0;
  for (int q0 = 0; q0 < total; q0 += kWave) {
    const int q = q0 + lane_id();
    bool hit = false;
    if (q < total) {
      const int j = stencil_atom(q, t, cell_atoms);
      int8_t sh[3];
      hit = j != i && pair_within(pos, i, j, g, sh);
    }
    cnt += __popcll(__ballot(hit));
  }
  if (lane_id() == 0) row_count[i] = cnt;
}

// Fill of rows of at most kNbrRowCap neighbours: the wave compacts atom i's neighbours
// into LDS (in candidate order, ballot-ranked) and writes each at its rank among them by
// sender id, so the row comes out sorted by j (the ids of one row are distinct).
__global__ void __launch_bounds__(kNbrWaves * kWave) nbr_fill_wave_kernel(
    const float* __restrict__ pos, int n, GridArgs g, const int32_t* __restrict__ atom_cell,
    const int32_t* __restrict__ cell_start, const int32_t* __restrict__ cell_atoms,
    const int32_t* __restrict__ row_ptr, int32_t* __restrict__ col, int8_t* __restrict__ shift) {
  __shared__ StencilTable tab[kNbrWaves];
  __shared__ int s_j[kNbrWaves][kNbrRowCap];
  __shared__ int s_code[kNbrWaves][kNbrRowCap];   // (s0 + 1) 9 + (s1 + 1) 3 + (s2 + 1)
  const int wave = threadIdx.x / kWave;
  const int lane = lane_id();
  const int i = __builtin_amdgcn_readfirstlane(int(blockIdx.x) * kNbrWaves + wave);
  if (i >= n) return;
  const int rb = row_ptr[i], deg = row_ptr[i + 1] - rb;
  if (deg > kNbrRowCap || deg == 0) return;   // long rows: nbr_fill_kernel
  StencilTable& t = tab[wave];
  const int total = stencil_table(atom_cell[i], g, cell_start, t);
  __builtin_amdgcn_wave_barrier();
  const unsigned long long lt = lane == 0 ? 0ull : (~0ull >> (64 - lane));
  int m = 0;
  for (int q0 = 0; q0 < total; q0 += kWave) {
    const int q = q0 + lane;
    bool hit = false;
    int j = 0;
    int8_t sh[3] = {0, 0, 0};
    if (q < total) {
      j = stencil_atom(q, t, cell_atoms);
      hit = j != i && pair_within(pos, i, j, g, sh);
    }
    const unsigned long long bal = __ballot(hit);
    const int at = m + __popcll(bal & lt);
    if (hit && at < deg) {   // at < deg always: the count pass used the same predicate
      s_j[wave][at] = j;
      s_code[wave][at] = (sh[0] + 1) * 9 + (sh[1] + 1) * 3 + (sh[2] + 1);
    }
    m += __popcll(bal);
  }
  m = min(m, deg);
  __builtin_amdgcn_wave_barrier();
  for (int k = lane; k < m; k += kWave) {
    const int jk = s_j[wave][k];
    int r = 0;
    for (int u = 0; u < m; ++u) r += s_j[wave][u] < jk;
    const int code = s_code[wave][k];
    const int at = rb + r;
    col[at] = jk;
    shift[3 * at + 0] = int8_t(code / 9 - 1);
    shift[3 * at + 1] = int8_t((code / 3) % 3 - 1);
    shift[3 * at + 2] = int8_t(code % 3 - 1);
  }
}

__global__ void nbr_count_kernel(const float* __restrict__ pos, int n, GridArgs g,
                                 const int32_t* __restrict__ atom_cell,
                                 const int32_t* __restrict__ cell_start,
                                 const int32_t* __restrict__ cell_atoms, int32_t* __restrict__ row_count) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  int cnt = 0;
  for_each_stencil_cell(atom_cell[i], g, [&](int c) {
    for (int k = cell_start[c]; k < cell_start[c + 1]; ++k) {
      const int j = cell_atoms[k];
      int8_t s[3];
      if (j != i && pair_within(pos, i, j, g, s)) ++cnt;
    }
  });
  row_count[i] = cnt;
}

__global__ void nbr_fill_kernel(const float* __restrict__ pos, int n, GridArgs g,
                                const int32_t* __restrict__ atom_cell,
                                const int32_t* __restrict__ cell_start,
                                const int32_t* __restrict__ cell_atoms,
                                const int32_t* __restrict__ row_ptr, int32_t* __restrict__ col,
                                int8_t* __restrict__ shift) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const int beg = row_ptr[i];
  if (row_ptr[i + 1] - beg <= kNbrRowCap) return;   // filled by nbr_fill_wave_kernel
  int end = beg;
  for_each_stencil_cell(atom_cell[i], g, [&](int c) {
    for (int k = cell_start[c]; k < cell_start[c + 1]; ++k) {
      const int j = cell_atoms[k];
      int8_t s[3];
      if (j != i && pair_within(pos, i, j, g, s)) {
        col[end] = j;
        shift[3 * end + 0] = s[0];
        shift[3 * end + 1] = s[1];
        shift[3 * end + 2] = s[2];
        ++end;
      }
    }
  });
  // rows are short: insertion sort by j (j values within a row are distinct)
  for (int a = beg + 1; a < end; ++a) {
    const int key = col[a];
    const int8_t s0 = shift[3 * a], s1 = shift[3 * a + 1], s2 = shift[3 * a + 2];
    int b = a - 1;
    while (b >= beg && col[b] > key) {
      col[b + 1] = col[b];
      shift[3 * (b + 1) + 0] = shift[3 * b + 0];
      shift[3 * (b + 1) + 1] = shift[3 * b + 1];
      shift[3 * (b + 1) + 2] = shift[3 * b + 2];
      --b;
    }
    col[b + 1] = key;
    shift[3 * (b + 1) + 0] = s0;
    shift[3 * (b + 1) + 1] = s1;
    shift[3 * (b + 1) + 2] = s2;
  }
}

// ---------------------------------------------------------------------------------
// Mask prepare.
// ---------------------------------------------------------------------------------

// One workgroup: act_row_ptr = exclusive scan of deg (if requested); order = node ids
// sorted by deg descending, ties by id ascending (stable LSD radix sort on
// maxdeg - deg, 8-bit digits, ranks inside a wave from ballots, across waves from an
// LDS table).
// Degrees are cached in LDS when n <= kDegCache, so each radix pass reads LDS only.
__global__ void __launch_bounds__(kScanThreads) prep_scan_order_kernel(const int32_t* __restrict__ deg, int n,
                                                                      int32_t* __restrict__ act_row_ptr,
                                                                      int32_t* __restrict__ order,
                                                                      int32_t* __restrict__ tmp_a,
                                                                      int32_t* __restrict__ tmp_b) {
  __shared__ int wsum[kScanWaves + 1];
  __shared__ int s_max;
  __shared__ int hist[256];
  __shared__ int base[256];
  __shared__ int tile_tot[256];
  __shared__ int wcnt[kScanWaves][256];
  __shared__ int s_deg[kDegCache];

  const int tid = threadIdx.x;
  const bool cached = n <= kDegCache;
  const int lane = lane_id();
  const int wave = tid / kWave;

  // 1. scan (optional) and maximum
  if (tid == 0) s_max = 0;
  __syncthreads();
  int carry = 0;
  int local_max = 0;
  for (int b0 = 0; b0 < n; b0 += kScanThreads) {
    const int idx = b0 + tid;
    const int v = idx < n ? deg[idx] : 0;
    if (cached && idx < n) s_deg[idx] = v;
    local_max = v > local_max ? v : local_max;
    if (act_row_ptr) {
      int total;
      const int ex = block_exclusive_scan(v, wsum, total);
      if (idx < n) act_row_ptr[idx] = carry + ex;
      carry += total;
    }
  }
  if (act_row_ptr && tid == 0) act_row_ptr[n] = carry;
  atomicMax(&s_max, local_max);
  __syncthreads();
  const int maxdeg = s_max;

  int passes = 0;
  for (int m = maxdeg; m > 0; m >>= 8) ++passes;
  if (passes == 0) {
    for (int idx = tid; idx < n; idx += kScanThreads)
      if (order) order[idx] = idx;
    return;
  }

  const unsigned long long lt_mask = (lane == 0) ? 0ull : ((~0ull) >> (64 - lane));
  for (int p = 0; p < passes; ++p) {
    const int32_t* src = (p == 0) ? nullptr : ((p - 1) % 2 == 0 ? tmp_a : tmp_b);
    const bool last = p == passes - 1;
    int32_t* dst = last ? order : (p % 2 == 0 ? tmp_a : tmp_b);
    const int shift = 8 * p;
    for (int k = tid; k < 256; k += kScanThreads) hist[k] = 0;
    __syncthreads();
    for (int idx = tid; idx < n; idx += kScanThreads) {
      const int id = src ? src[idx] : idx;
      const int digit = ((maxdeg - (cached ? s_deg[id] : deg[id])) >> shift) & 255;
      atomicAdd(&hist[digit], 1);
    }
    __syncthreads();
    {
      int total;
      const int ex = block_exclusive_scan(tid < 256 ? hist[tid] : 0, wsum, total);
      if (tid < 256) base[tid] = ex;
    }
    __syncthreads();
    for (int b0 = 0; b0 < n; b0 += kScanThreads) {
      const int idx = b0 + tid;
      const bool valid = idx < n;
      const int id = valid ? (src ? src[idx] : idx) : 0;
      const int digit = valid ? (((maxdeg - (cached ? s_deg[id] : deg[id])) >> shift) & 255) : 0;
      unsigned long long same = __ballot(valid);
#pragma unroll
      for (int bit = 0; bit < 8; ++bit) {
        const bool on = (digit >> bit) & 1;
        const unsigned long long bb = __ballot(on);
        same &= on ? bb : ~bb;
      }
      const int rank = __popcll(same & lt_mask);
      const int cnt = __popcll(same);
      for (int k = tid; k < kScanWaves * 256; k += kScanThreads) (&wcnt[0][0])[k] = 0;
      __syncthreads();
      if (valid && rank == 0) wcnt[wave][digit] = cnt;
      __syncthreads();
      if (tid < 256) {
        int run = 0;
        for (int w = 0; w < kScanWaves; ++w) {
          const int t = wcnt[w][tid];
          wcnt[w][tid] = run;
          run += t;
        }
        tile_tot[tid] = run;
      }
      __syncthreads();
      if (valid) {
        const int at = base[digit] + wcnt[wave][digit] + rank;
        if (dst) dst[at] = id;
      }
      __syncthreads();
      if (tid < 256) base[tid] += tile_tot[tid];
      __syncthreads();
    }
  }
}

// ---------------------------------------------------------------------------------
// Node records of the forward: node_info[pos] = {node, row_ptr[node], deg[node], 0} in
// descending degree order (LunaTP Table 9), as a one-pass counting sort in one
// workgroup: LDS histogram of the degrees, scan from the largest degree down, and each
// node placed by an LDS atomic on its degree's cursor.  Nodes of equal degree land in
// any order (the convolution of a receiver does not depend on its position); degrees
// above kOrderBins - 1 share the top bin.
// ---------------------------------------------------------------------------------

constexpr int kOrderBins = kScanThreads;

// Graphs of up to kOrderCache nodes keep each node's degree and row start in LDS from
// the counting pass to the placing pass, which then reads no global memory (one memory
// round trip per launch instead of two); every load of the counting pass is issued before
// the first is used.
constexpr int kOrderCache = 6144;
constexpr int kOrderUnroll = (kOrderCache + kScanThreads - 1) / kScanThreads;

// deg may be null: then every edge is active and deg[i] = row_ptr[i + 1] - row_ptr[i]
__device__ inline void degree_order_body(const int32_t* __restrict__ deg, int n, const int32_t* __restrict__ row_ptr,
                                         int4* __restrict__ node_info) {
  __shared__ int wsum[kScanWaves + 1];
  __shared__ int cursor[kOrderBins];
  __shared__ int c_deg[kOrderCache];
  __shared__ int c_row[kOrderCache];
  if (n <= 0) return;   // (uniform)
  const int tid = threadIdx.x;
  auto degree = [&](int i) { return deg ? deg[i] : row_ptr[i + 1] - row_ptr[i]; };
  const bool cached = n <= kOrderCache;
  cursor[tid] = 0;
  __syncthreads();
  if (cached) {
    int d[kOrderUnroll], r[kOrderUnroll];
#pragma unroll
    for (int u = 0; u < kOrderUnroll; ++u) {
      const int i = min(tid + u * kScanThreads, n - 1);
      r[u] = row_ptr[i];
      d[u] = deg ? deg[i] : row_ptr[i + 1];
    }
#pragma unroll
    for (int u = 0; u < kOrderUnroll; ++u) {
      const int i = tid + u * kScanThreads;
      if (i < n) {
        const int dd = deg ? d[u] : d[u] - r[u];
        c_deg[i] = dd;
        c_row[i] = r[u];
        atomicAdd(&cursor[min(dd, kOrderBins - 1)], 1);
      }
    }
  } else {
    for (int i = tid; i < n; i += kScanThreads) atomicAdd(&cursor[min(degree(i), kOrderBins - 1)], 1);
  }
  __syncthreads();
  // exclusive scan over the bins from the top degree down
  const int b = kOrderBins - 1 - tid;
  const int cnt = cursor[b];
  int total;
  const int ex = block_exclusive_scan(cnt, wsum, total);
  cursor[b] = ex;
  __syncthreads();
  for (int i = tid; i < n; i += kScanThreads) {
    const int d = cached ? c_deg[i] : degree(i);
    const int pos = atomicAdd(&cursor[min(d, kOrderBins - 1)], 1);
    node_info[pos] = make_int4(i, cached ? c_row[i] : row_ptr[i], d, 0);
  }
}

__global__ void __launch_bounds__(kScanThreads) degree_order_kernel(const int32_t* __restrict__ deg, int n,
                                                                    const int32_t* __restrict__ row_ptr,
                                                                    int4* __restrict__ node_info) {
  degree_order_body(deg, n, row_ptr, node_info);
}

// ---------------------------------------------------------------------------------
// Per-row pass (one wave per receiver row, lanes over its edges): active-edge count and
// the real harmonics of every active edge, stored in CSR edge order.  Geometry and
// harmonics in fp64, stored fp32.
// ---------------------------------------------------------------------------------

// P: element type of the positions, the gate and the stored harmonics (float or double)
template <typename P>
struct RowArgs {
  const P* pos;
  const int32_t* row_ptr;
  const int32_t* col;
  const int8_t* shift;
  const uint8_t* mask;
  const P* gate;   // may be null: continuation gate per edge (0 = inactive)
  int32_t* deg;    // may be null
  int32_t* act_e;  // may be null
  int32_t* act_j;  // may be null
  P* sh;           // may be null
  int n_nodes;
  int has_cell;
  int sh_stride;
  double cell[9];
};

constexpr int kRowThreads = 256;

// Row i's active edges are written compacted within the row's own CSR segment: the
// q-th active edge of row i goes to slot row_ptr[i] + q (q from a ballot prefix).  With
// no mask the slot is the edge itself.
template <int L, typename P>
__device__ inline void edge_rows_body(const RowArgs<P>& a, int row) {
  if (row >= a.n_nodes) return;
  const int lane = lane_id();
  const unsigned long long lt_mask = (lane == 0) ? 0ull : ((~0ull) >> (64 - lane));
  const int rb = a.row_ptr[row], re = a.row_ptr[row + 1];
  const double pi0 = a.pos ? a.pos[3 * row + 0] : 0.0;
  const double pi1 = a.pos ? a.pos[3 * row + 1] : 0.0;
  const double pi2 = a.pos ? a.pos[3 * row + 2] : 0.0;
  int cnt = 0;
  for (int b0 = rb; b0 < re; b0 += kWave) {
    const int e = b0 + lane;
    const bool act = e < re && (!a.mask || a.mask[e] != 0) && (!a.gate || a.gate[e] != P(0));
    const unsigned long long bal = __ballot(act);
    const int slot = rb + cnt + __popcll(bal & lt_mask);
    cnt += __popcll(bal);
    if (!act) continue;
    const int j = (a.act_j || a.sh) ? a.col[e] : 0;
    if (a.act_e) a.act_e[slot] = e;
    if (a.act_j) a.act_j[slot] = j;
    if (!a.sh) continue;
    double r[3] = {double(a.pos[3 * j + 0]) - pi0, double(a.pos[3 * j + 1]) - pi1, double(a.pos[3 * j + 2]) - pi2};
    if (a.has_cell && a.shift) {
      const double s0 = a.shift[3 * e + 0], s1 = a.shift[3 * e + 1], s2 = a.shift[3 * e + 2];
#pragma unroll
      for (int k = 0; k < 3; ++k) r[k] = r[k] + s0 * a.cell[k] + s1 * a.cell[3 + k] + s2 * a.cell[6 + k];
    }
    const double rr = sqrt(r[0] * r[0] + r[1] * r[1] + r[2] * r[2]);
    constexpr int NY = (L + 1) * (L + 1);
    double Y[NY];
    if (rr > 0.0) {
      const double inv = 1.0 / rr;
      sh_unit<L>(r[0] * inv, r[1] * inv, r[2] * inv, Y);
    } else {
#pragma unroll
      for (int q = 0; q < NY; ++q) Y[q] = 0.0;
      Y[0] = 1.0;
    }
    // a continuation gate scales the edge's harmonics, hence its message (the product
    // is linear in them)
    if (a.gate) {
      const double g = a.gate[e];
#pragma unroll
      for (int q = 0; q < NY; ++q) Y[q] *= g;
    }
    P* out = a.sh + (long)slot * a.sh_stride;
#pragma unroll
    for (int q = 0; q < NY; ++q) out[q] = P(Y[q]);
    for (int q = NY; q < a.sh_stride; ++q) out[q] = P(0);
  }
  if (a.deg && lane == 0) a.deg[row] = cnt;
}

template <int L, typename P>
__global__ void __launch_bounds__(kRowThreads) edge_rows_kernel(RowArgs<P> a) {
  edge_rows_body<L, P>(a, __builtin_amdgcn_readfirstlane(int(blockIdx.x) * (kRowThreads / kWave) +
                                                         int(threadIdx.x) / kWave));
}

// The per-row pass and the node order in one launch, for a forward without mask and gate
// (every edge active, so the degrees are the row lengths): workgroup 0 builds the node
// records from row_ptr while the others run the per-row pass, one wave per row.
template <int L, typename P>
__global__ void __launch_bounds__(kScanThreads) rows_order_kernel(RowArgs<P> a, int4* node_info) {
  if (blockIdx.x == 0) {
    degree_order_body(nullptr, a.n_nodes, a.row_ptr, node_info);
    return;
  }
  edge_rows_body<L, P>(a, __builtin_amdgcn_readfirstlane(int(blockIdx.x - 1) * kScanWaves +
                                                         int(threadIdx.x) / kWave));
}

// ---------------------------------------------------------------------------------
// Compaction of the active edges (ids in CSR order) for the exported prepare: the
// receiver of each edge by binary search over row_ptr, its rank among the active
// edges of its row, and the slot act_row_ptr[i] + rank.
// ---------------------------------------------------------------------------------

__global__ void compact_kernel(const int32_t* __restrict__ row_ptr, const uint8_t* __restrict__ mask,
                               const int32_t* __restrict__ act_row_ptr, int n_nodes, int n_edges,
                               int32_t* __restrict__ act_eid) {
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= n_edges) return;
  if (mask && mask[e] == 0) return;
  int lo = 0, hi = n_nodes;  // find i with row_ptr[i] <= e < row_ptr[i+1]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (row_ptr[mid] <= e) lo = mid; else hi = mid;
  }
  const int rbeg = row_ptr[lo];
  int rank = e - rbeg;
  if (mask) {
    rank = 0;
    for (int q = rbeg; q < e; ++q) rank += (mask[q] != 0);
  }
  act_eid[act_row_ptr[lo] + rank] = e;
}

// One wave per row: the w-gradient rows of the row's inactive edges set to zero, the
// lanes over the row's columns (16-byte stores when the rows allow).
__global__ void __launch_bounds__(256) zero_inactive_kernel(const int32_t* __restrict__ row_ptr,
                                                            const uint8_t* __restrict__ mask,
                                                            const float* __restrict__ gate, int n_nodes,
                                                            float* __restrict__ grad_w, int w_stride) {
  const int row = __builtin_amdgcn_readfirstlane(int(blockIdx.x) * 4 + int(threadIdx.x) / kWave);
  if (row >= n_nodes) return;
  const int lane = lane_id();
  const int rb = row_ptr[row], re = row_ptr[row + 1];
  const bool vec = (w_stride % 4) == 0 && (reinterpret_cast<uintptr_t>(grad_w) % 16) == 0;
  for (int b0 = rb; b0 < re; b0 += kWave) {
    const int e = b0 + lane;
    const bool off = e < re && ((mask && mask[e] == 0) || (gate && gate[e] == 0.0f));
    unsigned long long bal = __ballot(off);
    while (bal) {
      const int k = __ffsll((long long)bal) - 1;
      bal &= bal - 1;
      float* r = grad_w + (long)(b0 + k) * w_stride;
      if (vec) {
        for (int c = lane; c < w_stride / 4; c += kWave) reinterpret_cast<float4*>(r)[c] = make_float4(0, 0, 0, 0);
      } else {
        for (int c = lane; c < w_stride; c += kWave) r[c] = 0.0f;
      }
    }
  }
}

}  // namespace

// ---------------------------------------------------------------------------------
// Host launchers
// ---------------------------------------------------------------------------------

NbrGrid make_nbr_grid(int64_t n, const float box[3], float cutoff) {
  NbrGrid g{};
  const double rc = double(cutoff);
  g.rc2 = rc * rc;
  // cells no smaller than the cutoff (with a margin for rounding in the binning),
  // and no more cells than about 2 per atom
  const double cap = std::max(1.0, std::cbrt(2.0 * double(std::max<int64_t>(n, 1))) + 1.0);
  for (int k = 0; k < 3; ++k) {
    g.box[k] = double(box[k]);
    int nc = int(std::floor(g.box[k] / (rc * (1.0 + 1e-6))));
    nc = std::max(1, std::min(nc, int(cap)));
    g.nc[k] = nc;
  }
  return g;
}

static size_t align256(size_t b) { return (b + 255) & ~size_t(255); }

size_t nbr_workspace_bytes(int64_t n, const NbrGrid& g) {
  const size_t nc = size_t(g.n_cells());
  return align256(nc * 4) + align256((nc + 1) * 4) + 3 * align256(size_t(n) * 4 + 4) + 256;
}

NbrWorkspace carve_nbr_workspace(void* ws, int64_t n, const NbrGrid& g) {
  char* p = static_cast<char*>(ws);
  const size_t nc = size_t(g.n_cells());
  NbrWorkspace w{};
  w.cell_count = reinterpret_cast<int32_t*>(p);
  p += align256(nc * 4);
  w.cell_start = reinterpret_cast<int32_t*>(p);
  p += align256((nc + 1) * 4);
  w.atom_cell = reinterpret_cast<int32_t*>(p);
  p += align256(size_t(n) * 4 + 4);
  w.cell_atoms = reinterpret_cast<int32_t*>(p);
  p += align256(size_t(n) * 4 + 4);
  w.row_count = reinterpret_cast<int32_t*>(p);
  p += align256(size_t(n) * 4 + 4);
  w.stats = reinterpret_cast<int32_t*>(p);
  return w;
}

static GridArgs to_args(const NbrGrid& g) {
  GridArgs a{};
  for (int k = 0; k < 3; ++k) {
    a.nc[k] = g.nc[k];
    a.box[k] = g.box[k];
  }
  a.rc2 = g.rc2;
  return a;
}

hipError_t launch_nbr_count(const float* pos, int n, const NbrGrid& g, const NbrWorkspace& w,
                            int32_t* row_ptr, hipStream_t s) {
  const GridArgs a = to_args(g);
  const int nc = g.n_cells();
  const int tb = 256;
  // cell_count doubles as the fill cursor: clear, count, scan, clear, bin
  fill_i32_kernel<<<ceil_div(nc, tb), tb, 0, s>>>(w.cell_count, nc, 0);
  if (n > 0) nbr_assign_kernel<<<ceil_div(n, tb), tb, 0, s>>>(pos, n, a, w.atom_cell, w.cell_count);
  scan_exclusive_kernel<<<1, kScanThreads, 0, s>>>(w.cell_count, w.cell_start, nc, nullptr);
  fill_i32_kernel<<<ceil_div(nc, tb), tb, 0, s>>>(w.cell_count, nc, 0);
  if (n > 0) {
    nbr_bin_kernel<<<ceil_div(n, tb), tb, 0, s>>>(n, w.atom_cell, w.cell_start, w.cell_count, w.cell_atoms);
    nbr_count_wave_kernel<<<ceil_div(n, kNbrWaves), kNbrWaves * kWave, 0, s>>>(pos, n, a, w.atom_cell, w.cell_start,
                                                                              w.cell_atoms, w.row_count);
  }
  scan_exclusive_kernel<<<1, kScanThreads, 0, s>>>(w.row_count, row_ptr, n, w.stats);
  return hipGetLastError();
}

hipError_t launch_nbr_fill(const float* pos, int n, const NbrGrid& g, const NbrWorkspace& w,
                           const int32_t* row_ptr, int32_t* col, int8_t* shift, int max_degree, hipStream_t s) {
  if (n == 0) return hipSuccess;
  const GridArgs a = to_args(g);
  nbr_fill_wave_kernel<<<ceil_div(n, kNbrWaves), kNbrWaves * kWave, 0, s>>>(pos, n, a, w.atom_cell, w.cell_start,
                                                                           w.cell_atoms, row_ptr, col, shift);
  if (max_degree > kNbrRowCap) {   // rows too long for the wave's LDS list: one thread each
    const int tb = 256;
    nbr_fill_kernel<<<ceil_div(n, tb), tb, 0, s>>>(pos, n, a, w.atom_cell, w.cell_start, w.cell_atoms, row_ptr,
                                                   col, shift);
  }
  return hipGetLastError();
}

template <typename P>
static RowArgs<P> row_args(const RowPass& p, const P* pos, const P* gate, P* sh, int l_sh_max) {
  RowArgs<P> a{};
  a.pos = pos;
  a.row_ptr = p.row_ptr;
  a.col = p.col;
  a.shift = p.shift;
  a.mask = p.mask;
  a.gate = gate;
  a.deg = p.deg;
  a.act_e = p.act_e;
  a.act_j = p.act_j;
  a.sh = sh;
  a.n_nodes = p.n_nodes;
  a.has_cell = p.has_cell;
  a.sh_stride = p.sh_stride > 0 ? p.sh_stride : (l_sh_max + 1) * (l_sh_max + 1);
  for (int k = 0; k < 9; ++k) a.cell[k] = p.cell[k];
  return a;
}

hipError_t launch_rows(const RowPass& p, int l_sh_max, hipStream_t s) {
  if (p.n_nodes == 0) return hipSuccess;
  if (!p.row_ptr) return hipErrorInvalidValue;
  const bool f64 = p.pos64 || p.gate64 || p.sh64;
  if (f64 && (p.pos || p.gate || p.sh)) return hipErrorInvalidValue;   // one element type per pass
  const bool has_sh = p.sh || p.sh64;
  if ((has_sh || p.act_j) && p.n_edges > 0 && !p.col) return hipErrorInvalidValue;
  if (has_sh && p.n_edges > 0 && !(p.pos || p.pos64)) return hipErrorInvalidValue;
  const int nb = ceil_div(p.n_nodes, kRowThreads / kWave);
  if (f64) {
    const RowArgs<double> a = row_args<double>(p, p.pos64, p.gate64, p.sh64, l_sh_max);
    switch (l_sh_max) {
      case 0: edge_rows_kernel<0, double><<<nb, kRowThreads, 0, s>>>(a); break;
      case 1: edge_rows_kernel<1, double><<<nb, kRowThreads, 0, s>>>(a); break;
      case 2: edge_rows_kernel<2, double><<<nb, kRowThreads, 0, s>>>(a); break;
      case 3: edge_rows_kernel<3, double><<<nb, kRowThreads, 0, s>>>(a); break;
      case 4: edge_rows_kernel<4, double><<<nb, kRowThreads, 0, s>>>(a); break;
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  const RowArgs<float> a = row_args<float>(p, p.pos, p.gate, p.sh, l_sh_max);
  switch (l_sh_max) {
    case 0: edge_rows_kernel<0, float><<<nb, kRowThreads, 0, s>>>(a); break;
    case 1: edge_rows_kernel<1, float><<<nb, kRowThreads, 0, s>>>(a); break;
    case 2: edge_rows_kernel<2, float><<<nb, kRowThreads, 0, s>>>(a); break;
    case 3: edge_rows_kernel<3, float><<<nb, kRowThreads, 0, s>>>(a); break;
    case 4: edge_rows_kernel<4, float><<<nb, kRowThreads, 0, s>>>(a); break;
    case 5: edge_rows_kernel<5, float><<<nb, kRowThreads, 0, s>>>(a); break;
    case 6: edge_rows_kernel<6, float><<<nb, kRowThreads, 0, s>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_rows_order(const RowPass& p, int l_sh_max, int4* node_info, hipStream_t s) {
  if (p.n_nodes == 0) return hipSuccess;
  if (!p.row_ptr || p.mask || p.gate || p.gate64 || !node_info) return hipErrorInvalidValue;
  const bool f64 = p.pos64 || p.sh64;
  if (f64 && (p.pos || p.sh)) return hipErrorInvalidValue;
  const bool has_sh = p.sh || p.sh64;
  if ((has_sh || p.act_j) && p.n_edges > 0 && !p.col) return hipErrorInvalidValue;
  if (has_sh && p.n_edges > 0 && !(p.pos || p.pos64)) return hipErrorInvalidValue;
  const int nb = 1 + ceil_div(p.n_nodes, kScanWaves);
  if (f64) {
    const RowArgs<double> a = row_args<double>(p, p.pos64, nullptr, p.sh64, l_sh_max);
    switch (l_sh_max) {
      case 0: rows_order_kernel<0, double><<<nb, kScanThreads, 0, s>>>(a, node_info); break;
      case 1: rows_order_kernel<1, double><<<nb, kScanThreads, 0, s>>>(a, node_info); break;
      case 2: rows_order_kernel<2, double><<<nb, kScanThreads, 0, s>>>(a, node_info); break;
      case 3: rows_order_kernel<3, double><<<nb, kScanThreads, 0, s>>>(a, node_info); break;
      case 4: rows_order_kernel<4, double><<<nb, kScanThreads, 0, s>>>(a, node_info); break;
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  const RowArgs<float> a = row_args<float>(p, p.pos, nullptr, p.sh, l_sh_max);
  switch (l_sh_max) {
    case 0: rows_order_kernel<0, float><<<nb, kScanThreads, 0, s>>>(a, node_info); break;
    case 1: rows_order_kernel<1, float><<<nb, kScanThreads, 0, s>>>(a, node_info); break;
    case 2: rows_order_kernel<2, float><<<nb, kScanThreads, 0, s>>>(a, node_info); break;
    case 3: rows_order_kernel<3, float><<<nb, kScanThreads, 0, s>>>(a, node_info); break;
    case 4: rows_order_kernel<4, float><<<nb, kScanThreads, 0, s>>>(a, node_info); break;
    case 5: rows_order_kernel<5, float><<<nb, kScanThreads, 0, s>>>(a, node_info); break;
    case 6: rows_order_kernel<6, float><<<nb, kScanThreads, 0, s>>>(a, node_info); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_order(const int32_t* deg, int n, int32_t* act_row_ptr, int32_t* order, int32_t* tmp_a,
                        int32_t* tmp_b, hipStream_t s) {
  prep_scan_order_kernel<<<1, kScanThreads, 0, s>>>(deg, n, act_row_ptr, order, tmp_a, tmp_b);
  return hipGetLastError();
}

hipError_t launch_degree_order(const int32_t* deg, int n, const int32_t* row_ptr, int4* node_info, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  degree_order_kernel<<<1, kScanThreads, 0, s>>>(deg, n, row_ptr, node_info);
  return hipGetLastError();
}

hipError_t launch_zero_inactive(const int32_t* row_ptr, const uint8_t* mask, const float* gate, int n_nodes,
                                float* grad_w, int w_stride, hipStream_t s) {
  if (n_nodes == 0 || !grad_w || (!mask && !gate)) return hipSuccess;
  zero_inactive_kernel<<<ceil_div(n_nodes, 4), 256, 0, s>>>(row_ptr, mask, gate, n_nodes, grad_w, w_stride);
  return hipGetLastError();
}

hipError_t launch_compact(const int32_t* row_ptr, const uint8_t* mask, const int32_t* act_row_ptr, int n_nodes,
                          int n_edges, int32_t* act_eid, hipStream_t s) {
  if (n_edges == 0 || n_nodes == 0) return hipSuccess;
  const int tb = 256;
  compact_kernel<<<ceil_div(n_edges, tb), tb, 0, s>>>(row_ptr, mask, act_row_ptr, n_nodes, n_edges, act_eid);
  return hipGetLastError();
}

hipError_t launch_conv(const ConvArgsT<float>& args, int cls, hipStream_t s, hipEvent_t b, hipEvent_t e) {
  switch (cls) {
    case 0: return launch_conv_class<0, float>(args, s, b, e);
    case 1: return launch_conv_class<1, float>(args, s, b, e);
    case 2: return launch_conv_class<2, float>(args, s, b, e);
    case 3: return launch_conv_class<3, float>(args, s, b, e);
    case 4: return launch_conv_class<4, float>(args, s, b, e);
    case 5: return launch_conv_class<5, float>(args, s, b, e);
    case 6: return launch_conv_class<6, float>(args, s, b, e);
    case 7: return launch_conv_class<7, float>(args, s, b, e);
    case 8: return launch_conv_class<8, float>(args, s, b, e);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_conv(const ConvArgsT<double>& args, int cls, hipStream_t s, hipEvent_t b, hipEvent_t e) {
  switch (cls) {
    case 0: return launch_conv_class<0, double>(args, s, b, e);
    case 1: return launch_conv_class<1, double>(args, s, b, e);
    case 2: return launch_conv_class<2, double>(args, s, b, e);
    case 3: return launch_conv_class<3, double>(args, s, b, e);
    case 4: return launch_conv_class<4, double>(args, s, b, e);
    case 5: return launch_conv_class<5, double>(args, s, b, e);
    case 6: return launch_conv_class<6, double>(args, s, b, e);
    default: return hipErrorInvalidValue;
  }
}
static_assert(kNumClassesF64 == 7, "launch_conv covers every fp64 kernel class");

static_assert(kNumClasses == 9, "launch_conv covers every kernel class");

hipError_t launch_conv_bwd(const ConvArgsT<float>& args, int cls, hipStream_t s) {
  switch (cls) {
    case 0: return launch_conv_bwd_class<0>(args, s);
    case 1: return launch_conv_bwd_class<1>(args, s);
    case 2: return launch_conv_bwd_class<2>(args, s);
    case 3: return launch_conv_bwd_class<3>(args, s);
    case 4: return launch_conv_bwd_class<4>(args, s);
    case 5: return launch_conv_bwd_class<5>(args, s);
    case 6: return launch_conv_bwd_class<6>(args, s);
    default: return hipErrorInvalidValue;
  }
}
static_assert(kNumClassesBwd == 7, "launch_conv_bwd covers every class with l <= kBwdLmax");

}  // namespace cgtp
