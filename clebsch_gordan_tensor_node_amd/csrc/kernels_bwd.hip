// Backward of the CGTP convolution (fp32, plans whose largest l is kBwdLmax = 4 or less):
// the passes after the edge pass (which is the fused conv kernel in its backward mode,
// conv_kernel.hpp).
//
// LunaTP's abstract puts the derivatives that forces need within the scope of its
// kernels.  The forward is trilinear in (x_j, w_e, Y(r_e)), so with dL/d out = g:
//   dL/dw[e, c]      = sum C x_j Y g_i             (one value per edge and channel)
//   dL/dx[j, u, m1] += w sum_{m2,m3} C Y g_i        (summed over the sender's edges)
//   dL/dY[e, m2]    += w sum_{m1,m3} C x_j g_i      (summed over paths and channels)
//   dL/dr_e          = gate_e sum_m2 dL/dY[e, m2] dY_m2/dr,   dL/dpos = +dL/dr at the
//                      sender, -dL/dr at the receiver.
// The harmonics used are the forward's stored ones (already scaled by the gate), so the
// w and x gradients carry the gate; dL/dY is taken with respect to the stored values,
// hence the gate factor in dL/dr.
//
// gfx950 mapping: every pass is deterministic (no floating-point atomics; every sum runs
// in a fixed order):
//   * the edge pass (conv_kernel_bwd<C>) runs on the forward's workgroups,
//     producer wave and schedule, each consumer holding its receiver's g; per active
//     slot it writes the edge's w-gradient, each job's dL/dY of the slot and each job
//     group's x-gradient of the edge into one row of partials (zero_inactive_kernel
//     clears the w-gradient rows of inactive edges);
//   * the active slots are regrouped by sender (counts, scan, placement, per-sender sort
//     by slot); bwd_gather_x_kernel runs one workgroup per sender and column block,
//     dL/dx[j] being the sum of its slots' x-gradient blocks (rows of partials read in
//     slot order), and bwd_force_kernel one per sender: each slot's dL/dY (its jobs'
//     partials in job order) goes through dY/dr, evaluated by running the harmonics'
//     recurrence on dual numbers (exact derivatives of the same polynomials);
//   * bwd_pos_kernel sums each node's +/- contributions in slot order.
#include <hip/hip_runtime.h>

#include "launch.hpp"
#include "sh_eval.hpp"

namespace cgtp {

namespace {

// ---------------------------------------------------------------------------------
// active slots grouped by sender
// ---------------------------------------------------------------------------------

__global__ void fill_zero_kernel(int32_t* p, int n) {
  const int k = int(blockIdx.x * blockDim.x + threadIdx.x);
  if (k < n) p[k] = 0;
}

// one wave per row: count (place == 0) or place (place == 1) the row's active slots
__global__ void __launch_bounds__(256) bwd_t_count_kernel(BwdArgs a, int32_t* cnt, int32_t* t_slot, int32_t* t_recv,
                                                          int place) {
  const int i = int(blockIdx.x) * (256 / kWave) + int(threadIdx.x) / kWave;
  if (i >= a.n_nodes) return;
  const int lane = int(threadIdx.x) & (kWave - 1);
  const int rb = a.row_ptr[i], d = a.deg[i];
  for (int q = lane; q < d; q += kWave) {
    const int s = rb + q;
    const int j = a.act_j[s];
    const int k = atomicAdd(&cnt[j], 1);
    if (place) {
      t_slot[a.t_row_ptr[j] + k] = s;
      t_recv[a.t_row_ptr[j] + k] = i;
    }
  }
}

// one workgroup: out[k] = sum_{q < k} in[q], k <= n; in is reset to zero
__global__ void __launch_bounds__(1024) bwd_scan_kernel(int32_t* in, int32_t* out, int n) {
  __shared__ int wsum[1024 / kWave + 1];
  const int lane = int(threadIdx.x) & (kWave - 1), wave = int(threadIdx.x) / kWave;
  int carry = 0;
  for (int base = 0; base < n; base += 1024) {
    const int idx = base + int(threadIdx.x);
    const int v = idx < n ? in[idx] : 0;
    int inc = v;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
      const int t = __shfl_up(inc, d, kWave);
      if (lane >= d) inc += t;
    }
    if (lane == kWave - 1) wsum[wave] = inc;
    __syncthreads();
    if (threadIdx.x == 0) {
      int run = 0;
      for (int k = 0; k < 1024 / kWave; ++k) {
        const int t = wsum[k];
        wsum[k] = run;
        run += t;
      }
      wsum[1024 / kWave] = run;
    }
    __syncthreads();
    if (idx < n) {
      out[idx] = carry + wsum[wave] + inc - v;
      in[idx] = 0;   // the counts become the placement cursors
    }
    carry += wsum[1024 / kWave];
    __syncthreads();
  }
  if (threadIdx.x == 0) out[n] = carry;
}

// one wave per sender: its entries in slot order.  Slots are distinct, so an entry's
// position is the number of entries with a smaller slot (counted over an LDS copy of
// the row); rows longer than the LDS copy are sorted by insertion by one lane.
constexpr int kSortCap = 512;
__global__ void __launch_bounds__(kWave) bwd_t_sort_kernel(const int32_t* t_row_ptr, int32_t* t_slot,
                                                          int32_t* t_recv, int n) {
  __shared__ int ss[kSortCap], rr[kSortCap];
  const int j = int(blockIdx.x);
  const int lane = int(threadIdx.x);
  const int b = t_row_ptr[j], e = t_row_ptr[j + 1], len = e - b;
  if (len <= 1) return;
  if (len <= kSortCap) {
    for (int k = lane; k < len; k += kWave) {
      ss[k] = t_slot[b + k];
      rr[k] = t_recv[b + k];
    }
    __syncthreads();
    for (int k = lane; k < len; k += kWave) {
      const int v = ss[k];
      int rank = 0;
      for (int m = 0; m < len; ++m) rank += ss[m] < v ? 1 : 0;
      t_slot[b + rank] = v;
      t_recv[b + rank] = rr[k];
    }
    return;
  }
  if (lane != 0) return;
  for (int k = b + 1; k < e; ++k) {
    const int s = t_slot[k], r = t_recv[k];
    int m = k - 1;
    while (m >= b && t_slot[m] > s) {
      t_slot[m + 1] = t_slot[m];
      t_recv[m + 1] = t_recv[m];
      --m;
    }
    t_slot[m + 1] = s;
    t_recv[m + 1] = r;
  }
}

// ---------------------------------------------------------------------------------
// dL/dr per active slot, and the position gradient
// ---------------------------------------------------------------------------------

// dL/dr of active slot s (edge j -> i) from its dL/dY, g[0 .. (L + 1)^2)
template <int L>
__device__ __forceinline__ void slot_grad_r(const BwdArgs& a, int i, int j, int s, const float* g) {
  constexpr int NY = (L + 1) * (L + 1);
  const int e = a.act_e[s];
  double r[3];
#pragma unroll
  for (int k = 0; k < 3; ++k) r[k] = double(a.pos[3 * j + k]) - double(a.pos[3 * i + k]);
  if (a.has_cell && a.shift) {
    const double s0 = a.shift[3 * e + 0], s1 = a.shift[3 * e + 1], s2 = a.shift[3 * e + 2];
#pragma unroll
    for (int k = 0; k < 3; ++k) r[k] = r[k] + s0 * a.cell[k] + s1 * a.cell[3 + k] + s2 * a.cell[6 + k];
  }
  const double rr = sqrt(r[0] * r[0] + r[1] * r[1] + r[2] * r[2]);
  double gr[3] = {0.0, 0.0, 0.0};
  if (rr > 0.0) {   // a zero-length edge has constant harmonics: no gradient
    const double inv = 1.0 / rr;
    const double rh[3] = {r[0] * inv, r[1] * inv, r[2] * inv};
    // the unit vector's components with d rhat_a / d r_k = (delta_ak - rhat_a rhat_k) / |r|
    Dual3 u[3];
#pragma unroll
    for (int c = 0; c < 3; ++c) {
      u[c] = Dual3(rh[c]);
#pragma unroll
      for (int k = 0; k < 3; ++k) u[c].d[k] = ((c == k ? 1.0 : 0.0) - rh[c] * rh[k]) * inv;
    }
    Dual3 Y[NY];
    sh_unit<L, Dual3>(u[0], u[1], u[2], Y);
    const double gt = a.gate ? double(a.gate[e]) : 1.0;
#pragma unroll
    for (int q = 1; q < NY; ++q)
#pragma unroll
      for (int k = 0; k < 3; ++k) gr[k] += double(g[q]) * Y[q].d[k];
#pragma unroll
    for (int k = 0; k < 3; ++k) gr[k] *= gt;
  }
#pragma unroll
  for (int k = 0; k < 3; ++k) a.grad_r[(long)s * 3 + k] = float(gr[k]);
}

// One workgroup per (sender j, block of kGatherThreads columns of x).  dL/dx[j, c] is
// the sum over j's active slots, in slot order, of the entries of column c in the slot's
// row of partials (the x-gradient blocks of the groups that read c, in group order).
// The sender's slots are staged in LDS by chunks and each thread keeps its column's
// entry offsets in registers, so that the loads of several slots are in flight at once.
constexpr int kGatherThreads = 256;
constexpr int kMaxCover = 4;   // x-gradient blocks per column held in registers
// slots whose loads are issued together: a sender's whole slot list at the common
// degrees (one memory latency per workgroup instead of one per four slots), in as
// many registers as NQ entries allow
template <int NQ>
constexpr int gather_batch() {
  return NQ <= 2 ? 16 : 8;
}

// acc + the column's entries of the n staged slots, NQ entries per slot loaded for every
// lane (lanes with fewer, nq, repeat a valid offset and drop the extra values): all
// loads of a batch are unconditional, so they are in flight together
template <int NQ>
__device__ __forceinline__ float gather_cols(const BwdArgs& a, const int* ss, int n, const int* off, int nq,
                                             float acc) {
  constexpr int kGatherBatch = gather_batch<NQ>();
  for (int t = 0; t < n; t += kGatherBatch) {
    float v[kGatherBatch][NQ];
#pragma unroll
    for (int u = 0; u < kGatherBatch; ++u) {
      const float* row = a.part + (long)ss[t + u < n ? t + u : t] * a.part_stride;
#pragma unroll
      for (int q = 0; q < NQ; ++q) v[u][q] = row[off[q]];
    }
#pragma unroll
    for (int u = 0; u < kGatherBatch; ++u)
#pragma unroll
      for (int q = 0; q < NQ; ++q) acc = (t + u < n && q < nq) ? acc + v[u][q] : acc;
  }
  return acc;
}

__global__ void __launch_bounds__(kGatherThreads) bwd_gather_x_kernel(BwdArgs a) {
  __shared__ int ss[kGatherThreads];
  const int j = int(blockIdx.x);
  const int tid = int(threadIdx.x);
  const int tb = a.t_row_ptr[j], te = a.t_row_ptr[j + 1];
  const int c = int(blockIdx.y) * kGatherThreads + tid;
  const bool col_ok = c < a.f_in;
  int q0 = 0, nq = 0;
  if (col_ok) {
    q0 = a.xcol_ptr[c];
    nq = a.xcol_ptr[c + 1] - q0;
  }
  int off[kMaxCover];
#pragma unroll
  for (int q = 0; q < kMaxCover; ++q) off[q] = nq > 0 ? a.xcol_off[q0 + (q < nq ? q : 0)] : 0;
  // the wave's largest cover selects the unrolled form (uniform)
  int nqw = nq;
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) nqw = max(nqw, __shfl_xor(nqw, o, kWave));
  nqw = __builtin_amdgcn_readfirstlane(nqw);
  float acc = 0.0f;
  for (int t0 = tb; t0 < te; t0 += kGatherThreads) {
    const int n = min(kGatherThreads, te - t0);
    __syncthreads();   // the previous chunk is consumed
    if (tid < n) ss[tid] = a.t_slot[t0 + tid];
    __syncthreads();
    switch (nqw) {
      case 0: break;
      case 1: acc = gather_cols<1>(a, ss, n, off, nq, acc); break;
      case 2: acc = gather_cols<2>(a, ss, n, off, nq, acc); break;
      case 3: acc = gather_cols<3>(a, ss, n, off, nq, acc); break;
      case 4: acc = gather_cols<4>(a, ss, n, off, nq, acc); break;
      default:
        if (col_ok)
          for (int t = 0; t < n; ++t) {
            const float* row = a.part + (long)ss[t] * a.part_stride;
            for (int q = 0; q < nq; ++q) acc += row[a.xcol_off[q0 + q]];
          }
        break;
    }
  }
  if (col_ok) a.grad_x[(long)j * a.f_in + c] = acc;
}

// One workgroup per sender j: dL/dr of its active slots.  Per chunk of kForceSlots slots,
// their dL/dY (each harmonic component's job partials, in job order, read from the
// slots' rows of partials) is summed into LDS, then one thread per slot evaluates dL/dr.
constexpr int kForceThreads = 256;
constexpr int kForceSlots = 16;
constexpr int kMaxGyLen = 1024;   // dL/dY entries of a row whose offsets are staged in LDS

template <int L>
__global__ void __launch_bounds__(kForceThreads) bwd_force_kernel(BwdArgs a) {
  const int j = int(blockIdx.x);
  const int tid = int(threadIdx.x);
  const int tb = a.t_row_ptr[j], te = a.t_row_ptr[j + 1];
  if constexpr (L == 0) {   // l = 0 harmonics only: constant, no gradient
    for (int t = tb + tid; t < te; t += kForceThreads)
#pragma unroll
      for (int k = 0; k < 3; ++k) a.grad_r[(long)a.t_slot[t] * 3 + k] = 0.0f;
  } else {
    constexpr int NY = (L + 1) * (L + 1);
    __shared__ float gys[kForceSlots][NY];
    __shared__ int yoff[kMaxGyLen];
    __shared__ int yptr[NY + 1];
    if (tb == te) return;
    const int ny_len = a.ycol_ptr[NY];
    const bool staged = ny_len <= kMaxGyLen;
    if (tid <= NY) yptr[tid] = a.ycol_ptr[tid];
    if (staged)
      for (int q = tid; q < ny_len; q += kForceThreads) yoff[q] = a.ycol_off[q];
    __syncthreads();
    for (int t0 = tb; t0 < te; t0 += kForceSlots) {
      const int n = min(kForceSlots, te - t0);
      for (int idx = tid; idx < n * NY; idx += kForceThreads) {
        const int r = idx / NY, m = idx - r * NY;
        const float* row = a.part + (long)a.t_slot[t0 + r] * a.part_stride;
        float v = 0.0f;
        if (staged) {
#pragma unroll 4
          for (int q = yptr[m]; q < yptr[m + 1]; ++q) v += row[yoff[q]];
        } else {
          for (int q = yptr[m]; q < yptr[m + 1]; ++q) v += row[a.ycol_off[q]];
        }
        gys[r][m] = v;
      }
      __syncthreads();
      if (tid < n) slot_grad_r<L>(a, a.t_recv[t0 + tid], j, a.t_slot[t0 + tid], gys[tid]);
      __syncthreads();
    }
  }
}

__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int d = kWave / 2; d > 0; d >>= 1) v += __shfl_xor(v, d, kWave);
  return v;
}

// one wave per node: + its edges as sender, - its edges as receiver; lanes take the
// entries in slot order and a fixed butterfly sums them (fp64)
__global__ void __launch_bounds__(256) bwd_pos_kernel(BwdArgs a) {
  const int n = int(blockIdx.x) * (256 / kWave) + int(threadIdx.x) / kWave;
  if (n >= a.n_nodes) return;
  const int lane = int(threadIdx.x) & (kWave - 1);
  double g[3] = {0.0, 0.0, 0.0};
  for (int k = a.t_row_ptr[n] + lane; k < a.t_row_ptr[n + 1]; k += kWave) {
    const int s = a.t_slot[k];
#pragma unroll
    for (int c = 0; c < 3; ++c) g[c] += double(a.grad_r[(long)s * 3 + c]);
  }
  const int rb = a.row_ptr[n], d = a.deg[n];
  for (int q = lane; q < d; q += kWave)
#pragma unroll
    for (int c = 0; c < 3; ++c) g[c] -= double(a.grad_r[(long)(rb + q) * 3 + c]);
#pragma unroll
  for (int c = 0; c < 3; ++c) {
    const double v = wave_sum_f64(g[c]);
    if (lane == 0) a.grad_pos[3 * n + c] = float(v);
  }
}


}  // namespace

hipError_t launch_bwd_transpose(const BwdArgs& a, int32_t* t_cnt, int32_t* t_row_ptr, int32_t* t_slot,
                                int32_t* t_recv, hipStream_t s) {
  const int n = a.n_nodes;
  if (n == 0) return hipSuccess;
  const int zb = ceil_div(n, 256), rb = ceil_div(n, 256 / kWave);
  fill_zero_kernel<<<zb, 256, 0, s>>>(t_cnt, n);
  bwd_t_count_kernel<<<rb, 256, 0, s>>>(a, t_cnt, nullptr, nullptr, 0);
  bwd_scan_kernel<<<1, 1024, 0, s>>>(t_cnt, t_row_ptr, n);
  BwdArgs b = a;
  b.t_row_ptr = t_row_ptr;
  bwd_t_count_kernel<<<rb, 256, 0, s>>>(b, t_cnt, t_slot, t_recv, 1);
  bwd_t_sort_kernel<<<n, kWave, 0, s>>>(t_row_ptr, t_slot, t_recv, n);
  return hipGetLastError();
}

hipError_t launch_bwd_gather_x(const BwdArgs& a, hipStream_t s) {
  if (a.n_nodes == 0 || a.f_in == 0) return hipSuccess;
  bwd_gather_x_kernel<<<dim3(a.n_nodes, ceil_div(a.f_in, kGatherThreads)), kGatherThreads, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_bwd_force(const BwdArgs& a, hipStream_t s) {
  const int n = a.n_nodes;
  if (n == 0) return hipSuccess;
  switch (a.l_sh_max) {
    case 0: bwd_force_kernel<0><<<n, kForceThreads, 0, s>>>(a); break;
    case 1: bwd_force_kernel<1><<<n, kForceThreads, 0, s>>>(a); break;
    case 2: bwd_force_kernel<2><<<n, kForceThreads, 0, s>>>(a); break;
    case 3: bwd_force_kernel<3><<<n, kForceThreads, 0, s>>>(a); break;
    case 4: bwd_force_kernel<4><<<n, kForceThreads, 0, s>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_bwd_pos(const BwdArgs& a, hipStream_t s) {
  const int n = a.n_nodes;
  if (n == 0) return hipSuccess;
  bwd_pos_kernel<<<ceil_div(n, 256 / kWave), 256, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace cgtp
