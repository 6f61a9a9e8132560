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
// in a fixed order), and each path's coupling is a compile-time specialisation (the real
// CG coefficients and their sparsity are constants):
//   * the edge pass (conv_kernel<C, float, true>): the forward's workgroups, producer wave
//     and schedule, with consumers that write each active edge's w-gradient for their
//     channels and the job's dL/dY of the edge's slot, reduced over the receiver's lanes
//     by a fixed butterfly (zero_inactive_kernel clears the rows of inactive edges);
//   * the active slots are regrouped by sender (counts, scan, placement, per-sender sort
//     by slot), so that the x-gradient is a gather: on large graphs bwd_x_kernel runs
//     one wave per (sender, input irrep) and accumulates all of the irrep's paths in
//     registers; on graphs too small to fill the chip that way bwd_xp_kernel runs one
//     wave per (sender, path) and writes that path's partial, and bwd_x_sum_kernel adds
//     each input irrep's partials in path order (either way a path of 32 channels or
//     fewer puts several of the sender's edges side by side in one wave and adds their
//     sums by a fixed butterfly);
//   * bwd_force_kernel evaluates dY/dr by running the harmonics' recurrence on dual
//     numbers (exact derivatives of the same polynomials), and bwd_pos_kernel sums each
//     node's +/- contributions in slot order.
#include <hip/hip_runtime.h>

#include "launch.hpp"
#include "sh_eval.hpp"
#include "variants.hpp"

namespace cgtp {

namespace {


template <int N>
struct IC {
  static constexpr int value = N;
};

template <int B, int E, typename F>
__device__ __forceinline__ void sfor(F&& f) {
  if constexpr (B < E) {
    f(IC<B>{});
    sfor<B + 1, E>(f);
  }
}

template <int L1, int L2, int L3>
inline constexpr RealCG<L1, L2, L3> kCGb{};

// Runs f(IC<v>) for the variant v of a path: the scalar (K = 1) form of a triple whose
// largest l is at most LMAX (the kernels here specialise on (l1, l2, l3) only).  Each
// kernel below is built twice, for l <= 3 and for l = 4 paths, so that the registers
// the l = 4 code needs do not lower the occupancy of the l <= 3 code.
constexpr int kBwdLowLmax = 3;
static_assert(kBwdLmax == kBwdLowLmax + 1, "one high instantiation covers l = kBwdLmax");

template <int LO, int HI, int LMAX, typename F>
__device__ __forceinline__ void by_variant(int v, F&& f) {
  if constexpr (HI - LO == 1) {
    if constexpr (variant_lmax(LO) <= LMAX && variant_desc(LO).k == 1) f(IC<LO>{});
  } else {
    constexpr int MID = (LO + HI) / 2;
    if (v < MID)
      by_variant<LO, MID, LMAX>(v, f);
    else
      by_variant<MID, HI, LMAX>(v, f);
  }
}

__device__ __forceinline__ int path_lmax(const PathDev& P) { return max(P.l1, max(P.l2, P.l3)); }

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int d = kWave / 2; d > 0; d >>= 1) v += __shfl_xor(v, d, kWave);
  return v;
}

__device__ __forceinline__ bool edge_active(const BwdArgs& a, int e) {
  return (!a.mask || a.mask[e] != 0) && (!a.gate || a.gate[e] != 0.0f);
}

// A[m1][m3] = sum_m2 C[m1,m2,m3] Y[m2]
template <int L1, int L2, int L3>
__device__ __forceinline__ void form_a(const float* Y, float (*A)[2 * L3 + 1]) {
  constexpr int N1 = 2 * L1 + 1, N2 = 2 * L2 + 1, N3 = 2 * L3 + 1;
  sfor<0, N1>([&](auto M1) {
    sfor<0, N3>([&](auto M3) {
      float s = 0.0f;
      sfor<0, N2>([&](auto M2) {
        constexpr float c = kCGb<L1, L2, L3>.at(decltype(M1)::value, decltype(M2)::value, decltype(M3)::value);
        if constexpr (c != 0.0f) s = __builtin_fmaf(c, Y[decltype(M2)::value], s);
      });
      A[decltype(M1)::value][decltype(M3)::value] = s;
    });
  });
}


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
// x-gradient
// ---------------------------------------------------------------------------------

// entries k0 .. k0 + cnt - 1 of the sender's list: slot, receiver and edge id of entry
// k0 + lane are held by that lane.  The lanes form nsub sub-groups (sub = this lane's):
// sub-group g takes entries g, g + nsub, ... (uniform trip count, idle at the tail).
template <int L1, int L2, int L3>
__device__ __forceinline__ void bwd_x_path(const BwdArgs& a, const PathDev& P, int cnt, int sub, int nsub,
                                           int my_s, int my_i, int my_e, int u, bool ok, float* acc) {
  constexpr int N1 = 2 * L1 + 1, N2 = 2 * L2 + 1, N3 = 2 * L3 + 1;
  // D-deep pipeline: the harmonics, weight and grad_out rows of the next D entries of
  // this sub-group are in flight (loaded at clamped indices, unconditionally) while one
  // entry is used; D from the registers an entry holds
  struct Entry {
    float Y[N2];
    float w;
    float go[N3];
  };
  constexpr int D = 48 / (N2 + 1 + N3) < 2 ? 2 : (48 / (N2 + 1 + N3) > 4 ? 4 : 48 / (N2 + 1 + N3));
  const int uu = ok ? u : 0;
  auto load = [&](int k, Entry& d) {
    const int s = __shfl(my_s, k, kWave), i = __shfl(my_i, k, kWave), e = __shfl(my_e, k, kWave);
#pragma unroll
    for (int m = 0; m < N2; ++m) d.Y[m] = a.sh[(long)s * a.sh_stride + P.sh_off + m];
    d.w = a.w[(long)e * a.w_stride + P.w_off + uu];
#pragma unroll
    for (int m = 0; m < N3; ++m) d.go[m] = a.grad_out[(long)i * a.f_out + P.out_off + uu * N3 + m];
  };
  const int steps = (cnt + nsub - 1) / nsub;
  Entry ring[D];
#pragma unroll
  for (int r = 0; r < D; ++r) load(min(sub + r * nsub, cnt - 1), ring[r]);
  for (int t0 = 0; t0 < steps; t0 += D) {
#pragma unroll
    for (int r = 0; r < D; ++r) {
      const int t = t0 + r;
      if (t < steps) {   // uniform over the wave
        const int k = t * nsub + sub;
        const Entry cur = ring[r];
        load(min(k + D * nsub, cnt - 1), ring[r]);
        float A[N1][N3];
        form_a<L1, L2, L3>(cur.Y, A);
        if (ok && k < cnt) {
#pragma unroll
          for (int m1 = 0; m1 < N1; ++m1) {
            float v = 0.0f;
#pragma unroll
            for (int m3 = 0; m3 < N3; ++m3) v = __builtin_fmaf(A[m1][m3], cur.go[m3], v);
            acc[m1] = __builtin_fmaf(cur.w, v, acc[m1]);
          }
        }
      }
    }
  }
}

template <int L1, int LMAX>
__device__ __forceinline__ void bwd_x_irrep(const BwdArgs& a, int j, int ir) {
  constexpr int N1 = 2 * L1 + 1;
  const int mul = a.irrep_mul[ir], off = a.irrep_off[ir];
  const int p0 = a.irrep_start[ir], p1 = a.irrep_start[ir + 1];
  // lanes per entry: the next power of two of the multiplicity, at most 64; the
  // 64 / cw sub-groups of a wave walk interleaved entries of the sender's list and their
  // partial sums are added by a fixed butterfly before the store
  int cw = 1;
  while (cw < mul && cw < kWave) cw <<= 1;
  const int lane = int(threadIdx.x), sub = lane / cw, nsub = kWave / cw;
  for (int u0 = 0; u0 < mul; u0 += kWave) {
    const int u = u0 + (lane & (cw - 1));
    const bool ok = u < mul;
    float acc[N1];
#pragma unroll
    for (int m = 0; m < N1; ++m) acc[m] = 0.0f;
    const int tb = a.t_row_ptr[j], te = a.t_row_ptr[j + 1];
    for (int k0 = tb; k0 < te; k0 += kWave) {
      const int cnt = min(kWave, te - k0);
      const int kk = k0 + min(int(threadIdx.x), cnt - 1);
      const int my_s = a.t_slot[kk], my_i = a.t_recv[kk];
      const int my_e = a.act_e[my_s];
      for (int pp = p0; pp < p1; ++pp) {
        const PathDev P = a.paths[a.irrep_paths[pp]];
        by_variant<0, kNumVariants, LMAX>(P.variant, [&](auto V) {
          constexpr VariantDesc d = variant_desc(decltype(V)::value);
          if constexpr (d.l1 == L1) bwd_x_path<L1, d.l2, d.l3>(a, P, cnt, sub, nsub, my_s, my_i, my_e, u, ok, acc);
        });
      }
    }
    for (int d = cw; d < kWave; d <<= 1) {
#pragma unroll
      for (int m = 0; m < N1; ++m) acc[m] += __shfl_xor(acc[m], d, kWave);
    }
    if (ok && sub == 0) {
#pragma unroll
      for (int m = 0; m < N1; ++m) a.grad_x[(long)j * a.f_in + off + u * N1 + m] = acc[m];
    }
  }
}

// One wave per (sender, input irrep), all of the irrep's paths accumulated in registers
// and stored once (no partials).  HIGH: the instantiation for the input irreps with a
// path of l = kBwdLmax.
template <bool HIGH>
__global__ void __launch_bounds__(kWave) bwd_x_kernel(BwdArgs a) {
  const int j = int(blockIdx.x), ir = int(blockIdx.y);
  int lm = 0;
  for (int pp = a.irrep_start[ir]; pp < a.irrep_start[ir + 1]; ++pp) lm = max(lm, path_lmax(a.paths[a.irrep_paths[pp]]));
  if ((lm > kBwdLowLmax) != HIGH) return;
  constexpr int LM = HIGH ? kBwdLmax : kBwdLowLmax;
  switch (a.irrep_l[ir]) {
    case 0: bwd_x_irrep<0, LM>(a, j, ir); break;
    case 1: bwd_x_irrep<1, LM>(a, j, ir); break;
    case 2: bwd_x_irrep<2, LM>(a, j, ir); break;
    case 3: bwd_x_irrep<3, LM>(a, j, ir); break;
    case 4:
      if constexpr (HIGH) bwd_x_irrep<4, LM>(a, j, ir);
      break;
    default: break;
  }
}

// One wave per (sender, path): the path's x-gradient partial of every channel of the
// sender, over its entries in slot order, written to the path's block of the sender's
// row of partials.  A path of 32 channels or fewer runs 64 / 2^ceil(log2 mul) of the
// sender's entries side by side and adds the sub-groups' sums by a fixed butterfly.
template <bool HIGH>
__global__ void __launch_bounds__(kWave) bwd_xp_kernel(BwdArgs a) {
  const int j = int(blockIdx.x);
  const PathDev P = a.paths[blockIdx.y];
  if ((path_lmax(P) > kBwdLowLmax) != HIGH) return;
  int cw = 1;
  while (cw < P.mul && cw < kWave) cw <<= 1;
  const int lane = int(threadIdx.x), sub = lane / cw, nsub = kWave / cw;
  const int tb = a.t_row_ptr[j], te = a.t_row_ptr[j + 1];
  by_variant<0, kNumVariants, HIGH ? kBwdLmax : kBwdLowLmax>(P.variant, [&](auto V) {
    constexpr VariantDesc d = variant_desc(decltype(V)::value);
    constexpr int N1 = 2 * d.l1 + 1;
    for (int u0 = 0; u0 < P.mul; u0 += kWave) {
      const int u = u0 + (lane & (cw - 1));
      const bool ok = u < P.mul;
      float acc[N1];
#pragma unroll
      for (int m = 0; m < N1; ++m) acc[m] = 0.0f;
      for (int k0 = tb; k0 < te; k0 += kWave) {
        const int cnt = min(kWave, te - k0);
        const int kk = k0 + min(lane, cnt - 1);
        const int my_s = a.t_slot[kk], my_i = a.t_recv[kk];
        const int my_e = a.act_e[my_s];
        bwd_x_path<d.l1, d.l2, d.l3>(a, P, cnt, sub, nsub, my_s, my_i, my_e, u, ok, acc);
      }
      for (int dd = cw; dd < kWave; dd <<= 1) {
#pragma unroll
        for (int m = 0; m < N1; ++m) acc[m] += __shfl_xor(acc[m], dd, kWave);
      }
      if (ok && sub == 0) {
#pragma unroll
        for (int m = 0; m < N1; ++m) a.xp[(long)j * a.xp_stride + P.xp_off + u * N1 + m] = acc[m];
      }
    }
  });
}

// x-gradient: per node and input-feature column, the partials of the column's irrep's
// paths added in path order (an irrep without paths gets 0)
__global__ void __launch_bounds__(256) bwd_x_sum_kernel(BwdArgs a) {
  const long idx = long(blockIdx.x) * 256 + threadIdx.x;
  if (idx >= long(a.n_nodes) * a.f_in) return;
  const int j = int(idx / a.f_in), c = int(idx - long(j) * a.f_in);
  int ir = 0;
  while (ir + 1 < a.n_irreps && a.irrep_off[ir + 1] <= c) ++ir;
  const int r = c - a.irrep_off[ir];
  float v = 0.0f;
  for (int pp = a.irrep_start[ir]; pp < a.irrep_start[ir + 1]; ++pp)
    v += a.xp[(long)j * a.xp_stride + a.paths[a.irrep_paths[pp]].xp_off + r];
  a.grad_x[idx] = v;
}

// ---------------------------------------------------------------------------------
// dL/dr per active slot, and the position gradient
// ---------------------------------------------------------------------------------

template <int L>
__device__ __forceinline__ void slot_grad_r(const BwdArgs& a, int i, int s) {
  constexpr int NY = (L + 1) * (L + 1);
  // dL/dY of the slot: the jobs' partials (one per path and channel block) in job order
  float g[NY];
#pragma unroll
  for (int k = 0; k < NY; ++k) g[k] = 0.0f;
  for (int q = 0; q < a.n_gy; ++q) {
    const int2 jb = a.gy_list[q];   // {l2, offset in a row of partials}
    sfor<1, L + 1>([&](auto L2c) {
      constexpr int L2 = decltype(L2c)::value;
      if (jb.x == L2) {
#pragma unroll
        for (int m = 0; m < 2 * L2 + 1; ++m) g[L2 * L2 + m] += a.gyp[(long)s * a.gy_stride + jb.y + m];
      }
    });
  }
  const int e = a.act_e[s], j = a.act_j[s];
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

// one wave per row, lanes over its active slots
__global__ void __launch_bounds__(256) bwd_force_kernel(BwdArgs a) {
  const int i = int(blockIdx.x) * (256 / kWave) + int(threadIdx.x) / kWave;
  if (i >= a.n_nodes) return;
  const int lane = int(threadIdx.x) & (kWave - 1);
  const int rb = a.row_ptr[i], d = a.deg[i];
  for (int q = lane; q < d; q += kWave) {
    switch (a.l_sh_max) {
      case 1: slot_grad_r<1>(a, i, rb + q); break;
      case 2: slot_grad_r<2>(a, i, rb + q); break;
      case 3: slot_grad_r<3>(a, i, rb + q); break;
      case 4: slot_grad_r<4>(a, i, rb + q); break;
      default:   // l = 0 harmonics only: constant, no gradient
#pragma unroll
        for (int k = 0; k < 3; ++k) a.grad_r[(long)(rb + q) * 3 + k] = 0.0f;
        break;
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

hipError_t launch_bwd_x(const BwdArgs& a, bool high, hipStream_t s) {
  if (a.n_nodes == 0 || a.n_irreps == 0) return hipSuccess;
  // With enough (sender, irrep) waves to fill the chip (4 per SIMD) each wave takes a
  // whole irrep; otherwise one wave per (sender, path) and a fixed-order sum, which
  // shortens each wave's chain of dependent loads at the price of the partials' traffic.
  constexpr long kFillWaves = 4L * 1024;
  if (long(a.n_nodes) * a.n_irreps >= kFillWaves) {
    bwd_x_kernel<false><<<dim3(a.n_nodes, a.n_irreps), kWave, 0, s>>>(a);
    if (high) bwd_x_kernel<true><<<dim3(a.n_nodes, a.n_irreps), kWave, 0, s>>>(a);
    return hipGetLastError();
  }
  if (a.n_paths > 0) {
    bwd_xp_kernel<false><<<dim3(a.n_nodes, a.n_paths), kWave, 0, s>>>(a);
    if (high) bwd_xp_kernel<true><<<dim3(a.n_nodes, a.n_paths), kWave, 0, s>>>(a);
  }
  const long total = long(a.n_nodes) * a.f_in;
  bwd_x_sum_kernel<<<int((total + 255) / 256), 256, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_bwd_pos(const BwdArgs& a, hipStream_t s) {
  const int n = a.n_nodes;
  if (n == 0) return hipSuccess;
  bwd_force_kernel<<<ceil_div(n, 256 / kWave), 256, 0, s>>>(a);
  bwd_pos_kernel<<<ceil_div(n, 256 / kWave), 256, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace cgtp
