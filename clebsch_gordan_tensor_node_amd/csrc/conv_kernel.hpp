// The fused node-centric CGTP convolution kernel.
//
// LunaTP ("Enabling Efficient and Scalable Tensor Product for Equivariant MLIPs")
// Figure 3: (a) node-centric execution sums the messages of all incoming edges on chip
// and stores each output once; (b) paths are grouped and mapped to SIMD lanes by
// channel block; (c) products are reused and equal coefficients factored; Table 8:
// inputs shared across paths.  This is the gfx950 design, not a translation:
//   * a workgroup serves one group (up to 7 paths of one input irrep and channel block;
//     3 in the backward) on S consecutive receivers of the degree-sorted order (LunaTP
//     Table 9: descending degree first): its first waves are consumers, wave p running
//     path p with T = 64 / S lanes per receiver, each lane owning K channels, and its
//     last wave is the producer that gathers the operands the paths share, once for all
//     of them;
//   * the receivers' active edges are walked in lock step, one edge per receiver per
//     step.  Per step the workgroup gathers the senders' x_j segments and the edges'
//     harmonics once, each thread one 16-byte share, into a double-buffered LDS stage;
//     one barrier publishes it and every wave reads its operands from LDS.  The only
//     per-path stream is the lane's own K weights of the edge;
//   * loads run D steps ahead of use in a register ring that holds only the thread's
//     shares and weights, so the pipeline is deep for few VGPRs; the edge and sender
//     indices of the receivers are staged in LDS first, so no index load waits behind
//     data loads in the wave's in-order memory counter;
//   * the path is a compile-time specialisation: the real CG coefficients and their
//     sparsity are constants, so A[m1,m3] = sum_m2 C[m1,m2,m3] Y[m2] is a short FMA
//     chain with immediate coefficients and structural zeros removed, applied to the K
//     channels as acc[k,m3] += w[k] * sum_m1 A[m1,m3] x[k,m1], scaling whichever side
//     (x or the partial result) is shorter;
//   * accumulators live in VGPRs for the whole edge loop; one coalesced store per
//     receiver and channel block at the end.  No atomics: the result is bitwise
//     reproducible.
// The uvu coupling is not a dense contraction, so no MFMA is used.
//
// This header is compiled once per kernel class (kernels_conv.hip with
// CGTP_CONV_CLASS = 0 .. kNumClasses-1); each build instantiates the class's conv_kernel
// for fp32 and, for the classes whose variants reach l <= 4, for fp64 (T = double: the
// same design with 16-byte chunks of two elements).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include "launch.hpp"
#include "variants.hpp"

namespace cgtp {

namespace {

constexpr int kConvThreadsFwd = kConvWavesMax * kWave;          // forward workgroups: up to 8 waves
constexpr int kConvThreadsBwd = (kConvJobsBwd + 1) * kWave;     // backward edge pass: up to 4
// (edge, sender) pairs staged per workgroup and window: fewer in the backward, whose
// x-gradient hand-off takes the LDS (three workgroups of the l1 <= 3 class per CU)
template <bool BWD>
constexpr int stage_log2() {
  return BWD ? 8 : 10;
}

template <int N>
struct IntC {
  static constexpr int value = N;
};

template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(IntC<B>{});
    static_for<B + 1, E>(f);
  }
}

template <int L1, int L2, int L3>
inline constexpr RealCG<L1, L2, L3> kCG{};

// Elements of T in one 16-byte vector access (4 floats, 2 doubles).  A job's K is either
// that (16-byte aligned data) or 1.
template <typename T>
inline constexpr int kVec = int(16 / sizeof(T));

template <typename T>
__device__ __forceinline__ T fma_t(T a, T b, T c) {
  if constexpr (sizeof(T) == 4)
    return __builtin_fmaf(a, b, c);
  else
    return __builtin_fma(a, b, c);
}

// A[M1, M3] = sum_m2 C[M1, m2, M3] Y[m2], structural zeros skipped.
template <typename T, int L1, int L2, int L3, int M1, int M3>
__device__ __forceinline__ T a_entry(const T* Y) {
  T s = T(0);
  bool first = true;
  static_for<0, 2 * L2 + 1>([&](auto M2) {
    constexpr T c = kCG<L1, L2, L3>.template coef<T>(M1, decltype(M2)::value, M3);
    if constexpr (c != T(0)) {
      if (first) {
        s = c * Y[decltype(M2)::value];
        first = false;
      } else {
        s = fma_t(c, Y[decltype(M2)::value], s);
      }
    }
  });
  return s;
}

template <typename T>
using vec16_t = T __attribute__((ext_vector_type(kVec<T>)));

template <typename T, int K>
__device__ __forceinline__ void load_k(const T* __restrict__ p, T* v) {
  if constexpr (K == kVec<T>) {
    const vec16_t<T> q = *reinterpret_cast<const vec16_t<T>*>(p);
#pragma unroll
    for (int k = 0; k < K; ++k) v[k] = q[k];
  } else {
#pragma unroll
    for (int k = 0; k < K; ++k) v[k] = p[k];
  }
}

// K elements read once (the weights): a non-temporal load, so that the stream does not
// evict the x rows and harmonics that the producer gathers again and again from L2
template <typename T, int K>
__device__ __forceinline__ void load_k_stream(const T* __restrict__ p, T* v) {
  if constexpr (K == kVec<T>) {
    const vec16_t<T> q = __builtin_nontemporal_load(reinterpret_cast<const vec16_t<T>*>(p));
#pragma unroll
    for (int k = 0; k < K; ++k) v[k] = q[k];
  } else {
#pragma unroll
    for (int k = 0; k < K; ++k) v[k] = __builtin_nontemporal_load(p + k);
  }
}

// N contiguous elements, in 16-byte vectors when K is the vector width (16-byte aligned
// source, N a multiple of K)
template <typename T, int K, int N>
__device__ __forceinline__ void load_run(const T* __restrict__ p, T* v) {
  if constexpr (K == kVec<T>) {
    static_assert(N % K == 0, "vector run");
#pragma unroll
    for (int q = 0; q < N / K; ++q) {
      const vec16_t<T> t = reinterpret_cast<const vec16_t<T>*>(p)[q];
#pragma unroll
      for (int k = 0; k < K; ++k) v[K * q + k] = t[k];
    }
  } else {
#pragma unroll
    for (int q = 0; q < N; ++q) v[q] = p[q];
  }
}

template <typename T, int K, int N>
__device__ __forceinline__ void store_run(T* __restrict__ p, const T* v) {
  if constexpr (K == kVec<T>) {
    static_assert(N % K == 0, "vector run");
#pragma unroll
    for (int q = 0; q < N / K; ++q) {
      vec16_t<T> t;
#pragma unroll
      for (int k = 0; k < K; ++k) t[k] = v[K * q + k];
      reinterpret_cast<vec16_t<T>*>(p)[q] = t;
    }
  } else {
#pragma unroll
    for (int q = 0; q < N; ++q) p[q] = v[q];
  }
}

// acc[k, m3] += w[k] sum_m1 A[m1, m3] x[k, m1] with A = C . Y (one edge, K channels)
template <typename T, int L1, int L2, int L3, int K>
__device__ __forceinline__ void accumulate_edge(T* acc, T* xv, const T* wv, const T* Y) {
  constexpr int N1 = 2 * L1 + 1, N3 = 2 * L3 + 1;
  if constexpr (N1 <= N3) {
    // scale the input side (2l1+1 products per channel), accumulate A x directly
#pragma unroll
    for (int q = 0; q < K * N1; ++q) xv[q] *= wv[q / N1];
    static_for<0, N3>([&](auto M3c) {
      constexpr int M3 = decltype(M3c)::value;
      static_for<0, N1>([&](auto M1c) {
        constexpr int M1 = decltype(M1c)::value;
        if constexpr (kCG<L1, L2, L3>.a_nonzero(M1, M3)) {
          const T A = a_entry<T, L1, L2, L3, M1, M3>(Y);
#pragma unroll
          for (int k = 0; k < K; ++k) acc[k * N3 + M3] = fma_t(A, xv[k * N1 + M1], acc[k * N3 + M3]);
        }
      });
    });
  } else {
    // form sum_m1 A x per output component, then scale by w (2l3+1 per channel)
    static_for<0, N3>([&](auto M3c) {
      constexpr int M3 = decltype(M3c)::value;
      T tk[K];
#pragma unroll
      for (int k = 0; k < K; ++k) tk[k] = T(0);
      static_for<0, N1>([&](auto M1c) {
        constexpr int M1 = decltype(M1c)::value;
        if constexpr (kCG<L1, L2, L3>.a_nonzero(M1, M3)) {
          const T A = a_entry<T, L1, L2, L3, M1, M3>(Y);
#pragma unroll
          for (int k = 0; k < K; ++k) tk[k] = fma_t(A, xv[k * N1 + M1], tk[k]);
        }
      });
#pragma unroll
      for (int k = 0; k < K; ++k) acc[k * N3 + M3] = fma_t(wv[k], tk[k], acc[k * N3 + M3]);
    });
  }
}

// The backward's x-gradient hand-off: per step parity, the lane values of the group's
// jobs other than the last, as [value][lane] (16-byte values for the vector form)
template <int C, typename T, bool BWD>
struct XgStage {
  T v[2][kConvJobsBwd - 1][kWave * (2 * class_max_l1(C) + 1) * kVec<T>];
};
template <int C, typename T>
struct XgStage<C, T, false> {};

// LDS of one workgroup of class C (sized by the class's largest l1).  Per step the
// producer wave stores N1 x chunks and one harmonic chunk per lane; chunk c of a step
// sits at c * (chunk elements), so the stage is receiver-major.  Chunks past the step's
// data land in the padding.
template <int C, typename T, bool BWD>
struct ConvSmem {
  static constexpr int kN1 = 2 * class_max_l1(C) + 1;
  static constexpr int kStage = (1 << stage_log2<BWD>()) + kWave;
  T x[2][kWave * kN1 * kVec<T>];    // x_j segments of one step (double-buffered)
  T y[2][kWave * kVec<T>];          // harmonics of one step (double-buffered)
  // staged offsets, receiver r's window at r (cap + 1): the odd row stride puts the
  // receivers of one read on different LDS banks
  uint32_t sx[kStage];              // j f_in (x element offset of the sender's row)
  uint32_t sw[kStage];              // (e - row start) W (w offset from the receiver's rows)
  uint32_t sy[kStage];              // q sh_stride (SH offset from the receiver's rows)
  uint32_t sg[BWD ? kStage : 1];    // backward: q part_stride (row of partials)
  int4 slot[kWave];                 // receiver records {node or -1, row start, active degree, 0}
  XgStage<C, T, BWD> xg;
};

// Pipeline depths (edge steps whose loads are in flight while one step is used), sized
// by the 32-bit registers a step holds.  The producer's loads (x_j rows, harmonics)
// mostly hit the L2 cache and need few steps; the consumers' weight loads come from HBM
// once and get a ring of K elements a slot.
template <typename T, int N1, int K>
constexpr int producer_depth() {
  constexpr int d = 72 / ((N1 * K + kVec<T>) * int(sizeof(T) / 4));
  return d < 2 ? 2 : (d > 4 ? 4 : d);
}
template <typename T, int K>
constexpr int consumer_depth() {
  return K == kVec<T> ? 4 : 6;
}

// v plus its copy from the lane that the DPP control CTRL selects (every lane active,
// full row and bank masks)
template <int CTRL>
__device__ __forceinline__ float add_dpp(float v) {
  return v + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

// Sum over aligned groups of 2^lg lanes (lg wave-uniform, at most 6); every lane of a
// group ends with the group's sum.  Within a row of 16 lanes the pairs are exchanged by
// DPP (lane ^ 1 and lane ^ 2 by quad permutes, then the half-row and the row mirrors,
// each pairing lanes whose partial sums cover disjoint halves), across the two rows of a
// 32-lane half by a swizzle (lane ^ 16), and across the halves by a permute.  Each stage
// adds the same two values on both lanes of a pair, so the result is reproducible.
__device__ __forceinline__ float group_sum(float v, int lg) {
  if (lg > 0) v = add_dpp<0xB1>(v);    // quad_perm [1, 0, 3, 2]
  if (lg > 1) v = add_dpp<0x4E>(v);    // quad_perm [2, 3, 0, 1]
  if (lg > 2) v = add_dpp<0x141>(v);   // row_half_mirror: lane 7 - i of each 8
  if (lg > 3) v = add_dpp<0x140>(v);   // row_mirror: lane 15 - i of each 16
  // swizzle bit mode, and-mask 0x1f, xor-mask 0x10: lane ^ 16 within each 32
  if (lg > 4) v += __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v), 0x401F));
  if (lg > 5) v += __shfl_xor(v, 32, kWave);
  return v;
}

template <typename T>
__device__ __forceinline__ const T* byte_off(const T* base, uint32_t bytes) {
  return reinterpret_cast<const T*>(reinterpret_cast<const char*>(base) + bytes);
}

// The backward of one edge for K channels (the lane's share), with g the receiver's
// output gradient [K][N3], x the sender's features [K][N1], w the edge's weights and Y its
// harmonics, in two parts.  With h[k][m1] = sum_m3 A[m1][m3] g[k][m3] (A = C . Y):
//   backward_edge_wx:  gw[k]     = sum_m1 x[k][m1] h[k][m1]                 (dL/dw)
//                      xg[k][m1] = w[k] h[k][m1]                            (the edge's dL/dx_j)
//   backward_edge_y:   gy[m2]    = sum_k w[k] sum_{m1,m3} C[m1,m2,m3] x[k][m1] g[k][m3]
//                      (this lane's part of dL/dY; x is scaled by w on return)
template <typename T, int L1, int L2, int L3, int K>
__device__ __forceinline__ void backward_edge_wx(const T* g, const T* x, const T* w, const T* Y, T* gw, T* xg) {
  constexpr int N1 = 2 * L1 + 1, N3 = 2 * L3 + 1;
#pragma unroll
  for (int q = 0; q < K * N1; ++q) xg[q] = T(0);
  static_for<0, N1>([&](auto M1c) {
    constexpr int M1 = decltype(M1c)::value;
    static_for<0, N3>([&](auto M3c) {
      constexpr int M3 = decltype(M3c)::value;
      if constexpr (kCG<L1, L2, L3>.a_nonzero(M1, M3)) {
        const T A = a_entry<T, L1, L2, L3, M1, M3>(Y);
#pragma unroll
        for (int k = 0; k < K; ++k) xg[k * N1 + M1] = fma_t(A, g[k * N3 + M3], xg[k * N1 + M1]);
      }
    });
  });
  // xg holds h here
#pragma unroll
  for (int k = 0; k < K; ++k) {
    T s = x[k * N1] * xg[k * N1];
#pragma unroll
    for (int m = 1; m < N1; ++m) s = fma_t(x[k * N1 + m], xg[k * N1 + m], s);
    gw[k] = s;
  }
#pragma unroll
  for (int q = 0; q < K * N1; ++q) xg[q] *= w[q / N1];
}

template <typename T, int L1, int L2, int L3, int K>
__device__ __forceinline__ void backward_edge_y(const T* g, T* x, const T* w, T* gy) {
  constexpr int N1 = 2 * L1 + 1, N2 = 2 * L2 + 1, N3 = 2 * L3 + 1;
#pragma unroll
  for (int q = 0; q < K * N1; ++q) x[q] *= w[q / N1];
#pragma unroll
  for (int m = 0; m < N2; ++m) gy[m] = T(0);
  static_for<0, N1>([&](auto M1c) {
    constexpr int M1 = decltype(M1c)::value;
    static_for<0, N3>([&](auto M3c) {
      constexpr int M3 = decltype(M3c)::value;
      if constexpr (kCG<L1, L2, L3>.a_nonzero(M1, M3)) {
        T pq = T(0);   // sum over the lane's channels of w x[m1] g[m3]
#pragma unroll
        for (int k = 0; k < K; ++k) pq = fma_t(x[k * N1 + M1], g[k * N3 + M3], pq);
        static_for<0, N2>([&](auto M2c) {
          constexpr int M2 = decltype(M2c)::value;
          constexpr T c = kCG<L1, L2, L3>.template coef<T>(M1, M2, M3);
          if constexpr (c != T(0)) gy[M2] = fma_t(c, pq, gy[M2]);
        });
      }
    });
  });
}

// One wave of a workgroup.  Waves 0 .. n_waves-2 are consumers, one job each (or idle
// when the group has fewer jobs); the last wave is the producer.  Consumer lane layout:
// lane = (receiver slot ns, channel lane t) with T = 2^lg channel lanes and S = 64 / T
// receivers (node positions ng S .. ng S + S - 1).  Stage layout per step: receiver r's
// x_j segment (n_ch N1 elements) at r n_ch N1, cut into chunks of K elements, chunk c
// loaded by producer lane c mod 64; receiver r's harmonics Y[y0 .. y0 + V y4) at r V y4,
// V = kVec<T> (the schedule keeps S y4 <= 64: one 16-byte chunk per producer lane).
//
// Steps past a receiver's last active edge repeat that edge (its offsets are staged
// again) with the weight replaced by zero, so every load is of real, finite data; a
// receiver without active edges stores zeros.  Every load of a pipeline step is issued
// unconditionally: a skipped load would make the wave's in-order memory counter
// ambiguous and force full waits.
template <int C, typename T, bool BWD, int L1, int L2, int L3, int K>
__device__ __forceinline__ void run_job(const ConvArgsT<T>& a, const Job& J, int job, int ng, int lg, int y0, int y4,
                                        int wave, bool has_job, int nj, ConvSmem<C, T, BWD>& sm) {
  constexpr int N1 = 2 * L1 + 1, N2 = 2 * L2 + 1, N3 = 2 * L3 + 1;
  constexpr int V = kVec<T>;
  constexpr uint32_t B = sizeof(T);
  static_assert(N1 <= ConvSmem<C, T, BWD>::kN1, "x stage too small for this variant");
  const int tid = int(threadIdx.x);
  const int lane = tid & (kWave - 1);
  const int S = kWave >> lg;
  const int n_ch = J.n_ch;
  const int cap_log2 = stage_log2<BWD>() - (6 - lg);   // staged entries per receiver and window
  const int srow = (1 << cap_log2) + 1;             // stage row stride

  __syncthreads();   // the receiver records (stored by the kernel entry) are visible
  // the edge steps of the node group: the largest active degree among its S receivers.
  // The node order is descending only up to its top bin (degrees past the bin count
  // share one bin in any order), so the first record is not always the largest.
  int qmax = lane < S ? sm.slot[lane].z : 0;
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) qmax = max(qmax, __shfl_xor(qmax, o, kWave));
  qmax = __builtin_amdgcn_readfirstlane(qmax);

  // stage the element offsets of every (receiver, step) of a window; a step past the
  // receiver's last edge repeats that edge, a receiver with no edge uses zeros
  auto stage = [&](int qw, int steps) {
    const int spl = steps > 1 ? 32 - __clz(steps - 1) : 0;
    for (int idx = tid; idx < (S << spl); idx += int(blockDim.x)) {
      const int r = idx >> spl, k = idx & ((1 << spl) - 1);
      if (k < steps) {
        const int4 si = sm.slot[r];
        uint32_t ox = 0, ow = 0, oy = 0;
        if (si.z > 0) {
          const int q = min(qw + k, si.z - 1);
          const int e = a.act_e[si.y + q];
          const int j = a.act_j[si.y + q];
          ox = uint32_t(j) * uint32_t(a.f_in);
          ow = uint32_t(e - si.y) * uint32_t(a.w_stride);
          oy = uint32_t(q) * uint32_t(a.sh_stride);
        }
        const int at = r * srow + k;
        sm.sx[at] = ox;
        sm.sw[at] = ow;
        sm.sy[at] = oy;
        if constexpr (BWD) sm.sg[at] = oy / uint32_t(a.sh_stride) * uint32_t(a.part_stride);
      }
    }
  };

  if (wave == int(blockDim.x) / kWave - 1) {
    // ---------------- producer: x_j segments and harmonics of every step ----------------
    constexpr int D = producer_depth<T, N1, K>();
    const int cps = n_ch * N1 / K;                  // x chunks per receiver
    uint32_t x_off[N1];
    int x_sl[N1];
#pragma unroll
    for (int i = 0; i < N1; ++i) {
      const int c = lane + kWave * i;
      x_sl[i] = 0;
      x_off[i] = uint32_t(J.in_off);
      if (c < S * cps) {
        const int r = c / cps;
        x_sl[i] = r * srow;
        x_off[i] = uint32_t(J.in_off + (c - r * cps) * K);
      }
    }
    int y_sl = 0;
    const T* ybase = a.sh + y0;
    if (lane < S * y4) {
      const int r = lane / y4;
      const int4 si = sm.slot[r];
      y_sl = r * srow;
      ybase = a.sh + (long)(si.z > 0 ? si.y : 0) * a.sh_stride + y0 + V * (lane - r * y4);
    }
    struct PSlot {
      T x[N1 * K];
      T y[V];
    };
    struct PIdx {
      uint32_t x[N1];
      uint32_t y;
    };
    PSlot ring[D];
    for (int qw = 0; qw < qmax; qw += (1 << cap_log2)) {
      const int steps = min(1 << cap_log2, qmax - qw);
      stage(qw, steps);
      __syncthreads();
      auto fetch = [&](int k, PIdx& ix) {
        const int kk = min(k, steps - 1);
#pragma unroll
        for (int i = 0; i < N1; ++i) ix.x[i] = (sm.sx[x_sl[i] + kk] + x_off[i]) * B;
        ix.y = sm.sy[y_sl + kk] * B;
      };
      auto issue = [&](const PIdx& ix, PSlot& b) {
#pragma unroll
        for (int i = 0; i < N1; ++i) load_k<T, K>(byte_off(a.x, ix.x[i]), b.x + i * K);
        load_k<T, V>(byte_off(ybase, ix.y), b.y);
        // keep the steps' loads in program order: the memory counter is in order, and a
        // step's loads scheduled after a later step's would make that step wait for both
        __builtin_amdgcn_sched_barrier(0);
      };
      auto publish = [&](int k, PSlot& b) {
        T* xs = sm.x[k & 1];
#pragma unroll
        for (int i = 0; i < N1; ++i) store_run<T, K, K>(xs + (lane + kWave * i) * K, b.x + i * K);
        store_run<T, V, V>(sm.y[k & 1] + lane * V, b.y);
        __syncthreads();
      };
      // every step issues its loads unconditionally (past the window's end they repeat
      // its last step), so the wave's memory counter is exact on every path; only the
      // publishing, which holds no load, is skipped past the end
      PIdx ix;
      static_for<0, D - 1>([&](auto P) {
        constexpr int p = decltype(P)::value;
        fetch(p, ix);
        issue(ix, ring[p]);
      });
      fetch(D - 1, ix);
      for (int k0 = 0; k0 < steps; k0 += D) {
        static_for<0, D>([&](auto Sx) {
          constexpr int s = decltype(Sx)::value;
          issue(ix, ring[(s + D - 1) % D]);
          fetch(k0 + s + D, ix);
          if (k0 + s < steps) publish(k0 + s, ring[s]);
        });
      }
      __syncthreads();   // every staged offset and stage buffer consumed before re-staging
    }
    return;
  }

  if (!has_job) {
    // ---------------- idle consumer: keep the workgroup's barrier count ----------------
    for (int qw = 0; qw < qmax; qw += (1 << cap_log2)) {
      const int steps = min(1 << cap_log2, qmax - qw);
      stage(qw, steps);
      __syncthreads();
      for (int k = 0; k < steps; ++k) __syncthreads();
      __syncthreads();
    }
    return;
  }

  if constexpr (BWD) {
    // ---------------- consumer (backward): dL/dw, dL/dY and dL/dx per edge ----------
    // As the forward's consumer, but per edge step it writes the edge's w-gradient for
    // its K channels, the job's dL/dY of the edge's slot (summed over the receiver's
    // lanes by group_sum) and the edge's x-gradient of its channels, added over
    // the group's jobs in job order: the jobs before the last hand theirs to the last
    // job's wave through LDS (buffer by step parity), which adds them one step later and
    // stores the sum, one block per (active slot, group).  Steps past a receiver's last
    // edge repeat that edge (its weights are kept), so they store the same values
    // again; lanes without edges or channels store into a scratch row.
    constexpr int D = consumer_depth<T, K>();
    constexpr int NX = K * N1;
    const int t = lane & ((1 << lg) - 1);
    const int ns = lane >> lg;
    const int ch0 = t * K;
    const int4 my = sm.slot[ns];
    const bool mine = my.z > 0 && ch0 < n_ch;
    const int w_sl = ns * srow;
    const long rowoff = (long)(my.z > 0 ? my.y : 0) * a.w_stride + J.w_off + (ch0 < n_ch ? ch0 : 0);
    const T* __restrict__ wbase = a.w + rowoff;
    T* gwbase = a.grad_w ? a.grad_w + rowoff : nullptr;
    const long prow = (long)(my.z > 0 ? my.y : 0) * a.part_stride;
    T* gybase = a.gyp ? a.gyp + prow + a.job_gy[job] : nullptr;
    T* xgbase = a.xgp ? a.xgp + prow + a.job_xg[job] + ch0 * N1 : nullptr;
    const bool last = wave == nj - 1;            // the job that adds the group's x-gradients
    const bool defer = a.xgp && last && nj > 1;  // uniform
    const int x_rd = (ns * n_ch + ch0) * N1;
    const int y_rd = ns * V * y4 + J.sh_off - y0;
    T g[K * N3];
    if (ch0 < n_ch && my.x >= 0) {
      load_run<T, K, K * N3>(a.grad_out + (long)my.x * a.f_out + J.out_off + ch0 * N3, g);
    } else {
#pragma unroll
      for (int q = 0; q < K * N3; ++q) g[q] = T(0);
    }
    // the hand-off: value q of this lane at [q][lane] (16-byte values for K = kVec)
    auto put = [&](int kg, const T* v) {
      T* dst = sm.xg.v[kg & 1][wave];
      if constexpr (K == V) {
#pragma unroll
        for (int c = 0; c < N1; ++c) {
          vec16_t<T> q;
#pragma unroll
          for (int m = 0; m < V; ++m) q[m] = v[V * c + m];
          reinterpret_cast<vec16_t<T>*>(dst)[c * kWave + lane] = q;
        }
      } else {
#pragma unroll
        for (int c = 0; c < NX; ++c) dst[c * kWave + lane] = v[c];
      }
    };
    // the last job's x-gradient of the previous step and where its group sum goes
    T pend[NX];
    T* pend_dst = a.scratch_row;
    // stores step kg's group sum, (job 0 + job 1) + the last job's own value, one 16-byte
    // chunk at a time (few registers live)
    auto flush = [&](int kg) {
      const T* x0 = sm.xg.v[kg & 1][0];
      const T* x1 = sm.xg.v[kg & 1][1];
      if constexpr (K == V) {
#pragma unroll
        for (int c = 0; c < N1; ++c) {
          vec16_t<T> q = reinterpret_cast<const vec16_t<T>*>(x0)[c * kWave + lane];
          if (nj > 2) q += reinterpret_cast<const vec16_t<T>*>(x1)[c * kWave + lane];
#pragma unroll
          for (int m = 0; m < V; ++m) q[m] += pend[V * c + m];
          reinterpret_cast<vec16_t<T>*>(pend_dst)[c] = q;
        }
      } else {
#pragma unroll
        for (int c = 0; c < NX; ++c) {
          T v = x0[c * kWave + lane];
          if (nj > 2) v += x1[c * kWave + lane];
          pend_dst[c] = v + pend[c];
        }
      }
    };
    T ring[D][K];
    for (int qw = 0; qw < qmax; qw += (1 << cap_log2)) {
      const int steps = min(1 << cap_log2, qmax - qw);
      stage(qw, steps);
      __syncthreads();
      auto fetch = [&](int k) { return sm.sw[w_sl + min(k, steps - 1)] * B; };
      auto issue = [&](uint32_t ow, T* b) {
        load_k_stream<T, K>(byte_off(wbase, ow), b);
        __builtin_amdgcn_sched_barrier(0);
      };
      auto use = [&](int k, T* b) {
        __syncthreads();   // the producer has published step k; the hand-off of step k - 1 is complete
#pragma unroll
        for (int m = 0; m < K; ++m) asm volatile("" : "+v"(b[m]));
        const int kg = qw + k;
        if (defer && kg > 0) flush(kg - 1);
        // the flush stays apart from this step's work: interleaved, both sets of values
        // would be live at once
        __builtin_amdgcn_sched_barrier(0);
        T wv[K];
#pragma unroll
        for (int m = 0; m < K; ++m) wv[m] = mine ? b[m] : T(0);
        T xv[K * N1];
        load_run<T, K, K * N1>(sm.x[k & 1] + x_rd, xv);
        T Y[N2];
        const T* ys = sm.y[k & 1] + y_rd;
#pragma unroll
        for (int m = 0; m < N2; ++m) Y[m] = ys[m];
        T gw[K], xg[NX];
        backward_edge_wx<T, L1, L2, L3, K>(g, xv, wv, Y, gw, xg);
        const uint32_t prow_k = sm.sg[w_sl + k];
        T* xdst = mine && a.xgp ? xgbase + prow_k : a.scratch_row;
        if (a.xgp) {      // uniform: the x-gradient is requested
          if (!last)
            put(kg, xg);
          else if (nj == 1)
            store_run<T, K, NX>(xdst, xg);
        }
        // kept by every wave (only the deferring one uses it): assigned on every path, the
        // previous value is dead once the flush above has run
#pragma unroll
        for (int q = 0; q < NX; ++q) pend[q] = xg[q];
        pend_dst = xdst;
        if (a.grad_w) {   // uniform: the w-gradient is requested
          T* dst = mine ? reinterpret_cast<T*>(reinterpret_cast<char*>(gwbase) + sm.sw[w_sl + k] * B) : a.scratch_row;
          store_run<T, K, K>(dst, gw);
        }
        if (a.gyp) {      // uniform: dL/dY is requested (for the position gradient)
          T gy[N2];
          backward_edge_y<T, L1, L2, L3, K>(g, xv, wv, gy);
#pragma unroll
          for (int m = 0; m < N2; ++m) gy[m] = group_sum(gy[m], lg);
          if (t == 0) {
            T* gdst = my.z > 0 ? gybase + prow_k : a.scratch_row;
#pragma unroll
            for (int m = 0; m < N2; ++m) gdst[m] = gy[m];
          }
        }
      };
      static_for<0, D - 1>([&](auto P) {
        constexpr int p = decltype(P)::value;
        issue(fetch(p), ring[p]);
      });
      uint32_t ow = fetch(D - 1);
      for (int k0 = 0; k0 < steps; k0 += D) {
        static_for<0, D>([&](auto Sx) {
          constexpr int s = decltype(Sx)::value;
          issue(ow, ring[(s + D - 1) % D]);
          ow = fetch(k0 + s + D);
          if (k0 + s < steps) use(k0 + s, ring[s]);
        });
      }
      __syncthreads();
    }
    // the last step's group sum (its hand-off is complete after the window's last barrier)
    if (defer && qmax > 0) flush(qmax - 1);
    return;
  }

  // ---------------- consumer: this job's weights and accumulation ----------------
  constexpr int D = consumer_depth<T, K>();
  const int t = lane & ((1 << lg) - 1);
  const int ns = lane >> lg;
  const int ch0 = t * K;
  const int4 my = sm.slot[ns];
  const int w_n = ch0 < n_ch ? my.z : 0;
  const int w_sl = ns * srow;
  const T* __restrict__ wbase =
      a.w + (long)(my.z > 0 ? my.y : 0) * a.w_stride + J.w_off + (ch0 < n_ch ? ch0 : 0);
  const int x_rd = (ns * n_ch + ch0) * N1;          // this lane's operands in the x stage
  const int y_rd = ns * V * y4 + J.sh_off - y0;     // ... and its Y_l2 in the harmonic stage

  T acc[K * N3];
#pragma unroll
  for (int q = 0; q < K * N3; ++q) acc[q] = T(0);
  T ring[D][K];
  for (int qw = 0; qw < qmax; qw += (1 << cap_log2)) {
    const int steps = min(1 << cap_log2, qmax - qw);
    stage(qw, steps);
    __syncthreads();
    auto fetch = [&](int k) { return sm.sw[w_sl + min(k, steps - 1)] * B; };
    auto issue = [&](uint32_t ow, T* b) {
      load_k_stream<T, K>(byte_off(wbase, ow), b);
      __builtin_amdgcn_sched_barrier(0);   // loads stay in step order (see the producer)
    };
    auto use = [&](int k, T* b) {
      __syncthreads();   // the producer has published step k
      // the weights are first touched here, after the barrier: without this the
      // scheduler hoists the selects of all unrolled steps above the loop's barriers and
      // waits for every weight load at once
#pragma unroll
      for (int m = 0; m < K; ++m) asm volatile("" : "+v"(b[m]));
      const bool live = qw + k < w_n;
      T wv[K];
#pragma unroll
      for (int m = 0; m < K; ++m) wv[m] = live ? b[m] : T(0);
      T xv[K * N1];
      load_run<T, K, K * N1>(sm.x[k & 1] + x_rd, xv);
      T Y[N2];
      const T* ys = sm.y[k & 1] + y_rd;
#pragma unroll
      for (int m = 0; m < N2; ++m) Y[m] = ys[m];
      accumulate_edge<T, L1, L2, L3, K>(acc, xv, wv, Y);
    };
    // as in the producer: loads unconditional, only the use skipped past the end
    static_for<0, D - 1>([&](auto P) {
      constexpr int p = decltype(P)::value;
      issue(fetch(p), ring[p]);
    });
    uint32_t ow = fetch(D - 1);
    for (int k0 = 0; k0 < steps; k0 += D) {
      static_for<0, D>([&](auto Sx) {
        constexpr int s = decltype(Sx)::value;
        issue(ow, ring[(s + D - 1) % D]);
        ow = fetch(k0 + s + D);
        if (k0 + s < steps) use(k0 + s, ring[s]);
      });
    }
    __syncthreads();
  }
  if (ch0 < n_ch && my.x >= 0) {
    if (my.z == 0) {
#pragma unroll
      for (int q = 0; q < K * N3; ++q) acc[q] = T(0);
    }
    store_run<T, K, K * N3>(a.out + (long)my.x * a.f_out + J.out_off + ch0 * N3, acc);
  }
}

template <int C, typename T, bool BWD, int LO, int HI>
__device__ __forceinline__ void dispatch(int v, const ConvArgsT<T>& a, const Job& J, int job, int ng, int lg, int y0,
                                         int y4, int wave, bool has_job, int nj, ConvSmem<C, T, BWD>& sm) {
  if constexpr (HI - LO == 1) {
    if constexpr (class_contains(C, LO) && (sizeof(T) == 4 || variant_lmax(LO) <= kF64Lmax) &&
                  (!BWD || variant_lmax(LO) <= kBwdLmax)) {
      constexpr VariantDesc d = variant_desc(LO);
      constexpr int K = d.k == 1 ? 1 : kVec<T>;   // the vector form moves 16 bytes per lane
      run_job<C, T, BWD, d.l1, d.l2, d.l3, K>(a, J, job, ng, lg, y0, y4, wave, has_job, nj, sm);
    }
  } else {
    constexpr int MID = (LO + HI) / 2;
    if (v < MID)
      dispatch<C, T, BWD, LO, MID>(v, a, J, job, ng, lg, y0, y4, wave, has_job, nj, sm);
    else
      dispatch<C, T, BWD, MID, HI>(v, a, J, job, ng, lg, y0, y4, wave, has_job, nj, sm);
  }
}

// One workgroup per (group, node group): the producer wave and one consumer wave per job
// (consumer waves past the group's job count only keep the barrier count).  The producer
// runs the first job's code path, which fixes l1, K and the channel block it gathers.
// BWD: the backward's edge pass (dL/dw, the per-job dL/dY and the per-group dL/dx of
// every active slot) instead of the forward.
template <int C, typename T, bool BWD>
__device__ __forceinline__ void conv_workgroup(const ConvArgsT<T>& a) {
  // the hardware deals workgroups to the XCDs round-robin by index; the numbering puts
  // every workgroup of one receiver block on the same XCD, so that the block's groups
  // share the senders' rows and the edges' harmonics in that XCD's L2
  const int xcd = int(blockIdx.x) % kXcds;
  const int rr = int(blockIdx.x) / kXcds;
  const int rb = rr / a.blk_wgs;
  const int wg = rr - rb * a.blk_wgs;
  const int blk = rb * kXcds + xcd;
  if (blk >= a.n_blocks) return;   // padding of the last round of blocks
  // the workgroup's group: the last g with g_start[g] <= wg (g_start is increasing, and
  // INT32_MAX past the launch's groups); the sign bit of g_start - wg - 1 counts it
  uint32_t g = 0;
#pragma unroll
  for (int k = 1; k < kMaxGroupsPerLaunch; ++k) g += uint32_t(a.g_start[k] - wg - 1) >> 31;
  // read through the kernel-argument segment pointer: a dynamic index into the by-value
  // argument would make the compiler copy the whole argument block to scratch first
  const GroupArgs G = reinterpret_cast<const GroupArgs*>(
      (const char*)__builtin_amdgcn_kernarg_segment_ptr() + offsetof(ConvArgsT<T>, grp))[g];
  const int lg = G.lanes_log2;
  const int S = kWave >> lg;
  const int ng = (blk << (lg - a.blk_lg_min)) + (wg - G.start);   // node group of this group
  const int wave = __builtin_amdgcn_readfirstlane(int(threadIdx.x) / kWave);
  const bool has_job = wave < G.n_jobs;
  // the receiver records and the job descriptor are independent loads: both in flight
  // before either is waited for
  // (branch-free: every thread loads a valid record and stores it, the threads of one
  // slot storing the same value, so that no divergent region separates the two loads)
  const int tid = int(threadIdx.x);
  const int pos = ng * S + (tid & (S - 1));
  const int4 rec = a.node_info[min(pos, a.n_nodes - 1)];
  const int job = G.first_job + (has_job ? wave : 0);
  const Job J = a.jobs[job];
  __shared__ ConvSmem<C, T, BWD> sm;
  sm.slot[tid & (S - 1)] = pos < a.n_nodes ? rec : make_int4(-1, 0, 0, 0);
  dispatch<C, T, BWD, 0, kNumVariants>(J.variant, a, J, job, ng, lg, G.y0, G.y4, wave, has_job, G.n_jobs, sm);
}

template <int C, typename T>
__global__ void __launch_bounds__(kConvThreadsFwd) conv_kernel(ConvArgsT<T> a) {
  conv_workgroup<C, T, false>(a);
}

// The backward's workgroups per CU as the LDS allows them (at most 3): the register
// budget is set to match, so that registers never lower the occupancy below what the
// LDS permits and the l1 <= 3 code (about 170 registers unconstrained) fits 3 per SIMD.
template <int C>
constexpr int bwd_waves_per_eu() {
  constexpr int by_lds = int((160 * 1024) / sizeof(ConvSmem<C, float, true>));
  return by_lds < 1 ? 1 : (by_lds > 3 ? 3 : by_lds);
}

template <int C>
__global__ void __launch_bounds__(kConvThreadsBwd) __attribute__((amdgpu_waves_per_eu(bwd_waves_per_eu<C>())))
conv_kernel_bwd(ConvArgsT<float> a) {
  conv_workgroup<C, float, true>(a);
}

}  // namespace

template <int C, typename T>
hipError_t launch_conv_class(const ConvArgsT<T>& args, hipStream_t s, hipEvent_t ev_start, hipEvent_t ev_stop) {
  if (args.total_wgs <= 0) return hipSuccess;
  const int blocks = args.total_wgs;
  if (ev_start || ev_stop) {
    // the events are stamped by the dispatch itself: kernel time without launch gaps
    hipExtLaunchKernelGGL(conv_kernel<C, T>, dim3(blocks), dim3(args.n_waves * kWave), 0, s, ev_start, ev_stop,
                          0, args);
  } else {
    conv_kernel<C, T><<<blocks, args.n_waves * kWave, 0, s>>>(args);
  }
  return hipGetLastError();
}

template <int C>
hipError_t launch_conv_bwd_class(const ConvArgsT<float>& args, hipStream_t s) {
  if (args.total_wgs <= 0) return hipSuccess;
  conv_kernel_bwd<C><<<args.total_wgs, args.n_waves * kWave, 0, s>>>(args);
  return hipGetLastError();
}

}  // namespace cgtp
