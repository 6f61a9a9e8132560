// The fused node-centric CGTP convolution kernel.
//
// LunaTP ("Enabling Efficient and Scalable Tensor Product for Equivariant MLIPs")
// Figure 3: (a) node-centric execution sums the messages of all incoming edges on chip
// and stores each output once; (b) paths are grouped and mapped to SIMD lanes by
// channel block; (c) products are reused and equal coefficients factored.  This is
// the gfx950 design, not a translation:
//   * a wave (64 lanes) runs one job = (path, channel block) for Sn consecutive
//     receivers of the degree-sorted node order (LunaTP Table 9: descending degree
//     first); each receiver gets Se edge slots of T lanes (Sn Se T = 64), each lane
//     owning K channels; the edge slots split the receiver's edges round robin and are
//     summed by a butterfly at the end, so long rows do not set the kernel's tail;
//   * the path is a compile-time specialisation: the real CG coefficients and their
//     sparsity are constants, so A[m1,m3] = sum_m2 C[m1,m2,m3] Y[m2] is a short FMA
//     chain with immediate coefficients and structural zeros removed;
//   * per edge a lane loads its K weights (one 16-byte load when K = 4), its K x_j
//     channel vectors and the edge's Y_l2, forms A once, and applies it to its K
//     channels: acc[k,m3] += w[k] * sum_m1 A[m1,m3] x[k,m1], scaling whichever side
//     (x or the partial result) is shorter;
//   * the edge loop is a software pipeline: the operands of the next D-1 edges are in
//     flight (a ring of register buffers) while one edge is accumulated; the edge and
//     sender indices of the receivers are staged in a wave-private LDS area first, so
//     no index load waits behind data loads in the in-order memory counter and no
//     register that a load is still filling is ever copied;
//   * accumulators live in VGPRs for the whole edge loop; one coalesced store per
//     receiver and channel block at the end.  No atomics: the result is bitwise
//     reproducible.
// The uvu coupling is not a dense contraction, so no MFMA is used.
//
// This header is compiled once per kernel class (kernels_conv.hip with
// CGTP_CONV_CLASS = 0 .. kNumClasses-1); each build instantiates one conv_kernel.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include "launch.hpp"
#include "variants.hpp"

namespace cgtp {

namespace {

constexpr int kConvThreads = 256;
constexpr int kConvWaves = kConvThreads / kWave;


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

// A[M1, M3] = sum_m2 C[M1, m2, M3] Y[m2], structural zeros skipped.
template <int L1, int L2, int L3, int M1, int M3>
__device__ __forceinline__ float a_entry(const float* Y) {
  float s = 0.0f;
  bool first = true;
  static_for<0, 2 * L2 + 1>([&](auto M2) {
    constexpr float c = kCG<L1, L2, L3>.at(M1, decltype(M2)::value, M3);
    if constexpr (c != 0.0f) {
      if (first) {
        s = c * Y[decltype(M2)::value];
        first = false;
      } else {
        s = __builtin_fmaf(c, Y[decltype(M2)::value], s);
      }
    }
  });
  return s;
}

template <int K>
__device__ __forceinline__ void load_k(const float* __restrict__ p, float* v) {
  if constexpr (K == 4) {
    const float4 q = *reinterpret_cast<const float4*>(p);
    v[0] = q.x;
    v[1] = q.y;
    v[2] = q.z;
    v[3] = q.w;
  } else {
#pragma unroll
    for (int k = 0; k < K; ++k) v[k] = p[k];
  }
}

// n contiguous floats, n a multiple of 4 when K == 4 (16-byte aligned source)
template <int K, int N>
__device__ __forceinline__ void load_run(const float* __restrict__ p, float* v) {
  if constexpr (K == 4) {
    static_assert(N % 4 == 0, "vector run");
#pragma unroll
    for (int q = 0; q < N / 4; ++q) {
      const float4 t = reinterpret_cast<const float4*>(p)[q];
      v[4 * q + 0] = t.x;
      v[4 * q + 1] = t.y;
      v[4 * q + 2] = t.z;
      v[4 * q + 3] = t.w;
    }
  } else {
#pragma unroll
    for (int q = 0; q < N; ++q) v[q] = p[q];
  }
}

template <int K, int N>
__device__ __forceinline__ void store_run(float* __restrict__ p, const float* v) {
  if constexpr (K == 4) {
    static_assert(N % 4 == 0, "vector run");
#pragma unroll
    for (int q = 0; q < N / 4; ++q) {
      float4 t;
      t.x = v[4 * q + 0];
      t.y = v[4 * q + 1];
      t.z = v[4 * q + 2];
      t.w = v[4 * q + 3];
      reinterpret_cast<float4*>(p)[q] = t;
    }
  } else {
#pragma unroll
    for (int q = 0; q < N; ++q) p[q] = v[q];
  }
}

// acc[k, m3] += w[k] sum_m1 A[m1, m3] x[k, m1] with A = C . Y (one edge, K channels)
template <int L1, int L2, int L3, int K>
__device__ __forceinline__ void accumulate_edge(float* acc, float* xv, const float* wv, const float* Y) {
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
          const float A = a_entry<L1, L2, L3, M1, M3>(Y);
#pragma unroll
          for (int k = 0; k < K; ++k) acc[k * N3 + M3] = __builtin_fmaf(A, xv[k * N1 + M1], acc[k * N3 + M3]);
        }
      });
    });
  } else {
    // form sum_m1 A x per output component, then scale by w (2l3+1 per channel)
    static_for<0, N3>([&](auto M3c) {
      constexpr int M3 = decltype(M3c)::value;
      float tk[K];
#pragma unroll
      for (int k = 0; k < K; ++k) tk[k] = 0.0f;
      static_for<0, N1>([&](auto M1c) {
        constexpr int M1 = decltype(M1c)::value;
        if constexpr (kCG<L1, L2, L3>.a_nonzero(M1, M3)) {
          const float A = a_entry<L1, L2, L3, M1, M3>(Y);
#pragma unroll
          for (int k = 0; k < K; ++k) tk[k] = __builtin_fmaf(A, xv[k * N1 + M1], tk[k]);
        }
      });
#pragma unroll
      for (int k = 0; k < K; ++k) acc[k * N3 + M3] = __builtin_fmaf(wv[k], tk[k], acc[k * N3 + M3]);
    });
  }
}

template <int K, int N1, int N2>
struct EdgeBuf {
  float x[K * N1];
  float w[K];
  float y[N2];
};

// Ring depth: edges whose operands are in flight while one edge is accumulated.
template <int N1>
constexpr int ring_depth() {
  return N1 <= 5 ? 3 : 2;
}

// Wave-private LDS staging of edge indices: kStageEntries (edge, sender) pairs per
// wave, shared by its receivers (kStageEntries / Sn each).
constexpr int kStageEntries = 512;

// Lane layout of a wave: lane = (node slot, edge slot, channel lane) with T = 2^lg
// channel lanes, Se = 2^sg edge slots and Sn = 64 / (T Se) node slots.  Edge slot es
// of a receiver takes its active edges es, es + Se, ...; the edge slots are summed by a
// butterfly at the end.
template <int L1, int L2, int L3, int K>
__device__ __forceinline__ void run_job(const ConvArgs& a, const Job& J, int node_pos, int lane, int lg, int sg,
                                        int2* __restrict__ stage) {
  constexpr int N1 = 2 * L1 + 1, N2 = 2 * L2 + 1, N3 = 2 * L3 + 1;
  constexpr int D = ring_depth<N1>();
  const int T = 1 << lg;
  const int Se = 1 << sg;
  const int t = lane & (T - 1);
  const int es = (lane >> lg) & (Se - 1);
  const int nslot = lane >> (lg + sg);
  const int cap = kStageEntries >> (6 - lg - sg);   // staged edges per receiver and window
  int2* __restrict__ my_stage = stage + nslot * cap;
  const int ch0 = t * K;
  const bool ok = (node_pos < a.n_nodes) && (ch0 < J.n_ch);
  int i = 0, rb = 0, n_act = 0;
  if (node_pos < a.n_nodes) {
    const int4 ni = a.node_info[node_pos];
    i = ni.x;
    rb = ni.y;
    n_act = ni.z;
  }
  // active edges of row i, compacted within the row: edge ids act_e[rb + q], senders
  // act_j[rb + q], harmonics sh[(rb + q) * sh_stride], q < n_act
  int qmax = n_act;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) qmax = max(qmax, __shfl_xor(qmax, off, kWave));
  qmax = __builtin_amdgcn_readfirstlane(qmax);

  float acc[K * N3];
#pragma unroll
  for (int q = 0; q < K * N3; ++q) acc[q] = 0.0f;

  const float* __restrict__ xb = a.x + J.in_off + ch0 * N1;
  const float* __restrict__ wb = a.w + J.w_off + ch0;
  const float* __restrict__ shb = a.sh + J.sh_off + (long)rb * a.sh_stride;
  const int32_t* __restrict__ ae = a.act_e + rb;
  const int32_t* __restrict__ aj = a.act_j + rb;

  // Ring buffers start at zero; a lane with no edge at some step accumulates with a zero
  // weight, so the accumulate step has no branch and the compiler can track every
  // buffer's outstanding loads exactly.
  EdgeBuf<K, N1, N2> ring[D];
#pragma unroll
  for (int d = 0; d < D; ++d) {
#pragma unroll
    for (int m = 0; m < K * N1; ++m) ring[d].x[m] = 0.0f;
#pragma unroll
    for (int m = 0; m < K; ++m) ring[d].w[m] = 0.0f;
#pragma unroll
    for (int m = 0; m < N2; ++m) ring[d].y[m] = 0.0f;
  }
  // step k of a window: this lane's edge is q = qw + k Se + es
  auto issue = [&](int k, int qw, EdgeBuf<K, N1, N2>& b) {
    const int q = qw + (k << sg) + es;
    if (ok && q < n_act) {
      const int2 ej = my_stage[q - qw];
      load_run<K, K * N1>(xb + (long)ej.y * a.f_in, b.x);
      load_k<K>(wb + (long)ej.x * a.w_stride, b.w);
      const float* ys = shb + (long)q * a.sh_stride;
#pragma unroll
      for (int m = 0; m < N2; ++m) b.y[m] = ys[m];
    }
  };
  auto consume = [&](int k, int qw, EdgeBuf<K, N1, N2>& b) {
    const bool live = ok && (qw + (k << sg) + es) < n_act;
    float wv[K];
#pragma unroll
    for (int m = 0; m < K; ++m) wv[m] = live ? b.w[m] : 0.0f;
    accumulate_edge<L1, L2, L3, K>(acc, b.x, wv, b.y);
  };

  for (int qw = 0; qw < qmax; qw += cap) {   // windows of `cap` edges (one for short rows)
    const int qend = min(qmax, qw + cap);
    const int steps = (qend - qw + Se - 1) >> sg;
    // stage this window's indices: the receiver's lanes copy them cooperatively; LDS
    // operations of one wave complete in order, so the fences only order the compiler
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    for (int q = qw + (lane & (T * Se - 1)); q < min(n_act, qend); q += T * Se)
      my_stage[q - qw] = make_int2(ae[q], aj[q]);
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // software pipeline: the operands of the next D-1 edges are in flight while one
    // edge is accumulated; ring slots are static after unrolling by D
    static_for<0, D - 1>([&](auto P) {
      constexpr int p = decltype(P)::value;
      if (p < steps) issue(p, qw, ring[p]);
    });
    int k0 = 0;
    for (; k0 + 2 * D - 2 < steps; k0 += D) {   // steady state: every step issues
      static_for<0, D>([&](auto Sx) {
        constexpr int s = decltype(Sx)::value;
        issue(k0 + s + D - 1, qw, ring[(s + D - 1) % D]);
        consume(k0 + s, qw, ring[s]);
      });
    }
    for (; k0 < steps; k0 += D) {               // drain
      static_for<0, D>([&](auto Sx) {
        constexpr int s = decltype(Sx)::value;
        const int k = k0 + s;
        if (k < steps) {
          if (k + D - 1 < steps) issue(k + D - 1, qw, ring[(s + D - 1) % D]);
          consume(k, qw, ring[s]);
        }
      });
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");  // staged entries consumed
  }
  // sum the edge slots of each receiver (lane bits lg .. lg+sg-1); slot 0 stores
  for (int off = T; off < (T << sg); off <<= 1) {
#pragma unroll
    for (int q = 0; q < K * N3; ++q) acc[q] += __shfl_xor(acc[q], off, kWave);
  }
  if (ok && es == 0) store_run<K, K * N3>(a.out + (long)i * a.f_out + J.out_off + ch0 * N3, acc);
}

template <int C, int LO, int HI>
__device__ __forceinline__ void dispatch(int v, const ConvArgs& a, const Job& J, int node_pos, int lane, int lg,
                                         int sg, int2* stage) {
  if constexpr (HI - LO == 1) {
    if constexpr (class_contains(C, LO)) {
      constexpr VariantDesc d = variant_desc(LO);
      run_job<d.l1, d.l2, d.l3, d.k>(a, J, node_pos, lane, lg, sg, stage);
    }
  } else {
    constexpr int MID = (LO + HI) / 2;
    if (v < MID)
      dispatch<C, LO, MID>(v, a, J, node_pos, lane, lg, sg, stage);
    else
      dispatch<C, MID, HI>(v, a, J, node_pos, lane, lg, sg, stage);
  }
}

template <int C>
__global__ void __launch_bounds__(kConvThreads) conv_kernel(ConvArgs a) {
  const int task = __builtin_amdgcn_readfirstlane(int(blockIdx.x) * kConvWaves + int(threadIdx.x) / kWave);
  if (task >= a.total_tasks) return;
  // the wave's group: last g with g_start[g] <= task (unrolled, kernel-argument reads)
  int g_base = 0, g_first = 0, g_nj = 1, lg = 0;
#pragma unroll
  for (int g = 0; g < kMaxGroupsPerLaunch; ++g) {
    if (g < a.n_groups && task >= a.g_start[g]) {
      g_base = a.g_start[g];
      g_first = a.g_first_job[g];
      g_nj = a.g_n_jobs[g];
      lg = a.g_lanes_log2[g];
    }
  }
  const int r = task - g_base;
  const int ng = r / g_nj;                     // node group
  const Job J = a.jobs[g_first + (r - ng * g_nj)];
  const int lane = int(threadIdx.x) & (kWave - 1);
  const int sg = min(a.edge_slots_log2, 6 - lg);
  const int node_pos = (ng << (6 - lg - sg)) + (lane >> (lg + sg));
  __shared__ int2 stage[kConvWaves][kStageEntries];
  dispatch<C, 0, kNumVariants>(J.variant, a, J, node_pos, lane, lg, sg, stage[threadIdx.x / kWave]);
}

}  // namespace

template <int C>
hipError_t launch_conv_class(const ConvArgs& args, hipStream_t s, hipEvent_t ev_start, hipEvent_t ev_stop) {
  if (args.total_tasks <= 0) return hipSuccess;
  const int blocks = ceil_div(args.total_tasks, kConvWaves);
  if (ev_start || ev_stop) {
    // the events are stamped by the dispatch itself: kernel time without launch gaps
    hipExtLaunchKernelGGL(conv_kernel<C>, dim3(blocks), dim3(kConvThreads), 0, s, ev_start, ev_stop, 0, args);
  } else {
    conv_kernel<C><<<blocks, kConvThreads, 0, s>>>(args);
  }
  return hipGetLastError();
}

}  // namespace cgtp
