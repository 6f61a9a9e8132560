// The fused node-centric CGTP convolution kernel.
//
// LunaTP ("Enabling Efficient and Scalable Tensor Product for Equivariant MLIPs")
// Figure 3: (a) node-centric execution sums the messages of all incoming edges on chip
// and stores each output once; (b) paths are grouped and mapped to SIMD lanes by
// channel block; (c) products are reused and equal coefficients factored.  This is
// the gfx950 design, not a translation:
//   * a wave (64 lanes) runs one job = (path, channel block) for S = 64 / lanes
//     consecutive receivers of the degree-sorted node order (LunaTP Table 9: descending
//     degree first); `lanes` lanes serve one receiver and each lane owns K channels;
//   * the path is a compile-time specialisation: the real CG coefficients and their
//     sparsity are constants, so A[m1,m3] = sum_m2 C[m1,m2,m3] Y[m2] is a short FMA
//     chain with immediate coefficients and structural zeros removed;
//   * per edge a lane loads its K weights (one 16-byte load when K = 4), its K x_j
//     channel vectors and the edge's Y_l2, forms A once, and applies it to its K
//     channels: acc[k,m3] += w[k] * sum_m1 A[m1,m3] x[k,m1], scaling whichever side
//     (x or the partial result) is shorter;
//   * accumulators live in VGPRs for the whole edge loop; one coalesced store per
//     receiver and channel block at the end.  No atomics: the result is bitwise
//     reproducible.
// The uvu coupling is not a dense contraction, so no MFMA is used.
//
// This header is compiled once per kernel class (kernels_conv.hip with
// CGTP_CONV_CLASS = 0 .. kNumClasses-1); each build instantiates one conv_kernel.
#pragma once

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

template <int L1, int L2, int L3, int K>
__device__ __forceinline__ void run_job(const ConvArgs& a, const Job& J, int node_pos, int t) {
  constexpr int N1 = 2 * L1 + 1, N2 = 2 * L2 + 1, N3 = 2 * L3 + 1;
  const int ch0 = t * K;
  const bool ok = (node_pos < a.n_nodes) && (ch0 < J.n_ch);
  int i = 0, e_beg = 0, e_end = 0;
  if (ok) {
    i = a.order[node_pos];
    e_beg = a.act_row_ptr[i];
    e_end = a.act_row_ptr[i + 1];
  }
  float acc[K * N3];
#pragma unroll
  for (int q = 0; q < K * N3; ++q) acc[q] = 0.0f;

  const float* __restrict__ xb = a.x + J.in_off + ch0 * N1;
  const float* __restrict__ wb = a.w + J.w_off + ch0;
  const float* __restrict__ shb = a.sh + J.sh_off;

  for (int e = e_beg; e < e_end; ++e) {
    const int eid = a.act_eid[e];
    const int j = a.act_col[e];
    float Y[N2];
    const float* ys = shb + (long)e * a.sh_stride;
#pragma unroll
    for (int q = 0; q < N2; ++q) Y[q] = ys[q];
    float xv[K * N1];
    load_run<K, K * N1>(xb + (long)j * a.f_in, xv);
    float wv[K];
    load_k<K>(wb + (long)eid * a.w_stride, wv);

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
  if (ok) store_run<K, K * N3>(a.out + (long)i * a.f_out + J.out_off + ch0 * N3, acc);
}

template <int C, int LO, int HI>
__device__ __forceinline__ void dispatch(int v, const ConvArgs& a, const Job& J, int node_pos, int t) {
  if constexpr (HI - LO == 1) {
    if constexpr (variant_class(LO) == C) {
      constexpr VariantDesc d = variant_desc(LO);
      run_job<d.l1, d.l2, d.l3, d.k>(a, J, node_pos, t);
    }
  } else {
    constexpr int MID = (LO + HI) / 2;
    if (v < MID)
      dispatch<C, LO, MID>(v, a, J, node_pos, t);
    else
      dispatch<C, MID, HI>(v, a, J, node_pos, t);
  }
}

template <int C>
__global__ void __launch_bounds__(kConvThreads) conv_kernel(ConvArgs a) {
  const int task = __builtin_amdgcn_readfirstlane(int(blockIdx.x) * kConvWaves + int(threadIdx.x) / kWave);
  if (task >= a.total_tasks) return;
  // task_start holds the prefix over all jobs of the plan; this launch starts at ts[0]
  const int32_t* __restrict__ ts = a.task_start;
  const int t0 = ts[0];
  int lo = 0, hi = a.n_jobs;  // last job whose first task is <= task
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (ts[mid] - t0 <= task) lo = mid; else hi = mid;
  }
  const Job J = a.jobs[lo];
  const int lane = int(threadIdx.x) & (kWave - 1);
  const int lg = J.lanes_log2;
  const int slot = lane >> lg;
  const int t = lane & ((1 << lg) - 1);
  const int node_pos = ((task - (ts[lo] - t0)) << (6 - lg)) + slot;
  dispatch<C, 0, kNumVariants>(J.variant, a, J, node_pos, t);
}

}  // namespace

template <int C>
hipError_t launch_conv_class(const ConvArgs& args, hipStream_t s) {
  if (args.total_tasks <= 0) return hipSuccess;
  const int blocks = ceil_div(args.total_tasks, kConvWaves);
  conv_kernel<C><<<blocks, kConvThreads, 0, s>>>(args);
  return hipGetLastError();
}

}  // namespace cgtp
