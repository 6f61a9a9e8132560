// Shared definitions of libcgtp: wave-job descriptor, kernel argument blocks and
// small helpers used by the host plan and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "cg_real.hpp"

namespace cgtp {

constexpr int kWave = 64;            // CDNA wavefront width
constexpr int kMaxShL = kMaxL;       // harmonics up to l = 6

// One wave job: a path p and a block of its channels.  A wave runs one job for S
// consecutive nodes of the degree-sorted node order; 2^lanes_log2 lanes
// serve one node, each lane owning K consecutive channels.  (LunaTP Figure 3(b): paths
// mapped to SIMD lanes by channel block; here sized to the 64-lane wavefront.)
struct Job {
  int32_t variant;     // index of the (l1, l2, l3, K) specialisation
  int32_t lanes_log2;  // log2 of the lanes serving one node (lanes <= 64)
  int32_t n_ch;      // channels in this job (multiple of K)
  int32_t in_off;    // float offset of the job's first channel in a row of x
  int32_t out_off;   // float offset of the job's first channel in a row of out
  int32_t w_off;     // column of w of the job's first channel
  int32_t sh_off;    // offset of Y_{l2} in a row of the SH table (= l2*l2)
  int32_t path;      // path index (diagnostics)
};
static_assert(sizeof(Job) == 32, "Job is 32 bytes");

struct ConvArgs {
  const float* x;
  const float* w;
  const float* sh;
  const int32_t* act_row_ptr;
  const int32_t* act_eid;
  const int32_t* act_col;
  const int32_t* order;
  const int32_t* task_start;  // [n_jobs + 1] prefix of wave tasks per job (device)
  float* out;
  const Job* jobs;            // first job of this launch
  int32_t n_nodes;
  int32_t f_in;
  int32_t f_out;
  int32_t w_stride;
  int32_t sh_stride;
  int32_t n_jobs;
  int32_t total_tasks;
  int32_t pad;
};

__host__ __device__ constexpr int ceil_div(int a, int b) { return (a + b - 1) / b; }

}  // namespace cgtp
