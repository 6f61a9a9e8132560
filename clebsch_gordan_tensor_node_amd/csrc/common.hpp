// Shared definitions of libcgtp: wave-job descriptor, kernel argument blocks and
// small helpers used by the host plan and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "cg_real.hpp"

namespace cgtp {

constexpr int kWave = 64;            // CDNA wavefront width
constexpr int kMaxShL = kMaxL;       // harmonics up to l = 6

// One wave job: a path p and a block of its channels.  2^lanes_log2 lanes serve one
// receiver, each lane owning K consecutive channels, so one wave covers
// S = 64 / 2^lanes_log2 receivers of the degree-sorted order.  (LunaTP Figure 3(b):
// paths mapped to SIMD lanes by channel block; sized to the 64-lane wavefront.)
struct Job {
  int32_t variant;     // index of the (l1, l2, l3, K) specialisation
  int32_t lanes_log2;  // log2 of the lanes serving one receiver (<= 64)
  int32_t n_ch;      // channels in this job (multiple of K)
  int32_t in_off;    // float offset of the job's first channel in a row of x
  int32_t out_off;   // float offset of the job's first channel in a row of out
  int32_t w_off;     // column of w of the job's first channel
  int32_t sh_off;    // offset of Y_{l2} in a row of the SH table (= l2*l2)
  int32_t path;      // path index (diagnostics)
};
static_assert(sizeof(Job) == 32, "Job is 32 bytes");

// A group: jobs of one input irrep, one channel block, one K and one kernel class, run by
// one workgroup per node group: one consumer wave per job and one producer wave (the
// workgroup's last).  The jobs read the same x_j rows and the same harmonics, which the
// producer gathers once per edge step into LDS (LunaTP Table 8: cross-path input reuse);
// each consumer streams only its own path's weights.  The forward's groups hold up to
// kConvJobsFwd jobs; the backward's edge pass, whose LDS also carries the jobs'
// x-gradient hand-off, up to kConvJobsBwd.
constexpr int kConvJobsFwd = 7;
constexpr int kConvJobsBwd = 3;
constexpr int kConvWavesMax = kConvJobsFwd + 1;
struct Group {
  int32_t first_job;   // index into the schedule's job table
  int32_t n_jobs;      // 1 .. jobs per group of the schedule
  int32_t lanes_log2;  // lanes per receiver, common to the jobs
  int32_t y0;          // first harmonic (float offset in an SH row, multiple of 4) staged
  int32_t y4;          // 16-byte chunks of harmonics staged per receiver
};

// Groups of one launch, carried in the kernel arguments.  Workgroups come in blocks of
// 64 / 2^blk_lg_min consecutive receivers of the degree order; a block holds
// 2^(lanes_log2 - blk_lg_min) workgroups of each group.  A workgroup counts the groups
// whose range starts at or before it in g_start (two wide scalar loads, no dependent
// loads), then reads its group's record with one more.
constexpr int kMaxGroupsPerLaunch = 32;
constexpr int kXcds = 8;   // accelerator dies of an MI355X, each with its own L2

struct alignas(32) GroupArgs {
  int32_t start;       // first workgroup of the group inside a block
  int32_t first_job;
  int32_t n_jobs;
  int32_t lanes_log2;
  int32_t y0;
  int32_t y4;
  int32_t pad[2];
};

template <typename T>
struct ConvArgsT {
  const T* x;
  const T* w;
  const T* sh;                // harmonics of active edges, compacted within each row
  const int4* node_info;      // per order position: {node, row_ptr[node], active degree, 0}
  const int32_t* act_e;       // active edge ids, compacted within each row (at row_ptr[i] + q)
  const int32_t* act_j;       // their senders
  T* out;
  const Job* jobs;            // the plan's job table
  // backward edge pass only (else null): dL/d out, dL/dw, and rows of per-slot partials
  // [active slot, part_stride]: job j's dL/dY block at job_gy[j] (written when gyp is
  // set) and the x-gradient block of j's group at job_xg[j] (written when xgp is set;
  // gyp and xgp both point at the rows); a scratch row for lanes with nothing to store
  const T* grad_out;
  T* grad_w;
  T* gyp;
  T* xgp;
  const int32_t* job_gy;
  const int32_t* job_xg;
  T* scratch_row;
  int32_t part_stride;
  int32_t n_waves;            // waves of a workgroup of this launch (consumers + producer)
  int32_t n_nodes;
  int32_t f_in;
  int32_t f_out;
  int32_t w_stride;
  int32_t sh_stride;          // elements per SH row (a multiple of 16 / sizeof(T))
  int32_t n_groups;           // groups of this launch (<= kMaxGroupsPerLaunch)
  int32_t total_wgs;          // workgroups of this launch (whole blocks)
  int32_t blk_wgs;            // workgroups per block of 64 / 2^blk_lg_min receivers
  int32_t blk_lg_min;         // smallest lanes_log2 of the launch's groups
  int32_t n_blocks;           // receiver blocks (workgroup b of block k runs on XCD k mod kXcds)
  int32_t g_start[kMaxGroupsPerLaunch];       // first workgroup of each group inside a block
                                              // (INT32_MAX past the launch's groups)
  GroupArgs grp[kMaxGroupsPerLaunch];
};
using ConvArgs = ConvArgsT<float>;
// fp64 is built for the variants with l <= kF64Lmax: the kernel classes below
// kNumClassesF64 (l <= 2, l <= 3, and l1 = 0 .. kF64Lmax of the l >= 4 classes)
constexpr int kF64Lmax = 4;
constexpr int kNumClassesF64 = 3 + kF64Lmax;

// Arguments of the backward kernels (fp32).  Active slots are those of the forward's
// per-row pass: slot row_ptr[i] + q for the q-th active edge of row i.
struct BwdArgs {
  const float* pos;
  const int32_t* row_ptr;
  const int8_t* shift;
  const float* gate;
  const int32_t* deg;         // active edges per row
  const int32_t* act_e;       // edge id per active slot
  const int32_t* act_j;       // sender per active slot
  const int32_t* t_row_ptr;   // active slots grouped by sender
  const int32_t* t_slot;
  const int32_t* t_recv;
  const float* part;          // [slot, part_stride] the edge pass's partials
  const int32_t* xcol_ptr;    // per column c of x: its x-gradient blocks' entries in a row
  const int32_t* xcol_off;    //   of partials, xcol_off[xcol_ptr[c] .. xcol_ptr[c + 1])
  const int32_t* ycol_ptr;    // per harmonic component m: its dL/dY entries in a row,
  const int32_t* ycol_off;    //   ycol_off[ycol_ptr[m] .. ycol_ptr[m + 1])
  float* grad_x;
  float* grad_r;              // [slot, 3] dL/dr
  float* grad_pos;
  int32_t n_nodes, f_in, part_stride, l_sh_max;
  int32_t want_gy, has_cell;
  double cell[9];
};

__host__ __device__ constexpr int ceil_div(int a, int b) { return (a + b - 1) / b; }

}  // namespace cgtp
