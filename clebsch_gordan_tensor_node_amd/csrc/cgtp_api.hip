// C ABI of libcgtp (declared in include/cgtp.h): plan construction (irreps parser,
// path enumerator, real-CG tables, wave-job scheduler), argument validation and the
// launch sequence of the neighbour list, mask prepare, edge harmonics and the fused
// convolution.  No allocation happens outside cgtp_plan_create.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/cgtp.h"
#include "launch.hpp"
#include "nbr.hpp"
#include "variants.hpp"

namespace cgtp {
namespace {

thread_local std::string g_last_error;

// CGTP_LOG in the environment: 1 copies every failing call's message to stderr, 2 adds
// a line per created plan (paths, jobs, groups, launches and their streams).
int log_level() {
  static const int level = [] {
    const char* e = std::getenv("CGTP_LOG");
    return e ? std::atoi(e) : 0;
  }();
  return level;
}

void log_line(int level, const char* fmt, ...) {
  if (log_level() < level) return;
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  std::fprintf(stderr, "cgtp: %s\n", buf);
}

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  log_line(1, "error %d: %s", code, buf);
  return code;
}

int ok() {
  g_last_error.clear();
  return CGTP_OK;
}

#define CGTP_HIP(call)                                                                  \
  do {                                                                                  \
    hipError_t e_ = (call);                                                             \
    if (e_ != hipSuccess) return fail(CGTP_ERR_HIP, "%s: %s", #call, hipGetErrorString(e_)); \
  } while (0)

struct Irrep {
  int mul, l, p;
};

struct PathInfo {
  int l1, p1, l2, p2, l3, p3, mul, i_in, i_sh, in_off, out_off, w_off;
};

// Parse "128x0e+64x1o" (a bare "1o" means multiplicity 1).
bool parse_irreps(const char* spec, std::vector<Irrep>& out, std::string& err) {
  out.clear();
  if (!spec || !*spec) {
    err = "empty irreps spec";
    return false;
  }
  std::string s;
  for (const char* c = spec; *c; ++c)
    if (*c != ' ') s.push_back(*c);
  size_t pos = 0;
  while (true) {
    size_t plus = s.find('+', pos);
    std::string term = s.substr(pos, plus == std::string::npos ? std::string::npos : plus - pos);
    if (term.empty()) {
      err = "empty term in '" + s + "'";
      return false;
    }
    long mul = 1;
    std::string ir = term;
    size_t x = term.find('x');
    if (x != std::string::npos) {
      std::string m = term.substr(0, x);
      if (m.empty() || m.find_first_not_of("0123456789") != std::string::npos || m.size() > 9) {
        err = "bad multiplicity in '" + term + "'";
        return false;
      }
      mul = std::stol(m);
      ir = term.substr(x + 1);
    }
    if (ir.size() < 2 || (ir.back() != 'e' && ir.back() != 'o')) {
      err = "bad irrep '" + term + "'";
      return false;
    }
    std::string ls = ir.substr(0, ir.size() - 1);
    if (ls.empty() || ls.find_first_not_of("0123456789") != std::string::npos || ls.size() > 4) {
      err = "bad irrep '" + term + "'";
      return false;
    }
    out.push_back(Irrep{int(mul), std::stoi(ls), ir.back() == 'e' ? 1 : -1});
    if (plus == std::string::npos) break;
    pos = plus + 1;
  }
  return true;
}

std::string format_irreps(const std::vector<Irrep>& v) {
  std::string s;
  for (size_t k = 0; k < v.size(); ++k) {
    if (k) s += "+";
    s += std::to_string(v[k].mul) + "x" + std::to_string(v[k].l) + (v[k].p == 1 ? "e" : "o");
  }
  return s;
}

int sign_pow(int l) { return (l % 2 == 0) ? 1 : -1; }

// Real CG of a path as a dense fp32 table (run-time evaluation of the same
// constexpr formulas the kernels are specialised with).
void dense_cg(int l1, int l2, int l3, std::vector<float>& out) {
  const int n1 = 2 * l1 + 1, n2 = 2 * l2 + 1, n3 = 2 * l3 + 1;
  out.assign(size_t(n1) * n2 * n3, 0.0f);
  for (int a = 0; a < n1; ++a)
    for (int b = 0; b < n2; ++b)
      for (int c = 0; c < n3; ++c) {
        double v = real_cg(l1, l2, l3, a - l1, b - l2, c - l3);
        if (v < 1e-12 && v > -1e-12) v = 0.0;
        out[(size_t(a) * n2 + b) * n3 + c] = float(v);
      }
}

int next_pow2(int v) {
  int p = 1;
  while (p < v) p <<= 1;
  return p;
}
int ilog2(int v) {
  int r = 0;
  while ((1 << r) < v) ++r;
  return r;
}

}  // namespace
}  // namespace cgtp

using namespace cgtp;

// streams a plan may add beside the caller's: with it, four, the hardware queues a
// process gets by default
constexpr int kAuxStreams = 3;

// Launches of the fused conv kernel: a kernel class, a range of its groups and the
// workgroup's waves (its largest group's jobs plus the producer).  Launches write disjoint
// output columns and only read the inputs, so the forward spreads them over the caller's
// stream (stream 0) and up to kAuxStreams streams of the plan (stream k = aux stream
// k - 1), forked from and joined back into the caller's stream by events; the small
// latency-bound launches of the l >= 4 classes then run beside the large one.
struct ConvLaunch {
  int cls, g0, g1, stream, waves;
};
// per group: its heaviest job's cost (per-step work of a lane), its work (cost times
// lanes, summed over its jobs) and its weight columns
struct GroupLoad {
  double max_cost, work, cols;
};
// One schedule of the plan's jobs into groups of at most jobs_per_group[class] jobs: the
// forward's and the backward's edge pass's (at most kConvJobsBwd: the jobs whose
// x-gradients its LDS hand-off adds).  In the forward the l <= 3 class (class 1) takes
// groups of up to kConvJobsFwd jobs, so that one producer wave gathers each sender's
// x_j segment (up to 7 components per channel) for all paths of its input irrep; the
// other classes (and the fp64 forward) keep groups of kConvJobsBwd, as more and smaller
// workgroups measured faster there.  Conv kernel time, groups of 3 against groups of 7: c1_768 (l <= 2)
// 27.1 against 28.0 us; highl_768 (mostly the l >= 4 classes, whose few hundred
// workgroups are bound by their arithmetic and edge chains) 414 against 470 us; for
// l <= 3, c2_768 56.2 against 51.3 us and si_mask 108.3 against 105.0 us.
struct Schedule {
  int jobs_per_group[kNumClasses] = {};
  bool balance_simds = false;        // jobs of a group placed for SIMD balance (the forward)
  std::vector<Job> jobs;             // ordered by group
  std::vector<Group> groups;         // by kernel class, heavy groups first
  std::vector<int> class_begin;      // [kNumClasses + 1] first group of each class
  std::vector<GroupLoad> group_load;
  std::vector<ConvLaunch> launches;  // in enqueue order
  int n_variants = 0;
  int n_aux = 0;                     // streams beside the caller's that the launches use
  Job* d_jobs = nullptr;             // device copy of jobs
};

struct cgtp_plan_s {
  std::vector<Irrep> in, sh, out;
  std::vector<PathInfo> paths;
  int64_t f_in = 0, f_out = 0, w = 0;
  int l_sh_max = 0;
  int sh_stride = 1;                 // floats per SH row of cgtp_edge_sh: (l_sh_max + 1)^2
  int sh_pad = 4;                    // elements per SH row of the forward workspace (16-byte rows)
  int elem = 4;                      // bytes per element of x, w, out and the workspace SH
  std::string irreps_out;
  Schedule fwd, bwd;                 // the forward's and the backward edge pass's schedules
  bool host_only = true;
  int device = -1;
  void* d_tables = nullptr;          // device copy of the job tables and the backward tables
  int lmax = 0;                      // largest l of the plan
  // backward tables.  A row of the edge pass's partials (one per active slot) holds
  // [each job's dL/dY block (2 l2 + 1, job order) | padding to 4 | each group's
  // x-gradient block (n_ch (2 l1 + 1) in x's layout, padded to 4; group order)], jobs
  // and groups of the backward's schedule;
  // job_gy / job_xg give each job's block (a group's jobs share one x-gradient block).
  // xcol: per column of x, the row entries of the blocks that read it (CSR, group
  // order); ycol: per harmonic component, the entries of its jobs' dL/dY (job order).
  int part_stride = 0;
  std::vector<int32_t> job_gy, job_xg, xcol_ptr, xcol_off, ycol_ptr, ycol_off;
  int32_t *d_job_gy = nullptr, *d_job_xg = nullptr;
  int32_t *d_xcol_ptr = nullptr, *d_xcol_off = nullptr, *d_ycol_ptr = nullptr, *d_ycol_off = nullptr;
  hipStream_t aux[kAuxStreams] = {};   // the forward's streams beside the caller's
  hipEvent_t fork = nullptr;
  hipEvent_t join[kAuxStreams] = {};
  // the backward's side stream (fp32 plans with l <= kBwdLmax): the zeroing of inactive
  // w-gradient rows and the grouping of slots by sender run on it beside the edge pass
  hipStream_t bwd_side = nullptr;
  hipEvent_t bwd_ev[2] = {};
  std::mutex enqueue;                // held while a forward or backward forks, launches and joins
};

namespace {

// Job schedule.  Per path: K = 4 channels per lane when every offset and stride is
// 16-byte aligned, else K = 1; lanes per receiver = next power of two of mul/K, at most
// 64 (larger multiplicities are cut into channel blocks of 64*K).  Jobs of one kernel
// class, input irrep, channel block and K form a set that shares x_j rows; each set is
// cut into groups of at most S.jobs_per_group[class] jobs, one workgroup per group and
// node group.
// Jobs keep their weight-column order inside a set (the forward's schedule then places
// a group's jobs on waves for SIMD balance, below); groups are ordered heaviest first inside a class
// (LunaTP Table 9: ordering by descending CG-term count was fastest).
void schedule(const cgtp_plan_s& P, Schedule& S) {
  S.jobs.clear();
  struct Tmp {
    Job j;
    int cls, irrep, block, l2;
    double cost;
  };
  std::vector<Tmp> tmp;
  std::vector<int> used(kNumVariants, 0);
  const int VE = 16 / P.elem;        // elements per 16-byte access
  const bool strides4 = (P.f_in % VE == 0) && (P.f_out % VE == 0) && (P.w % VE == 0);
  int plan_lmax = 0;
  for (const PathInfo& p : P.paths) plan_lmax = std::max(plan_lmax, std::max(p.l1, std::max(p.l2, p.l3)));
  for (size_t pi = 0; pi < P.paths.size(); ++pi) {
    const PathInfo& p = P.paths[pi];
    const bool al = strides4 && p.mul % VE == 0 && p.in_off % VE == 0 && p.out_off % VE == 0 && p.w_off % VE == 0;
    const int K = al ? VE : 1;
    const int v = variant_index(p.l1, p.l2, p.l3, al ? 4 : 1);   // the vector or the scalar form
    const int cls = job_class(v, plan_lmax);
    used[v] = 1;
    std::vector<float> cg;
    dense_cg(p.l1, p.l2, p.l3, cg);
    const int n1 = 2 * p.l1 + 1, n2 = 2 * p.l2 + 1, n3 = 2 * p.l3 + 1;
    int nnz_c = 0, nnz_a = 0;
    for (int a = 0; a < n1; ++a)
      for (int c = 0; c < n3; ++c) {
        bool any = false;
        for (int b = 0; b < n2; ++b)
          if (cg[(size_t(a) * n2 + b) * n3 + c] != 0.0f) {
            ++nnz_c;
            any = true;
          }
        nnz_a += any;
      }
    const double cost = nnz_c + K * (nnz_a + std::min(n1, n3));
    const int block = 64 * K;
    for (int c0 = 0; c0 < p.mul; c0 += block) {
      const int n_ch = std::min(block, p.mul - c0);
      const int lanes = next_pow2((n_ch + K - 1) / K);
      Job j{};
      j.variant = v;
      j.lanes_log2 = ilog2(lanes);
      j.n_ch = n_ch;
      j.in_off = p.in_off + c0 * n1;
      j.out_off = p.out_off + c0 * n3;
      j.w_off = p.w_off + c0;
      j.sh_off = p.l2 * p.l2;
      j.path = int(pi);
      tmp.push_back(Tmp{j, cls, p.i_in, c0, p.l2, cost});
    }
  }
  // sets of jobs sharing (class, input irrep, channel block, K)
  auto key_less = [&](const Tmp& x, const Tmp& y) {
    if (x.cls != y.cls) return x.cls < y.cls;
    if (x.irrep != y.irrep) return x.irrep < y.irrep;
    if (x.block != y.block) return x.block < y.block;
    const int kx = variant_desc(x.j.variant).k, ky = variant_desc(y.j.variant).k;
    if (kx != ky) return kx < ky;
    return x.j.w_off < y.j.w_off;   // weight-column order inside a set
  };
  std::stable_sort(tmp.begin(), tmp.end(), key_less);
  struct G {
    int cls, begin, n;
    double cost;
  };
  std::vector<G> gs;
  for (size_t b = 0; b < tmp.size();) {
    size_t e = b + 1;
    while (e < tmp.size() && tmp[b].cls == tmp[e].cls && tmp[b].irrep == tmp[e].irrep &&
           tmp[b].block == tmp[e].block && variant_desc(tmp[b].j.variant).k == variant_desc(tmp[e].j.variant).k)
      ++e;
    // cut the set [b, e) into ceil(n / jobs_per_group) groups of balanced size
    // large groups only where a workgroup serves several receivers (fewer than 64 lanes
    // per receiver): with one receiver per workgroup its chain is that receiver's whole
    // edge list, which more and smaller groups shorten (c4_768, 256 channels: 141.5
    // against 151.2 us)
    const int jpg = tmp[b].j.lanes_log2 < 6 ? S.jobs_per_group[tmp[b].cls] : kConvJobsBwd;
    const int n = int(e - b), ng = (n + jpg - 1) / jpg;
    int at = int(b);
    for (int g = 0; g < ng; ++g) {
      const int sz = n / ng + (g < n % ng ? 1 : 0);
      double c = 0.0;
      for (int k = at; k < at + sz; ++k) c = std::max(c, tmp[k].cost);
      gs.push_back(G{tmp[b].cls, at, sz, c});
      at += sz;
    }
    b = e;
  }
  std::stable_sort(gs.begin(), gs.end(), [](const G& x, const G& y) {
    if (x.cls != y.cls) return x.cls < y.cls;
    return x.cost > y.cost;
  });
  S.groups.clear();
  S.group_load.clear();
  S.class_begin.assign(kNumClasses + 1, 0);
  std::vector<double> jcost;   // per job of S.jobs: its lane's work per edge step
  for (const G& g : gs) {
    Group G{};
    G.first_job = int(S.jobs.size());
    G.n_jobs = g.n;
    G.lanes_log2 = tmp[g.begin].j.lanes_log2;
    int l2lo = kMaxL, l2hi = 0;
    for (int k = g.begin; k < g.begin + g.n; ++k) {
      S.jobs.push_back(tmp[k].j);
      jcost.push_back(tmp[k].cost);
      l2lo = std::min(l2lo, tmp[k].l2);
      l2hi = std::max(l2hi, tmp[k].l2);
    }
    G.y0 = (l2lo * l2lo) / VE * VE;
    G.y4 = ((l2hi + 1) * (l2hi + 1) - G.y0 + VE - 1) / VE;
    // at least y4 lanes per receiver, so that the S y4 harmonic chunks of a step fit the
    // producer wave's 64 lanes (extra lanes idle)
    G.lanes_log2 = std::max(G.lanes_log2, ilog2(next_pow2(G.y4)));
    for (int k = G.first_job; k < G.first_job + G.n_jobs; ++k) S.jobs[k].lanes_log2 = G.lanes_log2;
    S.groups.push_back(G);
    double work = 0.0, cols = 0.0;
    for (int k = g.begin; k < g.begin + g.n; ++k) {
      work += tmp[k].cost * tmp[k].j.n_ch / (64.0 * variant_desc(tmp[k].j.variant).k);
      cols += tmp[k].j.n_ch;
    }
    S.group_load.push_back({g.cost, work, cols});
    S.class_begin[g.cls + 1]++;
  }
  for (int c = 0; c < kNumClasses; ++c) S.class_begin[c + 1] += S.class_begin[c];
  S.n_variants = 0;
  for (int u : used) S.n_variants += u;

  // launches of up to kMaxGroupsPerLaunch groups of one class, spread over the streams
  // longest first onto the least loaded (the first, the longest, stays on the caller's
  // stream).  A launch's time is modelled as the largest of three bounds, in
  // microseconds for a graph of about 20 000 edges (only their ratios matter): the
  // receiver with the most edges walks them in sequence at a step time set by the
  // heaviest group, the arithmetic of all groups, and the weight stream.
  S.launches.clear();
  for (int c = 0; c < kNumClasses; ++c)
    for (int g0 = S.class_begin[c]; g0 < S.class_begin[c + 1]; g0 += kMaxGroupsPerLaunch)
      S.launches.push_back({c, g0, std::min(S.class_begin[c + 1], g0 + kMaxGroupsPerLaunch), 0, 0});
  for (ConvLaunch& L : S.launches) {
    int most = 1;
    for (int k = L.g0; k < L.g1; ++k) most = std::max(most, S.groups[k].n_jobs);
    L.waves = most + 1;
  }
  // SIMD balance.  A CU deals the waves of a workgroup to its four SIMDs in turn, so
  // waves w and w + 4 share a SIMD, and the producer (the last wave) shares one with a
  // consumer; every wave meets the others at each step's barrier, so a step lasts as
  // long as the busiest SIMD's waves.  The jobs of a group are placed heaviest first on
  // the least loaded SIMD that still has a consumer position (conv kernel time against
  // weight-column order: si_mask 104.9 -> 103.2 us, c5_768 147.5 -> 144.7, c2_768
  // 51.8 -> 51.5).  Only the forward's schedule is rearranged: the backward's tables
  // follow its own job order.
  if (S.balance_simds) {
    constexpr double kStepOverhead = 25.0;   // LDS reads, weight select and addressing
    for (const ConvLaunch& L : S.launches) {
      for (int k = L.g0; k < L.g1; ++k) {
        const Group& G = S.groups[k];
        if (G.n_jobs < 2 || L.waves <= 4) continue;
        const int n = G.n_jobs;
        const int l1 = variant_desc(S.jobs[G.first_job].variant).l1;
        double load[4] = {};
        load[(L.waves - 1) % 4] += 4.0 * (2 * l1 + 2);   // the producer's loads and stores
        std::vector<int> ord(n);
        for (int q = 0; q < n; ++q) ord[q] = q;
        std::stable_sort(ord.begin(), ord.end(), [&](int a, int b) {
          return jcost[G.first_job + a] > jcost[G.first_job + b];
        });
        std::vector<int> pos_of(n, -1);
        std::vector<char> used(n, 0);
        for (int q : ord) {
          int best = -1;
          for (int p = 0; p < n; ++p)
            if (!used[p] && (best < 0 || load[p % 4] < load[best % 4])) best = p;
          used[best] = 1;
          pos_of[q] = best;
          load[best % 4] += jcost[G.first_job + q] + kStepOverhead;
        }
        std::vector<Job> js(n);
        std::vector<double> cs(n);
        for (int q = 0; q < n; ++q) {
          js[pos_of[q]] = S.jobs[G.first_job + q];
          cs[pos_of[q]] = jcost[G.first_job + q];
        }
        for (int q = 0; q < n; ++q) {
          S.jobs[G.first_job + q] = js[q];
          jcost[G.first_job + q] = cs[q];
        }
      }
    }
  }
  std::vector<double> est(S.launches.size(), 0.0);
  for (size_t li = 0; li < S.launches.size(); ++li) {
    double chain = 0.0, work = 0.0, cols = 0.0;
    for (int k = S.launches[li].g0; k < S.launches[li].g1; ++k) {
      chain = std::max(chain, S.group_load[k].max_cost);
      work += S.group_load[k].work;
      cols += S.group_load[k].cols;
    }
    est[li] = std::max(10.0 + 0.075 * chain, std::max(0.072 * work, 0.026 * cols));
  }
  std::vector<int> ord(S.launches.size());
  for (size_t li = 0; li < ord.size(); ++li) ord[li] = int(li);
  std::stable_sort(ord.begin(), ord.end(), [&](int x, int y) { return est[x] > est[y]; });
  double load[kAuxStreams + 1] = {};
  std::vector<ConvLaunch> sorted;
  S.n_aux = 0;
  for (int li : ord) {
    int best = 0;
    for (int k = 1; k <= kAuxStreams; ++k)
      if (load[k] < load[best]) best = k;
    load[best] += est[li];
    ConvLaunch L = S.launches[li];
    L.stream = best;
    S.n_aux = std::max(S.n_aux, best);
    sorted.push_back(L);
  }
  S.launches = sorted;
}


size_t align256(size_t b) { return (b + 255) & ~size_t(255); }

// Workspace of the forward and of the exported prepare (one layout, 256-byte aligned
// sections): per-node degree, the position-indexed node records of the degree order,
// radix scratch, and the active edge ids, senders and harmonics compacted within each
// row.
struct FwdWorkspace {
  int32_t *deg, *tmp_a, *tmp_b, *act_e, *act_j;
  int4* node_info;
  void* sh;                          // [e, sh_pad] of the plan's element type
  size_t bytes;
};

FwdWorkspace carve(const cgtp_plan_s& P, int64_t n, int64_t e, void* base) {
  FwdWorkspace w{};
  char* p = static_cast<char*>(base);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    char* r = p ? p + off : nullptr;
    off += align256(bytes);
    return r;
  };
  w.deg = reinterpret_cast<int32_t*>(take(size_t(n) * 4));
  w.node_info = reinterpret_cast<int4*>(take(size_t(n) * 16));
  w.tmp_a = reinterpret_cast<int32_t*>(take(size_t(n) * 4));
  w.tmp_b = reinterpret_cast<int32_t*>(take(size_t(n) * 4));
  w.act_e = reinterpret_cast<int32_t*>(take(size_t(e) * 4));
  w.act_j = reinterpret_cast<int32_t*>(take(size_t(e) * 4));
  w.sh = take(size_t(e) * size_t(P.sh_pad) * size_t(P.elem));
  w.bytes = off;
  return w;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int check_device(const cgtp_plan_s* P) {
  int dev = -1;
  CGTP_HIP(hipGetDevice(&dev));
  if (dev != P->device) return fail(CGTP_ERR_INVALID_ARG, "plan was created on device %d, current device is %d", P->device, dev);
  return CGTP_OK;
}

const int kMaxInt32 = 0x7fffffff;

// frees a device plan's tables, streams and events (its device is current)
void release_device(cgtp_plan_s* P) {
  if (P->d_tables) (void)hipFree(P->d_tables);
  for (int k = 0; k < kAuxStreams; ++k) {
    if (P->aux[k]) (void)hipStreamDestroy(P->aux[k]);
    if (P->join[k]) (void)hipEventDestroy(P->join[k]);
  }
  if (P->fork) (void)hipEventDestroy(P->fork);
  if (P->bwd_side) (void)hipStreamDestroy(P->bwd_side);
  for (hipEvent_t ev : P->bwd_ev)
    if (ev) (void)hipEventDestroy(ev);
  P->d_tables = nullptr;
}

}  // namespace

extern "C" {

const char* cgtp_last_error(void) { return g_last_error.c_str(); }

const char* cgtp_version(void) { return "cgtp 0.1 gfx950"; }

int cgtp_plan_create(const char* irreps_in, const char* irreps_sh, int l_out_max, int path_rule,
                     unsigned flags, cgtp_plan_t* out) {
  if (!out) return fail(CGTP_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  if (path_rule != CGTP_PATHS_ALL && path_rule != CGTP_PATHS_PARITY)
    return fail(CGTP_ERR_INVALID_ARG, "unknown path rule %d", path_rule);
  if (flags & ~unsigned(CGTP_PLAN_HOST_ONLY | CGTP_PLAN_FP64))
    return fail(CGTP_ERR_INVALID_ARG, "unknown flags 0x%x", flags);
  if (l_out_max < 0) return fail(CGTP_ERR_INVALID_ARG, "l_out_max < 0");
  auto P = new cgtp_plan_s();
  std::string err;
  if (!parse_irreps(irreps_in, P->in, err) || !parse_irreps(irreps_sh, P->sh, err)) {
    delete P;
    return fail(CGTP_ERR_PARSE, "%s", err.c_str());
  }
  for (const Irrep& r : P->in)
    if (r.l > kMaxL || r.mul <= 0) {
      const Irrep bad = r;   // copied: r refers into the plan deleted below
      delete P;
      return fail(CGTP_ERR_UNSUPPORTED, "input irrep %dx%d: need l <= %d and mul > 0", bad.mul, bad.l, kMaxL);
    }
  for (const Irrep& r : P->sh)
    if (r.l > kMaxL || r.mul != 1) {
      const Irrep bad = r;
      delete P;
      return fail(CGTP_ERR_UNSUPPORTED, "edge SH irrep %dx%d: need l <= %d and multiplicity 1", bad.mul, bad.l,
                  kMaxL);
    }
  std::vector<int> in_off;
  int64_t off = 0;
  for (const Irrep& r : P->in) {
    in_off.push_back(int(off));
    off += int64_t(r.mul) * (2 * r.l + 1);
  }
  P->f_in = off;
  struct Raw {
    int l1, p1, l2, p2, l3, p3, mul, i_in, i_sh;
  };
  std::vector<Raw> raw;
  for (size_t a = 0; a < P->in.size(); ++a)
    for (size_t b = 0; b < P->sh.size(); ++b) {
      const Irrep &x = P->in[a], &y = P->sh[b];
      const int lo = std::abs(x.l - y.l), hi = std::min(x.l + y.l, l_out_max);
      for (int l3 = lo; l3 <= hi; ++l3) {
        const int p3 = x.p * y.p;
        if (path_rule == CGTP_PATHS_PARITY && p3 != sign_pow(l3)) continue;
        raw.push_back(Raw{x.l, x.p, y.l, y.p, l3, p3, x.mul, int(a), int(b)});
      }
    }
  if (raw.empty()) {
    delete P;
    return fail(CGTP_ERR_UNSUPPORTED, "no path survives the path rule");
  }
  // output irreps sorted by (l3, e before o); path blocks in path order
  std::vector<std::pair<int, int>> keys;
  for (const Raw& r : raw) keys.emplace_back(r.l3, r.p3 == 1 ? 0 : 1);
  std::sort(keys.begin(), keys.end());
  keys.erase(std::unique(keys.begin(), keys.end()), keys.end());
  std::vector<int> out_off(raw.size()), w_off(raw.size());
  int64_t fo = 0, ch = 0;
  for (auto& k : keys) {
    const int l3 = k.first, p3 = k.second == 0 ? 1 : -1;
    int64_t c_in = 0;
    for (size_t q = 0; q < raw.size(); ++q)
      if (raw[q].l3 == l3 && raw[q].p3 == p3) {
        out_off[q] = int(fo + c_in * (2 * l3 + 1));
        w_off[q] = int(ch + c_in);
        c_in += raw[q].mul;
      }
    P->out.push_back(Irrep{int(c_in), l3, p3});
    fo += c_in * (2 * l3 + 1);
    ch += c_in;
  }
  P->f_out = fo;
  P->w = ch;
  if (P->f_in > kMaxInt32 || P->f_out > kMaxInt32) {
    delete P;
    return fail(CGTP_ERR_UNSUPPORTED, "feature width exceeds int32");
  }
  for (size_t q = 0; q < raw.size(); ++q) {
    const Raw& r = raw[q];
    P->paths.push_back(PathInfo{r.l1, r.p1, r.l2, r.p2, r.l3, r.p3, r.mul, r.i_in, r.i_sh, in_off[r.i_in],
                                out_off[q], w_off[q]});
  }
  P->l_sh_max = 0;
  for (const Irrep& r : P->sh) P->l_sh_max = std::max(P->l_sh_max, r.l);
  P->sh_stride = (P->l_sh_max + 1) * (P->l_sh_max + 1);
  P->elem = (flags & CGTP_PLAN_FP64) ? 8 : 4;
  P->sh_pad = (P->sh_stride + 16 / P->elem - 1) / (16 / P->elem) * (16 / P->elem);
  if (P->elem == 8) {
    int lmax = 0;
    for (const PathInfo& p : P->paths) lmax = std::max(lmax, std::max(p.l1, std::max(p.l2, p.l3)));
    if (lmax > kF64Lmax) {
      delete P;
      return fail(CGTP_ERR_UNSUPPORTED, "fp64 plans support l <= %d (this plan reaches l = %d)", kF64Lmax, lmax);
    }
  }
  P->irreps_out = format_irreps(P->out);
  for (int c = 0; c < kNumClasses; ++c) {
    // groups of 7 for the fp32 l <= 3 class only: in fp64 (K = 2, twice the lanes per
    // channel block) groups of 3 measured faster (si_mask conv 231 -> 205 us, c5_768
    // 247 -> 233 us; c2_768 unchanged)
    P->fwd.jobs_per_group[c] = c == 1 && P->elem == 4 ? kConvJobsFwd : kConvJobsBwd;
    P->bwd.jobs_per_group[c] = kConvJobsBwd;
  }
  P->fwd.balance_simds = true;
  schedule(*P, P->fwd);
  schedule(*P, P->bwd);
  // backward tables
  P->lmax = 0;
  for (const PathInfo& p : P->paths) P->lmax = std::max(P->lmax, std::max(p.l1, std::max(p.l2, p.l3)));
  {
    auto pad4 = [](int v) { return (v + 3) & ~3; };
    int at = 0;
    const Schedule& B = P->bwd;
    for (const Job& j : B.jobs) {
      P->job_gy.push_back(at);
      at += 2 * variant_desc(j.variant).l2 + 1;
    }
    at = pad4(at);
    P->job_xg.assign(B.jobs.size(), 0);
    std::vector<std::vector<int32_t>> xcover(size_t(P->f_in)), ycover(size_t(P->sh_stride));
    for (const Group& G : B.groups) {
      const Job& J = B.jobs[G.first_job];
      const int n1 = 2 * variant_desc(J.variant).l1 + 1, len = J.n_ch * n1;
      for (int k = G.first_job; k < G.first_job + G.n_jobs; ++k) P->job_xg[k] = at;
      for (int c = 0; c < len; ++c) xcover[size_t(J.in_off + c)].push_back(at + c);
      at += pad4(len);
    }
    P->part_stride = at;
    for (size_t k = 0; k < B.jobs.size(); ++k) {
      const int l2 = variant_desc(B.jobs[k].variant).l2;
      for (int m = 0; m < 2 * l2 + 1; ++m) ycover[size_t(l2 * l2 + m)].push_back(P->job_gy[k] + m);
    }
    auto flatten = [](const std::vector<std::vector<int32_t>>& cov, std::vector<int32_t>& ptr,
                      std::vector<int32_t>& off) {
      ptr.assign(1, 0);
      for (const auto& v : cov) {
        off.insert(off.end(), v.begin(), v.end());
        ptr.push_back(int32_t(off.size()));
      }
    };
    flatten(xcover, P->xcol_ptr, P->xcol_off);
    flatten(ycover, P->ycol_ptr, P->ycol_off);
  }

  P->host_only = (flags & CGTP_PLAN_HOST_ONLY) != 0;
  if (!P->host_only) {
    int ndev = 0;
    if (hipGetDeviceCount(&ndev) != hipSuccess || ndev <= 0) {
      delete P;
      return fail(CGTP_ERR_NO_DEVICE, "no HIP device");
    }
    int dev = 0;
    hipDeviceProp_t prop;
    if (hipGetDevice(&dev) != hipSuccess || hipGetDeviceProperties(&prop, dev) != hipSuccess ||
        std::strncmp(prop.gcnArchName, "gfx950", 6) != 0) {
      delete P;
      return fail(CGTP_ERR_NO_DEVICE, "current device is not gfx950");
    }
    P->device = dev;
    // one allocation: the two job tables, then the backward tables, each 256-byte aligned
    const std::vector<int32_t>* tabs[] = {&P->job_gy, &P->job_xg, &P->xcol_ptr, &P->xcol_off, &P->ycol_ptr,
                                          &P->ycol_off};
    int32_t** dtabs[] = {&P->d_job_gy, &P->d_job_xg, &P->d_xcol_ptr, &P->d_xcol_off, &P->d_ycol_ptr,
                         &P->d_ycol_off};
    Schedule* scheds[] = {&P->fwd, &P->bwd};
    size_t total = 0;
    for (const Schedule* S : scheds) total += align256(S->jobs.size() * sizeof(Job));
    for (const auto* t : tabs) total += align256(std::max<size_t>(t->size(), 1) * sizeof(int32_t));
    hipError_t e = hipMalloc(&P->d_tables, total);
    if (e == hipSuccess) {
      char* base = static_cast<char*>(P->d_tables);
      size_t off = 0;
      for (Schedule* S : scheds) {
        S->d_jobs = reinterpret_cast<Job*>(base + off);
        if (e == hipSuccess)
          e = hipMemcpy(S->d_jobs, S->jobs.data(), S->jobs.size() * sizeof(Job), hipMemcpyHostToDevice);
        off += align256(S->jobs.size() * sizeof(Job));
      }
      for (int k = 0; k < 6 && e == hipSuccess; ++k) {
        *dtabs[k] = reinterpret_cast<int32_t*>(base + off);
        if (!tabs[k]->empty())
          e = hipMemcpy(*dtabs[k], tabs[k]->data(), tabs[k]->size() * sizeof(int32_t), hipMemcpyHostToDevice);
        off += align256(std::max<size_t>(tabs[k]->size(), 1) * sizeof(int32_t));
      }
    }
    // auxiliary streams (default priority, not synchronising with the null stream) and
    // the fork/join events of the concurrent launches
    for (int k = 0; e == hipSuccess && k < P->fwd.n_aux; ++k) {
      e = hipStreamCreateWithFlags(&P->aux[k], hipStreamNonBlocking);
      if (e == hipSuccess) e = hipEventCreateWithFlags(&P->join[k], hipEventDisableTiming);
    }
    if (e == hipSuccess && P->fwd.n_aux > 0) e = hipEventCreateWithFlags(&P->fork, hipEventDisableTiming);
    if (e == hipSuccess && P->elem == 4 && P->lmax <= kBwdLmax) {
      e = hipStreamCreateWithFlags(&P->bwd_side, hipStreamNonBlocking);
      for (int k = 0; e == hipSuccess && k < 2; ++k) e = hipEventCreateWithFlags(&P->bwd_ev[k], hipEventDisableTiming);
    }
    if (e != hipSuccess) {
      release_device(P);
      delete P;
      return fail(CGTP_ERR_HIP, "plan device set-up: %s", hipGetErrorString(e));
    }
  }
  log_line(2, "plan %s x %s -> %s: %zu paths, %zu jobs, %zu groups, %zu launches on %d streams%s",
           irreps_in, irreps_sh, P->irreps_out.c_str(), P->paths.size(), P->fwd.jobs.size(), P->fwd.groups.size(),
           P->fwd.launches.size(), P->fwd.n_aux + 1, P->host_only ? " (host only)" : "");
  *out = P;
  return ok();
}

void cgtp_plan_destroy(cgtp_plan_t plan) {
  if (!plan) return;
  if (!plan->host_only) {
    int cur = -1;
    (void)hipGetDevice(&cur);
    if (cur != plan->device) (void)hipSetDevice(plan->device);
    release_device(plan);
    if (cur != plan->device && cur >= 0) (void)hipSetDevice(cur);
  }
  delete plan;
}

int cgtp_plan_info(cgtp_plan_t P, int64_t* f_in, int64_t* f_out, int64_t* w_per_edge, int* n_paths,
                   int* l_sh_max, char* irreps_out, size_t cap) {
  if (!P) return fail(CGTP_ERR_INVALID_ARG, "plan is NULL");
  if (f_in) *f_in = P->f_in;
  if (f_out) *f_out = P->f_out;
  if (w_per_edge) *w_per_edge = P->w;
  if (n_paths) *n_paths = int(P->paths.size());
  if (l_sh_max) *l_sh_max = P->l_sh_max;
  if (irreps_out && cap > 0) {
    std::strncpy(irreps_out, P->irreps_out.c_str(), cap - 1);
    irreps_out[cap - 1] = '\0';
  }
  return ok();
}

int cgtp_plan_paths(cgtp_plan_t P, int32_t* rows) {
  if (!P || !rows) return fail(CGTP_ERR_INVALID_ARG, "NULL argument");
  for (size_t k = 0; k < P->paths.size(); ++k) {
    const PathInfo& p = P->paths[k];
    const int32_t r[10] = {p.l1, p.p1, p.l2, p.p2, p.l3, p.p3, p.mul, p.in_off, p.out_off, p.w_off};
    std::memcpy(rows + 10 * k, r, sizeof(r));
  }
  return ok();
}

int cgtp_plan_cg(cgtp_plan_t P, int path, float* dense) {
  if (!P || !dense) return fail(CGTP_ERR_INVALID_ARG, "NULL argument");
  if (path < 0 || size_t(path) >= P->paths.size()) return fail(CGTP_ERR_INVALID_ARG, "path %d out of range", path);
  const PathInfo& p = P->paths[path];
  std::vector<float> t;
  dense_cg(p.l1, p.l2, p.l3, t);
  std::memcpy(dense, t.data(), t.size() * sizeof(float));
  return ok();
}

int cgtp_plan_schedule(cgtp_plan_t P, int* n_jobs, int* n_variants) {
  if (!P) return fail(CGTP_ERR_INVALID_ARG, "plan is NULL");
  if (n_jobs) *n_jobs = int(P->fwd.jobs.size());
  if (n_variants) *n_variants = P->fwd.n_variants;
  return ok();
}

int cgtp_workspace_size(cgtp_plan_t P, int64_t n_nodes, int64_t n_edges, int has_mask, size_t* bytes) {
  (void)has_mask;
  if (!P || !bytes) return fail(CGTP_ERR_INVALID_ARG, "NULL argument");
  if (n_nodes < 0 || n_edges < 0) return fail(CGTP_ERR_INVALID_ARG, "negative size");
  *bytes = carve(*P, n_nodes, n_edges, nullptr).bytes;
  return ok();
}

int cgtp_neighbors_workspace_size(int64_t n_nodes, const float box[3], float cutoff, size_t* bytes) {
  if (!box || !bytes) return fail(CGTP_ERR_INVALID_ARG, "NULL argument");
  if (n_nodes < 0 || n_nodes > kMaxInt32 - 1) return fail(CGTP_ERR_INVALID_ARG, "bad n_nodes");
  if (!(cutoff > 0.0f) || !(box[0] > 0.0f) || !(box[1] > 0.0f) || !(box[2] > 0.0f))
    return fail(CGTP_ERR_INVALID_ARG, "box and cutoff must be positive");
  *bytes = nbr_workspace_bytes(n_nodes, make_nbr_grid(n_nodes, box, cutoff));
  return ok();
}

int cgtp_neighbors_build(const float* pos, int64_t n_nodes, const float box[3], float cutoff, int32_t* row_ptr,
                         int32_t* col, int8_t* shift, int64_t edge_capacity, int64_t* n_edges, void* workspace,
                         size_t ws_bytes, void* stream) {
  if (!box || !row_ptr || !n_edges) return fail(CGTP_ERR_INVALID_ARG, "NULL argument");
  if (n_nodes < 0 || n_nodes > kMaxInt32 - 1) return fail(CGTP_ERR_INVALID_ARG, "bad n_nodes");
  if (n_nodes > 0 && !pos) return fail(CGTP_ERR_INVALID_ARG, "pos is NULL");
  if (edge_capacity < 0) return fail(CGTP_ERR_INVALID_ARG, "negative edge capacity");
  if (!(cutoff > 0.0f) || !(box[0] > 0.0f) || !(box[1] > 0.0f) || !(box[2] > 0.0f))
    return fail(CGTP_ERR_INVALID_ARG, "box and cutoff must be positive");
  if (!aligned(pos, 4) || !aligned(row_ptr, 4) || !aligned(col, 4))
    return fail(CGTP_ERR_INVALID_ARG, "misaligned pointer");
  const NbrGrid g = make_nbr_grid(n_nodes, box, cutoff);
  const size_t need = nbr_workspace_bytes(n_nodes, g);
  if (!workspace || ws_bytes < need)
    return fail(CGTP_ERR_WORKSPACE, "workspace %zu bytes < %zu required", ws_bytes, need);
  if (!aligned(workspace, 256)) return fail(CGTP_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  const NbrWorkspace w = carve_nbr_workspace(workspace, n_nodes, g);
  CGTP_HIP(launch_nbr_count(pos, int(n_nodes), g, w, row_ptr, s));
  int32_t stats[2] = {0, 0};   // edges, longest row
  if (n_nodes > 0) {
    CGTP_HIP(hipMemcpyAsync(stats, w.stats, sizeof(stats), hipMemcpyDeviceToHost, s));
    CGTP_HIP(hipStreamSynchronize(s));
  }
  const int32_t e_host = stats[0];
  *n_edges = e_host;
  if (e_host > edge_capacity)
    return fail(CGTP_ERR_CAPACITY, "edge list needs %d entries, capacity is %lld", e_host, (long long)edge_capacity);
  if (e_host > 0) {
    if (!col || !shift) return fail(CGTP_ERR_INVALID_ARG, "col/shift NULL with edges present");
    CGTP_HIP(launch_nbr_fill(pos, int(n_nodes), g, w, row_ptr, col, shift, stats[1], s));
  }
  return ok();
}

static int check_graph_args(const cgtp_plan_s* P, int64_t n_nodes, int64_t n_edges, const int32_t* row_ptr) {
  if (!P) return fail(CGTP_ERR_INVALID_ARG, "plan is NULL");
  if (P->host_only) return fail(CGTP_ERR_INVALID_ARG, "plan was created with CGTP_PLAN_HOST_ONLY");
  if (n_nodes < 0 || n_edges < 0) return fail(CGTP_ERR_INVALID_ARG, "negative size");
  if (n_nodes > kMaxInt32 - 1 || n_edges > kMaxInt32 - 1) return fail(CGTP_ERR_INVALID_ARG, "size exceeds int32");
  if (!row_ptr) return fail(CGTP_ERR_INVALID_ARG, "row_ptr is NULL");
  if (!aligned(row_ptr, 4)) return fail(CGTP_ERR_INVALID_ARG, "misaligned row_ptr");
  return check_device(P);
}

int cgtp_conv_prepare(cgtp_plan_t P, const int32_t* row_ptr, const uint8_t* mask, int64_t n_nodes, int64_t n_edges,
                      int32_t* act_row_ptr, int32_t* act_eid, int32_t* order, void* workspace, size_t ws_bytes,
                      void* stream) {
  int rc = check_graph_args(P, n_nodes, n_edges, row_ptr);
  if (rc != CGTP_OK) return rc;
  if (!act_row_ptr || !order || (n_edges > 0 && !act_eid)) return fail(CGTP_ERR_INVALID_ARG, "NULL output");
  const FwdWorkspace w = carve(*P, n_nodes, n_edges, workspace);
  if (!workspace || ws_bytes < w.bytes)
    return fail(CGTP_ERR_WORKSPACE, "workspace %zu bytes < %zu required", ws_bytes, w.bytes);
  if (!aligned(workspace, 256)) return fail(CGTP_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  RowPass rp{};
  rp.row_ptr = row_ptr;
  rp.mask = mask;
  rp.deg = w.deg;
  rp.n_nodes = int(n_nodes);
  rp.n_edges = int(n_edges);
  CGTP_HIP(launch_rows(rp, P->l_sh_max, s));
  CGTP_HIP(launch_order(w.deg, int(n_nodes), act_row_ptr, order, w.tmp_a, w.tmp_b, s));
  CGTP_HIP(launch_compact(row_ptr, mask, act_row_ptr, int(n_nodes), int(n_edges), act_eid, s));
  return ok();
}

}  // extern "C"

template <typename T>
static void fill_cell(RowPass& g, const T* cell) {
  g.has_cell = cell != nullptr;
  for (int k = 0; k < 9; ++k) g.cell[k] = cell ? double(cell[k]) : 0.0;
}

extern "C" {

int cgtp_edge_sh(cgtp_plan_t P, const float* pos, int64_t n_nodes, const float cell[9], const int32_t* row_ptr,
                 const int32_t* col, const int8_t* shift, int64_t n_edges, float* sh, void* stream) {
  int rc = check_graph_args(P, n_nodes, n_edges, row_ptr);
  if (rc != CGTP_OK) return rc;
  if (n_edges > 0 && (!pos || !col || !sh)) return fail(CGTP_ERR_INVALID_ARG, "NULL argument");
  RowPass g{};
  g.pos = pos;
  g.row_ptr = row_ptr;
  g.col = col;
  g.shift = shift;
  g.sh = sh;
  g.n_nodes = int(n_nodes);
  g.n_edges = int(n_edges);
  fill_cell(g, cell);
  CGTP_HIP(launch_rows(g, P->l_sh_max, static_cast<hipStream_t>(stream)));
  return ok();
}

}  // extern "C"

// The workgroup layout of one launch of the fused conv kernel (its groups and blocks) in
// a; returns its workgroup count.  Workgroups are dispatched block by block: a block of
// B = 64 / 2^lg_min receivers (the largest node group of the launch) holds B / S_g node
// groups of every group g, so the groups of one block, which read the same weight rows,
// run at the same time.
template <typename T>
static int64_t fill_launch(const Schedule& S, const ConvLaunch& L, int64_t n_nodes, ConvArgsT<T>& a) {
  a.n_groups = L.g1 - L.g0;
  for (int k = 0; k < kMaxGroupsPerLaunch; ++k) a.g_start[k] = kMaxInt32;   // past the groups
  int lg_min = 6;
  for (int k = L.g0; k < L.g1; ++k) lg_min = std::min(lg_min, S.groups[k].lanes_log2);
  int per_block = 0;
  for (int k = L.g0; k < L.g1; ++k) {
    const Group& G = S.groups[k];
    a.g_start[k - L.g0] = per_block;
    GroupArgs& ga = a.grp[k - L.g0];
    ga.start = per_block;
    ga.first_job = G.first_job;
    ga.n_jobs = G.n_jobs;
    ga.lanes_log2 = G.lanes_log2;
    ga.y0 = G.y0;
    ga.y4 = G.y4;
    per_block += 1 << (G.lanes_log2 - lg_min);
  }
  const int64_t block = 64 >> lg_min;
  const int64_t nblocks = (n_nodes + block - 1) / block;
  // whole rounds of kXcds blocks: blocks past the last are empty workgroups
  const int64_t wgs = (nblocks + kXcds - 1) / kXcds * kXcds * per_block;
  a.jobs = S.d_jobs;
  a.n_waves = L.waves;
  a.blk_wgs = per_block;
  a.blk_lg_min = lg_min;
  a.n_blocks = int(nblocks);
  a.total_wgs = int(std::min<int64_t>(wgs, kMaxInt32));
  return wgs;
}

// The forward in element type T (float, or double for plans made with CGTP_PLAN_FP64).
template <typename T>
static int conv_forward_impl(cgtp_plan_t P, const T* pos, int64_t n_nodes, const T cell[9],
                             const int32_t* row_ptr, const int32_t* col, const int8_t* shift, int64_t n_edges,
                             const T* x, const T* w, const uint8_t* mask, const T* gate, T* out,
                             void* workspace, size_t ws_bytes, void* stream, hipEvent_t ev_begin,
                             hipEvent_t ev_end) {
  int rc = check_graph_args(P, n_nodes, n_edges, row_ptr);
  if (rc != CGTP_OK) return rc;
  if (P->elem != int(sizeof(T)))
    return fail(CGTP_ERR_INVALID_ARG, "the plan's precision (%s) does not match this entry point (%s)",
                P->elem == 8 ? "fp64" : "fp32", sizeof(T) == 8 ? "fp64" : "fp32");
  if (n_nodes > 0 && (!out || !x || !pos)) return fail(CGTP_ERR_INVALID_ARG, "NULL node array");
  if (n_edges > 0 && (!col || !w)) return fail(CGTP_ERR_INVALID_ARG, "NULL edge array");
  if (!aligned(x, 16) || !aligned(w, 16) || !aligned(out, 16) || !aligned(pos, sizeof(T)) || !aligned(col, 4))
    return fail(CGTP_ERR_INVALID_ARG, "x, w and out must be 16-byte aligned");
  if (!aligned(gate, sizeof(T))) return fail(CGTP_ERR_INVALID_ARG, "gate must be aligned to its element size");
  if (double(n_nodes) * double(P->f_in) * double(sizeof(T)) >= 4294967296.0)
    return fail(CGTP_ERR_UNSUPPORTED, "x is 4 GiB or larger (32-bit byte offsets)");
  const FwdWorkspace ws = carve(*P, n_nodes, n_edges, workspace);
  if (!workspace || ws_bytes < ws.bytes)
    return fail(CGTP_ERR_WORKSPACE, "workspace %zu bytes < %zu required", ws_bytes, ws.bytes);
  if (!aligned(workspace, 256)) return fail(CGTP_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  if (n_nodes == 0) return ok();
  hipStream_t s = static_cast<hipStream_t>(stream);

  // 1. per row: active degree and the harmonics of its active edges (CSR order)
  RowPass g{};
  if constexpr (sizeof(T) == 8) {
    g.pos64 = pos;
    g.gate64 = gate;
    g.sh64 = static_cast<double*>(ws.sh);
  } else {
    g.pos = pos;
    g.gate = gate;
    g.sh = static_cast<float*>(ws.sh);
  }
  g.row_ptr = row_ptr;
  g.col = col;
  g.shift = shift;
  g.mask = mask;
  g.deg = ws.deg;
  g.act_e = ws.act_e;
  g.act_j = ws.act_j;
  g.sh_stride = P->sh_pad;
  g.n_nodes = int(n_nodes);
  g.n_edges = int(n_edges);
  fill_cell(g, cell);
  // 2. node order by active degree (LunaTP Table 9), as position-indexed node records;
  //    without mask and gate every edge is active and the order needs only row_ptr, so
  //    it runs in the same launch as the per-row pass
  if (!mask && !gate) {
    CGTP_HIP(launch_rows_order(g, P->l_sh_max, ws.node_info, s));
  } else {
    CGTP_HIP(launch_rows(g, P->l_sh_max, s));
    CGTP_HIP(launch_degree_order(ws.deg, int(n_nodes), row_ptr, ws.node_info, s));
  }
  // 3. the fused convolution: per kernel class, launches of up to kMaxGroupsPerLaunch
  //    job groups whose workgroup ranges travel in the kernel arguments
  ConvArgsT<T> a{};
  a.x = x;
  a.w = w;
  a.sh = static_cast<const T*>(ws.sh);
  a.node_info = ws.node_info;
  a.act_e = ws.act_e;
  a.act_j = ws.act_j;
  a.out = out;
  a.n_nodes = int(n_nodes);
  a.f_in = int(P->f_in);
  a.f_out = int(P->f_out);
  a.w_stride = int(P->w);
  a.sh_stride = P->sh_pad;
  const Schedule& F = P->fwd;
  auto fill = [&](const ConvLaunch& L) -> int64_t { return fill_launch(F, L, n_nodes, a); };
  const auto& launches = F.launches;
  for (const auto& L : launches)
    if (fill(L) > kMaxInt32) return fail(CGTP_ERR_UNSUPPORTED, "too many workgroups");
  // With auxiliary streams: fork them from the caller's stream after the per-row pass,
  // launch, and join them back; the events then bracket the whole set (enqueue-time
  // records).  On one stream the events are stamped by the first and last launches.
  const bool forked = F.n_aux > 0;
  std::unique_lock<std::mutex> lock(P->enqueue, std::defer_lock);
  if (forked) {
    lock.lock();
    if (ev_begin) CGTP_HIP(hipEventRecord(ev_begin, s));
    CGTP_HIP(hipEventRecord(P->fork, s));
    for (int k = 0; k < F.n_aux; ++k) CGTP_HIP(hipStreamWaitEvent(P->aux[k], P->fork, 0));
  }
  hipError_t launch_err = hipSuccess;
  for (size_t li = 0; li < launches.size() && launch_err == hipSuccess; ++li) {
    const auto& L = launches[li];
    fill(L);
    hipStream_t ls = L.stream == 0 ? s : P->aux[L.stream - 1];
    launch_err = launch_conv(a, L.cls, ls, !forked && li == 0 ? ev_begin : nullptr,
                             !forked && li + 1 == launches.size() ? ev_end : nullptr);
  }
  if (forked) {   // joined even after a failed launch, so that `stream` follows what ran
    for (int k = 0; k < F.n_aux; ++k) {
      CGTP_HIP(hipEventRecord(P->join[k], P->aux[k]));
      CGTP_HIP(hipStreamWaitEvent(s, P->join[k], 0));
    }
    if (ev_end) CGTP_HIP(hipEventRecord(ev_end, s));
  }
  CGTP_HIP(launch_err);
  if (launches.empty()) {  // no wave task (cannot happen with n_nodes > 0): keep the events valid
    if (ev_begin) CGTP_HIP(hipEventRecord(ev_begin, s));
    if (ev_end) CGTP_HIP(hipEventRecord(ev_end, s));
  }
  return ok();
}

extern "C" {

int cgtp_conv_forward(cgtp_plan_t P, const float* pos, int64_t n_nodes, const float cell[9], const int32_t* row_ptr,
                      const int32_t* col, const int8_t* shift, int64_t n_edges, const float* x, const float* w,
                      const uint8_t* mask, float* out, void* workspace, size_t ws_bytes, void* stream) {
  return conv_forward_impl<float>(P, pos, n_nodes, cell, row_ptr, col, shift, n_edges, x, w, mask, nullptr, out,
                           workspace, ws_bytes, stream, nullptr, nullptr);
}

int cgtp_conv_forward_gated(cgtp_plan_t P, const float* pos, int64_t n_nodes, const float cell[9],
                            const int32_t* row_ptr, const int32_t* col, const int8_t* shift, int64_t n_edges,
                            const float* x, const float* w, const uint8_t* mask, const float* gate, float* out,
                            void* workspace, size_t ws_bytes, void* stream) {
  return conv_forward_impl<float>(P, pos, n_nodes, cell, row_ptr, col, shift, n_edges, x, w, mask, gate, out,
                           workspace, ws_bytes, stream, nullptr, nullptr);
}

int cgtp_conv_forward_f64(cgtp_plan_t P, const double* pos, int64_t n_nodes, const double cell[9],
                          const int32_t* row_ptr, const int32_t* col, const int8_t* shift, int64_t n_edges,
                          const double* x, const double* w, const uint8_t* mask, const double* gate, double* out,
                          void* workspace, size_t ws_bytes, void* stream, void* ev_conv_begin,
                          void* ev_conv_end) {
  return conv_forward_impl<double>(P, pos, n_nodes, cell, row_ptr, col, shift, n_edges, x, w, mask, gate, out, workspace,
                           ws_bytes, stream, static_cast<hipEvent_t>(ev_conv_begin),
                           static_cast<hipEvent_t>(ev_conv_end));
}

}  // extern "C"

// Scratch of the no-allocation forward: one copy of this array per GPU, held until the
// process ends.  Host code never uses its name as an address (in host code the name is
// a host-side stand-in): kernels and copies get the device address that
// hipGetSymbolAddress returns for the current device, looked up once per device.
static __device__ __align__(256) unsigned char scratch[CGTP_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_addr[kMaxDevices] = {};   // device address of `scratch`, per device

// The current device's address of `scratch` (the plan's device, already checked to be
// current).
int scratch_address(int dev, void** out) {
  if (dev < 0 || dev >= kMaxDevices) return fail(CGTP_ERR_UNSUPPORTED, "device %d beyond %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_addr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(CGTP_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
    g_scratch_addr[dev] = p;
  }
  *out = g_scratch_addr[dev];
  return CGTP_OK;
}
}  // namespace

extern "C" int cgtp_conv_forward_noalloc(cgtp_plan_t P, const float* pos, int64_t n_nodes, const float cell[9],
                                         const int32_t* row_ptr, const int32_t* col, const int8_t* shift,
                                         int64_t n_edges, const float* x, const float* w, const uint8_t* mask,
                                         const float* gate, float* out, void* stream) {
  int rc = check_graph_args(P, n_nodes, n_edges, row_ptr);
  if (rc != CGTP_OK) return rc;
  const size_t need = carve(*P, n_nodes, n_edges, nullptr).bytes;
  if (need > CGTP_NOALLOC_SCRATCH_BYTES)
    return fail(CGTP_ERR_WORKSPACE, "this graph needs %zu bytes of scratch; the no-allocation forward has %zu",
                need, size_t(CGTP_NOALLOC_SCRATCH_BYTES));
  void* ws = nullptr;
  rc = scratch_address(P->device, &ws);
  if (rc != CGTP_OK) return rc;
  return conv_forward_impl<float>(P, pos, n_nodes, cell, row_ptr, col, shift, n_edges, x, w, mask, gate, out, ws,
                                  CGTP_NOALLOC_SCRATCH_BYTES, stream, nullptr, nullptr);
}

// Workspace of the backward: the forward's sections, then the sender-grouped slots, the
// edge pass's rows of partials (one per slot) and dL/dr per slot.
struct BwdWorkspace {
  FwdWorkspace fwd;
  int32_t *t_cnt, *t_row_ptr, *t_slot, *t_recv;
  float *part, *grad_r;
  float* scratch_row;   // the edge pass's stores of lanes with nothing to store
  size_t bytes;
};

static BwdWorkspace carve_bwd(const cgtp_plan_s& P, int64_t n, int64_t e, void* base) {
  BwdWorkspace w{};
  w.fwd = carve(P, n, e, base);
  char* p = static_cast<char*>(base);
  size_t off = w.fwd.bytes;
  auto take = [&](size_t bytes) {
    char* r = p ? p + off : nullptr;
    off += align256(bytes);
    return r;
  };
  w.t_cnt = reinterpret_cast<int32_t*>(take(size_t(n) * 4));
  w.t_row_ptr = reinterpret_cast<int32_t*>(take(size_t(n + 1) * 4));
  w.t_slot = reinterpret_cast<int32_t*>(take(size_t(e) * 4));
  w.t_recv = reinterpret_cast<int32_t*>(take(size_t(e) * 4));
  w.part = reinterpret_cast<float*>(take(size_t(e) * size_t(P.part_stride) * 4));
  w.grad_r = reinterpret_cast<float*>(take(size_t(e) * 12));
  w.scratch_row = reinterpret_cast<float*>(take(64 * 4));
  w.bytes = off;
  return w;
}

extern "C" {

int cgtp_backward_workspace_size(cgtp_plan_t P, int64_t n_nodes, int64_t n_edges, size_t* bytes) {
  if (!P || !bytes) return fail(CGTP_ERR_INVALID_ARG, "NULL argument");
  if (n_nodes < 0 || n_edges < 0) return fail(CGTP_ERR_INVALID_ARG, "negative size");
  *bytes = carve_bwd(*P, n_nodes, n_edges, nullptr).bytes;
  return ok();
}

int cgtp_conv_backward(cgtp_plan_t P, const float* pos, int64_t n_nodes, const float cell[9], const int32_t* row_ptr,
                       const int32_t* col, const int8_t* shift, int64_t n_edges, const float* x, const float* w,
                       const uint8_t* mask, const float* gate, const float* grad_out, float* grad_x, float* grad_w,
                       float* grad_pos, void* workspace, size_t ws_bytes, void* stream) {
  int rc = check_graph_args(P, n_nodes, n_edges, row_ptr);
  if (rc != CGTP_OK) return rc;
  if (P->elem != 4) return fail(CGTP_ERR_INVALID_ARG, "the backward is fp32: the plan's precision is fp64");
  if (P->lmax > kBwdLmax)
    return fail(CGTP_ERR_UNSUPPORTED, "the backward supports plans with l <= %d (this one reaches %d)", kBwdLmax,
                P->lmax);
  const bool any = grad_x || grad_w || grad_pos;
  if (n_nodes > 0 && any && (!grad_out || !x || !pos)) return fail(CGTP_ERR_INVALID_ARG, "NULL node array");
  if (n_edges > 0 && any && (!col || !w)) return fail(CGTP_ERR_INVALID_ARG, "NULL edge array");
  if (!aligned(x, 16) || !aligned(w, 16) || !aligned(grad_out, 16) || !aligned(grad_w, 16))
    return fail(CGTP_ERR_INVALID_ARG, "x, w, grad_out and grad_w must be 16-byte aligned");
  if (!aligned(pos, 4) || !aligned(col, 4) || !aligned(gate, 4) || !aligned(grad_x, 4) || !aligned(grad_pos, 4))
    return fail(CGTP_ERR_INVALID_ARG, "misaligned pointer");
  if (double(n_nodes) * double(P->f_in) * 4.0 >= 4294967296.0)
    return fail(CGTP_ERR_UNSUPPORTED, "x is 4 GiB or larger (32-bit byte offsets)");
  const BwdWorkspace ws = carve_bwd(*P, n_nodes, n_edges, workspace);
  if (!workspace || ws_bytes < ws.bytes)
    return fail(CGTP_ERR_WORKSPACE, "workspace %zu bytes < %zu required", ws_bytes, ws.bytes);
  if (!aligned(workspace, 256)) return fail(CGTP_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  if (n_nodes == 0 || !any) return ok();
  hipStream_t s = static_cast<hipStream_t>(stream);
  // 1. the forward's per-row pass: active slots, senders and gate-scaled harmonics
  RowPass g{};
  g.pos = pos;
  g.row_ptr = row_ptr;
  g.col = col;
  g.shift = shift;
  g.mask = mask;
  g.gate = gate;
  g.deg = ws.fwd.deg;
  g.act_e = ws.fwd.act_e;
  g.act_j = ws.fwd.act_j;
  g.sh = static_cast<float*>(ws.fwd.sh);
  g.sh_stride = P->sh_pad;
  g.n_nodes = int(n_nodes);
  g.n_edges = int(n_edges);
  fill_cell(g, cell);
  // and the node order by active degree that the edge pass walks, as in the forward
  if (!mask && !gate) {
    CGTP_HIP(launch_rows_order(g, P->l_sh_max, ws.fwd.node_info, s));
  } else {
    CGTP_HIP(launch_rows(g, P->l_sh_max, s));
    CGTP_HIP(launch_degree_order(ws.fwd.deg, int(n_nodes), row_ptr, ws.fwd.node_info, s));
  }
  // 2. beside the edge pass, on the plan's side stream: the zeroing of the inactive
  //    edges' w-gradient rows and the grouping of the active slots by sender
  BwdArgs a{};
  a.pos = pos;
  a.row_ptr = row_ptr;
  a.shift = shift;
  a.gate = gate;
  a.deg = ws.fwd.deg;
  a.act_e = ws.fwd.act_e;
  a.act_j = ws.fwd.act_j;
  a.t_row_ptr = ws.t_row_ptr;
  a.t_slot = ws.t_slot;
  a.t_recv = ws.t_recv;
  a.part = ws.part;
  a.xcol_ptr = P->d_xcol_ptr;
  a.xcol_off = P->d_xcol_off;
  a.ycol_ptr = P->d_ycol_ptr;
  a.ycol_off = P->d_ycol_off;
  a.grad_x = grad_x;
  a.grad_r = ws.grad_r;
  a.grad_pos = grad_pos;
  a.n_nodes = int(n_nodes);
  a.f_in = int(P->f_in);
  a.part_stride = P->part_stride;
  a.l_sh_max = P->l_sh_max;
  a.want_gy = grad_pos != nullptr;
  a.has_cell = cell != nullptr;
  for (int k = 0; k < 9; ++k) a.cell[k] = cell ? double(cell[k]) : 0.0;
  std::lock_guard<std::mutex> lock(P->enqueue);
  hipStream_t b = P->bwd_side;
  CGTP_HIP(hipEventRecord(P->bwd_ev[0], s));
  CGTP_HIP(hipStreamWaitEvent(b, P->bwd_ev[0], 0));
  if (grad_w) CGTP_HIP(launch_zero_inactive(row_ptr, mask, gate, int(n_nodes), grad_w, int(P->w), b));
  if (grad_x || grad_pos) CGTP_HIP(launch_bwd_transpose(a, ws.t_cnt, ws.t_row_ptr, ws.t_slot, ws.t_recv, b));
  CGTP_HIP(hipEventRecord(P->bwd_ev[1], b));
  // 3. the edge pass: the fused conv kernel's workgroups in their backward mode write the
  //    w-gradient of every active edge and, per active slot, the jobs' dL/dY and the job
  //    groups' x-gradients of the edge
  {
    ConvArgsT<float> c{};
    c.x = x;
    c.w = w;
    c.sh = static_cast<const float*>(ws.fwd.sh);
    c.node_info = ws.fwd.node_info;
    c.act_e = ws.fwd.act_e;
    c.act_j = ws.fwd.act_j;
    c.n_nodes = int(n_nodes);
    c.f_in = int(P->f_in);
    c.f_out = int(P->f_out);
    c.w_stride = int(P->w);
    c.sh_stride = P->sh_pad;
    c.grad_out = grad_out;
    c.grad_w = grad_w;
    c.gyp = grad_pos ? ws.part : nullptr;
    c.xgp = grad_x ? ws.part : nullptr;
    c.job_gy = P->d_job_gy;
    c.job_xg = P->d_job_xg;
    c.scratch_row = ws.scratch_row;
    c.part_stride = P->part_stride;
    for (const auto& L : P->bwd.launches) {
      if (fill_launch(P->bwd, L, n_nodes, c) > kMaxInt32) return fail(CGTP_ERR_UNSUPPORTED, "too many workgroups");
      CGTP_HIP(launch_conv_bwd(c, L.cls, s));
    }
  }
  // 4. per sender: its x-gradient and its slots' dL/dr, then the position gradient (in
  //    the caller's stream once the side stream is joined back: run beside each other or
  //    beside the edge pass, these passes only slowed it by as much as they took)
  CGTP_HIP(hipStreamWaitEvent(s, P->bwd_ev[1], 0));
  if (grad_x) CGTP_HIP(launch_bwd_gather_x(a, s));
  if (grad_pos) {
    CGTP_HIP(launch_bwd_force(a, s));
    CGTP_HIP(launch_bwd_pos(a, s));
  }
  return ok();
}

int cgtp_conv_forward_timed(cgtp_plan_t P, const float* pos, int64_t n_nodes, const float cell[9],
                            const int32_t* row_ptr, const int32_t* col, const int8_t* shift, int64_t n_edges,
                            const float* x, const float* w, const uint8_t* mask, const float* gate, float* out,
                            void* workspace, size_t ws_bytes, void* stream, void* ev_conv_begin,
                            void* ev_conv_end) {
  if (!ev_conv_begin || !ev_conv_end) return fail(CGTP_ERR_INVALID_ARG, "events must not be NULL");
  return conv_forward_impl<float>(P, pos, n_nodes, cell, row_ptr, col, shift, n_edges, x, w, mask, gate, out,
                           workspace, ws_bytes, stream, static_cast<hipEvent_t>(ev_conv_begin),
                           static_cast<hipEvent_t>(ev_conv_end));
}

}  // extern "C"
