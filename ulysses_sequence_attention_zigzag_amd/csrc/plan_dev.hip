// Device tile planner: the ring calls plan their tiles on the GPU, into the
// caller's workspace, on every call, so a call allocates nothing, copies
// nothing from the host and never waits for the device (and can be recorded
// into a HIP graph as it stands).  The host only sizes the buffers.
//
// plan_items_kernel: one thread per candidate item (a tile of query rows, or
//   of keys for the dK / dV kernel) runs the shared per-item planner
//   (plan_core.h) and writes the item, its runs (into the candidate's run
//   slots) and its cost; items with nothing to do get q_rows = 0.
// plan_sort_kernel: orders the items of each plan by decreasing cost, ties
//   by candidate index (the rank of an item is the number of items before it
//   in that order), dropped items last; plans of more than kMaxSortItems
//   candidates keep candidate order.
// plan_small_kernel: both steps in one workgroup per job when every job has
//   at most kSmallPlan candidates (the window and varlen calls): items and
//   costs stay in LDS between them, and one launch replaces two.
// The kernels read cu_seqlens from LDS when it fits: the planner's binary
// searches over it are chains of dependent loads.

#include <hip/hip_runtime.h>

#include <algorithm>

#include "plan_core.h"

namespace usp {
namespace {

constexpr int kSmallPlan = 1024;
constexpr int kCuLds = 2048;  // cu_seqlens entries staged in LDS

// Sequences of job J, with cu_seqlens copied into cu_s when it fits (a
// workgroup barrier: every thread of the workgroup calls this).
__device__ SeqView stage_seq(const PlanJob& J, int32_t* cu_s) {
  SeqView seq{J.mask.nseq > 0 ? J.cu : nullptr, J.mask.nseq, J.mask.S};
  if (J.mask.nseq > 0 && J.mask.nseq + 1 <= kCuLds) {
    for (int i = threadIdx.x; i <= J.mask.nseq; i += blockDim.x) cu_s[i] = J.cu[i];
    seq.cu = cu_s;
  }
  __syncthreads();
  return seq;
}

__global__ __launch_bounds__(256) void plan_items_kernel(const PlanJobs jobs) {
  const PlanJob& J = blockIdx.y ? jobs.j[1] : jobs.j[0];
  __shared__ int32_t cu_s[kCuLds];
  const SeqView seq = stage_seq(J, cu_s);
  const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (g >= J.candidates()) return;
  Run* slot = J.runs + g * J.cap;
  int64_t cost = 0;
  const WorkItem it = plan_candidate(J, seq, g, [&](int32_t i, const Run& r) { slot[i] = r; }, &cost);
  J.tmp[g] = it;
  J.cost[g] = cost;
}

__global__ __launch_bounds__(256) void plan_sort_kernel(const PlanJobs jobs) {
  const PlanJob& J = blockIdx.z ? jobs.j[1] : jobs.j[0];
  const int32_t s = blockIdx.y;
  const int64_t cpp = J.cpp();
  const int64_t i0 = (int64_t)blockIdx.x * 256;
  if (s >= J.n_steps || i0 >= cpp) return;  // whole workgroup
  const int64_t base = (int64_t)s * cpp;
  const int64_t i = i0 + threadIdx.x;
  if (cpp > kMaxSortItems) {
    if (i < cpp) J.items[base + i] = J.tmp[base + i];
    return;
  }
  __shared__ int64_t sc[256];
  const int64_t mine = i < cpp ? J.cost[base + i] : 0;
  int64_t rank = 0;
  for (int64_t c0 = 0; c0 < cpp; c0 += 256) {
    __syncthreads();
    if (c0 + threadIdx.x < cpp) sc[threadIdx.x] = J.cost[base + c0 + threadIdx.x];
    __syncthreads();
    const int n = (int)(cpp - c0 < 256 ? cpp - c0 : 256);
    for (int k = 0; k < n; ++k) {
      const int64_t c = sc[k];
      rank += (c > mine) || (c == mine && c0 + k < i);
    }
  }
  if (i < cpp) J.items[base + rank] = J.tmp[base + i];
}

__global__ __launch_bounds__(kSmallPlan) void plan_small_kernel(const PlanJobs jobs) {
  const PlanJob& J = blockIdx.x ? jobs.j[1] : jobs.j[0];
  __shared__ int32_t cu_s[kCuLds];
  __shared__ int64_t cost_s[kSmallPlan];
  __shared__ WorkItem item_s[kSmallPlan];
  const SeqView seq = stage_seq(J, cu_s);
  const int64_t cand = J.candidates();
  for (int64_t g = threadIdx.x; g < cand; g += blockDim.x) {
    Run* slot = J.runs + g * J.cap;
    int64_t cost = 0;
    item_s[g] = plan_candidate(J, seq, g, [&](int32_t i, const Run& r) { slot[i] = r; }, &cost);
    cost_s[g] = cost;
  }
  __syncthreads();
  const int64_t cpp = J.cpp();
  for (int64_t g = threadIdx.x; g < cand; g += blockDim.x) {
    const int64_t s = g / cpp;
    const int64_t base = s * cpp, i = g - base;
    const int64_t mine = cost_s[g];
    int64_t rank = 0;
    for (int64_t k = 0; k < cpp; ++k) {
      const int64_t c = cost_s[base + k];
      rank += (c > mine) || (c == mine && k < i);
    }
    J.items[base + rank] = item_s[g];
  }
}

}  // namespace

usp_status launch_plan(const PlanJobs& jobs, hipStream_t stream) {
  int64_t cand = 0, cpp = 0;
  int32_t steps = 0;
  for (int k = 0; k < jobs.n; ++k) {
    cand = std::max<int64_t>(cand, jobs.j[k].candidates());
    cpp = std::max<int64_t>(cpp, jobs.j[k].cpp());
    steps = std::max<int32_t>(steps, jobs.j[k].n_steps);
  }
  if (cand == 0) return USP_OK;
  TimingScope ts(K_PLAN, stream);
  if (cand <= kSmallPlan) {
    // (cpp <= cand <= kMaxSortItems: every plan is ordered)
    hipLaunchKernelGGL(plan_small_kernel, dim3((unsigned)jobs.n), dim3(kSmallPlan), 0, stream, jobs);
  } else {
    hipLaunchKernelGGL(plan_items_kernel, dim3((unsigned)((cand + 255) / 256), (unsigned)jobs.n), dim3(256), 0,
                       stream, jobs);
    hipLaunchKernelGGL(plan_sort_kernel, dim3((unsigned)((cpp + 255) / 256), (unsigned)steps, (unsigned)jobs.n),
                       dim3(256), 0, stream, jobs);
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    set_error("tile planner launch failed: %s", hipGetErrorString(e));
    return USP_ERR_HIP;
  }
  return USP_OK;
}

}  // namespace usp
