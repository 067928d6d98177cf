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

#include <hip/hip_runtime.h>

#include <algorithm>

#include "plan_core.h"

namespace usp {
namespace {

__global__ __launch_bounds__(256) void plan_items_kernel(const PlanJobs jobs) {
  const PlanJob& J = blockIdx.y ? jobs.j[1] : jobs.j[0];
  const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (g >= J.candidates()) return;
  const SeqView seq{J.mask.nseq > 0 ? J.cu : nullptr, J.mask.nseq, J.mask.S};
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
  hipLaunchKernelGGL(plan_items_kernel, dim3((unsigned)((cand + 255) / 256), (unsigned)jobs.n), dim3(256), 0,
                     stream, jobs);
  hipLaunchKernelGGL(plan_sort_kernel, dim3((unsigned)((cpp + 255) / 256), (unsigned)steps, (unsigned)jobs.n),
                     dim3(256), 0, stream, jobs);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    set_error("tile planner launch failed: %s", hipGetErrorString(e));
    return USP_ERR_HIP;
  }
  return USP_OK;
}

}  // namespace usp
