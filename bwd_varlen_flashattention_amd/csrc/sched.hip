// Device-built, cost-sorted work list for the persistent attention kernels.
//
// Jagged batches give tiles of very different cost.  The list is built on the
// device straight from the offsets (no host round trip): every (sequence, tile)
// entry gets a cost equal to the number of inner-loop tiles it will visit
// (causal tiles stop at the diagonal), entries are counting-sorted longest
// first, and persistent workgroups then pull them in that order from an atomic
// counter, which is a longest-processing-time-first greedy schedule.  This is
// the software load balancing of jagged tiles and the persistent, on-demand
// tile hand-out of "Optimizing Jagged Flash Attention with TLX" (fourth and
// fifth paragraphs), done with a global atomic instead of Cluster Launch Control.
#include "jfa_internal.h"
#include "device_common.h"

namespace jfa {

constexpr int kSchedThreads = 1024;
constexpr int kMaxBuckets = 4096;

__device__ __forceinline__ int entry_cost(const SchedArgs& a, int lq, int lk, int t) {
  if (a.mode == 0) {               // query tile t, loop over key tiles
    if (!a.causal) return cdiv(lk, a.loop_tile);
    const int kmax = min(lk, (t + 1) * a.stat_tile + lk - lq);   // keys visible to the tile's last row
    return kmax > 0 ? cdiv(kmax, a.loop_tile) : 0;
  }
  // key tile t, loop over query tiles
  const int ntq = cdiv(lq, a.loop_tile);
  if (!a.causal) return ntq;
  const int first_q = max(0, t * a.stat_tile - (lk - lq));       // first query that sees key t*stat_tile
  return first_q < lq ? ntq - first_q / a.loop_tile : 0;
}

__global__ __launch_bounds__(kSchedThreads) void sched_kernel(SchedArgs a) {
  __shared__ int hist[kMaxBuckets];
  __shared__ int part[kSchedThreads];
  const int tid = threadIdx.x;
  const int nb = a.n_buckets;
  for (int i = tid; i < nb; i += kSchedThreads) hist[i] = 0;
  __syncthreads();

  // pass 1: histogram of costs (bucket index counts down so the scan sorts longest first)
  for (int b = tid; b < a.batch; b += kSchedThreads) {
    const int lq = a.bcast_nq > 0 ? a.bcast_nq : a.cu_q[b + 1] - a.cu_q[b];
    const int lk = a.cu_k[b + 1] - a.cu_k[b];
    const int stat_len = a.mode == 0 ? lq : lk;
    const int nt = cdiv(stat_len, a.stat_tile);
    for (int t = 0; t < nt; ++t) {
      const int c = min(entry_cost(a, lq, lk, t), nb - 1);
      atomicAdd(&hist[nb - 1 - c], 1);
    }
  }
  __syncthreads();

  // pass 2: exclusive scan of the histogram (each thread owns a contiguous run of buckets)
  const int per = cdiv(nb, kSchedThreads);
  const int lo = min(tid * per, nb), hi = min(lo + per, nb);
  int run = 0;
  for (int i = lo; i < hi; ++i) run += hist[i];
  part[tid] = run;
  __syncthreads();
  for (int off = 1; off < kSchedThreads; off <<= 1) {
    const int add = tid >= off ? part[tid - off] : 0;
    __syncthreads();
    part[tid] += add;
    __syncthreads();
  }
  int base = part[tid] - run;            // exclusive prefix of this thread's run
  for (int i = lo; i < hi; ++i) {
    const int c = hist[i];
    hist[i] = base;
    base += c;
  }
  const int total = part[kSchedThreads - 1];
  __syncthreads();

  // pass 3: scatter the entries into their buckets
  for (int b = tid; b < a.batch; b += kSchedThreads) {
    const int lq = a.bcast_nq > 0 ? a.bcast_nq : a.cu_q[b + 1] - a.cu_q[b];
    const int lk = a.cu_k[b + 1] - a.cu_k[b];
    const int stat_len = a.mode == 0 ? lq : lk;
    const int nt = cdiv(stat_len, a.stat_tile);
    for (int t = 0; t < nt; ++t) {
      const int c = min(entry_cost(a, lq, lk, t), nb - 1);
      const int pos = atomicAdd(&hist[nb - 1 - c], 1);
      if (pos < a.max_entries) a.entries[pos] = WorkEntry{b, t};
    }
  }
  if (tid == 0) {
    *a.n_entries = min(total, a.max_entries);
    *a.counter = 0u;
  }
}

hipError_t launch_sched(const SchedArgs& a, hipStream_t stream) {
  if (a.n_buckets < 1 || a.n_buckets > kMaxBuckets) return hipErrorInvalidValue;
  hipLaunchKernelGGL(sched_kernel, dim3(1), dim3(kSchedThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace jfa
