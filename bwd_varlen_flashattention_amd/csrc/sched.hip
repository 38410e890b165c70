// Device-built work list for the persistent attention kernels.
//
// Jagged batches give tiles of very different cost.  The list is built on the
// device straight from the offsets (no host round trip).  Every tile gets a cost
// equal to the number of inner-loop tiles it will visit (causal tiles stop at the
// diagonal).  This is the software load balancing of jagged tiles and the
// persistent, on-demand tile hand-out of "Optimizing Jagged Flash Attention with
// TLX" (fourth and fifth paragraphs), with global atomics in place of Cluster
// Launch Control.
//
// The list is organised for the L2 caches as well as for balance.  All tiles of
// one (sequence, KV head) read the same K/V (query-stationary kernels) or the
// same Q/dO (key-stationary kernel), so they form a group that is kept together
// in one queue and handed out back to back.  Groups are counting-sorted by cost,
// longest first, and dealt to the kQueues per-XCD queues in snake order
// (0..7, 7..0, ...), which balances the queues while each stays in descending
// cost order.  Workgroup i serves queue i % kQueues (the XCD it is dispatched
// to) and steals from the other queues once its own is empty.
#include <algorithm>

#include "jfa_internal.h"
#include "device_common.h"

namespace jfa {

constexpr int kSchedThreads = 1024;
constexpr int kMaxBuckets = 4096;
constexpr int kPerQueue = kSchedThreads / kQueues;
static_assert(kPerQueue % 64 == 0 && kSchedThreads % 64 == 0, "scan segments are whole waves");
constexpr int kLdsGroups = 6144;              // per-group arrays in LDS up to this many groups (96 KB)

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

// Rank r of the cost-sorted groups goes to queue snake(r) as that queue's group r / kQueues.
__device__ __forceinline__ int snake_queue(int r) {
  const int round = r / kQueues, pos = r % kQueues;
  return (round & 1) ? kQueues - 1 - pos : pos;
}
__device__ __forceinline__ int snake_rank(int q, int j) {
  return j * kQueues + ((j & 1) ? kQueues - 1 - q : q);
}

// Exclusive scan of one value per thread over segments of `seg` consecutive
// threads (seg a multiple of 64).  Returns the exclusive prefix; *seg_total
// receives the segment's total.  Each wave scans its 64 values with lane
// shuffles; the wave totals go through LDS, so the whole scan costs two
// barriers instead of two per doubling step.
__device__ int segmented_scan(int* part, int x, int seg, int* seg_total) {
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  int incl = x;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(incl, off, 64);
    if (lane >= off) incl += y;
  }
  if (lane == 63) part[wave] = incl;             // wave totals
  __syncthreads();
  const int waves_per_seg = seg >> 6;
  const int first = wave - wave % waves_per_seg;   // first wave of this segment
  int before = 0, total = 0;
  for (int w = first; w < first + waves_per_seg; ++w) {
    const int t = part[w];
    before += w < wave ? t : 0;
    total += t;
  }
  *seg_total = total;
  __syncthreads();                                  // part is reused by the next scan
  return before + incl - x;
}

// Total cost of the nt tiles of one group member.
__device__ __forceinline__ int tiles_cost(const SchedArgs& a, int lq, int lk, int nt) {
  if (!a.causal) return nt * (a.mode == 0 ? cdiv(lk, a.loop_tile) : cdiv(lq, a.loop_tile));
  int cost = 0;
  for (int t = 0; t < nt; ++t) cost += entry_cost(a, lq, lk, t);
  return cost;
}

// One block builds one work list (block i: list i).  LDS_SCRATCH keeps the
// per-group arrays in LDS (up to kLdsGroups groups), otherwise they live in the
// list's global scratch.
template <bool LDS_SCRATCH>
__global__ __launch_bounds__(kSchedThreads) void sched_kernel(SchedBatch batch) {
  __shared__ int hist[kMaxBuckets];
  __shared__ int part[kSchedThreads];
  __shared__ int q_start[kQueues], q_size[kQueues];
  __shared__ int lds_scratch[LDS_SCRATCH ? 4 * kLdsGroups : 1];
  const SchedArgs a = batch.list[blockIdx.x];
  const int tid = threadIdx.x;
  const int nb = a.n_buckets;
  const int n_groups = a.batch * a.groups_per_seq;
  const int per_tile = a.per_tile;
  int* scratch = LDS_SCRATCH ? lds_scratch : a.scratch;
  int* g_items = scratch;                     // [n_groups] items of each group
  int* g_bucket = scratch + n_groups;         // [n_groups] cost bucket, -1 when empty
  int* order = scratch + 2 * n_groups;        // [n_groups] group of each rank
  int* r_off = scratch + 3 * n_groups;        // [n_groups] item offset of each rank in its queue

  for (int i = tid; i < nb; i += kSchedThreads) hist[i] = 0;
  __syncthreads();

  // pass 1: cost and size of every group, histogram of costs (bucket index counts
  // down so the scan sorts longest first)
  for (int gi = tid; gi < n_groups; gi += kSchedThreads) {
    const int b = gi / a.groups_per_seq;
    const int lq = a.bcast ? a.bcast_nq : a.cu_q[b + 1] - a.cu_q[b];
    const int lk = a.cu_k[b + 1] - a.cu_k[b];
    const int nt = cdiv(a.mode == 0 ? lq : lk, a.stat_tile);
    const int cost = tiles_cost(a, lq, lk, nt);
    const int n = nt * per_tile;
    g_items[gi] = n;
    int bucket = -1;
    if (n > 0) {
      bucket = nb - 1 - min(cost * per_tile, nb - 1);
      atomicAdd(&hist[bucket], 1);
    }
    g_bucket[gi] = bucket;
  }
  __syncthreads();

  // pass 2: exclusive scan of the histogram (each thread owns a contiguous run of buckets)
  {
    const int per = cdiv(nb, kSchedThreads);
    const int lo = min(tid * per, nb), hi = min(lo + per, nb);
    int run = 0;
    for (int i = lo; i < hi; ++i) run += hist[i];
    int total;
    int base = segmented_scan(part, run, kSchedThreads, &total);
    for (int i = lo; i < hi; ++i) {
      const int c = hist[i];
      hist[i] = base;
      base += c;
    }
  }
  __syncthreads();

  // pass 3: place the groups by rank
  for (int gi = tid; gi < n_groups; gi += kSchedThreads) {
    const int bucket = g_bucket[gi];
    if (bucket >= 0) order[atomicAdd(&hist[bucket], 1)] = gi;
  }
  __syncthreads();
  // after the scatter hist[nb - 1] is one past the last rank: the number of ranked groups
  const int ranked = hist[nb - 1];

  // pass 4: item offsets of the groups inside their queue (kPerQueue threads per
  // queue, each owning a contiguous run of that queue's groups)
  {
    const int q = tid / kPerQueue, i = tid % kPerQueue;
    const int per_q = cdiv(cdiv(ranked, kQueues), kPerQueue);
    const int lo = i * per_q, hi = lo + per_q;
    int run = 0;
    for (int j = lo; j < hi; ++j) {
      const int r = snake_rank(q, j);
      if (r < ranked) run += g_items[order[r]];
    }
    int q_total;
    int base = segmented_scan(part, run, kPerQueue, &q_total);
    for (int j = lo; j < hi; ++j) {
      const int r = snake_rank(q, j);
      if (r < ranked) {
        r_off[r] = base;
        base += g_items[order[r]];
      }
    }
    if (i == 0) q_size[q] = q_total;
  }
  __syncthreads();
  if (tid == 0) {
    int s = 0;
    for (int q = 0; q < kQueues; ++q) {
      const int n = max(0, min(q_size[q], a.max_items - s));
      q_start[q] = s;
      q_size[q] = n;
      s += n;
    }
  }
  __syncthreads();
  if (tid < kQueues) {
    a.queues->start[tid] = q_start[tid];
    a.queues->size[tid] = q_size[tid];
    a.queues->next[tid].value = 0u;
  }

  // pass 5: write the items of every group, tiles in descending cost order
  // (query-stationary causal tiles grow with t, key-stationary ones shrink),
  // the query heads of a tile next to each other
  for (int r = tid; r < ranked; r += kSchedThreads) {
    const int gi = order[r];
    const int q = snake_queue(r);
    const int b = gi / a.groups_per_seq, g = gi % a.groups_per_seq;
    const int n = g_items[gi];
    const int nt = n / per_tile;
    const int base = q_start[q] + r_off[r];
    const int end = min(q_start[q] + q_size[q], base + n);
    const int q_base = a.bcast ? 0 : a.cu_q[b];
    const int lq = a.bcast ? a.bcast_nq : a.cu_q[b + 1] - q_base;
    const int k_base = a.cu_k[b];
    const int lk = a.cu_k[b + 1] - k_base;
    for (int idx = 0; base + idx < end; ++idx) {
      const int tt = idx / per_tile, hi = idx % per_tile;
      WorkItem it;
      it.b = b;
      it.t = (a.causal && a.mode == 0) ? nt - 1 - tt : tt;
      it.h = g * per_tile + hi;
      it.pad = 0;
      it.q_base = q_base;
      it.lq = lq;
      it.k_base = k_base;
      it.lk = lk;
      a.items[base + idx] = it;
    }
  }
}

hipError_t launch_sched(const SchedArgs* lists, int n, hipStream_t stream) {
  if (n < 1 || n > kMaxSchedLists) return hipErrorInvalidValue;
  SchedBatch batch{};
  int64_t max_groups = 0;
  for (int i = 0; i < n; ++i) {
    const SchedArgs& a = lists[i];
    if (a.n_buckets < 1 || a.n_buckets > kMaxBuckets) return hipErrorInvalidValue;
    if (a.groups_per_seq < 1 || a.per_tile < 1 || a.batch < 0) return hipErrorInvalidValue;
    batch.list[i] = a;
    max_groups = std::max<int64_t>(max_groups, (int64_t)a.batch * a.groups_per_seq);
  }
  if (max_groups <= kLdsGroups)
    hipLaunchKernelGGL(sched_kernel<true>, dim3(n), dim3(kSchedThreads), 0, stream, batch);
  else
    hipLaunchKernelGGL(sched_kernel<false>, dim3(n), dim3(kSchedThreads), 0, stream, batch);
  return hipGetLastError();
}

}  // namespace jfa
