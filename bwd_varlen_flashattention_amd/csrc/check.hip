// Device-side checks of the input contents that the entry points take on trust:
// packed offsets (the jagged layout of "Optimizing Jagged Flash Attention with
// TLX": sequences stored back to back, boundaries in an offsets tensor) and a
// paged KV cache's lengths and page table ("Optimizing FlashAttention-4 for
// Efficient Inference", PR 1999: arbitrary page size through a page table).
// Each check is one 1024-thread workgroup that reads only the array it checks,
// within the sizes the host passes, and writes one int32 bitmask of violations
// (JFA_CHECK_* in jfa.h; 0 = valid): bad contents can make it report, never fault.
#include "jfa.h"
#include "jfa_internal.h"

namespace jfa {

constexpr int kCheckThreads = 1024;

__global__ __launch_bounds__(kCheckThreads) void check_offsets_kernel(const int32_t* cu, int32_t batch, int32_t total,
                                                                      int32_t* result) {
  __shared__ int mask;
  if (threadIdx.x == 0) mask = 0;
  __syncthreads();
  int m = 0;
  if (threadIdx.x == 0) {
    if (cu[0] != 0) m |= JFA_CHECK_OFFSETS_START;
    if (cu[batch] != total) m |= JFA_CHECK_OFFSETS_END;
  }
  for (int b = threadIdx.x; b < batch; b += kCheckThreads)
    if (cu[b + 1] < cu[b]) m |= JFA_CHECK_OFFSETS_ORDER;
  if (m) atomicOr(&mask, m);
  __syncthreads();
  if (threadIdx.x == 0) *result = mask;
}

__global__ __launch_bounds__(kCheckThreads) void check_paged_kernel(const int32_t* page_table, const int32_t* seqlens,
                                                                    int32_t batch, int32_t max_pages, int32_t page_size,
                                                                    int32_t num_pages, int32_t* result) {
  __shared__ int mask;
  if (threadIdx.x == 0) mask = 0;
  __syncthreads();
  int m = 0;
  const int64_t cap = (int64_t)max_pages * page_size;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int b = wave; b < batch; b += kCheckThreads / 64) {   // one wave per sequence
    const int32_t L = seqlens[b];
    if (L < 0 || L > cap) {
      if (lane == 0) m |= JFA_CHECK_SEQLEN_RANGE;
      continue;   // its page-table row is not read past max_pages
    }
    const int pages = (int)(((int64_t)L + page_size - 1) / page_size);
    for (int j = lane; j < pages; j += 64) {
      const int32_t id = page_table[(int64_t)b * max_pages + j];
      if (id < 0 || id >= num_pages) m |= JFA_CHECK_PAGE_RANGE;
    }
  }
  if (m) atomicOr(&mask, m);
  __syncthreads();
  if (threadIdx.x == 0) *result = mask;
}

hipError_t launch_check_offsets(const int32_t* cu, int32_t batch, int32_t total, int32_t* result, hipStream_t stream) {
  hipLaunchKernelGGL(check_offsets_kernel, dim3(1), dim3(kCheckThreads), 0, stream, cu, batch, total, result);
  return hipGetLastError();
}

hipError_t launch_check_paged(const int32_t* page_table, const int32_t* seqlens, int32_t batch, int32_t max_pages,
                              int32_t page_size, int32_t num_pages, int32_t* result, hipStream_t stream) {
  hipLaunchKernelGGL(check_paged_kernel, dim3(1), dim3(kCheckThreads), 0, stream, page_table, seqlens, batch, max_pages,
                     page_size, num_pages, result);
  return hipGetLastError();
}

}  // namespace jfa
