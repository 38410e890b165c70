// C ABI of libjfa.so (declared in include/jfa.h): argument validation, workspace
// carve-up, kernel selection and launch on the caller's stream.
//
// Head dims outside the compiled set are reported as JFA_ERR_UNSUPPORTED rather
// than failing an assertion, the failure mode that the B300 page describes for
// FlashAttention-4's head-dim support in March 2026.
#include <hip/hip_runtime.h>

#include <math.h>
#include <algorithm>

#include "jfa.h"
#include "jfa_internal.h"

using namespace jfa;

namespace {

constexpr size_t kAlign = 256;
constexpr int kMaxDevices = 64;
constexpr int kMaxBuckets = 4096;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
int cdiv_i(int64_t a, int64_t b) { return (int)((a + b - 1) / b); }

int g_cu_count[kMaxDevices] = {0};

int cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
  int n = __atomic_load_n(&g_cu_count[dev], __ATOMIC_ACQUIRE);
  if (n <= 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    __atomic_store_n(&g_cu_count[dev], n, __ATOMIC_RELEASE);
  }
  return n;
}

bool supported_dim(int d) { return d == 64 || d == 96 || d == 128 || d == 192 || d == 256; }

// ------------------------------------------------------------------ timing
// The caller's events (jfa_kernel_events_t): recorded on the call's stream around
// one kernel launch; the library keeps no reference to them.
hipError_t record(void* ev, hipStream_t s) { return ev ? hipEventRecord((hipEvent_t)ev, s) : hipSuccess; }

// ------------------------------------------------------------------ validation
bool positive_finite(float x) { return x > 0.f && !isinf(x); }   // false for NaN as well

jfa_status_t check_attn(const jfa_attn_params_t* p) {
  if (!p) return JFA_ERR_INVALID_ARGUMENT;
  if (p->batch < 1 || p->num_heads_q < 1 || p->num_heads_kv < 1) return JFA_ERR_INVALID_ARGUMENT;
  if (p->num_heads_q % p->num_heads_kv != 0) return JFA_ERR_INVALID_ARGUMENT;
  if (p->total_q < 0 || p->total_k < 0 || p->max_seqlen_q < 0 || p->max_seqlen_k < 0) return JFA_ERR_INVALID_ARGUMENT;
  if ((p->causal != 0 && p->causal != 1) || (p->broadcast_q != 0 && p->broadcast_q != 1)) return JFA_ERR_INVALID_ARGUMENT;
  if (!(p->softmax_scale == p->softmax_scale) || isinf(p->softmax_scale)) return JFA_ERR_INVALID_ARGUMENT;
  if (p->qkv_dtype != JFA_DTYPE_BF16 && p->qkv_dtype != JFA_DTYPE_FP8_E4M3) return JFA_ERR_INVALID_ARGUMENT;
  if (p->qkv_dtype == JFA_DTYPE_FP8_E4M3 && !(positive_finite(p->q_scale) && positive_finite(p->k_scale) &&
                                              positive_finite(p->v_scale)))
    return JFA_ERR_INVALID_ARGUMENT;
  if (!supported_dim(p->head_dim)) return JFA_ERR_UNSUPPORTED;
  if (p->qkv_dtype == JFA_DTYPE_FP8_E4M3 && p->head_dim % 64 != 0) return JFA_ERR_UNSUPPORTED;
  if (p->broadcast_q && p->causal) return JFA_ERR_UNSUPPORTED;
  if (p->query_tile != 0 && p->query_tile != 128 && p->query_tile != 256) return JFA_ERR_INVALID_ARGUMENT;
  // 32-bit element offsets of packed rows stay within int64 math; row counts must fit int32 tiles
  if ((int64_t)p->total_q * p->num_heads_q * p->head_dim > (int64_t)1 << 40) return JFA_ERR_INVALID_ARGUMENT;
  return JFA_OK;
}

float eff_scale(float s, int d) { return s > 0.f ? s : 1.0f / sqrtf((float)d); }

// ------------------------------------------------------------------ workspace layouts
struct SchedLayout {
  size_t items = 0, scratch = 0, queues = 0, end = 0;
  int max_items = 0;
};

// Work list of one persistent kernel: max_items items, per-group scratch for
// `groups` (sequence, KV head) groups, and the per-XCD queue descriptors.
SchedLayout sched_layout(size_t base, int64_t max_items, int64_t groups) {
  SchedLayout l;
  l.max_items = (int)max_items;
  l.items = align_up(base);
  l.scratch = align_up(l.items + (size_t)max_items * sizeof(WorkItem));
  l.queues = align_up(l.scratch + (size_t)groups * 4 * sizeof(int32_t));
  l.end = align_up(l.queues + sizeof(WorkQueues));
  return l;
}

// Tile shape per call.  When the sequences are short (mean query rows per
// sequence at most JFA_NARROW_ROWS; broadcast-Q: the shared query rows), an
// item of the 8-wave, 256-row forward / dQ workgroup is mostly empty rows and a
// few tiles long, so its time is load latency: the 4-wave, 128-row shape, two
// workgroups per CU, halves the idle rows and overlaps two items per CU.  Only
// bf16 at d = 64 / 128 has both shapes; the choice is a function of the
// parameters alone, so workspace sizing and launch agree.  A nonzero
// query_tile in the params overrides it.
#ifndef JFA_NARROW_ROWS
#define JFA_NARROW_ROWS 160
#endif
bool narrow_tiles(const jfa_attn_params_t* p) {
  if (p->qkv_dtype != JFA_DTYPE_BF16 || (p->head_dim != 64 && p->head_dim != 128)) return false;
  if (p->query_tile != 0) return p->query_tile == 128;   // the caller's choice
  if (p->broadcast_q) return p->total_q <= JFA_NARROW_ROWS;
  return (int64_t)p->total_q <= (int64_t)JFA_NARROW_ROWS * p->batch;
}

int64_t fwd_max_entries(const jfa_attn_params_t* p) {
  const int bm = fwd_block_rows(p->head_dim, p->qkv_dtype == JFA_DTYPE_FP8_E4M3, narrow_tiles(p));
  if (p->broadcast_q) return (int64_t)p->batch * cdiv_i(p->total_q, bm);
  return cdiv_i(p->total_q, bm) + (int64_t)p->batch;
}

int64_t dkdv_max_entries(const jfa_attn_params_t* p) {
  return (cdiv_i(p->total_k, bwd_dkdv_tile()) + (int64_t)p->batch) * bwd_dkdv_slices(p->head_dim);
}

int64_t dq_max_entries(const jfa_attn_params_t* p) {
  if (p->broadcast_q) return 0;   // broadcast-Q dQ work is indexed directly
  return cdiv_i(p->total_q, bwd_dq_rows(p->head_dim, narrow_tiles(p))) + (int64_t)p->batch;
}

SchedLayout fwd_list(const jfa_attn_params_t* p) {
  return sched_layout(0, fwd_max_entries(p) * p->num_heads_q, (int64_t)p->batch * p->num_heads_kv);
}

int64_t lse_elems(const jfa_attn_params_t* p) {
  return p->broadcast_q ? (int64_t)p->batch * p->num_heads_q * p->total_q : (int64_t)p->num_heads_q * p->total_q;
}

// Broadcast-Q dQ: items split into chunks, enough (query tile, head, chunk) units
// for two per CU; each chunk owns an fp32 partial of dQ.
int bcast_dq_chunks(const jfa_attn_params_t* p) {
  const int64_t tiles_heads = (int64_t)cdiv_i(p->total_q, bwd_dq_rows(p->head_dim, narrow_tiles(p))) * p->num_heads_q;
  if (tiles_heads == 0) return 0;   // no query rows: no dQ work
  const int64_t want = std::max<int64_t>(1, (2LL * cu_count() + tiles_heads - 1) / tiles_heads);
  const int per = cdiv_i(p->batch, std::min<int64_t>(p->batch, want));
  return cdiv_i(p->batch, per);
}

struct BwdLayout {
  size_t delta = 0, dq_part = 0;
  int chunks = 0;
  SchedLayout dq_list, dkdv_list;
  size_t end = 0;
};

BwdLayout bwd_layout(const jfa_attn_params_t* p) {
  BwdLayout l;
  l.delta = 0;
  size_t next = align_up((size_t)lse_elems(p) * sizeof(float));
  if (p->broadcast_q) {
    l.chunks = bcast_dq_chunks(p);
    l.dq_part = next;
    next = align_up(next + (size_t)l.chunks * p->total_q * p->num_heads_q * p->head_dim * sizeof(float));
  }
  const int64_t groups = (int64_t)p->batch * p->num_heads_kv;
  l.dq_list = sched_layout(next, dq_max_entries(p) * p->num_heads_q, p->broadcast_q ? 0 : groups);
  l.dkdv_list = sched_layout(l.dq_list.end, dkdv_max_entries(p) * p->num_heads_kv, groups);
  l.end = l.dkdv_list.end;
  return l;
}

template <typename T>
T* at(void* ws, size_t off) { return (T*)((char*)ws + off); }

// Work-list fields of the scheduler arguments shared by every launch.
void set_lists(SchedArgs& sa, const jfa_attn_params_t* p, void* ws, const SchedLayout& L) {
  // one item group per (sequence, KV head); a query-stationary tile has one item
  // per query head of the GQA group, a key-stationary tile one per head-dim slice
  sa.groups_per_seq = p->num_heads_kv;
  sa.per_tile = sa.mode == 0 ? p->num_heads_q / p->num_heads_kv : bwd_dkdv_slices(p->head_dim);
  sa.n_buckets = kMaxBuckets;
  sa.max_items = L.max_items;
  sa.scratch = at<int32_t>(ws, L.scratch);
  sa.items = at<WorkItem>(ws, L.items);
  sa.queues = at<WorkQueues>(ws, L.queues);
}

jfa_status_t hip_status(hipError_t e) { return e == hipSuccess ? JFA_OK : JFA_ERR_HIP; }

// ------------------------------------------------------------------ decode helpers
jfa_status_t check_decode(const jfa_decode_params_t* p) {
  if (!p) return JFA_ERR_INVALID_ARGUMENT;
  if (p->batch < 1 || p->num_heads_q < 1 || p->num_heads_kv < 1) return JFA_ERR_INVALID_ARGUMENT;
  if (p->num_heads_q % p->num_heads_kv != 0) return JFA_ERR_INVALID_ARGUMENT;
  if (p->page_size < 1 || p->num_pages < 1 || p->max_pages_per_seq < 1) return JFA_ERR_INVALID_ARGUMENT;
  if (p->num_splits < 0 || p->num_splits > kMaxDecodeSplits) return JFA_ERR_INVALID_ARGUMENT;
  if (!(p->softmax_scale == p->softmax_scale) || isinf(p->softmax_scale)) return JFA_ERR_INVALID_ARGUMENT;
  if (!supported_dim(p->head_dim)) return JFA_ERR_UNSUPPORTED;
  if (p->q_len < 1 || p->q_len > 16 || (p->causal != 0 && p->causal != 1)) return JFA_ERR_INVALID_ARGUMENT;
  if (p->single_launch != 0 && p->single_launch != 1) return JFA_ERR_INVALID_ARGUMENT;
  if (p->kv_dtype != JFA_KV_BF16 && p->kv_dtype != JFA_KV_FP8_E4M3) return JFA_ERR_INVALID_ARGUMENT;
  if (p->q_dtype != JFA_DTYPE_BF16 && p->q_dtype != JFA_DTYPE_FP8_E4M3) return JFA_ERR_INVALID_ARGUMENT;
  if (!(p->q_scale == p->q_scale) || isinf(p->q_scale)) return JFA_ERR_INVALID_ARGUMENT;
  if (!(p->k_scale == p->k_scale) || isinf(p->k_scale) || !(p->v_scale == p->v_scale) || isinf(p->v_scale))
    return JFA_ERR_INVALID_ARGUMENT;
  if ((int64_t)(p->num_heads_q / p->num_heads_kv) * p->q_len > 256) return JFA_ERR_UNSUPPORTED;
  if ((int64_t)p->num_pages * p->page_size * p->num_heads_kv * p->head_dim > ((int64_t)1 << 40)) return JFA_ERR_INVALID_ARGUMENT;
  return JFA_OK;
}

// Units (sequence, 16-column query unit, KV head) of one decode split: one arrival
// counter each.
int64_t decode_units(const jfa_decode_params_t* p) {
  const int cols = p->num_heads_q / p->num_heads_kv * p->q_len;
  const int64_t col_units = cdiv_i(cdiv_i(cols, 16), decode_col_groups(cols, p->head_dim));
  return (int64_t)p->batch * p->num_heads_kv * col_units;
}

int resolve_splits(const jfa_decode_params_t* p) {
  if (p->num_splits > 0) return p->num_splits;
  // about two workgroups per resident slot: the later ones fill in behind units
  // of short sequences, which balances mixed lengths
  const int cols = p->num_heads_q / p->num_heads_kv * p->q_len;
  const int64_t units = decode_units(p);
  int s = cdiv_i(2 * (int64_t)cu_count() * decode_blocks_per_cu(cols, p->head_dim), units);
  const int64_t max_len = (int64_t)p->max_pages_per_seq * p->page_size;
  const int cap = (int)std::max<int64_t>(1, (max_len + 1023) / 1024);   // at least ~1k keys per split
  if (s > cap) s = cap;
  if (s > 32) s = 32;
  if (s < 1) s = 1;
  return s;
}

// Split partials: [arrival counters, JFA_DECODE_COUNTER_BYTES][O_s fp32][LSE_s fp32].
// The counters sit at a fixed offset with a fixed size, so a workspace reused by
// decode calls of any shape keeps them zero between calls.
size_t decode_ws(const jfa_decode_params_t* p, int splits) {
  if (splits <= 1) return 0;
  const size_t plane = (size_t)p->batch * p->q_len * p->num_heads_q;
  return JFA_DECODE_COUNTER_BYTES + align_up(plane * splits * p->head_dim * sizeof(float)) +
         align_up(plane * splits * sizeof(float));
}
static_assert(JFA_DECODE_COUNTER_BYTES == kDecodeCounterSlots * sizeof(uint32_t), "counter region");
static_assert(JFA_DECODE_COUNTER_BYTES % kAlign == 0, "partials stay aligned");

// ------------------------------------------------------------------ static scratch
// jfa_decode_paged_noalloc keeps its split partials in this array instead of a
// caller workspace.  Each GPU holds its own copy for the life of the process; host
// code uses only the device address hipGetSymbolAddress reports for it (the
// array's name on the host is a stand-in, not that address), looked up once per
// device and cached.
static __device__ __align__(256) unsigned char scratch[JFA_DECODE_SCRATCH_BYTES];
void* g_scratch[kMaxDevices] = {nullptr};

jfa_status_t scratch_address(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return JFA_ERR_HIP;
  void* ptr = __atomic_load_n(&g_scratch[dev], __ATOMIC_ACQUIRE);
  if (!ptr) {
    // two threads racing here store the same address
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return JFA_ERR_HIP;
    __atomic_store_n(&g_scratch[dev], ptr, __ATOMIC_RELEASE);
  }
  *out = ptr;
  return JFA_OK;
}

}  // namespace

// ====================================================================== exported
extern "C" {

int jfa_abi_version(void) { return JFA_ABI_VERSION; }

const char* jfa_status_string(jfa_status_t s) {
  switch (s) {
    case JFA_OK: return "JFA_OK";
    case JFA_ERR_INVALID_ARGUMENT: return "JFA_ERR_INVALID_ARGUMENT";
    case JFA_ERR_UNSUPPORTED: return "JFA_ERR_UNSUPPORTED";
    case JFA_ERR_WORKSPACE_TOO_SMALL: return "JFA_ERR_WORKSPACE_TOO_SMALL";
    case JFA_ERR_HIP: return "JFA_ERR_HIP";
  }
  return "JFA_ERR_UNKNOWN";
}

size_t jfa_fwd_workspace_size(const jfa_attn_params_t* p) {
  if (check_attn(p) != JFA_OK) return 0;
  return fwd_list(p).end;
}

jfa_status_t jfa_fwd(const jfa_attn_params_t* p, const void* q, const void* k, const void* v,
                     const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, void* o, float* lse,
                     void* workspace, size_t workspace_bytes, jfa_stream_t stream_) {
  jfa_status_t st = check_attn(p);
  if (st != JFA_OK) return st;
  if (p->total_q == 0) return JFA_OK;                           // nothing to write
  if (!q || !o || !lse || !cu_seqlens_k) return JFA_ERR_INVALID_ARGUMENT;
  if (!p->broadcast_q && !cu_seqlens_q) return JFA_ERR_INVALID_ARGUMENT;
  if (p->total_k > 0 && (!k || !v)) return JFA_ERR_INVALID_ARGUMENT;
  const SchedLayout L = fwd_list(p);
  if (!workspace || ((uintptr_t)workspace % kAlign) != 0) return JFA_ERR_INVALID_ARGUMENT;
  if (workspace_bytes < L.end) return JFA_ERR_WORKSPACE_TOO_SMALL;
  hipStream_t stream = (hipStream_t)stream_;

  const int bn = fwd_kv_tile(p->head_dim);
  SchedArgs sa{};
  sa.cu_q = cu_seqlens_q;
  sa.cu_k = cu_seqlens_k;
  sa.batch = p->batch;
  const bool narrow = narrow_tiles(p);
  sa.stat_tile = fwd_block_rows(p->head_dim, p->qkv_dtype == JFA_DTYPE_FP8_E4M3, narrow);
  sa.loop_tile = bn;
  sa.mode = 0;
  sa.causal = p->causal;
  sa.bcast = p->broadcast_q;
  sa.bcast_nq = p->broadcast_q ? p->total_q : 0;
  set_lists(sa, p, workspace, L);
  hipError_t e = launch_sched(&sa, 1, stream);
  if (e != hipSuccess) return JFA_ERR_HIP;

  FwdArgs fa{};
  fa.q = (const __bf16*)q;
  fa.k = (const __bf16*)k;
  fa.v = (const __bf16*)v;
  fa.cu_q = cu_seqlens_q;
  fa.cu_k = cu_seqlens_k;
  fa.o = (__bf16*)o;
  fa.lse = lse;
  fa.items = sa.items;
  fa.queues = sa.queues;
  fa.hq = p->num_heads_q;
  fa.hkv = p->num_heads_kv;
  fa.group = p->num_heads_q / p->num_heads_kv;
  fa.bcast = sa.bcast;
  fa.bcast_nq = sa.bcast_nq;
  fa.total_q = p->total_q;
  fa.causal = p->causal;
  const bool fp8 = p->qkv_dtype == JFA_DTYPE_FP8_E4M3;
  fa.scale_log2 = eff_scale(p->softmax_scale, p->head_dim) * 1.4426950408889634f * (fp8 ? p->q_scale * p->k_scale : 1.f);
  fa.fp8 = fp8;
  fa.v_scale = fp8 ? p->v_scale : 1.f;
  fa.narrow = narrow;
  const int64_t max_items = L.max_items;
  const int grid = (int)std::min<int64_t>((int64_t)cu_count() * fwd_blocks_per_cu(p->head_dim, fp8, narrow), max_items);
  const jfa_kernel_events_t* ev = p->events;
  if (ev && record(ev->fwd_start, stream) != hipSuccess) return JFA_ERR_HIP;
  e = launch_fwd(fa, p->head_dim, std::max(grid, 1), stream);
  if (e != hipSuccess) return JFA_ERR_HIP;
  if (ev && record(ev->fwd_stop, stream) != hipSuccess) return JFA_ERR_HIP;
  return JFA_OK;
}

// The backward is a bf16 computation (e4m3 is an inference input format).
jfa_status_t check_bwd(const jfa_attn_params_t* p) {
  const jfa_status_t st = check_attn(p);
  if (st != JFA_OK) return st;
  return p->qkv_dtype == JFA_DTYPE_BF16 ? JFA_OK : JFA_ERR_UNSUPPORTED;
}

size_t jfa_bwd_workspace_size(const jfa_attn_params_t* p) {
  if (check_bwd(p) != JFA_OK) return 0;
  return bwd_layout(p).end;
}

jfa_status_t jfa_bwd(const jfa_attn_params_t* p, const void* q, const void* k, const void* v,
                     const void* o, const float* lse, const void* dout,
                     const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                     void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes, jfa_stream_t stream_) {
  jfa_status_t st = check_bwd(p);
  if (st != JFA_OK) return st;
  if (p->total_q == 0 && p->total_k == 0) return JFA_OK;
  if (!cu_seqlens_k || (!p->broadcast_q && !cu_seqlens_q)) return JFA_ERR_INVALID_ARGUMENT;
  if (p->total_q > 0 && (!q || !o || !lse || !dout || !dq)) return JFA_ERR_INVALID_ARGUMENT;
  if (p->total_k > 0 && (!k || !v || !dk || !dv)) return JFA_ERR_INVALID_ARGUMENT;
  const BwdLayout L = bwd_layout(p);
  if (!workspace || ((uintptr_t)workspace % kAlign) != 0) return JFA_ERR_INVALID_ARGUMENT;
  if (workspace_bytes < L.end) return JFA_ERR_WORKSPACE_TOO_SMALL;
  hipStream_t stream = (hipStream_t)stream_;
  const jfa_kernel_events_t* ev = p->events;
  if (p->broadcast_q && p->total_q == 0) {
    // no query rows: no key is seen by any query, so dK = dV = 0 (there is no dQ)
    const int64_t bytes = (int64_t)p->total_k * p->num_heads_kv * p->head_dim * 2;
    if (launch_zero_fill(dk, bytes, stream) != hipSuccess || launch_zero_fill(dv, bytes, stream) != hipSuccess)
      return JFA_ERR_HIP;
    return JFA_OK;
  }
  const float scale = eff_scale(p->softmax_scale, p->head_dim);
  float* delta = at<float>(workspace, L.delta);
  float* dq_part = p->broadcast_q ? at<float>(workspace, L.dq_part) : nullptr;
  const int64_t dq_elems = (int64_t)p->total_q * p->num_heads_q * p->head_dim;
  const int cus = cu_count();
  const bool narrow = narrow_tiles(p);
  const int dq_per_cu = bwd_dq_blocks_per_cu(p->head_dim, narrow);

  BwdArgs ba{};
  ba.q = (const __bf16*)q;
  ba.k = (const __bf16*)k;
  ba.v = (const __bf16*)v;
  ba.dout = (const __bf16*)dout;
  ba.o = (const __bf16*)o;
  ba.lse = lse;
  ba.delta = delta;
  ba.cu_q = cu_seqlens_q;
  ba.cu_k = cu_seqlens_k;
  ba.dq = (__bf16*)dq;
  ba.dq_part = dq_part;
  ba.dk = (__bf16*)dk;
  ba.dv = (__bf16*)dv;
  ba.batch = p->batch;
  ba.hq = p->num_heads_q;
  ba.hkv = p->num_heads_kv;
  ba.group = p->num_heads_q / p->num_heads_kv;
  ba.bcast = p->broadcast_q;
  ba.bcast_nq = p->broadcast_q ? p->total_q : 0;
  ba.total_q = p->total_q;
  ba.causal = p->causal;
  ba.scale = scale;
  ba.scale_log2 = scale * 1.4426950408889634f;
  ba.narrow = narrow;

  // Both work lists (dQ: query-stationary, dK/dV: key-stationary) in one launch.
  const bool dq_list = p->total_q > 0 && !p->broadcast_q;
  const bool dkdv_list = p->total_k > 0;
  SchedArgs lists[kMaxSchedLists];
  int n_lists = 0;
  SchedArgs dq_sa{}, dkdv_sa{};
  if (dq_list) {
    dq_sa.cu_q = cu_seqlens_q;
    dq_sa.cu_k = cu_seqlens_k;
    dq_sa.batch = p->batch;
    dq_sa.stat_tile = bwd_dq_rows(p->head_dim, narrow);
    dq_sa.loop_tile = bwd_dq_tile(p->head_dim);
    dq_sa.mode = 0;
    dq_sa.causal = p->causal;
    dq_sa.bcast = 0;
    dq_sa.bcast_nq = 0;
    set_lists(dq_sa, p, workspace, L.dq_list);
    lists[n_lists++] = dq_sa;
  }
  if (dkdv_list) {
    dkdv_sa.cu_q = cu_seqlens_q;
    dkdv_sa.cu_k = cu_seqlens_k;
    dkdv_sa.batch = p->batch;
    dkdv_sa.stat_tile = bwd_dkdv_tile();
    dkdv_sa.loop_tile = bwd_dkdv_rows(p->head_dim);
    dkdv_sa.mode = 1;
    dkdv_sa.causal = p->causal;
    dkdv_sa.bcast = p->broadcast_q;
    dkdv_sa.bcast_nq = p->broadcast_q ? p->total_q : 0;
    set_lists(dkdv_sa, p, workspace, L.dkdv_list);
    lists[n_lists++] = dkdv_sa;
  }
  hipError_t e;
  if (n_lists > 0) {
    e = launch_sched(lists, n_lists, stream);
    if (e != hipSuccess) return JFA_ERR_HIP;
  }

  if (p->total_q > 0) {
    // Broadcast-Q: delta = rowsum(dO * O) for every item.  Self-attention
    // computes delta inside the dQ kernel.
    if (p->broadcast_q) {
      BwdPreArgs pa{};
      pa.o = (const __bf16*)o;
      pa.dout = (const __bf16*)dout;
      pa.delta = delta;
      pa.rows = (int64_t)p->batch * p->total_q;   // [B, Nq] rows of O and dO
      pa.hq = p->num_heads_q;
      pa.head_dim = p->head_dim;
      pa.lse_cols = p->total_q;
      pa.bcast = 1;
      e = launch_bwd_pre(pa, stream);
      if (e != hipSuccess) return JFA_ERR_HIP;
    }

    // dQ: query-stationary
    if (p->broadcast_q) {
      const int qtiles = cdiv_i(p->total_q, bwd_dq_rows(p->head_dim, narrow));
      const int64_t tiles_heads = (int64_t)qtiles * p->num_heads_q;
      ba.bcast_chunks = L.chunks;
      ba.bcast_chunk = cdiv_i(p->batch, L.chunks);
      ba.bcast_units = (int)(tiles_heads * ba.bcast_chunks);
      if (ev && record(ev->bwd_dq_start, stream) != hipSuccess) return JFA_ERR_HIP;
      e = launch_bwd_dq(ba, p->head_dim, std::max(1, std::min(ba.bcast_units, dq_per_cu * cus)), stream);
      if (e != hipSuccess) return JFA_ERR_HIP;
      if (ev && record(ev->bwd_dq_stop, stream) != hipSuccess) return JFA_ERR_HIP;
    } else {
      ba.items = dq_sa.items;
      ba.queues = dq_sa.queues;
      const int64_t max_items = L.dq_list.max_items;
      if (ev && record(ev->bwd_dq_start, stream) != hipSuccess) return JFA_ERR_HIP;
      e = launch_bwd_dq(ba, p->head_dim, (int)std::max<int64_t>(1, std::min<int64_t>((int64_t)dq_per_cu * cus, max_items)), stream);
      if (e != hipSuccess) return JFA_ERR_HIP;
      if (ev && record(ev->bwd_dq_stop, stream) != hipSuccess) return JFA_ERR_HIP;
    }
  }

  if (p->total_k > 0) {
    // dK, dV: key-stationary
    ba.items = dkdv_sa.items;
    ba.queues = dkdv_sa.queues;
    const int64_t max_items = L.dkdv_list.max_items;
    if (ev && record(ev->bwd_dkdv_start, stream) != hipSuccess) return JFA_ERR_HIP;
    e = launch_bwd_dkdv(ba, p->head_dim, (int)std::max<int64_t>(1, std::min<int64_t>(cus, max_items)), stream);
    if (e != hipSuccess) return JFA_ERR_HIP;
    if (ev && record(ev->bwd_dkdv_stop, stream) != hipSuccess) return JFA_ERR_HIP;
  }

  if (p->broadcast_q && p->total_q > 0) {
    DqConvertArgs ca{};
    ca.dq_part = dq_part;
    ca.dq = (__bf16*)dq;
    ca.n = dq_elems;
    ca.chunks = L.chunks;
    ca.scale = scale;
    e = launch_dq_convert(ca, stream);
    if (e != hipSuccess) return JFA_ERR_HIP;
  }
  return JFA_OK;
}

jfa_status_t jfa_check_offsets(const int32_t* offsets, int32_t batch, int32_t total, int32_t* result,
                               jfa_stream_t stream) {
  if (!offsets || !result || batch < 0 || total < 0) return JFA_ERR_INVALID_ARGUMENT;
  return hip_status(launch_check_offsets(offsets, batch, total, result, (hipStream_t)stream));
}

jfa_status_t jfa_check_paged_cache(const jfa_decode_params_t* p, const int32_t* page_table,
                                   const int32_t* seqlens_k, int32_t* result, jfa_stream_t stream) {
  if (!p || !page_table || !seqlens_k || !result) return JFA_ERR_INVALID_ARGUMENT;
  if (p->batch < 1 || p->page_size < 1 || p->num_pages < 1 || p->max_pages_per_seq < 1) return JFA_ERR_INVALID_ARGUMENT;
  return hip_status(launch_check_paged(page_table, seqlens_k, p->batch, p->max_pages_per_seq, p->page_size,
                                       p->num_pages, result, (hipStream_t)stream));
}

int32_t jfa_decode_num_splits(const jfa_decode_params_t* p) {
  if (check_decode(p) != JFA_OK) return 0;
  return resolve_splits(p);
}

size_t jfa_decode_workspace_size(const jfa_decode_params_t* p) {
  if (check_decode(p) != JFA_OK) return 0;
  return decode_ws(p, resolve_splits(p));
}

jfa_status_t jfa_decode_paged_noalloc(const jfa_decode_params_t* p, const void* q, const void* k_cache,
                                      const void* v_cache, const int32_t* page_table, const int32_t* seqlens_k,
                                      void* o, float* lse, jfa_stream_t stream) {
  const jfa_status_t st = check_decode(p);
  if (st != JFA_OK) return st;
  if (decode_ws(p, resolve_splits(p)) > JFA_DECODE_SCRATCH_BYTES) return JFA_ERR_WORKSPACE_TOO_SMALL;
  void* ptr = nullptr;
  if (scratch_address(&ptr) != JFA_OK) return JFA_ERR_HIP;
  return jfa_decode_paged(p, q, k_cache, v_cache, page_table, seqlens_k, o, lse, ptr, JFA_DECODE_SCRATCH_BYTES,
                          stream);
}

jfa_status_t jfa_decode_paged(const jfa_decode_params_t* p, const void* q, const void* k_cache,
                              const void* v_cache, const int32_t* page_table, const int32_t* seqlens_k,
                              void* o, float* lse, void* workspace, size_t workspace_bytes,
                              jfa_stream_t stream_) {
  jfa_status_t st = check_decode(p);
  if (st != JFA_OK) return st;
  if (!q || !k_cache || !v_cache || !page_table || !seqlens_k || !o || !lse) return JFA_ERR_INVALID_ARGUMENT;
  const int splits = resolve_splits(p);
  const size_t need = decode_ws(p, splits);
  if (need > 0 && (!workspace || ((uintptr_t)workspace % kAlign) != 0)) return JFA_ERR_INVALID_ARGUMENT;
  if (workspace_bytes < need) return JFA_ERR_WORKSPACE_TOO_SMALL;
  hipStream_t stream = (hipStream_t)stream_;

  DecodeArgs a{};
  a.q = (const __bf16*)q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.page_table = page_table;
  a.seqlens = seqlens_k;
  a.o = (__bf16*)o;
  a.lse = lse;
  const size_t plane = (size_t)p->batch * p->q_len * p->num_heads_q;
  char* parts = splits > 1 ? (char*)workspace + JFA_DECODE_COUNTER_BYTES : nullptr;
  a.o_part = (float*)parts;
  a.lse_part = splits > 1 ? (float*)(parts + align_up(plane * splits * p->head_dim * sizeof(float))) : nullptr;
  // single-launch mode: the last split of each unit merges inside the decode
  // launch, unless there are more units than counters (then, as by default,
  // decode_combine_kernel runs after the decode kernel)
  const bool fused = p->single_launch == 1 && splits > 1 && decode_units(p) <= kDecodeCounterSlots;
  a.counters = fused ? (uint32_t*)workspace : nullptr;
  a.batch = p->batch;
  a.hq = p->num_heads_q;
  a.hkv = p->num_heads_kv;
  a.group = p->num_heads_q / p->num_heads_kv;
  a.page_size = p->page_size;
  a.max_pages = p->max_pages_per_seq;
  a.splits = splits;
  a.q_len = p->q_len;
  a.causal = p->causal;
  a.kv_fp8 = p->kv_dtype == JFA_KV_FP8_E4M3;
  a.q_fp8 = p->q_dtype == JFA_DTYPE_FP8_E4M3;
  const float k_scale = (a.kv_fp8 && p->k_scale > 0.f) ? p->k_scale : 1.f;
  const float q_scale = (a.q_fp8 && p->q_scale > 0.f) ? p->q_scale : 1.f;
  a.v_scale = (a.kv_fp8 && p->v_scale > 0.f) ? p->v_scale : 1.f;
  a.scale_log2 = eff_scale(p->softmax_scale, p->head_dim) * 1.4426950408889634f * k_scale * q_scale;
  const jfa_kernel_events_t* ev = p->events;
  if (ev && record(ev->decode_start, stream) != hipSuccess) return JFA_ERR_HIP;
  hipError_t e = launch_decode(a, p->head_dim, stream);
  if (e != hipSuccess) return JFA_ERR_HIP;
  if (ev && record(ev->decode_stop, stream) != hipSuccess) return JFA_ERR_HIP;
  if (splits > 1 && !fused) {
    e = launch_decode_combine(a, p->head_dim, stream);
    if (e != hipSuccess) return JFA_ERR_HIP;
  }
  return JFA_OK;
}

}  // extern "C"
