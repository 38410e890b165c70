// C ABI of libjfa.so (declared in include/jfa.h): argument validation, workspace
// carve-up, kernel selection and launch on the caller's stream.
//
// Head dims outside the compiled set are reported as JFA_ERR_UNSUPPORTED rather
// than failing an assertion, the failure mode that the B300 page describes for
// FlashAttention-4's head-dim support in March 2026.
#include <hip/hip_runtime.h>

#include <math.h>
#include <algorithm>
#include <mutex>
#include <vector>

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

bool supported_dim(int d) { return d == 64 || d == 96 || d == 128; }

// ------------------------------------------------------------------ timing
struct Timing {
  std::mutex mu;
  bool enabled = false;
  std::vector<hipEvent_t> start[JFA_TIMING_SLOTS], stop[JFA_TIMING_SLOTS];
};
Timing& timing() {
  static Timing t;
  return t;
}

struct TimedRegion {
  int which;
  hipStream_t stream;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  TimedRegion(int w, hipStream_t s) : which(w), stream(s) {
    Timing& t = timing();
    std::lock_guard<std::mutex> g(t.mu);
    if (!t.enabled) return;
    if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) { e0 = e1 = nullptr; return; }
    hipEventRecord(e0, stream);
  }
  void finish() {
    if (!e0) return;
    hipEventRecord(e1, stream);
    Timing& t = timing();
    std::lock_guard<std::mutex> g(t.mu);
    t.start[which].push_back(e0);
    t.stop[which].push_back(e1);
    e0 = e1 = nullptr;
  }
};

// ------------------------------------------------------------------ validation
jfa_status_t check_attn(const jfa_attn_params_t* p) {
  if (!p) return JFA_ERR_INVALID_ARGUMENT;
  if (p->batch < 1 || p->num_heads_q < 1 || p->num_heads_kv < 1) return JFA_ERR_INVALID_ARGUMENT;
  if (p->num_heads_q % p->num_heads_kv != 0) return JFA_ERR_INVALID_ARGUMENT;
  if (p->total_q < 0 || p->total_k < 0 || p->max_seqlen_q < 0 || p->max_seqlen_k < 0) return JFA_ERR_INVALID_ARGUMENT;
  if ((p->causal != 0 && p->causal != 1) || (p->broadcast_q != 0 && p->broadcast_q != 1)) return JFA_ERR_INVALID_ARGUMENT;
  if (!(p->softmax_scale == p->softmax_scale) || isinf(p->softmax_scale)) return JFA_ERR_INVALID_ARGUMENT;
  if (!supported_dim(p->head_dim)) return JFA_ERR_UNSUPPORTED;
  if (p->broadcast_q && p->causal) return JFA_ERR_UNSUPPORTED;
  // 32-bit element offsets of packed rows stay within int64 math; row counts must fit int32 tiles
  if ((int64_t)p->total_q * p->num_heads_q * p->head_dim > (int64_t)1 << 40) return JFA_ERR_INVALID_ARGUMENT;
  return JFA_OK;
}

float eff_scale(float s, int d) { return s > 0.f ? s : 1.0f / sqrtf((float)d); }

// ------------------------------------------------------------------ workspace layouts
struct SchedLayout {
  size_t entries = 0, n_entries = 0, counter = 0, end = 0;
  int max_entries = 0;
};

SchedLayout sched_layout(size_t base, int64_t max_entries) {
  SchedLayout l;
  l.max_entries = (int)max_entries;
  l.entries = base;
  l.n_entries = align_up(l.entries + (size_t)max_entries * sizeof(WorkEntry));
  l.counter = align_up(l.n_entries + sizeof(int32_t));
  l.end = align_up(l.counter + sizeof(uint32_t));
  return l;
}

int64_t fwd_max_entries(const jfa_attn_params_t* p) {
  const int bm = fwd_block_rows();
  if (p->broadcast_q) return (int64_t)p->batch * cdiv_i(p->total_q, bm);
  return cdiv_i(p->total_q, bm) + (int64_t)p->batch;
}

int64_t dkdv_max_entries(const jfa_attn_params_t* p) {
  return cdiv_i(p->total_k, bwd_dkdv_tile()) + (int64_t)p->batch;
}

int64_t dq_max_entries(const jfa_attn_params_t* p) {
  if (p->broadcast_q) return 0;   // broadcast-Q dQ work is indexed directly
  return cdiv_i(p->total_q, bwd_dq_rows()) + (int64_t)p->batch;
}

int64_t lse_elems(const jfa_attn_params_t* p) {
  return p->broadcast_q ? (int64_t)p->batch * p->num_heads_q * p->total_q : (int64_t)p->num_heads_q * p->total_q;
}

struct BwdLayout {
  size_t delta = 0, dq_acc = 0;
  SchedLayout dq_list, dkdv_list;
  size_t end = 0;
};

BwdLayout bwd_layout(const jfa_attn_params_t* p) {
  BwdLayout l;
  l.delta = 0;
  size_t next = align_up((size_t)lse_elems(p) * sizeof(float));
  if (p->broadcast_q) {
    l.dq_acc = next;
    next = align_up(next + (size_t)p->total_q * p->num_heads_q * p->head_dim * sizeof(float));
  }
  l.dq_list = sched_layout(next, dq_max_entries(p));
  l.dkdv_list = sched_layout(l.dq_list.end, dkdv_max_entries(p));
  l.end = l.dkdv_list.end;
  return l;
}

template <typename T>
T* at(void* ws, size_t off) { return (T*)((char*)ws + off); }

jfa_status_t hip_status(hipError_t e) { return e == hipSuccess ? JFA_OK : JFA_ERR_HIP; }

// ------------------------------------------------------------------ decode helpers
jfa_status_t check_decode(const jfa_decode_params_t* p) {
  if (!p) return JFA_ERR_INVALID_ARGUMENT;
  if (p->batch < 1 || p->num_heads_q < 1 || p->num_heads_kv < 1) return JFA_ERR_INVALID_ARGUMENT;
  if (p->num_heads_q % p->num_heads_kv != 0) return JFA_ERR_INVALID_ARGUMENT;
  if (p->page_size < 1 || p->num_pages < 1 || p->max_pages_per_seq < 1) return JFA_ERR_INVALID_ARGUMENT;
  if (p->num_splits < 0 || p->num_splits > 128) return JFA_ERR_INVALID_ARGUMENT;
  if (!(p->softmax_scale == p->softmax_scale) || isinf(p->softmax_scale)) return JFA_ERR_INVALID_ARGUMENT;
  if (!supported_dim(p->head_dim)) return JFA_ERR_UNSUPPORTED;
  if (p->num_heads_q / p->num_heads_kv > 16) return JFA_ERR_UNSUPPORTED;
  if ((int64_t)p->num_pages * p->page_size * p->num_heads_kv * p->head_dim > ((int64_t)1 << 40)) return JFA_ERR_INVALID_ARGUMENT;
  return JFA_OK;
}

int resolve_splits(const jfa_decode_params_t* p) {
  if (p->num_splits > 0) return p->num_splits;
  const int64_t units = (int64_t)p->batch * p->num_heads_kv;
  int s = cdiv_i(4 * (int64_t)cu_count(), units);
  const int64_t max_len = (int64_t)p->max_pages_per_seq * p->page_size;
  const int cap = (int)std::max<int64_t>(1, (max_len + 1023) / 1024);   // at least ~1k keys per split
  if (s > cap) s = cap;
  if (s > 32) s = 32;
  if (s < 1) s = 1;
  return s;
}

size_t decode_ws(const jfa_decode_params_t* p, int splits) {
  if (splits <= 1) return 0;
  const size_t plane = (size_t)p->batch * p->num_heads_q;
  return align_up(plane * splits * p->head_dim * sizeof(float)) + align_up(plane * splits * sizeof(float));
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
  return sched_layout(0, fwd_max_entries(p)).end;
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
  const SchedLayout L = sched_layout(0, fwd_max_entries(p));
  if (!workspace) return JFA_ERR_INVALID_ARGUMENT;
  if (workspace_bytes < L.end) return JFA_ERR_WORKSPACE_TOO_SMALL;
  hipStream_t stream = (hipStream_t)stream_;

  const int bn = fwd_kv_tile();
  SchedArgs sa{};
  sa.cu_q = cu_seqlens_q;
  sa.cu_k = cu_seqlens_k;
  sa.batch = p->batch;
  sa.stat_tile = fwd_block_rows();
  sa.loop_tile = bn;
  sa.mode = 0;
  sa.causal = p->causal;
  sa.bcast_nq = p->broadcast_q ? p->total_q : 0;
  sa.n_buckets = std::min(kMaxBuckets, cdiv_i(p->max_seqlen_k, bn) + 1);
  sa.max_entries = L.max_entries;
  sa.entries = at<WorkEntry>(workspace, L.entries);
  sa.n_entries = at<int32_t>(workspace, L.n_entries);
  sa.counter = at<uint32_t>(workspace, L.counter);
  hipError_t e = launch_sched(sa, stream);
  if (e != hipSuccess) return JFA_ERR_HIP;

  FwdArgs fa{};
  fa.q = (const __bf16*)q;
  fa.k = (const __bf16*)k;
  fa.v = (const __bf16*)v;
  fa.cu_q = cu_seqlens_q;
  fa.cu_k = cu_seqlens_k;
  fa.o = (__bf16*)o;
  fa.lse = lse;
  fa.entries = sa.entries;
  fa.n_entries = sa.n_entries;
  fa.counter = sa.counter;
  fa.hq = p->num_heads_q;
  fa.hkv = p->num_heads_kv;
  fa.group = p->num_heads_q / p->num_heads_kv;
  fa.bcast_nq = sa.bcast_nq;
  fa.total_q = p->total_q;
  fa.causal = p->causal;
  fa.scale_log2 = eff_scale(p->softmax_scale, p->head_dim) * 1.4426950408889634f;
  const int64_t max_items = (int64_t)L.max_entries * p->num_heads_q;
  const int grid = (int)std::min<int64_t>((int64_t)cu_count() * fwd_blocks_per_cu(p->head_dim), max_items);
  TimedRegion tr(JFA_TIMING_FWD, stream);
  e = launch_fwd(fa, p->head_dim, std::max(grid, 1), stream);
  tr.finish();
  return hip_status(e);
}

size_t jfa_bwd_workspace_size(const jfa_attn_params_t* p) {
  if (check_attn(p) != JFA_OK) return 0;
  return bwd_layout(p).end;
}

jfa_status_t jfa_bwd(const jfa_attn_params_t* p, const void* q, const void* k, const void* v,
                     const void* o, const float* lse, const void* dout,
                     const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                     void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes, jfa_stream_t stream_) {
  jfa_status_t st = check_attn(p);
  if (st != JFA_OK) return st;
  if (p->total_q == 0 && p->total_k == 0) return JFA_OK;
  if (!cu_seqlens_k || (!p->broadcast_q && !cu_seqlens_q)) return JFA_ERR_INVALID_ARGUMENT;
  if (p->total_q > 0 && (!q || !o || !lse || !dout || !dq)) return JFA_ERR_INVALID_ARGUMENT;
  if (p->total_k > 0 && (!k || !v || !dk || !dv)) return JFA_ERR_INVALID_ARGUMENT;
  const BwdLayout L = bwd_layout(p);
  if (!workspace) return JFA_ERR_INVALID_ARGUMENT;
  if (workspace_bytes < L.end) return JFA_ERR_WORKSPACE_TOO_SMALL;
  hipStream_t stream = (hipStream_t)stream_;
  const float scale = eff_scale(p->softmax_scale, p->head_dim);
  float* delta = at<float>(workspace, L.delta);
  float* dq_acc = p->broadcast_q ? at<float>(workspace, L.dq_acc) : nullptr;
  const int64_t dq_elems = (int64_t)p->total_q * p->num_heads_q * p->head_dim;
  const int cus = cu_count();

  BwdArgs ba{};
  ba.q = (const __bf16*)q;
  ba.k = (const __bf16*)k;
  ba.v = (const __bf16*)v;
  ba.dout = (const __bf16*)dout;
  ba.lse = lse;
  ba.delta = delta;
  ba.cu_q = cu_seqlens_q;
  ba.cu_k = cu_seqlens_k;
  ba.dq = (__bf16*)dq;
  ba.dq_acc = dq_acc;
  ba.dk = (__bf16*)dk;
  ba.dv = (__bf16*)dv;
  ba.batch = p->batch;
  ba.hq = p->num_heads_q;
  ba.hkv = p->num_heads_kv;
  ba.group = p->num_heads_q / p->num_heads_kv;
  ba.bcast_nq = p->broadcast_q ? p->total_q : 0;
  ba.total_q = p->total_q;
  ba.causal = p->causal;
  ba.scale = scale;
  ba.scale_log2 = scale * 1.4426950408889634f;

  hipError_t e;
  if (p->total_q > 0) {
    // delta = rowsum(dO * O); for broadcast-Q also zero the fp32 dQ accumulator
    BwdPreArgs pa{};
    pa.o = (const __bf16*)o;
    pa.dout = (const __bf16*)dout;
    pa.delta = delta;
    pa.dq_acc = dq_acc;
    pa.rows = p->broadcast_q ? (int64_t)p->batch * p->total_q : p->total_q;
    pa.hq = p->num_heads_q;
    pa.head_dim = p->head_dim;
    pa.lse_cols = p->total_q;
    pa.bcast = p->broadcast_q;
    pa.dq_elems = dq_elems;
    e = launch_bwd_pre(pa, stream);
    if (e != hipSuccess) return JFA_ERR_HIP;

    // dQ: query-stationary
    if (p->broadcast_q) {
      const int qtiles = cdiv_i(p->total_q, bwd_dq_rows());
      const int64_t tiles_heads = (int64_t)qtiles * p->num_heads_q;
      int chunks = (int)std::min<int64_t>(p->batch, std::max<int64_t>(1, (2LL * cus + tiles_heads - 1) / tiles_heads));
      ba.bcast_chunk = cdiv_i(p->batch, chunks);
      ba.bcast_chunks = cdiv_i(p->batch, ba.bcast_chunk);
      ba.bcast_units = (int)(tiles_heads * ba.bcast_chunks);
      TimedRegion tr(JFA_TIMING_BWD_DQ, stream);
      e = launch_bwd_dq(ba, p->head_dim, std::max(1, std::min(ba.bcast_units, 2 * cus)), stream);
      tr.finish();
      if (e != hipSuccess) return JFA_ERR_HIP;
    } else {
      SchedArgs sa{};
      sa.cu_q = cu_seqlens_q;
      sa.cu_k = cu_seqlens_k;
      sa.batch = p->batch;
      sa.stat_tile = bwd_dq_rows();
      sa.loop_tile = bwd_dq_tile();
      sa.mode = 0;
      sa.causal = p->causal;
      sa.bcast_nq = 0;
      sa.n_buckets = std::min(kMaxBuckets, cdiv_i(p->max_seqlen_k, bwd_dq_tile()) + 1);
      sa.max_entries = L.dq_list.max_entries;
      sa.entries = at<WorkEntry>(workspace, L.dq_list.entries);
      sa.n_entries = at<int32_t>(workspace, L.dq_list.n_entries);
      sa.counter = at<uint32_t>(workspace, L.dq_list.counter);
      e = launch_sched(sa, stream);
      if (e != hipSuccess) return JFA_ERR_HIP;
      ba.entries = sa.entries;
      ba.n_entries = sa.n_entries;
      ba.counter = sa.counter;
      const int64_t max_items = (int64_t)L.dq_list.max_entries * p->num_heads_q;
      TimedRegion tr(JFA_TIMING_BWD_DQ, stream);
      e = launch_bwd_dq(ba, p->head_dim, (int)std::max<int64_t>(1, std::min<int64_t>(2LL * cus, max_items)), stream);
      tr.finish();
      if (e != hipSuccess) return JFA_ERR_HIP;
    }
  }

  if (p->total_k > 0) {
    // dK, dV: key-stationary
    SchedArgs sa{};
    sa.cu_q = cu_seqlens_q;
    sa.cu_k = cu_seqlens_k;
    sa.batch = p->batch;
    sa.stat_tile = bwd_dkdv_tile();
    sa.loop_tile = bwd_dkdv_rows();
    sa.mode = 1;
    sa.causal = p->causal;
    sa.bcast_nq = p->broadcast_q ? p->total_q : 0;
    const int maxq = p->broadcast_q ? p->total_q : p->max_seqlen_q;
    sa.n_buckets = std::min(kMaxBuckets, cdiv_i(maxq, bwd_dkdv_rows()) + 1);
    sa.max_entries = L.dkdv_list.max_entries;
    sa.entries = at<WorkEntry>(workspace, L.dkdv_list.entries);
    sa.n_entries = at<int32_t>(workspace, L.dkdv_list.n_entries);
    sa.counter = at<uint32_t>(workspace, L.dkdv_list.counter);
    e = launch_sched(sa, stream);
    if (e != hipSuccess) return JFA_ERR_HIP;
    ba.entries = sa.entries;
    ba.n_entries = sa.n_entries;
    ba.counter = sa.counter;
    const int64_t max_items = (int64_t)L.dkdv_list.max_entries * p->num_heads_kv;
    TimedRegion tr(JFA_TIMING_BWD_DKDV, stream);
    e = launch_bwd_dkdv(ba, p->head_dim, (int)std::max<int64_t>(1, std::min<int64_t>(cus, max_items)), stream);
    tr.finish();
    if (e != hipSuccess) return JFA_ERR_HIP;
  }

  if (p->broadcast_q && p->total_q > 0) {
    DqConvertArgs ca{};
    ca.dq_acc = dq_acc;
    ca.dq = (__bf16*)dq;
    ca.n = dq_elems;
    ca.scale = scale;
    e = launch_dq_convert(ca, stream);
    if (e != hipSuccess) return JFA_ERR_HIP;
  }
  return JFA_OK;
}

int32_t jfa_decode_num_splits(const jfa_decode_params_t* p) {
  if (check_decode(p) != JFA_OK) return 0;
  return resolve_splits(p);
}

size_t jfa_decode_workspace_size(const jfa_decode_params_t* p) {
  if (check_decode(p) != JFA_OK) return 0;
  return decode_ws(p, resolve_splits(p));
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
  if (need > 0 && !workspace) return JFA_ERR_INVALID_ARGUMENT;
  if (workspace_bytes < need) return JFA_ERR_WORKSPACE_TOO_SMALL;
  hipStream_t stream = (hipStream_t)stream_;

  DecodeArgs a{};
  a.q = (const __bf16*)q;
  a.k_cache = (const __bf16*)k_cache;
  a.v_cache = (const __bf16*)v_cache;
  a.page_table = page_table;
  a.seqlens = seqlens_k;
  a.o = (__bf16*)o;
  a.lse = lse;
  const size_t plane = (size_t)p->batch * p->num_heads_q;
  a.o_part = splits > 1 ? (float*)workspace : nullptr;
  a.lse_part = splits > 1 ? (float*)((char*)workspace + align_up(plane * splits * p->head_dim * sizeof(float))) : nullptr;
  a.batch = p->batch;
  a.hq = p->num_heads_q;
  a.hkv = p->num_heads_kv;
  a.group = p->num_heads_q / p->num_heads_kv;
  a.page_size = p->page_size;
  a.max_pages = p->max_pages_per_seq;
  a.splits = splits;
  a.scale_log2 = eff_scale(p->softmax_scale, p->head_dim) * 1.4426950408889634f;
  TimedRegion tr(JFA_TIMING_DECODE, stream);
  hipError_t e = launch_decode(a, p->head_dim, stream);
  tr.finish();
  if (e != hipSuccess) return JFA_ERR_HIP;
  if (splits > 1) {
    e = launch_decode_combine(a, p->head_dim, stream);
    if (e != hipSuccess) return JFA_ERR_HIP;
  }
  return JFA_OK;
}

jfa_status_t jfa_timing_enable(int enable) {
  Timing& t = timing();
  std::lock_guard<std::mutex> g(t.mu);
  t.enabled = enable != 0;
  return JFA_OK;
}

jfa_status_t jfa_timing_collect(double total_ms[JFA_TIMING_SLOTS], int64_t count[JFA_TIMING_SLOTS]) {
  Timing& t = timing();
  std::lock_guard<std::mutex> g(t.mu);
  jfa_status_t st = JFA_OK;
  for (int w = 0; w < JFA_TIMING_SLOTS; ++w) {
    double ms_sum = 0.0;
    int64_t n = 0;
    for (size_t i = 0; i < t.start[w].size(); ++i) {
      float ms = 0.f;
      if (hipEventSynchronize(t.stop[w][i]) != hipSuccess ||
          hipEventElapsedTime(&ms, t.start[w][i], t.stop[w][i]) != hipSuccess) {
        st = JFA_ERR_HIP;
      } else {
        ms_sum += ms;
        ++n;
      }
      hipEventDestroy(t.start[w][i]);
      hipEventDestroy(t.stop[w][i]);
    }
    t.start[w].clear();
    t.stop[w].clear();
    if (total_ms) total_ms[w] = ms_sum;
    if (count) count[w] = n;
  }
  return st;
}

}  // extern "C"
