// Internal (host-side) interface between the C ABI layer and the kernel launchers.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace jfa {

// Workgroups are dispatched to the MI355X's 8 XCDs (each with its own L2) round
// robin by block index.
constexpr int kXcds = 8;

// Work queues: one per XCD.  Block i serves queue i % kQueues first and steals
// from the others when its own queue runs dry.
constexpr int kQueues = kXcds;

// One work item: sequence b, tile t, head (or head/slice) h, and the sequence's
// packed offsets and lengths, so a consumer needs one 32-byte load per item.
struct WorkItem {
  int32_t b;
  int32_t t;
  int32_t h;
  int32_t pad;
  int32_t q_base;   // first packed query row (broadcast-Q: 0)
  int32_t lq;       // query rows (broadcast-Q: Nq)
  int32_t k_base;   // first packed key row
  int32_t lk;       // key rows
};

// Queue descriptors.  start/size are read once per workgroup; each consumer
// counter sits on a 256-byte line of its own, because every item hand-out is an
// atomic on it and a shared line becomes the bottleneck of the whole grid.
struct QueueCounter {
  uint32_t value;
  uint32_t pad[63];
};
struct WorkQueues {
  int32_t start[kQueues];   // first item of each queue in the item array
  int32_t size[kQueues];    // items in each queue
  uint32_t pad[64 - 2 * kQueues];
  QueueCounter next[kQueues];   // consumer counters (reset by the scheduler)
};

// Shape of the work list built on the device from the offsets.
struct SchedArgs {
  const int32_t* cu_q;      // [B+1] (unused in broadcast-Q mode)
  const int32_t* cu_k;      // [B+1]
  int32_t batch;
  int32_t groups_per_seq;   // item groups per sequence (the tiles of a group share K/V or Q/dO)
  int32_t per_tile;         // items per tile of a group: head h = (group index) * per_tile + i
  int32_t stat_tile;        // rows per tile on the stationary axis
  int32_t loop_tile;        // rows per tile on the inner-loop axis
  int32_t mode;             // 0: query-stationary (one item per query head), 1: key-stationary (per KV head)
  int32_t causal;
  int32_t bcast;            // 1: broadcast-Q (cu_q is not read)
  int32_t bcast_nq;         // broadcast-Q: every item has Lq = bcast_nq
  int32_t n_buckets;        // cost buckets (costs above are clamped into the last one)
  int32_t max_items;        // capacity of `items`
  int32_t* scratch;         // 4 * batch * groups_per_seq ints (used when they do not fit in LDS)
  WorkItem* items;          // queue by queue
  WorkQueues* queues;
};

// Several work lists built by one launch (one block each).
constexpr int kMaxSchedLists = 2;
struct SchedBatch {
  SchedArgs list[kMaxSchedLists];
};
hipError_t launch_sched(const SchedArgs* lists, int n, hipStream_t stream);

// Forward kernel arguments.
struct FwdArgs {
  const __bf16* q;
  const __bf16* k;
  const __bf16* v;
  const int32_t* cu_q;
  const int32_t* cu_k;
  __bf16* o;
  float* lse;
  const WorkItem* items;
  WorkQueues* queues;
  int32_t hq, hkv, group;   // group = hq / hkv
  int32_t bcast;            // 1: broadcast-Q
  int32_t bcast_nq;         // broadcast-Q: query rows shared by every item
  int32_t total_q;          // LSE row stride for self-attention
  int32_t causal;
  float scale_log2;         // softmax scale * log2(e) (e4m3: times the Q and K scales)
  int32_t fp8;              // Q, K, V are e4m3 bytes
  float v_scale;            // e4m3: V scale, applied to O
  int32_t narrow;           // 1: the 4-wave, 128-row workgroups (short sequences; d = 64 / 128, bf16)
};

hipError_t launch_fwd(const FwdArgs& a, int head_dim, int grid, hipStream_t stream);
// forward kernels of the iterative-ILP unit (causal d = 128, all d >= 192); called by launch_fwd
hipError_t launch_fwd_ilp(const FwdArgs& a, int head_dim, bool fp8, int grid, hipStream_t stream);
int fwd_block_rows(int head_dim, bool fp8, bool narrow);   // BM of the forward kernel
int fwd_kv_tile(int head_dim);   // BN of the forward kernel
int fwd_blocks_per_cu(int head_dim, bool fp8, bool narrow);

// Backward.
struct BwdPreArgs {
  const __bf16* o;
  const __bf16* dout;
  float* delta;             // same layout as lse
  int64_t rows;             // rows of o / dout (self: total_q, broadcast: B * Nq)
  int32_t hq;
  int32_t head_dim;
  int32_t lse_cols;         // self: total_q; broadcast: Nq
  int32_t bcast;
};
hipError_t launch_bwd_pre(const BwdPreArgs& a, hipStream_t stream);

struct BwdArgs {
  const __bf16* q;
  const __bf16* k;
  const __bf16* v;
  const __bf16* dout;
  const __bf16* o;          // forward output: the self-attention dQ kernel computes delta from it
  const float* lse;
  float* delta;             // broadcast-Q: written by bwd_pre_kernel; self-attention: by the dQ kernel
  const int32_t* cu_q;
  const int32_t* cu_k;
  __bf16* dq;
  float* dq_part;           // broadcast-Q: fp32 dQ partial per chunk of items [chunks, Nq, Hq, d]
  __bf16* dk;
  __bf16* dv;
  const WorkItem* items;    // work list of the kernel being launched
  WorkQueues* queues;
  int32_t batch;
  int32_t hq, hkv, group;
  int32_t bcast;            // 1: broadcast-Q
  int32_t bcast_nq;         // broadcast-Q: query rows shared by every item
  int32_t bcast_chunk;      // broadcast-Q dQ: items per chunk
  int32_t bcast_chunks;     // number of chunks
  int32_t bcast_units;      // query tiles * heads * chunks
  int32_t total_q;
  int32_t causal;
  float scale;
  float scale_log2;
  int32_t narrow;           // dQ, d = 128: the 4-wave, 128-row workgroups (short sequences)
};
hipError_t launch_bwd_dkdv(const BwdArgs& a, int head_dim, int grid, hipStream_t stream);
hipError_t launch_bwd_dq(const BwdArgs& a, int head_dim, int grid, hipStream_t stream);
// emitted by bwd_wide.hip (called by the two above): dK/dV at d = 192 and 256,
// dQ at d = 192
hipError_t launch_bwd_dkdv_wide(const BwdArgs& a, int head_dim, int grid, hipStream_t stream);
hipError_t launch_bwd_dq_wide(const BwdArgs& a, int head_dim, int grid, hipStream_t stream);
int bwd_dkdv_tile();                       // keys per dK/dV item
int bwd_dkdv_rows(int head_dim);           // query rows per dK/dV step
int bwd_dkdv_slices(int head_dim);         // head-dim slices (dK/dV items) per key tile
int bwd_dq_rows(int head_dim, bool narrow);            // query rows per dQ item
int bwd_dq_tile(int head_dim);             // keys per dQ tile
int bwd_dq_blocks_per_cu(int head_dim, bool narrow);    // resident dQ workgroups per CU

struct DqConvertArgs {
  const float* dq_part;     // [chunks, n] fp32 partials
  __bf16* dq;
  int64_t n;                // elements of dQ
  int32_t chunks;
  float scale;
};
hipError_t launch_dq_convert(const DqConvertArgs& a, hipStream_t stream);
// bytes (a multiple of 16, 16-byte aligned) of zeros at p
hipError_t launch_zero_fill(void* p, int64_t bytes, hipStream_t stream);

// Decode.
struct DecodeArgs {
  const __bf16* q;
  const void* k_cache;      // bf16 or e4m3 bytes
  const void* v_cache;
  const int32_t* page_table;
  const int32_t* seqlens;
  __bf16* o;                // final output when splits == 1
  float* lse;
  float* o_part;            // [splits, B, Hq, d] when splits > 1
  float* lse_part;          // [splits, B, Hq]
  uint32_t* counters;       // per (b, column unit, KV head) arrival counters, zero at the
                            // start (then the last split merges), or null (decode_combine)
  int32_t batch, hq, hkv, group;
  int32_t page_size;
  int32_t max_pages;
  int32_t splits;
  int32_t q_len;            // query tokens per sequence (1 = single-token decode)
  int32_t causal;           // bottom-right mask over the q_len tokens
  int32_t kv_fp8;           // caches hold OCP e4m3 bytes
  int32_t q_fp8;            // q holds OCP e4m3 bytes (its scale is folded into scale_log2)
  float v_scale;            // fp8 V dequantisation scale (K's is folded into scale_log2)
  float scale_log2;
};
hipError_t launch_decode(const DecodeArgs& a, int head_dim, hipStream_t stream);
hipError_t launch_decode_combine(const DecodeArgs& a, int head_dim, hipStream_t stream);
constexpr int kMaxDecodeSplits = 128;   // largest num_splits the decode accepts
constexpr int64_t kDecodeCounterSlots = 65536;   // arrival counters at the workspace start
int decode_chunk_align();
hipError_t launch_check_offsets(const int32_t* cu, int32_t batch, int32_t total, int32_t* result, hipStream_t stream);
hipError_t launch_check_paged(const int32_t* page_table, const int32_t* seqlens, int32_t batch, int32_t max_pages,
                              int32_t page_size, int32_t num_pages, int32_t* result, hipStream_t stream);
int decode_col_groups(int columns, int head_dim);      // 16-column query groups per decode workgroup
int decode_blocks_per_cu(int columns, int head_dim);   // decode workgroups resident per CU

}  // namespace jfa
