/*
 * jfa.h -- C ABI of libjfa.so: exact jagged (packed variable-length) FlashAttention
 * forward and backward, and split-KV paged decode, for AMD MI355X (gfx950).
 *
 * Sources of the operations (page title, then section):
 *   - "Optimizing Jagged Flash Attention with TLX: The Road Toward SOTA FA4 on
 *     Blackwell": attention over jagged user sequences packed contiguously with
 *     their boundaries in an offsets tensor, no padded tokens materialised; the
 *     broadcast-Q production case in which one dense Q serves the whole batch and
 *     dQ is summed over the batch (third paragraph); persistent passes, load
 *     balancing of jagged tiles, bulk + masked-tail KV loop (fourth and fifth).
 *   - "Cutting edge isn't plug-and-play: customising FlashAttention-4 on B300":
 *     the tiled forward with saved LSE and the backward that rebuilds P from the
 *     saved LSE and uses delta, dP and dS (Flash Attention recap; Phase 2
 *     chunked-backward pseudocode and buffer list); unsupported head dims must not
 *     end in an assertion (the March 2026 head-dim support remark).
 *   - "Optimizing FlashAttention-4 for Efficient Inference": decode with
 *     parallelism over the KV dimension (PR 1940), arbitrary KV page sizes with a
 *     page table (PR 1999 / PR 2104), only real query rows in the tile (PR 1993)
 *     and GQA packing of the query heads that share a KV head (PR 2186).
 *
 * Conventions shared by every entry point
 *   - Every tensor pointer is a DEVICE pointer to contiguous row-major memory in
 *     the layout stated, aligned to 16 bytes.  bf16 tensors are passed as void*.
 *   - The workspace pointer must be aligned to 256 bytes (torch and hipMalloc
 *     allocations are); a misaligned one is rejected with
 *     JFA_ERR_INVALID_ARGUMENT.
 *   - The caller owns all memory (inputs, outputs, workspace) and the optional
 *     timing events.  The library allocates no device memory and keeps no state
 *     beyond a per-device cache of the compute-unit count; the one exception is
 *     jfa_decode_paged_noalloc, whose static device array (and its cached
 *     per-device address) is described with it.  Calls with distinct workspaces
 *     may run concurrently on different streams.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and
 *     runs asynchronously: no call synchronises with the host.
 *   - Outputs are fully overwritten, never accumulated into.
 *   - Host-checkable errors are returned before anything is launched.  The
 *     library never aborts, throws or prints.  A failed launch returns
 *     JFA_ERR_HIP.
 *   - Device contents are the caller's contract and are not checked by the
 *     compute entry points: offsets start at 0, do not decrease and end at the
 *     packed total; page ids are < num_pages; seqlens_k[b] <= max_pages_per_seq *
 *     page_size.  jfa_check_offsets and jfa_check_paged_cache check them on the
 *     device on request.
 *   - Sequences (or items) of length 0 are legal.  A query row that sees no key
 *     gets O = 0 and LSE = -inf, and contributes no gradient.
 */
#ifndef JFA_H
#define JFA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define JFA_ABI_VERSION 6

/* Same type as hipStream_t, declared without including the HIP headers. */
struct ihipStream_t;
typedef struct ihipStream_t* jfa_stream_t;

typedef enum {
  JFA_OK = 0,
  JFA_ERR_INVALID_ARGUMENT = 1,   /* null pointer, negative size, Hq % Hkv != 0, ... */
  JFA_ERR_UNSUPPORTED = 2,        /* head_dim outside {64, 96, 128, 192, 256}, causal broadcast-Q, ... */
  JFA_ERR_WORKSPACE_TOO_SMALL = 3,
  JFA_ERR_HIP = 4                 /* a HIP call or kernel launch failed */
} jfa_status_t;

/* Element types of the q/k/v (and KV-cache) tensors. */
enum { JFA_DTYPE_BF16 = 0, JFA_DTYPE_FP8_E4M3 = 1 };

/*
 * Optional kernel timing, owned by the caller.  Every member is a hipEvent_t that
 * the caller created (passed as void*), or NULL.  A call whose params point at
 * this struct records `*_start` on its stream right before it launches the named
 * kernel and `*_stop` right after, so hipEventElapsedTime(start, stop) is that
 * kernel's time; a call never launches the named kernel leaves its pair alone.
 * The library keeps no reference to the events.  A failed record returns
 * JFA_ERR_HIP.
 */
typedef struct {
  void* fwd_start;        /* jfa_fwd: the attention kernel */
  void* fwd_stop;
  void* bwd_dq_start;     /* jfa_bwd: the dQ kernel */
  void* bwd_dq_stop;
  void* bwd_dkdv_start;   /* jfa_bwd: the dK/dV kernel */
  void* bwd_dkdv_stop;
  void* decode_start;     /* jfa_decode_paged: the split-KV kernel */
  void* decode_stop;
} jfa_kernel_events_t;

/*
 * Problem description for jfa_fwd / jfa_bwd.
 *
 * Self-attention (broadcast_q = 0), B = batch sequences:
 *   q, o, dout, dq   [total_q, Hq, d]   bf16, sequence b owns rows cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1
 *   k, v, dk, dv     [total_k, Hkv, d]  bf16, rows cu_seqlens_k[b] .. cu_seqlens_k[b+1]-1
 *   lse              [Hq, total_q]      fp32, natural-log log-sum-exp of the scaled scores
 * Broadcast-Q (broadcast_q = 1), B = batch items sharing one dense Q of Nq = total_q rows:
 *   q, dq            [Nq, Hq, d]        dq = sum over all B items
 *   k, v, dk, dv     [total_k, Hkv, d]  jagged by cu_seqlens_k
 *   o, dout          [B, Nq, Hq, d]
 *   lse              [B, Hq, Nq]
 *   cu_seqlens_q is ignored (may be NULL); causal must be 0.
 * Query head h uses KV head h / (Hq / Hkv) (grouped-query attention).
 * Scores: S = Q K^T * scale with scale = softmax_scale, or 1/sqrt(d) when
 * softmax_scale <= 0.  Causal masking is aligned bottom-right: key j is visible
 * to query i of a sequence iff j <= i + (Lk - Lq).
 */
typedef struct {
  int32_t batch;          /* B >= 1 */
  int32_t num_heads_q;    /* Hq >= 1 */
  int32_t num_heads_kv;   /* Hkv >= 1, Hq % Hkv == 0 */
  int32_t head_dim;       /* d in {64, 96, 128, 192, 256}; anything else is JFA_ERR_UNSUPPORTED */
  int32_t total_q;        /* packed query rows (broadcast-Q: Nq) */
  int32_t total_k;        /* packed key rows */
  int32_t max_seqlen_q;   /* upper bound on any Lq (broadcast-Q: ignored, Nq is used) */
  int32_t max_seqlen_k;   /* upper bound on any Lk; sizes the scheduler's cost buckets */
  int32_t causal;         /* 0 or 1 */
  int32_t broadcast_q;    /* 0 or 1 */
  float softmax_scale;    /* <= 0 selects 1/sqrt(d) */
  int32_t qkv_dtype;      /* JFA_DTYPE_BF16 (0), or JFA_DTYPE_FP8_E4M3: q, k, v hold OCP e4m3
                             bytes in the same layouts (jfa_fwd only, d a multiple of 64;
                             jfa_bwd returns JFA_ERR_UNSUPPORTED) */
  float q_scale;          /* e4m3 only: per-tensor scales, each tensor's value = scale x its */
  float k_scale;          /* e4m3 value; finite and > 0.  Ignored for bf16 */
  float v_scale;
  int32_t query_tile;     /* query rows per forward / dQ work item.  0: chosen from the
                             lengths (128 when the mean query rows per sequence -- or
                             broadcast-Q's Nq -- is at most 160, else 256).  128 or 256:
                             that size wherever the kernel has both (bf16 forward at
                             d = 64 / 128, dQ at d = 128), ignored elsewhere.  Any other
                             value is JFA_ERR_INVALID_ARGUMENT.  The result does not
                             depend on it; the workspace size does, so pass the same
                             value to the size query and the call. */
  const jfa_kernel_events_t* events;   /* optional kernel timing (NULL: none) */
} jfa_attn_params_t;

/* Bytes of workspace jfa_fwd needs for this problem (0 if the params are invalid). */
size_t jfa_fwd_workspace_size(const jfa_attn_params_t* p);

/*
 * Forward: O = softmax(S) V per sequence and head, plus LSE, with no score
 * matrix or padding ever written to memory.  With e4m3 inputs ("Optimizing
 * FlashAttention-4 for Efficient Inference", PR 2109: FP8 inputs) the result is
 * that of attention on the scaled e4m3 values: Q K^T runs on the e4m3 matrix
 * cores with fp32 accumulation, V is widened exactly to bf16 for P V; o stays
 * bf16 and lse fp32.  Work items (sequence, query tile,
 * head) are listed on the device from the offsets.  The tiles of one (sequence,
 * KV head) form a group that shares its K/V; groups are sorted by cost (longest
 * first) and dealt to one queue per XCD, and persistent workgroups pull from
 * their XCD's queue, then from the others.
 * workspace: device memory of at least jfa_fwd_workspace_size(p) bytes, used
 * only during this call (stream-ordered).
 */
jfa_status_t jfa_fwd(const jfa_attn_params_t* p,
                     const void* q, const void* k, const void* v,
                     const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                     void* o, float* lse,
                     void* workspace, size_t workspace_bytes, jfa_stream_t stream);

/* Bytes of workspace jfa_bwd needs (delta, the two work lists, and for broadcast-Q
 * one fp32 partial of dQ per chunk of items). */
size_t jfa_bwd_workspace_size(const jfa_attn_params_t* p);

/*
 * Backward: given q, k, v, the forward's o and lse, and dout, writes dq, dk, dv.
 * P is rebuilt from lse; delta = rowsum(dout * o); dP = dout V^T;
 * dS = P * (dP - delta); dV = P^T dout; dK = scale dS^T Q; dQ = scale dS K.
 * dK/dV of a KV head sum over the Hq/Hkv query heads of its group.  Results
 * are deterministic (no atomics): in broadcast-Q mode dQ, the sum over all
 * items, is accumulated per chunk of items in fp32 and the chunk partials are
 * added in a fixed order.  Keys that no query sees get dK = dV = 0; queries
 * that see no key get dQ = 0.  A broadcast-Q problem with Nq = total_q = 0
 * writes dK = dV = 0 (q, o, lse, dout, dq and cu_seqlens_q are not read and may
 * be NULL); a self-attention problem with total_q = 0 likewise writes dK = dV =
 * 0 through the regular kernels.  For d = 256 the dK/dV work is split along the
 * head dimension ("Cutting edge isn't plug-and-play", Phase 2 chunked
 * backward): each slice of 128 columns is a work item of its own that rebuilds
 * S and dP from the whole head; the results are the same.
 */
jfa_status_t jfa_bwd(const jfa_attn_params_t* p,
                     const void* q, const void* k, const void* v,
                     const void* o, const float* lse, const void* dout,
                     const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                     void* dq, void* dk, void* dv,
                     void* workspace, size_t workspace_bytes, jfa_stream_t stream);

/* KV-cache element types of jfa_decode_paged (the JFA_DTYPE_* values). */
enum { JFA_KV_BF16 = JFA_DTYPE_BF16, JFA_KV_FP8_E4M3 = JFA_DTYPE_FP8_E4M3 };

/*
 * Split-KV paged decode of q_len (1..16) new tokens per sequence: single-token
 * decode, and the few-token shapes of speculative decoding or chunked prefill
 * ("Optimizing FlashAttention-4 for Efficient Inference": one or a few tokens
 * at a time against cached KV, PR 1940 and PR 1993).
 *   q           [B, q_len, Hq, d]                     bf16 (q_len = 1: [B, Hq, d])
 *   k_cache,
 *   v_cache     [num_pages, page_size, Hkv, d]        bf16
 *   page_table  [B, max_pages_per_seq]                int32, physical page of each logical page
 *   seqlens_k   [B]                                   int32, KV length of each sequence
 *                                                      (the new tokens included)
 *   o           [B, q_len, Hq, d]                     bf16
 *   lse         [B, q_len, Hq]                        fp32, natural log
 * Token t of sequence b lives in slot t % page_size of page
 * page_table[b][t / page_size].  With causal = 1 the q_len tokens are the last
 * ones of the sequence: token i (0-based) sees keys j <= i + seqlens_k[b] - q_len
 * (bottom-right alignment); a token that sees no key gets O = 0, LSE = -inf.
 * The Hq/Hkv query heads that share a KV head, for all q_len tokens, form the
 * columns of one query tile (only real rows: no padding to a fixed tile height),
 * so every KV byte is read once per 64 such columns.  Each sequence's tokens are
 * cut into num_splits contiguous chunks processed in parallel; every chunk
 * leaves a normalised partial output and its LSE in the workspace, and they are
 * merged with weights exp(LSE_s - LSE): by a second kernel launch (default), or
 * with single_launch = 1 by the last chunk of each (sequence, KV head) to
 * finish, inside the decode launch.  num_splits = 0 picks a count from the
 * problem size; 1 writes o/lse directly and needs no workspace.
 * Workspace (num_splits > 1): JFA_DECODE_COUNTER_BYTES of per-unit arrival
 * counters, then the fp32 partials.  Only single_launch = 1 uses the counters,
 * which must then be zero when the call starts; a call that runs to completion
 * leaves them zero, so zero-filling a workspace once when it is allocated
 * (hipMemset, torch.zeros) suffices for every later decode call on it, of any
 * shape and either mode; anything else written into that region (another entry
 * point's use of the same buffer) must be cleared again before the next
 * single-launch call.  The rest of the workspace needs no initialisation.
 * Problems with more than JFA_DECODE_COUNTER_BYTES / 4 units
 * (B * Hkv * ceil(ceil(Hq / Hkv * q_len / 16) / 2) at d <= 128) merge in a
 * second launch in either mode and do not touch the counters.
 * FP8 caches ("Optimizing FlashAttention-4 for Efficient Inference", PR 2109:
 * FP8 inputs): k_cache / v_cache hold OCP e4m3 bytes (same shapes, one byte per
 * element) with per-tensor scales; the result is that of bf16 attention on the
 * dequantised values (every e4m3 value is exact in bf16), for half the KV bytes.
 */
typedef struct {
  int32_t batch;              /* B >= 1 */
  int32_t num_heads_q;        /* Hq >= 1 */
  int32_t num_heads_kv;       /* Hkv >= 1, Hq % Hkv == 0, (Hq / Hkv) * q_len <= 256 */
  int32_t head_dim;           /* d in {64, 96, 128, 192, 256} */
  int32_t page_size;          /* >= 1, any value */
  int32_t num_pages;          /* pages in the cache, >= 1 */
  int32_t max_pages_per_seq;  /* columns of page_table, >= 1 */
  int32_t num_splits;         /* 0 = automatic, else 1 .. 128 */
  float softmax_scale;        /* <= 0 selects 1/sqrt(d) */
  int32_t q_len;              /* new tokens per sequence, 1 .. 16 */
  int32_t causal;             /* 0 or 1: bottom-right mask over the q_len tokens */
  int32_t kv_dtype;           /* JFA_KV_BF16 or JFA_KV_FP8_E4M3 (k_cache / v_cache element type) */
  float k_scale;              /* fp8 caches: K = k_scale * e4m3 value (<= 0 means 1) */
  float v_scale;              /* fp8 caches: V = v_scale * e4m3 value (<= 0 means 1) */
  int32_t q_dtype;            /* JFA_DTYPE_BF16 or JFA_DTYPE_FP8_E4M3 (q element type) */
  float q_scale;              /* e4m3 q: Q = q_scale * e4m3 value (<= 0 means 1) */
  int32_t single_launch;      /* 0: split partials merged by a second launch; 1: by the
                                 last split of each unit inside the decode launch (needs
                                 the workspace's counters zero, see above) */
  const jfa_kernel_events_t* events;   /* optional kernel timing (NULL: none) */
} jfa_decode_params_t;

/* Bytes at the start of a decode workspace that hold arrival counters. */
#define JFA_DECODE_COUNTER_BYTES ((size_t)256 << 10)

/* Bytes of workspace jfa_decode_paged needs: 0 without splits, else
 * JFA_DECODE_COUNTER_BYTES + the fp32 partials (0 if the params are invalid). */
size_t jfa_decode_workspace_size(const jfa_decode_params_t* p);

jfa_status_t jfa_decode_paged(const jfa_decode_params_t* p,
                              const void* q, const void* k_cache, const void* v_cache,
                              const int32_t* page_table, const int32_t* seqlens_k,
                              void* o, float* lse,
                              void* workspace, size_t workspace_bytes, jfa_stream_t stream);

/*
 * jfa_decode_paged without a workspace, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).  The same computation and arguments as jfa_decode_paged;
 * the split partials live in a static device array of
 * JFA_DECODE_SCRATCH_BYTES that the library holds on every GPU it runs on (on
 * the current device; `stream` must belong to it) until the process ends.  The
 * call allocates nothing.  A problem whose partials (jfa_decode_workspace_size)
 * exceed JFA_DECODE_SCRATCH_BYTES returns JFA_ERR_WORKSPACE_TOO_SMALL before
 * any launch; failing to look up the array's address returns JFA_ERR_HIP.
 * Every call on one GPU uses the same array: calls that overlap in time on one
 * GPU (concurrent streams, or host threads) race and must be serialised by the
 * caller.  The array's counter region (its first JFA_DECODE_COUNTER_BYTES) is
 * zero when the library is loaded and every completed call leaves it zero.
 */
#define JFA_DECODE_SCRATCH_BYTES ((size_t)8 << 20)
jfa_status_t jfa_decode_paged_noalloc(const jfa_decode_params_t* p,
                                      const void* q, const void* k_cache, const void* v_cache,
                                      const int32_t* page_table, const int32_t* seqlens_k,
                                      void* o, float* lse, jfa_stream_t stream);

/*
 * Device-side checks of the input contents the entry points take on trust (the
 * "device contents" convention above), for debugging a caller: each enqueues one
 * small kernel on `stream` that reads only the array it checks, within the sizes
 * passed, and writes to *result (a device int32) the OR of the JFA_CHECK_* bits
 * of every violation found, 0 if there is none.  Nothing else is written, and
 * bad contents are reported, never dereferenced.  Host-checkable errors (null
 * pointers, negative sizes) return JFA_ERR_INVALID_ARGUMENT before any launch.
 *
 * jfa_check_offsets: offsets [batch + 1] of a packed layout (cu_seqlens_q or
 *   cu_seqlens_k of jfa_fwd / jfa_bwd) must start at 0, not decrease and end at
 *   total (T_q or T_k).
 * jfa_check_paged_cache: with p's batch, page_size, num_pages and
 *   max_pages_per_seq, every seqlens_k[b] must lie in
 *   [0, max_pages_per_seq * page_size] and every page id a sequence uses
 *   (page_table[b][0 .. ceil(seqlens_k[b] / page_size) - 1]) in [0, num_pages).
 */
#define JFA_CHECK_OFFSETS_START 1    /* offsets[0] != 0 */
#define JFA_CHECK_OFFSETS_ORDER 2    /* some offsets[b + 1] < offsets[b] */
#define JFA_CHECK_OFFSETS_END 4      /* offsets[batch] != total */
#define JFA_CHECK_SEQLEN_RANGE 8     /* some seqlens_k[b] < 0 or > max_pages_per_seq * page_size */
#define JFA_CHECK_PAGE_RANGE 16      /* some used page id < 0 or >= num_pages */
jfa_status_t jfa_check_offsets(const int32_t* offsets, int32_t batch, int32_t total, int32_t* result,
                               jfa_stream_t stream);
jfa_status_t jfa_check_paged_cache(const jfa_decode_params_t* p, const int32_t* page_table,
                                   const int32_t* seqlens_k, int32_t* result, jfa_stream_t stream);

/* The split count jfa_decode_paged uses for p (resolves num_splits = 0). */
int32_t jfa_decode_num_splits(const jfa_decode_params_t* p);

/* Static string naming a status code. */
const char* jfa_status_string(jfa_status_t s);

/* JFA_ABI_VERSION of the built library. */
int jfa_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* JFA_H */
