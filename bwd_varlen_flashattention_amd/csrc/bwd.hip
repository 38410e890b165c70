// Jagged FlashAttention backward for gfx950.
//
// What is computed ("Cutting edge isn't plug-and-play: customising
// FlashAttention-4 on B300", Phase 2 chunked-backward pseudocode and its buffer
// list; the head-dim slicing is used for dK/dV at d = 256, see DkvTile):
//   P = exp(S - LSE) rebuilt from the forward's saved LSE, S = Q K^T * scale,
//   delta = rowsum(dO * O), dP = dO V^T, dS = P * (dP - delta),
//   dV = P^T dO, dK = scale dS^T Q, dQ = scale dS K.
// Broadcast-Q ("Optimizing Jagged Flash Attention with TLX", third paragraph):
// every item adds its dQ into the one shared dQ.
//
// Kernels:
//   bwd_pre_kernel   broadcast-Q only: delta (fp32, laid out like LSE) for
//                    every item; self-attention computes delta in the dQ kernel
//   bwd_dkdv_kernel  persistent, key-stationary: a workgroup owns 128 keys of one
//                    KV head; K/V fragments stay in VGPRs and the dK^T/dV^T
//                    accumulators in registers across all query tiles and all
//                    query heads of the GQA group.  64-row Q/dO tiles (32 above
//                    d = 128) are staged
//                    into double-buffered LDS both row-major (A operands of
//                    S = Q K^T and dP = dO V^T) and transposed (A operands of
//                    dV^T += dO^T P and dK^T += Q^T dS, with P and dS taken
//                    straight from the S/dP accumulators), so every MFMA operand
//                    is a single ds_read_b128.
//   bwd_dq_kernel    persistent, query-stationary (the forward's structure):
//                    recomputes S^T = K Q^T and dP^T = V dO^T per 32-key tile
//                    and accumulates dQ^T += K^T dS^T in registers, with dS^T
//                    straight from the accumulators and K^T staged transposed.
//                    dQ is written once per query tile: no atomics, so dQ is
//                    deterministic.  Broadcast-Q splits the items into chunks;
//                    each chunk writes its fp32 partial dQ to a slice of its
//                    own and dq_convert adds the slices in chunk order, so
//                    broadcast-Q dQ is deterministic as well.
//
// The dQ kernel repeats S and dP (4d of the 14d flops per query-key pair); the
// alternative -- dS K accumulated with fp32 atomics from the key-stationary
// kernel -- measured ~1.2 ms of atomic traffic on the GEM s=0.5 workload,
// more than the repeated MFMA work.  Neither kernel refills an LDS stage while
// any reader of it is unfinished (one barrier per stage), the single-buffer
// K hazard described in the bug-hunting section of the B300 page.
//
// Two compilation units.  bwd_wide.hip includes this file with
// JFA_BWD_WIDE_UNIT defined and emits only the d >= 192 dK/dV kernels and the
// d = 192 dQ kernels, built with the MFMA builtins in their VGPR form: there the
// dK/dV accumulators live in AGPRs through hand-written MFMAs
// (DkvTile::ACC_AGPR).  This unit emits the rest.
#include <algorithm>
#include <type_traits>

#include "jfa_internal.h"
#include "device_common.h"

namespace jfa {

#ifndef JFA_BWD_WIDE_UNIT
// ----------------------------------------------------------------------------- preprocess
constexpr int kPreThreads = 256;

__global__ __launch_bounds__(kPreThreads) void bwd_pre_kernel(BwdPreArgs a) {
  // 16 lanes per (row, head) pair; lane l reads the 8-column chunks l, l + 16, ...
  // of O and dO (one chunk up to d = 128, two for d = 256).
  const int64_t gtid = (int64_t)blockIdx.x * kPreThreads + threadIdx.x;
  const int lane16 = threadIdx.x & 15;
  const int64_t pair = gtid >> 4;
  const int64_t n_pairs = a.rows * a.hq;
  const int chunks = a.head_dim / 8;
  float acc = 0.f;
  if (pair < n_pairs) {
    for (int c = lane16; c < chunks; c += 16) {
      const int64_t base = pair * a.head_dim + c * 8;
      const bf16x8 o = *(const bf16x8*)(a.o + base);
      const bf16x8 d = *(const bf16x8*)(a.dout + base);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc = fmaf((float)o[i], (float)d[i], acc);
    }
  }
#pragma unroll
  for (int m = 8; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, 16);
  if (pair < n_pairs && lane16 == 0) {
    const int64_t row = pair / a.hq;
    const int h = (int)(pair % a.hq);
    int64_t di;
    if (a.bcast) {
      const int64_t b = row / a.lse_cols, qi = row % a.lse_cols;
      di = (b * a.hq + h) * a.lse_cols + qi;
    } else {
      di = (int64_t)h * a.lse_cols + row;
    }
    a.delta[di] = acc;
  }
}

hipError_t launch_bwd_pre(const BwdPreArgs& a, hipStream_t stream) {
  const int64_t threads = a.rows * a.hq * 16;
  int64_t blocks = (threads + kPreThreads - 1) / kPreThreads;
  if (blocks < 1) blocks = 1;
  if (blocks > (1 << 30)) return hipErrorInvalidValue;
  hipLaunchKernelGGL(bwd_pre_kernel, dim3((unsigned)blocks), dim3(kPreThreads), 0, stream, a);
  return hipGetLastError();
}

// ----------------------------------------------------------------------------- zero fill
// dK = dV = 0 for a broadcast-Q backward without query rows (no key sees a query).
// n16 16-byte chunks; a fill kernel rather than a memset, so that a caller may
// capture the call in a graph.
__global__ __launch_bounds__(256) void zero_fill_kernel(u32x4* p, int64_t n16) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += (int64_t)gridDim.x * 256)
    p[i] = u32x4{0u, 0u, 0u, 0u};
}

hipError_t launch_zero_fill(void* p, int64_t bytes, hipStream_t stream) {
  if (bytes <= 0) return hipSuccess;
  if (bytes % 16 != 0 || ((uintptr_t)p % 16) != 0) return hipErrorInvalidValue;
  const int64_t n16 = bytes / 16;
  const int64_t blocks = std::min<int64_t>((n16 + 255) / 256, 4096);
  hipLaunchKernelGGL(zero_fill_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, (u32x4*)p, n16);
  return hipGetLastError();
}

// ----------------------------------------------------------------------------- dQ convert (broadcast-Q)
// dQ = scale * sum of the chunk partials, added in chunk order: the result does
// not depend on which workgroup finished first.
__global__ __launch_bounds__(256) void dq_convert_kernel(DqConvertArgs a) {
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i + 3 < a.n) {
    f32x4 x = *(const f32x4*)(a.dq_part + i);
    for (int c = 1; c < a.chunks; ++c) x += *(const f32x4*)(a.dq_part + (int64_t)c * a.n + i);
    bf16x4 y;
#pragma unroll
    for (int e = 0; e < 4; ++e) y[e] = (__bf16)(x[e] * a.scale);
    *(bf16x4*)(a.dq + i) = y;
  } else {
    for (int64_t j = i; j < a.n; ++j) {
      float x = a.dq_part[j];
      for (int c = 1; c < a.chunks; ++c) x += a.dq_part[(int64_t)c * a.n + j];
      a.dq[j] = (__bf16)(x * a.scale);
    }
  }
}

hipError_t launch_dq_convert(const DqConvertArgs& a, hipStream_t stream) {
  if (a.n <= 0) return hipSuccess;
  const int64_t blocks = (a.n + 1023) / 1024;
  hipLaunchKernelGGL(dq_convert_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, a);
  return hipGetLastError();
}
#endif  // JFA_BWD_WIDE_UNIT

// Stored order of the four 4-row quarters of a 16-row group in a transposed
// tile: an S/dP accumulator hands lane half h the rows {4h..4h+3, 8+4h..8+4h+3}
// of each group as one 8-slot MFMA operand, so quarters go in the order 0, 2, 1, 3.
__device__ __forceinline__ int quarter_pos(int q) { return ((q & 1) << 1) | (q >> 1); }

// Transpose a 4-row x 8-column bf16 block held as four 16-byte rows and write it
// as 8 rows of 4 values (8 bytes each) at dst, dst + pitch, ... (pitch in elements).
__device__ __forceinline__ void store_transposed_4x8(__bf16* dst, int pitch, const u32x4 (&r)[4]) {
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const uint32_t lo01 = __builtin_amdgcn_perm(r[1][c], r[0][c], 0x05040100u);
    const uint32_t lo23 = __builtin_amdgcn_perm(r[3][c], r[2][c], 0x05040100u);
    const uint32_t hi01 = __builtin_amdgcn_perm(r[1][c], r[0][c], 0x07060302u);
    const uint32_t hi23 = __builtin_amdgcn_perm(r[3][c], r[2][c], 0x07060302u);
    *(uint2*)(dst + (2 * c) * pitch) = make_uint2(lo01, lo23);
    *(uint2*)(dst + (2 * c + 1) * pitch) = make_uint2(hi01, hi23);
  }
}

// Staging block of a thread: (row block, 8-column block) of a tile staged as
// 4-row x 8-column blocks, each written row-major (16-byte stores) and
// transposed (8-byte stores).  gfx950's LDS serves 16-byte accesses 8 lanes and
// 8-byte accesses 16 lanes per cycle over 32 banks (measured with in-bounds store
// probes).  With 16 row blocks: the transposed stores' bank depends only on the
// row block, so the 16 lanes of a group take 16 row blocks (thread bits 0-3);
// the row-major stores need (4 * row block + column block) mod 8 distinct in
// each 8-lane group, which the column block gets from bits 1-2 xor bits 4-5
// (bits 6-7 give its high half).  Both stores are then free of bank conflicts;
// stepping the lanes down rows alone made the row-major stores 4-way.  With 8
// row blocks (head dims above 128) the same construction (row block = bits 0-2,
// column block from bits 1-2 xor 3-4) frees the row-major stores; the transposed
// stores stay 2-way, as 16 lanes cannot hold 16 distinct row blocks.
__device__ __forceinline__ void staging_block(int tid, int row_blocks, int& rb, int& cb) {
  if (row_blocks == 16) {
    rb = tid & 15;
    cb = (((tid >> 1) ^ (tid >> 4)) & 3) | ((tid >> 6) << 2);
  } else {   // 8 row blocks
    rb = tid & 7;
    cb = (((tid >> 1) ^ (tid >> 3)) & 3) | ((tid >> 5) << 2);
  }
}

// ============================================================================= dK / dV
// Head-dim chunking ("Cutting edge isn't plug-and-play: customising
// FlashAttention-4 on B300", Phase 2): for d = 256 one work item owns the dK/dV
// columns of one DC-wide slice of the head dimension.  S = Q K^T and dP = dO V^T
// are still summed over the whole head dimension (every item reads all of Q, K,
// V and dO), and P, dS are rebuilt from them and the saved LSE; only the dK/dV
// accumulators and the transposed Q/dO tiles are per slice.  d <= 192 keeps the
// whole head in one item.  Above d = 128 a step takes 32 query rows, so that the
// double-buffered full-width Q/dO tiles fit in LDS.
template <int D>
struct DkvTile {
  static constexpr int NT = 256;             // 4 waves, 32 keys each
  static constexpr int BN = 128;             // keys per item
  static constexpr int BM = D <= 128 ? 64 : 32;   // query rows per step
  static constexpr int DC = D <= 192 ? D : 128;   // head-dim slice owned by one item
  static constexpr int NC = D / DC;               // slices per key tile
  static constexpr int QP = D + 8;           // row pitch of Q / dO tiles (elements)
  static constexpr int QTP = BM + 8;         // row pitch of Q^T / dO^T tiles
  static constexpr int QBLOCKS = (BM / 4) * (D / 8);   // 4-row x 8-column staging blocks
  static constexpr int KS = D / 16;
  static constexpr int DB = DC / 32;         // 32-wide blocks of the owned slice
  // d >= 192: the dV^T/dK^T MFMAs are hand-written with their accumulators in
  // AGPRs, while the S/dP products stay compiler-generated in VGPRs (the MFMA
  // form bwd_wide.hip, which builds these kernels, asks for).  With every MFMA in AGPR form each S/dP entry needed its own
  // v_accvgpr_read before the softmax; here those copies go and fewer registers
  // are needed (no spills at d = 192): dK/dV 6-7.5 % faster at d = 192 and 256.
  // At d <= 128 the fixed MFMA order of the hand-written statements cost more
  // than that (5-7 % slower), so those kernels keep the compiler's MFMAs.
  static constexpr bool ACC_AGPR = D >= 192;
  static_assert(QBLOCKS <= NT, "one Q block per thread");
  static_assert(D % DC == 0 && DC % 32 == 0, "slice width");
  static_assert(2 * (2 * BM * QP + 2 * DC * QTP) * 2 + 4 * BM * 4 <= 160 * 1024, "LDS budget");
};

template <int D, bool CAUSAL, bool BCAST>
__global__ __launch_bounds__(256) void bwd_dkdv_kernel(BwdArgs a) {
  using T = DkvTile<D>;
  constexpr int BN = T::BN, BM = T::BM, QP = T::QP, QTP = T::QTP, KS = T::KS, DB = T::DB, DC = T::DC;
  __shared__ __attribute__((aligned(16))) __bf16 q_lds[2][BM * QP];
  __shared__ __attribute__((aligned(16))) __bf16 do_lds[2][BM * QP];
  __shared__ __attribute__((aligned(16))) __bf16 qt_lds[2][DC * QTP];
  __shared__ __attribute__((aligned(16))) __bf16 dot_lds[2][DC * QTP];
  __shared__ __attribute__((aligned(16))) float lse_lds[2][BM];
  __shared__ __attribute__((aligned(16))) float dlt_lds[2][BM];
  __shared__ int s_item[2];   // claims alternate between the entries: a wave still
  // reading claim k's entry has not passed the barrier that follows claim k + 1, so
  // claim k + 2, the next write to that entry, cannot overtake the read even when
  // item k + 1 has no tiles (and so no barrier of its own)
  __shared__ int s_queue[2 * kQueues];

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, hh = lane >> 5;
  const float INF = __builtin_inff();

  // Staging.  Up to d = 128 (64-row steps) a thread owns 8 rows x 8 columns of
  // one tile (threads 0-127 Q, 128-255 dO): rows 16*(sq/2) + 4*(sq%2) + {0-3,
  // 8-11}, the two quarters an S/dP accumulator hands one lane half, so each
  // transposed column is 16 contiguous bytes and every LDS store is b128 (16 per
  // thread instead of 8 b128 + 16 b64).  Bank map: transposed stores need sq
  // distinct in each 8-lane group (sq = thread bits 0-2); row-major stores need
  // 4*(sq%2) + sd distinct mod 8, which sd gets from bits 0-2 xor 3-5 plus
  // 4*(sq%2) (bit 6 gives its high half).  Above d = 128 (32-row steps) a thread
  // owns rows 4*sq..4*sq+3 of both tiles.
  constexpr bool ST8 = D <= 128;
  int sq, sd;
  const int ts = ST8 ? __builtin_amdgcn_readfirstlane(tid >> 7) : 0;   // staged tile (8-row map)
  if constexpr (ST8) {
    static_assert(BM == 64, "8-row staging map covers 64 rows");
    const int lt = tid & 127;
    sq = lt & 7;
    sd = ((((sq ^ (lt >> 3)) & 7) + 4 * (sq & 1)) & 7) | ((lt >> 6) << 3);
  } else {
    staging_block(tid, BM / 4, sq, sd);
  }
  const bool stager = sd < D / 8;
  const int qrs = a.hq * D;                           // elements between query rows
  const int srow0 = ST8 ? 16 * (sq >> 1) + 4 * (sq & 1) : 4 * sq;   // first staged row
  const uint32_t qoff = (uint32_t)((srow0 * qrs + 8 * sd) * 2);   // byte offsets stay in the
  // vector offset: the buffer range check that zeroes rows past Lq covers only that
  auto srow = [&](int i) { return ST8 ? (i & 3) + 8 * (i >> 2) : i; };   // row of register i - srow0

  int home_q = blockIdx.x % kQueues, drained = 0;   // work-queue state (thread 0)
  load_queues(a.queues, s_queue);
  __syncthreads();
  if (tid == 0) s_item[0] = next_work_item(a.queues, s_queue, home_q, drained);
  __syncthreads();
  int slot = 0;   // s_item entry of the current claim (uniform)
  int item = __builtin_amdgcn_readfirstlane(s_item[0]);   // uniform: the item loads are scalar
  while (item >= 0) {
    const WorkItem e = a.items[item];
    const int g = e.h / T::NC;
    const int c0 = (e.h % T::NC) * DC;         // first head-dim column of the owned slice
    const int b = e.b;
    const int lq = e.lq, q_base = e.q_base;
    const int k_base = e.k_base, lk = e.lk;
    const int off = lk - lq;
    const int kt0 = e.t * BN;
    const int my_key = kt0 + 32 * w + l32;
    const bool key_ok = my_key < lk;

    int i_first = 0;
    if (CAUSAL) i_first = max(0, kt0 - off) / BM;
    const int ntq = cdiv(lq, BM);
    const int n_qt = (CAUSAL && max(0, kt0 - off) >= lq) ? 0 : ntq - i_first;
    const int n_steps = n_qt * a.group;

    // K/V fragments for this wave's 32 keys: B operands of S = Q K^T and dP = dO V^T.
    // Up to d = 128 the rows are loaded whole (D / 8 lanes per row, rows past Lk
    // read as zero through the buffer range) and moved into the fragment layout
    // through LDS stage 1, which the item's first tile leaves alone; a fragment
    // load would touch 32 rows per instruction.
    bf16x8 kf[KS], vf[KS];
    constexpr bool KV_VIA_LDS = D <= 128;
    constexpr int KV_CPR = D / 8, KV_PER = 32 * KV_CPR / 64;   // 16-byte chunks per row / per lane
    u32x4 kraw[KV_VIA_LDS ? KV_PER : 1], vraw[KV_VIA_LDS ? KV_PER : 1];
    if constexpr (KV_VIA_LDS) {
      const int key0 = kt0 + 32 * w;
      const uint32_t nbytes = (uint32_t)(max(0, min(32, lk - key0)) * a.hkv * D * 2);
      const int64_t off0 = ((int64_t)(k_base + key0) * a.hkv + g) * D;
      const auto krs = uniform_rsrc(a.k + off0, nbytes);
      const auto vrs = uniform_rsrc(a.v + off0, nbytes);
#pragma unroll
      for (int i = 0; i < KV_PER; ++i) {
        const int id = lane + 64 * i, row = id / KV_CPR, col = id % KV_CPR;
        const uint32_t voff = (uint32_t)((row * a.hkv * D + 8 * col) * 2);
        kraw[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(krs, voff, 0, 0));
        vraw[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(vrs, voff, 0, 0));
      }
    } else {
      const int64_t base = ((int64_t)(k_base + min(my_key, lk - 1)) * a.hkv + g) * D + 8 * hh;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        kf[ks] = key_ok ? *(const bf16x8*)(a.k + base + 16 * ks) : zero_bf16x8();
        vf[ks] = key_ok ? *(const bf16x8*)(a.v + base + 16 * ks) : zero_bf16x8();
      }
    }
    f32x16 dkt[DB], dvt[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) { dkt[db] = f32x16{}; dvt[db] = f32x16{}; }

    // step s -> unit s -> (query head, query tile); rows past Lq read as zero
    // (buffer range).  All key tiles of a (sequence, KV head) walk the query
    // tiles in the same order, so the ones running together on an XCD find the
    // same Q/dO tiles in its L2.
    // Causal: only the first n_diag query tiles of each head reach past this key
    // tile's diagonal and need the mask.  Those steps run first, for every head,
    // then the unmasked ones (one head at a time, tiles in increasing order).
    // (d = 192 keeps one masked step body: the second one makes it spill.)
    constexpr bool SPLIT_MASK = CAUSAL && D != 192;
    int n_diag = 0;
    if constexpr (SPLIT_MASK) {
      const int last_key = kt0 + BN - 1 - off;   // the tile's last key, in query-row units
      n_diag = last_key < 0 ? 0 : max(0, min(n_qt, last_key / BM - i_first + 1));
    }
    const int n_mask = n_diag * a.group;
    const int n_rest = n_qt - n_diag;
    auto unit_of = [&](int s) {
      if (!SPLIT_MASK) return s;
      if (s < n_mask) return (s / n_diag) * n_qt + s % n_diag;
      const int r = s - n_mask;
      return (r / n_rest) * n_qt + n_diag + r % n_rest;
    };
    u32x4 sr[8];   // staged rows: 8 rows of one tile, or 4 rows of Q then 4 of dO
    // LSE and delta travel raw (range-checked buffer loads) and are only looked
    // at when they are written to LDS: consuming them right after the load would
    // make the in-order vmcnt wait cover this step's Q/dO prefetch as well.
    // Rows past Lq read LSE = delta = 0 with zero Q and dO rows, so they add
    // nothing to dK or dV.
    float lse_raw = 0.f, dlt_raw = 0.f;
    auto load_regs = [&](int s) {
      const int u = unit_of(s);
      const int h = g * a.group + u / n_qt;
      const int qt = i_first + u % n_qt;
      const int row0 = qt * BM;
      const int rows = min(lq - row0, BM);
      if (tid < BM) {
        const int64_t li0 = BCAST ? ((int64_t)b * a.hq + h) * lq + row0 : (int64_t)h * a.total_q + q_base + row0;
        const auto lrsrc = uniform_rsrc(a.lse + li0, (uint32_t)(rows * 4));
        const auto drsrc = uniform_rsrc(a.delta + li0, (uint32_t)(rows * 4));
        lse_raw = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(lrsrc, tid * 4, 0, 0));
        dlt_raw = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(drsrc, tid * 4, 0, 0));
      }
      const uint32_t nbytes = (uint32_t)(rows * qrs * 2);
      const __bf16* qb = a.q + ((int64_t)(q_base + row0) * a.hq + h) * D;
      const int64_t orow0 = BCAST ? (int64_t)b * lq + row0 : (int64_t)(q_base + row0);
      const __bf16* ob = a.dout + (orow0 * a.hq + h) * D;
      const auto qrsrc = uniform_rsrc(qb, nbytes);
      const auto orsrc = uniform_rsrc(ob, nbytes);
      if (stager) {
        if constexpr (ST8) {
          const auto rs = ts == 0 ? qrsrc : orsrc;
#pragma unroll
          for (int i = 0; i < 8; ++i)
            sr[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, qoff + (uint32_t)(srow(i) * qrs * 2), 0, 0));
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            sr[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(qrsrc, qoff + (uint32_t)(i * qrs * 2), 0, 0));
            sr[4 + i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(orsrc, qoff + (uint32_t)(i * qrs * 2), 0, 0));
          }
        }
      }
    };
    auto store_lds = [&](int buf) {
      if (stager) {
        if constexpr (ST8) {
          __bf16* rm = ts == 0 ? &q_lds[buf][0] : &do_lds[buf][0];
          __bf16* tr = ts == 0 ? &qt_lds[buf][0] : &dot_lds[buf][0];
#pragma unroll
          for (int i = 0; i < 8; ++i) *(u32x4*)&rm[(srow0 + srow(i)) * QP + 8 * sd] = sr[i];
          // column c of the block: its 8 values in register order, at transposed
          // row 8*sd + c, columns 16*(sq/2) + 8*(sq%2) + 0..7
          __bf16* tp = &tr[(8 * sd) * QTP + 8 * sq];
#pragma unroll
          for (int c = 0; c < 8; ++c) {
            const uint32_t sel = (c & 1) ? 0x07060302u : 0x05040100u;
            u32x4 col;
#pragma unroll
            for (int j = 0; j < 4; ++j) col[j] = __builtin_amdgcn_perm(sr[2 * j + 1][c >> 1], sr[2 * j][c >> 1], sel);
            *(u32x4*)(tp + c * QTP) = col;
          }
        } else {
          const u32x4 qr[4] = {sr[0], sr[1], sr[2], sr[3]};
          const u32x4 dr[4] = {sr[4], sr[5], sr[6], sr[7]};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            *(u32x4*)&q_lds[buf][(4 * sq + i) * QP + 8 * sd] = qr[i];
            *(u32x4*)&do_lds[buf][(4 * sq + i) * QP + 8 * sd] = dr[i];
          }
          // the transposed tiles hold the owned slice only (whole 8-column blocks)
          const int col = 16 * (sq >> 2) + 4 * quarter_pos(sq & 3);
          const int trow = 8 * sd - c0;
          if (trow >= 0 && trow < DC) {
            store_transposed_4x8(&qt_lds[buf][trow * QTP + col], QTP, qr);
            store_transposed_4x8(&dot_lds[buf][trow * QTP + col], QTP, dr);
          }
        }
      }
      if (tid < BM) {
        lse_lds[buf][tid] = (lse_raw == -INF) ? INF : lse_raw * kLog2e;   // rows that saw no key get P = 0
        dlt_lds[buf][tid] = dlt_raw;
      }
    };

    // MASK (a std::bool_constant): the step applies the causal mask
    auto step = [&](int s, auto mask_tag) {
      constexpr bool MASK = decltype(mask_tag)::value;
      const int buf = s & 1;
      const int qt = i_first + unit_of(s) % n_qt;
      if (s + 1 < n_steps) load_regs(s + 1);
      // S[q][key], dP[q][key] of query block qb: A = Q / dO rows, B = K / V fragments
      auto scores = [&](int qb, f32x16& sacc, f32x16& pacc) {
        sacc = f32x16{};
        pacc = f32x16{};
        const __bf16* qp = &q_lds[buf][(32 * qb + l32) * QP + 8 * hh];
        const __bf16* dp = &do_lds[buf][(32 * qb + l32) * QP + 8 * hh];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          sacc = mfma32x32x16(*(const bf16x8*)(qp + 16 * ks), kf[ks], sacc);
          pacc = mfma32x32x16(*(const bf16x8*)(dp + 16 * ks), vf[ks], pacc);
        }
      };
      // P = exp2(S*c - LSE*log2e); dS = P * (dP - delta); then
      // dV^T[d][key] += dO^T P ; dK^T[d][key] += Q^T dS  (A operands from the transposed tiles)
      auto grads = [&](int qb, const f32x16& sacc, const f32x16& pacc) {
        // AGPR path: the A operands first, so their LDS reads complete under the
        // softmax VALU work (the hand-written MFMAs keep their program order)
        bf16x8 dfr[DB][2], qfr[DB][2];
        if constexpr (T::ACC_AGPR) {
#pragma unroll
          for (int db = 0; db < DB; ++db) {
            const __bf16* dtp = &dot_lds[buf][(32 * db + l32) * QTP + 32 * qb + 8 * hh];
            const __bf16* qtp = &qt_lds[buf][(32 * db + l32) * QTP + 32 * qb + 8 * hh];
            dfr[db][0] = *(const bf16x8*)(dtp);
            dfr[db][1] = *(const bf16x8*)(dtp + 16);
            qfr[db][0] = *(const bf16x8*)(qtp);
            qfr[db][1] = *(const bf16x8*)(qtp + 16);
          }
        }
        float pv[16], dsv[16];
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const int q0 = 32 * qb + 8 * r4 + 4 * hh;
          const f32x4 l4 = *(const f32x4*)&lse_lds[buf][q0];
          const f32x4 d4 = *(const f32x4*)&dlt_lds[buf][q0];
#pragma unroll
          for (int x = 0; x < 4; ++x) {
            const int r = 4 * r4 + x;
            float p = fast_exp2(fmaf(sacc[r], a.scale_log2, -l4[x]));
            if constexpr (MASK) p = (my_key <= qt * BM + q0 + x + off) ? p : 0.f;
            pv[r] = p;
            dsv[r] = p * (pacc[r] - d4[x]);
          }
        }
        const bf16x8 pb0 = to_bf16x8(pv), pb1 = to_bf16x8(pv + 8);
        const bf16x8 sb0 = to_bf16x8(dsv), sb1 = to_bf16x8(dsv + 8);
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          if constexpr (T::ACC_AGPR) {
            mfma4_acc_agpr(dvt[db], dkt[db], dfr[db][0], dfr[db][1], qfr[db][0], qfr[db][1], pb0, pb1, sb0, sb1);
          } else {
            const __bf16* dtp = &dot_lds[buf][(32 * db + l32) * QTP + 32 * qb + 8 * hh];
            const __bf16* qtp = &qt_lds[buf][(32 * db + l32) * QTP + 32 * qb + 8 * hh];
            dvt[db] = mfma32x32x16(*(const bf16x8*)(dtp), pb0, dvt[db]);
            dvt[db] = mfma32x32x16(*(const bf16x8*)(dtp + 16), pb1, dvt[db]);
            dkt[db] = mfma32x32x16(*(const bf16x8*)(qtp), sb0, dkt[db]);
            dkt[db] = mfma32x32x16(*(const bf16x8*)(qtp + 16), sb1, dkt[db]);
          }
        }
      };
      if constexpr (BM == 64) {
        // both query blocks' S/dP first: the second block's MFMAs run while the
        // first block's softmax occupies the VALU
        f32x16 s0, p0, s1, p1;
        scores(0, s0, p0);
        scores(1, s1, p1);
        grads(0, s0, p0);
        grads(1, s1, p1);
      } else {
#pragma unroll
        for (int qb = 0; qb < BM / 32; ++qb) {
          f32x16 sacc, pacc;
          scores(qb, sacc, pacc);
          grads(qb, sacc, pacc);
        }
      }
      // Every path out of the step (to the next step, the other step loop or the
      // epilogue) starts after this wait, so the copies of the accumulators the
      // compiler may place where those paths join read finished results.
      if constexpr (T::ACC_AGPR) agpr_settle(dkt, dvt);
      debug_barrier();
      // Self-attention: unconditional, so the staging shares the step's basic block
      // and the scheduler can interleave it with the gradient MFMAs (dense causal
      // and GEM s = 0.1 dK/dV -1.3 %); the last step writes stale registers into
      // the stage nobody reads again before the barrier.  Broadcast-Q items are
      // Nq / 64 steps long (4 at Nq = 256), where that wasted last staging costs
      // more than the interleaving saves (+1 %), so they skip it.
      if constexpr (BCAST) {
        if (s + 1 < n_steps) store_lds(buf ^ 1);
      } else {
        store_lds(buf ^ 1);
      }
      __syncthreads();
    };

    if (n_steps > 0) {
      load_regs(0);   // in flight together with the K/V rows: one round trip
      wait_vmem_all();
      if constexpr (KV_VIA_LDS) {
        // wave w's K and V blocks (32 rows, pitch D + 8) in one stage-1 array
        constexpr int EP = D + 8;
        static_assert(2 * 32 * EP <= BM * QP && 2 * 32 * EP <= DC * QTP, "K/V blocks fit a stage");
        __bf16* kvb = w == 0 ? &q_lds[1][0] : w == 1 ? &do_lds[1][0] : w == 2 ? &qt_lds[1][0] : &dot_lds[1][0];
#pragma unroll
        for (int i = 0; i < KV_PER; ++i) {
          const int id = lane + 64 * i, row = id / KV_CPR, col = id % KV_CPR;
          *(u32x4*)(kvb + row * EP + 8 * col) = kraw[i];
          *(u32x4*)(kvb + (32 + row) * EP + 8 * col) = vraw[i];
        }
        store_lds(0);
        __syncthreads();
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          kf[ks] = *(const bf16x8*)(kvb + l32 * EP + 16 * ks + 8 * hh);
          vf[ks] = *(const bf16x8*)(kvb + (32 + l32) * EP + 16 * ks + 8 * hh);
        }
        __syncthreads();   // every wave holds its fragments before step 0 restages stage 1
      } else {
        store_lds(0);
        __syncthreads();
      }
      // Causal: only the query tiles of a head that reach past this key tile's
      // diagonal (the first n_diag of each head's n_qt) need the mask; the
      // others run the step without it.
      if constexpr (SPLIT_MASK) {
        int s = 0;
        for (; s < n_mask; ++s) step(s, std::true_type{});
        for (; s < n_steps; ++s) step(s, std::false_type{});
      } else {
        for (int s = 0; s < n_steps; ++s) step(s, std::bool_constant<CAUSAL>{});
      }
    }

    // epilogue: dK = scale * dK^T, dV = dV^T of the owned slice.  A lane holds 4
    // consecutive columns of one key per register quad, so direct stores would
    // write 32 rows in 8-byte pieces per instruction; the wave's 32 x DC block is
    // transposed through LDS instead (free after the last step's barrier) and
    // written back 16 bytes per lane, DC / 8 lanes covering one row.
    debug_barrier();
    {
      constexpr int EP = DC + 8;                 // row pitch of the epilogue blocks
      static_assert(2 * 32 * EP <= 2 * BM * QP && 2 * 32 * EP <= 2 * DC * QTP, "epilogue blocks fit");
      __bf16* kblk = (w < 2 ? &q_lds[0][0] : &do_lds[0][0]) + (w & 1) * 32 * EP;
      __bf16* vblk = (w < 2 ? &qt_lds[0][0] : &dot_lds[0][0]) + (w & 1) * 32 * EP;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          bf16x4 kv4, vv4;
#pragma unroll
          for (int x = 0; x < 4; ++x) {
            kv4[x] = (__bf16)(dkt[db][4 * r4 + x] * a.scale);
            vv4[x] = (__bf16)(dvt[db][4 * r4 + x]);
          }
          const int d0 = 32 * db + 8 * r4 + 4 * hh;
          *(bf16x4*)(kblk + l32 * EP + d0) = kv4;
          *(bf16x4*)(vblk + l32 * EP + d0) = vv4;
        }
      // Claim the next item before the global stores: waiting for the atomic's
      // result then waits for no store (the memory counter drains in order).
      if (tid == 0) s_item[slot ^ 1] = next_work_item(a.queues, s_queue, home_q, drained);
      __syncthreads();
      constexpr int CPR = DC / 8;                // 16-byte chunks per row
      static_assert(CPR % 2 == 0, "whole chunks per lane");
#pragma unroll 1
      for (int i = 0; i < CPR / 2; ++i) {   // not unrolled: per-lane addresses are not kept across items
        const int id = lane + 64 * i, row = id / CPR, col = id % CPR;
        const int key = kt0 + 32 * w + row;
        if (key < lk) {
          const int64_t dst = ((int64_t)(k_base + key) * a.hkv + g) * D + c0 + 8 * col;
          *(u32x4*)(a.dk + dst) = *(const u32x4*)(kblk + row * EP + 8 * col);
          *(u32x4*)(a.dv + dst) = *(const u32x4*)(vblk + row * EP + 8 * col);
        }
      }
    }
    __syncthreads();   // next item published; the epilogue blocks are read
    slot ^= 1;
    item = __builtin_amdgcn_readfirstlane(s_item[slot]);
  }
}

// ============================================================================= dQ
// Broadcast-Q dQ splits the items into chunks of about equal cost (key tiles,
// plus one for an item's own loads): the cost prefix over the items lives in LDS
// for up to kBcastPrefixItems items, beyond which chunks hold equal item counts.
constexpr int kBcastPrefixItems = 2048;

// Exclusive prefix sum of one value per thread over the workgroup (blockDim a
// multiple of 64, at most 16 waves); *total receives the sum.  wave_tot: 16 ints
// of LDS.  Two barriers.
__device__ int block_exclusive_scan(int x, int* wave_tot, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  int incl = x;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(incl, off, 64);
    if (lane >= off) incl += y;
  }
  if (lane == 63) wave_tot[wave] = incl;
  __syncthreads();
  int before = 0, sum = 0;
  for (int w = 0; w < nw; ++w) {
    const int t = wave_tot[w];
    before += w < wave ? t : 0;
    sum += t;
  }
  *total = sum;
  __syncthreads();
  return before + incl - x;
}

// NARROW (d = 128): the 4-wave, 128-row workgroup, two per CU, for problems of
// short sequences, whose items are a few tiles long: two resident workgroups per
// CU overlap one item's load latency with the other's work.
template <int D, bool NARROW = false>
struct DqTile {
  // keys per tile: 32, with the LDS stage double-buffered (one barrier per tile;
  // the next tile's stores leave the critical path); d = 96 splits evenly over
  // the 256 staging threads only with 64-key tiles, of which two workgroups per
  // CU fit a single stage
  static constexpr int BN = D == 96 ? 64 : 32;
  static constexpr int NSTAGE = BN == 32 ? 2 : 1;
  static constexpr int CH = D / 8;
  // d = 128: one workgroup of 8 waves per CU owning 256 query rows, so that each
  // K/V tile brought into the CU serves 256 rows (as in the forward); d = 64 /
  // 96: two 4-wave workgroups of 128 rows (their tiles do not split over 512
  // threads); d = 192 / 256 keep Q, dO and dQ^T of the whole head in the
  // registers of one wave per SIMD
  static constexpr int NT = (!NARROW && D <= 128 && (BN * CH) % 512 == 0) ? 512 : 256;
  static constexpr int BM = NT / 2;          // query rows per item (32 per wave)
  static constexpr int WG_PER_CU = (NT == 256 && D <= 128) ? 2 : 1;
  static constexpr int KP = D + 8;           // row pitch of K / V tiles
  static constexpr int KTP = BN + 8;         // row pitch of the K^T tile
  static constexpr int VLOADS = BN * CH / NT;
  static constexpr int KBLOCKS = (BN / 4) * (D / 8);
  static constexpr int KS = D / 16;
  static constexpr int DB = D / 32;
  static constexpr int EP = D + 8;           // row pitch of the epilogue blocks
  // the 8-wave epilogue blocks get LDS of their own (one workgroup per CU)
  static constexpr int EP_EL = NT == 512 ? (NT / 64) * 32 * EP : 1;
  static_assert(BN * CH % NT == 0 && KBLOCKS <= NT, "tile load split");
  static_assert(WG_PER_CU * (NSTAGE * (2 * BN * KP + D * KTP) + EP_EL) * 2 <= 160 * 1024, "LDS budget");
};

template <int D, bool CAUSAL, bool BCAST, bool NARROW>
__global__ __launch_bounds__((DqTile<D, NARROW>::NT), (DqTile<D, NARROW>::WG_PER_CU)) void bwd_dq_kernel(BwdArgs a) {
  using T = DqTile<D, NARROW>;
  constexpr int BM = T::BM, BN = T::BN, KP = T::KP, KTP = T::KTP, KS = T::KS, DB = T::DB;
  constexpr int NSTAGE = T::NSTAGE;
  __shared__ __attribute__((aligned(16))) __bf16 k_lds[NSTAGE][BN * KP];
  __shared__ __attribute__((aligned(16))) __bf16 v_lds[NSTAGE][BN * KP];
  __shared__ __attribute__((aligned(16))) __bf16 kt_lds[NSTAGE][D * KTP];
  __shared__ __attribute__((aligned(16))) __bf16 ep_lds[T::EP_EL];
  __shared__ int s_item[2];   // claims alternate between the entries: a wave still
  // reading claim k's entry has not passed the barrier that follows claim k + 1, so
  // claim k + 2, the next write to that entry, cannot overtake the read even when
  // item k + 1 has no tiles (and so no barrier of its own)
  __shared__ int s_queue[2 * kQueues];

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, hh = lane >> 5;
  const float NEG_INF = -__builtin_inff(), INF = __builtin_inff();

  // staging: K as one 4-key x 8-column block per thread (written row-major and
  // transposed); V as row-major 16-byte chunks
  const int rs = a.hkv * D;
  int skb, skd;
  staging_block(tid, BN / 4, skb, skd);
  const bool k_stager = skd < D / 8;
  uint32_t koff[4], voff[T::VLOADS];
#pragma unroll
  for (int i = 0; i < 4; ++i) koff[i] = (uint32_t)(((4 * skb + i) * rs + 8 * skd) * 2);
#pragma unroll
  for (int i = 0; i < T::VLOADS; ++i) {
    const int id = tid + i * T::NT;
    voff[i] = (uint32_t)(((id / T::CH) * rs + (id % T::CH) * 8) * 2);
  }

  // Broadcast-Q chunks: item b owns the cost positions [s_pre[b], s_pre[b + 1]):
  // one for its own loads, then one per key tile.  Chunk c takes the positions
  // [c, c + 1) * total / chunks, so an item's key tiles may be split between two
  // chunks.  Every workgroup derives the same cuts from the offsets, so the
  // chunking (and the chunk-ordered dQ sum) depends on the lengths alone.
  __shared__ int s_pre[BCAST ? kBcastPrefixItems + 1 : 1];
  __shared__ int s_wave_tot[16];
  const bool by_cost = BCAST && a.batch <= kBcastPrefixItems;
  if (BCAST && by_cost) {
    const int per = cdiv(a.batch, T::NT);
    const int lo = min(tid * per, a.batch), hi = min(lo + per, a.batch);
    auto cost = [&](int b) {
      const int lk = a.cu_k[b + 1] - a.cu_k[b];
      return lk > 0 ? cdiv(lk, BN) + 1 : 0;
    };
    int run = 0;
    for (int b = lo; b < hi; ++b) run += cost(b);
    int total;
    int base = block_exclusive_scan(run, s_wave_tot, &total);
    for (int b = lo; b < hi; ++b) {
      s_pre[b] = base;
      base += cost(b);
    }
    if (tid == 0) s_pre[a.batch] = total;
    __syncthreads();
  }
  // first cost position of chunk c, and the smallest b in [lo, batch] with
  // s_pre[b] > pos (strict) or >= pos
  auto chunk_pos = [&](int c) {
    return (int)(((int64_t)c * s_pre[a.batch] + a.bcast_chunks - 1) / a.bcast_chunks);
  };
  auto first_item = [&](int lo, int pos, bool strict) {
    int hi = a.batch;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (strict ? s_pre[mid] > pos : s_pre[mid] >= pos) hi = mid;
      else lo = mid + 1;
    }
    return lo;
  };

  // Work: self-attention pulls (sequence, query tile, head) items from the per-XCD
  // work queues; broadcast-Q owns (query tile, head, chunk of items) by block index.
  int bcast_item = blockIdx.x;
  int home_q = blockIdx.x % kQueues, drained = 0;   // work-queue state (thread 0)
  int item = -1, slot = 0;   // slot: s_item entry of the current claim (uniform)
  if (!BCAST) {   // broadcast-Q runs without a work list (a.queues is null)
    load_queues(a.queues, s_queue);
    __syncthreads();
    if (tid == 0) s_item[0] = next_work_item(a.queues, s_queue, home_q, drained);
    __syncthreads();
    item = __builtin_amdgcn_readfirstlane(s_item[0]);   // uniform: the item loads are scalar
  }
  for (;;) {
    int b_lo, b_hi, h, qtile, chunk = 0;
    int pos_lo = 0, pos_hi = 0;   // broadcast-Q, by cost: the chunk's cost positions
    int e_qbase = 0, e_lq = 0, e_kbase = 0, e_lk = 0;   // self-attention: the item's sequence
    if (BCAST) {
      if (bcast_item >= a.bcast_units) break;
      const int per_tile = a.hq * a.bcast_chunks;
      qtile = bcast_item / per_tile;
      const int rem = bcast_item % per_tile;
      h = rem / a.bcast_chunks;
      chunk = rem % a.bcast_chunks;
      if (by_cost) {
        pos_lo = chunk_pos(chunk);
        pos_hi = chunk_pos(chunk + 1);
        b_lo = max(0, first_item(1, pos_lo, true) - 1);   // the item holding position pos_lo
        b_hi = first_item(0, pos_hi, false);               // the first item starting at or past pos_hi
      } else {
        b_lo = min(a.batch, chunk * a.bcast_chunk);
        b_hi = min(a.batch, b_lo + a.bcast_chunk);
      }
      bcast_item += gridDim.x;
    } else {
      if (item < 0) break;
      const WorkItem e = a.items[item];
      h = e.h;
      b_lo = e.b;
      b_hi = e.b + 1;
      qtile = e.t;
      e_qbase = e.q_base;
      e_lq = e.lq;
      e_kbase = e.k_base;
      e_lk = e.lk;
    }
    const int g = h / a.group;
    const int row0 = qtile * BM;
    const int my_row = row0 + w * 32 + l32;

    f32x16 dqt[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) dqt[db] = f32x16{};

    // Q fragment: B operand of S^T = K Q^T.  Broadcast-Q shares one Q among all
    // items, so it is loaded once per unit; self-attention loads it per item below.
    bf16x8 qf[KS];
    if constexpr (BCAST) {
      const bool q_ok = my_row < a.bcast_nq;
      const __bf16* qp = a.q + ((int64_t)my_row * a.hq + h) * D + 8 * hh;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) qf[ks] = q_ok ? *(const bf16x8*)(qp + 16 * ks) : zero_bf16x8();
    }

    for (int b = b_lo; b < b_hi; ++b) {
      int lq, q_base, k_base, lk;
      if (BCAST) { lq = a.bcast_nq; q_base = 0; k_base = a.cu_k[b]; lk = a.cu_k[b + 1] - k_base; }
      else { lq = e_lq; q_base = e_qbase; k_base = e_kbase; lk = e_lk; }
      const bool row_ok = my_row < lq;
      const bool wave_rows = row0 + w * 32 < lq;   // uniform per wave
      const int off = lk - lq;

      int n_tiles, n_bulk;
      if (CAUSAL) {
        const int kmax = min(lk, row0 + BM + off);
        n_tiles = kmax > 0 ? cdiv(kmax, BN) : 0;
        const int full = min(lk, row0 + off + 1);
        n_bulk = full > 0 ? full / BN : 0;
      } else {
        n_tiles = cdiv(lk, BN);
        n_bulk = lk / BN;
      }
      // broadcast-Q by cost: the item's key tiles [t0, t0 + n_tiles) that fall
      // into this chunk's positions (the item's first position is its own loads)
      int t0 = 0;
      if (BCAST && by_cost) {
        const int pb = s_pre[b] + 1;
        t0 = max(0, pos_lo - pb);
        const int t1 = min(n_tiles, pos_hi - pb);
        n_bulk = max(0, min(n_bulk, t1) - t0);
        n_tiles = max(0, t1 - t0);
      }
      if (BCAST && n_tiles == 0) continue;   // uniform

      const __bf16* kbase = a.k + ((int64_t)k_base * a.hkv + g) * D;
      const __bf16* vbase = a.v + ((int64_t)k_base * a.hkv + g) * D;
      u32x4 kr[4], vr[T::VLOADS];
      auto load_regs = [&](int j) {
        const int64_t tile_off = (int64_t)j * BN * rs;
        const uint32_t nbytes = (uint32_t)(min(lk - j * BN, BN) * rs * 2);
        const auto krs = uniform_rsrc(kbase + tile_off, nbytes);
        const auto vrs = uniform_rsrc(vbase + tile_off, nbytes);
        if (k_stager) {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            kr[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(krs, koff[i], 0, 0));
        }
#pragma unroll
        for (int i = 0; i < T::VLOADS; ++i)
          vr[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(vrs, voff[i], 0, 0));
      };
      auto store_lds = [&](int st) {
        if (k_stager) {
#pragma unroll
          for (int i = 0; i < 4; ++i) *(u32x4*)&k_lds[st][(4 * skb + i) * KP + 8 * skd] = kr[i];
          store_transposed_4x8(&kt_lds[st][(8 * skd) * KTP + 16 * (skb >> 2) + 4 * quarter_pos(skb & 3)], KTP, kr);
        }
#pragma unroll
        for (int i = 0; i < T::VLOADS; ++i) {
          const int id = tid + i * T::NT;
          *(u32x4*)&v_lds[st][(id / T::CH) * KP + (id % T::CH) * 8] = vr[i];
        }
      };

      // Key-tile order: bulk tiles first, masked tiles last, the same order for
      // every item sharing this K/V (they run together on one XCD and find the
      // same K/V tiles in its L2).
      auto tile_of = [&](int s) { return t0 + s; };
      // the first K/V tile travels with the Q / dO / O fragments: one round trip
      if (n_tiles > 0) load_regs(tile_of(0));

      // per-row state: Q and dO fragments (B operands of S^T = K Q^T, dP^T = V dO^T), LSE, delta
      bf16x8 df[KS];
      float lse2 = INF, dlt = 0.f;
      {
        const __bf16* qp = a.q + ((int64_t)(q_base + my_row) * a.hq + h) * D + 8 * hh;
        const int64_t orow = BCAST ? (int64_t)b * lq + my_row : (int64_t)(q_base + my_row);
        const __bf16* op = a.dout + (orow * a.hq + h) * D + 8 * hh;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          if constexpr (!BCAST) qf[ks] = row_ok ? *(const bf16x8*)(qp + 16 * ks) : zero_bf16x8();
          df[ks] = row_ok ? *(const bf16x8*)(op + 16 * ks) : zero_bf16x8();
        }
        const int64_t li = BCAST ? ((int64_t)b * a.hq + h) * lq + my_row : (int64_t)h * a.total_q + q_base + my_row;
        if (BCAST) {
          if (row_ok) dlt = a.delta[li];   // written by bwd_pre_kernel
        } else {
          // delta = rowsum(dO * O): each lane holds half of the row, its partner lane the other half.
          // Written for every row, also of tiles that see no key, for the dK/dV kernel.
          const __bf16* orp = a.o + ((int64_t)(q_base + my_row) * a.hq + h) * D + 8 * hh;
          float part = 0.f;
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) {
            const bf16x8 ov = row_ok ? *(const bf16x8*)(orp + 16 * ks) : zero_bf16x8();
#pragma unroll
            for (int e = 0; e < 8; ++e) part = fmaf((float)ov[e], (float)df[ks][e], part);
          }
          dlt = xhalf_sum(part);
          if (row_ok && hh == 0) a.delta[li] = dlt;
        }
        if (row_ok) {
          const float l = a.lse[li];
          lse2 = (l == NEG_INF) ? INF : l * kLog2e;
        }
      }
      if (!BCAST && n_tiles == 0) continue;   // uniform; delta is written


      auto tile = [&](int s, auto mask_tag) {
        constexpr bool MASK = decltype(mask_tag)::value;
        const int j = tile_of(s);
        const int stg = NSTAGE == 2 ? (s & 1) : 0;
        if (NSTAGE == 1) {   // one stage: fill it once every reader of the last tile is done
          store_lds(0);
          __syncthreads();
        }
        if (s + 1 < n_tiles) load_regs(tile_of(s + 1));
        const int kmax_ok = CAUSAL ? min(lk - 1, my_row + off) : lk - 1;
        // a wave whose 32 rows all lie past the sequence end only stages and syncs;
        // in a causal diagonal tile, so does a wave for the 32-key blocks past its
        // last row's diagonal (the blocks are in key order: the live ones come first)
        int live_kb = wave_rows ? BN / 32 : 0;
        if (CAUSAL && MASK && wave_rows)
          live_kb = max(0, min(BN / 32, cdiv(row0 + 32 * w + 31 + off + 1 - j * BN, 32)));
#pragma unroll
        for (int kb = 0; kb < live_kb; ++kb) {
          // S^T[key][q] = K Q^T and dP^T[key][q] = V dO^T for 32 keys
          f32x16 st = f32x16{}, pt = f32x16{};
          const __bf16* kp = &k_lds[stg][(32 * kb + l32) * KP + 8 * hh];
          const __bf16* vp = &v_lds[stg][(32 * kb + l32) * KP + 8 * hh];
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) {
            st = mfma32x32x16(*(const bf16x8*)(kp + 16 * ks), qf[ks], st);
            pt = mfma32x32x16(*(const bf16x8*)(vp + 16 * ks), df[ks], pt);
          }
          float dsv[16];
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            float p = fast_exp2(fmaf(st[r], a.scale_log2, -lse2));
            if constexpr (MASK) {
              const int key = j * BN + 32 * kb + 8 * (r >> 2) + 4 * hh + (r & 3);
              p = key <= kmax_ok ? p : 0.f;
            }
            dsv[r] = p * (pt[r] - dlt);
          }
          const bf16x8 sb0 = to_bf16x8(dsv), sb1 = to_bf16x8(dsv + 8);
          // dQ^T[d][q] += K^T[d][key] dS^T[key][q]
#pragma unroll
          for (int db = 0; db < DB; ++db) {
            const __bf16* ktp = &kt_lds[stg][(32 * db + l32) * KTP + 32 * kb + 8 * hh];
            dqt[db] = mfma32x32x16(*(const bf16x8*)(ktp), sb0, dqt[db]);
            dqt[db] = mfma32x32x16(*(const bf16x8*)(ktp + 16), sb1, dqt[db]);
          }
        }
        // two stages: the next tile goes into the other stage, whose readers
        // finished before the previous barrier; one stage: refilled next tile
        debug_barrier();
        if (NSTAGE == 2 && s + 1 < n_tiles) store_lds(stg ^ 1);
        __syncthreads();
      };

      if (NSTAGE == 2) {
        store_lds(0);
        __syncthreads();
      }
      for (int s = 0; s < n_bulk; ++s) tile(s, std::false_type{});
      for (int s = n_bulk; s < n_tiles; ++s) tile(s, std::true_type{});
    }

    // epilogue: dQ = scale * dQ^T
    if (BCAST && my_row < a.bcast_nq) {
      // this chunk's partial, 4 consecutive d per store (summed in order by dq_convert)
      float* dst = a.dq_part + (((int64_t)chunk * a.bcast_nq + my_row) * a.hq + h) * D;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4)
          *(f32x4*)(dst + 32 * db + 8 * r4 + 4 * hh) =
              f32x4{dqt[db][4 * r4], dqt[db][4 * r4 + 1], dqt[db][4 * r4 + 2], dqt[db][4 * r4 + 3]};
    }
    debug_barrier();
    if (!BCAST) {
      // A lane holds 4 consecutive columns of its row per register quad; the
      // wave's 32 x D block goes through LDS (4 waves: the stages, free after the
      // last tile's closing barrier, waves 0-1 in the K stages and 2-3 in the V
      // stages; 8 waves: LDS of their own) and out 16 bytes per lane, D / 8 lanes
      // covering one row.
      constexpr int EP = T::EP;
      static_assert(T::NT == 512 || 2 * 32 * EP <= NSTAGE * BN * KP, "epilogue blocks fit");
      __bf16* blk = T::NT == 512 ? &ep_lds[0] + w * 32 * EP
                                 : (w < 2 ? &k_lds[0][0] : &v_lds[0][0]) + (w & 1) * 32 * EP;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          bf16x4 v4;
#pragma unroll
          for (int x = 0; x < 4; ++x) v4[x] = (__bf16)(dqt[db][4 * r4 + x] * a.scale);
          *(bf16x4*)(blk + l32 * EP + 32 * db + 8 * r4 + 4 * hh) = v4;
        }
      // claim the next item before any global store: waiting for the atomic's
      // result then waits for no store (the memory counter drains in order)
      if (tid == 0) s_item[slot ^ 1] = next_work_item(a.queues, s_queue, home_q, drained);
      __syncthreads();
      constexpr int CPR = D / 8;             // 16-byte chunks per row
      static_assert(CPR % 2 == 0, "whole chunks per lane");
#pragma unroll 1
      for (int i = 0; i < CPR / 2; ++i) {    // not unrolled: per-lane addresses are not kept across items
        const int id = lane + 64 * i, row = id / CPR, col = id % CPR;
        const int r = row0 + 32 * w + row;
        if (r < e_lq)
          *(u32x4*)(a.dq + ((int64_t)(e_qbase + r) * a.hq + h) * D + 8 * col) = *(const u32x4*)(blk + row * EP + 8 * col);
      }
      __syncthreads();   // next item published; the LDS blocks are read
      slot ^= 1;
      item = __builtin_amdgcn_readfirstlane(s_item[slot]);
    }
  }
}

#ifndef JFA_BWD_WIDE_UNIT
int bwd_dkdv_tile() { return DkvTile<128>::BN; }
int bwd_dkdv_rows(int head_dim) { return head_dim <= 128 ? DkvTile<128>::BM : DkvTile<256>::BM; }
int bwd_dkdv_slices(int head_dim) {
  return head_dim <= 128 ? DkvTile<128>::NC : head_dim <= 192 ? DkvTile<192>::NC : DkvTile<256>::NC;
}
int bwd_dq_rows(int head_dim, bool narrow) {
  if (head_dim == 128 && narrow) return DqTile<128, true>::BM;
  return head_dim == 64 ? DqTile<64>::BM : head_dim == 96 ? DqTile<96>::BM : head_dim == 128 ? DqTile<128>::BM : DqTile<256>::BM;
}
int bwd_dq_tile(int head_dim) {
  return head_dim == 64 ? DqTile<64>::BN : head_dim == 96 ? DqTile<96>::BN : head_dim == 128 ? DqTile<128>::BN : DqTile<256>::BN;
}
int bwd_dq_blocks_per_cu(int head_dim, bool narrow) {
  if (head_dim == 128 && narrow) return DqTile<128, true>::WG_PER_CU;
  return head_dim == 64 ? DqTile<64>::WG_PER_CU : head_dim == 96 ? DqTile<96>::WG_PER_CU
       : head_dim == 128 ? DqTile<128>::WG_PER_CU : DqTile<256>::WG_PER_CU;
}
#endif  // JFA_BWD_WIDE_UNIT

template <int D>
static hipError_t launch_dkdv_d(const BwdArgs& a, int grid, hipStream_t stream) {
  const dim3 g(grid), blk(DkvTile<D>::NT);
  if (a.bcast) hipLaunchKernelGGL((bwd_dkdv_kernel<D, false, true>), g, blk, 0, stream, a);
  else if (a.causal) hipLaunchKernelGGL((bwd_dkdv_kernel<D, true, false>), g, blk, 0, stream, a);
  else hipLaunchKernelGGL((bwd_dkdv_kernel<D, false, false>), g, blk, 0, stream, a);
  return hipGetLastError();
}

template <int D, bool NARROW>
static hipError_t launch_dq_dn(const BwdArgs& a, int grid, hipStream_t stream) {
  const dim3 g(grid), blk(DqTile<D, NARROW>::NT);
  if (a.bcast) hipLaunchKernelGGL((bwd_dq_kernel<D, false, true, NARROW>), g, blk, 0, stream, a);
  else if (a.causal) hipLaunchKernelGGL((bwd_dq_kernel<D, true, false, NARROW>), g, blk, 0, stream, a);
  else hipLaunchKernelGGL((bwd_dq_kernel<D, false, false, NARROW>), g, blk, 0, stream, a);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_dq_d(const BwdArgs& a, int grid, hipStream_t stream) {
  if constexpr (D == 128) {
    if (a.narrow) return launch_dq_dn<D, true>(a, grid, stream);
  }
  return launch_dq_dn<D, false>(a, grid, stream);
}

#ifndef JFA_BWD_WIDE_UNIT
hipError_t launch_bwd_dkdv(const BwdArgs& a, int head_dim, int grid, hipStream_t stream) {
  switch (head_dim) {
    case 64: return launch_dkdv_d<64>(a, grid, stream);
    case 96: return launch_dkdv_d<96>(a, grid, stream);
    case 128: return launch_dkdv_d<128>(a, grid, stream);
    case 192:
    case 256: return launch_bwd_dkdv_wide(a, head_dim, grid, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_bwd_dq(const BwdArgs& a, int head_dim, int grid, hipStream_t stream) {
  switch (head_dim) {
    case 64: return launch_dq_d<64>(a, grid, stream);
    case 96: return launch_dq_d<96>(a, grid, stream);
    case 128: return launch_dq_d<128>(a, grid, stream);
    case 192: return launch_bwd_dq_wide(a, head_dim, grid, stream);
    case 256: return launch_dq_d<256>(a, grid, stream);
    default: return hipErrorInvalidValue;
  }
}
#else
hipError_t launch_bwd_dkdv_wide(const BwdArgs& a, int head_dim, int grid, hipStream_t stream) {
  switch (head_dim) {
    case 192: return launch_dkdv_d<192>(a, grid, stream);
    case 256: return launch_dkdv_d<256>(a, grid, stream);
    default: return hipErrorInvalidValue;
  }
}

// The dQ kernel has no hand-written MFMAs; at d = 192 it is 2 % faster built here
// (equal or slower at d = 256, which stays in the other unit).
hipError_t launch_bwd_dq_wide(const BwdArgs& a, int head_dim, int grid, hipStream_t stream) {
  return head_dim == 192 ? launch_dq_d<192>(a, grid, stream) : hipErrorInvalidValue;
}
#endif  // JFA_BWD_WIDE_UNIT

}  // namespace jfa
