// Split-KV paged decode for gfx950 ("Optimizing FlashAttention-4 for Efficient
// Inference": KV-dimension parallelism of PR 1940, arbitrary page sizes of
// PR 1999/2104, a query tile holding only real rows as in PR 1993, and GQA
// packing of PR 2186).
//
// One workgroup handles one (sequence b, KV head g, split s) unit: the Hq/Hkv
// query heads of group g form the columns of a 16-wide query tile, so every K/V
// byte of the chunk is read once for the whole group.  The chunk's keys are
// gathered row by row through the page table (any page size; rows are never
// read past the sequence end) into LDS, 64 keys per tile, with the next tile's
// loads in flight while the current one is consumed.  Each of the 4 waves takes
// 16 keys of a tile:
//   S^T[key][q]  = K Q^T      v_mfma_f32_16x16x32_bf16, A = K rows from LDS
//   online softmax over the 16 keys x query column (per-lane + cross-lane)
//   O^T[d][q]   += V^T P^T    v_mfma_f32_16x16x16_f16, A = V (staged as fp16)
//                             through the transposed LDS read, B = P^T rounded
//                             to fp16 straight from the S^T accumulator (P keeps
//                             11 significant bits; a unit whose V holds a value
//                             beyond the fp16 range is computed again with P V
//                             in bf16, as in the forward)
// The four waves' (max, sum, accumulator) states are merged through LDS at the
// end.  With one split the result is final (bf16 O, LSE); otherwise each split
// leaves its normalised fp32 partial and its LSE, and the partials are merged
// with weights exp(LSE_s - LSE) (the LSE-weighted combine the split-KV scheme of
// PR 1940 implies): by decode_combine_kernel in a second launch, or (single-
// launch mode) by the unit's last split to finish, in the decode launch itself,
// which learns that it is last from a per-unit arrival counter.  The second
// launch is the default: on the MI355X the single-launch merge measured 1-2 %
// slower on 32 sequences of 4k-16k tokens and 5-17 % on batches of 1-8, as every
// workgroup then waits for its partial stores and the counter before it exits.
#include <type_traits>

#include "jfa_internal.h"
#include "device_common.h"

namespace jfa {

template <int D>
struct DecTile {
  static constexpr int NT = 256;
  static constexpr int BN = 64;           // keys per tile, 16 per wave
  static constexpr int KP = D + 8;        // K row pitch (elements)
  static constexpr int VP = D + 16;       // V row pitch
  static constexpr int CH = D / 8;
  static constexpr int LOADS = BN * CH / NT;
  static constexpr int KK = D / 32;       // k-steps of K Q^T
  static constexpr int DB = D / 16;       // 16-wide output blocks
  static_assert(BN * CH % NT == 0, "tile load split");
};

// Resident workgroups per CU: d <= 128 runs four one-group workgroups (two with
// two column groups); d = 192 / 256 run one column group at two per CU, where the
// K/V tile's LDS and the accumulator's registers allow no more.
template <int D, int NCG>
struct DecOcc {
  static constexpr int WG_PER_CU = D <= 128 ? (NCG == 1 ? 4 : 2) : 2;
  static_assert(D <= 128 || NCG == 1, "one column group above d = 128");
};

typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));

constexpr int kLptMaxBatch = 256;   // one rank per thread

__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16x16x16_f16(f16x4 a, f16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16x16x16_bf16(bf16x4 a, bf16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a), __builtin_bit_cast(s16x4, b), c, 0, 0, 0);
}

// NCG: 16-column query groups per workgroup (1 or 2).  A workgroup handles up to 16*NCG
// query columns (token, query head of the GQA group) of one (sequence, KV head,
// split); every K and V fragment it reads from LDS feeds all of its groups.
// FP8: the KV cache holds OCP e4m3 bytes; rows are widened exactly (every e4m3
// value is a bf16 and an fp16 value; K to bf16, V to fp16) when they are written
// to LDS, and the per-tensor scales are applied to the scores (K, folded into
// scale_log2 by the host) and to the output (V).
template <int D, int NCG, bool FP8>
__global__ __launch_bounds__(256, (DecOcc<D, NCG>::WG_PER_CU)) void decode_kernel(DecodeArgs a) {
  using T = DecTile<D>;
  constexpr int BN = T::BN, KP = T::KP, VP = T::VP, KK = T::KK, DB = T::DB;
  constexpr int KV_BYTES = BN * (KP + VP) * 2;
  constexpr int OP = D + 4;   // merge row pitch (floats): 16-byte stores of 8 lanes on distinct banks
  constexpr int MERGE_BYTES = 4 * 16 * OP * 4 + 2 * 4 * 16 * 4;
  constexpr int SMEM = KV_BYTES > MERGE_BYTES ? KV_BYTES : MERGE_BYTES;
  static_assert(DecOcc<D, NCG>::WG_PER_CU * SMEM <= 160 * 1024, "LDS budget");
  __shared__ __attribute__((aligned(16))) unsigned char smem[SMEM];
  __bf16* k_lds = (__bf16*)smem;
  __bf16* v_lds = k_lds + BN * KP;

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int l16 = lane & 15, g16 = lane >> 4;
  const float NEG_INF = -__builtin_inff();

  // Workgroup -> (chunk, KV head g) with g fastest; chunk = (b rank, split s,
  // column unit cu) with cu fastest.  The KV heads of one chunk share its token
  // rows (one row of the cache holds all Hkv heads) and are neighbouring
  // workgroups, dispatched together.  (Grouping them on one XCD instead --
  // workgroups go to the XCDs round robin -- was 1.5 % slower.)
  const int cols = a.group * a.q_len;               // query columns of one (sequence, KV head)
  const int n_cu = cdiv(cdiv(cols, 16), NCG);
  const int ci = blockIdx.x / a.hkv, g = blockIdx.x % a.hkv;
  const int cu = ci % n_cu;
  const int s = (ci / n_cu) % a.splits;
  const int b_rank = ci / n_cu / a.splits;
  // Longest sequences first: the workgroups are dispatched in index order, so the
  // units of long sequences start early and short ones fill in at the end.  The
  // rank is computed from the KV lengths by every workgroup (batches up to
  // kLptMaxBatch; larger ones keep the given order).
  __shared__ int s_b;
  // set when the fp16 accumulation was not finite (see the recomputation below)
  __shared__ int s_big;
  __shared__ int s_last;   // this workgroup is the last split of its unit to finish
  if (tid == 0) s_big = 0;
  int b = b_rank;
  if (a.batch <= kLptMaxBatch && tid < a.batch) {
    const int lt = a.seqlens[tid];
    int rank = 0;
    for (int j = 0; j < a.batch; ++j) {
      const int lj = a.seqlens[j];
      rank += (lj > lt || (lj == lt && j < tid)) ? 1 : 0;
    }
    if (rank == b_rank) s_b = tid;
  }
  __syncthreads();
  if (a.batch <= kLptMaxBatch) b = s_b;
  const int L = a.seqlens[b];
  const int chunk = cdiv(cdiv(L, a.splits), BN) * BN;
  const int k_lo = s * chunk;
  const int k_hi = min(L, k_lo + chunk);
  const int n_tiles = k_hi > k_lo ? cdiv(k_hi - k_lo, BN) : 0;

  // Query fragments.  Column c = (cu*NCG + cg)*16 + l16 is token t = c / group of
  // query head g*group + c % group; columns past the last one are zero.  With a
  // causal mask (bottom-right: the q_len tokens are the last ones of the
  // sequence) token t sees keys up to t + L - q_len.
  bf16x8 qf[NCG][KK];
  int kmax[NCG];
#pragma unroll
  for (int cg = 0; cg < NCG; ++cg) {
    const int c = (cu * NCG + cg) * 16 + l16;
    const bool ok = c < cols;
    const int t = ok ? c / a.group : 0;
    const int h = g * a.group + (ok ? c % a.group : 0);
    const int64_t qe = (((int64_t)b * a.q_len + t) * a.hq + h) * D + 8 * g16;   // element offset
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      if (!ok) qf[cg][kk] = zero_bf16x8();
      else if (a.q_fp8)   // e4m3 query: 8 bytes widened exactly to bf16
        qf[cg][kk] = __builtin_bit_cast(bf16x8, widen_e4m3x8(*(const uint2*)((const unsigned char*)a.q + qe + 32 * kk)));
      else qf[cg][kk] = *(const bf16x8*)(a.q + qe + 32 * kk);
    }
    kmax[cg] = min(k_hi - 1, a.causal ? t + L - a.q_len : L - 1);
  }

  f32x4 acc[NCG][DB];
  float m_run[NCG], l_run[NCG];
#pragma unroll
  for (int cg = 0; cg < NCG; ++cg) {
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[cg][db] = f32x4{0.f, 0.f, 0.f, 0.f};
    m_run[cg] = NEG_INF;
    l_run[cg] = 0.f;
  }

  const int32_t* pt = a.page_table + (int64_t)b * a.max_pages;
  // One 16-byte load per (row, chunk): 8 bf16 columns, or 16 fp8 columns.
  constexpr int EPL = FP8 ? 16 : 8;                  // elements per 16-byte load
  constexpr int CHL = D / EPL;                       // loads per row
  constexpr int NLD = (BN * CHL + T::NT - 1) / T::NT;
  u32x4 kr[NLD], vr[NLD];
  auto load_regs = [&](int j) {
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int id = tid + i * T::NT;
      if (BN * CHL % T::NT == 0 || id < BN * CHL) {
        const int r = id / CHL, c = id % CHL;
        const int key = min(k_lo + j * BN + r, k_hi - 1);   // never past the sequence end
        const int page = pt[key / a.page_size];
        const int slot = key - (key / a.page_size) * a.page_size;
        const int64_t el = (((int64_t)page * a.page_size + slot) * a.hkv + g) * D + c * EPL;
        const unsigned char* kb = (const unsigned char*)a.k_cache;
        const unsigned char* vb = (const unsigned char*)a.v_cache;
        kr[i] = *(const u32x4*)(kb + el * (FP8 ? 1 : 2));
        vr[i] = *(const u32x4*)(vb + el * (FP8 ? 1 : 2));
      }
    }
  };
  // 16 e4m3 bytes -> 16 bf16 (two 16-byte stores)
  auto widen = [&](const u32x4& x, u32x4& lo, u32x4& hi) {
#pragma unroll
    for (int w2 = 0; w2 < 4; ++w2) {
      typedef float f2_t __attribute__((ext_vector_type(2)));
      const f2_t p0 = __builtin_amdgcn_cvt_pk_f32_fp8(x[w2], false);
      const f2_t p1 = __builtin_amdgcn_cvt_pk_f32_fp8(x[w2], true);
      bf16x4 q;
      q[0] = (__bf16)p0[0]; q[1] = (__bf16)p0[1]; q[2] = (__bf16)p1[0]; q[3] = (__bf16)p1[1];
      const uint2 u = __builtin_bit_cast(uint2, q);
      if (w2 < 2) { lo[2 * w2] = u.x; lo[2 * w2 + 1] = u.y; }
      else { hi[2 * (w2 - 2)] = u.x; hi[2 * (w2 - 2) + 1] = u.y; }
    }
  };
  // F16 (a std::bool_constant): V is written as fp16 (e4m3 always is; a bf16
  // value beyond the fp16 range becomes infinite), otherwise as bf16.
  auto store_lds = [&](auto f16_tag) {
    constexpr bool F16 = decltype(f16_tag)::value;
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int id = tid + i * T::NT;
      if (BN * CHL % T::NT == 0 || id < BN * CHL) {
        const int r = id / CHL, c = id % CHL;
        if constexpr (FP8) {
          u32x4 k0, k1;
          widen(kr[i], k0, k1);
          const u32x4 v0 = widen_e4m3x8_f16(uint2{vr[i][0], vr[i][1]});
          const u32x4 v1 = widen_e4m3x8_f16(uint2{vr[i][2], vr[i][3]});
          *(u32x4*)&k_lds[r * KP + c * 16] = k0;
          *(u32x4*)&k_lds[r * KP + c * 16 + 8] = k1;
          *(u32x4*)&v_lds[r * VP + c * 16] = v0;
          *(u32x4*)&v_lds[r * VP + c * 16 + 8] = v1;
        } else {
          u32x4 vh = vr[i];
          if constexpr (F16) {
#pragma unroll
            for (int x = 0; x < 4; ++x) vh[x] = bf16x2_to_f16x2(vr[i][x]);
          }
          *(u32x4*)&k_lds[r * KP + c * 8] = kr[i];
          *(u32x4*)&v_lds[r * VP + c * 8] = vh;
        }
      }
    }
  };

  // The chunk's tiles; F16 selects the P V precision (fp16, or bf16 for the
  // recomputation of a unit whose V does not fit fp16).
  auto run_tiles = [&](auto f16_tag) {
    constexpr bool F16 = decltype(f16_tag)::value;
    if (n_tiles > 0) load_regs(0);
    for (int j = 0; j < n_tiles; ++j) {
      store_lds(f16_tag);
      __syncthreads();
      if (j + 1 < n_tiles) load_regs(j + 1);

      // S^T[key][column] for this wave's 16 keys and every column group
      f32x4 st[NCG];
#pragma unroll
      for (int cg = 0; cg < NCG; ++cg) st[cg] = f32x4{0.f, 0.f, 0.f, 0.f};
      const __bf16* kp = k_lds + (16 * w + l16) * KP + 8 * g16;
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        const bf16x8 kfrag = *(const bf16x8*)(kp + 32 * kk);
#pragma unroll
        for (int cg = 0; cg < NCG; ++cg) st[cg] = mfma16x16x32(kfrag, qf[cg][kk], st[cg]);
      }

      float pv[NCG][4];
      float alpha[NCG];
#pragma unroll
      for (int cg = 0; cg < NCG; ++cg) {
        float mx = NEG_INF;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int key = k_lo + j * BN + 16 * w + 4 * g16 + r;
          st[cg][r] = key <= kmax[cg] ? st[cg][r] : NEG_INF;
          mx = fmaxf(mx, st[cg][r]);
        }
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = xhalf_max(mx);
        const float m_new = fmaxf(m_run[cg], mx * a.scale_log2);
        alpha[cg] = (m_new == NEG_INF) ? 1.f : fast_exp2(m_run[cg] - m_new);
        const float m_sub = (m_new == NEG_INF) ? 0.f : m_new;
        float psum = 0.f;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          pv[cg][r] = fast_exp2(fmaf(st[cg][r], a.scale_log2, -m_sub));
          psum += pv[cg][r];
        }
        l_run[cg] = l_run[cg] * alpha[cg] + psum;
        m_run[cg] = m_new;
      }
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const __bf16* vp = v_lds + (16 * w + 4 * g16 + (l16 >> 2)) * VP + 16 * db + 4 * (l16 & 3);
#pragma unroll
        for (int cg = 0; cg < NCG; ++cg) {
          if constexpr (F16) {
            const f16x4 pb = {(_Float16)pv[cg][0], (_Float16)pv[cg][1], (_Float16)pv[cg][2], (_Float16)pv[cg][3]};
            acc[cg][db] = mfma16x16x16_f16(__builtin_bit_cast(f16x4, lds_read_tr4(vp)), pb, acc[cg][db] * alpha[cg]);
          } else {
            const bf16x4 pb = {(__bf16)pv[cg][0], (__bf16)pv[cg][1], (__bf16)pv[cg][2], (__bf16)pv[cg][3]};
            acc[cg][db] = mfma16x16x16_bf16(lds_read_tr4(vp), pb, acc[cg][db] * alpha[cg]);
          }
        }
      }
      __syncthreads();   // the tile buffer is refilled at the top of the next iteration
    }
  };
  run_tiles(std::true_type{});   // e4m3 V is widened to fp16 as well
  if constexpr (!FP8) {
    // A bf16 V value beyond the fp16 range became infinite in the fp16 tile, so
    // every accumulator it met is infinite or NaN; the flag is read after the
    // barrier below.
    float chk = 0.f;   // NaN iff some accumulator entry is not finite
#pragma unroll
    for (int cg = 0; cg < NCG; ++cg)
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 4; ++r) chk = fmaf(acc[cg][db][r], 0.f, chk);
    if (__builtin_amdgcn_ballot_w64(chk != chk) != 0 && lane == 0) s_big = 1;
  }
  __syncthreads();
  if (!FP8 && s_big) {
    // Rare: the whole unit again with P V in bf16 (for V that is itself not
    // finite this gives the result the first pass would have).
#pragma unroll
    for (int cg = 0; cg < NCG; ++cg) {
#pragma unroll
      for (int db = 0; db < DB; ++db) acc[cg][db] = f32x4{0.f, 0.f, 0.f, 0.f};
      m_run[cg] = NEG_INF;
      l_run[cg] = 0.f;
    }
    run_tiles(std::false_type{});
  }

  // merge the four waves, one column group at a time: lanes of one column share
  // m_run; l sums over the 4 row groups
  float* o_s = (float*)smem;                       // [4][16][OP]
  float* m_s = o_s + 4 * 16 * OP;                  // [4][16]
  float* l_s = m_s + 4 * 16;                       // [4][16]
  // (the tiles' LDS is free: the barrier after the check above, or the last one
  // of the recomputation, follows every read of it)
#pragma unroll
  for (int cg = 0; cg < NCG; ++cg) {
    float lr = l_run[cg];
    lr += __shfl_xor(lr, 16);
    lr = xhalf_sum(lr);
#pragma unroll
    for (int db = 0; db < DB; ++db) *(f32x4*)&o_s[(w * 16 + l16) * OP + 16 * db + 4 * g16] = acc[cg][db];
    if (g16 == 0) {
      m_s[w * 16 + l16] = m_run[cg];
      l_s[w * 16 + l16] = lr;
    }
    __syncthreads();

    const int c0 = (cu * NCG + cg) * 16;
    const int ncol = min(16, cols - c0);
    for (int e = tid; e < ncol * D; e += T::NT) {
      const int q = e / D, d = e % D;
      float M = NEG_INF;
#pragma unroll
      for (int ww = 0; ww < 4; ++ww) M = fmaxf(M, m_s[ww * 16 + q]);
      float Lsum = 0.f, O = 0.f;
#pragma unroll
      for (int ww = 0; ww < 4; ++ww) {
        const float mw = m_s[ww * 16 + q];
        const float wt = (mw == NEG_INF) ? 0.f : fast_exp2(mw - M);
        Lsum += wt * l_s[ww * 16 + q];
        O += wt * o_s[(ww * 16 + q) * OP + d];
      }
      const float inv = Lsum > 0.f ? (FP8 ? a.v_scale : 1.f) / Lsum : 0.f;
      const float lse = Lsum > 0.f ? (M + __log2f(Lsum)) * kLn2 : NEG_INF;
      const int c = c0 + q;
      const int t = c / a.group;
      const int h = g * a.group + c % a.group;
      const int64_t row = ((int64_t)b * a.q_len + t) * a.hq + h;     // [B, q_len, Hq]
      if (a.splits == 1) {
        a.o[row * D + d] = (__bf16)(O * inv);
        if (d == 0) a.lse[row] = lse;
      } else if (a.counters) {
        // single launch: device-scope stores, written through to memory, so that
        // another XCD's device-scope loads see them without an L2 write-back here
        const int64_t pi = (int64_t)s * a.batch * a.q_len * a.hq + row;
        __hip_atomic_store(a.o_part + pi * D + d, O * inv, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (d == 0) __hip_atomic_store(a.lse_part + pi, lse, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      } else {   // merged by decode_combine_kernel after this launch
        const int64_t pi = (int64_t)s * a.batch * a.q_len * a.hq + row;
        a.o_part[pi * D + d] = O * inv;
        if (d == 0) a.lse_part[pi] = lse;
      }
    }
    if (cg + 1 < NCG) __syncthreads();   // the merge buffers are rewritten by the next group
  }
  if (a.splits == 1 || a.counters == nullptr) return;

  // Arrival.  The XCDs' L2 caches are not coherent with one another, so the
  // partials were stored at device scope (through to memory) and are read back
  // at device scope below; every wave waits for its stores to complete before
  // the workgroup is counted.  (A device-scope fence would do the same by writing
  // back the whole L2 of the XCD, which cost 3x the decode's time.)  The counter
  // wraps to zero at the last arrival, so every call leaves it zero.
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);   // vmcnt = expcnt = lgkmcnt = 0: this wave's stores are done
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __syncthreads();
  if (tid == 0) {
    const int idx = (b * n_cu + cu) * a.hkv + g;
    const unsigned last = (unsigned)(a.splits - 1);
    s_last = atomicInc(a.counters + idx, last) == last;   // relaxed, device scope
  }
  __syncthreads();
  if (!s_last) return;

  // The unit's columns: weights exp(LSE_s - M) per (column, split) in LDS, then
  // O = sum_s w_s O_s / sum_s w_s, summed in split order as decode_combine does.
  const int c_beg = cu * NCG * 16;
  const int ncol = min(16 * NCG, cols - c_beg);
  const int64_t plane = (int64_t)a.batch * a.q_len * a.hq;
  float* w_s = (float*)smem;                               // [16 * NCG][kMaxDecodeSplits]
  float* mw_s = w_s + 16 * NCG * kMaxDecodeSplits;         // [16 * NCG]: M, then sum of weights
  float* sw_s = mw_s + 16 * NCG;
  static_assert((16 * NCG * kMaxDecodeSplits + 2 * 16 * NCG) * 4 <= SMEM, "combine weights fit");
  auto row_of = [&](int c) {
    const int t = c / a.group, h = g * a.group + c % a.group;
    return ((int64_t)b * a.q_len + t) * a.hq + h;
  };
  for (int i = tid; i < ncol * a.splits; i += T::NT) {
    const int c = i / a.splits, sp = i % a.splits;
    w_s[c * kMaxDecodeSplits + sp] =
        __hip_atomic_load(a.lse_part + sp * plane + row_of(c_beg + c), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  if (tid < ncol) {
    float* wc = w_s + tid * kMaxDecodeSplits;
    float M = NEG_INF;
    for (int sp = 0; sp < a.splits; ++sp) M = fmaxf(M, wc[sp]);
    float wsum = 0.f;
    for (int sp = 0; sp < a.splits; ++sp) {
      const float wt = (M == NEG_INF || wc[sp] == NEG_INF) ? 0.f : __expf(wc[sp] - M);
      wc[sp] = wt;
      wsum += wt;
    }
    mw_s[tid] = M;
    sw_s[tid] = wsum;
  }
  __syncthreads();
  const int64_t stride = plane * D;
  for (int e = tid; e < ncol * D; e += T::NT) {
    const int c = e / D, d = e % D;
    const int64_t row = row_of(c_beg + c);
    const float* op = a.o_part + row * D + d;
    const float* wc = w_s + c * kMaxDecodeSplits;
    float O = 0.f;
    int sp = 0;
    for (; sp + 8 <= a.splits; sp += 8) {   // eight loads in flight, then the sums in split order
      float x[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) x[u] = __hip_atomic_load(op + (sp + u) * stride, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
      for (int u = 0; u < 8; ++u) O = fmaf(wc[sp + u], x[u], O);
    }
    for (; sp < a.splits; ++sp)
      O = fmaf(wc[sp], __hip_atomic_load(op + sp * stride, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT), O);
    const float wsum = sw_s[c];
    a.o[row * D + d] = (__bf16)(wsum > 0.f ? O / wsum : 0.f);
    if (d == 0) a.lse[row] = wsum > 0.f ? mw_s[c] + __logf(wsum) : NEG_INF;
  }
}

// LSE-weighted merge of the split partials: LSE = log sum_s exp(LSE_s),
// O = sum_s exp(LSE_s - LSE) O_s.  Splits with LSE_s = -inf (no keys) weigh 0.
// One block per (b, token, h) row: the split LSEs are read in parallel into LDS,
// then every thread (one d each) sums its column with the partial loads unrolled,
// so a row costs a few memory round trips instead of two per split.
template <int D>
__global__ __launch_bounds__(D) void decode_combine_kernel(DecodeArgs a) {
  __shared__ float w_s[kMaxDecodeSplits];
  const int bh = blockIdx.x;            // (b * q_len + t) * hq + h
  const int d = threadIdx.x;
  const int64_t plane = (int64_t)a.batch * a.q_len * a.hq;
  const float NEG_INF = -__builtin_inff();
  const int splits = a.splits;
  for (int s = d; s < splits; s += D) w_s[s] = a.lse_part[s * plane + bh];
  __syncthreads();
  float M = NEG_INF;
  for (int s = 0; s < splits; ++s) M = fmaxf(M, w_s[s]);
  float wsum = 0.f, O = 0.f;
  if (M != NEG_INF) {
    const float* op = a.o_part + (int64_t)bh * D + d;
    const int64_t stride = plane * D;
#pragma unroll 4
    for (int s = 0; s < splits; ++s) {
      const float ls = w_s[s];
      const float wt = ls == NEG_INF ? 0.f : __expf(ls - M);
      wsum += wt;
      O = fmaf(wt, op[s * stride], O);
    }
  }
  a.o[(int64_t)bh * D + d] = (__bf16)(wsum > 0.f ? O / wsum : 0.f);
  if (d == 0) a.lse[bh] = wsum > 0.f ? M + __logf(wsum) : NEG_INF;
}

int decode_chunk_align() { return DecTile<128>::BN; }

// Two 16-column groups at most: four would spill at d = 128 with two waves per
// SIMD; wider query tiles use more column units (the KV chunk is then read once
// per unit).  Above d = 128 a workgroup holds one column group.
int decode_col_groups(int columns, int head_dim) { return (columns <= 16 || head_dim > 128) ? 1 : 2; }
int decode_blocks_per_cu(int columns, int head_dim) {
  if (head_dim > 128) return DecOcc<256, 1>::WG_PER_CU;
  return decode_col_groups(columns, head_dim) == 1 ? DecOcc<128, 1>::WG_PER_CU : DecOcc<128, 2>::WG_PER_CU;
}

template <int D, bool FP8>
static void launch_decode_d(const DecodeArgs& a, int ncg, unsigned grid, hipStream_t stream) {
  if constexpr (D > 128) {
    hipLaunchKernelGGL((decode_kernel<D, 1, FP8>), dim3(grid), dim3(256), 0, stream, a);
  } else {
    if (ncg == 1)
      hipLaunchKernelGGL((decode_kernel<D, 1, FP8>), dim3(grid), dim3(256), 0, stream, a);
    else
      hipLaunchKernelGGL((decode_kernel<D, 2, FP8>), dim3(grid), dim3(256), 0, stream, a);
  }
}
template <int D>
static void launch_decode_d(const DecodeArgs& a, int ncg, unsigned grid, hipStream_t stream) {
  if (a.kv_fp8) launch_decode_d<D, true>(a, ncg, grid, stream);
  else launch_decode_d<D, false>(a, ncg, grid, stream);
}

hipError_t launch_decode(const DecodeArgs& a, int head_dim, hipStream_t stream) {
  const int cols = a.group * a.q_len;
  const int ncg = decode_col_groups(cols, head_dim);
  const int n_cu = ((cols + 15) / 16 + ncg - 1) / ncg;
  const int64_t grid = (int64_t)a.batch * a.hkv * a.splits * n_cu;
  if (grid <= 0 || grid > (1ll << 31) - 1) return hipErrorInvalidValue;
  switch (head_dim) {
    case 64: launch_decode_d<64>(a, ncg, (unsigned)grid, stream); break;
    case 96: launch_decode_d<96>(a, ncg, (unsigned)grid, stream); break;
    case 128: launch_decode_d<128>(a, ncg, (unsigned)grid, stream); break;
    case 192: launch_decode_d<192>(a, ncg, (unsigned)grid, stream); break;
    case 256: launch_decode_d<256>(a, ncg, (unsigned)grid, stream); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_decode_combine(const DecodeArgs& a, int head_dim, hipStream_t stream) {
  const int64_t grid = (int64_t)a.batch * a.q_len * a.hq;
  switch (head_dim) {
    case 64: hipLaunchKernelGGL(decode_combine_kernel<64>, dim3((unsigned)grid), dim3(64), 0, stream, a); break;
    case 96: hipLaunchKernelGGL(decode_combine_kernel<96>, dim3((unsigned)grid), dim3(96), 0, stream, a); break;
    case 128: hipLaunchKernelGGL(decode_combine_kernel<128>, dim3((unsigned)grid), dim3(128), 0, stream, a); break;
    case 192: hipLaunchKernelGGL(decode_combine_kernel<192>, dim3((unsigned)grid), dim3(192), 0, stream, a); break;
    case 256: hipLaunchKernelGGL(decode_combine_kernel<256>, dim3((unsigned)grid), dim3(256), 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace jfa
