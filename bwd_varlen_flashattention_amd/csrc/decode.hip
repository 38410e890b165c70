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
//   O^T[d][q]   += V^T P^T    v_mfma_f32_16x16x16_bf16, A = V through the
//                             transposed LDS read, B = P^T straight from the
//                             S^T accumulator
// The four waves' (max, sum, accumulator) states are merged through LDS at the
// end.  With one split the result is final (bf16 O, LSE); otherwise each split
// leaves its normalised fp32 partial and its LSE, and decode_combine merges the
// partials with weights exp(LSE_s - LSE).
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

typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16x16x16(bf16x4 a, bf16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a), __builtin_bit_cast(s16x4, b), c, 0, 0, 0);
}

template <int D>
__global__ __launch_bounds__(256, 4) void decode_kernel(DecodeArgs a) {
  using T = DecTile<D>;
  constexpr int BN = T::BN, KP = T::KP, VP = T::VP, KK = T::KK, DB = T::DB;
  constexpr int KV_BYTES = BN * (KP + VP) * 2;
  constexpr int MERGE_BYTES = 4 * 16 * D * 4 + 2 * 4 * 16 * 4;
  constexpr int SMEM = KV_BYTES > MERGE_BYTES ? KV_BYTES : MERGE_BYTES;
  __shared__ __attribute__((aligned(16))) unsigned char smem[SMEM];
  __bf16* k_lds = (__bf16*)smem;
  __bf16* v_lds = k_lds + BN * KP;

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int l16 = lane & 15, g16 = lane >> 4;
  const float NEG_INF = -__builtin_inff();

  // unit = (b, s, g) with g fastest: the KV heads of one chunk are neighbouring
  // workgroups, dispatched together, so the token rows they share are read from
  // DRAM at about the same time
  const int unit = blockIdx.x;
  const int g = unit % a.hkv;
  const int bs = unit / a.hkv;
  const int s = bs % a.splits;
  const int b = bs / a.splits;
  const int L = a.seqlens[b];
  const int chunk = cdiv(cdiv(L, a.splits), BN) * BN;
  const int k_lo = s * chunk;
  const int k_hi = min(L, k_lo + chunk);
  const int n_tiles = k_hi > k_lo ? cdiv(k_hi - k_lo, BN) : 0;

  // query fragment: column q = l16 is query head g*group + q (zero when q >= group)
  bf16x8 qf[KK];
  {
    const bool q_ok = l16 < a.group;
    const __bf16* qp = a.q + ((int64_t)b * a.hq + g * a.group + (q_ok ? l16 : 0)) * D + 8 * g16;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) qf[kk] = q_ok ? *(const bf16x8*)(qp + 32 * kk) : zero_bf16x8();
  }

  f32x4 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = NEG_INF, l_run = 0.f;

  const int32_t* pt = a.page_table + (int64_t)b * a.max_pages;
  u32x4 kr[T::LOADS], vr[T::LOADS];
  auto load_regs = [&](int j) {
#pragma unroll
    for (int i = 0; i < T::LOADS; ++i) {
      const int id = tid + i * T::NT;
      const int r = id / T::CH, c = id % T::CH;
      const int key = min(k_lo + j * BN + r, k_hi - 1);   // never past the sequence end
      const int page = pt[key / a.page_size];
      const int slot = key - (key / a.page_size) * a.page_size;
      const int64_t off = (((int64_t)page * a.page_size + slot) * a.hkv + g) * D + c * 8;
      kr[i] = *(const u32x4*)(a.k_cache + off);
      vr[i] = *(const u32x4*)(a.v_cache + off);
    }
  };
  auto store_lds = [&]() {
#pragma unroll
    for (int i = 0; i < T::LOADS; ++i) {
      const int id = tid + i * T::NT;
      const int r = id / T::CH, c = id % T::CH;
      *(u32x4*)&k_lds[r * KP + c * 8] = kr[i];
      *(u32x4*)&v_lds[r * VP + c * 8] = vr[i];
    }
  };

  if (n_tiles > 0) load_regs(0);
  for (int j = 0; j < n_tiles; ++j) {
    store_lds();
    __syncthreads();
    if (j + 1 < n_tiles) load_regs(j + 1);

    f32x4 st = f32x4{0.f, 0.f, 0.f, 0.f};
    const __bf16* kp = k_lds + (16 * w + l16) * KP + 8 * g16;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) st = mfma16x16x32(*(const bf16x8*)(kp + 32 * kk), qf[kk], st);

    float mx = NEG_INF;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int key = k_lo + j * BN + 16 * w + 4 * g16 + r;
      st[r] = key < k_hi ? st[r] : NEG_INF;
      mx = fmaxf(mx, st[r]);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = xhalf_max(mx);
    const float m_new = fmaxf(m_run, mx * a.scale_log2);
    const float alpha = (m_new == NEG_INF) ? 1.f : fast_exp2(m_run - m_new);
    const float m_sub = (m_new == NEG_INF) ? 0.f : m_new;
    bf16x4 pb;
    float psum = 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float p = fast_exp2(fmaf(st[r], a.scale_log2, -m_sub));
      psum += p;
      pb[r] = (__bf16)p;
    }
    l_run = l_run * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const __bf16* vp = v_lds + (16 * w + 4 * g16 + (l16 >> 2)) * VP + 16 * db + 4 * (l16 & 3);
      acc[db] = mfma16x16x16(lds_read_tr4(vp), pb, acc[db] * alpha);
    }
    __syncthreads();   // the tile buffer is refilled at the top of the next iteration
  }

  // merge the four waves: lanes of one query column share m_run; sum l over the 4 row groups
  l_run += __shfl_xor(l_run, 16);
  l_run = xhalf_sum(l_run);
  float* o_s = (float*)smem;                       // [4][16][D]
  float* m_s = o_s + 4 * 16 * D;                   // [4][16]
  float* l_s = m_s + 4 * 16;                       // [4][16]
  if (n_tiles > 0) __syncthreads();
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 4; ++r) o_s[(w * 16 + l16) * D + 16 * db + 4 * g16 + r] = acc[db][r];
  if (g16 == 0) {
    m_s[w * 16 + l16] = m_run;
    l_s[w * 16 + l16] = l_run;
  }
  __syncthreads();

  for (int e = tid; e < a.group * D; e += T::NT) {
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
      O += wt * o_s[(ww * 16 + q) * D + d];
    }
    const float inv = Lsum > 0.f ? 1.f / Lsum : 0.f;
    const float lse = Lsum > 0.f ? (M + __log2f(Lsum)) * kLn2 : NEG_INF;
    const int h = g * a.group + q;
    if (a.splits == 1) {
      a.o[((int64_t)b * a.hq + h) * D + d] = (__bf16)(O * inv);
      if (d == 0) a.lse[(int64_t)b * a.hq + h] = lse;
    } else {
      const int64_t pi = ((int64_t)s * a.batch + b) * a.hq + h;
      a.o_part[pi * D + d] = O * inv;
      if (d == 0) a.lse_part[pi] = lse;
    }
  }
}

// LSE-weighted merge of the split partials: LSE = log sum_s exp(LSE_s),
// O = sum_s exp(LSE_s - LSE) O_s.  Splits with LSE_s = -inf (no keys) weigh 0.
template <int D>
__global__ __launch_bounds__(D) void decode_combine_kernel(DecodeArgs a) {
  const int bh = blockIdx.x;            // b * hq + h
  const int d = threadIdx.x;
  const int64_t plane = (int64_t)a.batch * a.hq;
  const float NEG_INF = -__builtin_inff();
  float M = NEG_INF;
  for (int s = 0; s < a.splits; ++s) M = fmaxf(M, a.lse_part[s * plane + bh]);
  float wsum = 0.f, O = 0.f;
  if (M != NEG_INF) {
    for (int s = 0; s < a.splits; ++s) {
      const float ls = a.lse_part[s * plane + bh];
      const float wt = ls == NEG_INF ? 0.f : __expf(ls - M);
      wsum += wt;
      O += wt * a.o_part[(s * plane + bh) * D + d];
    }
  }
  a.o[(int64_t)bh * D + d] = (__bf16)(wsum > 0.f ? O / wsum : 0.f);
  if (d == 0) a.lse[bh] = wsum > 0.f ? M + __logf(wsum) : NEG_INF;
}

int decode_chunk_align() { return DecTile<128>::BN; }
int decode_blocks_per_cu() { return 4; }   // LDS and registers of the d = 128 kernel allow four

hipError_t launch_decode(const DecodeArgs& a, int head_dim, hipStream_t stream) {
  const int64_t grid = (int64_t)a.batch * a.hkv * a.splits;
  if (grid <= 0 || grid > (1ll << 31) - 1) return hipErrorInvalidValue;
  switch (head_dim) {
    case 64: hipLaunchKernelGGL(decode_kernel<64>, dim3((unsigned)grid), dim3(256), 0, stream, a); break;
    case 96: hipLaunchKernelGGL(decode_kernel<96>, dim3((unsigned)grid), dim3(256), 0, stream, a); break;
    case 128: hipLaunchKernelGGL(decode_kernel<128>, dim3((unsigned)grid), dim3(256), 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_decode_combine(const DecodeArgs& a, int head_dim, hipStream_t stream) {
  const int64_t grid = (int64_t)a.batch * a.hq;
  switch (head_dim) {
    case 64: hipLaunchKernelGGL(decode_combine_kernel<64>, dim3((unsigned)grid), dim3(64), 0, stream, a); break;
    case 96: hipLaunchKernelGGL(decode_combine_kernel<96>, dim3((unsigned)grid), dim3(96), 0, stream, a); break;
    case 128: hipLaunchKernelGGL(decode_combine_kernel<128>, dim3((unsigned)grid), dim3(128), 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace jfa
