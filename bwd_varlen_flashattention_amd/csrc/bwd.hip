// Jagged FlashAttention backward for gfx950.
//
// What is computed ("Cutting edge isn't plug-and-play: customising
// FlashAttention-4 on B300", Phase 2 chunked-backward pseudocode and its buffer
// list, restated without the head-dim chunking because d <= 128 fits on chip):
//   P = exp(S - LSE) rebuilt from the forward's saved LSE, S = Q K^T * scale,
//   delta = rowsum(dO * O), dP = dO V^T, dS = P * (dP - delta),
//   dV = P^T dO, dK = scale dS^T Q, dQ = scale dS K.
// Broadcast-Q ("Optimizing Jagged Flash Attention with TLX", third paragraph):
// every item adds its dQ into the one shared dQ.
//
// Kernels:
//   bwd_pre_kernel   delta (fp32, laid out like LSE) and a zeroed fp32 dQ accumulator
//   bwd_kernel       persistent, key-stationary: a workgroup owns 128 keys of one
//                    KV head, keeps K/V fragments in VGPRs and the dK/dV
//                    accumulators in AGPR/VGPRs across all query tiles and all
//                    query heads of the GQA group, and streams 64-row Q/dO tiles
//                    through double-buffered LDS.  dQ partials (dS K) are
//                    atomically added in fp32 to the accumulator.
//   dq_convert       dQ = scale * accumulator -> bf16
//
// The K tile stays in LDS for the whole item: K is consumed twice per query
// tile, by S = Q K^T and again by dQ = dS K after dS exists, so no stage that
// holds K is refilled before its last reader (the single-stage K-buffer hazard
// described in the bug-hunting section of the B300 page).
#include "jfa_internal.h"
#include "device_common.h"

namespace jfa {

// ----------------------------------------------------------------------------- preprocess
constexpr int kPreThreads = 256;

__global__ __launch_bounds__(kPreThreads) void bwd_pre_kernel(BwdPreArgs a) {
  // 16 lanes per (row, head) pair; each lane reads 8 bf16 of O and dO.
  const int64_t gtid = (int64_t)blockIdx.x * kPreThreads + threadIdx.x;
  const int lane16 = threadIdx.x & 15;
  const int64_t pair = gtid >> 4;
  const int64_t n_pairs = a.rows * a.hq;
  const int chunks = a.head_dim / 8;
  float acc = 0.f;
  if (pair < n_pairs && lane16 < chunks) {
    const int64_t base = pair * a.head_dim + lane16 * 8;
    const bf16x8 o = *(const bf16x8*)(a.o + base);
    const bf16x8 d = *(const bf16x8*)(a.dout + base);
#pragma unroll
    for (int i = 0; i < 8; ++i) acc = fmaf((float)o[i], (float)d[i], acc);
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
  // zero the dQ accumulator (grid-stride over float4)
  const int64_t n4 = a.dq_elems / 4;
  const int64_t stride = (int64_t)gridDim.x * kPreThreads;
  for (int64_t i = gtid; i < n4; i += stride) ((f32x4*)a.dq_acc)[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int64_t i = n4 * 4 + gtid; i < a.dq_elems; i += stride) a.dq_acc[i] = 0.f;
}

hipError_t launch_bwd_pre(const BwdPreArgs& a, hipStream_t stream) {
  const int64_t threads = a.rows * a.hq * 16;
  int64_t blocks = (threads + kPreThreads - 1) / kPreThreads;
  if (blocks < 1024) blocks = 1024;                 // enough waves for the zero fill
  if (blocks > (1 << 30)) return hipErrorInvalidValue;
  hipLaunchKernelGGL(bwd_pre_kernel, dim3((unsigned)blocks), dim3(kPreThreads), 0, stream, a);
  return hipGetLastError();
}

// ----------------------------------------------------------------------------- dQ convert
__global__ __launch_bounds__(256) void dq_convert_kernel(DqConvertArgs a) {
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i + 3 < a.n) {
    const f32x4 x = *(const f32x4*)(a.dq_acc + i);
    bf16x4 y;
#pragma unroll
    for (int e = 0; e < 4; ++e) y[e] = (__bf16)(x[e] * a.scale);
    *(bf16x4*)(a.dq + i) = y;
  } else {
    for (int64_t j = i; j < a.n; ++j) a.dq[j] = (__bf16)(a.dq_acc[j] * a.scale);
  }
}

hipError_t launch_dq_convert(const DqConvertArgs& a, hipStream_t stream) {
  if (a.n <= 0) return hipSuccess;
  const int64_t blocks = (a.n + 1023) / 1024;
  hipLaunchKernelGGL(dq_convert_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, a);
  return hipGetLastError();
}

// ----------------------------------------------------------------------------- main kernel
template <int D>
struct BwdTile {
  static constexpr int NT = 256;           // 4 waves, 32 keys each
  static constexpr int BN = 128;           // keys per item
  static constexpr int BM = 64;            // query rows per inner step
  static constexpr int P = D + 16;         // LDS row pitch of Q, dO and K (elements)
  static constexpr int SP = BM + 16;       // LDS row pitch of the dS^T tile
  static constexpr int CH = D / 8;
  static constexpr int QLOADS = BM * CH / NT;
  static constexpr int KLOADS = BN * CH / NT;
  static constexpr int KS = D / 16;
  static constexpr int DB = D / 32;
  static constexpr int DQB = (2 * DB + 3) / 4;   // dQ output blocks per wave
  static_assert(BM * CH % NT == 0 && BN * CH % NT == 0, "tile load split");
};

template <int D, bool CAUSAL, bool BCAST>
__global__ __launch_bounds__(256) void bwd_kernel(BwdArgs a) {
  using T = BwdTile<D>;
  constexpr int BN = T::BN, BM = T::BM, P = T::P, SP = T::SP, KS = T::KS, DB = T::DB;
  __shared__ __attribute__((aligned(16))) __bf16 k_lds[BN * P];
  __shared__ __attribute__((aligned(16))) __bf16 q_lds[2][BM * P];
  __shared__ __attribute__((aligned(16))) __bf16 do_lds[2][BM * P];
  __shared__ __attribute__((aligned(16))) __bf16 dst_lds[BN * SP];
  __shared__ __attribute__((aligned(16))) float lse_lds[2][BM];
  __shared__ __attribute__((aligned(16))) float dlt_lds[2][BM];
  __shared__ int s_item;

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, hh = lane >> 5;
  const int g16 = lane >> 4, i16 = lane & 15;
  const int n_items = *a.n_entries * a.hkv;
  const float INF = __builtin_inff();

  for (;;) {
    if (tid == 0) s_item = (int)atomicAdd(a.counter, 1u);
    __syncthreads();
    const int item = s_item;
    if (item >= n_items) break;
    const WorkEntry e = a.entries[item / a.hkv];
    const int g = item % a.hkv;
    const int b = e.b;
    int lq, q_base;
    if (BCAST) { lq = a.bcast_nq; q_base = 0; }
    else { q_base = a.cu_q[b]; lq = a.cu_q[b + 1] - q_base; }
    const int k_base = a.cu_k[b];
    const int lk = a.cu_k[b + 1] - k_base;
    const int off = lk - lq;
    const int kt0 = e.t * BN;
    const int my_key = kt0 + 32 * w + l32;
    const bool key_ok = my_key < lk;

    int i_first = 0;
    if (CAUSAL) i_first = max(0, kt0 - off) / BM;
    const int ntq = cdiv(lq, BM);
    const int n_qt = (CAUSAL && max(0, kt0 - off) >= lq) ? 0 : ntq - i_first;
    const int n_steps = n_qt * a.group;

    // K/V fragments for this wave's 32 keys: B operands of S = Q K^T and dP = dO V^T
    bf16x8 kf[KS], vf[KS];
    {
      const int64_t base = ((int64_t)(k_base + min(my_key, lk - 1)) * a.hkv + g) * D + 8 * hh;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        kf[ks] = key_ok ? *(const bf16x8*)(a.k + base + 16 * ks) : zero_bf16x8();
        vf[ks] = key_ok ? *(const bf16x8*)(a.v + base + 16 * ks) : zero_bf16x8();
      }
    }
    f32x16 dkT[DB], dvT[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) { dkT[db] = f32x16{}; dvT[db] = f32x16{}; }

    if (n_steps > 0) {
      // stage the K tile (row-major, zero past the end) for the dQ contraction
#pragma unroll
      for (int i = 0; i < T::KLOADS; ++i) {
        const int id = tid + i * T::NT;
        const int r = id / T::CH, c = id % T::CH;
        u32x4 v = {0u, 0u, 0u, 0u};
        if (kt0 + r < lk) v = *(const u32x4*)(a.k + ((int64_t)(k_base + kt0 + r) * a.hkv + g) * D + c * 8);
        *(u32x4*)&k_lds[r * P + c * 8] = v;
      }
    }

    // step s -> (query head, query tile)
    u32x4 qr[T::QLOADS], dr[T::QLOADS];
    float lse_r = 0.f, dlt_r = 0.f;
    auto load_regs = [&](int s) {
      const int h = g * a.group + s / n_qt;
      const int qt = i_first + s % n_qt;
#pragma unroll
      for (int i = 0; i < T::QLOADS; ++i) {
        const int id = tid + i * T::NT;
        const int r = id / T::CH, c = id % T::CH;
        const int row = qt * BM + r;
        u32x4 qv = {0u, 0u, 0u, 0u}, dv = {0u, 0u, 0u, 0u};
        if (row < lq) {
          qv = *(const u32x4*)(a.q + ((int64_t)(q_base + row) * a.hq + h) * D + c * 8);
          const int64_t orow = BCAST ? (int64_t)b * lq + row : (int64_t)(q_base + row);
          dv = *(const u32x4*)(a.dout + (orow * a.hq + h) * D + c * 8);
        }
        qr[i] = qv;
        dr[i] = dv;
      }
      if (tid < BM) {
        const int row = qt * BM + tid;
        if (row < lq) {
          const int64_t li = BCAST ? ((int64_t)b * a.hq + h) * lq + row : (int64_t)h * a.total_q + q_base + row;
          const float l = a.lse[li];
          lse_r = (l == -INF) ? INF : l * kLog2e;   // rows that saw no key get P = 0
          dlt_r = a.delta[li];
        } else {
          lse_r = INF;
          dlt_r = 0.f;
        }
      }
    };
    auto store_lds = [&](int buf) {
#pragma unroll
      for (int i = 0; i < T::QLOADS; ++i) {
        const int id = tid + i * T::NT;
        const int r = id / T::CH, c = id % T::CH;
        *(u32x4*)&q_lds[buf][r * P + c * 8] = qr[i];
        *(u32x4*)&do_lds[buf][r * P + c * 8] = dr[i];
      }
      if (tid < BM) { lse_lds[buf][tid] = lse_r; dlt_lds[buf][tid] = dlt_r; }
    };

    if (n_steps > 0) {
      load_regs(0);
      store_lds(0);
      __syncthreads();
    }

    for (int s = 0; s < n_steps; ++s) {
      const int buf = s & 1;
      const int h = g * a.group + s / n_qt;
      const int qt = i_first + s % n_qt;
      if (s + 1 < n_steps) load_regs(s + 1);
      const __bf16* qt_lds = q_lds[buf];
      const __bf16* dot_lds = do_lds[buf];

      // S[q][key] and dP[q][key] for two 32-row query blocks
      f32x16 sacc[2], pacc[2];
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        sacc[qb] = f32x16{};
        pacc[qb] = f32x16{};
        const __bf16* qp = qt_lds + (32 * qb + l32) * P + 8 * hh;
        const __bf16* dp = dot_lds + (32 * qb + l32) * P + 8 * hh;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          sacc[qb] = mfma32x32x16(*(const bf16x8*)(qp + 16 * ks), kf[ks], sacc[qb]);
          pacc[qb] = mfma32x32x16(*(const bf16x8*)(dp + 16 * ks), vf[ks], pacc[qb]);
        }
      }

      // P = exp2(S*c - LSE*log2e), masked; dS = P * (dP - delta)
      bf16x8 pb[2][2], sb[2][2];
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        float pv[16], dsv[16];
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const int q0 = 32 * qb + 8 * r4 + 4 * hh;
          const f32x4 l4 = *(const f32x4*)&lse_lds[buf][q0];
          const f32x4 d4 = *(const f32x4*)&dlt_lds[buf][q0];
#pragma unroll
          for (int x = 0; x < 4; ++x) {
            const int r = 4 * r4 + x;
            bool ok = key_ok;
            if (CAUSAL) ok = ok && (my_key <= qt * BM + q0 + x + off);
            const float p = ok ? fast_exp2(fmaf(sacc[qb][r], a.scale_log2, -l4[x])) : 0.f;
            pv[r] = p;
            dsv[r] = p * (pacc[qb][r] - d4[x]);
          }
        }
        pb[qb][0] = to_bf16x8(pv);
        pb[qb][1] = to_bf16x8(pv + 8);
        sb[qb][0] = to_bf16x8(dsv);
        sb[qb][1] = to_bf16x8(dsv + 8);
      }

      // dV^T[d][key] += dO^T P ; dK^T[d][key] += Q^T dS   (A operands: transposed LDS reads)
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const int c0 = 32 * db + 16 * (g16 & 1) + 4 * (i16 & 3);
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            const int r0 = 32 * qb + 16 * t + 4 * (g16 >> 1) + (i16 >> 2);
            const __bf16* dp = dot_lds + r0 * P + c0;
            const __bf16* qp = qt_lds + r0 * P + c0;
            const bf16x8 doT = cat8(lds_read_tr4(dp), lds_read_tr4(dp + 8 * P));
            const bf16x8 qT = cat8(lds_read_tr4(qp), lds_read_tr4(qp + 8 * P));
            dvT[db] = mfma32x32x16(doT, pb[qb][t], dvT[db]);
            dkT[db] = mfma32x32x16(qT, sb[qb][t], dkT[db]);
          }
      }

      // dS^T[key][q] -> LDS (4 consecutive queries per 8-byte write)
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          bf16x4 v4;
#pragma unroll
          for (int x = 0; x < 4; ++x) v4[x] = sb[qb][r4 >> 1][4 * (r4 & 1) + x];
          *(bf16x4*)&dst_lds[(32 * w + l32) * SP + 32 * qb + 8 * r4 + 4 * hh] = v4;
        }
      __syncthreads();

      // dQ[q][d] = dS[q][key] K[key][d] over all 128 keys; this wave takes output blocks w, w+4, ...
#pragma unroll
      for (int bi = 0; bi < T::DQB; ++bi) {
        const int blk = w + 4 * bi;
        if (blk < 2 * DB) {
          const int qb = blk / DB, db = blk % DB;
          f32x16 dq = f32x16{};
          const __bf16* sp = dst_lds + (4 * (g16 >> 1) + (i16 >> 2)) * SP + 32 * qb + 16 * (g16 & 1) + 4 * (i16 & 3);
          const __bf16* kp = k_lds + (4 * (g16 >> 1) + (i16 >> 2)) * P + 32 * db + 16 * (g16 & 1) + 4 * (i16 & 3);
#pragma unroll
          for (int ks = 0; ks < BN / 16; ++ks) {
            const bf16x8 sa = cat8(lds_read_tr4(sp + 16 * ks * SP), lds_read_tr4(sp + (16 * ks + 8) * SP));
            const bf16x8 kb = cat8(lds_read_tr4(kp + 16 * ks * P), lds_read_tr4(kp + (16 * ks + 8) * P));
            dq = mfma32x32x16(sa, kb, dq);
          }
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int row = qt * BM + 32 * qb + 8 * (r >> 2) + 4 * hh + (r & 3);
            if (row < lq)
              unsafeAtomicAdd(a.dq_acc + ((int64_t)(q_base + row) * a.hq + h) * D + 32 * db + l32, dq[r]);
          }
        }
      }

      if (s + 1 < n_steps) store_lds(buf ^ 1);
      __syncthreads();
    }

    // epilogue: dK = scale * dK^T, dV = dV^T, 4 consecutive d per 8-byte store
    if (key_ok) {
      const int64_t base = ((int64_t)(k_base + my_key) * a.hkv + g) * D;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          bf16x4 kv4, vv4;
#pragma unroll
          for (int x = 0; x < 4; ++x) {
            kv4[x] = (__bf16)(dkT[db][4 * r4 + x] * a.scale);
            vv4[x] = (__bf16)(dvT[db][4 * r4 + x]);
          }
          const int d0 = 32 * db + 8 * r4 + 4 * hh;
          *(bf16x4*)(a.dk + base + d0) = kv4;
          *(bf16x4*)(a.dv + base + d0) = vv4;
        }
    }
    __syncthreads();   // s_item and LDS reuse
  }
}

int bwd_block_rows() { return BwdTile<128>::BM; }
int bwd_kv_tile() { return BwdTile<128>::BN; }
int bwd_blocks_per_cu(int) { return 1; }

template <int D>
static hipError_t launch_bwd_d(const BwdArgs& a, int grid, hipStream_t stream) {
  const dim3 g(grid), blk(BwdTile<D>::NT);
  if (a.bcast_nq > 0)
    hipLaunchKernelGGL((bwd_kernel<D, false, true>), g, blk, 0, stream, a);
  else if (a.causal)
    hipLaunchKernelGGL((bwd_kernel<D, true, false>), g, blk, 0, stream, a);
  else
    hipLaunchKernelGGL((bwd_kernel<D, false, false>), g, blk, 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_bwd(const BwdArgs& a, int head_dim, int grid, hipStream_t stream) {
  switch (head_dim) {
    case 64: return launch_bwd_d<64>(a, grid, stream);
    case 96: return launch_bwd_d<96>(a, grid, stream);
    case 128: return launch_bwd_d<128>(a, grid, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace jfa
