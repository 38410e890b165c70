// Jagged FlashAttention forward for gfx950.
//
// What is computed: for each packed sequence (or broadcast-Q item) and query head,
// O = softmax(Q K^T * scale) V and the natural-log LSE of the scaled scores,
// tiled along the key axis with an online softmax so that neither padding nor the
// score matrix ever reaches memory ("Optimizing Jagged Flash Attention with TLX",
// third paragraph; the tiling recap of "Cutting edge isn't plug-and-play:
// customising FlashAttention-4 on B300").
//
// How it maps to CDNA4:
//   * persistent workgroups pull (sequence, query tile, head) items from the
//     per-XCD queues built by sched.hip, where the tiles sharing one K/V run
//     back to back on one XCD and so share its L2;
//   * waves of 32 query rows whose Q fragment stays in VGPRs for the whole key
//     loop; two waves per SIMD for d <= 128 (one 8-wave workgroup of 256 rows
//     per CU, or two 4-wave ones of 128 rows where the K tile does not split
//     over 512 threads), so one wave's softmax VALU work overlaps the other's
//     MFMAs; d = 192 and 256 run one 4-wave workgroup per CU, whose Q fragment
//     and accumulator fill a SIMD's registers;
//   * K/V tiles of 64 keys are staged through LDS while earlier tiles are
//     consumed: at d >= 128 in four stages, loaded two tiles ahead, with one
//     workgroup barrier per two tiles; otherwise double-buffered, one barrier
//     per tile;
//   * S^T = K Q^T on v_mfma_f32_32x32x16_bf16 so each lane owns one query column:
//     the row max/sum reductions are in-lane plus one permlane32 swap;
//   * the S^T accumulator, rounded to fp16, is directly the B operand of
//     O^T += V^T P^T on v_mfma_f32_32x32x16_f16 (the fp16 rate equals the bf16
//     one; P keeps 11 significant bits instead of 8, which keeps O within 1e-2
//     of exact attention where bf16 rounding of P alone can exceed what the
//     output's own bf16 rounding leaves of that budget).  V is converted to
//     fp16 (exact below 65520 in magnitude; an item whose V holds a larger
//     value is computed again with bf16 P V) and staged into LDS
//     already transposed (each thread transposes a 4-key x 8-column block in
//     registers with v_perm_b32), with the keys of every 16-key group stored in
//     the order the accumulator hands them out, so every MFMA operand is one
//     16-byte ds_read_b128 -- on gfx950 the transposed LDS read delivers about
//     a third of the b128 bandwidth;
//   * the key loop is split into a branch-free bulk and masked tail/diagonal tiles
//     (loop peeling, TLX page fifth paragraph);
//   * the running max is only moved (and the accumulator rescaled) when it grows
//     by more than 2^8, which keeps the result exact because the final
//     normalisation uses the same stale max.
#include <type_traits>

#include "jfa_internal.h"
#include "device_common.h"

namespace jfa {

// FP8: Q, K and V are OCP e4m3 bytes.  K stays e4m3 in LDS and S^T = K Q^T runs
// on v_mfma_f32_32x32x64_f8f6f4 (64-deep k-steps, twice the bf16 rate); V is
// widened to fp16 (exactly: every e4m3 value is an fp16 value) while it is
// staged transposed, so P V is the fp16 contraction of the bf16 path.
// NARROW: the 4-wave, 128-row workgroup (two per CU) at head dims that otherwise
// take the 8-wave one; chosen per call for problems of short sequences, where an
// item is a few tiles long and the latency of its loads, not its work, sets the
// time: two resident workgroups per CU keep two items in flight.
template <int D, bool FP8 = false, bool NARROW = false>
struct FwdTile {
  static constexpr int BN = D <= 192 ? 64 : 32;   // keys per KV tile (d = 256: 32, so nothing spills)
  static constexpr int KB = BN / 32;        // 32-key blocks per tile
  static constexpr int EB = FP8 ? 1 : 2;    // bytes per Q/K/V element in memory
  static constexpr int KP = FP8 ? D + 16 : D + 8;   // K row pitch in LDS (elements): +16 B staggers banks
  static constexpr int VTP = BN + 8;        // V^T row pitch (elements): 144 B rows at 64 keys
  static constexpr int CH = D * EB / 16;    // 16-byte chunks per K row
  // d <= 128: one workgroup of 8 waves per CU (2 per SIMD) owning 256 query
  // rows, so that every K/V tile brought into the CU serves 256 rows (the L2 ->
  // CU path, not the HBM, limits the staging); otherwise 4 waves, 128 rows.
  // d = 96 and e4m3 at d = 64 keep 4 waves: their K tile does not split evenly
  // over 512 threads.
  static constexpr int NT = (!NARROW && D <= 128 && (BN * CH) % 512 == 0) ? 512 : 256;
  static constexpr int BM = NT / 2;         // query rows per item (32 per wave)
  static constexpr int KLOADS = BN * CH / NT;
  static constexpr int VBLOCKS = (BN / 4) * (D / 8);   // 4-key x 8-column blocks of V
  static constexpr int VPER = (VBLOCKS + NT - 1) / NT;  // V blocks per thread (2 for d > 128)
  static constexpr int KS = D / 16;         // k-steps of K Q^T (bf16)
  static constexpr int KS8 = D / 64;        // k-steps of K Q^T (e4m3)
  static constexpr int DB = D / 32;         // 32-wide output column blocks
  static constexpr int K_LDS_BYTES = BN * KP * EB;
  // 4-wave workgroups at d <= 128: two per CU; larger heads need the whole
  // register file of one wave per SIMD (Q fragment + output accumulator)
  static constexpr int WG_PER_CU = (NT == 256 && D <= 128) ? 2 : 1;
  static_assert(BN * CH % NT == 0, "tile load split");
  static_assert(!FP8 || D % 64 == 0, "e4m3 k-steps are 64 deep");
  // epilogue: each wave's 32 x D output block goes through LDS
  static constexpr int NW = NT / 64;
  static constexpr int EP = D + 8;
  // K/V stages: four for d >= 128 where they and the epilogue blocks (then all
  // in the V^T stages) fit, with tiles loaded two steps ahead and a workgroup
  // barrier after every second tile (dense causal forward -2.6 % at d = 128, -6 %
  // at d = 256); two, with a barrier after every tile, otherwise (at d = 64 a
  // tile's work is short and four stages were 2 % slower)
  static constexpr int NST = (D >= 128 && WG_PER_CU * 4 * (K_LDS_BYTES + D * VTP * 2) <= 159 * 1024 &&
                              NW * 32 * EP <= 4 * D * VTP) ? 4 : 2;   // 1 KB left for the small shared state
  // With two stages the blocks go in the V^T stages, or half of them in the K
  // stages, except for e4m3 with 8 waves (a smaller K stage), which then has LDS
  // of its own (one workgroup per CU).
  static constexpr bool EP_ALL_VT = NW * 32 * EP <= NST * D * VTP;
  static constexpr bool EP_SPLIT = (NW / 2) * 32 * EP <= 2 * D * VTP && (NW / 2) * 32 * EP <= K_LDS_BYTES;
  static constexpr int EP_OWN = (!EP_ALL_VT && !EP_SPLIT && NT == 512) ? NW * 32 * EP : 1;
  static constexpr int AHEAD = NST / 2;     // steps between a tile's load and its use
  static_assert(WG_PER_CU * (NST * (K_LDS_BYTES + D * VTP * 2) + 2 * EP_OWN) <= 160 * 1024, "LDS budget");
};

typedef int i32x8 __attribute__((ext_vector_type(8)));

// e4m3 x e4m3 -> fp32, 32x32x64; zero scale operands select the unscaled form.
// A and B hold their 64 k-values per row in the same lane/slot order, so any
// consistent placement of the head dimension gives the dot products.
__device__ __forceinline__ f32x16 mfma32x32x64_fp8(i32x8 a, i32x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}


// Position of a 4-key quarter inside its stored 16-key group: the S^T accumulator
// gives lane half h the keys {4h..4h+3, 8+4h..8+4h+3} of each group as one
// 8-slot MFMA operand, so quarters are stored in the order 0, 2, 1, 3.
__device__ __forceinline__ int vt_quarter_pos(int q) { return ((q & 1) << 1) | (q >> 1); }

constexpr float kRescaleThreshold = 8.0f;   // log2 units

template <int D, bool CAUSAL, bool BCAST, bool FP8, bool NARROW>
__global__ __launch_bounds__((FwdTile<D, FP8, NARROW>::NT), (FwdTile<D, FP8, NARROW>::WG_PER_CU)) void fwd_kernel(FwdArgs a) {
  using T = FwdTile<D, FP8, NARROW>;
  constexpr int BM = T::BM, BN = T::BN, KB = T::KB, KP = T::KP, VTP = T::VTP, KS = T::KS, DB = T::DB;
  constexpr int EB = T::EB;
  __shared__ __attribute__((aligned(16))) unsigned char k_raw[T::NST][T::K_LDS_BYTES];
  __shared__ __attribute__((aligned(16))) __bf16 vt_lds[T::NST][D * VTP];
  __shared__ __attribute__((aligned(16))) __bf16 ep_lds[T::EP_OWN];
  __shared__ int s_item[2];   // claims alternate between the entries: a wave still
  // reading claim k's entry has not passed the barrier that follows claim k + 1, so
  // claim k + 2, the next write to that entry, cannot overtake the read even when
  // item k + 1 has no tiles (and so no barrier of its own)
  __shared__ int s_queue[2 * kQueues];
  // Number (counted from 1 over the workgroup's lifetime) of the last item whose
  // fp16 accumulation was not finite; 0 = none
  __shared__ int s_big_item;

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, hh = lane >> 5;
  const float NEG_INF = -__builtin_inff();

  // byte offsets of this thread's staging loads inside a KV tile (row stride rs elements)
  const int rs = a.hkv * D;
  const unsigned char* const qb8 = (const unsigned char*)a.q;
  const unsigned char* const kb8 = (const unsigned char*)a.k;
  const unsigned char* const vb8 = (const unsigned char*)a.v;
  constexpr int VPER = T::VPER;
  bool v_stager[VPER];
  int vkb[VPER], vdb[VPER];
  uint32_t koff[T::KLOADS], voff[VPER][4];
#pragma unroll
  for (int i = 0; i < T::KLOADS; ++i) {
    const int id = tid + i * T::NT;
    koff[i] = (uint32_t)((id / T::CH) * rs * EB + (id % T::CH) * 16);
  }
#pragma unroll
  for (int vi = 0; vi < VPER; ++vi) {
    const int id = tid + vi * T::NT;
    v_stager[vi] = id < T::VBLOCKS;
    vkb[vi] = id % (BN / 4);
    vdb[vi] = id / (BN / 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) voff[vi][i] = (uint32_t)(((4 * vkb[vi] + i) * rs + vdb[vi] * 8) * EB);
  }

  int home_q = blockIdx.x % kQueues, drained = 0;   // work-queue state (thread 0)
  load_queues(a.queues, s_queue);
  if (tid == 0) s_big_item = 0;
  __syncthreads();
  if (tid == 0) s_item[0] = next_work_item(a.queues, s_queue, home_q, drained);
  __syncthreads();
  int slot = 0;   // s_item entry of the current claim (uniform)
  int item_no = 0;   // items taken by this workgroup (uniform)
  int item = __builtin_amdgcn_readfirstlane(s_item[0]);   // uniform: the item loads are scalar
  while (item >= 0) {
    ++item_no;
    const WorkItem e = a.items[item];
    const int h = e.h;
    const int g = h / a.group;
    const int b = e.b;
    const int lq = e.lq, q_base = e.q_base;
    const int k_base = e.k_base, lk = e.lk;
    const int row0 = e.t * BM;
    const int my_row = row0 + w * 32 + l32;
    const bool row_ok = my_row < lq;
    const bool wave_rows = row0 + w * 32 < lq;   // uniform per wave
    const int off = lk - lq;                 // bottom-right causal alignment

    // Q fragment: B operand of S^T = K Q^T, lane holds row my_row, d-slots
    // 16*ks + 8*hh + 0..7 (bf16) or 64*ks + 32*hh + 0..31 (e4m3)
    using QFrag = std::conditional_t<FP8, i32x8, bf16x8>;
    constexpr int QSTEPS = FP8 ? T::KS8 : KS;
    QFrag qf[QSTEPS];
    {
      const int64_t qrow = ((int64_t)(q_base + my_row) * a.hq + h) * D;
#pragma unroll
      for (int ks = 0; ks < QSTEPS; ++ks) {
        if constexpr (FP8) qf[ks] = row_ok ? *(const i32x8*)(qb8 + qrow + 64 * ks + 32 * hh) : i32x8{};
        else qf[ks] = row_ok ? *(const bf16x8*)(a.q + qrow + 16 * ks + 8 * hh) : zero_bf16x8();
      }
    }

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

    f32x16 acc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[db] = f32x16{};
    float m_run = NEG_INF, l_run = 0.f;

    // staging: K row-major chunks; V as one 4-key x 8-column block per thread.
    // Raw buffer loads: the per-thread byte offsets are fixed (koff/voff), the
    // tile base and its valid byte range live in the 4-SGPR resource, and rows
    // past the sequence end fall outside the range and read as zero.
    const unsigned char* kbase = kb8 + ((int64_t)k_base * a.hkv + g) * D * EB;
    const unsigned char* vbase = vb8 + ((int64_t)k_base * a.hkv + g) * D * EB;
    using VReg = std::conditional_t<FP8, uint2, u32x4>;   // one 8-column row piece of V
    u32x4 kr[T::KLOADS];
    VReg vr[VPER][4];
    auto load_regs = [&](int j) {
      const int64_t tile_off = (int64_t)j * BN * rs * EB;
      const uint32_t nbytes = (uint32_t)(min(lk - j * BN, BN) * rs * EB);
      const auto krs = uniform_rsrc(kbase + tile_off, nbytes);
      const auto vrs = uniform_rsrc(vbase + tile_off, nbytes);
#pragma unroll
      for (int i = 0; i < T::KLOADS; ++i)
        kr[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(krs, koff[i], 0, 0));
#pragma unroll
      for (int vi = 0; vi < VPER; ++vi)
        if (v_stager[vi]) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            if constexpr (FP8) vr[vi][i] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(vrs, voff[vi][i], 0, 0));
            else vr[vi][i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(vrs, voff[vi][i], 0, 0));
          }
        }
    };
    // F16 (a std::bool_constant): V is written as fp16 (e4m3 always is; a bf16
    // value beyond the fp16 range becomes infinite, see the recomputation below),
    // otherwise as bf16.
    auto store_lds = [&](int buf, auto f16_tag) {
      constexpr bool F16 = decltype(f16_tag)::value;
#pragma unroll
      for (int i = 0; i < T::KLOADS; ++i) {
        const int id = tid + i * T::NT;
        const int r = id / T::CH, c = id % T::CH;
        *(u32x4*)&k_raw[buf][r * KP * EB + c * 16] = kr[i];
      }
#pragma unroll
      for (int vi = 0; vi < VPER; ++vi) {
        if (!v_stager[vi]) continue;
        // 4 keys x 8 columns -> 8 rows of V^T holding 4 keys each
        const int col = 16 * (vkb[vi] >> 2) + 4 * vt_quarter_pos(vkb[vi] & 3);
        __bf16* dst = &vt_lds[buf][(8 * vdb[vi]) * VTP + col];
        // Per column pair (2c, 2c + 1): rows 0-1 and 2-3 of column 2c (lo01, lo23) and of
        // column 2c + 1 (hi01, hi23), two 16-bit values per register
        uint32_t lo01[4], lo23[4], hi01[4], hi23[4];
        if constexpr (!FP8 && F16) {
          // bf16 -> fp16 with each packed conversion taking two rows of one column,
          // so its result is already the transposed pair (no permutes)
          auto lo = [](uint32_t x) { return __uint_as_float(x << 16); };
          auto hi = [](uint32_t x) { return __uint_as_float(x & 0xffff0000u); };
          auto pk = [](float a, float b) {   // a in the low half
            return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a, b}, f16x2));
          };
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const uint32_t x0 = vr[vi][0][c], x1 = vr[vi][1][c], x2 = vr[vi][2][c], x3 = vr[vi][3][c];
            lo01[c] = pk(lo(x0), lo(x1));
            lo23[c] = pk(lo(x2), lo(x3));
            hi01[c] = pk(hi(x0), hi(x1));
            hi23[c] = pk(hi(x2), hi(x3));
          }
        } else {
          u32x4 r[4];   // 4 rows of 8 16-bit values
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            if constexpr (FP8) r[i] = widen_e4m3x8_f16(vr[vi][i]);
            else r[i] = vr[vi][i];
          }
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            lo01[c] = __builtin_amdgcn_perm(r[1][c], r[0][c], 0x05040100u);
            lo23[c] = __builtin_amdgcn_perm(r[3][c], r[2][c], 0x05040100u);
            hi01[c] = __builtin_amdgcn_perm(r[1][c], r[0][c], 0x07060302u);
            hi23[c] = __builtin_amdgcn_perm(r[3][c], r[2][c], 0x07060302u);
          }
        }
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          *(uint2*)(dst + (2 * c) * VTP) = make_uint2(lo01[c], lo23[c]);
          *(uint2*)(dst + (2 * c + 1) * VTP) = make_uint2(hi01[c], hi23[c]);
        }
      }
    };

    // Key-tile order: bulk tiles first, masked tiles last, the same order for every
    // item sharing this K/V (they run together on one XCD and find the same K/V
    // tiles in its L2).
    auto tile_of = [&](int s) { return s; };

    // Step s visits key tile j = tile_of(s).  MASK selects the tail / causal-diagonal
    // variant; the bulk variant has no per-element masking at all (loop peeling).
    // F16 selects the P V precision (fp16, or bf16 for the recomputation of an
    // item whose V does not fit fp16).
    auto tile = [&](int step, auto mask_tag, auto f16_tag) {
      constexpr bool MASK = decltype(mask_tag)::value;
      constexpr bool F16 = decltype(f16_tag)::value;
      const int buf = step & (T::NST - 1);
      const int j = tile_of(step);
      const bool fill = step + T::AHEAD < n_tiles;   // this step stages tile step + AHEAD
      if (fill) load_regs(tile_of(step + T::AHEAD));
      // a wave whose 32 rows all lie past the sequence end only stages and syncs,
      // and so does one whose rows all lie before a causal diagonal tile's first key
      if (wave_rows && !(CAUSAL && MASK && j * BN > row0 + 32 * w + 31 + off)) {
      // S^T[key][query] for the tile's 32-key blocks
      f32x16 s[KB];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        s[kb] = f32x16{};
        if constexpr (FP8) {
          const unsigned char* kp = &k_raw[buf][(32 * kb + l32) * KP + 32 * hh];
#pragma unroll
          for (int ks = 0; ks < QSTEPS; ++ks)
            s[kb] = mfma32x32x64_fp8(*(const i32x8*)(kp + 64 * ks), qf[ks], s[kb]);
        } else {
          const __bf16* kp = (const __bf16*)k_raw[buf] + (32 * kb + l32) * KP + 8 * hh;
#pragma unroll
          for (int ks = 0; ks < KS; ++ks)
            s[kb] = mfma32x32x16(*(const bf16x8*)(kp + 16 * ks), qf[ks], s[kb]);
        }
      }

      if constexpr (MASK) {
        const int kmax_ok = CAUSAL ? min(lk - 1, my_row + off) : lk - 1;   // last visible key
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = j * BN + 32 * kb + 8 * (r >> 2) + 4 * hh + (r & 3);
            s[kb][r] = key <= kmax_ok ? s[kb][r] : NEG_INF;
          }
      }

      float mx = NEG_INF;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
      mx = xhalf_max(mx);
      const float m_new = fmaxf(m_run, mx * a.scale_log2);
      const bool need = m_new > m_run + kRescaleThreshold;
      if (__builtin_amdgcn_ballot_w64(need) != 0) {
        asm volatile("" ::: "memory");   // keep this a real branch: the rescale is rare
        const float alpha = (m_new == NEG_INF) ? 1.f : fast_exp2(m_run - m_new);
#pragma unroll
        for (int db = 0; db < DB; ++db) acc[db] *= alpha;
        l_run *= alpha;
        m_run = m_new;
      }
      const float m_sub = (m_run == NEG_INF) ? 0.f : m_run;

      float psum = 0.f;
      using PFrag = std::conditional_t<F16, f16x8, bf16x8>;
      PFrag pb[KB][2];   // P^T: B operands of O^T += V^T P^T
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        float pv[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          pv[r] = fast_exp2(fmaf(s[kb][r], a.scale_log2, -m_sub));
          psum += pv[r];
        }
        if constexpr (F16) {
          pb[kb][0] = to_f16x8(pv);
          pb[kb][1] = to_f16x8(pv + 8);
        } else {
          pb[kb][0] = to_bf16x8(pv);
          pb[kb][1] = to_bf16x8(pv + 8);
        }
      }
      l_run += psum;

      // O^T[d][query] += V^T[d][key] P^T[key][query]; one b128 read per operand
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const __bf16* vp = &vt_lds[buf][(32 * db + l32) * VTP + 8 * hh];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            if constexpr (F16)
              acc[db] = mfma32x32x16_f16(*(const f16x8*)(vp + 16 * (2 * kb + t)), pb[kb][t], acc[db]);
            else
              acc[db] = mfma32x32x16(*(const bf16x8*)(vp + 16 * (2 * kb + t)), pb[kb][t], acc[db]);
          }
      }
      }   // wave_rows

      debug_barrier();
      // With four stages a step stages tile step + 2 into the stage that step - 2
      // read, and reads the stage step - 2 filled: a barrier after every odd step
      // (and after the last) separates each such pair.
      if (fill) store_lds((step + T::AHEAD) & (T::NST - 1), f16_tag);
      if (T::NST == 2 || (step & 1) || step + 1 == n_tiles) __syncthreads();
    };

    // The loops are only reachable through the prologue, whose wait covers the
    // Q-fragment loads; otherwise every tile would wait on all outstanding loads.
    auto key_loop = [&](auto f16_tag) {
      load_regs(tile_of(0));
      store_lds(0, f16_tag);
      if (T::NST == 4 && n_tiles > 1) {
        load_regs(tile_of(1));
        store_lds(1, f16_tag);
      }
      __syncthreads();
      for (int s = 0; s < n_bulk; ++s) tile(s, std::false_type{}, f16_tag);
      for (int s = n_bulk; s < n_tiles; ++s) tile(s, std::true_type{}, f16_tag);
    };
    if (n_tiles > 0) {
      key_loop(std::true_type{});   // e4m3 V is widened to fp16 as well
      if constexpr (!FP8) {
        // A bf16 V value beyond the fp16 range became infinite in the fp16 tile,
        // so every accumulator it met is infinite or NaN.  Rare: then the whole
        // item again with P V in bf16 (for V that is itself non-finite this gives
        // the same result as the first pass would have).
        float chk = 0.f;   // NaN iff some accumulator entry is not finite
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) chk = fmaf(acc[db][r], 0.f, chk);
        if (__builtin_amdgcn_ballot_w64(chk != chk) != 0 && lane == 0) s_big_item = item_no;
        __syncthreads();
      }
      if (!FP8 && s_big_item == item_no) {
#pragma unroll
        for (int db = 0; db < DB; ++db) acc[db] = f32x16{};
        m_run = NEG_INF;
        l_run = 0.f;
        key_loop(std::false_type{});
      }
    }

    // epilogue: O = acc / l, LSE = (m + log2 l) * ln 2
    const float l_tot = xhalf_sum(l_run);
    const float inv = l_tot > 0.f ? (FP8 ? a.v_scale : 1.f) / l_tot : 0.f;
    const float m_fin = (m_run == NEG_INF) ? 0.f : m_run;
    const float lse = l_tot > 0.f ? (m_fin + __log2f(l_tot)) * kLn2 : NEG_INF;
    auto o_row = [&](int r) -> __bf16* {   // output row r of this item
      return BCAST ? a.o + (((int64_t)b * lq + r) * a.hq + h) * D : a.o + ((int64_t)(q_base + r) * a.hq + h) * D;
    };
    // A lane holds 4 consecutive columns of its row per register quad, so direct
    // stores write 32 rows in 8-byte pieces per instruction.  The waves' 32 x D
    // blocks go through LDS instead (the stages, free after the last tile's
    // barrier, or LDS of their own, see FwdTile) and out 16 bytes per lane, D / 8
    // lanes covering one row; direct stores remain only where neither fits.
    constexpr int EP = T::EP, NW = T::NW;
    constexpr bool ALL_VT = T::EP_ALL_VT, OWN = T::EP_OWN > 1;
    constexpr bool VIA_LDS = ALL_VT || T::EP_SPLIT || OWN;
    debug_barrier();
    if constexpr (VIA_LDS) {
      __bf16* blk = OWN ? &ep_lds[0] + w * 32 * EP
                  : (ALL_VT || w < NW / 2) ? &vt_lds[0][0] + (ALL_VT ? w : w % (NW / 2)) * 32 * EP
                                           : (__bf16*)&k_raw[0][0] + (w % (NW / 2)) * 32 * EP;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          bf16x4 ov;
#pragma unroll
          for (int x = 0; x < 4; ++x) ov[x] = (__bf16)(acc[db][4 * r4 + x] * inv);
          *(bf16x4*)(blk + l32 * EP + 32 * db + 8 * r4 + 4 * hh) = ov;
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
        if (r < lq) *(u32x4*)(o_row(r) + 8 * col) = *(const u32x4*)(blk + row * EP + 8 * col);
      }
    } else {
      if (tid == 0) s_item[slot ^ 1] = next_work_item(a.queues, s_queue, home_q, drained);
      if (row_ok) {
        __bf16* op = o_row(my_row);
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4) {
            bf16x4 ov;
#pragma unroll
            for (int x = 0; x < 4; ++x) ov[x] = (__bf16)(acc[db][4 * r4 + x] * inv);
            *(bf16x4*)(op + 32 * db + 8 * r4 + 4 * hh) = ov;
          }
      }
    }
    if (row_ok && hh == 0) {
      const int64_t li = BCAST ? ((int64_t)b * a.hq + h) * lq + my_row
                               : (int64_t)h * a.total_q + q_base + my_row;
      a.lse[li] = lse;
    }
    __syncthreads();   // next item published; the LDS buffers are free for it
    slot ^= 1;
    item = __builtin_amdgcn_readfirstlane(s_item[slot]);
  }
}

// Scheduling units.  LLVM's iterative ILP scheduler suits the long-row kernels
// (causal at d = 128: 3-4 % faster; every kernel at d >= 192: 9-13 % faster)
// and the latency-first one the rest (non-causal d = 128: 3 % faster; d = 64:
// 2-7 % faster; d = 96: equal), measured in interleaved runs.  The first group
// is instantiated only by fwd_ilp.hip (this file included with JFA_FWD_ILP_UNIT
// defined), the second only here, so no kernel is emitted by both units.
constexpr bool fwd_in_ilp_unit(int d, bool causal) { return d >= 192 || (causal && d == 128); }

// Head dims with an 8-wave forward, which may run NARROW instead.
constexpr bool fwd_has_narrow(int d, bool fp8) { return !fp8 && (d == 64 || d == 128); }

#ifndef JFA_FWD_ILP_UNIT
template <bool FP8, bool NARROW>
static int fwd_rows_t(int head_dim) {
  switch (head_dim) {
    case 64: return FwdTile<64, FP8, NARROW>::BM;
    case 96: return FwdTile<96, false>::BM;
    case 128: return FwdTile<128, FP8, NARROW>::BM;
    case 192: return FwdTile<192, FP8>::BM;
    default: return FwdTile<256, FP8>::BM;
  }
}
template <bool FP8, bool NARROW>
static int fwd_wgs_t(int head_dim) {
  switch (head_dim) {
    case 64: return FwdTile<64, FP8, NARROW>::WG_PER_CU;
    case 96: return FwdTile<96, false>::WG_PER_CU;
    case 128: return FwdTile<128, FP8, NARROW>::WG_PER_CU;
    case 192: return FwdTile<192, FP8>::WG_PER_CU;
    default: return FwdTile<256, FP8>::WG_PER_CU;
  }
}
int fwd_block_rows(int head_dim, bool fp8, bool narrow) {
  narrow = narrow && fwd_has_narrow(head_dim, fp8);
  return fp8 ? fwd_rows_t<true, false>(head_dim) : narrow ? fwd_rows_t<false, true>(head_dim) : fwd_rows_t<false, false>(head_dim);
}
int fwd_kv_tile(int head_dim) { return head_dim <= 128 ? FwdTile<128>::BN : head_dim <= 192 ? FwdTile<192>::BN : FwdTile<256>::BN; }
int fwd_blocks_per_cu(int head_dim, bool fp8, bool narrow) {
  narrow = narrow && fwd_has_narrow(head_dim, fp8);
  return fp8 ? fwd_wgs_t<true, false>(head_dim) : narrow ? fwd_wgs_t<false, true>(head_dim) : fwd_wgs_t<false, false>(head_dim);
}

template <int D, bool FP8, bool NARROW>
static hipError_t launch_fwd_dt(const FwdArgs& a, int grid, hipStream_t stream) {
  if (fwd_in_ilp_unit(D, a.causal && !a.bcast)) return launch_fwd_ilp(a, D, FP8, grid, stream);
  const dim3 g(grid), blk(FwdTile<D, FP8, NARROW>::NT);
  if constexpr (!fwd_in_ilp_unit(D, false)) {
    if (a.bcast)
      hipLaunchKernelGGL((fwd_kernel<D, false, true, FP8, NARROW>), g, blk, 0, stream, a);
    else if (a.causal) {
      if constexpr (!fwd_in_ilp_unit(D, true)) hipLaunchKernelGGL((fwd_kernel<D, true, false, FP8, NARROW>), g, blk, 0, stream, a);
    } else
      hipLaunchKernelGGL((fwd_kernel<D, false, false, FP8, NARROW>), g, blk, 0, stream, a);
  }
  return hipGetLastError();
}

template <int D>
static hipError_t launch_fwd_d(const FwdArgs& a, int grid, hipStream_t stream) {
  if constexpr (D % 64 == 0) {
    if (a.fp8) return launch_fwd_dt<D, true, false>(a, grid, stream);
  } else {
    if (a.fp8) return hipErrorInvalidValue;   // e4m3 needs 64-deep k-steps
  }
  if constexpr (fwd_has_narrow(D, false)) {
    if (a.narrow) return launch_fwd_dt<D, false, true>(a, grid, stream);
  }
  return launch_fwd_dt<D, false, false>(a, grid, stream);
}

hipError_t launch_fwd(const FwdArgs& a, int head_dim, int grid, hipStream_t stream) {
  switch (head_dim) {
    case 64: return launch_fwd_d<64>(a, grid, stream);
    case 96: return launch_fwd_d<96>(a, grid, stream);
    case 128: return launch_fwd_d<128>(a, grid, stream);
    case 192: return launch_fwd_d<192>(a, grid, stream);
    case 256: return launch_fwd_d<256>(a, grid, stream);
    default: return hipErrorInvalidValue;
  }
}

#else
template <int D, bool FP8, bool NARROW>
static hipError_t launch_fwd_ilp_dt(const FwdArgs& a, int grid, hipStream_t stream) {
  const dim3 g(grid), blk(FwdTile<D, FP8, NARROW>::NT);
  const bool causal = a.causal && !a.bcast;
  if (!fwd_in_ilp_unit(D, causal)) return hipErrorInvalidValue;
  if constexpr (fwd_in_ilp_unit(D, false)) {
    if (a.bcast)
      hipLaunchKernelGGL((fwd_kernel<D, false, true, FP8, NARROW>), g, blk, 0, stream, a);
    else if (!causal)
      hipLaunchKernelGGL((fwd_kernel<D, false, false, FP8, NARROW>), g, blk, 0, stream, a);
  }
  if constexpr (fwd_in_ilp_unit(D, true)) {
    if (causal) hipLaunchKernelGGL((fwd_kernel<D, true, false, FP8, NARROW>), g, blk, 0, stream, a);
  }
  return hipGetLastError();
}

hipError_t launch_fwd_ilp(const FwdArgs& a, int head_dim, bool fp8, int grid, hipStream_t stream) {
  switch (head_dim) {
    case 128:
      if (fp8) return launch_fwd_ilp_dt<128, true, false>(a, grid, stream);
      return a.narrow ? launch_fwd_ilp_dt<128, false, true>(a, grid, stream) : launch_fwd_ilp_dt<128, false, false>(a, grid, stream);
    case 192: return fp8 ? launch_fwd_ilp_dt<192, true, false>(a, grid, stream) : launch_fwd_ilp_dt<192, false, false>(a, grid, stream);
    case 256: return fp8 ? launch_fwd_ilp_dt<256, true, false>(a, grid, stream) : launch_fwd_ilp_dt<256, false, false>(a, grid, stream);
    default: return hipErrorInvalidValue;
  }
}
#endif

}  // namespace jfa
