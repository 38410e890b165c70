// Device-side helpers shared by the gfx950 kernels of libjfa.
//
// MFMA lane layouts used throughout (checked on gfx950 with an in-bounds probe):
//   v_mfma_f32_32x32x16_bf16  A[m][k]: lane l holds row m = l%32 and 8 k-slots
//                             (half h = l/32, element j);  B[k][n]: column n = l%32,
//                             the same (h, j) k-slots;  C[m][n]: lane l, register r
//                             holds m = 8*(r/4) + 4*(l/32) + r%4, n = l%32.
//   Which logical k sits in slot (h, j) is the caller's choice as long as A and B
//   agree, so a C tile can feed the next contraction straight from registers.
//   ds_read_tr16_b64: inside each 16-lane group, lane i supplies an address of
//   four 16-bit values; call them M[i][0..3].  Lane i receives M[4e + i/4][i%4]
//   for e = 0..3.  With lane i pointing at row (r0 + i/4), column (c0 + 4*(i%4))
//   of a row-major bf16 tile, lane i receives the column c0 + i, rows r0..r0+3:
//   a transposed 4x16 read.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "jfa_internal.h"

namespace jfa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

#define JFA_LDS __attribute__((address_space(3)))

// Word 3 of a raw buffer resource (32-bit data format, no swizzle); loads past
// num_records return zero.
constexpr int kBufferFlags = 0x00020000;

// 8 e4m3 bytes -> 8 bf16 (exact), packed two per dword in column order.
__device__ __forceinline__ u32x4 widen_e4m3x8(uint2 x) {
  typedef float f2_t __attribute__((ext_vector_type(2)));
  u32x4 r;
  const f2_t p[4] = {__builtin_amdgcn_cvt_pk_f32_fp8(x.x, false), __builtin_amdgcn_cvt_pk_f32_fp8(x.x, true),
                     __builtin_amdgcn_cvt_pk_f32_fp8(x.y, false), __builtin_amdgcn_cvt_pk_f32_fp8(x.y, true)};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    bf16x2 q;
    q[0] = (__bf16)p[i][0];
    q[1] = (__bf16)p[i][1];
    r[i] = __builtin_bit_cast(uint32_t, q);
  }
  return r;
}

// 8 e4m3 bytes -> 8 fp16 (exact: every e4m3 value is an fp16 value), packed two
// per dword in column order.
__device__ __forceinline__ u32x4 widen_e4m3x8_f16(uint2 x) {
  u32x4 r;
  const f32x2 p[4] = {__builtin_amdgcn_cvt_pk_f32_fp8(x.x, false), __builtin_amdgcn_cvt_pk_f32_fp8(x.x, true),
                      __builtin_amdgcn_cvt_pk_f32_fp8(x.y, false), __builtin_amdgcn_cvt_pk_f32_fp8(x.y, true)};
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector(p[i], f16x2));
  return r;
}

// P V runs on the fp16 matrix cores: P in [0, 2^8] (the lazy rescale bounds it)
// keeps 11 significant bits instead of bf16's 8, and every bf16 V value of
// magnitude below 65520 is exactly an fp16 value (below 2^-14 it becomes an fp16
// subnormal, an absolute change under 2^-25).  Larger magnitudes become infinite:
// the forward and the decode detect the non-finite accumulators that follows and
// compute that work item again with P V in bf16.
constexpr float kF16Overflow = 65520.f;   // smallest magnitude that fp16 rounds to infinity

// Two bf16 values (one dword, low half first) -> two fp16 values.
__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t x) {
  const float lo = __uint_as_float(x << 16), hi = __uint_as_float(x & 0xffff0000u);
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, f16x2));
}

__device__ __forceinline__ f16x8 to_f16x8(const float* s) {
  f16x8 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const f16x2 h = __builtin_convertvector((f32x2){s[2 * i], s[2 * i + 1]}, f16x2);
    r[2 * i] = h[0];
    r[2 * i + 1] = h[1];
  }
  return r;
}

// Raw buffer resource for a wave-uniform base and byte range.  The base and range
// are moved to scalar registers explicitly: when a 64-bit address product ends up
// in vector registers, the compiler otherwise wraps every load through the
// resource in a readfirstlane loop.  Callers pass values that are the same in
// every lane of the wave.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t uniform_rsrc(const void* base, uint32_t nbytes) {
  const uint64_t a = (uint64_t)base;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  const uint32_t n = __builtin_amdgcn_readfirstlane(nbytes);
  return __builtin_amdgcn_make_buffer_rsrc((void*)(((uint64_t)hi << 32) | lo), (short)0, n, kBufferFlags);
}

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
// dv += a0 p0 + a1 p1 and dk += b0 s0 + b1 s1 on v_mfma_f32_32x32x16_bf16 with
// both accumulators in AGPRs (the caller's other MFMAs keep theirs in VGPRs).
// The compiler does not see MFMAs inside inline asm, so this statement carries
// the wait states it would otherwise place, as read from the code it emits for
// the same builtin sequences: two before an MFMA whose operand a VALU or
// v_accvgpr_write has just written (every statement starts with them); none
// between MFMAs chained on the same accumulator; agpr_settle's before anything
// else reads or writes the accumulators.  One statement holds the four MFMAs,
// so nothing the compiler emits can land between them; volatile keeps the
// statements in program order.
__device__ __forceinline__ void mfma4_acc_agpr(f32x16& dv, f32x16& dk, bf16x8 a0, bf16x8 a1, bf16x8 b0,
                                               bf16x8 b1, bf16x8 p0, bf16x8 p1, bf16x8 s0, bf16x8 s1) {
  asm volatile(
      "s_nop 1\n\t"
      "v_mfma_f32_32x32x16_bf16 %0, %2, %6, %0\n\t"
      "v_mfma_f32_32x32x16_bf16 %1, %4, %8, %1\n\t"
      "v_mfma_f32_32x32x16_bf16 %0, %3, %7, %0\n\t"
      "v_mfma_f32_32x32x16_bf16 %1, %5, %9, %1"
      : "+a"(dv), "+a"(dk)
      : "v"(a0), "v"(a1), "v"(b0), "v"(b1), "v"(p0), "v"(p1), "v"(s0), "v"(s1));
}

// 16 wait states after the last mfma4_acc_agpr (the compiler places 12 before
// reading a 32x32x16 result).  Every accumulator is an operand, so the statement
// follows every MFMA that writes one and precedes every later use of any of them.
template <int N>
__device__ __forceinline__ void agpr_settle(f32x16 (&x)[N], f32x16 (&y)[N]) {
#define JFA_SETTLE "s_nop 15"
  if constexpr (N == 4) {
    asm volatile(JFA_SETTLE : "+a"(x[0]), "+a"(x[1]), "+a"(x[2]), "+a"(x[3]), "+a"(y[0]), "+a"(y[1]), "+a"(y[2]),
                 "+a"(y[3]));
  } else {
    static_assert(N == 6, "accumulator blocks of the d >= 192 dK/dV kernels");
    asm volatile(JFA_SETTLE : "+a"(x[0]), "+a"(x[1]), "+a"(x[2]), "+a"(x[3]), "+a"(x[4]), "+a"(x[5]), "+a"(y[0]),
                 "+a"(y[1]), "+a"(y[2]), "+a"(y[3]), "+a"(y[4]), "+a"(y[5]));
  }
#undef JFA_SETTLE
}

__device__ __forceinline__ f32x16 mfma32x32x16_f16(f16x8 a, f16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// Transposed 4x16 read of a row-major bf16 tile in LDS (see the layout note above).
__device__ __forceinline__ bf16x4 lds_read_tr4(const __bf16* p) {
  s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((JFA_LDS s16x4*)(p));
  return __builtin_bit_cast(bf16x4, r);
}

__device__ __forceinline__ bf16x8 cat8(bf16x4 a, bf16x4 b) {
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Reductions across the two 32-lane halves of a wave: permlane32_swap(x, x)
// leaves {x[l], x[l^32]} in the pair (order depends on the half), so one
// combine of the pair gives the cross-half result in every lane.
__device__ __forceinline__ float xhalf_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xhalf_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ bf16x8 to_bf16x8(const float* s) {
  bf16x8 r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = (__bf16)s[i];
  return r;
}

__device__ __forceinline__ bf16x8 zero_bf16x8() {
  return __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
}

__device__ __forceinline__ int cdiv(int a, int b) { return (a + b - 1) / b; }

// s_waitcnt vmcnt(0): every vector-memory load of this wave has returned.  Used
// after loads made under a branch whose results feed a loop: on the path that
// skips the branch the waitcnt pass cannot prove those loads retired, and would
// otherwise wait for all outstanding loads, this iteration's prefetch included,
// inside the loop.  (gfx9 encoding: vmcnt 0, expcnt 7, lgkmcnt 15.)
__device__ __forceinline__ void wait_vmem_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Race-hunting build: with JFA_DEBUG_SYNC defined every kernel adds a workgroup
// barrier before it refills an LDS stage and before it reuses the stages for its
// epilogue.  Only called where the whole workgroup arrives (outside per-wave
// branches).  Outputs must match the normal build bit for bit; a difference
// points at a missing barrier in the normal one.
__device__ __forceinline__ void debug_barrier() {
#ifdef JFA_DEBUG_SYNC
  __syncthreads();
#endif
}

// Work-queue hand-out for persistent workgroups.  The queue starts and sizes
// are copied into LDS once (load_queues, by all threads, followed by a barrier);
// next_work_item is then called by one thread.  `q` starts at the block's home
// queue, blockIdx.x % kQueues, and `drained` at 0; queues are visited
// cyclically and a queue found empty stays empty, so after kQueues empty
// visits every queue is drained and -1 is returned.
__device__ __forceinline__ void load_queues(const WorkQueues* wq, int* s_queue) {
  const int t = threadIdx.x;
  if (t < 2 * kQueues) s_queue[t] = t < kQueues ? wq->start[t] : wq->size[t - kQueues];
}
__device__ __forceinline__ int next_work_item(WorkQueues* wq, const int* s_queue, int& q, int& drained) {
  while (drained < kQueues) {
    const uint32_t i = atomicAdd(&wq->next[q].value, 1u);
    if (i < (uint32_t)s_queue[kQueues + q]) return s_queue[q] + (int)i;
    q = (q + 1) & (kQueues - 1);
    ++drained;
  }
  return -1;
}

}  // namespace jfa
