// Shared device helpers of libvidattn: vector types, conversions and the
// 3D rotary angle of one (token, pair).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace vidattn {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kMaxPairs = 128;  // head dim up to 256

// Rotary parameters as kernel arguments. Pair p (elements 2p, 2p+1) is
// driven by the frame index when p < pair_t, by the row index when
// p < pair_th, else by the column index; it turns by pos * omega[p].
// omega[p] = theta^(-2j/d_a) for pair j of its axis chunk of width d_a,
// evaluated on the host in double precision.
struct RopeParams {
  int enabled;
  int F, H, W;
  int pair_t, pair_th;
  double omega[kMaxPairs];
};

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b16) { return __uint_as_float(b16 << 16); }

// Unpack 8 bf16 (one 16-byte load) to fp32.
__device__ __forceinline__ void unpack_bf16x8(const u32x4 w, float (&x)[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = __uint_as_float(w[i] << 16);
    x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

// Token index -> grid coordinates (frame-major order n = (f*H + y)*W + x),
// then the coordinate driving pair p.
__device__ __forceinline__ int rope_pos(const RopeParams& rp, int n, int p) {
  const int hw = rp.H * rp.W;
  const int f = n / hw;
  const int r = n - f * hw;
  const int y = r / rp.W;
  const int x = r - y * rp.W;
  return p < rp.pair_t ? f : (p < rp.pair_th ? y : x);
}

// cos/sin of the rotation angle of pair p of token n. The angle pos*omega is
// formed and reduced modulo 2*pi in double precision (|angle| < 2^24 here,
// so the reduced value is exact to ~1e-11), rounded to fp32 in [-pi, pi],
// and its cos/sin taken in fp32 (absolute error ~2e-7, far below the fp16 /
// bf16 rounding of the rotated values and within the fp32 path's bounds).
__device__ __forceinline__ void rope_angle_cos_sin(int pos, double omega, float& c, float& s) {
  const double ang = (double)pos * omega;
  const double turns = rint(ang * 0.15915494309189535);  // nearest multiple of 2*pi
  const float r = (float)fma(-turns, 6.283185307179586, ang);
  sincosf(r, &s, &c);
}
__device__ __forceinline__ void rope_cos_sin(const RopeParams& rp, int n, int p, float& c, float& s) {
  rope_angle_cos_sin(rope_pos(rp, n, p), rp.omega[p], c, s);
}

// A wave-uniform double kept in scalar registers (its halves read from the
// first lane), so that a per-lane choice between two of them stays a select
// instead of becoming one per-lane load from a chosen address.
__device__ __forceinline__ double uniform_f64(double v) {
  const uint64_t b = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)b);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// Rotate one pair in fp32: (x0, x1) -> (x0 c - x1 s, x0 s + x1 c).
__device__ __forceinline__ void rotate_pair(float& x0, float& x1, float c, float s) {
  const float a = __builtin_fmaf(x0, c, -(x1 * s));
  const float b = __builtin_fmaf(x0, s, x1 * c);
  x0 = a;
  x1 = b;
}

// Lanes l and l^32 exchange a value; returns the pair {x[l], x[l^32]} in
// some order (enough for symmetric reductions such as max and sum).
__device__ __forceinline__ float xor32_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// The same for lanes l and l^16 (rows of 16 lanes swapped pairwise).
__device__ __forceinline__ float xor16_max(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor16_sum(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Direct global -> LDS copy of 16 bytes per lane: lane i reads base + voff
// (base uniform, in SGPRs; voff per lane) and the data lands at LDS byte
// address lds + 16 i. Written as inline assembly so that the compiler does
// not track it: with a compiler-tracked LDS DMA in flight, every LDS read
// wait in the same loop becomes lgkmcnt(0), which drains the operand
// double buffer at every other MFMA batch. The caller orders these copies
// with explicit vmcnt waits and barriers. (m0 holds the LDS address; the
// nop covers the m0 write before the LDS DMA. The compiler reserves m0 and
// warns about the clobber; it is sound because the kernels use m0 nowhere
// else, which tests/test_sources.py checks on the generated assembly.)
__device__ __forceinline__ void lds_dma16(const void* base, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(base), "s"(lds)
               : "memory", "m0");
}

// Workgroup barrier without a memory fence. __syncthreads() also drains
// every outstanding global load (vmcnt(0)), which would wait for the
// direct-to-LDS prefetches of later pipeline stages too; callers wait with
// an explicit, counted vmcnt for exactly the loads that must have landed.
// The memory clobber keeps the compiler from moving LDS accesses across it,
// and lgkmcnt(0) retires this wave's LDS reads before others may refill.
// (The wait is the builtin, not inline asm, so the compiler's wait-count
// tracking knows every LDS/scalar load has retired here.)
__device__ __forceinline__ void lds_barrier() {
  constexpr int kLgkm0 = 0xF | (0x3 << 14) | (0x7 << 4);  // lgkmcnt(0), vmcnt/expcnt untouched
  // The scheduling barriers keep arithmetic on its side of the workgroup
  // barrier too (the s_barrier alone fences only memory operations).
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(kLgkm0);
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// Key of row i (< 16) of key block kb (< 4) in a 64-key tile's score
// product. The 16x16 accumulator gives lane i + 16r rows 4r .. 4r + 3 of a
// block; with this order those rows of blocks 2s and 2s + 1 are the 8
// consecutive keys 32s + 8r .. 32s + 8r + 7, which is exactly the k-slice
// the lane supplies as B operand of the 16x16x32 P.V product.
__device__ __host__ __forceinline__ int score_key(int kb, int i) {
  return 32 * (kb >> 1) + 8 * (i >> 2) + 4 * (kb & 1) + (i & 3);
}

}  // namespace vidattn
