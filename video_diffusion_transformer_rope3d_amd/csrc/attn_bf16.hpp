// Flash-attention forward for bf16 Q/K/V on gfx950 matrix cores.
//
// One workgroup = NW waves; each wave owns QB blocks of 32 queries of one
// (batch, head) slice, so a workgroup covers BR = NW*QB*32 queries. Keys and
// values stream through LDS in tiles of KT = 64 (double-buffered, copied by
// direct global->LDS 16-byte loads from the pre-pass workspace).
//
// Per tile and query block, with 32x32 MFMA blocks:
//   S^T (64 keys x 32 queries) = K' Q'^T     v_mfma_f32_32x32x16_f16, fp32 acc
//   online softmax in base 2 (Q' carries scale*log2 e), lazily rescaled
//   O^T (D x 32 queries) += V^T P^T           v_mfma_f32_32x32x16_bf16, fp32 acc
// Computing the transposed products puts every score and every output
// element of query q in the two lanes q and q+32: row max and row sum need a
// single cross-lane swap, the rescale factor is lane-local, and the
// probabilities feed the second product straight from registers.
#pragma once

#include "common.hpp"

namespace vidattn {

// Skip the O/l rescale while the running maximum grows by at most this much
// (log2 units): probabilities then stay below 2^8, exact algebra unchanged.
constexpr float kLazyRescale = 8.0f;

template <int D, int NW, int QB>
__global__ __launch_bounds__(NW * 64, 1) void attn_fwd_bf16_kernel(const uint16_t* __restrict__ Q,
                                                                    const uint8_t* __restrict__ ws,
                                                                    uint16_t* __restrict__ O, int N, int nkt, int ntq,
                                                                    int total_wg, float qscale, RopeParams rp) {
  constexpr int KT = 64;
  constexpr int BR = NW * QB * 32;
  constexpr int KSTEPS = D / 16;  // 16-wide head-dim steps of the score product
  constexpr int DB = D / 32;      // 32-wide head-dim blocks of the output
  constexpr int MS = KT / 16;     // 16-key steps of the P.V product
  constexpr int TILE = KT * D * 2;
  constexpr int TB = 2 * TILE;
  constexpr int LOADS = TB / (NW * 1024);
  static_assert(TB % (NW * 1024) == 0, "tile must split into whole 1 KB wave loads");
  __shared__ __attribute__((aligned(1024))) uint8_t lds[2 * TB];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 5, qi = lane & 31;

  // Workgroups are dealt to the 8 XCDs round-robin; give each XCD a
  // contiguous range of (bh, query tile) so the workgroups resident on one
  // XCD share the same K/V stream in its L2.
  const int wg = blockIdx.x;
  const int xcd = wg & 7, k8 = wg >> 3;
  const int per = total_wg >> 3, rem = total_wg & 7;
  const int logical = xcd * per + (xcd < rem ? xcd : rem) + k8;
  const int bh = logical / ntq;
  const int qt = logical - bh * ntq;
  const uint8_t* wsbh = ws + (int64_t)bh * nkt * TB;

  auto load_tile = [&](int kt, int buf) {
    const uint8_t* src = wsbh + (int64_t)kt * TB;
    uint8_t* dst = lds + buf * TB;
#pragma unroll
    for (int r = 0; r < LOADS; ++r) {
      const int blk = r * NW + wave;
      __builtin_amdgcn_global_load_lds(src + blk * 1024 + lane * 16,
                                       (__attribute__((address_space(3))) void*)(dst + blk * 1024), 16, 0, 0);
    }
  };
  load_tile(0, 0);

  // ---- queries: rotate, pre-scale by scale*log2(e), round to fp16 (B operand)
  half8 qreg[QB][KSTEPS];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int q = qt * BR + (wave * QB + qb) * 32 + qi;
    const uint16_t* qrow = Q + ((int64_t)bh * N + (q < N ? q : 0)) * D;
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) {
      float x[8];
      unpack_bf16x8(*reinterpret_cast<const u32x4*>(qrow + 16 * s + 8 * g), x);
      if (rp.enabled) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          float c, sn;
          rope_cos_sin(rp, q < N ? q : 0, 8 * s + 4 * g + j, c, sn);
          rotate_pair(x[2 * j], x[2 * j + 1], c, sn);
        }
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) qreg[qb][s][j] = (_Float16)(q < N ? x[j] * qscale : 0.f);
    }
  }

  f32x16 oacc[QB][DB];
  float m[QB], l[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m[qb] = -INFINITY;
    l[qb] = 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) oacc[qb][db][i] = 0.f;
  }
  const int tail = N - (nkt - 1) * KT;  // valid keys of the last tile, 1..KT

  for (int kt = 0; kt < nkt; ++kt) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (kt + 1 < nkt) load_tile(kt + 1, (kt + 1) & 1);
    const uint8_t* kl = lds + (kt & 1) * TB;
    const uint8_t* vl = kl + TILE;

    // ---- S^T = K' Q'^T
    f32x16 sacc[2][QB];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s) {
        const half8 a = *reinterpret_cast<const half8*>(kl + ((kb * KSTEPS + s) * 64 + lane) * 16);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          if (s == 0) {
            const f32x16 z = {};
            sacc[kb][qb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, qreg[qb][s], z, 0, 0, 0);
          } else {
            sacc[kb][qb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, qreg[qb][s], sacc[kb][qb], 0, 0, 0);
          }
        }
      }
    }

    // ---- keys past N in the last tile get -inf.
    // Score register i of lane (q, g) in key block kb is key 32kb + 16(i/8) + 8g + i%8.
    if (kt == nkt - 1 && tail < KT) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = 32 * kb + 16 * (i >> 3) + 8 * g + (i & 7);
          if (key >= tail)
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) sacc[kb][qb][i] = -INFINITY;
        }
    }

    // ---- online softmax, probabilities to bf16 B operands
    bf16x8 pk[QB][MS];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float mx = sacc[0][qb][0];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[kb][qb][i]);
      mx = xor32_max(mx);
      if (__builtin_amdgcn_ballot_w64(mx > m[qb] + kLazyRescale) != 0) {
        const float mnew = fmaxf(m[qb], mx);
        const float alpha = __builtin_amdgcn_exp2f(m[qb] - mnew);
        m[qb] = mnew;
        l[qb] *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int i = 0; i < 16; ++i) oacc[qb][db][i] *= alpha;
      }
      const float mm = m[qb];
      float ls = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float p = __builtin_amdgcn_exp2f(sacc[kb][qb][i] - mm);
          ls += p;
          pk[qb][2 * kb + (i >> 3)][i & 7] = (__bf16)p;
        }
      l[qb] += ls;
    }

    // ---- O^T += V^T P^T
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int ms = 0; ms < MS; ++ms) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(vl + ((db * MS + ms) * 64 + lane) * 16);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          oacc[qb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pk[qb][ms], oacc[qb][db], 0, 0, 0);
      }
    }
  }

  // ---- epilogue: O = O^T / l, rounded to bf16.
  // Output register i of lane (q, g) in head-dim block db is d = 32db + 8(i/4) + 4g + i%4.
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int q = qt * BR + (wave * QB + qb) * 32 + qi;
    const float inv = 1.0f / xor32_sum(l[qb]);
    if (q < N) {
      uint16_t* orow = O + ((int64_t)bh * N + q) * D;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int ib = 0; ib < 4; ++ib) {
          bf16x4 v;
#pragma unroll
          for (int j = 0; j < 4; ++j) v[j] = (__bf16)(oacc[qb][db][4 * ib + j] * inv);
          *reinterpret_cast<bf16x4*>(orow + 32 * db + 8 * ib + 4 * g) = v;
        }
    }
  }
}

}  // namespace vidattn
