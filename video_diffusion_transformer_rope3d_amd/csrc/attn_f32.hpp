// Flash-attention forward for fp32 Q/K/V on gfx950 fp32 matrix cores
// (v_mfma_f32_32x32x2_f32). Same transposed formulation as the bf16 kernel
// (S^T = K Q^T, O^T += V^T P^T, base-2 online softmax), in fp32 throughout.
// 4 waves x 32 queries per workgroup; key tiles of 32 staged in LDS (K
// transposed so the A operand of each step is one conflict-free row read).
#pragma once

#include "common.hpp"

namespace vidattn {

template <int D>
__global__ __launch_bounds__(256) void attn_fwd_f32_kernel(const float* __restrict__ Q, const float* __restrict__ K,
                                                           const float* __restrict__ V, float* __restrict__ O, int N,
                                                           int ntq, float qscale, RopeParams rp) {
  constexpr int KT = 32;
  constexpr int BR = 128;
  constexpr int DB = D / 32;
  __shared__ float kt_s[D][KT + 1];
  __shared__ float v_s[KT][D + 4];

  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const int g = lane >> 5, qi = lane & 31;
  const int bh = blockIdx.x / ntq;
  const int qt = blockIdx.x - bh * ntq;
  const int q = qt * BR + wave * 32 + qi;
  const int qc = q < N ? q : 0;

  // queries: lane (q, g) holds element 2s + g of its rotated, pre-scaled row
  float qreg[D / 2];
  {
    const float* qrow = Q + ((int64_t)bh * N + qc) * D;
#pragma unroll
    for (int s = 0; s < D / 2; ++s) {
      float x0 = qrow[2 * s], x1 = qrow[2 * s + 1];
      if (rp.enabled) {
        float c, sn;
        rope_cos_sin(rp, qc, s, c, sn);
        rotate_pair(x0, x1, c, sn);
      }
      qreg[s] = q < N ? (g ? x1 : x0) * qscale : 0.f;
    }
  }

  f32x16 oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[db][i] = 0.f;
  float m = -INFINITY, l = 0.f;

  const float* Kbh = K + (int64_t)bh * N * D;
  const float* Vbh = V + (int64_t)bh * N * D;
  const int nkt = (N + KT - 1) / KT;
  for (int kt = 0; kt < nkt; ++kt) {
    const int n0 = kt * KT;
    __syncthreads();
    for (int ch = t; ch < KT * D / 4; ch += 256) {
      const int row = ch / (D / 4), c4 = ch - row * (D / 4);
      f32x4 kv = {0.f, 0.f, 0.f, 0.f}, vv = {0.f, 0.f, 0.f, 0.f};
      if (n0 + row < N) {
        kv = *reinterpret_cast<const f32x4*>(Kbh + (int64_t)(n0 + row) * D + 4 * c4);
        vv = *reinterpret_cast<const f32x4*>(Vbh + (int64_t)(n0 + row) * D + 4 * c4);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        kt_s[4 * c4 + j][row] = kv[j];
        v_s[row][4 * c4 + j] = vv[j];
      }
    }
    __syncthreads();

    // S^T (32 keys x 32 queries); register i of lane (q, g) is key 8(i/4) + 4g + i%4
    f32x16 sacc = {};
#pragma unroll
    for (int s = 0; s < D / 2; ++s)
      sacc = __builtin_amdgcn_mfma_f32_32x32x2f32(kt_s[2 * s + g][qi], qreg[s], sacc, 0, 0, 0);

    if (n0 + KT > N) {
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (n0 + 8 * (i >> 2) + 4 * g + (i & 3) >= N) sacc[i] = -INFINITY;
    }
    float mx = sacc[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) mx = fmaxf(mx, sacc[i]);
    mx = xor32_max(mx);
    const float mnew = fmaxf(m, mx);
    const float alpha = __builtin_amdgcn_exp2f(m - mnew);
    m = mnew;
    float p[16], ls = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      p[i] = __builtin_amdgcn_exp2f(sacc[i] - mnew);
      ls += p[i];
    }
    l = l * alpha + ls;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;
      // step s: lane (., g) contributes key 8(s/4) + 4g + s%4
#pragma unroll
      for (int s = 0; s < 16; ++s)
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(v_s[8 * (s >> 2) + 4 * g + (s & 3)][32 * db + qi], p[s],
                                                        oacc[db], 0, 0, 0);
    }
  }

  const float inv = 1.0f / xor32_sum(l);
  if (q < N) {
    float* orow = O + ((int64_t)bh * N + q) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int ib = 0; ib < 4; ++ib) {
        f32x4 v;
#pragma unroll
        for (int j = 0; j < 4; ++j) v[j] = oacc[db][4 * ib + j] * inv;
        *reinterpret_cast<f32x4*>(orow + 32 * db + 8 * ib + 4 * g) = v;
      }
  }
}

}  // namespace vidattn
