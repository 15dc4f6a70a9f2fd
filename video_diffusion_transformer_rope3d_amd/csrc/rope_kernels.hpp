// 3D rotary embedding kernels (HBM-bound elementwise work):
//   rope3d_kernel    standalone rotation of a [B][heads][N][d] tensor;
//   prep_kv_kernel   the key/value pre-pass of the bf16 attention: rotated
//                    keys rounded to fp16 and a transposed copy of V, both
//                    written tile by tile in the order the matrix-core
//                    operands are read, so the attention kernel copies
//                    each tile linearly into LDS.
#pragma once

#include "common.hpp"

namespace vidattn {

// ---------------------------------------------------------------- loads/stores of 8 elements

template <typename T>
struct Elem8;

template <>
struct Elem8<uint16_t> {  // bf16 storage
  static __device__ __forceinline__ void load(const uint16_t* p, float (&x)[8]) {
    unpack_bf16x8(*reinterpret_cast<const u32x4*>(p), x);
  }
  static __device__ __forceinline__ void store(uint16_t* p, const float (&x)[8]) {
    bf16x8 v;
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = (__bf16)x[i];
    *reinterpret_cast<bf16x8*>(p) = v;
  }
};

template <>
struct Elem8<_Float16> {
  static __device__ __forceinline__ void store(_Float16* p, const float (&x)[8]) {
    half8 v;
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = (_Float16)x[i];
    *reinterpret_cast<half8*>(p) = v;
  }
};

template <>
struct Elem8<float> {
  static __device__ __forceinline__ void load(const float* p, float (&x)[8]) {
    const f32x4 a = reinterpret_cast<const f32x4*>(p)[0];
    const f32x4 b = reinterpret_cast<const f32x4*>(p)[1];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[i] = a[i];
      x[4 + i] = b[i];
    }
  }
  static __device__ __forceinline__ void store(float* p, const float (&x)[8]) {
    f32x4 a, b;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      a[i] = x[i];
      b[i] = x[4 + i];
    }
    reinterpret_cast<f32x4*>(p)[0] = a;
    reinterpret_cast<f32x4*>(p)[1] = b;
  }
};

// ---------------------------------------------------------------- standalone rotation

// One thread = one 8-element chunk (4 pairs) of one token; its 4 cos/sin
// pairs are evaluated once and reused over `bh_per_block` (batch, head)
// slices. Row n of each slice (n < N) is grid token n0 + n.
// grid = (ceil(N*d/8 / 256), ceil(B*heads / bh_per_block)).
template <typename TIn, typename TOut>
__global__ __launch_bounds__(256) void rope3d_kernel(const TIn* in, TOut* out, int64_t nbh, int N, int n0, int d,
                                                     float prescale, int bh_per_block, RopeParams rp) {
  const int cpt = d >> 3;
  const int64_t item = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (item >= (int64_t)N * cpt) return;
  const int n = (int)(item / cpt);
  const int c = (int)(item - (int64_t)n * cpt);
  float cs[4], sn[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) rope_cos_sin(rp, n0 + n, 4 * c + j, cs[j], sn[j]);
  const int64_t bh0 = (int64_t)blockIdx.y * bh_per_block;
  const int64_t bh1 = bh0 + bh_per_block < nbh ? bh0 + bh_per_block : nbh;
  for (int64_t bh = bh0; bh < bh1; ++bh) {
    const int64_t off = (bh * N + n) * d + 8 * c;
    float x[8];
    Elem8<TIn>::load(in + off, x);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      rotate_pair(x[2 * j], x[2 * j + 1], cs[j], sn[j]);
      x[2 * j] *= prescale;
      x[2 * j + 1] *= prescale;
    }
    Elem8<TOut>::store(out + off, x);
  }
}

// ---------------------------------------------------------------- bf16 attention pre-pass

// Workspace tile layout (per (b, head), per tile of KT = 64 keys; the
// K part and the V part are TILE = 64*D*2 bytes each, K first). Lane
// l = i + 16r (i < 16, r < 4) of a 1 KB block holds 16 bytes:
//   K part: block kb*(D/32) + s for key block kb < 4 (16 keys) and head-dim
//           step s < D/32; the lane holds K'[score_key(kb, i)][32s + 8r ..
//           32s + 8r + 7] (fp16, rotated): the A operand (row i, k-slice r)
//           of v_mfma_f32_16x16x32_f16.
//   V part: block ks*(D/16) + db for key step ks < 2 (32 keys) and head-dim
//           block db < D/16; the lane holds V[32ks + 8r + j][16db + i],
//           j < 8 (bf16): the A operand of the V^T.P^T product.
// Key slots that hold no token (past N, or outside the grid) are zero in
// both parts.
//
// Which tokens a tile holds: tile t holds tokens 64t .. 64t+63 (row order),
// or, in the patch order of the local-window attention, the 8 x 8 patch
// (tf, ty, tx) of the grid, t = (tf*tyn + ty)*txn + tx, whose key 8r + c is
// the token at frame tf, row 8ty + r, column 8tx + c.
struct TileMap {
  int patch;  // 0: row order, 1: patch order (the kernel's PATCH)
  int H, W, tyn, txn;

  // token of key kk < 64 of tile t, -1 for an empty slot
  template <bool PATCH>
  __device__ __forceinline__ int token(int t, int kk, int N) const {
    if (!PATCH) {
      const int n = t * 64 + kk;
      return n < N ? n : -1;
    }
    const int tf = t / (tyn * txn), rest = t - tf * (tyn * txn);
    const int ty = rest / txn, tx = rest - ty * txn;
    const int y = 8 * ty + (kk >> 3), x = 8 * tx + (kk & 7);
    return y < H && x < W ? (tf * H + y) * W + x : -1;
  }
};

template <int D, bool PATCH = false>
__global__ __launch_bounds__(256) void prep_kv_kernel(const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
                                                      uint8_t* __restrict__ ws, int N, int nkt, int64_t nbh,
                                                      int bh_per_block, RopeParams rp, TileMap map) {
  constexpr int KT = 64;
  constexpr int KS = D / 32;  // 32-wide head-dim steps
  constexpr int DB = D / 16;  // 16-wide head-dim blocks
  constexpr int TILE = KT * D * 2;
  constexpr int SLOTS = TILE / 16 / 256;  // 16-byte slots per thread per part
  constexpr int VPAD = D + 8;
  __shared__ __attribute__((aligned(16))) uint16_t vs[KT * VPAD];

  const int t = threadIdx.x;
  const int tile = blockIdx.x;

  int ksrc[SLOTS];  // source key of the slot (-1: past N)
  int kchunk[SLOTS];
  float cs[SLOTS][4], sn[SLOTS][4];
#pragma unroll
  for (int r = 0; r < SLOTS; ++r) {
    const int slot = t + 256 * r;
    const int blk = slot >> 6, lane = slot & 63;
    const int i = lane & 15, rr = lane >> 4;
    const int kb = blk / KS, s = blk - kb * KS;
    const int n = map.token<PATCH>(tile, score_key(kb, i), N);
    ksrc[r] = n;
    kchunk[r] = 4 * s + rr;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      cs[r][j] = 1.f;
      sn[r][j] = 0.f;
      if (rp.enabled && n >= 0) rope_cos_sin(rp, n, 4 * kchunk[r] + j, cs[r][j], sn[r][j]);
    }
  }

  const int64_t bh0 = (int64_t)blockIdx.y * bh_per_block;
  const int64_t bh1 = bh0 + bh_per_block < nbh ? bh0 + bh_per_block : nbh;
  for (int64_t bh = bh0; bh < bh1; ++bh) {
    const uint16_t* Kbh = K + bh * N * D;
    const uint16_t* Vbh = V + bh * N * D;
    uint8_t* wt = ws + (bh * nkt + tile) * (int64_t)(2 * TILE);

    // keys: rotate, round to fp16, scatter into operand order
#pragma unroll
    for (int r = 0; r < SLOTS; ++r) {
      half8 h;
      if (ksrc[r] >= 0) {
        float x[8];
        Elem8<uint16_t>::load(Kbh + (int64_t)ksrc[r] * D + 8 * kchunk[r], x);
#pragma unroll
        for (int j = 0; j < 4; ++j) rotate_pair(x[2 * j], x[2 * j + 1], cs[r][j], sn[r][j]);
#pragma unroll
        for (int j = 0; j < 8; ++j) h[j] = (_Float16)x[j];
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) h[j] = (_Float16)0.f;
      }
      *reinterpret_cast<half8*>(wt + (t + 256 * r) * 16) = h;
    }

    // values: stage the row-major tile in LDS, then gather 8 keys per slot.
    // The gather reads, per instruction, one head-dim column pair of 16 lanes
    // in each of the row groups 8r + j (r < 4); row R keeps its 16-byte chunk
    // c at chunk c ^ 2((R >> 3) & 3), so the four groups read four disjoint
    // 32-byte windows of LDS banks (padding alone cannot separate rows 8
    // apart while rows stay 16-byte aligned).
    auto swz = [](int row) __attribute__((always_inline)) { return 2 * ((row >> 3) & 3); };
    __syncthreads();
#pragma unroll
    for (int r = 0; r < SLOTS; ++r) {
      const int ch = t + 256 * r;
      const int row = ch / (D / 8), col8 = ch - row * (D / 8);
      u32x4 w = {0u, 0u, 0u, 0u};
      const int n = map.token<PATCH>(tile, row, N);
      if (n >= 0) w = *reinterpret_cast<const u32x4*>(Vbh + (int64_t)n * D + 8 * col8);
      *reinterpret_cast<u32x4*>(vs + row * VPAD + 8 * (col8 ^ swz(row))) = w;
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < SLOTS; ++r) {
      const int slot = t + 256 * r;
      const int blk = slot >> 6, lane = slot & 63;
      const int i = lane & 15, rr = lane >> 4;
      const int ks = blk / DB, db = blk - ks * DB;
      const int col = 16 * db + i;
      const int key0 = 32 * ks + 8 * rr;  // rows key0 .. key0 + 7 share swz = 2 rr
      const int scol = 8 * ((col >> 3) ^ (2 * rr)) + (col & 7);
      u32x4 w;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        w[j] = (uint32_t)vs[(key0 + 2 * j) * VPAD + scol] | ((uint32_t)vs[(key0 + 2 * j + 1) * VPAD + scol] << 16);
      *reinterpret_cast<u32x4*>(wt + TILE + slot * 16) = w;
    }
  }
}

}  // namespace vidattn
