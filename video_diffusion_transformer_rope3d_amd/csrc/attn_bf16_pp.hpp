// Flash-attention forward for bf16 Q/K/V on gfx950 matrix cores, with the
// two waves of each SIMD in ping-pong.
//
// One workgroup = 8 waves (two per SIMD), 32 queries per wave, 256 queries
// of one (batch, head) slice per workgroup. Keys and values stream through a
// ring of NS LDS stages of KT = 64 keys, filled by direct global->LDS 16-byte
// loads from the pre-pass workspace (already in matrix-core operand order:
// every LDS read is one conflict-free ds_read_b128 per lane).
//
// Per wave and tile j there are two phases:
//   GEMM_j     O^T += V_{j-1}^T P_{j-1}^T   (32 x v_mfma_f32_16x16x32_bf16)
//              S'^T = K_j Q'^T - m          (32 x v_mfma_f32_16x16x32_f16)
//   SOFTMAX_j  P_j = exp2(S'_j) -> bf16, rare exact rescale, row sums
//              (group B adds its row sums in its next GEMM phase)
// The 16x16 products take each LDS operand block twice, once per 16-query
// half of the wave, so a wave reads the same LDS bytes per tile as one
// 32x32 product would; measured on this chip, the 16x16x32 instructions
// draw less power per FLOP on real data, and the kernel is power-limited.
// Waves 0-3 (group A) and 4-7 (group B) sit one per SIMD each (the hardware
// places wave w and w+4 of a workgroup on the same SIMD). One barrier opens
// each tile period; in it group A runs GEMM then SOFTMAX and group B runs
// SOFTMAX (of the previous tile) then GEMM, so on each SIMD one wave feeds
// the matrix core while the other works on the vector ALU:
//   period  0          1             2            ...  T
//   A       G_0 S_0    G_1 S_1       G_2 S_2           G_T
//   B       G_0        S_0 G_1       S_1 G_2           S_T-1 G_T
// (G_T is the last P.V alone.) Stage s of the ring holds K_j and V_{j-1} for
// j = s mod NS and is read in period j only. In period j the waves of group
// A issue the direct-to-LDS loads that refill the stage of tile j-1 with
// tile j+NS-1, at the start of their softmax phase (the sparse variants
// split them with group B, which issues its share at the period start).
//
// Lanes: lane i + 16r (i < 16, r < 4) holds, for each half h < 2 of the
// wave, query 16h + i: its scores for keys 32s + 8r .. 32s + 8r + 7 of each
// 32-key step s (score_key order), its outputs for head dims 16db + 4r ..
// 16db + 4r + 3, and head dims 32s + 8r .. + 7 of its rotated query. A
// query's scores and outputs are thus spread over the four lanes i, i + 16,
// i + 32, i + 48.
//
// Numerics: m + 20 (m the running maximum, in log2 units) enters as the
// accumulator input of the first score MFMA, so P = exp2(s - m - 20) is at
// most 2^-20 at the maximum. m moves only when some probability of a tile
// reaches 2 (a score more than 21 above m, or a non-finite one), which one
// bit of the OR of the bf16 probabilities shows; then the tile is redone
// against the exact maximum and O, l are scaled. The common factor 2^-20
// cancels in O / l.
//
// Three variants share the loop. Query subset: Nq query rows (Nq may differ
// from the Nk keys) whose rotary positions are the token indices qidx[row]
// (qidx == nullptr: row r is token r). Block-sparse (SPARSE): each
// (b, head, 256-query block) visits only the 64-key tiles listed in
// kvb[.][0 .. kvc[.]-1] (ascending), so "tile j" of the loop is the j-th
// listed tile; a block with no listed tile gets O = 0; the lists may be
// shared by every (b, head) (lists_shared). Local window (WIN != kWinNone,
// on top of SPARSE): in the listed tiles, keys outside the box of radii
// (r_f, r_h, r_w) around the query's grid position get -inf (row layout) or
// a score below -3e38 (patch layout), which exp2 takes to 0 all the same.
// Indices read from device memory are clamped into range, so no input can
// address outside the workspace. A row's m is unset until its first tile with a visible key
// (in the dense case: the first tile); the exact step runs on that tile, so
// tiles whose keys are all masked for a row leave its m untouched.
#pragma once

#include <type_traits>


#include "common.hpp"

namespace vidattn {

// Box of a local window over the F x H x W token grid. With mode != 0 (the
// host sets it when every key index is below 2^22) a key index k is split
// into row k / W and column k % W as (int)fma(k, invW, invW / 2): the exact
// quotient plus (r + 1/2) / W lies at least 1/(2W) from an integer and the
// fp32 error stays below that for k < 2^22 (the same for row / H).
// mode 2 (W >= 64): a 64-key tile spans at most two grid rows and is tested
// as a whole; mode 1 (W >= 8): each run of 8 keys spans at most two rows;
// mode 0: any grid, integer division and per-key stepping.
// The patch layout (WIN == kWinPatch) does not use mode: key tile t is the
// 8 x 8 patch (tf, ty, tx), t = (tf*tyn + ty)*txn + tx, with key 8r + c at
// grid row 8ty + r, column 8tx + c (keys past the grid's edge are zero in
// the workspace and never visible), and query block b the 16 x 16 patch
// (f, py, px) of one frame, b = (f*pyn + py)*pxn + px, with row 16i + j of
// the block at grid row 16py + i, column 16px + j (rows past the edge
// compute nothing that is stored). The host uses it only when tile and block
// indices are below 2^22 (their decode uses the fp32 reciprocal split).
constexpr int kWinNone = 0, kWinRows = 1, kWinPatch = 2;
struct WindowParams {
  int F, H, W;
  int rf, rh, rw;
  int mode;
  float invW, invH;
  int tyn, txn, pyn, pxn;
  float invtxn, invtyn, invpxn, invpyn;
};

// (int)fma(k, inv, inv / 2) = k / n for 0 <= k < 2^22 and inv = 1/n in fp32,
// written as (int)((k + 0.5) * inv): k + 0.5 is exact in fp32 and the product
// rounds the same exact value once, so the bits agree, and a uniform inv
// stays a scalar operand (a vector instruction takes at most one).
__device__ __forceinline__ int div_small(int k, float inv) { return (int)(((float)k + 0.5f) * inv); }

typedef short s16x4 __attribute__((ext_vector_type(4)));

template <int D, int NS, bool SPARSE, int WIN = kWinNone>
__global__ __launch_bounds__(512, 1) void attn_fwd_bf16_pp_kernel(
    const uint16_t* __restrict__ Q, const uint8_t* __restrict__ ws, uint16_t* __restrict__ O, int N, int nkt, int Nq,
    int ntq, int total_wg, float qscale, RopeParams rp, const int32_t* __restrict__ qidx,
    const int32_t* __restrict__ kvb, const int32_t* __restrict__ kvc, int maxb, int lists_shared,
    WindowParams wp) {
  static_assert(SPARSE || WIN == kWinNone, "the window visits listed tiles");
  constexpr int NW = 8;
  constexpr int KT = 64;
  constexpr int BR = NW * 32;
  constexpr int KS = D / 32;    // 32-wide head-dim steps of the score product
  constexpr int DB = D / 16;    // 16-wide head-dim blocks of the output
  constexpr int NKB = KT / 16;  // 16-key blocks of a tile's scores
  constexpr int MS = KT / 32;   // 32-key steps of the P.V product
  constexpr int TILE = KT * D * 2;  // bytes of one K tile (and of one V tile)
  constexpr int STAGE = 2 * TILE;
  // Dense: the waves of group A refill the ring. Sparse variants, whose
  // scattered tiles have a longer fetch latency, spread it over all waves
  // so that half of it is issued at the start of the period.
  constexpr bool kFillB = SPARSE;
  constexpr int NLOADER = kFillB ? NW : NW / 2;
  constexpr int STAGE_LOADS = STAGE / (NLOADER * 1024);  // 1 KB loads per loader wave per stage
  static_assert(STAGE % (NLOADER * 1024) == 0, "stage must split into whole 1 KB wave loads");
  static_assert(NS >= 2 && STAGE_LOADS * (NS - 2) < 64, "vmcnt range");
  // The probabilities are exp2(s - m - kBias): at most 2^-20 for a score at
  // the running maximum m, so a tile needs the exact step only when some
  // probability reaches 2 (a score more than kBias + 1 above m, or a
  // non-finite one): one bit of its bf16 exponent.
  constexpr float kBias = 20.f;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[NS * STAGE];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int group = wave >> 2;  // 0: GEMM then softmax in each period, 1: the reverse
  const int qi = lane & 15, r4 = lane >> 4;

  // Workgroups are dealt to the 8 XCDs round-robin; give each XCD a
  // contiguous range of (bh, query tile) so the workgroups resident on one
  // XCD share the same K/V stream in its L2.
  const int wg = blockIdx.x;
  const int xcd = wg & 7, k8 = wg >> 3;
  const int per = total_wg >> 3, rem = total_wg & 7;
  const int logical = xcd * per + (xcd < rem ? xcd : rem) + k8;
  const int bh = logical / ntq;
  const int qt = logical - bh * ntq;
  const uint8_t* wsbh = ws + (int64_t)bh * nkt * STAGE;

  // Key tiles this workgroup visits: all nkt (dense) or its list (SPARSE).
  // Loop position j maps to workspace tile tile_at(j), clamped into range.
  const int64_t lrow = lists_shared ? (int64_t)qt : (int64_t)bh * ntq + qt;
  const int32_t* lst = SPARSE ? kvb + lrow * maxb : nullptr;
  int nt = nkt;
  if constexpr (SPARSE) {
    const int c = kvc[lrow];
    nt = c < 0 ? 0 : (c > maxb ? maxb : c);
  }
  auto tile_at = [&](int j) __attribute__((always_inline)) {
    j = j < 0 ? 0 : (j < nt ? j : nt - 1);
    if constexpr (SPARSE) {
      const int t = lst[j];
      return t < 0 ? 0 : (t < nkt ? t : nkt - 1);
    } else {
      return j;
    }
  };
  // This lane's two query rows (h = 0, 1: row wave*32 + 16h + qi of the
  // block): their row indices in Q and O, and whether they exist (in the
  // patch layout, rows past the grid's edge do not; their grid position
  // (pf, py0 + 2 wave + h, px0 + qi) still serves the rotation).
  int qtok[2];
  bool qvalid[2];
  int pf = 0, py0 = 0, px0 = 0;  // the patch's frame, first row and first column
  if constexpr (WIN == kWinPatch) {
    const int b2 = div_small(qt, wp.invpxn), px = qt - b2 * wp.pxn;
    pf = div_small(b2, wp.invpyn);
    const int py = b2 - pf * wp.pyn;
    py0 = 16 * py;
    px0 = 16 * px;
  }
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int r = wave * 32 + 16 * h + qi;
    if constexpr (WIN == kWinPatch) {
      const int y = py0 + (r >> 4), x = px0 + (r & 15);
      qvalid[h] = y < wp.H && x < wp.W;
      qtok[h] = qvalid[h] ? (pf * wp.H + y) * wp.W + x : 0;
    } else {
      qtok[h] = qt * BR + r;
      qvalid[h] = qtok[h] < Nq;
      if (!qvalid[h]) qtok[h] = 0;
    }
  }
  if (SPARSE && nt == 0) {  // no key visited: O = 0 for the block's rows
#pragma unroll
    for (int h = 0; h < 2; ++h)
      if (qvalid[h]) {
        uint16_t* orow = O + ((int64_t)bh * Nq + qtok[h]) * D;
#pragma unroll
        for (int c = 0; c < KS; ++c) *reinterpret_cast<u32x4*>(orow + 32 * c + 8 * r4) = u32x4{0u, 0u, 0u, 0u};
      }
    return;
  }

  // Fill the stage of loop tile j: K of tile j and V of tile j-1 (blocks
  // 0 .. STAGE/1024-1 of the stage; K first). Load r of loader wave w moves
  // block r*NLOADER + w. At the ends (no V_{-1}, no K_nt) a neighbouring
  // tile is copied into the unused half so that every stage costs each
  // loader wave exactly STAGE_LOADS loads (the vmcnt arithmetic below relies
  // on it). tk and tv are the workspace tiles of loop tiles j and j-1.
  auto issue_one = [&](int j, int r, int tk, int tv) __attribute__((always_inline)) {
    constexpr int KBLK = TILE / 1024;
    const int blk = r * NLOADER + wave;
    uint8_t* st = lds + (j % NS) * STAGE;
    const uint8_t* src = blk < KBLK ? wsbh + (int64_t)tk * STAGE + blk * 1024
                                    : wsbh + (int64_t)tv * STAGE + TILE + (blk - KBLK) * 1024;
    lds_dma16(src, (uint32_t)lane * 16u,
              (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)(st + blk * 1024));
  };
  auto issue = [&](int j, int tk, int tv) __attribute__((always_inline)) {
#pragma unroll
    for (int r = 0; r < STAGE_LOADS; ++r) issue_one(j, r, tk, tv);
  };
  // ---- queries: rotate, pre-scale by scale*log2(e), round to fp16 (B operand).
  // Their loads are issued before any tile load, so waiting for tile 0 covers them.
  half8 qreg[KS][2];
  {
    u32x4 raw[2][KS];
    int pos[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint16_t* qrow = Q + ((int64_t)bh * Nq + qtok[h]) * D;
#pragma unroll
      for (int s = 0; s < KS; ++s) raw[h][s] = *reinterpret_cast<const u32x4*>(qrow + 32 * s + 8 * r4);
      // rotary position of this row: its token index in the grid
      pos[h] = qtok[h];
      if (qidx) {
        const int t = qidx[pos[h]];
        pos[h] = t < 0 ? 0 : (t < N ? t : N - 1);
      }
    }
    if (kFillB || group == 0)
      for (int j = 0; j < NS - 1; ++j)
        if (j <= nt) issue(j, tile_at(j), tile_at(j - 1));
    // grid coordinates of the rows, once
    const int hw = rp.H * rp.W;
    int cf[2], cy[2], cx[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      if constexpr (WIN == kWinPatch) {
        cf[h] = pf;
        cy[h] = py0 + 2 * wave + h;
        cx[h] = px0 + qi;
      } else {
        cf[h] = rp.enabled ? pos[h] / hw : 0;
        cy[h] = rp.enabled ? (pos[h] - cf[h] * hw) / rp.W : 0;
        cx[h] = pos[h] - cf[h] * hw - cy[h] * rp.W;
      }
    }
    // Window variants: the cos/sin of every (axis position, pair) the
    // workgroup's rows can use, once per workgroup, in the ring stage the
    // prologue does not fill (stage NS-1, first refilled after the barrier
    // that opens tile period 0): per axis, extent x pairs entries of
    // (cos, sin), t then h then w, over the whole grid (row layout) or the
    // patch's frame, 16 rows and 16 columns (patch layout). The 256 rows of
    // a workgroup share few positions per axis, so this evaluates far fewer
    // angles than one per (row, pair), which matters where a workgroup
    // visits few tiles; the values are those of rope_angle_cos_sin, so the
    // rotation is the same bit for bit. Tables that do not fit the stage
    // give way to each lane's own angles.
    constexpr bool kPatch = WIN == kWinPatch;
    const int f0 = kPatch ? pf : 0, y0 = kPatch ? py0 : 0, x0 = kPatch ? px0 : 0;
    const int nf = kPatch ? 1 : rp.F, nh = kPatch ? 16 : rp.H, nw = kPatch ? 16 : rp.W;
    const int npt = rp.pair_t, nph = rp.pair_th - rp.pair_t, npw = D / 2 - rp.pair_th;
    const int base_h = nf * npt, base_w = base_h + nh * nph, n_ent = base_w + nw * npw;
    const bool table = WIN != kWinNone && NS >= 3 && rp.enabled && n_ent <= STAGE / 8;
    float2* tbl = reinterpret_cast<float2*>(lds + (NS - 1) * STAGE);
    if (table) {
      for (int e = threadIdx.x; e < n_ent; e += NW * 64) {
        int apos, pair;
        if (e < base_h) {
          apos = e / npt;
          pair = e - apos * npt;
          apos += f0;
        } else if (e < base_w) {
          apos = (e - base_h) / nph;
          pair = rp.pair_t + (e - base_h - apos * nph);
          apos += y0;
        } else {
          apos = (e - base_w) / npw;
          pair = rp.pair_th + (e - base_w - apos * npw);
          apos += x0;
        }
        float c, sn;
        rope_angle_cos_sin(apos, rp.omega[pair], c, sn);
        tbl[e] = float2{c, sn};
      }
      lds_barrier();
    }
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      float x[2][8];
#pragma unroll
      for (int h = 0; h < 2; ++h) unpack_bf16x8(raw[h][s], x[h]);
      if (rp.enabled) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          // pair 16s + 4r + j: its four candidates (r = 0..3) are
          // wave-uniform kernel arguments, read once into scalar registers
          const int p = 16 * s + 4 * r4 + j;
          if (table) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
              const int e = p < rp.pair_t ? (cf[h] - f0) * npt + p
                                          : (p < rp.pair_th ? base_h + (cy[h] - y0) * nph + (p - rp.pair_t)
                                                            : base_w + (cx[h] - x0) * npw + (p - rp.pair_th));
              const float2 cs = tbl[e];
              rotate_pair(x[h][2 * j], x[h][2 * j + 1], cs.x, cs.y);
            }
          } else {
            double wr[4];
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) wr[rr] = uniform_f64(rp.omega[16 * s + 4 * rr + j]);
            const double w = r4 == 0 ? wr[0] : (r4 == 1 ? wr[1] : (r4 == 2 ? wr[2] : wr[3]));
#pragma unroll
            for (int h = 0; h < 2; ++h) {
              const int a = p < rp.pair_t ? cf[h] : (p < rp.pair_th ? cy[h] : cx[h]);
              float c, sn;
              rope_angle_cos_sin(a, w, c, sn);
              rotate_pair(x[h][2 * j], x[h][2 * j + 1], c, sn);
            }
          }
        }
      }
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int j = 0; j < 8; ++j) qreg[s][h][j] = (_Float16)(qvalid[h] ? x[h][j] * qscale : 0.f);
    }
  }

  f32x4 oacc[DB][2];
  f32x4 negm[2];  // -m broadcast: accumulator input of the first score MFMA
  f32x4 sacc[NKB][2];
  bf16x8 pk[MS][2];
  float m[2] = {0.f, 0.f}, l[2] = {0.f, 0.f};
  bool m_valid[2] = {false, false};  // the row's m comes from a visible key
  // window bits of the tile whose scores the last GEMM phase produced (the
  // softmax phase that follows reads them): bit 16h + 4kb + i for score i of
  // key block kb of half h; in the patch layout all 16 bits of a half are
  // equal (whether its query sees any key of the tile); all keys count as
  // visible outside the window variants
  unsigned wvis = ~0u;
  // Window of this lane's queries (window variant): a key at (f, y, x) is
  // visible when f - flo, y - ylo and x - clo, as unsigned, are at most
  // 2 r_f, 2 r_h and 2 r_w. For the fast test, a run of 8 keys starting at
  // column c0 of row r0 sees columns [clo, cend) of row r0 and, after the
  // row wrap, [wlo, wend) counted from the run's start as W - c0 + column.
  // The patch layout tests rows and columns on their own: the query sees
  // grid rows [ylo, yend) and columns [clo, cend).
  int flo[2] = {0, 0}, ylo[2] = {0, 0}, clo[2] = {0, 0}, cend[2] = {0, 0}, yend[2] = {0, 0};
  // (wlo and wend follow from clo and cend; formed where used)
  auto wlo = [&](int h) __attribute__((always_inline)) { return wp.W + (clo[h] > 0 ? clo[h] : 0); };
  auto wend = [&](int h) __attribute__((always_inline)) { return wp.W + cend[h]; };
  if constexpr (WIN != kWinNone) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      int qf, qy, qx;
      if constexpr (WIN == kWinPatch) {
        qf = pf;
        qy = py0 + 2 * wave + h;
        qx = px0 + qi;
      } else {
        const int t = qtok[h];
        const int hw = wp.H * wp.W;
        qf = t / hw;
        qy = (t - qf * hw) / wp.W;
        qx = t - qf * hw - qy * wp.W;
      }
      flo[h] = qf - wp.rf;
      ylo[h] = qy - wp.rh;
      clo[h] = qx - wp.rw;
      const int chi = qx + wp.rw < wp.W - 1 ? qx + wp.rw : wp.W - 1;
      cend[h] = chi + 1;
      yend[h] = (qy + wp.rh < wp.H - 1 ? qy + wp.rh : wp.H - 1) + 1;
    }
  }
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int i = 0; i < 4; ++i) negm[h][i] = -kBias;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int i = 0; i < 4; ++i) oacc[db][h][i] = 0.f;

  // P = exp2(S') as bf16 B operands: pk[s][h] holds keys 32s + 8r .. + 7 of
  // half h (score blocks 2s and 2s + 1). Returns the OR of the
  // probabilities' bits (a balanced tree: it is on the path to the
  // exact-step test).
  auto probs = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int s = 0; s < MS; ++s)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        bf16x8 p;
#pragma unroll
        for (int e = 0; e < 8; ++e) p[e] = (__bf16)__builtin_amdgcn_exp2f(sacc[2 * s + (e >> 2)][h][e & 3]);
        pk[s][h] = p;
      }
    uint32_t w[16];
#pragma unroll
    for (int s = 0; s < MS; ++s)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const bf16x8 pv = pk[s][h];
        const u32x4 x = __builtin_bit_cast(u32x4, pv);
#pragma unroll
        for (int e = 0; e < 4; ++e) w[8 * s + 4 * h + e] = x[e];
      }
    // (the empty asm statements keep the compiler from re-associating the
    // tree into one serial chain)
    uint32_t a = w[0] | w[1] | w[2], b = w[3] | w[4] | w[5], c = w[6] | w[7] | w[8];
    uint32_t d = w[9] | w[10] | w[11], e = w[12] | w[13] | w[14];
    asm("" : "+v"(a), "+v"(b), "+v"(c), "+v"(d), "+v"(e));
    uint32_t f = a | b | c, g = d | e | w[15];
    asm("" : "+v"(f), "+v"(g));
    return f | g;
  };
  // Adds the lane's partial row sums of the rounded probabilities to l.
  auto rowsum = [&]() __attribute__((always_inline)) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      float part[MS];
#pragma unroll
      for (int s = 0; s < MS; ++s) {
        float acc = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const bf16x2 pp = {pk[s][h][2 * j], pk[s][h][2 * j + 1]};
          acc = __builtin_amdgcn_fdot2_f32_bf16(pp, one, acc, false);
        }
        part[s] = acc;
      }
      l[h] += part[0] + part[1];
    }
  };
  // The exact step's rescale: the tile's exact maximum (relative to the
  // current m) becomes part of m; a row that has seen no visible key yet
  // takes the tile's maximum as its m (and keeps m = 0 if the tile shows it
  // none). O and l are scaled, the scores are moved to the new m.
  auto rescale_to_tile_max = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      float mx = sacc[0][h][0];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) mx = fmaxf(mx, sacc[kb][h][i]);
      mx = xor32_max(xor16_max(mx)) + kBias;
      // (in the patch layout a hidden key's score is finite, and wvis, the
      // same in the four lanes of a row, decides; elsewhere the row maximum
      // does)
      const bool seen = WIN == kWinPatch ? ((wvis >> (16 * h)) & 0xFFFFu) != 0u : mx > -INFINITY;
      const float delta = !m_valid[h] ? (seen ? mx : 0.f) : fmaxf(mx, 0.f);
      const float alpha = !m_valid[h] ? 1.f : __builtin_amdgcn_exp2f(-delta);
      m_valid[h] = m_valid[h] || seen;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i) oacc[db][h][i] *= alpha;
      l[h] *= alpha;
      m[h] += delta;
#pragma unroll
      for (int i = 0; i < 4; ++i) negm[h][i] = -(m[h] + kBias);
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) sacc[kb][h][i] -= delta;
    }
  };

  constexpr int kWaitNewer = STAGE_LOADS * (NS - 2);
  constexpr int kVmcntNewer = (kWaitNewer & 0xF) | ((kWaitNewer >> 4) << 14) | (0x7 << 4) | (0xF << 8);
  constexpr int kVmcntZero = (0x7 << 4) | (0xF << 8);
  // valid keys of the last key tile, 1..KT (the patch layout's edge keys are
  // masked by the window test instead)
  const int tail = WIN == kWinPatch ? KT : N - (nkt - 1) * KT;

  // Barrier that opens tile period i: tile i must have landed (a loader's
  // loads of the newer tiles may stay in flight).
  auto tile_barrier = [&](int i) __attribute__((always_inline)) {
    if (i + NS - 2 <= nt)
      __builtin_amdgcn_s_waitcnt(kVmcntNewer);
    else
      __builtin_amdgcn_s_waitcnt(kVmcntZero);
    lds_barrier();
  };

  // Window variant: bit 16h + 8s + e of window_vis(t) is set when key
  // 32s + 8r + e of workspace tile t (this lane's run e < 8 of step s) lies
  // inside the box of its query of half h. It depends on the tile and the
  // queries only, so the GEMM phase folds it into the accumulator input of
  // the first score MFMA (-m, or -inf for a key outside the box) while the
  // matrix core runs the P.V products.
  auto window_vis = [&](int tile) __attribute__((always_inline)) {
    unsigned vis = 0;
    if constexpr (WIN == kWinRows) {
      const int base = tile * KT;
      const unsigned fspan = 2u * wp.rf, yspan = 2u * wp.rh, xspan = 2u * wp.rw;
      if (wp.mode == 2) {
        // the tile [base, base + 64) lies in rows rb and rb + 1; the visible
        // keys of each row form one range of tile offsets
        auto bits64 = [](int a, int b) __attribute__((always_inline)) {  // bits [a, b) of 0..63
          const int lo = a < 0 ? 0 : (a > 64 ? 64 : a);
          const int hi = b < lo ? lo : (b > 64 ? 64 : b);
          return hi == lo ? (uint64_t)0 : ((~(uint64_t)0 >> (64 - hi)) & (~(uint64_t)0 << lo));
        };
        const int rb = div_small(base, wp.invW);
        const int cb = base - __mul24(rb, wp.W);
        const int fb = div_small(rb, wp.invH);
        const int yb = rb - __mul24(fb, wp.H);
        const bool wrap = yb == wp.H - 1;
        const int y1 = wrap ? 0 : yb + 1;
        const int f1 = fb + (wrap ? 1 : 0);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const bool row0 = ((unsigned)(fb - flo[h]) <= fspan) & ((unsigned)(yb - ylo[h]) <= yspan);
          const bool row1 = ((unsigned)(f1 - flo[h]) <= fspan) & ((unsigned)(y1 - ylo[h]) <= yspan);
          const uint64_t mm = (row0 ? bits64(clo[h] - cb, cend[h] - cb) : (uint64_t)0) |
                              (row1 ? bits64(wlo(h) - cb, wend(h) - cb) : (uint64_t)0);
          // this lane's keys are the runs at tile offsets 8r and 32 + 8r:
          // bytes r and 4 + r of mm
          const unsigned lo = (unsigned)mm, hi = (unsigned)(mm >> 32);
          const unsigned run = ((lo >> (8 * r4)) & 0xFFu) | (((hi >> (8 * r4)) & 0xFFu) << 8);
          vis |= run << (16 * h);
        }
      } else if (wp.mode == 1) {
        // W >= 8: a run covers at most rows r0 and r0 + 1. Its visible keys
        // form one bit range per row; the row test gates each range.
        auto bits = [](int a, int b) __attribute__((always_inline)) {  // bits [a, b) of 0..7
          const int lo = a < 0 ? 0 : (a > 8 ? 8 : a);
          const int hi = b < lo ? lo : (b > 8 ? 8 : b);
          return (1u << hi) - (1u << lo);
        };
#pragma unroll
        for (int s = 0; s < MS; ++s) {
          const int k0 = base + 32 * s + 8 * r4;
          const int r0 = div_small(k0, wp.invW);
          const int c0 = k0 - __mul24(r0, wp.W);
          const int f0 = div_small(r0, wp.invH);
          const int y0 = r0 - __mul24(f0, wp.H);
          const bool wrap = y0 == wp.H - 1;
          const int y1 = wrap ? 0 : y0 + 1;
          const int f1 = f0 + (wrap ? 1 : 0);
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const bool row0 = ((unsigned)(f0 - flo[h]) <= fspan) & ((unsigned)(y0 - ylo[h]) <= yspan);
            const bool row1 = ((unsigned)(f1 - flo[h]) <= fspan) & ((unsigned)(y1 - ylo[h]) <= yspan);
            const unsigned rv =
                (row0 ? bits(clo[h] - c0, cend[h] - c0) : 0u) | (row1 ? bits(wlo(h) - c0, wend(h) - c0) : 0u);
            vis |= rv << (16 * h + 8 * s);
          }
        }
      } else {
        // general grid: decode each run's first key, then step the column
        // index with carries into row and frame
        const int hw = wp.H * wp.W;
#pragma unroll
        for (int s = 0; s < MS; ++s) {
          const int k0 = base + 32 * s + 8 * r4;
          int f = k0 / hw;
          int y = (k0 - f * hw) / wp.W;
          int x = k0 - f * hw - y * wp.W;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
              const bool in = ((unsigned)(f - flo[h]) <= fspan) & ((unsigned)(y - ylo[h]) <= yspan) &
                              ((unsigned)(x - clo[h]) <= xspan);
              vis |= (in ? 1u : 0u) << (16 * h + 8 * s + e);
            }
            const bool cx = x == wp.W - 1;
            x = cx ? 0 : x + 1;
            const bool cy = cx & (y == wp.H - 1);
            y = cy ? 0 : (cx ? y + 1 : y);
            f += cy ? 1 : 0;
          }
        }
      }
    }
    return vis;
  };

  // Patch layout: the box test runs on the matrix core. Key kk of a tile
  // lies in tile row kk/8 and column kk%8, so an extra 16x16x16 MFMA per key
  // block and query half, with a one-hot A operand (the key's row among
  // k = 0..7, its column among k = 8..15) and a B operand of per-query
  // penalties (0 for a tile row or column the query sees, -3.39e38 for one
  // it does not), turns the accumulator input -m into exactly -m for a
  // visible key and into at most -3.39e38 (or -inf) for a hidden one; the
  // score products that follow (at most 2^40 in size) cannot lift it. Its
  // products are 1 x pen or 0 x pen, never 0 x inf, so no NaN arises.
  // (16x16x16 operands: lane i + 16r holds k = 4r .. 4r + 3 of row/column i.)
  s16x4 onehot[NKB];
  if constexpr (WIN == kWinPatch) {
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      const int kk = score_key(kb, qi);  // the key of A row qi in key block kb
      const int hot = r4 < 2 ? (kk >> 3) - 4 * r4 : (kk & 7) - 4 * (r4 - 2);
      bf16x4 v;
#pragma unroll
      for (int j = 0; j < 4; ++j) v[j] = (__bf16)(j == hot ? 1.f : 0.f);
      onehot[kb] = __builtin_bit_cast(s16x4, v);
    }
  }
  // The penalty operands of the tile the next score product covers (this
  // lane's quarter: tile rows 4r .. 4r + 3 for r < 2, columns 4(r - 2) ..
  // for r >= 2) and whether each query sees any of its keys (it becomes
  // wvis once the scores exist).
  s16x4 pen_sc[2];
  unsigned vis_sc = ~0u;
  // Sets pen_sc and vis_sc for tile t and returns whether any query of the
  // wave sees a key of it. A wave that sees none skips the tile's score
  // product, softmax and P.V product: its probabilities would all be 0, so
  // the result is the same bit for bit. Outside the patch layout every tile
  // is needed (a constant, so the skips compile away).
  auto prep_scores = [&](int tile) __attribute__((always_inline)) -> bool {
    if constexpr (WIN == kWinPatch) {
      const int t2 = div_small(tile, wp.invtxn), tx = tile - t2 * wp.txn;
      const int tf = div_small(t2, wp.invtyn), ty = t2 - tf * wp.tyn;
      auto bits8 = [](int a, int b) __attribute__((always_inline)) {  // bits [a, b) of 0..7
        const int lo = a < 0 ? 0 : (a > 8 ? 8 : a);
        const int hi = b < lo ? lo : (b > 8 ? 8 : b);
        return (1u << hi) - (1u << lo);
      };
      const unsigned cols = bits8(clo[0] - 8 * tx, cend[0] - 8 * tx);  // (both rows share the column)
      const bool fok = (unsigned)(tf - flo[0]) <= 2u * wp.rf;
      unsigned vis = 0u;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const unsigned rows = bits8(ylo[h] - 8 * ty, yend[h] - 8 * ty);
        vis |= fok && rows != 0u && cols != 0u ? 0xFFFFu << (16 * h) : 0u;
        const unsigned hide = (fok ? ~(r4 < 2 ? rows : cols) : ~0u) >> (4 * (r4 & 1));
        u32x2 w;
#pragma unroll
        for (int e = 0; e < 2; ++e)  // bf16 0xFF7F = -3.39e38 for a hidden row or column
          w[e] = (((hide >> (2 * e)) & 1u) | (((hide >> (2 * e + 1)) & 1u) << 16)) * 0xFF7Fu;
        pen_sc[h] = __builtin_bit_cast(s16x4, w);
      }
      vis_sc = vis;
      return __builtin_amdgcn_ballot_w64(vis != 0u) != 0;
    } else {
      (void)tile;
      return true;
    }
  };

  // Workspace tiles of loop tiles j-1 .. j+NS-1 in tile period j:
  // tw[k] = tile_at(j - 1 + k). Each period reads one list entry, for the
  // next period, in a softmax phase: the list reads are scalar loads, and
  // one in flight during a GEMM phase would turn every LDS operand wait
  // there into a full drain.
  // (Dense: tile_at is the clamped loop index and tw is not used.)
  int tw[NS + 1];
#pragma unroll
  for (int k = 0; k <= NS; ++k) tw[k] = SPARSE ? tile_at(k - 1) : 0;
  int tnext = 0;  // tile_at(i + NS), read in period i
  auto advance = [&]() __attribute__((always_inline)) {
    if constexpr (SPARSE) {
#pragma unroll
      for (int k = 0; k < NS; ++k) tw[k] = tw[k + 1];
      tw[NS] = tnext;
    }
  };
  // workspace tile of loop tile j - 1 + k in period j
  auto tile_k = [&](int k, int j) __attribute__((always_inline)) { return SPARSE ? tw[k] : tile_at(j - 1 + k); };

  // GEMM phase of tile jj: O^T += V_{jj-1}^T P^T (PV), S'^T = K_jj Q'^T - m (SC).
  // The operands (16 B per lane each) stream from LDS in batches of RB,
  // double-buffered in registers: batch b+1 is read while the MFMAs of
  // batch b run, so each MFMA finds its operand already loaded. (Measured:
  // batches of 4 suit the dense kernel, 0.4 % ahead of 2; the list-driven
  // variants run 2 % faster with batches of 2.)
  constexpr int RB = SPARSE ? 2 : 4;
  struct Batch {
    u32x4 v[RB];
    const uint8_t* st;  // the stage the batch was read from
  };
  // one register holds this lane's address in the stage; the operand
  // offsets (< 32 KB) then fit the ds_read immediate field
  auto stage_ptr = [&](int jj) __attribute__((always_inline)) {
    uint32_t sb = (uint32_t)(uintptr_t)(lds + (jj % NS) * STAGE + lane * 16);
    asm volatile("" : "+v"(sb));
    return (const uint8_t*)(__attribute__((address_space(3))) const uint8_t*)(uintptr_t)sb;
  };
  // The first operand batch of a GEMM phase with the P.V product (V blocks
  // 0 .. RB-1). Group B reads it right after the barrier, ahead of its
  // softmax, so that its GEMM phase starts without an LDS wait.
  auto first_batch = [&](int jj) __attribute__((always_inline)) {
    const uint8_t* st = stage_ptr(jj);
    Batch b;
    b.st = st;
#pragma unroll
    for (int r = 0; r < RB; ++r) b.v[r] = *reinterpret_cast<const u32x4*>(st + TILE + r * 1024);
    __builtin_amdgcn_sched_barrier(0);  // issue the reads before what follows
    return b;
  };
  // GEMM phase of tile jj: O^T += V_{jj-1}^T P^T (PV), S'^T = K_jj Q'^T - m
  // (SC). SUM: add the row sums of the P being multiplied to l (in the shadow
  // of the MFMAs). PRE: the first operand batch was read ahead (pre).
  auto gemm = [&](auto PV, auto SC, int jj, auto SUM, auto PRE, const Batch& pre) __attribute__((always_inline)) {
    const uint8_t* st = decltype(PRE)::value ? pre.st : stage_ptr(jj);
    constexpr int NV = decltype(PV)::value ? DB * MS : 0;   // V^T operand blocks
    constexpr int NK = decltype(SC)::value ? NKB * KS : 0;  // K operand blocks
    constexpr int NOP = NV + NK;
    static_assert(NOP % RB == 0, "operand batches");
    constexpr int NB = NOP / RB;
    // scheduling groups that keep the batch structure of batches b0 .. b1:
    // the reads of batch b + 1, then the MFMAs of batch b (two per operand)
    constexpr bool kBox = WIN == kWinPatch && decltype(SC)::value;
    auto groups = [&](int b0, int b1) __attribute__((always_inline)) {
      for (int b = b0; b <= b1; ++b) {
        if (b + 1 < NB) __builtin_amdgcn_sched_group_barrier(0x100, RB, 0);  // DS read
        __builtin_amdgcn_sched_group_barrier(0x008, 2 * RB, 0);  // MFMA
      }
    };
    // Operand i < NV is V block i = (s, db) (db fastest, workspace order),
    // else K block kbs(i - NV) = (kb, s) (kb fastest). Each operand feeds
    // the two query halves; consecutive V blocks share their P operand.
    // Every accumulator still sums in head-dim (K) or key (V) order.
    auto kbs = [&](int i) __attribute__((always_inline)) { return (i % NKB) * KS + i / NKB; };
    auto addr = [&](int i) __attribute__((always_inline)) {
      return st + (i < NV ? TILE + i * 1024 : kbs(i - NV) * 1024);
    };
    // accumulator input of the first score MFMA of key block kb and half h:
    // -m, or -inf for a key outside the window (sign-extended bit, then a bit
    // select), formed right before that MFMA so that only the window bits
    // stay live through the P.V products
    if constexpr (kBox) wvis = vis_sc;
    if constexpr (WIN == kWinRows && decltype(SC)::value) wvis = window_vis(tw[1]);
    auto cneg = [&](int kb, int h) __attribute__((always_inline)) {
      f32x4 c;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const unsigned keep = (unsigned)((int)(wvis << (31 - (16 * h + 4 * kb + i))) >> 31);
        const float mv = negm[h][i];  // (bit-casting the element expression itself reads element 0)
        const unsigned mb = __builtin_bit_cast(unsigned, mv);
        c[i] = __builtin_bit_cast(float, (mb & keep) | (0xff800000u & ~keep));
      }
      return c;
    };
    // Patch layout: the box products run first, as a fenced group, so that
    // the P.V products stand between them and the score products that take
    // their results as accumulator input (a phase without P.V products waits
    // 32 cycles instead). With a 16x16x16 box product and a 16x16x32 score
    // product next to each other on one accumulator register (written, then
    // read as accumulator input one instruction later, or read, then
    // overwritten), the scores came out wrong on gfx950, and the compiler
    // inserted no wait states there; tests/test_sources.py checks the
    // generated code for such pairs.
    if constexpr (kBox) {
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int k2 = 0; k2 < NKB; ++k2)
#pragma unroll
        for (int h = 0; h < 2; ++h)
          sacc[k2][h] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(onehot[k2], pen_sc[h], negm[h], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (NV == 0) asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7");
      __builtin_amdgcn_sched_barrier(0);
    }
    u32x4 buf[2][RB];
#pragma unroll
    for (int r = 0; r < RB; ++r) buf[0][r] = decltype(PRE)::value ? pre.v[r] : *reinterpret_cast<const u32x4*>(addr(r));
#pragma unroll
    for (int b = 0; b < NOP / RB; ++b) {
      if (b + 1 < NOP / RB) {
#pragma unroll
        for (int r = 0; r < RB; ++r) buf[(b + 1) & 1][r] = *reinterpret_cast<const u32x4*>(addr((b + 1) * RB + r));
      }
#pragma unroll
      for (int r = 0; r < RB; ++r) {
        const int i = b * RB + r;
        const u32x4 a = buf[b & 1][r];
        if (i < NV) {
          const int db = i % DB, s = i / DB;
#pragma unroll
          for (int h = 0; h < 2; ++h)
            oacc[db][h] =
                __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), pk[s][h], oacc[db][h], 0, 0, 0);
        } else {
          const int kb = (i - NV) % NKB, s = (i - NV) / NKB;
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            f32x4 c0 = s == 0 ? negm[h] : sacc[kb][h];
            if constexpr (WIN == kWinPatch) c0 = sacc[kb][h];
            if constexpr (WIN == kWinRows)
              if (s == 0) c0 = cneg(kb, h);
            sacc[kb][h] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, a), qreg[s][h], c0, 0, 0, 0);
          }
        }
      }
    }
    if constexpr (decltype(SUM)::value) rowsum();
    // keep the batch structure: the first RB reads up front (unless read
    // ahead), then per batch the next RB reads and this batch's MFMAs
    if constexpr (!decltype(PRE)::value) __builtin_amdgcn_sched_group_barrier(0x100, RB, 0);
    groups(0, NB - 1);
  };

  // In the last key tile, keys past N get -inf.
  auto tail_mask = [&](int t) __attribute__((always_inline)) {
    if (tail < KT && t == nkt - 1) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = score_key(kb, 4 * r4 + i);
#pragma unroll
          for (int h = 0; h < 2; ++h)
            if (key >= tail) sacc[kb][h][i] = -INFINITY;
        }
    }
  };
  // SOFTMAX phase of the scores of workspace tile t. SUM: add the row sums
  // to l here (else the next GEMM phase does).
  auto softmax = [&](int t, auto SUM) __attribute__((always_inline)) {
    tail_mask(t);
    const bool big = (probs() & 0x40004000u) != 0u;  // some p >= 2 (or not finite)
    // the exact step: for a row's first tile with a visible key (a row with
    // no visible key in this tile keeps m unset), and when a score lies more
    // than kBias + 1 above m
    const bool first = (!m_valid[0] && (wvis & 0xFFFFu) != 0u) || (!m_valid[1] && (wvis >> 16) != 0u);
    if (__builtin_amdgcn_ballot_w64(first || big) != 0) {
      rescale_to_tile_max();
      probs();
    }
    if constexpr (decltype(SUM)::value) rowsum();
  };
  using T = std::true_type;
  using F = std::false_type;
  // One barrier per tile period i; within it group A runs GEMM_i then
  // SOFTMAX_i and group B runs SOFTMAX_{i-1} then GEMM_i, so on every SIMD
  // the matrix core and the vector ALU serve different waves.
  //   A: [b0] G_0 S_0 [b1] G_1 S_1 ... [b(T-1)] G_T-1 S_T-1 [bT] G_T(P.V)
  //   B: [b0] G_0     [b1] S_0 G_1 ... [b(T-1)] S_T-2 G_T-1 [bT] S_T-1 G_T(P.V)
  // Period i refills the ring with tile i+NS-1 while that is <= nkt (the
  // "refill" loops below; the "drain" loops follow). The waves of group A
  // issue it at the start of their softmax phase: group B's softmax runs
  // beside group A's GEMM phase, gets few vector issue slots there and is
  // the longer path through the period, so in the dense kernel it carries
  // none of the refill (sparse variants: its share, at the period start).
  // Softmax phase of workspace tile t in period i: the refill of tile
  // fill_tile (FILL), the list read for period i + 1, then the softmax
  // itself, during which the read lands. The scheduling barrier keeps the
  // list read out of the GEMM phase before.
  auto prefetch = [&](int i) __attribute__((always_inline)) {
    if constexpr (SPARSE) tnext = tile_at(i + NS);
  };
  // (scores: the wave needs tile t; else its probabilities are set to 0,
  // which is what the softmax would give, so a P.V product that still runs
  // adds exact zeros)
  auto sm = [&](bool fill, int t, int fill_tile, int i, auto SUM, bool scores) __attribute__((always_inline)) {
    if constexpr (SPARSE) __builtin_amdgcn_sched_barrier(0);
    if (fill) issue(fill_tile, tile_k(NS, i), tile_k(NS - 1, i));
    prefetch(i);
    if (scores) {
      softmax(t, SUM);
    } else {
#pragma unroll
      for (int s = 0; s < MS; ++s)
#pragma unroll
        for (int h = 0; h < 2; ++h) pk[s][h] = bf16x8{};
    }
  };
  // before a GEMM phase that no barrier precedes: no list read in flight
  auto lists_landed = [&]() __attribute__((always_inline)) {
    if constexpr (SPARSE) {
      constexpr int kLgkm0 = 0xF | (0x3 << 14) | (0x7 << 4);
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_waitcnt(kLgkm0);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  const Batch nob{};
  tile_barrier(0);
  // Patch layout: a wave skips a tile none of its queries sees. pv: the wave
  // needs the tile whose probabilities are in pk (its P.V product is still
  // to come); sc: it needs the tile of this period's score product. A GEMM
  // phase runs when either holds (the other half then multiplies zeros or
  // scores a hidden tile); a softmax runs when its tile is needed. need()
  // makes every test constant outside the patch layout.
  auto need = [](bool b) __attribute__((always_inline)) { return WIN != kWinPatch || b; };
  bool pv = false;
  if (group == 0) {  // period i: GEMM_i then SOFTMAX_i (with the row sums)
    {
      const bool sc = prep_scores(tile_k(1, 0));
      if (need(sc)) gemm(F{}, T{}, 0, F{}, F{}, nob);
      sm(NS - 1 <= nt, tile_k(1, 0), NS - 1, 0, T{}, need(sc));
      pv = sc;
    }
    // one loop for the refill periods and the drain periods (a uniform
    // branch skips the refill), so the accumulators keep one set of
    // registers throughout
    for (int j = 1; j < nt; ++j) {
      advance();
      tile_barrier(j);
      const bool sc = prep_scores(tile_k(1, j));
      if (need(pv || sc)) gemm(T{}, T{}, j, F{}, F{}, nob);
      sm(j + NS - 1 <= nt, tile_k(1, j), j + NS - 1, j, T{}, need(sc));
      pv = sc;
    }
    tile_barrier(nt);
    if (need(pv)) gemm(T{}, F{}, nt, F{}, F{}, nob);
  } else {  // period i: SOFTMAX_{i-1} then GEMM_i (period 0: GEMM_0 only)
    // Group B's softmax is the longer path through a period: it reads its
    // first GEMM operands before it, and leaves its row sums to the GEMM
    // phase that follows (where they run in the shadow of its MFMAs).
    if constexpr (kFillB) {
      if (NS - 1 <= nt) issue(NS - 1, tile_k(NS, 0), tile_k(NS - 1, 0));
      __builtin_amdgcn_sched_barrier(0);
    }
    prefetch(0);
    lists_landed();
    {
      const bool sc = prep_scores(tile_k(1, 0));
      if (need(sc)) gemm(F{}, T{}, 0, F{}, F{}, nob);
      pv = sc;
    }
    int j = 1;
    auto period_b = [&](int jj) __attribute__((always_inline)) {
      if constexpr (WIN == kWinPatch) {
        const bool sc = prep_scores(tile_k(1, jj));
        const bool run = pv || sc;
        Batch pre{};
        if (run) pre = first_batch(jj);
        sm(false, tile_k(0, jj), 0, jj, F{}, pv);
        lists_landed();
        if (run) gemm(T{}, T{}, jj, T{}, T{}, pre);
        pv = sc;
      } else {
        const Batch pre = first_batch(jj);
        sm(false, tile_k(0, jj), 0, jj, F{}, true);
        lists_landed();
        gemm(T{}, T{}, jj, T{}, T{}, pre);
      }
    };
    if constexpr (kFillB) {
      for (; j < nt && j + NS - 1 <= nt; ++j) {
        advance();
        tile_barrier(j);
        issue(j + NS - 1, tile_k(NS, j), tile_k(NS - 1, j));
        __builtin_amdgcn_sched_barrier(0);  // the refill share ahead of the softmax arithmetic
        period_b(j);
      }
    }
    for (; j < nt; ++j) {
      advance();
      tile_barrier(j);
      period_b(j);
    }
    advance();
    tile_barrier(nt);
    if (need(pv)) {
      const Batch pre = first_batch(nt);
      softmax(tile_k(0, nt), F{});
      gemm(T{}, F{}, nt, T{}, T{}, pre);
    }
  }

  // ---- epilogue: O = O^T / l, rounded to bf16.
  // Output register i of lane (qi, r) in head-dim block db of half h is
  // d = 16db + 4r + i of query 16h + qi.
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const float inv = 1.0f / xor32_sum(xor16_sum(l[h]));
    if (qvalid[h]) {
      uint16_t* orow = O + ((int64_t)bh * Nq + qtok[h]) * D;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        bf16x4 v;
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = (__bf16)(oacc[db][h][i] * inv);
        *reinterpret_cast<bf16x4*>(orow + 16 * db + 4 * r4) = v;
      }
    }
  }
}

}  // namespace vidattn
