// Key-tile lists of the local-window attention: for each query block, the
// 64-key tiles that can hold a key inside the window of one of its queries.
// A window is the box of radii (r_f, r_h, r_w) around a query's grid
// position (frame-major token order n = (f*H + y)*W + x). The lists are a
// superset per query; the attention kernel masks the keys outside each
// query's own box.
//
// Two layouts of queries and keys:
//   row order    query block i is tokens 256i .. 256i+255 and key tile t is
//                tokens 64t .. 64t+63; the list holds whole grid rows;
//   patch order  query block b is the 16 x 16 patch (f, py, px) of one frame
//                and key tile t the 8 x 8 patch (tf, ty, tx), so a block's
//                list follows the box in all three axes.
#pragma once

#include "common.hpp"

namespace vidattn {

// Row order: the tiles of query block i, as ascending, disjoint ranges
// [t0, t1] passed to range(t0, t1); host and device share this rule.
//
// The block's queries occupy rows ya..H-1 of frame fa, every row of the
// frames strictly between, and rows 0..yb of frame fb (ya..yb when fa == fb).
// Key frame f sees the query frames within r_f of it; its rows are those
// within r_h of their rows: all rows if one of them is a middle frame, else
// [ya - r_h, H-1] for fa and [0, yb + r_h] for fb, listed as two ranges
// (lower rows first) when both apply and they do not touch.
template <class Range>
__host__ __device__ inline void window_rows_plan(int i, int N, int F, int H, int W, int rf, int rh, Range range) {
  const int hw = H * W;
  const int q0 = i * 256, q1 = (q0 + 256 < N ? q0 + 256 : N) - 1;
  const int fa = q0 / hw, fb = q1 / hw;
  const int ya = (q0 - fa * hw) / W, yb = (q1 - fb * hw) / W;
  const int f0 = fa - rf < 0 ? 0 : fa - rf, f1 = fb + rf > F - 1 ? F - 1 : fb + rf;
  int last = -1;
  auto emit = [&](int f, int lo, int hi) {  // the tiles of rows lo..hi of frame f
    lo = lo < 0 ? 0 : lo;
    hi = hi > H - 1 ? H - 1 : hi;
    if (lo > hi) return;
    const int t0 = ((f * H + lo) * W) / 64, t1 = ((f * H + hi) * W + W - 1) / 64;
    const int a = t0 > last ? t0 : last + 1;
    if (a <= t1) range(a, t1);
    last = t1 > last ? t1 : last;
  };
  for (int f = f0; f <= f1; ++f) {
    const int ga = fa > f - rf ? fa : f - rf, gb = fb < f + rf ? fb : f + rf;  // query frames within reach
    const int ma = ga > fa + 1 ? ga : fa + 1, mb = gb < fb - 1 ? gb : fb - 1;
    if (ma <= mb) {  // a middle frame: all its rows hold queries
      emit(f, 0, H - 1);
    } else if (fa == fb) {
      emit(f, ya - rh, yb + rh);
    } else if (ga == fa && gb == fb) {  // both end frames
      if (yb + rh >= ya - rh - 1) {
        emit(f, 0, H - 1);
      } else {
        emit(f, 0, yb + rh);
        emit(f, ya - rh, H - 1);
      }
    } else if (ga == fa) {
      emit(f, ya - rh, H - 1);
    } else {
      emit(f, 0, yb + rh);
    }
  }
}

// One thread per query block i: kv_count[i] and kv_blocks[i*cap ..] (ascending,
// at most cap entries; the host sets cap to the most tiles any block lists).
__global__ __launch_bounds__(256) void window_plan_kernel(int32_t* __restrict__ kv_blocks,
                                                          int32_t* __restrict__ kv_count, int N, int nqb, int cap,
                                                          int F, int H, int W, int rf, int rh) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= nqb) return;
  int n = 0;
  int32_t* out = kv_blocks + (int64_t)i * cap;
  window_rows_plan(i, N, F, H, W, rf, rh, [&](int t0, int t1) {
    for (int t = t0; t <= t1 && n < cap; ++t) out[n++] = t;
  });
  kv_count[i] = n;
}

// Patch order: the axis ranges of key patches that query patch p (16
// queries wide) of an axis of extent n reaches with radius r, as tile
// indices [lo, hi] of 8-wide tiles.
__host__ __device__ inline void window_patch_span(int p, int n, int r, int& lo, int& hi) {
  const int a = 16 * p - r, b = (16 * p + 15 < n - 1 ? 16 * p + 15 : n - 1) + r;
  lo = (a < 0 ? 0 : a) / 8;
  hi = (b > n - 1 ? n - 1 : b) / 8;
}

// One thread per query patch b = (f*pyn + py)*pxn + px: every key patch of
// frames f - r_f .. f + r_f whose rows and columns meet the box of the
// patch's windows, frame-major (ascending tile index), at most cap entries.
__global__ __launch_bounds__(256) void window_plan_patch_kernel(int32_t* __restrict__ kv_blocks,
                                                                int32_t* __restrict__ kv_count, int nqb, int cap,
                                                                int F, int H, int W, int rf, int rh, int rw, int tyn,
                                                                int txn, int pyn, int pxn) {
  const int b = blockIdx.x * 256 + threadIdx.x;
  if (b >= nqb) return;
  const int px = b % pxn, py = (b / pxn) % pyn, f = b / (pxn * pyn);
  int ylo, yhi, xlo, xhi;
  window_patch_span(py, H, rh, ylo, yhi);
  window_patch_span(px, W, rw, xlo, xhi);
  const int f0 = f - rf < 0 ? 0 : f - rf, f1 = f + rf > F - 1 ? F - 1 : f + rf;
  int n = 0;
  int32_t* out = kv_blocks + (int64_t)b * cap;
  for (int tf = f0; tf <= f1; ++tf)
    for (int ty = ylo; ty <= yhi; ++ty)
      for (int tx = xlo; tx <= xhi && n < cap; ++tx) out[n++] = (tf * tyn + ty) * txn + tx;
  kv_count[b] = n;
}

}  // namespace vidattn
