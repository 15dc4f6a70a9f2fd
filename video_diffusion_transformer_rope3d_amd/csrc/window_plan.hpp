// Key-tile lists of the local-window attention: for each block of 256
// queries, the 64-key tiles that intersect the union of its queries'
// windows. A window is the box of radii (r_f, r_h, r_w) around a query's
// grid position (frame-major token order n = (f*H + y)*W + x). The list is
// a superset per query (whole rows: every row within r_h of a row that the
// block's queries of a frame within r_f occupy); the attention kernel masks
// the keys outside each query's own box.
#pragma once

#include "common.hpp"

namespace vidattn {

// One thread per query block i: kv_count[i] and kv_blocks[i*cap ..] (ascending,
// at most cap entries; cap >= the number of key tiles).
//
// The block's queries occupy rows ya..H-1 of frame fa, every row of the
// frames strictly between, and rows 0..yb of frame fb (ya..yb when fa == fb).
// Key frame f sees the query frames within r_f of it; its rows are those
// within r_h of their rows: all rows if one of them is a middle frame, else
// [ya - r_h, H-1] for fa and [0, yb + r_h] for fb, listed as two ranges
// (lower rows first) when both apply and they do not touch.
__global__ __launch_bounds__(256) void window_plan_kernel(int32_t* __restrict__ kv_blocks,
                                                          int32_t* __restrict__ kv_count, int N, int nqb, int cap,
                                                          int F, int H, int W, int rf, int rh) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= nqb) return;
  const int hw = H * W;
  const int q0 = i * 256, q1 = (q0 + 256 < N ? q0 + 256 : N) - 1;
  const int fa = q0 / hw, fb = q1 / hw;
  const int ya = (q0 - fa * hw) / W, yb = (q1 - fb * hw) / W;
  const int f0 = fa - rf < 0 ? 0 : fa - rf, f1 = fb + rf > F - 1 ? F - 1 : fb + rf;
  int n = 0, last = -1;
  int32_t* out = kv_blocks + (int64_t)i * cap;
  auto emit = [&](int f, int lo, int hi) {  // the tiles of rows lo..hi of frame f
    lo = lo < 0 ? 0 : lo;
    hi = hi > H - 1 ? H - 1 : hi;
    if (lo > hi) return;
    const int t0 = ((f * H + lo) * W) / 64, t1 = ((f * H + hi) * W + W - 1) / 64;
    for (int t = t0 > last ? t0 : last + 1; t <= t1 && n < cap; ++t) out[n++] = t;
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
  kv_count[i] = n;
}

}  // namespace vidattn
