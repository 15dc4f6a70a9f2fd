// Key-tile lists of the local-window attention: for each block of 256
// queries, the 64-key tiles that intersect the union of its queries'
// windows. A window is the box of radii (r_f, r_h, r_w) around a query's
// grid position (frame-major token order n = (f*H + y)*W + x). The list is
// a superset per query (whole rows of each frame in range); the attention
// kernel masks the keys outside each query's own box.
#pragma once

#include "common.hpp"

namespace vidattn {

// One thread per query block i: kv_count[i] and kv_blocks[i*cap ..] (ascending,
// at most cap entries; cap >= the number of key tiles).
__global__ __launch_bounds__(256) void window_plan_kernel(int32_t* __restrict__ kv_blocks,
                                                          int32_t* __restrict__ kv_count, int N, int nqb, int cap,
                                                          int F, int H, int W, int rf, int rh) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= nqb) return;
  const int hw = H * W;
  const int q0 = i * 256, q1 = (q0 + 256 < N ? q0 + 256 : N) - 1;
  const int fa = q0 / hw, fb = q1 / hw;
  int ya = 0, yb = H - 1;  // rows the block's queries occupy (all rows when it spans frames)
  if (fa == fb) {
    ya = (q0 - fa * hw) / W;
    yb = (q1 - fb * hw) / W;
  }
  const int f0 = fa - rf < 0 ? 0 : fa - rf, f1 = fb + rf > F - 1 ? F - 1 : fb + rf;
  const int y0 = ya - rh < 0 ? 0 : ya - rh, y1 = yb + rh > H - 1 ? H - 1 : yb + rh;
  int n = 0, last = -1;
  int32_t* out = kv_blocks + (int64_t)i * cap;
  for (int f = f0; f <= f1; ++f) {
    const int t0 = ((f * H + y0) * W) / 64, t1 = ((f * H + y1) * W + W - 1) / 64;
    for (int t = t0 > last ? t0 : last + 1; t <= t1 && n < cap; ++t) out[n++] = t;
    last = t1 > last ? t1 : last;
  }
  kv_count[i] = n;
}

}  // namespace vidattn
