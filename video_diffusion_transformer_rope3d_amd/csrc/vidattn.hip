// libvidattn: C ABI entry points (declared and documented in include/vidattn.h).
// Host side: argument validation (before any HIP call), rotary parameter
// setup, workspace sizing and kernel launches on the caller's stream.
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "vidattn.h"
#include "attn_bf16_pp.hpp"
#include "attn_f32.hpp"
#include "rope_kernels.hpp"
#include "window_plan.hpp"
#include "block_mask.hpp"

using namespace vidattn;

namespace {

thread_local std::string g_last_error;

vidattn_status fail(vidattn_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

vidattn_status ok() {
  g_last_error.clear();
  return VIDATTN_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t dtype_size(vidattn_dtype dt) {
  switch (dt) {
    case VIDATTN_BF16:
    case VIDATTN_F16:
      return 2;
    case VIDATTN_F32:
      return 4;
  }
  return 0;
}

bool mul_ok(int64_t a, int64_t b, int64_t* r) { return !__builtin_mul_overflow(a, b, r); }

// Limits that keep every in-kernel index within 32/64-bit range and the
// launch grid within the hardware's limits.
constexpr int64_t kMaxN = int64_t(1) << 24;
constexpr int64_t kMaxBH = int64_t(1) << 20;

// bf16 attention kernel: 8 waves of 32 queries per workgroup, a ring of
// VIDATTN_BF16_NS LDS stages of 64 keys (a compile-time tuning knob; the
// library ships three stages).
#ifndef VIDATTN_BF16_NS
#define VIDATTN_BF16_NS 3
#endif
constexpr int kKT = 64;  // keys per tile
constexpr int kNW = 8;   // waves per workgroup
constexpr int kQB = 1;   // 32-query blocks per wave
constexpr int kBR = kNW * kQB * 32;

vidattn_status check_rope(const vidattn_rope3d_desc* r, int64_t d, int64_t N_expected, bool check_n) {
  if (r->F < 1 || r->H < 1 || r->W < 1)
    return fail(VIDATTN_ERR_INVALID_ARG, "rope grid extents must be >= 1 (got %lld x %lld x %lld)", (long long)r->F,
                (long long)r->H, (long long)r->W);
  int64_t hw, fhw;
  if (!mul_ok(r->H, r->W, &hw) || !mul_ok(r->F, hw, &fhw) || fhw > kMaxN)
    return fail(VIDATTN_ERR_INVALID_ARG, "rope grid F*H*W overflows or exceeds %lld tokens", (long long)kMaxN);
  if (check_n && fhw != N_expected)
    return fail(VIDATTN_ERR_INVALID_ARG, "rope grid F*H*W = %lld does not equal N = %lld", (long long)fhw,
                (long long)N_expected);
  if (r->d_t < 0 || r->d_h < 0 || r->d_w < 0 || (r->d_t & 1) || (r->d_h & 1) || (r->d_w & 1))
    return fail(VIDATTN_ERR_INVALID_ARG, "rope split %d/%d/%d must be even, non-negative widths", r->d_t, r->d_h,
                r->d_w);
  if ((int64_t)r->d_t + r->d_h + r->d_w != d)
    return fail(VIDATTN_ERR_INVALID_ARG, "rope split %d+%d+%d does not sum to head dim %lld", r->d_t, r->d_h,
                r->d_w, (long long)d);
  if (!std::isfinite(r->theta) || !(r->theta > 0.0))
    return fail(VIDATTN_ERR_INVALID_ARG, "rope theta must be finite and > 0");
  return VIDATTN_OK;
}

RopeParams make_rope(const vidattn_rope3d_desc* r) {
  RopeParams p;
  std::memset(&p, 0, sizeof p);
  if (!r) return p;
  p.enabled = 1;
  p.F = (int)r->F;
  p.H = (int)r->H;
  p.W = (int)r->W;
  p.pair_t = r->d_t / 2;
  p.pair_th = (r->d_t + r->d_h) / 2;
  int k = 0;
  const int widths[3] = {r->d_t, r->d_h, r->d_w};
  for (int a = 0; a < 3; ++a)
    for (int j = 0; j < widths[a] / 2; ++j) p.omega[k++] = std::pow(r->theta, -2.0 * j / widths[a]);
  return p;
}

vidattn_status hip_check(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(VIDATTN_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return VIDATTN_OK;
}

int bh_group(int64_t items_blocks, int64_t nbh) {
  // Reuse each block's cos/sin over several (b, head) slices while keeping
  // at least ~4 blocks per CU in flight. Four slices per block measured best
  // for the K/V pre-pass at 2 x 40 x 75600 x 128 (1.12 ms, against 1.16 at
  // two or eight, 1.19 at sixteen and 1.44 at one).
  int g = 4;
  while (g > 1 && items_blocks * ((nbh + g - 1) / g) < 1024) g >>= 1;
  // keep the grid's y extent within 65535 for any number of slices
  while ((nbh + g - 1) / g > 65535) g <<= 1;
  return g;
}

}  // namespace

extern "C" {

int vidattn_abi_version(void) { return VIDATTN_ABI_VERSION; }

const char* vidattn_status_string(vidattn_status s) {
  switch (s) {
    case VIDATTN_OK:
      return "ok";
    case VIDATTN_ERR_INVALID_ARG:
      return "invalid argument";
    case VIDATTN_ERR_UNSUPPORTED:
      return "unsupported";
    case VIDATTN_ERR_WORKSPACE:
      return "workspace too small";
    case VIDATTN_ERR_HIP:
      return "HIP error";
  }
  return "unknown status";
}

const char* vidattn_last_error(void) { return g_last_error.c_str(); }

size_t vidattn_fwd_workspace_size(vidattn_dtype dt, int64_t B, int64_t heads, int64_t N, int64_t d, int use_rope) {
  if (B < 1 || heads < 1 || N < 1 || N > kMaxN || (d != 64 && d != 128)) return 0;
  int64_t nbh;
  if (!mul_ok(B, heads, &nbh) || nbh > kMaxBH) return 0;
  if (dt == VIDATTN_BF16) {
    const int64_t npad = (N + kKT - 1) / kKT * kKT;
    return (size_t)(4 * nbh * npad * d);
  }
  if (dt == VIDATTN_F32) return use_rope ? (size_t)(4 * nbh * N * d) : 0;
  return 0;
}

}  // extern "C"

namespace {

// The standalone rotation of n_tokens rows per (b, head) that are grid tokens
// token_offset .. token_offset + n_tokens - 1 (the whole grid: offset 0,
// F*H*W rows).
vidattn_status rope3d_rows(const void* in, vidattn_dtype in_dt, void* out, vidattn_dtype out_dt, int64_t B,
                           int64_t heads, int64_t n_tokens, int64_t token_offset, int64_t d,
                           const vidattn_rope3d_desc* rope, float prescale, void* hip_stream) {
  if (!in || !out || !rope) return fail(VIDATTN_ERR_INVALID_ARG, "in, out and rope must be non-null");
  if (!aligned16(in) || !aligned16(out)) return fail(VIDATTN_ERR_INVALID_ARG, "in and out must be 16-byte aligned");
  if (in_dt != VIDATTN_BF16 && in_dt != VIDATTN_F32)
    return fail(dtype_size(in_dt) ? VIDATTN_ERR_UNSUPPORTED : VIDATTN_ERR_INVALID_ARG,
                "input dtype must be BF16 or F32");
  if (!dtype_size(out_dt)) return fail(VIDATTN_ERR_INVALID_ARG, "unknown output dtype %d", (int)out_dt);
  if (B < 1 || heads < 1 || d < 1) return fail(VIDATTN_ERR_INVALID_ARG, "B, heads and d must be >= 1");
  int64_t nbh;
  if (!mul_ok(B, heads, &nbh) || nbh > kMaxBH)
    return fail(VIDATTN_ERR_INVALID_ARG, "B*heads overflows or exceeds %lld", (long long)kMaxBH);
  if ((d & 1) != 0) return fail(VIDATTN_ERR_INVALID_ARG, "head dim %lld must be even", (long long)d);
  if (d % 8 != 0 || d > 256)
    return fail(VIDATTN_ERR_UNSUPPORTED, "head dim %lld: rotation supports multiples of 8 up to 256", (long long)d);
  if (vidattn_status s = check_rope(rope, d, 0, false)) return s;
  if (!std::isfinite(prescale)) return fail(VIDATTN_ERR_INVALID_ARG, "prescale must be finite");
  const int64_t grid_n = rope->F * rope->H * rope->W;
  if (n_tokens < 1 || token_offset < 0 || token_offset > grid_n - n_tokens)
    return fail(VIDATTN_ERR_INVALID_ARG, "tokens %lld .. %lld + %lld lie outside the %lld-token grid",
                (long long)token_offset, (long long)token_offset, (long long)n_tokens, (long long)grid_n);
  const int64_t N = n_tokens;
  int64_t elems, bytes_in, bytes_out;
  if (!mul_ok(nbh, N * d, &elems) || !mul_ok(elems, (int64_t)dtype_size(in_dt), &bytes_in) ||
      !mul_ok(elems, (int64_t)dtype_size(out_dt), &bytes_out))
    return fail(VIDATTN_ERR_INVALID_ARG, "tensor size overflows");
  const char* ib = static_cast<const char*>(in);
  const char* ob = static_cast<const char*>(out);
  if (ib != ob && ib < ob + bytes_out && ob < ib + bytes_in)
    return fail(VIDATTN_ERR_INVALID_ARG, "in and out overlap without being the same buffer");
  if (ib == ob && dtype_size(in_dt) != dtype_size(out_dt))
    return fail(VIDATTN_ERR_INVALID_ARG, "in-place rotation needs equal input and output element sizes");

  const RopeParams rp = make_rope(rope);
  const int64_t items = N * (d / 8);
  const int64_t xblocks = (items + 255) / 256;
  const int grp = bh_group(xblocks, nbh);
  const dim3 grid((unsigned)xblocks, (unsigned)((nbh + grp - 1) / grp));
  hipStream_t st = static_cast<hipStream_t>(hip_stream);
#define VIDATTN_ROPE_LAUNCH(TI, TO)                                                                                 \
  hipLaunchKernelGGL((rope3d_kernel<TI, TO>), grid, dim3(256), 0, st, static_cast<const TI*>(in),                  \
                     static_cast<TO*>(out), nbh, (int)N, (int)token_offset, (int)d, prescale, grp, rp)
  if (in_dt == VIDATTN_BF16) {
    if (out_dt == VIDATTN_BF16) VIDATTN_ROPE_LAUNCH(uint16_t, uint16_t);
    else if (out_dt == VIDATTN_F16) VIDATTN_ROPE_LAUNCH(uint16_t, _Float16);
    else VIDATTN_ROPE_LAUNCH(uint16_t, float);
  } else {
    if (out_dt == VIDATTN_BF16) VIDATTN_ROPE_LAUNCH(float, uint16_t);
    else if (out_dt == VIDATTN_F16) VIDATTN_ROPE_LAUNCH(float, _Float16);
    else VIDATTN_ROPE_LAUNCH(float, float);
  }
#undef VIDATTN_ROPE_LAUNCH
  if (vidattn_status s = hip_check("rope3d launch")) return s;
  return ok();
}

}  // namespace

extern "C" {

vidattn_status vidattn_rope3d(const void* in, vidattn_dtype in_dt, void* out, vidattn_dtype out_dt, int64_t B,
                              int64_t heads, int64_t d, const vidattn_rope3d_desc* rope, float prescale,
                              void* hip_stream) {
  // the whole grid (a malformed descriptor is reported by the shared checks)
  int64_t hw = 0, n = 0;
  if (rope && rope->F >= 1 && rope->H >= 1 && rope->W >= 1 &&
      !(mul_ok(rope->H, rope->W, &hw) && mul_ok(rope->F, hw, &n)))
    n = 0;
  return rope3d_rows(in, in_dt, out, out_dt, B, heads, n, 0, d, rope, prescale, hip_stream);
}

vidattn_status vidattn_rope3d_tokens(const void* in, vidattn_dtype in_dt, void* out, vidattn_dtype out_dt, int64_t B,
                                     int64_t heads, int64_t n_tokens, int64_t token_offset, int64_t d,
                                     const vidattn_rope3d_desc* rope, float prescale, void* hip_stream) {
  return rope3d_rows(in, in_dt, out, out_dt, B, heads, n_tokens, token_offset, d, rope, prescale, hip_stream);
}

}  // extern "C"

namespace {

enum class Phase { kFused, kPrepare, kAttend };

// Shared argument checks of the three forward entry points; pointers that a
// phase does not take are passed as a non-null placeholder.
vidattn_status validate_fwd(Phase ph, const void* q, const void* k, const void* v, const void* o, vidattn_dtype dt,
                            int64_t B, int64_t heads, int64_t N, int64_t d, float softmax_scale,
                            const vidattn_rope3d_desc* rope, const void* workspace, size_t workspace_bytes,
                            int64_t Nq = -1, size_t extra_workspace = 0) {
  if (Nq < 0) Nq = N;  // rows of q and o (a query subset may have fewer or more than the N keys)
  if (!q || !k || !v || !o) return fail(VIDATTN_ERR_INVALID_ARG, "q, k, v and o must be non-null");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
    return fail(VIDATTN_ERR_INVALID_ARG, "q, k, v and o must be 16-byte aligned");
  if (dt != VIDATTN_BF16 && dt != VIDATTN_F32)
    return fail(dt == VIDATTN_F16 ? VIDATTN_ERR_UNSUPPORTED : VIDATTN_ERR_INVALID_ARG,
                "attention dtype must be BF16 or F32");
  if (B < 1 || heads < 1 || N < 1 || d < 1 || Nq < 1)
    return fail(VIDATTN_ERR_INVALID_ARG, "B, heads, N, Nq and d must be >= 1");
  int64_t nbh;
  if (!mul_ok(B, heads, &nbh) || nbh > kMaxBH)
    return fail(VIDATTN_ERR_INVALID_ARG, "B*heads overflows or exceeds %lld", (long long)kMaxBH);
  if (N > kMaxN || Nq > kMaxN)
    return fail(VIDATTN_ERR_UNSUPPORTED, "N = %lld or Nq = %lld exceeds %lld", (long long)N, (long long)Nq,
                (long long)kMaxN);
  if (d != 64 && d != 128) {
    if (d & 1) return fail(VIDATTN_ERR_INVALID_ARG, "head dim %lld must be even", (long long)d);
    return fail(VIDATTN_ERR_UNSUPPORTED, "head dim %lld: supported are 64 and 128", (long long)d);
  }
  if (ph != Phase::kPrepare && (!std::isfinite(softmax_scale) || !(softmax_scale > 0.f)))
    return fail(VIDATTN_ERR_INVALID_ARG, "softmax_scale must be finite and > 0");
  if (rope)
    if (vidattn_status s = check_rope(rope, d, N, true)) return s;
  const size_t need = vidattn_fwd_workspace_size(dt, B, heads, N, d, rope != nullptr) + extra_workspace;
  if (need > 0) {
    if (!workspace || workspace_bytes < need)
      return fail(VIDATTN_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given%s", need,
                  workspace ? workspace_bytes : (size_t)0, workspace ? "" : " (null)");
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
      return fail(VIDATTN_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  }
  const int64_t tensor_bytes = nbh * N * d * (int64_t)dtype_size(dt);
  const int64_t qo_bytes = nbh * Nq * d * (int64_t)dtype_size(dt);
  const char* w = static_cast<const char*>(workspace);
  if (ph != Phase::kPrepare) {
    const char* ob = static_cast<const char*>(o);
    const char* qb = static_cast<const char*>(q);
    if (qb < ob + qo_bytes && ob < qb + qo_bytes) return fail(VIDATTN_ERR_INVALID_ARG, "o overlaps q");
    const char* kv[2] = {static_cast<const char*>(k), static_cast<const char*>(v)};
    for (const char* p : kv)
      if (p != qb && p < ob + qo_bytes && ob < p + tensor_bytes)
        return fail(VIDATTN_ERR_INVALID_ARG, "o overlaps k or v");
    if (need > 0 && w < ob + qo_bytes && ob < w + (int64_t)need)
      return fail(VIDATTN_ERR_INVALID_ARG, "o overlaps the workspace");
    // the fused calls write the workspace (pre-pass, plans) before the
    // attention kernel reads q
    if (ph == Phase::kFused && need > 0 && w < qb + qo_bytes && qb < w + (int64_t)need)
      return fail(VIDATTN_ERR_INVALID_ARG, "q overlaps the workspace");
  }
  if (ph != Phase::kAttend && need > 0) {
    const char* ins[2] = {static_cast<const char*>(k), static_cast<const char*>(v)};
    for (const char* p : ins)
      if (p < w + (int64_t)need && w < p + tensor_bytes)
        return fail(VIDATTN_ERR_INVALID_ARG, "the workspace overlaps k or v");
  }
  if (dt == VIDATTN_BF16) {
    const int64_t ntq = (Nq + kBR - 1) / kBR;
    if (nbh * ntq > (int64_t)INT32_MAX / (kNW * 64))
      return fail(VIDATTN_ERR_UNSUPPORTED, "problem too large for one launch");
  } else {
    const int64_t ntq = (N + 127) / 128;
    if (nbh * ntq > (int64_t)INT32_MAX / 256) return fail(VIDATTN_ERR_UNSUPPORTED, "problem too large for one launch");
  }
  return VIDATTN_OK;
}

// Launch the key/value pre-pass (arguments already validated).
// map: the token order of the bf16 key tiles (row order unless given), with
// nkt tiles per (b, head).
vidattn_status launch_prepare(const void* k, const void* v, vidattn_dtype dt, int64_t nbh, int64_t N, int64_t d,
                              const RopeParams& rp, void* workspace, hipStream_t st,
                              const TileMap& map = TileMap{0, 1, 1, 1, 1}, int64_t nkt_map = 0) {
  if (dt == VIDATTN_BF16) {
    const int nkt = map.patch ? (int)nkt_map : (int)((N + kKT - 1) / kKT);
    const int grp = bh_group(nkt, nbh);
    const dim3 pgrid((unsigned)nkt, (unsigned)((nbh + grp - 1) / grp));
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    const uint16_t* kk = static_cast<const uint16_t*>(k);
    const uint16_t* vv = static_cast<const uint16_t*>(v);
    auto launch = [&](auto kernel) {
      hipLaunchKernelGGL(kernel, pgrid, dim3(256), 0, st, kk, vv, ws, (int)N, nkt, nbh, grp, rp, map);
    };
    if (d == 128)
      launch(map.patch ? prep_kv_kernel<128, true> : prep_kv_kernel<128, false>);
    else
      launch(map.patch ? prep_kv_kernel<64, true> : prep_kv_kernel<64, false>);
    return hip_check("bf16 key/value pre-pass launch");
  }
  if (!rp.enabled) return VIDATTN_OK;
  const int64_t xblocks = (N * (d / 8) + 255) / 256;
  const int grp = bh_group(xblocks, nbh);
  const dim3 grid((unsigned)xblocks, (unsigned)((nbh + grp - 1) / grp));
  hipLaunchKernelGGL((rope3d_kernel<float, float>), grid, dim3(256), 0, st, static_cast<const float*>(k),
                     static_cast<float*>(workspace), nbh, (int)N, 0, (int)d, 1.0f, grp, rp);
  return hip_check("f32 key rotation launch");
}

// Launch the attention kernel (arguments already validated).
// Optional inputs of the bf16 attention: a query subset (Nq rows with their
// token indices) and a block-sparse key-tile list.
struct AttendExtras {
  int64_t Nq = -1;  // -1: Nq = N
  const int32_t* qidx = nullptr;
  const int32_t* kvb = nullptr;  // non-null: block-sparse lists
  const int32_t* kvc = nullptr;
  int maxb = 0;
  int lists_shared = 0;  // one list per query block for every (b, head)
  bool window = false;   // mask keys outside each query's box
  bool patch = false;    // ... in the patch layout (else the row layout)
  WindowParams wp{1, 1, 1, 0, 0, 0, 0, 1.f, 1.f, 1, 1, 1, 1, 1.f, 1.f, 1.f, 1.f};
  int64_t nkt = 0, ntq = 0;  // > 0: key tiles and query blocks of the patch layout
};

template <int D, bool SPARSE, int WIN>
void launch_bf16(const void* q, const uint8_t* ws, void* o, int N, int nkt, int Nq, int ntq, int total, float qscale,
                 const RopeParams& rp, const AttendExtras& x, hipStream_t st) {
  hipLaunchKernelGGL((attn_fwd_bf16_pp_kernel<D, VIDATTN_BF16_NS, SPARSE, WIN>), dim3((unsigned)total),
                     dim3(kNW * 64), 0, st, static_cast<const uint16_t*>(q), ws, static_cast<uint16_t*>(o), N, nkt,
                     Nq, ntq, total, qscale, rp, x.qidx, x.kvb, x.kvc, x.maxb, x.lists_shared, x.wp);
}

vidattn_status launch_attend(const void* q, const void* k, const void* v, const void* workspace, void* o,
                             vidattn_dtype dt, int64_t nbh, int64_t N, int64_t d, float softmax_scale,
                             const RopeParams& rp, hipStream_t st, const AttendExtras& x = AttendExtras{}) {
  const float log2e = 1.4426950408889634f;
  const float qscale = softmax_scale * log2e;
  if (dt == VIDATTN_BF16) {
    const int64_t Nq = x.Nq < 0 ? N : x.Nq;
    const int nkt = x.nkt > 0 ? (int)x.nkt : (int)((N + kKT - 1) / kKT);
    const int ntq = x.ntq > 0 ? (int)x.ntq : (int)((Nq + kBR - 1) / kBR);
    const int total = (int)(nbh * ntq);
    const uint8_t* ws = static_cast<const uint8_t*>(workspace);
    const bool sparse = x.kvb != nullptr;
    const int n = (int)N, nq = (int)Nq;
    const bool patch = x.window && x.patch;
    if (d == 128) {
      if (patch)
        launch_bf16<128, true, kWinPatch>(q, ws, o, n, nkt, nq, ntq, total, qscale, rp, x, st);
      else if (x.window)
        launch_bf16<128, true, kWinRows>(q, ws, o, n, nkt, nq, ntq, total, qscale, rp, x, st);
      else if (sparse)
        launch_bf16<128, true, kWinNone>(q, ws, o, n, nkt, nq, ntq, total, qscale, rp, x, st);
      else
        launch_bf16<128, false, kWinNone>(q, ws, o, n, nkt, nq, ntq, total, qscale, rp, x, st);
    } else {
      if (patch)
        launch_bf16<64, true, kWinPatch>(q, ws, o, n, nkt, nq, ntq, total, qscale, rp, x, st);
      else if (x.window)
        launch_bf16<64, true, kWinRows>(q, ws, o, n, nkt, nq, ntq, total, qscale, rp, x, st);
      else if (sparse)
        launch_bf16<64, true, kWinNone>(q, ws, o, n, nkt, nq, ntq, total, qscale, rp, x, st);
      else
        launch_bf16<64, false, kWinNone>(q, ws, o, n, nkt, nq, ntq, total, qscale, rp, x, st);
    }
    return hip_check("bf16 attention launch");
  }
  const float* kk = rp.enabled ? static_cast<const float*>(workspace) : static_cast<const float*>(k);
  const int ntq = (int)((N + 127) / 128);
  const unsigned total = (unsigned)(nbh * ntq);
  if (d == 128)
    hipLaunchKernelGGL((attn_fwd_f32_kernel<128>), dim3(total), dim3(256), 0, st, static_cast<const float*>(q), kk,
                       static_cast<const float*>(v), static_cast<float*>(o), (int)N, ntq, qscale, rp);
  else
    hipLaunchKernelGGL((attn_fwd_f32_kernel<64>), dim3(total), dim3(256), 0, st, static_cast<const float*>(q), kk,
                       static_cast<const float*>(v), static_cast<float*>(o), (int)N, ntq, qscale, rp);
  return hip_check("f32 attention launch");
}

}  // namespace

extern "C" {

vidattn_status vidattn_fwd(const void* q, const void* k, const void* v, void* o, vidattn_dtype dt, int64_t B,
                           int64_t heads, int64_t N, int64_t d, float softmax_scale, const vidattn_rope3d_desc* rope,
                           void* workspace, size_t workspace_bytes, void* hip_stream) {
  if (vidattn_status s = validate_fwd(Phase::kFused, q, k, v, o, dt, B, heads, N, d, softmax_scale, rope, workspace,
                                      workspace_bytes))
    return s;
  const RopeParams rp = make_rope(rope);
  hipStream_t st = static_cast<hipStream_t>(hip_stream);
  if (vidattn_status s = launch_prepare(k, v, dt, B * heads, N, d, rp, workspace, st)) return s;
  if (vidattn_status s = launch_attend(q, k, v, workspace, o, dt, B * heads, N, d, softmax_scale, rp, st)) return s;
  return ok();
}

vidattn_status vidattn_fwd_prepare(const void* k, const void* v, vidattn_dtype dt, int64_t B, int64_t heads, int64_t N,
                                   int64_t d, const vidattn_rope3d_desc* rope, void* workspace, size_t workspace_bytes,
                                   void* hip_stream) {
  // q and o are not arguments of this phase: k stands in for both in the shared checks.
  if (vidattn_status s = validate_fwd(Phase::kPrepare, k, k, v, k, dt, B, heads, N, d, 1.0f, rope, workspace,
                                      workspace_bytes))
    return s;
  const RopeParams rp = make_rope(rope);
  if (vidattn_status s = launch_prepare(k, v, dt, B * heads, N, d, rp, workspace, static_cast<hipStream_t>(hip_stream)))
    return s;
  return ok();
}

vidattn_status vidattn_fwd_attend(const void* q, const void* k, const void* v, const void* workspace, void* o,
                                  vidattn_dtype dt, int64_t B, int64_t heads, int64_t N, int64_t d, float softmax_scale,
                                  const vidattn_rope3d_desc* rope, size_t workspace_bytes, void* hip_stream) {
  if (vidattn_status s = validate_fwd(Phase::kAttend, q, k, v, o, dt, B, heads, N, d, softmax_scale, rope, workspace,
                                      workspace_bytes))
    return s;
  const RopeParams rp = make_rope(rope);
  if (vidattn_status s = launch_attend(q, k, v, workspace, o, dt, B * heads, N, d, softmax_scale, rp,
                                       static_cast<hipStream_t>(hip_stream)))
    return s;
  return ok();
}

vidattn_status vidattn_fwd_attend_subset(const void* q, const int32_t* q_index, int64_t Nq, const void* workspace,
                                         void* o, vidattn_dtype dt, int64_t B, int64_t heads, int64_t N, int64_t d,
                                         float softmax_scale, const vidattn_rope3d_desc* rope, size_t workspace_bytes,
                                         void* hip_stream) {
  if (dt != VIDATTN_BF16)
    return fail(dt == VIDATTN_F32 || dt == VIDATTN_F16 ? VIDATTN_ERR_UNSUPPORTED : VIDATTN_ERR_INVALID_ARG,
                "query-subset attention is implemented for BF16");
  if (!q_index || (reinterpret_cast<uintptr_t>(q_index) & 3u) != 0)
    return fail(VIDATTN_ERR_INVALID_ARG, "q_index must be non-null and 4-byte aligned");
  // k and v are not arguments of this phase: q stands in for both in the shared checks.
  if (vidattn_status s = validate_fwd(Phase::kAttend, q, q, q, o, dt, B, heads, N, d, softmax_scale, rope, workspace,
                                      workspace_bytes, Nq))
    return s;
  const RopeParams rp = make_rope(rope);
  AttendExtras x;
  x.Nq = Nq;
  x.qidx = q_index;
  if (vidattn_status s = launch_attend(q, q, q, workspace, o, dt, B * heads, N, d, softmax_scale, rp,
                                       static_cast<hipStream_t>(hip_stream), x))
    return s;
  return ok();
}

vidattn_status vidattn_fwd_attend_block_sparse(const void* q, const void* workspace, void* o, vidattn_dtype dt,
                                               int64_t B, int64_t heads, int64_t N, int64_t d, float softmax_scale,
                                               const vidattn_rope3d_desc* rope, const int32_t* kv_blocks,
                                               const int32_t* kv_count, int64_t max_blocks, size_t workspace_bytes,
                                               void* hip_stream) {
  if (dt != VIDATTN_BF16)
    return fail(dt == VIDATTN_F32 || dt == VIDATTN_F16 ? VIDATTN_ERR_UNSUPPORTED : VIDATTN_ERR_INVALID_ARG,
                "block-sparse attention is implemented for BF16");
  if (!kv_blocks || !kv_count || (reinterpret_cast<uintptr_t>(kv_blocks) & 3u) != 0 ||
      (reinterpret_cast<uintptr_t>(kv_count) & 3u) != 0)
    return fail(VIDATTN_ERR_INVALID_ARG, "kv_blocks and kv_count must be non-null and 4-byte aligned");
  if (vidattn_status s = validate_fwd(Phase::kAttend, q, q, q, o, dt, B, heads, N, d, softmax_scale, rope, workspace,
                                      workspace_bytes))
    return s;
  const int64_t nkb = (N + VIDATTN_SPARSE_K_BLOCK - 1) / VIDATTN_SPARSE_K_BLOCK;
  if (max_blocks < 1 || max_blocks > nkb)
    return fail(VIDATTN_ERR_INVALID_ARG, "max_blocks = %lld must be in [1, ceil(N/%d) = %lld]", (long long)max_blocks,
                VIDATTN_SPARSE_K_BLOCK, (long long)nkb);
  static_assert(VIDATTN_SPARSE_K_BLOCK == kKT && VIDATTN_SPARSE_Q_BLOCK == kBR, "block sizes are the kernel's tiles");
  const RopeParams rp = make_rope(rope);
  AttendExtras x;
  x.kvb = kv_blocks;
  x.kvc = kv_count;
  x.maxb = (int)max_blocks;
  if (vidattn_status s = launch_attend(q, q, q, workspace, o, dt, B * heads, N, d, softmax_scale, rp,
                                       static_cast<hipStream_t>(hip_stream), x))
    return s;
  return ok();
}

// Tile lists built from a block bit mask, in the workspace tail after the
// prepared key/value image: counts [B*heads*nqb] (256-byte padded), then
// lists [B*heads*nqb][nkt].
static size_t block_mask_list_bytes(int64_t nbh, int64_t N) {
  const int64_t nqb = (N + kBR - 1) / kBR, nkt = (N + kKT - 1) / kKT;
  return (size_t)((nbh * nqb * 4 + 255) / 256 * 256 + nbh * nqb * nkt * 4);
}

// Layout of one local-window call and its tile counts (see
// vidattn_window_desc and window_plan.hpp). Its workspace: the key/value
// image of nkt tiles per (b, head), then the per-query-block tile counts
// (padded to 256 bytes), then the tile lists (nqb rows of cap entries, cap
// the most tiles any block lists, so the lists grow with N, not N^2).
struct WindowGeom {
  int layout = VIDATTN_WINDOW_ROWS;
  int64_t nkt = 0, nqb = 0;          // key tiles per (b, head), query blocks
  int64_t cap = 1;                   // entries per list row
  int tyn = 1, txn = 1, pyn = 1, pxn = 1;  // patch counts per axis (patch layout)
  int rf = 0, rh = 0, rw = 0;        // radii clipped to the grid
};

// Key tiles a layout lists: in all, and the most for one query block.
struct TileCount {
  int64_t total = 0, most = 0;
};

// The row layout (host count of window_plan_kernel's lists).
static TileCount rows_tiles_listed(int64_t N, int F, int H, int W, int rf, int rh) {
  const int nqb = (int)((N + kBR - 1) / kBR);
  TileCount c;
  for (int i = 0; i < nqb; ++i) {
    int64_t n = 0;
    window_rows_plan(i, (int)N, F, H, W, rf, rh, [&](int t0, int t1) { n += t1 - t0 + 1; });
    c.total += n;
    c.most = std::max(c.most, n);
  }
  return c;
}

// The patch layout: the count of patch (f, py, px) is the product of its
// frame, row and column spans, so the sum and the maximum factor.
static TileCount patch_tiles_listed(const WindowGeom& g, int F, int H, int W) {
  int64_t sf = 0, sy = 0, sx = 0, mf = 0, my = 0, mx = 0;
  for (int f = 0; f < F; ++f) {
    const int64_t n = std::min(F - 1, f + g.rf) - std::max(0, f - g.rf) + 1;
    sf += n;
    mf = std::max(mf, n);
  }
  for (int p = 0; p < g.pyn; ++p) {
    int lo, hi;
    window_patch_span(p, H, g.rh, lo, hi);
    sy += hi - lo + 1;
    my = std::max<int64_t>(my, hi - lo + 1);
  }
  for (int p = 0; p < g.pxn; ++p) {
    int lo, hi;
    window_patch_span(p, W, g.rw, lo, hi);
    sx += hi - lo + 1;
    mx = std::max<int64_t>(mx, hi - lo + 1);
  }
  return TileCount{sf * sy * sx, mf * my * mx};
}

// Checks the window against N and rope and resolves its layout.
static vidattn_status window_geom(const vidattn_window_desc* w, int64_t N, const vidattn_rope3d_desc* rope,
                                  WindowGeom* g) {
  if (!w) return fail(VIDATTN_ERR_INVALID_ARG, "window must be non-null");
  if (w->F < 1 || w->H < 1 || w->W < 1) return fail(VIDATTN_ERR_INVALID_ARG, "window grid extents must be >= 1");
  int64_t hw, fhw;
  if (!mul_ok(w->H, w->W, &hw) || !mul_ok(w->F, hw, &fhw) || fhw != N)
    return fail(VIDATTN_ERR_INVALID_ARG, "window grid F*H*W does not equal N = %lld", (long long)N);
  if (w->r_f < 0 || w->r_h < 0 || w->r_w < 0) return fail(VIDATTN_ERR_INVALID_ARG, "window radii must be >= 0");
  if (rope && (rope->F != w->F || rope->H != w->H || rope->W != w->W))
    return fail(VIDATTN_ERR_INVALID_ARG, "window and rotary grids differ");
  if (w->layout != VIDATTN_WINDOW_AUTO && w->layout != VIDATTN_WINDOW_ROWS && w->layout != VIDATTN_WINDOW_PATCHES)
    return fail(VIDATTN_ERR_INVALID_ARG, "window layout %d is not a VIDATTN_WINDOW_* value", (int)w->layout);
  // N <= kMaxN (checked by the caller) bounds every extent and count below
  const int F = (int)w->F, H = (int)w->H, W = (int)w->W;
  // a radius at or beyond the grid extent reaches the whole axis
  g->rf = (int)std::min<int64_t>(w->r_f, F);
  g->rh = (int)std::min<int64_t>(w->r_h, H);
  g->rw = (int)std::min<int64_t>(w->r_w, W);
  g->layout = VIDATTN_WINDOW_ROWS;
  g->nkt = (N + kKT - 1) / kKT;
  g->nqb = (N + kBR - 1) / kBR;
  const int tyn = (H + 7) / 8, txn = (W + 7) / 8, pyn = (H + 15) / 16, pxn = (W + 15) / 16;
  const int64_t pnkt = (int64_t)F * tyn * txn, pnqb = (int64_t)F * pyn * pxn;
  // the kernel decodes patch indices with an fp32 reciprocal split
  const bool patch_ok = pnkt < (int64_t(1) << 22) && pnqb < (int64_t(1) << 22);
  if (w->layout == VIDATTN_WINDOW_PATCHES && !patch_ok)
    return fail(VIDATTN_ERR_UNSUPPORTED, "patch layout needs fewer than 2^22 key and query patches");
  WindowGeom p = *g;
  p.layout = VIDATTN_WINDOW_PATCHES;
  p.nkt = pnkt;
  p.nqb = pnqb;
  p.tyn = tyn;
  p.txn = txn;
  p.pyn = pyn;
  p.pxn = pxn;
  const TileCount pc = patch_ok && w->layout != VIDATTN_WINDOW_ROWS ? patch_tiles_listed(p, F, H, W) : TileCount{};
  p.cap = pc.most;
  if (w->layout == VIDATTN_WINDOW_PATCHES) {
    *g = p;
    return VIDATTN_OK;
  }
  const TileCount rc = rows_tiles_listed(N, F, H, W, g->rf, g->rh);
  g->cap = rc.most;
  // every listed tile costs the same (256 queries x 64 keys) in both layouts
  if (w->layout == VIDATTN_WINDOW_AUTO && patch_ok && pc.total < rc.total) *g = p;
  return VIDATTN_OK;
}

// bf16 key/value image and tile lists of a window call.
static size_t window_image_bytes(int64_t nbh, int64_t d, const WindowGeom& g) {
  return (size_t)(4 * nbh * g.nkt * kKT * d);
}
static size_t window_plan_bytes(const WindowGeom& g) {
  return (size_t)((g.nqb * 4 + 255) / 256 * 256 + g.nqb * g.cap * 4);
}

size_t vidattn_fwd_window_workspace_size(vidattn_dtype dt, int64_t B, int64_t heads, int64_t N, int64_t d,
                                         int use_rope, const vidattn_window_desc* window) {
  if (dt != VIDATTN_BF16) return 0;
  const size_t base = vidattn_fwd_workspace_size(dt, B, heads, N, d, use_rope);
  if (!base) return 0;
  WindowGeom g;
  const std::string saved = g_last_error;  // a size query leaves the last error alone
  const vidattn_status s = window_geom(window, N, nullptr, &g);
  g_last_error = saved;
  if (s != VIDATTN_OK) return 0;
  return window_image_bytes(B * heads, d, g) + window_plan_bytes(g);
}

vidattn_status vidattn_fwd_window(const void* q, const void* k, const void* v, void* o, vidattn_dtype dt, int64_t B,
                                  int64_t heads, int64_t N, int64_t d, float softmax_scale,
                                  const vidattn_rope3d_desc* rope, const vidattn_window_desc* window,
                                  void* workspace, size_t workspace_bytes, void* hip_stream) {
  if (dt != VIDATTN_BF16)
    return fail(dt == VIDATTN_F32 || dt == VIDATTN_F16 ? VIDATTN_ERR_UNSUPPORTED : VIDATTN_ERR_INVALID_ARG,
                "local-window attention is implemented for BF16");
  WindowGeom g;
  size_t extra = 0;  // workspace beyond vidattn_fwd_workspace_size
  const bool sizes_ok = N >= 1 && N <= kMaxN && B >= 1 && heads >= 1 && B <= kMaxBH && heads <= kMaxBH &&
                        B * heads <= kMaxBH && (d == 64 || d == 128);
  if (N >= 1 && N <= kMaxN) {
    if (vidattn_status s = window_geom(window, N, rope, &g)) return s;
    if (sizes_ok)
      extra = window_image_bytes(B * heads, d, g) + window_plan_bytes(g) -
              vidattn_fwd_workspace_size(dt, B, heads, N, d, rope != nullptr);
  }
  if (vidattn_status s = validate_fwd(Phase::kFused, q, k, v, o, dt, B, heads, N, d, softmax_scale, rope, workspace,
                                      workspace_bytes, -1, extra))
    return s;
  if (!window) return fail(VIDATTN_ERR_INVALID_ARG, "window must be non-null");
  const int64_t nbh = B * heads;
  if (nbh * g.nqb > (int64_t)INT32_MAX / (kNW * 64))
    return fail(VIDATTN_ERR_UNSUPPORTED, "problem too large for one launch");
  const RopeParams rp = make_rope(rope);
  hipStream_t st = static_cast<hipStream_t>(hip_stream);
  const bool patch = g.layout == VIDATTN_WINDOW_PATCHES;
  const int F = (int)window->F, H = (int)window->H, W = (int)window->W;
  const TileMap map{patch ? 1 : 0, H, W, g.tyn, g.txn};
  if (vidattn_status s = launch_prepare(k, v, dt, nbh, N, d, rp, workspace, st, map, g.nkt)) return s;
  uint8_t* tail = static_cast<uint8_t*>(workspace) + window_image_bytes(nbh, d, g);
  int32_t* kvc = reinterpret_cast<int32_t*>(tail);
  int32_t* kvb = reinterpret_cast<int32_t*>(tail + (g.nqb * 4 + 255) / 256 * 256);
  const dim3 pgrid((unsigned)((g.nqb + 255) / 256));
  if (patch)
    hipLaunchKernelGGL(window_plan_patch_kernel, pgrid, dim3(256), 0, st, kvb, kvc, (int)g.nqb, (int)g.cap, F, H, W,
                       g.rf, g.rh, g.rw, g.tyn, g.txn, g.pyn, g.pxn);
  else
    hipLaunchKernelGGL(window_plan_kernel, pgrid, dim3(256), 0, st, kvb, kvc, (int)N, (int)g.nqb, (int)g.cap, F, H,
                       W, g.rf, g.rh);
  if (vidattn_status s = hip_check("window plan launch")) return s;
  AttendExtras x;
  x.kvb = kvb;
  x.kvc = kvc;
  x.maxb = (int)g.cap;
  x.lists_shared = 1;
  x.window = true;
  int mode = 0;  // the row layout's key decode (the patch layout has its own)
  if (patch) {
    x.patch = true;
    x.nkt = g.nkt;
    x.ntq = g.nqb;
  } else {
    // key decode (see WindowParams): the fp32 split needs key indices (up to
    // nkt * 64 - 1) below 2^22; rows of >= 64 tokens allow the whole-tile test
    const bool small_n = g.nkt * kKT < (int64_t(1) << 22);
    mode = !small_n ? 0 : (W >= 64 ? 2 : (W >= 8 ? 1 : 0));
  }
  auto inv = [](int n) { return (float)(1.0 / (double)n); };
  x.wp = WindowParams{F, H, W, g.rf, g.rh, g.rw, mode, inv(W), inv(H), g.tyn, g.txn, g.pyn, g.pxn,
                      inv(g.txn), inv(g.tyn), inv(g.pxn), inv(g.pyn)};
  if (vidattn_status s = launch_attend(q, k, v, workspace, o, dt, nbh, N, d, softmax_scale, rp, st, x)) return s;
  return ok();
}

size_t vidattn_fwd_block_mask_workspace_size(vidattn_dtype dt, int64_t B, int64_t heads, int64_t N, int64_t d,
                                             int use_rope) {
  if (dt != VIDATTN_BF16) return 0;
  const size_t base = vidattn_fwd_workspace_size(dt, B, heads, N, d, use_rope);
  return base ? base + block_mask_list_bytes(B * heads, N) : 0;
}

vidattn_status vidattn_fwd_attend_block_mask(const void* q, const uint32_t* mask, void* workspace, void* o,
                                             vidattn_dtype dt, int64_t B, int64_t heads, int64_t N, int64_t d,
                                             float softmax_scale, const vidattn_rope3d_desc* rope,
                                             size_t workspace_bytes, void* hip_stream) {
  if (dt != VIDATTN_BF16)
    return fail(dt == VIDATTN_F32 || dt == VIDATTN_F16 ? VIDATTN_ERR_UNSUPPORTED : VIDATTN_ERR_INVALID_ARG,
                "block-sparse attention is implemented for BF16");
  if (!mask || (reinterpret_cast<uintptr_t>(mask) & 3u) != 0)
    return fail(VIDATTN_ERR_INVALID_ARG, "mask must be non-null and 4-byte aligned");
  const size_t lists = N >= 1 && N <= kMaxN && B >= 1 && heads >= 1 && B <= kMaxBH && heads <= kMaxBH &&
                               B * heads <= kMaxBH
                           ? block_mask_list_bytes(B * heads, N)
                           : 0;
  if (vidattn_status s = validate_fwd(Phase::kAttend, q, q, q, o, dt, B, heads, N, d, softmax_scale, rope, workspace,
                                      workspace_bytes, -1, lists))
    return s;
  const int64_t nbh = B * heads, nqb = (N + kBR - 1) / kBR, nkt = (N + kKT - 1) / kKT;
  const int64_t rows = nbh * nqb;
  const int words = (int)((nkt + 31) / 32);
  {  // the lists are written into the workspace while the mask is read
    const char* mb = reinterpret_cast<const char*>(mask);
    const char* wb = static_cast<const char*>(workspace);
    const int64_t mask_bytes = rows * words * 4;
    const int64_t ws_bytes = (int64_t)vidattn_fwd_block_mask_workspace_size(dt, B, heads, N, d, rope != nullptr);
    if (mb < wb + ws_bytes && wb < mb + mask_bytes) return fail(VIDATTN_ERR_INVALID_ARG, "mask overlaps the workspace");
    // the lists are written into the workspace tail before q is read
    const char* qb = static_cast<const char*>(q);
    const int64_t q_bytes = nbh * N * d * 2;
    const char* tail0 = wb + vidattn_fwd_workspace_size(dt, B, heads, N, d, rope != nullptr);
    if (qb < wb + ws_bytes && tail0 < qb + q_bytes)
      return fail(VIDATTN_ERR_INVALID_ARG, "q overlaps the list part of the workspace");
  }
  uint8_t* tail = static_cast<uint8_t*>(workspace) + vidattn_fwd_workspace_size(dt, B, heads, N, d, rope != nullptr);
  int32_t* kvc = reinterpret_cast<int32_t*>(tail);
  int32_t* kvb = reinterpret_cast<int32_t*>(tail + (rows * 4 + 255) / 256 * 256);
  hipStream_t st = static_cast<hipStream_t>(hip_stream);
  hipLaunchKernelGGL(block_mask_lists_kernel, dim3((unsigned)((rows + 255) / 256)), dim3(256), 0, st, mask, kvb, kvc,
                     rows, words, (int)nkt);
  if (vidattn_status s = hip_check("block mask lists launch")) return s;
  const RopeParams rp = make_rope(rope);
  AttendExtras x;
  x.kvb = kvb;
  x.kvc = kvc;
  x.maxb = (int)nkt;
  if (vidattn_status s = launch_attend(q, q, q, workspace, o, dt, nbh, N, d, softmax_scale, rp, st, x)) return s;
  return ok();
}

}  // extern "C"


// ---------------------------------------------------------------- fixed scratch (no allocation)

// The workspace of vidattn_fwd_noalloc: a fixed array in device memory, one
// copy per GPU the library runs on, held until the process ends. In host
// code its name stands for a host-side shadow, not a device address; the
// device address is looked up once per device (hipGetSymbolAddress) and
// only that address is passed to kernels.
static __device__ __align__(256) uint8_t scratch[VIDATTN_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// Device address of `scratch` on the current device (looked up once per device).
vidattn_status scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return fail(VIDATTN_ERR_HIP, "no usable current HIP device (%d)", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(VIDATTN_ERR_HIP, "device address of the fixed scratch: %s", hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return VIDATTN_OK;
}

}  // namespace

extern "C" {

vidattn_status vidattn_fwd_noalloc(const void* q, const void* k, const void* v, void* o, vidattn_dtype dt, int64_t B,
                                   int64_t heads, int64_t N, int64_t d, float softmax_scale,
                                   const vidattn_rope3d_desc* rope, void* hip_stream) {
  // 0 for arguments vidattn_fwd rejects by dtype or size: it reports them
  const size_t need = vidattn_fwd_workspace_size(dt, B, heads, N, d, rope != nullptr);
  if (need > (size_t)VIDATTN_NOALLOC_SCRATCH_BYTES)
    return fail(VIDATTN_ERR_WORKSPACE,
                "this call needs %zu bytes of workspace; the fixed scratch of vidattn_fwd_noalloc holds %zu "
                "(use vidattn_fwd with a caller workspace)",
                need, (size_t)VIDATTN_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  if (need > 0)
    if (vidattn_status s = scratch_address(&ws)) return s;
  return vidattn_fwd(q, k, v, o, dt, B, heads, N, d, softmax_scale, rope, ws, need, hip_stream);
}

}  // extern "C"
