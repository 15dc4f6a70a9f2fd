/*
 * vidattn.h — C ABI of libvidattn: 3D rotary position embedding and full
 * (non-causal) spatiotemporal self-attention for video diffusion
 * transformer blocks, on AMD Instinct MI355X (gfx950).
 *
 * What is computed. The vidax paper summary (paperlayer.ai/abs/2609.18077v1,
 * section 2 "System Architecture & Design", heading "3D RoPE, 3D VAEs, and
 * flash attention") names 3D rotary embeddings and a flash-attention kernel
 * that never materialises the quadratic query-key matrix; section 1
 * ("Motivation and gap") describes the input as tens of thousands of tokens
 * cut from a video latent as 3D patches. The pages do not write the rotary
 * rule out; this library fixes it as follows (the plainest reading):
 *
 *   token order   n = (f*H + y)*W + x for a grid of F frames, H rows, W
 *                 columns (frame-major);
 *   chunks        the head dimension d splits into contiguous chunks
 *                 [0, d_t) | [d_t, d_t+d_h) | [d_t+d_h, d) driven by the
 *                 frame index f, row index y and column index x;
 *   pairs         inside a chunk of width d_a starting at c0, the adjacent
 *                 pair (c0+2j, c0+2j+1), j < d_a/2, is rotated by the angle
 *                 phi = pos_a * theta^(-2j/d_a):
 *                   x'[c0+2j]   = x[c0+2j]*cos(phi) - x[c0+2j+1]*sin(phi)
 *                   x'[c0+2j+1] = x[c0+2j]*sin(phi) + x[c0+2j+1]*cos(phi)
 *                 with 0-based integer positions (position (0,0,0) is the
 *                 identity).
 *
 * Attention is O[i] = sum_j softmax_j(scale * <q'_i, k'_j>) v_j over all N
 * tokens of one (batch, head) slice, with q', k' the rotated queries and
 * keys (v is not rotated).
 *
 * Layout. Q, K, V and O are dense, contiguous [B][heads][N][d] row-major
 * arrays (token rows of d elements, head-major: the layout an attention
 * kernel sees after a sequence-to-head all-to-all).
 *
 * Memory. Every pointer argument is a device pointer owned by the caller
 * (for example from PyTorch). The library allocates no device memory and
 * keeps no state besides its code objects; q, k and v are only read.
 *
 * Streams. Work is enqueued on `hip_stream` (a hipStream_t; NULL means the
 * null stream) and the call returns without synchronising. Faults of a
 * kernel surface on the caller's next synchronisation.
 *
 * Errors. Every entry point returns a vidattn_status. Arguments are
 * validated before any HIP call, so a malformed call returns INVALID_ARG or
 * UNSUPPORTED without touching the device (and works without a GPU); no
 * entry point aborts, throws or prints. vidattn_last_error() gives a
 * human-readable detail of the last non-OK status on the calling thread.
 *
 * Numerics (bf16 path). Rotation and softmax run in fp32. The rotated keys
 * and the rotated queries pre-multiplied by scale*log2(e) are rounded once,
 * to nearest-even, to fp16 and multiplied on fp16 matrix cores with fp32
 * accumulation (fp16 keeps 3 more mantissa bits than bf16; bf16 operands
 * here lose the peaky-key accuracy bound). Softmax probabilities are
 * rounded to nearest-even bf16 and multiplied with the bf16 V on bf16
 * matrix cores with fp32 accumulation; O is rounded once to bf16.
 * Finite results need |rotated k| < 65504 and |rotated q*scale*log2 e| <
 * 65504. (fp32 path) Everything in fp32, fp32 matrix cores.
 * Results are bitwise reproducible run to run for the same inputs.
 */
#ifndef VIDATTN_H
#define VIDATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define VIDATTN_ABI_VERSION 7

typedef enum {
  VIDATTN_OK = 0,
  VIDATTN_ERR_INVALID_ARG = 1,  /* null/misaligned pointer, bad size, inconsistent grid or split */
  VIDATTN_ERR_UNSUPPORTED = 2,  /* well-formed but not implemented (e.g. head dim 96) */
  VIDATTN_ERR_WORKSPACE = 3,    /* workspace missing or smaller than vidattn_fwd_workspace_size */
  VIDATTN_ERR_HIP = 4           /* a HIP runtime call or kernel launch failed */
} vidattn_status;

typedef enum {
  VIDATTN_BF16 = 0,
  VIDATTN_F16 = 1,
  VIDATTN_F32 = 2
} vidattn_dtype;

/* Token grid and rotary parameters.
 *   F, H, W       grid extents (frames, rows, columns), each >= 1; the
 *                 sequence length N must equal F*H*W.
 *   d_t, d_h, d_w widths of the frame, row and column chunks of the head
 *                 dimension: each even and >= 0, d_t + d_h + d_w == d.
 *   theta         frequency base (> 0 and finite), e.g. 10000.0. */
typedef struct {
  int64_t F, H, W;
  int32_t d_t, d_h, d_w;
  double theta;
} vidattn_rope3d_desc;

/* Standalone 3D rotary embedding (the rule above), for queries or keys.
 *   in       [B][heads][N][d] with N = F*H*W, dtype in_dt (BF16 or F32).
 *   out      same shape, dtype out_dt (BF16, F16 or F32); out == in is
 *            allowed when both dtypes have the same size, any other overlap
 *            is not.
 *   prescale multiplies every rotated element (1.0f = none); finite.
 *   d        even, a multiple of 8, at most 256.
 * The rotation is computed in fp32: the angle is formed and reduced modulo
 * 2*pi in fp64, and its cos/sin are evaluated in fp32 (absolute error about
 * 2e-7); the result is multiplied by prescale and rounded to nearest-even
 * to out_dt.
 * Pointers must be 16-byte aligned. */
vidattn_status vidattn_rope3d(const void* in, vidattn_dtype in_dt, void* out, vidattn_dtype out_dt,
                              int64_t B, int64_t heads, int64_t d, const vidattn_rope3d_desc* rope,
                              float prescale, void* hip_stream);

/* The same rotation for a contiguous run of tokens of the grid: row r of
 * each (b, head) slice is grid token token_offset + r, and turns by that
 * token's position. This is the rotation of one GPU's sequence shard before
 * the all-to-all of Ulysses sequence parallelism (the vidax summary,
 * paperlayer.ai/abs/2609.18077v1, section 2, heading "Spatiotemporal tensor
 * and sequence sharding": tokens are partitioned across devices and
 * all-to-all transposes give head-sharded views for attention), so that
 * every shard uses global positions.
 *   in, out      [B][heads][n_tokens][d]; dtypes, overlap, prescale and d
 *                as for vidattn_rope3d.
 *   n_tokens     >= 1; token_offset >= 0 and token_offset + n_tokens <=
 *                F*H*W (else INVALID_ARG).
 * Offset 0 with n_tokens = F*H*W is vidattn_rope3d, bit for bit. */
vidattn_status vidattn_rope3d_tokens(const void* in, vidattn_dtype in_dt, void* out, vidattn_dtype out_dt,
                                     int64_t B, int64_t heads, int64_t n_tokens, int64_t token_offset, int64_t d,
                                     const vidattn_rope3d_desc* rope, float prescale, void* hip_stream);

/* Attention forward: o = softmax(scale * rot(q) rot(k)^T) v per (b, head).
 *   q, k, v, o    [B][heads][N][d], dtype dt (BF16 or F32); o has dtype dt.
 *   d             64 or 128.
 *   softmax_scale finite, > 0 (typically 1/sqrt(d)).
 *   rope          NULL: q and k are used as given (already rotated or no
 *                 rotary embedding). Otherwise the rotation is applied to q
 *                 at tile load and to k by a pre-pass into the workspace;
 *                 rope->F*H*W must equal N.
 *   workspace     device buffer of at least
 *                 vidattn_fwd_workspace_size(dt, B, heads, N, d, rope != NULL)
 *                 bytes, 256-byte aligned; it may be NULL only when that size
 *                 is 0. Its contents on entry are irrelevant and are
 *                 overwritten.
 * All N keys are attended by every query (no mask, no causal order).
 * Pointers must be 16-byte aligned; o must not overlap q, k, v or the
 * workspace, and the workspace (which the pre-pass writes before q is read)
 * must not overlap q, k or v; INVALID_ARG otherwise. */
vidattn_status vidattn_fwd(const void* q, const void* k, const void* v, void* o, vidattn_dtype dt,
                           int64_t B, int64_t heads, int64_t N, int64_t d, float softmax_scale,
                           const vidattn_rope3d_desc* rope, void* workspace, size_t workspace_bytes,
                           void* hip_stream);

/* The two phases of vidattn_fwd, for callers that time them apart or attend
 * several times against one key/value set.
 *
 * vidattn_fwd_prepare writes the key/value operand image into the
 * workspace: for BF16 the rotated keys rounded to fp16 and a transposed copy
 * of v, both tiled in matrix-core operand order; for F32 the rotated keys
 * (nothing when rope is NULL). Arguments as for vidattn_fwd.
 *
 * vidattn_fwd_attend runs the attention kernel on q against a workspace
 * that vidattn_fwd_prepare filled for the same dt, B, heads, N, d, rope and
 * the same k, v contents (not checked: a workspace prepared from other
 * arguments gives meaningless output). k and v must be the tensors given to
 * vidattn_fwd_prepare; they are read only on the F32 path. The workspace is
 * only read. Argument rules as for vidattn_fwd.
 *
 * vidattn_fwd(...) is vidattn_fwd_prepare(...) followed by
 * vidattn_fwd_attend(...) on the same stream, bit for bit. */
vidattn_status vidattn_fwd_prepare(const void* k, const void* v, vidattn_dtype dt, int64_t B, int64_t heads,
                                   int64_t N, int64_t d, const vidattn_rope3d_desc* rope, void* workspace,
                                   size_t workspace_bytes, void* hip_stream);
vidattn_status vidattn_fwd_attend(const void* q, const void* k, const void* v, const void* workspace, void* o,
                                  vidattn_dtype dt, int64_t B, int64_t heads, int64_t N, int64_t d,
                                  float softmax_scale, const vidattn_rope3d_desc* rope, size_t workspace_bytes,
                                  void* hip_stream);

/* Block sizes of the block-sparse attention below: queries are grouped in
 * blocks of 256 tokens, keys in blocks of 64 tokens (the tiles of the bf16
 * attention kernel). */
#define VIDATTN_SPARSE_Q_BLOCK 256
#define VIDATTN_SPARSE_K_BLOCK 64

/* Query-subset attention against a prepared key/value set: Nq gathered
 * query tokens attend to all N keys: the key/value-cache synchronisation of
 * Heterogeneous Step Allocation (HSA; its abstract on the paper listing
 * thelatestinai.com/papers/2606.17566), where the active tokens attend to
 * the whole sequence (the page names the operation, not an interface). Same
 * operation as
 * vidattn_fwd_attend restricted to the rows q_index[0 .. Nq-1], for query
 * rows supplied in that order.
 *   q         [B][heads][Nq][d] BF16; row r is the query of token q_index[r].
 *   q_index   int32 [Nq], device memory, shared by every (b, head): the
 *             token index in [0, N) of each query row; it gives the row's
 *             rotary position (frame, row, column under the token order
 *             above). Repeated and unordered indices are allowed. Entries
 *             outside [0, N) are clamped into it (the library does not read
 *             the array on the host); callers must pass valid indices.
 *   o         [B][heads][Nq][d] BF16.
 *   workspace filled by vidattn_fwd_prepare for (BF16, B, heads, N, d, rope)
 *             and the keys/values to attend; only read.
 * With q_index = 0 .. N-1 and Nq = N the result is bit-identical to
 * vidattn_fwd_attend. Only BF16 is implemented (F32: UNSUPPORTED). Pointers
 * 16-byte aligned (q_index 4-byte); o must not overlap q or the workspace. */
vidattn_status vidattn_fwd_attend_subset(const void* q, const int32_t* q_index, int64_t Nq, const void* workspace,
                                         void* o, vidattn_dtype dt, int64_t B, int64_t heads, int64_t N, int64_t d,
                                         float softmax_scale, const vidattn_rope3d_desc* rope, size_t workspace_bytes,
                                         void* hip_stream);

/* Block-sparse attention against a prepared key/value set: each query block
 * attends only to the key blocks listed for it: the block-sparse video-DiT
 * attention of ScalingAttention (a bit-wise block-sparse kernel driven by a
 * per-head block mask; its abstract on thelatestinai.com/papers/2606.17566)
 * and of Sparse Forcing's Persistent Block-Sparse Attention (its abstract on
 * thelatestinai.com/papers/2609.18077). Logits of unlisted key blocks are
 * -inf before the softmax; a query block with no listed key block gets O = 0
 * (a reading: the pages do not define that case).
 *   q, o        [B][heads][N][d] BF16.
 *   kv_blocks   int32 [B][heads][ceil(N/256)][max_blocks], device memory:
 *               for query block (b, head, i) (tokens 256i .. 256i+255) the
 *               indices of its key blocks (tokens 64j .. 64j+63), strictly
 *               ascending, in the first kv_count[b][head][i] entries; the
 *               other entries are ignored.
 *   kv_count    int32 [B][heads][ceil(N/256)], device memory, each in
 *               [0, max_blocks].
 *   max_blocks  in [1, ceil(N/64)].
 *   workspace   as for vidattn_fwd_attend_subset.
 * Counts and indices are not read on the host: counts outside [0,
 * max_blocks] and indices outside [0, ceil(N/64)) are clamped into range,
 * and the result for lists that are not strictly ascending is unspecified
 * (but stays inside the buffers). Listing every key block gives the dense
 * result bit for bit. Only BF16 is implemented (F32: UNSUPPORTED).
 * Pointers 16-byte aligned (the two index arrays 4-byte); o must not overlap
 * q or the workspace. */
vidattn_status vidattn_fwd_attend_block_sparse(const void* q, const void* workspace, void* o, vidattn_dtype dt,
                                               int64_t B, int64_t heads, int64_t N, int64_t d, float softmax_scale,
                                               const vidattn_rope3d_desc* rope, const int32_t* kv_blocks,
                                               const int32_t* kv_count, int64_t max_blocks, size_t workspace_bytes,
                                               void* hip_stream);

/* Local window over the token grid: a query at grid position (f, y, x)
 * attends to the keys (f', y', x') with |f - f'| <= r_f, |y - y'| <= r_h and
 * |x - x'| <= r_w (a centred box, clipped at the grid border; every query
 * sees at least itself). F, H, W as in vidattn_rope3d_desc (F*H*W == N);
 * radii >= 0, and a radius at or beyond its extent reaches the whole axis.
 * layout picks how the attention tiles queries and keys; it changes the work
 * done, never the result beyond rounding order (the keys of a query are
 * summed in another order):
 *   VIDATTN_WINDOW_AUTO     the layout that visits fewer key tiles (ties:
 *                           rows), computed on the host from the grid and
 *                           radii;
 *   VIDATTN_WINDOW_ROWS     blocks of 256 consecutive queries, tiles of 64
 *                           consecutive keys, whole grid rows listed;
 *   VIDATTN_WINDOW_PATCHES  16 x 16 query patches and 8 x 8 key patches of
 *                           one frame (unsupported when the grid has 2^22 or
 *                           more key patches or query patches). */
typedef struct {
  int64_t F, H, W;
  int32_t r_f, r_h, r_w;
  int32_t layout;
} vidattn_window_desc;

#define VIDATTN_WINDOW_AUTO 0
#define VIDATTN_WINDOW_ROWS 1
#define VIDATTN_WINDOW_PATCHES 2

/* Block-sparse attention driven by a bit mask, the form of ScalingAttention's
 * bit-wise block-sparse kernel (a per-head block mask; its abstract on the
 * paper listing thelatestinai.com/papers/2606.17566): query block i (tokens
 * 256i .. 256i+255) of each (b, head) attends only to the key blocks (64
 * tokens each) whose bit is set. Same results as vidattn_fwd_attend_block_
 * sparse given the set bits as ascending lists (bit for bit).
 *   mask       uint32 [B][heads][ceil(N/256)][ceil(ceil(N/64)/32)], device
 *              memory, 4-byte aligned: bit j%32 of word j/32 is key block j;
 *              bits at or past ceil(N/64) are ignored. Must not overlap the
 *              workspace.
 *   workspace  the prepared key/value image (vidattn_fwd_prepare) in its
 *              first vidattn_fwd_workspace_size bytes, and room after it for
 *              the lists built from the mask: at least
 *              vidattn_fwd_block_mask_workspace_size(...) bytes in all.
 *   q, o       [B][heads][N][d] BF16; o must not overlap q or the workspace,
 *              and q must not overlap the list part of the workspace (it is
 *              written before q is read).
 * A query block with no bit set gets O = 0. Only BF16 is implemented (F32:
 * UNSUPPORTED). Other arguments as for vidattn_fwd_attend. */
vidattn_status vidattn_fwd_attend_block_mask(const void* q, const uint32_t* mask, void* workspace, void* o,
                                             vidattn_dtype dt, int64_t B, int64_t heads, int64_t N, int64_t d,
                                             float softmax_scale, const vidattn_rope3d_desc* rope,
                                             size_t workspace_bytes, void* hip_stream);

/* Workspace bytes vidattn_fwd_attend_block_mask needs: vidattn_fwd_workspace_size
 * plus the lists, 4*B*heads*ceil(N/256)*ceil(N/64) bytes and a 256-byte-padded
 * count array. 0 for arguments it would reject by dtype or size. */
size_t vidattn_fwd_block_mask_workspace_size(vidattn_dtype dt, int64_t B, int64_t heads, int64_t N, int64_t d,
                                             int use_rope);

/* Local-window attention: vidattn_fwd with every query restricted to its
 * window, the windowed-attention primitive of the vidax summary
 * (paperlayer.ai/abs/2609.18077v1, "2 System Architecture & Design", heading
 * "3D RoPE, 3D VAEs, and flash attention") and the sliding local windows of
 * Sparse Forcing (its abstract on thelatestinai.com/papers/2609.18077); the
 * pages fix no window shape, the centred box above is the plainest reading.
 * One call runs the key/value pre-pass (its key tiles in the layout's
 * order), a planning kernel that lists per query block the key tiles its
 * queries' windows can reach (in the workspace), and the attention over those
 * tiles with the keys outside each query's box masked. Arguments as for
 * vidattn_fwd, plus:
 *   window     non-null; its grid must equal rope's when rope is given, and
 *              its layout must be one of the VIDATTN_WINDOW_* values.
 *   workspace  at least vidattn_fwd_window_workspace_size(..., window) bytes;
 *              as for vidattn_fwd it must not overlap q, k, v or o.
 * An unbounded window in the row layout gives the vidattn_fwd result bit for
 * bit. Only BF16 is implemented (F32: UNSUPPORTED). */
vidattn_status vidattn_fwd_window(const void* q, const void* k, const void* v, void* o, vidattn_dtype dt, int64_t B,
                                  int64_t heads, int64_t N, int64_t d, float softmax_scale,
                                  const vidattn_rope3d_desc* rope, const vidattn_window_desc* window,
                                  void* workspace, size_t workspace_bytes, void* hip_stream);

/* Workspace bytes vidattn_fwd_window needs for this window (its layout, as
 * resolved for VIDATTN_WINDOW_AUTO): the key/value image of nkt key tiles per
 * (b, head), 256*d*B*heads*nkt bytes, then a 256-byte-padded count array of
 * nqb entries and the tile lists, 4*nqb*cap bytes, where cap is the most key
 * tiles any query block lists (found on the host from the grid and radii).
 * Rows: nkt = ceil(N/64), nqb = ceil(N/256) (the image is
 * vidattn_fwd_workspace_size bytes); patches: nkt = F*ceil(H/8)*ceil(W/8),
 * nqb = F*ceil(H/16)*ceil(W/16). 0 for arguments vidattn_fwd_window would
 * reject by dtype, size or window. */
size_t vidattn_fwd_window_workspace_size(vidattn_dtype dt, int64_t B, int64_t heads, int64_t N, int64_t d,
                                         int use_rope, const vidattn_window_desc* window);

/* Workspace bytes vidattn_fwd needs for these sizes (0 if none). Returns 0
 * also for arguments vidattn_fwd would reject; a positive size never
 * depends on the data. BF16: the rotated fp16 keys and a transposed copy of
 * V, tiled; 4*B*heads*ceil(N/64)*64*d bytes. F32: the rotated fp32 keys
 * when use_rope, 4*B*heads*N*d bytes; else 0. */
size_t vidattn_fwd_workspace_size(vidattn_dtype dt, int64_t B, int64_t heads, int64_t N, int64_t d,
                                  int use_rope);

/* Static text for a status code (never NULL). */
const char* vidattn_status_string(vidattn_status s);

/* Detail of the last non-OK status returned on the calling thread ("" if
 * none). The pointer stays valid until the next vidattn_* call on that
 * thread. */
const char* vidattn_last_error(void);

/* vidattn_fwd without a workspace argument, for callers that cannot
 * allocate device memory (code under stream capture, tight serving loops,
 * harnesses that forbid allocation). The workspace is a fixed array of
 * VIDATTN_NOALLOC_SCRATCH_BYTES in device memory inside the library, one
 * copy per GPU, held until the process ends; the call allocates nothing.
 * Its first call on a device looks up that array's device address (on the
 * current device: hip_stream must belong to it). Everything else is as for
 * vidattn_fwd, whose results it gives bit for bit. A call whose workspace
 * (vidattn_fwd_workspace_size) exceeds the scratch returns
 * VIDATTN_ERR_WORKSPACE. Every call on one GPU uses the same scratch, so
 * calls that overlap in time on one GPU (different streams, or threads)
 * race and give wrong results: serialize them. Nothing in the scratch has to
 * start at zero (each call rewrites what it reads). */
#define VIDATTN_NOALLOC_SCRATCH_BYTES (64u << 20)
vidattn_status vidattn_fwd_noalloc(const void* q, const void* k, const void* v, void* o, vidattn_dtype dt,
                                   int64_t B, int64_t heads, int64_t N, int64_t d, float softmax_scale,
                                   const vidattn_rope3d_desc* rope, void* hip_stream);

/* VIDATTN_ABI_VERSION of the loaded library. */
int vidattn_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* VIDATTN_H */
