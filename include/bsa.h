/*
 * bsa.h - C ABI of libbsa, training-free block-sparse self-attention for video diffusion
 * transformers on AMD Instinct MI355X (gfx950).
 *
 * The method (FVAttn page, abstract): a sparse-routing frontend made of video-aware block
 * organization, Top-p routing and a Top-k safety floor materializes a block mask; attention
 * then runs exactly over the kept blocks with an online softmax (the row maximum and row sum
 * that an online softmax keeps: VC-Attention page, abstract; block-sparse kernels: PSA page,
 * "Approach", DFSAttn abstract).  The library splits this into three calls:
 *
 *   bsa_reorder          token permutation into 3D tiles (and its inverse)
 *   bsa_score_and_route  per-block mean pooling, pooled block scores, Top-p/Top-k -> CSR
 *   bsa_sparse_attn_fwd  exact block-sparse attention over the CSR lists
 *
 * Two more calls split the same work differently: bsa_reorder_pool does the forward
 * permutation of Q (or K) and its block means in one pass, and bsa_route_pooled routes from
 * those means, so Q and K are read once instead of twice.  bsa_stripe_mask emits static
 * periodic-stripe masks (PSA page) in the same CSR format, as a second workload for
 * bsa_sparse_attn_fwd.
 *
 * Conventions shared by every call
 *   - Tensor arguments are DEVICE pointers (HIP device memory of the current device).  The
 *     caller allocates and owns every buffer, workspaces included; the library never
 *     allocates device memory and keeps no state between calls apart from a read-only
 *     per-device property cache.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).  Every call only
 *     enqueues work on it and returns; no call synchronizes the host or reads device data.
 *   - bf16 is IEEE bfloat16 (uint16 storage).  Results are written with round-to-nearest-even.
 *   - Arguments are validated on the host before anything is enqueued.  A non-OK status
 *     means nothing was enqueued (except BSA_ERR_HIP, returned when a launch itself fails);
 *     bsa_last_error() then returns a message for the calling thread.
 *   - Calls are thread-safe.  Calls that write the same buffers must not overlap.
 *
 * Token layout
 *   raster   [batch, N, heads, D]      token n = (t*H + h)*W + w of the T x H x W latent grid
 *   tiled    [batch, heads, Npad, D]   tile order; n_blk = ceil(N / block), Npad = n_blk*block;
 *                                      positions N..Npad-1 are padding (zero after reorder)
 *   Rows of the routing are (batch, head, query block) triples, numbered
 *   r = (b*heads + h)*n_blk + i.
 */
#ifndef BSA_H
#define BSA_H

#include <stddef.h>
#include <stdint.h>

/* Every entry point below is exported from libbsa.so; the library's other symbols are hidden. */
#ifndef BSA_API
#define BSA_API __attribute__((visibility("default")))
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    BSA_OK = 0,
    BSA_ERR_INVALID_ARG = -1,   /* null pointer, non-positive size, p outside [0,1], ...   */
    BSA_ERR_UNSUPPORTED = -2,   /* head_dim or block size the kernels are not built for     */
    BSA_ERR_WORKSPACE = -3,     /* workspace pointer NULL or smaller than the query returns */
    BSA_ERR_HIP = -4            /* a HIP launch or device query failed                      */
} bsa_status;

/* Latent grid and block organization.  Tiles are visited in (it, ih, iw) order, the last tile
 * along an axis is truncated to what is left of the grid, and tokens inside a tile are
 * row-major (t, h, w).  Blocks are `block` consecutive tokens of that order.  The tile volume
 * need not equal `block` (a block may then straddle tiles).
 * `order` replaces that token order when not NULL: a DEVICE table of N int32, order[p] = the
 * raster token at position p (a permutation of 0..N-1, not checked), e.g. the Hilbert-curve
 * order of bsa_hilbert_order; every call that maps positions to tokens (the reorders, the
 * fused quantization, the stripe masks' block coordinates) then uses it.  4-byte aligned.
 * Zero-initialising the struct's trailing members keeps the 3D-tile order. */
typedef struct {
    int32_t T, H, W;                  /* latent grid, N = T*H*W real tokens            */
    int32_t tile_t, tile_h, tile_w;   /* 3D tile extent, each >= 1                     */
    int32_t block;                    /* tokens per block: 64 or 128                   */
    const int32_t* order;             /* optional token order table (device), or NULL  */
} bsa_grid;

typedef struct {
    int32_t batch, heads, head_dim;   /* head_dim: 64 or 128                           */
} bsa_shape;

/* ---- host-only helpers ------------------------------------------------------------- */
/* ceil(N / block) and n_blk * block; 0 for an invalid grid. */
BSA_API int32_t bsa_num_blocks(const bsa_grid* grid);
BSA_API int32_t bsa_padded_len(const bsa_grid* grid);

/* ---- 1. video-aware block organization (FVAttn abstract) --------------------------- */
/* inverse == 0: src raster bf16 [batch, N, heads, D] -> dst tiled bf16 [batch, heads, Npad, D];
 *               dst pad rows (positions >= N) are written with zeros.
 * inverse != 0: src tiled [batch, heads, Npad, D] -> dst raster [batch, N, heads, D]; pad rows
 *               of src are not read.
 * src and dst must not overlap.  Supported head_dim: any multiple of 8 in [8, 1024]. */
BSA_API bsa_status bsa_reorder(const void* src, void* dst, const bsa_shape* shape,
                       const bsa_grid* grid, int32_t inverse, void* stream);

/* Forward reorder fused with the block pooling of routing (FVAttn abstract: video-aware
 * blocks, pooled into one mean per block for the router) and, optionally, with the E4M3
 * quantization of the FP8 path.  One pass over src (raster bf16 [batch, N, heads, D]); each
 * output may be NULL (at least one must be set):
 *   dst       as bsa_reorder(inverse = 0): tiled bf16 [batch, heads, Npad, D], pad rows zero;
 *   pooled    fp64 [batch, heads, n_blk, D]: pooled[b][h][j] = mean of the tiled rows j*block ..
 *             min((j+1)*block, N) - 1 (the block's real tokens).  Bit-identical to the pooling
 *             inside bsa_score_and_route whenever, in every column of a block, the nonzero
 *             bf16 values lie within a factor 2^38 of each other: every fp64 partial sum of
 *             at most 128 such values is then exact, whatever the order.  For wider spreads
 *             the two sums may round differently in the last bit of the mean;
 *   x8, x8_scales (both or neither): the E4M3 codes and per-block scales that
 *             bsa_quantize_fp8(v_layout = 0) writes for the tiled tensor (head_dim 128 and
 *             block 128 only, else BSA_ERR_UNSUPPORTED).
 * head_dim 64 or 128, block 64 or 128.  src, dst, x8 16-byte aligned, pooled 8-byte,
 * x8_scales 4-byte aligned; no two buffers may overlap (BSA_ERR_INVALID_ARG).  n_blk x heads
 * above 2^24 -> BSA_ERR_UNSUPPORTED. */
BSA_API bsa_status bsa_reorder_pool(const void* src, void* dst, double* pooled, void* x8,
                                    float* x8_scales, const bsa_shape* shape,
                                    const bsa_grid* grid, void* stream);

/* Forward reorder of V fused with its E4M3 quantization (head_dim 128, block 128): v8 and
 * v_scales exactly as bsa_quantize_fp8(v_layout = 1) writes them for the tiled V, and, when dst
 * is not NULL, the tiled bf16 V as bsa_reorder.  Reads the raster V twice (head maxima, then
 * codes).  Alignment and overlap rules as bsa_reorder_pool; n_blk x heads above 2^24 (a V of
 * more than 512 GiB) -> BSA_ERR_UNSUPPORTED. */
BSA_API bsa_status bsa_reorder_quantize_v(const void* src, void* dst, void* v8, float* v_scales,
                                          const bsa_shape* shape, const bsa_grid* grid,
                                          void* stream);

/* Hilbert-curve token order (DFSAttn page, abstract: tokens reordered along a Hilbert curve
 * so blocks of consecutive tokens are compact).  Writes order[N] (device int32): the tokens of
 * the T x H x W grid sorted by their index on the 3D Hilbert curve of the smallest 2^b cube
 * holding the grid (axes t, h, w; J. Skilling's construction, "Programming the Hilbert curve",
 * 2004), cells outside the grid skipped.  Built on the device (mark, scan, place), enqueued on
 * stream; ws of at least bsa_hilbert_order_workspace_bytes() bytes (8^b cells x 8 bytes),
 * 256-byte aligned.  Axes above 256 -> BSA_ERR_UNSUPPORTED.  The grid's own `order` and tile
 * extents are ignored. */
BSA_API size_t bsa_hilbert_order_workspace_bytes(const bsa_grid* grid);
BSA_API bsa_status bsa_hilbert_order(const bsa_grid* grid, int32_t* order, void* ws,
                                     size_t ws_bytes, void* stream);

/* ---- 2. routing frontend: pooled block scores, Top-p with a Top-k floor (FVAttn) ---- */
/* Workspace bytes bsa_score_and_route needs (depends on shape and grid only). */
BSA_API size_t bsa_route_workspace_bytes(const bsa_shape* shape, const bsa_grid* grid);

/* For every row (b, h, i):
 *   qbar_i, kbar_j = means of the tiled Q and K over the real tokens of block i / j (fp64),
 *   s_ij = scale * <qbar_i, kbar_j>  (fp64),  mass_ij = softmax_j(s_ij) over all n_blk blocks,
 *   order j by s_ij descending (equal scores: smaller j first), keep the shortest prefix
 *   whose cumulative mass reaches top_p (top_p >= 1: all; top_p == 0: none; all if rounding
 *   never reaches top_p), then raise the count to min(n_blk, k_floor).
 *   Rows of up to 2048 blocks rank by the score's order-preserving 64-bit image with its low
 *   log2(P) bits (P = max(64, next power of two >= n_blk), at most 11 bits) dropped, so two
 *   scores within 2^-41 of each other (relative) may rank by index instead; the masses and
 *   the prefix use the exact scores.  Longer rows rank by the exact scores.
 * Outputs, CSR over rows:
 *   row_ptr [rows + 1] int32, row_ptr[0] = 0;
 *   col_idx capacity rows*n_blk int32 (worst case), kept key blocks of each row ascending;
 *   nnz     [1] int32 = row_ptr[rows];
 *   block_scores (optional, may be NULL) [batch, heads, n_blk, n_blk] fp64 s_ij.
 * q_t, k_t: tiled bf16 [batch, heads, Npad, D] (pad rows are ignored).
 * Errors: top_p NaN or outside [0, 1], k_floor < 1, scale not finite -> BSA_ERR_INVALID_ARG;
 * rows*n_blk must fit int32; n_blk <= 4096.
 * ws: device workspace of at least bsa_route_workspace_bytes() bytes, 256-byte aligned. */
BSA_API bsa_status bsa_score_and_route(const void* q_t, const void* k_t, const bsa_shape* shape,
                               const bsa_grid* grid, double top_p, int32_t k_floor,
                               double scale, int32_t* row_ptr, int32_t* col_idx,
                               int32_t* nnz, double* block_scores, void* ws,
                               size_t ws_bytes, void* stream);

/* bsa_score_and_route without its pooling step: qbar and kbar are the block means
 * [batch, heads, n_blk, D] fp64 (as bsa_reorder_pool writes them, 16-byte aligned); every
 * other argument, output, error and the workspace (bsa_route_workspace_bytes) are those of
 * bsa_score_and_route, and for the same Q and K the outputs are identical. */
BSA_API bsa_status bsa_route_pooled(const double* qbar, const double* kbar,
                                    const bsa_shape* shape, const bsa_grid* grid, double top_p,
                                    int32_t k_floor, double scale, int32_t* row_ptr,
                                    int32_t* col_idx, int32_t* nnz, double* block_scores,
                                    void* ws, size_t ws_bytes, void* stream);

/* ---- 2b. static periodic-stripe masks (PSA page, "Approach") ----------------------- */
/* One six-parameter mask M(Tw, To, Ts, Sw, So, Ss) per head.  The page names the parameters
 * without defining them; reading used here (T = temporal, S = spatial; w = stripe width,
 * o = offset, s = period): a block's coordinates are those of the 3D tile holding its first
 * token, bt = t / tile_t and bs = (h / tile_h) * nW + w / tile_w with nW = ceil(W / tile_w);
 * query block i keeps key block j iff
 *     (bt_j - bt_i - To) mod Ts < Tw   and   (bs_j - bs_i - So) mod Ss < Sw
 * (non-negative remainders).  Requires 1 <= Tw <= Ts and 1 <= Sw <= Ss. */
typedef struct {
    int32_t Tw, To, Ts, Sw, So, Ss;
} bsa_stripe;

/* Workspace bytes bsa_stripe_mask needs (depends on shape and grid only). */
BSA_API size_t bsa_stripe_workspace_bytes(const bsa_shape* shape, const bsa_grid* grid);

/* The stripe masks of every (batch, head) as CSR, in the format bsa_score_and_route writes
 * (rows r = (b*heads + h)*n_blk + i, columns ascending, nnz = row_ptr[rows] on the device),
 * ready for bsa_sparse_attn_fwd.
 * params: HOST array of `heads` parameter sets (head h uses params[h] for every batch); it is
 *         validated on the host, then copied into the workspace on `stream`, so the caller may
 *         reuse it when the call returns.
 * Errors: NULL pointers or a parameter set outside the ranges above -> BSA_ERR_INVALID_ARG;
 * head_dim/block/size limits as bsa_score_and_route; ws smaller than
 * bsa_stripe_workspace_bytes() or not 256-byte aligned -> BSA_ERR_WORKSPACE. */
BSA_API bsa_status bsa_stripe_mask(const bsa_stripe* params, const bsa_shape* shape,
                                   const bsa_grid* grid, int32_t* row_ptr, int32_t* col_idx,
                                   int32_t* nnz, void* ws, size_t ws_bytes, void* stream);

/* ---- 3. exact block-sparse attention (online softmax over the kept blocks) --------- */
/* Workspace bytes bsa_sparse_attn_fwd needs: worst case over every possible CSR, so the host
 * never needs nnz. */
BSA_API size_t bsa_attn_workspace_bytes(const bsa_shape* shape, const bsa_grid* grid);

/* For every real query position p of block i in row r = (b, h, i):
 *   U = real key positions of the blocks col_idx[row_ptr[r] .. row_ptr[r+1]),
 *   logit_pu = scale * <Q_p, K_u>  (bf16 inputs, fp32 accumulation),
 *   out_t[p] = sum_u softmax_u(logit_pu) V_u  (bf16),  lse[p] = log sum_u exp(logit_pu) (fp32).
 * Pad query rows (p >= N) of out_t and lse are written with zeros.
 * q_t, k_t, v_t, out_t: tiled bf16 [batch, heads, Npad, D]; lse: [batch, heads, Npad] fp32 or
 * NULL.  The pad rows (positions N..Npad-1) of k_t and v_t are read and must hold finite
 * values (bsa_reorder writes zeros there); their logits are masked out.  A row that keeps no
 * block (row_ptr[r] == row_ptr[r+1]; bsa_score_and_route never emits one) has no softmax: its
 * rows of out_t and lse are written with zeros, like pad rows.  col_idx values must lie in
 * [0, n_blk) and be distinct within a row (bsa_score_and_route guarantees it; other CSRs are
 * the caller's responsibility and are not checked on the device).
 * The heavy-row scheduler is persistent: work items are built on the device from the CSR row
 * lengths, long rows are split and their partial results merged in a fixed order, so the
 * output is bitwise deterministic.
 * scale must be finite and > 0 (BSA_ERR_INVALID_ARG otherwise).
 * ws: device workspace of at least bsa_attn_workspace_bytes() bytes, 256-byte aligned. */
BSA_API bsa_status bsa_sparse_attn_fwd(const void* q_t, const void* k_t, const void* v_t,
                               const int32_t* row_ptr, const int32_t* col_idx,
                               const bsa_shape* shape, const bsa_grid* grid, float scale,
                               void* out_t, float* lse, void* ws, size_t ws_bytes,
                               void* stream);

/* bsa_sparse_attn_fwd for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same computation, the
 * same arguments without ws / ws_bytes, and the same output bit for bit.  Instead of a caller's
 * workspace it uses a static scratch array of 136 MiB per device (allocated when the library's
 * device code is loaded onto that device, held until the process ends; its address is looked
 * up once per device on the first call made with that device current).  The call itself
 * allocates nothing.  The schedule kernels rewrite every scratch word the attention reads, so
 * no state carries over from an earlier call.  Calls that overlap on one device (on different
 * streams, or from several threads without ordering) share the one array and race: order them.
 * A call whose workspace (bsa_attn_workspace_bytes) exceeds 136 MiB -> BSA_ERR_WORKSPACE
 * (on a 256-CU MI355X that is more than about 390,000 rows batch*heads*n_blk at block 128);
 * every other error as bsa_sparse_attn_fwd. */
BSA_API bsa_status bsa_sparse_attn_fwd_noalloc(const void* q_t, const void* k_t,
                                               const void* v_t, const int32_t* row_ptr,
                                               const int32_t* col_idx, const bsa_shape* shape,
                                               const bsa_grid* grid, float scale, void* out_t,
                                               float* lse, void* stream);

/* ---- 4. FP8 (E4M3) attention (VC-Attention page, abstract) ------------------------- */
/* Both products on FP8 matrix cores with fp32 accumulation; head_dim 128 and block 128 only
 * (other shapes -> BSA_ERR_UNSUPPORTED).  E4M3 is the OCP 8-bit format (4 exponent bits,
 * bias 7, 3 mantissa bits, largest finite 448); conversions round to nearest even.
 *
 * Quantize one tiled bf16 tensor x_t [batch, heads, Npad, 128]:
 *   v_layout == 0 (Q, K): one scale per block of 128 tokens, scales [batch, heads, n_blk] fp32,
 *     s = amax / 448 over the block, x8[...] = e4m3(x * (448 / amax)) in the same
 *     [batch, heads, Npad, 128] byte layout;
 *   v_layout == 1 (V): one scale per (batch, head), scales [batch, heads] fp32, and every block
 *     stored transposed, x8 [batch, heads, n_blk, 128 (feature), 128 (key)] bytes, the keys of
 *     a row in the order 64c + 32(b / 16) + 8((b % 16) / 4) + 4h + b % 4 for byte 64c + 32h + b.
 *   A block (or head) of zeros gets scale 0 and codes 0.  x_t and x8 16-byte aligned, not
 *   overlapping; scales 4-byte aligned. */
BSA_API bsa_status bsa_quantize_fp8(const void* x_t, void* x8, float* scales, int32_t v_layout,
                                    const bsa_shape* shape, const bsa_grid* grid, void* stream);

/* Workspace bytes bsa_sparse_attn_fwd_fp8 needs (queries the current device); 0 if the shape
 * is unsupported. */
BSA_API size_t bsa_attn_fp8_workspace_bytes(const bsa_shape* shape, const bsa_grid* grid);

/* bsa_sparse_attn_fwd over the quantized tensors of bsa_quantize_fp8 (q8/k8 with per-block
 * scales, v8 transposed with per-head scales): logits from the dequantized Q and K; the
 * probabilities 2^8 exp(logit - m) (m the running maximum over the row's blocks in CSR
 * order) are cast to E4M3 before the product with the dequantized V.
 *   expcast == 0: exp in fp32, then round to nearest even; the row sum is the fp32 sum of the
 *                 uncast probabilities;
 *   expcast == 1: ExpCast (VC-Attention page, abstract): the code is 8 y + 56 for the log2
 *                 probability y, converted to an unsigned byte, with no exponential (each
 *                 cast value is 0.917-1.109x the probability, or within 2^-6 of it below
 *                 2^-6); the row sum is the sum of the cast values, so the output is their
 *                 normalized average and lse is biased by up to ln 1.109.
 * Outputs, CSR requirements and errors as bsa_sparse_attn_fwd (expcast not 0 or 1 ->
 * BSA_ERR_INVALID_ARG); ws of at least bsa_attn_fp8_workspace_bytes() bytes. */
BSA_API bsa_status bsa_sparse_attn_fwd_fp8(const void* q8, const float* q_scale, const void* k8,
                                           const float* k_scale, const void* v8,
                                           const float* v_scale, const int32_t* row_ptr,
                                           const int32_t* col_idx, const bsa_shape* shape,
                                           const bsa_grid* grid, float scale,
                                           int32_t expcast, void* out_t, float* lse, void* ws,
                                           size_t ws_bytes, void* stream);

/* ---- diagnostics ------------------------------------------------------------------- */
/* Message of the calling thread's last non-OK status ("" if none).  Valid until the next
 * call on the same thread. */
BSA_API const char* bsa_last_error(void);
BSA_API const char* bsa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* BSA_H */
