/*
 * bsa.h -- C ABI of the MI355X (gfx950) content-adaptive block-sparse
 * attention library (libbsa.so).
 *
 * The library implements, as hand-written HIP kernels, the two-stage hot path
 * described for video diffusion transformers:
 *
 *   1. a dynamic block mask (NABLA summary "Riepilogo Tecnico: NABLA -
 *      Neighborhood Adaptive Block-Level Attention ...", Metodologia section
 *      2): Q and K are average-pooled into blocks, a reduced attention map is
 *      computed over the pooled blocks, each row is binarised by its CDF
 *      against 1 - thr, optionally OR'd with a static sliding-tile window
 *      (section 3, M = M_nabla OR M_STA);
 *   2. block-sparse attention that computes only the kept query x key tiles
 *      (section 2, "Espansione"), with an online softmax.
 *
 * plus the token reorder helpers and the semantic-clustering variant of the
 * Sparse VideoGen2 summary (Metodologia A-C): fractal flattening (NABLA
 * section 1), k-means of Q and K, cluster-contiguous permutation and its
 * inverse, centroid top-p selection and attention over variable-size blocks;
 * and around them: the attention backward over the same kept tiles (NABLA
 * summary, training), k-means warm-started from the previous step's
 * centroids (Sparse VideoGen2 summary, Metodologia C.1), per-head box
 * layouts (head-aware tiling, Veda summary 2.2) and a mask-quality
 * diagnostic against the full attention's tile map (Veda summary 2.1).
 *
 * Conventions for every entry point
 * ---------------------------------
 *  - Tensors are dense and row-major. Q, K, V, O are bf16 (raw 16-bit
 *    storage) with shape [B, H, N, d]: batch, head, token, channel.
 *  - Device pointers are HIP device memory owned by the caller. The library
 *    never allocates or frees memory and keeps no pointer after return.
 *  - All device work is enqueued asynchronously on the caller's stream
 *    `stream` (0 = the null stream); the library never synchronises. Buffers
 *    must stay valid until the stream has passed the work.
 *  - The first `n_valid` tokens of each sequence are real; rows
 *    n_valid..N-1 are padding. Padding is never read as a key or value, and
 *    output padding rows are written as zero.
 *  - Return value: BSA_OK (0) or an error code. Argument checks are done on
 *    the host before any launch; on error nothing is enqueued and
 *    bsa_last_error_message() describes the problem. BSA_EHIP reports a HIP
 *    launch/runtime error. No C++ exception crosses the ABI.
 *  - The library is thread-safe; its only mutable global state is a
 *    thread-local error message.
 */
#ifndef BSA_H
#define BSA_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define BSA_ABI_VERSION 2   /* 2: bsa_blocks.max_len */

enum bsa_status {
  BSA_OK = 0,
  BSA_EINVAL = 1,        /* invalid argument (null pointer, bad size, ...)   */
  BSA_EUNSUPPORTED = 2,  /* valid but unsupported (head dim, block size ...) */
  BSA_ENOSPC = 3,        /* workspace or output capacity too small           */
  BSA_EHIP = 4           /* HIP launch or runtime error                      */
};

/*
 * Block descriptors: block i covers tokens [start[i], start[i] + len[i]) of
 * the (possibly reordered) token axis. `start` and `len` are int32 device
 * arrays of shape [nblocks], or [B*H*nblocks] (row-major over b, h, i) when
 * `per_head` is non-zero. Blocks may have any length >= 0; blocks of one
 * side must not overlap. Passing NULL for a bsa_blocks* means uniform
 * blocks: block i = [block*i, min(block*(i+1), n_valid)),
 * nblocks = ceil(n_valid / block).
 * `max_len` is an optional bound the caller vouches for: 1..64 means no block
 * is longer (fractal patches, head-aware tiling boxes), and the attention
 * then takes every block as one 64-row tile, longest rows first, with no
 * gathering of key rows; a longer block would be cut to its first 64 tokens
 * (unspecified output). 0 (or > 64) means any length.
 */
typedef struct bsa_blocks {
  int32_t nblocks;
  int32_t per_head;
  const int32_t* start;
  const int32_t* len;
  int32_t max_len;
} bsa_blocks;

/*
 * Static sliding-tile window (NABLA summary, Metodologia section 3). Blocks
 * lie on an nt x ny x nx grid with block index (t*ny + y)*nx + x; key block
 * J is inside query block I's window when |t_I - t_J| <= rt,
 * |y_I - y_J| <= ry and |x_I - x_J| <= rx (clipped at the grid edges, no
 * wrap-around). nt*ny*nx must equal the number of query and of key blocks.
 */
typedef struct bsa_window {
  int32_t nt, ny, nx;
  int32_t rt, ry, rx;
} bsa_window;

int bsa_abi_version(void);

/* Test-only: the swizzle of the attention kernels' LDS tiles. A 64-row tile
 * of d bf16 channels keeps row r's 16-byte data piece p at piece position
 * p ^ bsa_lds_swizzle(d, r) (d in {64, 128}; -1 otherwise). Exposed so that
 * host tests can map each LDS access pattern of the kernels to banks. */
int bsa_lds_swizzle(int d, int row);
const char* bsa_strerror(int status);
/* Detail of the last error raised on the calling thread ("" if none). */
const char* bsa_last_error_message(void);

/* ------------------------------------------------------------------------
 * Mask stage
 * ------------------------------------------------------------------------ */

/*
 * Block mean pooling (NABLA summary, Metodologia section 2,
 * "Sottocampionamento"): out[b,h,i,:] = mean of x[b,h,t,:] over the tokens t
 * of block i, accumulated in fp32 in a fixed order (bit-reproducible).
 *   x    bf16 [B,H,N,d] (device), d in {64, 128}
 *   out  fp32 [B,H,nblocks,d] (device)
 *   blocks  NULL = uniform blocks of `block` tokens (block = 64)
 * Blocks of length 0 produce zeros.
 */
int bsa_pool_blocks(const void* x, int B, int H, int N, int d, int n_valid,
                    int block, const bsa_blocks* blocks, float* out,
                    hipStream_t stream);

/*
 * Reduced attention and CDF selection (NABLA summary, Metodologia section 2,
 * "Attenzione Ridotta" and "CDF Thresholding"; section 3 window union;
 * Sparse VideoGen2 summary, Metodologia B, for the size-weighted variant).
 *
 * For every row (b,h,I): s_J = scale * qbar_I . kbar_J with fp32 sums (+ log
 * n_J when k_sizes is given; rows of 1025..2048 key blocks at d = 128 form
 * the products from exact three-way bf16 splits of the fp32 operands, every
 * cross term but the smallest), p_J = exp(s_J - max s), and the kept set is
 * computed exactly on the fp32 values p_J: order the blocks lightest first
 * (equal p: higher J lighter), drop J exactly when the inclusive cumulative
 * mass up to J is below thr times the row total. Masses are summed in
 * 2^-31 fixed point (m_J = floor(p_J * 2^31), 64-bit sums), so the result
 * does not depend on summation order and is bit-reproducible. thr = 0 keeps every block; the heaviest block is
 * always kept. The window, if any, is OR'd in afterwards.
 *
 *   qbar     fp32 [B,H,nqb,d], kbar fp32 [B,H,nkb,d] (device), d in {64,128}
 *   q_sizes  int32 [B,H,nqb] or NULL: rows with size 0 keep nothing
 *   k_sizes  int32 [B,H,nkb] or NULL: NULL = equal weights; otherwise key J
 *            is weighted by k_sizes[J] (log-weight added to s_J) and never
 *            kept when its size is 0
 *   thr      in [0, 1]; scale > 0, or <= 0 for 1/sqrt(d)
 *   win      NULL or a window on the block grid (nqb == nkb required)
 *   kv_count int32 [B,H,nqb] (device): number of kept key blocks per row
 *   kv_index int32 [B,H,nqb,kv_stride] (device): the first kv_count entries
 *            of each row are the kept key-block ids in ascending order; the
 *            rest of the row is left untouched. kv_stride >= nkb.
 * Supports nkb <= 8192.
 */
int bsa_select_blocks(const float* qbar, const float* kbar, int B, int H,
                      int nqb, int nkb, int d, const int32_t* q_sizes,
                      const int32_t* k_sizes, float thr, float scale,
                      const bsa_window* win, int32_t* kv_count,
                      int32_t* kv_index, int kv_stride, hipStream_t stream);

/* Workspace bytes needed by bsa_build_block_mask (pooled Q and K). */
size_t bsa_build_block_mask_workspace(int B, int H, int nqb, int nkb, int d);

/*
 * Whole mask stage: bsa_pool_blocks on q and k, then bsa_select_blocks with
 * equal weights. q, k bf16 [B,H,N,d]; qb/kb block descriptors (NULL =
 * uniform `block`-token blocks); a descriptor block of length 0 has no
 * average and takes no part: never kept as a key block (unless the window
 * covers it), and as a query block it keeps nothing; ws of at least
 * bsa_build_block_mask_workspace(...) bytes (device, 256-byte aligned).
 * Outputs as in bsa_select_blocks.
 */
int bsa_build_block_mask(const void* q, const void* k, int B, int H, int N,
                         int d, int n_valid, int block, const bsa_blocks* qb,
                         const bsa_blocks* kb, float thr, const bsa_window* win,
                         int32_t* kv_count, int32_t* kv_index, int kv_stride,
                         void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * Centroid top-p mask (Sparse VideoGen2 summary, Metodologia B): weights
 * w_ab proportional to k_sizes[b] * exp(scale * cq_a . ck_b); key clusters
 * are kept heaviest first until the mass reaches top_p (the CDF rule above
 * with thr = 1 - top_p). Empty key clusters are never kept; empty query
 * clusters keep nothing.
 *   cq fp32 [B,H,Cq,d], ck fp32 [B,H,Ck,d], q_sizes int32 [B,H,Cq],
 *   k_sizes int32 [B,H,Ck] (device); top_p in [0,1].
 */
int bsa_build_centroid_mask(const float* cq, const int32_t* q_sizes,
                            const float* ck, const int32_t* k_sizes, int B,
                            int H, int Cq, int Ck, int d, float top_p,
                            float scale, int32_t* kv_count, int32_t* kv_index,
                            int kv_stride, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Block-sparse attention
 * ------------------------------------------------------------------------ */

/* Workspace bytes of bsa_block_sparse_attn_fwd with every path available.
 * The call needs at least int32 B*H*(nqb+1) entries (the processing order
 * of uniform query blocks, or the tile table of variable-size query
 * blocks); with the bytes returned here it also runs, for uniform blocks
 * over rows of at least 1024 key blocks at d = 128, the split over key
 * segments (its tables and fp32 partial results). nqb: number of query
 * blocks (uniform: ceil(N / 64)). */
size_t bsa_block_sparse_attn_fwd_workspace(int B, int H, int nqb,
                                           const bsa_blocks* qb);

/*
 * Block-sparse attention forward (NABLA summary, Metodologia section 2,
 * "Espansione"; Sparse VideoGen2 summary, Metodologia C.2 for variable-size
 * blocks). For every query block I and query token i in it:
 *   o_i = sum_j softmax_j(scale * q_i . k_j) v_j
 * over exactly the key tokens j of the key blocks listed in
 * kv_index[b,h,I,0..kv_count-1]; every other score is -inf. QK^T and PV run
 * on bf16 MFMA with fp32 accumulation; the softmax is an fp32 online
 * softmax. A query block with no kept key block gets zero rows.
 *
 *   q, k, v   bf16 [B,H,N,d] (device), d in {64, 128}, finite values (the
 *             kernel is built without NaN semantics)
 *   o         bf16 [B,H,N,d] (device); every row of every query block is
 *             written, rows n_valid..N-1 are zeroed, other rows untouched
 *   qb, kb    block descriptors (NULL = uniform `block`-token blocks,
 *             block = 64). Query blocks of any length are tiled by 64 rows.
 *             Key blocks of any length are cut into 64-key chunks from
 *             their starts where that takes at most twice the chunks of
 *             packing the keys densely, else gathered row by row into
 *             packed 64-key chunks (decided per query block).
 *   kv_count, kv_index, kv_stride   as produced by the mask stage; ids must
 *             be valid key blocks (the caller's contract)
 *   scale     > 0, or <= 0 for 1/sqrt(d)
 *   ws        workspace of bsa_block_sparse_attn_fwd_workspace(...) bytes,
 *             or at least 4*B*H*(nqb+1) bytes (then without the split);
 *             device, 16-byte aligned, contents overwritten
 * Limits: one head of K or V (N*d*2 bytes) must stay below 4 GiB
 * (BSA_EUNSUPPORTED otherwise).
 * Uniform query blocks are scheduled longest first (most kept key blocks
 * first, per head); the order does not change any output bit.
 */
int bsa_block_sparse_attn_fwd(const void* q, const void* k, const void* v,
                              void* o, int B, int H, int N, int d, int n_valid,
                              int block, const bsa_blocks* qb,
                              const bsa_blocks* kb, const int32_t* kv_count,
                              const int32_t* kv_index, int kv_stride,
                              float scale, void* ws, size_t ws_bytes,
                              hipStream_t stream);

/*
 * The forward above for callers that cannot allocate memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same kernels and results as bsa_block_sparse_attn_fwd, with no workspace
 * argument. The int32 table that the workspace would hold (B*H*(nqb+1)
 * entries) lives in a fixed device array inside the library, one per GPU,
 * held until the process ends; the call allocates nothing.
 * Limit: B*H*(nqb+1) <= bsa_block_sparse_attn_fwd_noalloc_capacity() / 4
 * (262144 entries, 1 MiB); larger problems get BSA_ENOSPC before anything is
 * launched (use bsa_block_sparse_attn_fwd with a workspace).
 * Every call on one GPU shares that GPU's array: calls that overlap on one
 * GPU (concurrent streams or threads) race and must be serialised by the
 * caller. The first call on a device looks up the array's device address
 * (hipGetSymbolAddress). Every other argument, limit and error is that of
 * bsa_block_sparse_attn_fwd.
 */
size_t bsa_block_sparse_attn_fwd_noalloc_capacity(void);
int bsa_block_sparse_attn_fwd_noalloc(const void* q, const void* k,
                                      const void* v, void* o, int B, int H,
                                      int N, int d, int n_valid, int block,
                                      const bsa_blocks* qb,
                                      const bsa_blocks* kb,
                                      const int32_t* kv_count,
                                      const int32_t* kv_index, int kv_stride,
                                      float scale, hipStream_t stream);

/*
 * The forward above, also writing each row's softmax log-normaliser, which
 * the backward needs (NABLA summary, Contributi Chiave, "Accelerazione a Due
 * Fasi": the sparse attention runs in training as well):
 *   lse[b,h,i] = log sum_j exp(scale * q_i . k_j)   over the same kept keys
 *   lse       fp32 [B,H,N] (device, 16-byte aligned); -inf for rows of a
 *             query block with no kept key block and for rows n_valid..N-1
 * Every other argument, limit and error is that of bsa_block_sparse_attn_fwd.
 */
int bsa_block_sparse_attn_fwd_lse(const void* q, const void* k, const void* v,
                                  void* o, float* lse, int B, int H, int N,
                                  int d, int n_valid, int block,
                                  const bsa_blocks* qb, const bsa_blocks* kb,
                                  const int32_t* kv_count,
                                  const int32_t* kv_index, int kv_stride,
                                  float scale, void* ws, size_t ws_bytes,
                                  hipStream_t stream);

/* Workspace bytes needed by bsa_block_sparse_attn_bwd: fp32 row terms
 * [B,H,N,2] (lse in log2 units, rowsum(dO o O)) plus the transposed block lists (int32 [B,H,nkb] counts,
 * [B,H,nkb,nqb] ids, a [B,H,nkb,ceil(nqb/32)] bit matrix) and two
 * processing orders; nqb, nkb from the descriptors, ceil(N/64) for NULL. */
size_t bsa_block_sparse_attn_bwd_workspace(int B, int H, int N,
                                           const bsa_blocks* qb,
                                           const bsa_blocks* kb);

/*
 * Block-sparse attention backward (NABLA summary, Contributi Chiave,
 * "Accelerazione a Due Fasi"; Risultati Sperimentali 2, pre-training): the
 * gradients of bsa_block_sparse_attn_fwd with respect to q, k and v for an
 * upstream gradient dout, over the same kept tiles. Per query block I and
 * kept key block J:
 *   P = exp(scale Q_I K_J^T - lse_I),  dP = dO_I V_J^T,  Dr_i = dO_i . O_i
 *   dS = P (dP - Dr),  dQ_I += scale dS K_J,  dK_J += scale dS^T Q_I,
 *   dV_J += P^T dO_I
 * MFMA bf16 products with fp32 accumulation; deterministic (no atomics on
 * the gradients). Blocks: uniform (qb / kb NULL, block = 64), or descriptors
 * bounded to 64 tokens (max_len in 1..64: fractal patches, head-aware
 * boxes) that cover [0, n_valid) once each (every valid token in exactly
 * one query block and one key block; rows of no block are not written).
 *
 *   q, k, v, o, dout  bf16 [B,H,N,d] (device), d in {64, 128}; o is the
 *             forward's output
 *   lse       fp32 [B,H,N] from bsa_block_sparse_attn_fwd_lse with the same
 *             lists
 *   kv_count, kv_index, kv_stride   the mask lists of the forward; ids must
 *             be valid key blocks
 *   scale     > 0, or <= 0 for 1/sqrt(d) (the forward's)
 *   dq, dk, dv  bf16 [B,H,N,d] (device), fully written: rows n_valid..N-1,
 *             query rows with no kept key block and key rows no query block
 *             kept are zero
 *   qb, kb    query / key block descriptors as in the forward (NULL =
 *             uniform); the lists index them
 *   ws        workspace of bsa_block_sparse_attn_bwd_workspace(B, H, N, qb,
 *             kb) bytes (device, 16-byte aligned; contents are overwritten)
 * All pointers 16-byte aligned. Errors: BSA_EINVAL (null or misaligned
 * pointers, bad kv_stride), BSA_EUNSUPPORTED (d, block, descriptors without
 * a length bound, 4 GiB head limit), BSA_ENOSPC (workspace).
 */
int bsa_block_sparse_attn_bwd(const void* q, const void* k, const void* v,
                              const void* o, const void* dout,
                              const float* lse, int B, int H, int N, int d,
                              int n_valid, int block, const bsa_blocks* qb,
                              const bsa_blocks* kb, const int32_t* kv_count,
                              const int32_t* kv_index, int kv_stride,
                              float scale, void* dq, void* dk, void* dv,
                              void* ws, size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Mask-quality diagnostic
 * ------------------------------------------------------------------------ */

/*
 * Tile statistics of the full attention (Veda summary, section 2.1: the
 * reference tile mask max-pools the full attention matrix over every
 * query-tile x key-tile region; a tile is described by the mean, maximum and
 * minimum of its values). Second of two passes: lse must hold the natural-log
 * normaliser of every full attention row (bsa_block_sparse_attn_fwd_lse with
 * every block kept). For uniform 64-token blocks, per tile (I, J):
 *   tile_max = max, tile_sum = sum, tile_min = min of
 *   P_ij = exp(scale q_i . k_j - lse_i) over its valid query rows i and keys j.
 *   q, k     bf16 [B,H,N,d] (device), d in {64, 128}
 *   lse      fp32 [B,H,N] (device)
 *   scale    > 0, or 0 for 1/sqrt(d)
 *   tile_max, tile_sum, tile_min  fp32 [B,H,nb,nb] out, nb = ceil(n_valid/64)
 * Deterministic (fixed reduction orders).
 */
int bsa_attention_tile_stats(const void* q, const void* k, const float* lse,
                             int B, int H, int N, int d, int n_valid,
                             float scale, float* tile_max, float* tile_sum,
                             float* tile_min, hipStream_t stream);

/*
 * Recall of a block mask against the full attention's tile map (Veda
 * summary, sections 2.1 and 3: sparse-mask quality is its alignment with the
 * tile geometry of the full attention). Per query block row with k kept key
 * blocks (ids in range; others count as not kept):
 *   oracle_recall = share of the k tiles with the largest tile_max (equal
 *                   values: lower key-block id first) that the row keeps
 *                   (0 for a row that keeps nothing);
 *   mass_recall   = kept tiles' tile_sum / the row's total tile_sum (0 when
 *                   the total is 0).
 *   tile_max, tile_sum  fp32 [B,H,nqb,nkb] (device), from
 *                       bsa_attention_tile_stats
 *   kv_count, kv_index  the mask lists as in bsa_select_blocks
 *   oracle_recall, mass_recall  fp32 [B,H,nqb] out
 *   nkb <= 8192
 */
int bsa_mask_recall(const float* tile_max, const float* tile_sum,
                    const int32_t* kv_count, const int32_t* kv_index,
                    int kv_stride, int B, int H, int nqb, int nkb,
                    float* oracle_recall, float* mass_recall,
                    hipStream_t stream);

/*
 * Validator of block lists, for tests (the lists' contract: the NABLA
 * summary's CDF thresholding keeps a set of key blocks per query block, which
 * the mask stage writes as ascending ids). Over the B*H*nqb rows:
 *   bad[0] = rows whose kv_count lies outside [0, kv_stride];
 *   bad[1] = ids outside [0, nkb) among the first kv_count entries of the
 *            other rows;
 *   bad[2] = entries of those rows not greater than the entry before them
 *            (the list is not strictly ascending there).
 *   kv_count  int32 [B,H,nqb], kv_index int32 [B,H,nqb,kv_stride] (device)
 *   bad       int32 [3] (device), overwritten
 * Exact integer counts. The attention entry points do not check their lists;
 * a caller that builds or edits them can run this first.
 */
int bsa_check_mask(const int32_t* kv_count, const int32_t* kv_index,
                   int B, int H, int nqb, int nkb, int kv_stride,
                   int32_t* bad, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Token reorder helpers
 * ------------------------------------------------------------------------ */

/*
 * Gather rows: y[b,h,i,:] = x[b,h,perm[i],:] (NABLA summary, Metodologia
 * section 1; Sparse VideoGen2 summary, Metodologia A "Permutazione").
 *   x, y  bf16 [B,H,N,d] (device, must not overlap); d a multiple of 8
 *   perm  int32 [N], or [B,H,N] when perm_per_head != 0 (device); must be a
 *         permutation of 0..N-1 (the caller's contract)
 */
int bsa_permute_tokens(const void* x, void* y, const int32_t* perm, int B,
                       int H, int N, int d, int perm_per_head,
                       hipStream_t stream);

/*
 * Inverse of bsa_permute_tokens, a scatter: y[b,h,perm[i],:] = x[b,h,i,:]
 * (Sparse VideoGen2 summary, Metodologia A "Equivalenza Matematica": the
 * output is permuted back to the original token order).
 */
int bsa_unpermute_tokens(const void* x, void* y, const int32_t* perm, int B,
                         int H, int N, int d, int perm_per_head,
                         hipStream_t stream);

/*
 * Fractal flattening order (NABLA summary, Metodologia section 1), a pure
 * host function on caller-owned HOST arrays. The T x Hl x Wl latent video
 * (raster order, t slowest) is reordered so that every P x P spatial patch
 * of a frame is contiguous (patches row-major on a ceil(Hl/P) x ceil(Wl/P)
 * grid, tokens row-major inside a patch, time order kept; edge patches are
 * smaller, no tokens are inserted).
 *   perm        int32 [N] out: perm[new] = old raster index; positions
 *               >= T*Hl*Wl map to themselves (N >= T*Hl*Wl)
 *   blk_start, blk_len  int32 [max_blocks] out: one block per patch
 *   blk_coords  int32 [max_blocks*3] out or NULL: (t, patch_row, patch_col)
 *   nblocks     out: T * ceil(Hl/P) * ceil(Wl/P); BSA_ENOSPC if larger than
 *               max_blocks
 */
int bsa_fractal_order(int T, int Hl, int Wl, int P, int N, int32_t* perm,
                      int32_t* blk_start, int32_t* blk_len,
                      int32_t* blk_coords, int max_blocks, int* nblocks);

/*
 * Head-aware tiling layout (Veda summary, section 2.2 "Tiling Consapevole
 * delle Teste"): a pure host function on caller-owned HOST arrays. Each
 * pt x ph x pw box of the T x Hl x Wl latent (a factorisation of the
 * hardware tile, e.g. 1x8x8, 2x4x8 or 4x4x4 for 64-token tiles) becomes one
 * contiguous block. Boxes are numbered row-major over the
 * ceil(T/pt) x ceil(Hl/ph) x ceil(Wl/pw) grid (frame boxes slowest); tokens
 * inside a box keep raster order; edge boxes are smaller, no tokens are
 * inserted. A caller gives each head its own factorisation by calling this
 * once per head and stacking the results into per-head permutations
 * ([B,H,N], see bsa_permute_tokens) and per-head block descriptors
 * ([B,H,nblocks], padded to a common count with blocks of length 0, which
 * take no part in the mask). bsa_fractal_order is the (1, P, P) case.
 *   perm        int32 [N] out: perm[new] = old raster index; positions
 *               >= T*Hl*Wl map to themselves (N >= T*Hl*Wl)
 *   blk_start, blk_len  int32 [max_blocks] out: one block per box
 *   blk_coords  int32 [max_blocks*3] out or NULL: (box_t, box_y, box_x)
 *   nblocks     out: the box count; BSA_ENOSPC if larger than max_blocks
 * Errors: BSA_EINVAL for non-positive sizes, N < T*Hl*Wl or a null pointer.
 */
int bsa_tile_order(int T, int Hl, int Wl, int pt, int ph, int pw, int N,
                   int32_t* perm, int32_t* blk_start, int32_t* blk_len,
                   int32_t* blk_coords, int max_blocks, int* nblocks);

/* ------------------------------------------------------------------------
 * Semantic clustering (Sparse VideoGen2 summary, Metodologia A)
 * ------------------------------------------------------------------------ */

/* Workspace bytes needed by bsa_kmeans. */
size_t bsa_kmeans_workspace(int B, int H, int N, int C, int d);

/*
 * k-means of the first n_valid token vectors of every (b,h): k-means++
 * seeding (D^2 inverse-CDF draws over token order driven by the given
 * uniforms), then `iters` rounds of (assign to the nearest centroid by
 * squared Euclidean distance, ties to the lower index; update to the cluster
 * means, an empty cluster keeps its centroid). The outputs are the last
 * assignment and its cluster means. Deterministic (fixed reduction orders).
 *   x         bf16 [B,H,N,d] (device), d in {64, 128}
 *   uniforms  fp32 [B,H,C] in [0,1) (device)
 *   centroids fp32 [B,H,C,d] out; assign int32 [B,H,N] out (-1 for padding
 *             rows); sizes int32 [B,H,C] out
 *   1 <= C <= 1024, C <= n_valid
 */
int bsa_kmeans(const void* x, int B, int H, int N, int d, int n_valid, int C,
               int iters, const float* uniforms, float* centroids,
               int32_t* assign, int32_t* sizes, void* ws, size_t ws_bytes,
               hipStream_t stream);

/*
 * Warm-started k-means (Sparse VideoGen2 summary, Metodologia C.1 "Cache dei
 * Centroidi": the centroids of the previous denoising step initialise the
 * clustering of the next one). No seeding: up to max_iters rounds of the
 * Lloyd step of bsa_kmeans (same assignment and update rules) start from the
 * given centroids. A head stops after the first round that moves at most
 * tol_moves tokens (that round's update included): its later rounds do
 * nothing on the GPU. With tol_moves = 0 that round moved nothing, the
 * clustering is a fixed point and the result equals running every round.
 *   x          bf16 [B,H,N,d] (device), d in {64, 128}
 *   centroids  fp32 [B,H,C,d] in: initial centroids; out: final
 *   assign     int32 [B,H,N] out (-1 for padding rows); sizes int32 [B,H,C] out
 *   changes    int32 [B,H,max_iters] out: tokens whose assignment changed in
 *              each round (round 0 counts all n_valid tokens; 0 after the
 *              stopping round)
 *   ws         bsa_kmeans_workspace(...) bytes (device)
 *   1 <= C <= 1024, C <= n_valid, max_iters >= 1, tol_moves >= 0
 */
int bsa_kmeans_warm(const void* x, int B, int H, int N, int d, int n_valid,
                    int C, int max_iters, int tol_moves, float* centroids,
                    int32_t* assign,
                    int32_t* sizes, int32_t* changes, void* ws,
                    size_t ws_bytes, hipStream_t stream);

/* Workspace bytes needed by bsa_cluster_order. */
size_t bsa_cluster_order_workspace(int B, int H, int N, int C);

/*
 * Cluster-contiguous token order (Sparse VideoGen2 summary, Metodologia A,
 * "Permutazione"): a stable counting sort of the first n_valid tokens of
 * every (b,h) by cluster id.
 *   assign  int32 [B,H,N] (device), ids in [0, C) for the first n_valid rows
 *   perm    int32 [B,H,N] out: perm[new] = old; rows >= n_valid map to
 *           themselves
 *   start, len  int32 [B,H,C] out: cluster c occupies
 *           [start[c], start[c] + len[c]) of the new order
 */
int bsa_cluster_order(const int32_t* assign, int B, int H, int N, int n_valid,
                      int C, int32_t* perm, int32_t* start, int32_t* len,
                      void* ws, size_t ws_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* BSA_H */
