/*
 * ring_attn.h -- C ABI of the MI355X (gfx950) ring-attention step library.
 *
 * Ring attention keeps one query block per device and passes key/value blocks
 * around a ring of N devices; at step s device i holds key/value block
 * j = (i - s) mod N, and the partial softmax results are combined with the same
 * running-maximum softmax that blockwise attention uses inside one GPU
 * (Ultralytics glossary page "Ring Attention", section "Come funziona", and its
 * worked example).  The per-row running state is the maximum m, the
 * denominator l and the unnormalised output O ("Ring Attention simulation"
 * gist: running maxima and partial denominators per query row; GitHub issue
 * "A ring attention with flash attention kernel implementation": outputs, row
 * maxima and lse are stored and passed back in on the next ring pass).  Here
 * all N ring blocks live on one GPU as virtual devices.
 *
 * Conventions for every entry point:
 *  - Pointers are DEVICE pointers unless the comment says "host".
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream); all
 *    GPU work is enqueued on it asynchronously.
 *  - The caller owns every buffer; the library never allocates or frees memory.
 *  - Arguments are checked before anything is enqueued: a bad argument returns
 *    RA_E_ARG (or RA_E_UNSUPPORTED for a valid but unimplemented combination)
 *    with no side effects.  A failed launch returns RA_E_HIP.
 *  - An empty sequence (T = 0) or empty query block needs no buffers: its
 *    tensor, output, state and gradient pointers may be NULL, and the call
 *    returns RA_OK after the argument checks without any GPU work.
 *  - Tensors are [tokens, heads, head_dim] views with element strides; the
 *    head_dim stride must be 1.  This covers plain [T, H, d] tensors, striped
 *    ring blocks (token stride multiplied by N) and the packed [T, 3, H, d]
 *    qkv layout (flash-attention's "qkvpacked" inputs, named in the GitHub
 *    issue) without copies.
 *  - Query head h reads key/value head h / (Hq / Hkv) (grouped-query
 *    attention, named on the flash-attention scrape page).
 *  - Scores are scale * q.k; scale must be finite and > 0.
 *  - Supported: 16-bit inputs (bf16 or fp16, the two data types the
 *    flash-attention scrape page lists) with head_dim 64 or 128 (matrix-core
 *    path, fp32 accumulation); f32 inputs with head_dim 1..128 (exact fp32
 *    path).
 */
#ifndef RING_ATTN_H
#define RING_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    RA_OK = 0,
    RA_E_ARG = 1,          /* invalid argument (shape, stride, pointer, value) */
    RA_E_UNSUPPORTED = 2,  /* valid but not implemented (dtype / head_dim / mask combination) */
    RA_E_HIP = 3,          /* a HIP runtime call or kernel launch failed */
    RA_E_WORKSPACE = 4,    /* workspace missing or smaller than ring_attn_forward_workspace_size */
    RA_E_TOO_LARGE = 5     /* shapes need more scratch than ring_attn_forward_noalloc holds */
} ra_status;

/* Element types.  16-bit values round to nearest even wherever the library
 * writes them (P before the P.V product, 16-bit outputs and gradients). */
typedef enum { RA_F32 = 0, RA_BF16 = 1, RA_F16 = 2 } ra_dtype;

/* Masks act on global token positions t (query) and t' (key):
 *  NONE: every key; CAUSAL: t' <= t; DOC_CAUSAL: t' <= t and both in the same
 *  document, documents given by cu_seqlens (int32, n_docs + 1 cumulative
 *  lengths starting at 0, as described on the flash-attention scrape page). */
typedef enum { RA_MASK_NONE = 0, RA_MASK_CAUSAL = 1, RA_MASK_DOC_CAUSAL = 2 } ra_mask;

/* Assignment of tokens to the N ring blocks: CONTIGUOUS puts tokens
 * [i*B, (i+1)*B) in block i; STRIPED puts token t in block t mod N (the
 * glossary page's striped attention, which spreads every device's tokens over
 * the whole sequence to balance causal work). */
typedef enum { RA_LAYOUT_CONTIGUOUS = 0, RA_LAYOUT_STRIPED = 1 } ra_layout;

typedef struct {
    const void* data;      /* device pointer to element [0, 0, 0] */
    ra_dtype dtype;
    int64_t n_tok, n_head, head_dim;
    int64_t stride_tok, stride_head; /* element strides; head_dim stride is 1 */
} ra_tensor;

/* Work tallies of a forward pass.  A block pair is one (query block i, key
 * block j) visited at some ring step; a tile is tile_q query rows x tile_k key
 * columns of a block pair (the last tile on each side may be short).  SKIP: no
 * allowed (query, key) pair, never computed; FULL: every pair allowed,
 * computed without a mask; PARTIAL: computed with a per-element mask.
 * tile_q / tile_k: the tile shape counted.  ring_attn_forward's 16-bit
 * one-launch ring gives each work item the h query heads of a kv head that
 * share its key/value tiles (h the largest power of two <= 8 dividing
 * Hq / Hkv; grouped-query attention, named on the flash-attention scrape
 * page), and tiles of tile_q / h rows: its tallies count those (tile_q =
 * 256 / h); ring_attn_plan and ring_attn_tile_shape give the 256-row tile. */
typedef struct {
    int64_t block_pairs_visited, block_pairs_skipped, block_pairs_full, block_pairs_partial;
    int64_t tiles_skipped, tiles_full, tiles_partial;
    int64_t allowed_pairs;     /* (query, key) pairs per head that pass mask and ring */
    int32_t tile_q, tile_k;
} ra_stats;

/*
 * One ring step: the query block q_blk against one key/value block, updating
 * the running state in place.
 *   q_blk [Bq, Hq, d], k_blk / v_blk [Bk, Hkv, d]: same dtype, same d.
 *   O [Hq, Bq, d], m [Hq, Bq], l [Hq, Bq]: fp32, contiguous.  After the call,
 *     for every row: m = max over all keys seen so far of scale*q.k (-inf if
 *     none), l = sum of exp(scale*q.k - m), O = sum of exp(scale*q.k - m) v.
 *     With first_step != 0 the incoming state is ignored (treated as empty),
 *     so O/m/l need no initialisation.
 *   Positions for the mask: query row u sits at q_offset + u * pos_stride, key
 *     row w at kv_offset + w * pos_stride (pos_stride = 1 for contiguous
 *     blocks, N for striped ones).  DOC_CAUSAL needs pos_stride = 1 and
 *     cu_seqlens (device, n_docs + 1 entries) covering every position used.
 *   key_bits: nullable device pointer, 8-byte aligned: the key block's
 *     key-padding mask as ring_attn_pack_key_mask writes it (bit w % 32 of
 *     word w / 32 set when key row w takes part).  It belongs to the key
 *     block and travels with it around the ring.  Padded keys leave the
 *     tile tallies unchanged (they are masked inside the computed tiles).
 *   stats_dev: nullable device int64[3]; the step ADDS its tile counts
 *     {skipped, full, partial} (tile shape as ring_attn_tile_shape reports).
 */
ra_status ring_attn_step(const ra_tensor* q_blk, const ra_tensor* k_blk, const ra_tensor* v_blk,
                         float* O, float* m, float* l, int first_step, float scale,
                         ra_mask mask_mode, int64_t q_offset, int64_t kv_offset, int64_t pos_stride,
                         const int32_t* cu_seqlens, int32_t n_docs, const uint32_t* key_bits,
                         int64_t* stats_dev, void* stream);

/*
 * Key-padding mask of one key block as bits: key_bits[w / 32] bit w % 32 =
 * (key_valid[w * stride] != 0) for w < n_keys; 2 * ceil(n_keys / 64) words
 * are written (whole 64-key tiles, zero past n_keys).  Both pointers are
 * device pointers; key_bits 8-byte aligned.  A key-padding mask leaves out
 * the keys of padding tokens (GitHub issue "A ring attention with flash
 * attention kernel implementation": a comment names the key padding mask
 * beside the causal one); it combines with every ra_mask.
 */
ra_status ring_attn_pack_key_mask(const uint8_t* key_valid, int64_t n_keys, int64_t stride, uint32_t* key_bits,
                                  void* stream);

/*
 * Normalise a running state: out[u, h, :] = O[h, u, :] / l[h, u] and
 * lse[h, u] = m[h, u] + ln l[h, u]; a row with l = 0 (no key seen) gets
 * out = 0 and lse = -inf (the glossary page's worked example divides the
 * accumulated weighted values by the accumulated weights at the end).
 *   O [Hq, Bq, d], m/l [Hq, Bq] fp32 contiguous; out is written at
 *   out + u*out_stride_tok + h*out_stride_head (+ c), dtype out_dtype
 *   (16-bit types round to nearest even); lse nullable, [Hq, Bq] contiguous.
 */
ra_status ring_attn_finalize(const float* O, const float* m, const float* l, int64_t Hq, int64_t Bq,
                             int64_t d, void* out, ra_dtype out_dtype, int64_t out_stride_tok,
                             int64_t out_stride_head, float* lse, void* stream);

/*
 * Merge a normalised partial result into an accumulator through log-sum-exp
 * (GitHub issue: returning lse is what lets blockwise attention results be
 * combined): with w_x = exp(lse_x - max(lse_acc, lse_blk)),
 *   out_acc = (w_acc out_acc + w_blk out_blk) / (w_acc + w_blk),
 *   lse_acc = max + ln(w_acc + w_blk);
 * a side with lse = -inf has weight 0, both -inf gives out 0, lse -inf.
 *   out_acc / out_blk: [rows, Hq, d] contiguous, dtype `dtype`;
 *   lse_acc / lse_blk: [Hq, rows] fp32 contiguous.  Updated in place.
 */
ra_status ring_attn_merge(void* out_acc, float* lse_acc, const void* out_blk, const float* lse_blk,
                          ra_dtype dtype, int64_t Hq, int64_t rows, int64_t d, void* stream);

/* Bytes of device workspace ring_attn_forward needs for these shapes.  The
 * fp32 per-step state (O [T, Hq, d], m and l [Hq, T]) is included only when
 * the per-step path can run: fp32 inputs, prefetch != 0, n_blocks > 64, or
 * more query tiles x heads x blocks than fit an int32.  16-bit inputs
 * otherwise need the packed V^T, the chain tables and the key bits only. */
size_t ring_attn_forward_workspace_size(const ra_tensor* q, const ra_tensor* k, int32_t n_blocks,
                                        int32_t n_docs, int prefetch);

/*
 * The whole ring on one GPU: the sequence of T tokens is split into n_blocks
 * ring blocks (virtual devices) by `layout`; for s = 0 .. min(P, N) - 1 every
 * virtual device i runs one step against block (i - s) mod N, with P =
 * max_ring_passes (GitHub issue: the maximum number of ring passes; one pass
 * is one step).  Pairs the mask skips entirely are not run.  16-bit inputs
 * without prefetch: one launch runs the whole ring, every query tile of
 * every virtual device taking its device's blocks with the state kept on
 * chip, then writing its normalised output; as every block is resident it
 * takes them in ring order but the device's own block last (striped
 * layout: in ascending block order), the merged result being the same sum
 * in any order, rounding aside.  Otherwise one
 * launch per step covers every active virtual device, the state goes
 * through the workspace between steps, and a device's last active step
 * writes its normalised output.
 *   q [T, Hq, d], k/v [T, Hkv, d] (views allowed, e.g. of a packed qkv).
 *   out: [T, Hq, d] contiguous, out_dtype (RA_F32 always allowed; for 16-bit
 *     inputs also their own type).  lse: nullable, [Hq, T] fp32 (natural log).
 *   cu_seqlens_host: HOST pointer, n_docs + 1 entries, needed for DOC_CAUSAL
 *     (contiguous layout only); copied into the workspace.
 *   key_valid: nullable device pointer, T bytes: key token t takes part only
 *     if key_valid[t] != 0 (a key-padding mask, on top of mask_mode; rows
 *     left with no key get out 0, lse -inf).  Packed into the workspace as
 *     bits; the tallies in stats ignore it.
 *   prefetch != 0: one launch per step; every step's key/value blocks are
 *     first copied, on a side stream, into a double buffer in the workspace
 *     while the previous step computes (the ring's transfer of the next
 *     block, modelled on one GPU).  For fp32 inputs the results are
 *     bit-identical to prefetch = 0; for 16-bit inputs they agree to 16-bit rounding
 *     (the state hand-off changes the reference P is rounded against).
 *     Each GPU has one copy stream and one pair of event sets for this path:
 *     concurrent prefetch calls on one device (any host threads, any
 *     streams) enqueue one after another and their copies share that
 *     stream.
 *   stats: nullable HOST pointer; when given the call synchronises `stream`
 *     and fills it.
 * Host tables (the chain tables the call plans, cu_seqlens) reach the device
 * through pinned host buffers of the library (a ring of 8 per GPU, allocated
 * on first use and grown as needed, held until the process ends) by copies
 * enqueued on `stream`: the caller's host arrays may be reused as soon as the
 * call returns, and the host may run up to 8 calls ahead of the GPU before a
 * call waits for the copies of an earlier one.  The staging is per call, so a
 * call is not meant for capture into a HIP graph (a replay would copy
 * whatever a later call left in the buffer).
 */
ra_status ring_attn_forward(const ra_tensor* q, const ra_tensor* k, const ra_tensor* v, void* out,
                            ra_dtype out_dtype, float* lse, int32_t n_blocks, ra_layout layout,
                            ra_mask mask_mode, int32_t max_ring_passes, const int32_t* cu_seqlens_host,
                            int32_t n_docs, const uint8_t* key_valid, float scale, int prefetch, void* workspace,
                            size_t workspace_bytes, ra_stats* stats, void* stream);

/*
 * ring_attn_forward without any device allocation, for callers that cannot
 * allocate: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.  Same arguments and results as ring_attn_forward
 * with prefetch = 0, except that the workspace is a fixed array of
 * ring_attn_forward_noalloc_scratch_bytes() (64 MiB) of device memory inside
 * the library, one per GPU, which each GPU holds until the process ends.
 * Shapes whose forward workspace (ring_attn_forward_workspace_size with
 * prefetch = 0) exceeds it return RA_E_TOO_LARGE before any GPU work.  The
 * caller still passes every input and output.  The call makes no device
 * or pinned host allocation: its host-side planning uses ordinary host
 * memory, and its tables are copied to the array straight from that memory.
 * Every call on one GPU uses that GPU's one array, which keeps the last
 * call's contents: calls that overlap on one GPU (several streams or host
 * threads) race and must be ordered by the caller.
 */
ra_status ring_attn_forward_noalloc(const ra_tensor* q, const ra_tensor* k, const ra_tensor* v, void* out,
                                    ra_dtype out_dtype, float* lse, int32_t n_blocks, ra_layout layout,
                                    ra_mask mask_mode, int32_t max_ring_passes,
                                    const int32_t* cu_seqlens_host, int32_t n_docs,
                                    const uint8_t* key_valid, float scale, ra_stats* stats, void* stream);

/* Bytes of the fixed scratch ring_attn_forward_noalloc works in. */
size_t ring_attn_forward_noalloc_scratch_bytes(void);

/*
 * Test hook, for checking the prefetch path's event ordering (not for
 * production use): from now on every prefetch forward enqueues a bounded
 * wait of copy_delay_us microseconds on its copy stream before each step's
 * copies, and of compute_delay_us on the caller's stream before each step's
 * compute (0 = none, the default; at most 100000 each, else RA_E_ARG).  The
 * results must not change: each step's compute waits for its copies, and
 * each copy waits until the step that last read its buffer is done (the
 * "Ring Attention simulation" gist waits twice per step so that a receive
 * buffer is never read before it is written nor overwritten while read).
 * Process-wide; no GPU work at the call.
 */
ra_status ring_attn_test_prefetch_delays(uint32_t copy_delay_us, uint32_t compute_delay_us);

/* Bytes of device workspace ring_attn_backward needs for these shapes. */
size_t ring_attn_backward_workspace_size(const ra_tensor* q, int32_t n_blocks, int32_t n_docs);

/*
 * Gradients of ring_attn_forward's output for a given output gradient
 * (GitHub issue "A ring attention with flash attention kernel
 * implementation": the backward pass produces the gradients of full
 * attention and reuses the forward's lse).  With P_tj = exp(scale q_t.k_j -
 * lse_t) over the pairs the forward attends (its mask and its
 * max_ring_passes) and D_t = dout_t . out_t:
 *   dS_tj = P_tj (dout_t . v_j - D_t),
 *   dq_t = scale sum_j dS_tj k_j,  dk_j = scale sum_t dS_tj q_t,
 *   dv_j = sum_t P_tj dout_t
 * (the chain rule through the row softmax); a grouped kv head sums over the
 * query heads that read it.  No atomics: the results do not depend on
 * scheduling.
 *   q, k, v, n_blocks, layout, mask_mode, max_ring_passes, cu_seqlens_host,
 *     n_docs, key_valid, scale: as given to ring_attn_forward.  16-bit
 *     inputs (bf16 or fp16, all the same type) with head_dim 64 or 128,
 *     n_blocks <= 64, T < 2^31 and T / n_blocks < 2^21 only
 *     (RA_E_UNSUPPORTED otherwise).  A padded key gets dk = dv = 0.
 *   out: the forward's output [T, Hq, d] view, f32 or the inputs' type
 *     (16-byte aligned rows); dout: [T, Hq, d] view of the inputs' type.
 *   lse: the forward's lse, [Hq, T] fp32 (natural log).
 *   dq [T, Hq, d], dk / dv [T, Hkv, d]: contiguous, 16-byte aligned,
 *     grad_dtype (fp32 or the inputs' type), every element written.
 *   workspace: ring_attn_backward_workspace_size bytes, 256-byte aligned.
 * Its host tables travel as ring_attn_forward's do (pinned buffers, the same
 * ring per GPU).
 */
ra_status ring_attn_backward(const ra_tensor* q, const ra_tensor* k, const ra_tensor* v, const ra_tensor* out,
                             const ra_tensor* dout, const float* lse, void* dq, void* dk, void* dv,
                             ra_dtype grad_dtype, int32_t n_blocks, ra_layout layout, ra_mask mask_mode,
                             int32_t max_ring_passes, const int32_t* cu_seqlens_host, int32_t n_docs,
                             const uint8_t* key_valid, float scale, void* workspace, size_t workspace_bytes,
                             void* stream);

/*
 * Host-only planning (no GPU work): fills `stats` with the tallies and the
 * allowed-pair count that ring_attn_forward would produce for these shapes,
 * from the exact per-tile mask classification.  dtype and head_dim select the
 * kernel (and so the tile shape).  cu_seqlens_host as for ring_attn_forward.
 */
ra_status ring_attn_plan(int64_t T, int32_t n_blocks, ra_layout layout, ra_mask mask_mode,
                         int32_t max_ring_passes, const int32_t* cu_seqlens_host, int32_t n_docs,
                         ra_dtype dtype, int64_t head_dim, ra_stats* stats);

/* Tile shape (query rows x key columns) of the kernel for dtype / head_dim;
 * returns RA_E_UNSUPPORTED when no kernel covers the combination. */
ra_status ring_attn_tile_shape(ra_dtype dtype, int64_t head_dim, int32_t* tile_q, int32_t* tile_k);

const char* ring_attn_status_string(ra_status s);

#ifdef __cplusplus
}
#endif
#endif /* RING_ATTN_H */
