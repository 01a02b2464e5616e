/*
 * ring_oracle.c -- plain fp64 CPU oracle for the ring-attention step.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path links, loads or calls
 * this file; only the test suite, the smoke check and the benchmark's CPU
 * baseline do.  It shares no code, header or constant with the HIP library.
 *
 * What it computes is the plain definition of (masked) softmax attention, with
 * the ring-attention block structure entering only through which keys a query
 * may see:
 *
 *   Ultralytics glossary page "Ring Attention", section "Come funziona": after
 *   the N ring steps each query block has met every key/value block and the
 *   result equals full softmax(q k^T / sqrt(d)) v; the worked example's code
 *   compares against exactly that.
 *   "Ring Attention simulation" gist (ring_attention_simulation.py): the same
 *   equality with the scaling factor omitted.
 *   Zhihu article "Attention的分块计算", section on local vs. global softmax:
 *   softmax is unchanged when a constant is subtracted from every score, and
 *   the usual implementation subtracts the maximum before exponentiating.
 *
 * For one query row t (head h, KV head g = h / (Hq/Hkv)) the oracle
 *   1. builds the allowed key set A(t) = { t' : mask(t,t') and visible(t,t') },
 *   2. s_j = scale * sum_c q[t,h,c] k[j,g,c]            for j in A(t),
 *   3. M = max_j s_j,  w_j = exp(s_j - M),  L = sum_j w_j,
 *   4. O = sum_j w_j v[j,g,:],  out = O / L,  lse = M + ln L,
 * and for an empty A(t): M = -inf, L = 0, O = 0, out = 0, lse = -inf.
 * (M, L, O) is also the running state a ring step carries (gist: running
 * maximum and partial denominator per query row; the GitHub issue
 * "A ring attention with flash attention kernel implementation": outputs, row
 * maxima and lse are stored and handed back on the next ring pass).
 *
 * Masks act on global token positions:
 *   none:        every key;
 *   causal:      t' <= t (the glossary page: devices holding early query
 *                blocks skip most key blocks under a causal mask);
 *   doc-causal:  t' <= t and t, t' in the same document, documents given by
 *                cumulative lengths cu_seqlens of shape (n_docs + 1,) (the
 *                flash-attention scrape page's description of cu_seqlens).
 * and, with a key-padding mask key_valid (one byte per key, nonzero = a real
 * token), every key with key_valid = 0 is left out as well (GitHub issue "A
 * ring attention with flash attention kernel implementation": a comment
 * names the key padding mask beside the causal one).  The whole-sequence
 * entry points index key_valid by global position t', the block entry point
 * by the key's row in its block.  The tile tallies below ignore it.
 * Ring visibility with N blocks and P = max ring passes (GitHub issue: the
 * maximum number of ring passes): at step s the device holding query block b
 * holds key block (b - s) mod N (glossary page code), and only steps
 * s < min(P, N) run, so t' is visible from t iff (blk(t) - blk(t')) mod N <
 * min(P, N); blk(t) = t / B for contiguous blocks of B = T/N tokens and
 * t mod N for the striped assignment (glossary page: striped attention gives
 * every device tokens spread evenly over the sequence).
 *
 * Tile tallies: for every visited (query block, key block) pair and every
 * tile of tile_q query rows x tile_k key columns (the last tile of each side
 * may be short), the tile is SKIP if no pair in it is allowed, FULL if all
 * are, else PARTIAL; a block pair is SKIP / FULL when all its tiles are, else
 * PARTIAL.  Brute force over every pair.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { RO_F32 = 0, RO_BF16 = 1 };
enum { RO_MASK_NONE = 0, RO_MASK_CAUSAL = 1, RO_MASK_DOC_CAUSAL = 2 };
enum { RO_LAYOUT_CONTIGUOUS = 0, RO_LAYOUT_STRIPED = 1 };
enum { RO_OK = 0, RO_BAD_ARG = 1, RO_NO_MEM = 2 };

/* One element of a [tokens, heads, dim] tensor, decoded to fp64.  bf16 is the
 * top half of an IEEE binary32, so the decode is exact. */
static double load_elem(const void* base, int dtype, int64_t idx) {
    if (dtype == RO_F32) return (double)((const float*)base)[idx];
    uint32_t bits = ((uint32_t)((const uint16_t*)base)[idx]) << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

typedef struct {
    const void* ptr;
    int dtype;
    int64_t stride_tok, stride_head; /* element strides; dim stride is 1 */
} ro_view;

static double view_at(const ro_view* v, int64_t tok, int64_t head, int64_t c) {
    return load_elem(v->ptr, v->dtype, tok * v->stride_tok + head * v->stride_head + c);
}

/* Document index of every position 0..T-1 from cu_seqlens. */
static int32_t* make_doc_of(const int32_t* cu, int64_t n_docs, int64_t T) {
    int32_t* doc_of = (int32_t*)malloc(sizeof(int32_t) * (size_t)(T > 0 ? T : 1));
    if (!doc_of) return NULL;
    for (int64_t t = 0; t < T; t++) doc_of[t] = -1;
    for (int64_t i = 0; i < n_docs; i++)
        for (int64_t t = cu[i]; t < cu[i + 1]; t++) doc_of[t] = (int32_t)i;
    return doc_of;
}

static int mask_allows(int mask, const int32_t* doc_of, int64_t t, int64_t tk) {
    if (mask == RO_MASK_NONE) return 1;
    if (tk > t) return 0;
    if (mask == RO_MASK_DOC_CAUSAL && doc_of[tk] != doc_of[t]) return 0;
    return 1;
}

typedef struct {
    int64_t T, n_blocks, passes; /* passes = min(P, N) */
    int layout;
} ro_ring;

static int64_t block_of(const ro_ring* r, int64_t t) {
    if (r->layout == RO_LAYOUT_STRIPED) return t % r->n_blocks;
    return t / (r->T / r->n_blocks);
}

static int ring_visible(const ro_ring* r, int64_t t, int64_t tk) {
    int64_t step = ((block_of(r, t) - block_of(r, tk)) % r->n_blocks + r->n_blocks) % r->n_blocks;
    return step < r->passes;
}

/* Steps 2-4 above for one query row against the keys listed in idx[0..n). */
static void attend_one(const ro_view* q, int64_t q_tok, int64_t h, const ro_view* k,
                       const ro_view* v, int64_t g, int64_t d, double scale,
                       const int64_t* idx, int64_t n, double* sbuf,
                       double* out, double* lse, double* m_out, double* l_out, double* O_out) {
    for (int64_t c = 0; c < d; c++) O_out[c] = 0.0;
    if (n == 0) {
        for (int64_t c = 0; c < d; c++) out[c] = 0.0;
        *lse = -INFINITY;
        *m_out = -INFINITY;
        *l_out = 0.0;
        return;
    }
    double M = -INFINITY;
    for (int64_t a = 0; a < n; a++) {
        double s = 0.0;
        for (int64_t c = 0; c < d; c++) s += view_at(q, q_tok, h, c) * view_at(k, idx[a], g, c);
        s *= scale;
        sbuf[a] = s;
        if (s > M) M = s;
    }
    double L = 0.0;
    for (int64_t a = 0; a < n; a++) {
        double w = exp(sbuf[a] - M);
        L += w;
        for (int64_t c = 0; c < d; c++) O_out[c] += w * view_at(v, idx[a], g, c);
    }
    for (int64_t c = 0; c < d; c++) out[c] = O_out[c] / L;
    *lse = M + log(L);
    *m_out = M;
    *l_out = L;
}

/*
 * Whole-sequence attention under the ring's visibility for the requested rows.
 * q: [T, Hq, d], k/v: [T, Hkv, d] (element strides given), positions 0..T-1.
 * rows: n_rows (head, token) pairs; outputs per row: out[d], lse, m, l, O[d]
 * (O is the unnormalised state sum w_j v_j; any output pointer may be NULL).
 */
int ro_forward_rows(const void* q, const void* k, const void* v, int dtype,
                    int64_t T, int64_t Hq, int64_t Hkv, int64_t d,
                    int64_t q_st, int64_t q_sh, int64_t k_st, int64_t k_sh,
                    int64_t v_st, int64_t v_sh, double scale, int mask, int layout,
                    int64_t n_blocks, int64_t max_ring_passes,
                    const int32_t* cu_seqlens, int64_t n_docs, const uint8_t* key_valid,
                    int64_t n_rows, const int64_t* row_head, const int64_t* row_tok,
                    double* out, double* lse, double* m, double* l, double* O) {
    if (T < 0 || Hq < 1 || Hkv < 1 || Hq % Hkv || d < 1 || n_blocks < 1 || max_ring_passes < 1)
        return RO_BAD_ARG;
    if (T % n_blocks) return RO_BAD_ARG;
    if (mask == RO_MASK_DOC_CAUSAL && (!cu_seqlens || n_docs < 1 || cu_seqlens[0] != 0 ||
                                       cu_seqlens[n_docs] != T))
        return RO_BAD_ARG;
    ro_view qv = {q, dtype, q_st, q_sh}, kv = {k, dtype, k_st, k_sh}, vv = {v, dtype, v_st, v_sh};
    ro_ring ring = {T, n_blocks, max_ring_passes < n_blocks ? max_ring_passes : n_blocks, layout};
    int32_t* doc_of = NULL;
    if (mask == RO_MASK_DOC_CAUSAL) {
        doc_of = make_doc_of(cu_seqlens, n_docs, T);
        if (!doc_of) return RO_NO_MEM;
    }
    int64_t group = Hq / Hkv;
    int status = RO_OK;
#pragma omp parallel
    {
        int64_t* idx = (int64_t*)malloc(sizeof(int64_t) * (size_t)(T > 0 ? T : 1));
        double* sbuf = (double*)malloc(sizeof(double) * (size_t)(T > 0 ? T : 1));
        double* Obuf = (double*)malloc(sizeof(double) * (size_t)d);
        double* obuf = (double*)malloc(sizeof(double) * (size_t)d);
        if (!idx || !sbuf || !Obuf || !obuf) {
#pragma omp atomic write
            status = RO_NO_MEM;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int64_t r = 0; r < n_rows; r++) {
                int64_t h = row_head[r], t = row_tok[r];
                int64_t n = 0;
                for (int64_t tk = 0; tk < T; tk++)
                    if (mask_allows(mask, doc_of, t, tk) && ring_visible(&ring, t, tk) &&
                        (!key_valid || key_valid[tk]))
                        idx[n++] = tk;
                double lse_r, m_r, l_r;
                attend_one(&qv, t, h, &kv, &vv, h / group, d, scale, idx, n, sbuf, obuf, &lse_r,
                           &m_r, &l_r, Obuf);
                if (out) memcpy(out + r * d, obuf, sizeof(double) * (size_t)d);
                if (O) memcpy(O + r * d, Obuf, sizeof(double) * (size_t)d);
                if (lse) lse[r] = lse_r;
                if (m) m[r] = m_r;
                if (l) l[r] = l_r;
            }
        }
        free(idx);
        free(sbuf);
        free(Obuf);
        free(obuf);
    }
    free(doc_of);
    return status;
}

/*
 * One query block against one key/value block, with explicit global
 * positions: q rows u = 0..nq-1 sit at q_pos[u], keys w = 0..nk-1 at k_pos[w].
 * This is what a single ring step sees: the mask acts on global positions and
 * there is no ring-visibility filter (the step is told which block it holds).
 * Outputs are laid out [Hq, nq] (lse, m, l) and [Hq, nq, d] (out, O).
 * doc_T is the length covered by cu_seqlens (needed only for doc-causal).
 */
int ro_block_rows(const void* q, const void* k, const void* v, int dtype,
                  int64_t nq, int64_t nk, int64_t Hq, int64_t Hkv, int64_t d,
                  int64_t q_st, int64_t q_sh, int64_t k_st, int64_t k_sh,
                  int64_t v_st, int64_t v_sh, const int64_t* q_pos, const int64_t* k_pos,
                  double scale, int mask, const int32_t* cu_seqlens, int64_t n_docs, int64_t doc_T,
                  const uint8_t* key_valid, double* out, double* lse, double* m, double* l, double* O) {
    if (nq < 0 || nk < 0 || Hq < 1 || Hkv < 1 || Hq % Hkv || d < 1) return RO_BAD_ARG;
    int32_t* doc_of = NULL;
    if (mask == RO_MASK_DOC_CAUSAL) {
        if (!cu_seqlens || n_docs < 1 || cu_seqlens[0] != 0 || cu_seqlens[n_docs] != doc_T)
            return RO_BAD_ARG;
        for (int64_t u = 0; u < nq; u++) if (q_pos[u] < 0 || q_pos[u] >= doc_T) return RO_BAD_ARG;
        for (int64_t w = 0; w < nk; w++) if (k_pos[w] < 0 || k_pos[w] >= doc_T) return RO_BAD_ARG;
        doc_of = make_doc_of(cu_seqlens, n_docs, doc_T);
        if (!doc_of) return RO_NO_MEM;
    }
    ro_view qv = {q, dtype, q_st, q_sh}, kv = {k, dtype, k_st, k_sh}, vv = {v, dtype, v_st, v_sh};
    int64_t group = Hq / Hkv;
    int status = RO_OK;
#pragma omp parallel
    {
        int64_t* idx = (int64_t*)malloc(sizeof(int64_t) * (size_t)(nk > 0 ? nk : 1));
        double* sbuf = (double*)malloc(sizeof(double) * (size_t)(nk > 0 ? nk : 1));
        double* obuf = (double*)malloc(sizeof(double) * (size_t)d);
        double* Obuf = (double*)malloc(sizeof(double) * (size_t)d);
        if (!idx || !sbuf || !obuf || !Obuf) {
#pragma omp atomic write
            status = RO_NO_MEM;
        } else {
#pragma omp for schedule(dynamic, 4)
            for (int64_t r = 0; r < Hq * nq; r++) {
                int64_t h = r / nq, u = r % nq;
                int64_t n = 0;
                for (int64_t w = 0; w < nk; w++)
                    if (mask_allows(mask, doc_of, q_pos[u], k_pos[w]) && (!key_valid || key_valid[w])) idx[n++] = w;
                double lse_r, m_r, l_r;
                attend_one(&qv, u, h, &kv, &vv, h / group, d, scale, idx, n, sbuf, obuf, &lse_r, &m_r,
                           &l_r, Obuf);
                if (out) memcpy(out + r * d, obuf, sizeof(double) * (size_t)d);
                if (O) memcpy(O + r * d, Obuf, sizeof(double) * (size_t)d);
                if (lse) lse[r] = lse_r;
                if (m) m[r] = m_r;
                if (l) l[r] = l_r;
            }
        }
        free(idx);
        free(sbuf);
        free(obuf);
        free(Obuf);
    }
    free(doc_of);
    return status;
}

/*
 * Tile tallies for the ring forward, brute force over every (query, key) pair
 * of every visited block pair.  counts[7] = {block pairs visited, skipped,
 * full, partial, tiles skipped, tiles full, tiles partial}.
 */
int ro_tile_tallies(int64_t T, int64_t n_blocks, int layout, int mask, int64_t max_ring_passes,
                    const int32_t* cu_seqlens, int64_t n_docs, int64_t tile_q, int64_t tile_k,
                    int64_t* counts) {
    if (T < 0 || n_blocks < 1 || T % n_blocks || max_ring_passes < 1 || tile_q < 1 || tile_k < 1)
        return RO_BAD_ARG;
    if (mask == RO_MASK_DOC_CAUSAL && (!cu_seqlens || n_docs < 1 || cu_seqlens[0] != 0 ||
                                       cu_seqlens[n_docs] != T))
        return RO_BAD_ARG;
    int32_t* doc_of = NULL;
    if (mask == RO_MASK_DOC_CAUSAL) {
        doc_of = make_doc_of(cu_seqlens, n_docs, T);
        if (!doc_of) return RO_NO_MEM;
    }
    const int64_t N = n_blocks, B = T / N;
    const int64_t passes = max_ring_passes < N ? max_ring_passes : N;
    const int64_t nqt = (B + tile_q - 1) / tile_q, nkt = (B + tile_k - 1) / tile_k;
    int64_t c[7] = {0, 0, 0, 0, 0, 0, 0};
    for (int64_t i = 0; i < N; i++) {
        for (int64_t s = 0; s < passes; s++) {
            int64_t j = ((i - s) % N + N) % N;
            int64_t t_skip = 0, t_full = 0, t_part = 0;
#pragma omp parallel for collapse(2) schedule(dynamic, 1) reduction(+ : t_skip, t_full, t_part)
            for (int64_t a = 0; a < nqt; a++) {
                for (int64_t b = 0; b < nkt; b++) {
                    /* every tile holds at least one pair, so "none allowed" and
                       "none denied" cannot both hold */
                    int any_allowed = 0, any_denied = 0;
                    for (int64_t u = a * tile_q; u < (a + 1) * tile_q && u < B; u++) {
                        int64_t t = layout == RO_LAYOUT_STRIPED ? u * N + i : i * B + u;
                        for (int64_t w = b * tile_k; w < (b + 1) * tile_k && w < B; w++) {
                            int64_t tk = layout == RO_LAYOUT_STRIPED ? w * N + j : j * B + w;
                            if (mask_allows(mask, doc_of, t, tk)) any_allowed = 1;
                            else any_denied = 1;
                            if (any_allowed && any_denied) goto classified;
                        }
                    }
                classified:
                    if (!any_allowed) t_skip++;
                    else if (!any_denied) t_full++;
                    else t_part++;
                }
            }
            c[0]++;
            if (t_full == 0 && t_part == 0) c[1]++;
            else if (t_skip == 0 && t_part == 0) c[2]++;
            else c[3]++;
            c[4] += t_skip;
            c[5] += t_full;
            c[6] += t_part;
        }
    }
    free(doc_of);
    memcpy(counts, c, sizeof c);
    return RO_OK;
}

/*
 * Number of allowed (query, key) pairs per head over the whole ring forward,
 * brute force over every pair: sum over t of |A(t)|.  The algorithmic FLOP of
 * the two contractions is 4 * d * Hq times this.
 */
int ro_allowed_pairs(int64_t T, int64_t n_blocks, int layout, int mask, int64_t max_ring_passes,
                     const int32_t* cu_seqlens, int64_t n_docs, int64_t* pairs) {
    if (T < 0 || n_blocks < 1 || T % n_blocks || max_ring_passes < 1) return RO_BAD_ARG;
    if (mask == RO_MASK_DOC_CAUSAL && (!cu_seqlens || n_docs < 1 || cu_seqlens[0] != 0 ||
                                       cu_seqlens[n_docs] != T))
        return RO_BAD_ARG;
    int32_t* doc_of = NULL;
    if (mask == RO_MASK_DOC_CAUSAL) {
        doc_of = make_doc_of(cu_seqlens, n_docs, T);
        if (!doc_of) return RO_NO_MEM;
    }
    ro_ring ring = {T, n_blocks, max_ring_passes < n_blocks ? max_ring_passes : n_blocks, layout};
    int64_t total = 0;
#pragma omp parallel for schedule(dynamic, 64) reduction(+ : total)
    for (int64_t t = 0; t < T; t++)
        for (int64_t tk = 0; tk < T; tk++)
            total += mask_allows(mask, doc_of, t, tk) && ring_visible(&ring, t, tk);
    free(doc_of);
    *pairs = total;
    return RO_OK;
}

/*
 * Gradients of the ring forward above with respect to q, k and v, given the
 * gradient dout of its output (GitHub issue "A ring attention with flash
 * attention kernel implementation": the backward pass of ring attention
 * yields the gradients of full attention, and the saved lse is what lets the
 * backward recompute the probabilities).  For one query row t of head h
 * (KV head g) with allowed keys A(t), P_j = exp(s_j - M) / L and
 * out = sum_j P_j v_j, so by the chain rule
 *   dv_j     += P_j dout
 *   dP_j      = dout . v_j
 *   dS_j      = P_j (dP_j - D),   D = sum_j P_j dP_j = dout . out
 *   dq       += scale sum_j dS_j k_j
 *   dk_j     += scale dS_j q
 * (the softmax Jacobian is diag(P) - P P^T).  Rows with no allowed key give
 * no gradient.  backward_row adds one row's terms: dq_row always, dk / dv
 * when non-null.
 */
typedef struct {
    const ro_view *q, *k, *v, *dout;
    const ro_ring* ring;
    const int32_t* doc_of;
    const uint8_t* key_valid;  /* nullable, by global position */
    int mask;
    int64_t T, Hkv, d;
    double scale;
} ro_bwd_ctx;

static void backward_row(const ro_bwd_ctx* c, int64_t t, int64_t h, int64_t g, int64_t* idx, double* sbuf,
                         double* Obuf, double* obuf, double* dq_row, double* dk, double* dv) {
    const int64_t T = c->T, d = c->d, Hkv = c->Hkv;
    int64_t n = 0;
    for (int64_t tk = 0; tk < T; tk++)
        if (mask_allows(c->mask, c->doc_of, t, tk) && ring_visible(c->ring, t, tk) &&
            (!c->key_valid || c->key_valid[tk]))
            idx[n++] = tk;
    if (n == 0) return;
    double lse_r, m_r, l_r;
    attend_one(c->q, t, h, c->k, c->v, g, d, c->scale, idx, n, sbuf, obuf, &lse_r, &m_r, &l_r, Obuf);
    double D = 0.0;
    for (int64_t x = 0; x < d; x++) D += view_at(c->dout, t, h, x) * obuf[x];
    for (int64_t a = 0; a < n; a++) {
        int64_t j = idx[a];
        double p = exp(sbuf[a] - m_r) / l_r;
        double dp = 0.0;
        for (int64_t x = 0; x < d; x++) dp += view_at(c->dout, t, h, x) * view_at(c->v, j, g, x);
        double ds = p * (dp - D);
        for (int64_t x = 0; x < d; x++) dq_row[x] += c->scale * ds * view_at(c->k, j, g, x);
        if (dk) {
            double* dkr = dk + (j * Hkv + g) * d;
            double* dvr = dv + (j * Hkv + g) * d;
            for (int64_t x = 0; x < d; x++) {
                dkr[x] += c->scale * ds * view_at(c->q, t, h, x);
                dvr[x] += p * view_at(c->dout, t, h, x);
            }
        }
    }
}

static int bwd_check(int64_t T, int64_t Hq, int64_t Hkv, int64_t d, int mask, int64_t n_blocks,
                     int64_t max_ring_passes, const int32_t* cu_seqlens, int64_t n_docs) {
    if (T < 0 || Hq < 1 || Hkv < 1 || Hq % Hkv || d < 1 || n_blocks < 1 || max_ring_passes < 1)
        return RO_BAD_ARG;
    if (T % n_blocks) return RO_BAD_ARG;
    if (mask == RO_MASK_DOC_CAUSAL && (!cu_seqlens || n_docs < 1 || cu_seqlens[0] != 0 ||
                                       cu_seqlens[n_docs] != T))
        return RO_BAD_ARG;
    return RO_OK;
}

/* Full gradients: fp64 arrays dq [T, Hq, d], dk and dv [T, Hkv, d] (dense,
 * overwritten); the work is split over KV heads so that the dk / dv sums of
 * one head stay in one thread. */
int ro_backward(const void* q, const void* k, const void* v, const void* dout, int dtype, int dout_dtype,
                int64_t T, int64_t Hq, int64_t Hkv, int64_t d,
                int64_t q_st, int64_t q_sh, int64_t k_st, int64_t k_sh,
                int64_t v_st, int64_t v_sh, int64_t o_st, int64_t o_sh,
                double scale, int mask, int layout, int64_t n_blocks, int64_t max_ring_passes,
                const int32_t* cu_seqlens, int64_t n_docs, const uint8_t* key_valid,
                double* dq, double* dk, double* dv) {
    int rc = bwd_check(T, Hq, Hkv, d, mask, n_blocks, max_ring_passes, cu_seqlens, n_docs);
    if (rc != RO_OK) return rc;
    ro_view qv = {q, dtype, q_st, q_sh}, kv = {k, dtype, k_st, k_sh}, vv = {v, dtype, v_st, v_sh};
    ro_view ov = {dout, dout_dtype, o_st, o_sh};
    ro_ring ring = {T, n_blocks, max_ring_passes < n_blocks ? max_ring_passes : n_blocks, layout};
    int32_t* doc_of = NULL;
    if (mask == RO_MASK_DOC_CAUSAL) {
        doc_of = make_doc_of(cu_seqlens, n_docs, T);
        if (!doc_of) return RO_NO_MEM;
    }
    ro_bwd_ctx c = {&qv, &kv, &vv, &ov, &ring, doc_of, key_valid, mask, T, Hkv, d, scale};
    memset(dq, 0, sizeof(double) * (size_t)(T * Hq * d));
    memset(dk, 0, sizeof(double) * (size_t)(T * Hkv * d));
    memset(dv, 0, sizeof(double) * (size_t)(T * Hkv * d));
    int64_t group = Hq / Hkv;
    int status = RO_OK;
#pragma omp parallel
    {
        int64_t* idx = (int64_t*)malloc(sizeof(int64_t) * (size_t)(T > 0 ? T : 1));
        double* sbuf = (double*)malloc(sizeof(double) * (size_t)(T > 0 ? T : 1));
        double* Obuf = (double*)malloc(sizeof(double) * (size_t)d);
        double* obuf = (double*)malloc(sizeof(double) * (size_t)d);
        if (!idx || !sbuf || !Obuf || !obuf) {
#pragma omp atomic write
            status = RO_NO_MEM;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int64_t g = 0; g < Hkv; g++)
                for (int64_t h = g * group; h < (g + 1) * group; h++)
                    for (int64_t t = 0; t < T; t++)
                        backward_row(&c, t, h, g, idx, sbuf, Obuf, obuf, dq + (t * Hq + h) * d, dk, dv);
        }
        free(idx);
        free(sbuf);
        free(Obuf);
        free(obuf);
    }
    free(doc_of);
    return status;
}

/* The terms of selected query rows only: row r is query head row_head[r] at
 * token row_tok[r] (each (head, token) listed once).  dq_rows [n_rows, d]
 * gets those rows' dq (a row's dq depends on that row alone, so these equal
 * the full gradients' rows); dk / dv, when non-null, [T, Hkv, d], get the
 * sums of those rows' terms only, which are the full gradients when dout is
 * zero on every other row.  dk / dv are summed serially in row order. */
int ro_backward_rows(const void* q, const void* k, const void* v, const void* dout, int dtype, int dout_dtype,
                        int64_t T, int64_t Hq, int64_t Hkv, int64_t d,
                        int64_t q_st, int64_t q_sh, int64_t k_st, int64_t k_sh,
                        int64_t v_st, int64_t v_sh, int64_t o_st, int64_t o_sh,
                        double scale, int mask, int layout, int64_t n_blocks, int64_t max_ring_passes,
                        const int32_t* cu_seqlens, int64_t n_docs, const uint8_t* key_valid,
                        const int64_t* row_head, const int64_t* row_tok, int64_t n_rows, double* dq_rows,
                        double* dk, double* dv) {
    int rc = bwd_check(T, Hq, Hkv, d, mask, n_blocks, max_ring_passes, cu_seqlens, n_docs);
    if (rc != RO_OK) return rc;
    for (int64_t r = 0; r < n_rows; r++)
        if (row_head[r] < 0 || row_head[r] >= Hq || row_tok[r] < 0 || row_tok[r] >= T) return RO_BAD_ARG;
    ro_view qv = {q, dtype, q_st, q_sh}, kv = {k, dtype, k_st, k_sh}, vv = {v, dtype, v_st, v_sh};
    ro_view ov = {dout, dout_dtype, o_st, o_sh};
    ro_ring ring = {T, n_blocks, max_ring_passes < n_blocks ? max_ring_passes : n_blocks, layout};
    int32_t* doc_of = NULL;
    if (mask == RO_MASK_DOC_CAUSAL) {
        doc_of = make_doc_of(cu_seqlens, n_docs, T);
        if (!doc_of) return RO_NO_MEM;
    }
    ro_bwd_ctx c = {&qv, &kv, &vv, &ov, &ring, doc_of, key_valid, mask, T, Hkv, d, scale};
    memset(dq_rows, 0, sizeof(double) * (size_t)(n_rows * d));
    if (dk) memset(dk, 0, sizeof(double) * (size_t)(T * Hkv * d));
    if (dv) memset(dv, 0, sizeof(double) * (size_t)(T * Hkv * d));
    if (!dk != !dv) {
        free(doc_of);
        return RO_BAD_ARG;
    }
    int64_t group = Hq / Hkv;
    int status = RO_OK;
#pragma omp parallel if (!dk)
    {
        int64_t* idx = (int64_t*)malloc(sizeof(int64_t) * (size_t)(T > 0 ? T : 1));
        double* sbuf = (double*)malloc(sizeof(double) * (size_t)(T > 0 ? T : 1));
        double* Obuf = (double*)malloc(sizeof(double) * (size_t)d);
        double* obuf = (double*)malloc(sizeof(double) * (size_t)d);
        if (!idx || !sbuf || !Obuf || !obuf) {
#pragma omp atomic write
            status = RO_NO_MEM;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int64_t r = 0; r < n_rows; r++)
                backward_row(&c, row_tok[r], row_head[r], row_head[r] / group, idx, sbuf, Obuf, obuf,
                             dq_rows + r * d, dk, dv);
        }
        free(idx);
        free(sbuf);
        free(Obuf);
        free(obuf);
    }
    free(doc_of);
    return status;
}
