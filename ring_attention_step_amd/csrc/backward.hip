// Backward of the ring forward on the matrix cores (bf16 inputs, fp32
// accumulation): the gradients dq, dk, dv of out = ring attention(q, k, v)
// for a given dout, from the forward's saved lse.
//
// For a query row t and an allowed key j (the forward's masks and ring
// visibility), P_tj = exp(scale q_t.k_j - lse_t); with D_t = dout_t . out_t
//   dP_tj = dout_t . v_j,   dS_tj = P_tj (dP_tj - D_t),
//   dq_t = scale sum_j dS_tj k_j,  dk_j = scale sum_t dS_tj q_t,  dv_j = sum_t P_tj dout_t
// (GitHub issue "A ring attention with flash attention kernel
// implementation": the backward pass yields the gradients of full attention
// and is where the saved lse is used; these are the chain rule through the
// forward's softmax).
//
// Three kernels, no atomics:
//  * bwd_prep: D_t for every (head, row).
//  * bwd_dq: one workgroup per (virtual device, head, 128-row query tile),
//    walking the device's visited key/value blocks in ring order (the
//    forward's chain tables) in 32-key tiles.  Per wave (32 query rows),
//    with S^T = K Q^T so that one query row sits in each lane:
//      S^T = K Q^T, dP^T = V dout^T, dS^T = P^T (dP^T - D), dq^T += K^T dS^T,
//    the last through transposing LDS reads of the K tile.
//  * bwd_dkdv: one workgroup per (key/value block, KV head, 128-key tile),
//    walking the query blocks that visit the block, every query head of the
//    KV head's group, in 32-row query tiles.  Per wave (32 keys), with
//    S = Q K^T so that one key sits in each lane:
//      S = Q K^T, dP = dout V^T, dS = P (dP - D),
//      dv^T += dout^T P, dk^T += q^T dS,
//    the last two through transposing reads of the dout and q tiles.
// The lane layouts of the 32x32x16 bf16 MFMA are those of the forward
// kernel: accumulator register i of lane l holds row 8 (i/4) + 4 (l/32) + i%4
// and column l % 32; an A operand holds row l % 32 and k = 8 (l/32) .. + 7;
// a B operand k = 8 (l/32) .. + 7 and column l % 32.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "kernels.h"
#include "plan.h"

namespace ra {
namespace {

typedef __bf16 bf16;
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int BW_WAVES = 4;
constexpr int BW_THREADS = 64 * BW_WAVES;
constexpr int BW_TQ = 32 * BW_WAVES;  // query rows per dq workgroup
constexpr int BW_TK = 32 * BW_WAVES;  // keys per dk/dv workgroup
constexpr int BW_T = 32;              // the tile streamed per iteration (keys for dq, queries for dk/dv)

// A [32 rows][D] bf16 tile in LDS, 16-byte chunks XOR-swizzled per row:
// logical chunk c of row r at slot c ^ (r & (D/8 - 1)).
template <int D>
__device__ __forceinline__ int swz(int r) {
    return r & (D / 8 - 1);
}

__device__ __forceinline__ i16x4 lds_read_tr(const bf16* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(p));
}

// Document end (start of the next document) of global position t.
__device__ __forceinline__ int64_t doc_end(const int32_t* cu, int64_t n_docs, int64_t t) {
    int64_t lo = 0, hi = n_docs - 1;
    while (lo < hi) {
        int64_t mid = (lo + hi + 1) >> 1;
        if (cu[mid] <= t) lo = mid; else hi = mid - 1;
    }
    return cu[lo + 1];
}

// Cooperative copy of rows [r0, r0 + 32) of a [rows][D] bf16 matrix (row
// stride rs elements) into a swizzled LDS tile; rows at or past n_rows copy
// row n_rows - 1 (callers mask them), and n_rows == 0 copies zeros.
template <int D>
__device__ __forceinline__ void load_tile(bf16* dst, const bf16* src, int64_t rs, int64_t r0, int64_t n_rows) {
    constexpr int CH = D / 8;
    for (int x = threadIdx.x; x < BW_T * CH; x += BW_THREADS) {
        const int r = x / CH, c = x % CH;
        int64_t row = r0 + r;
        if (row > n_rows - 1) row = n_rows - 1;
        u32x4 val = u32x4{0, 0, 0, 0};
        if (row >= 0) val = *(const u32x4*)(src + row * rs + 8 * c);
        *(u32x4*)(dst + r * D + 8 * (c ^ swz<D>(r))) = val;
    }
}

// MFMA operand offsets (elements) into a swizzled [rows][D] tile:
//  row operand (A or B) of row 32 rb + col, dims 16 kc + 8 half .. + 7;
//  transposing pair for rows 16 q + vrow (+8), dims 32 db + 16 g + 4 (j % 4).
template <int D>
struct TileOps {
    int row_off[D / 16];   // + 32 rb D for row block rb
    int tr_off0[D / 32];   // rows 16 q + vrow      (+ 16 q D)
    int tr_off1[D / 32];   // rows 16 q + vrow + 8  (+ 16 q D)
    __device__ TileOps(int lane) {
        const int col = lane & 31, half = lane >> 5;
#pragma unroll
        for (int kc = 0; kc < D / 16; kc++) row_off[kc] = col * D + 8 * ((2 * kc + half) ^ swz<D>(col));
        const int j16 = lane & 15, g16 = (lane >> 4) & 1, vrow = 4 * half + (j16 >> 2);
#pragma unroll
        for (int db = 0; db < D / 32; db++) {
            const int chunk = 4 * db + 2 * g16 + ((j16 & 3) >> 1);
            tr_off0[db] = vrow * D + 8 * (chunk ^ swz<D>(vrow)) + 4 * (j16 & 1);
            tr_off1[db] = (vrow + 8) * D + 8 * (chunk ^ swz<D>(vrow + 8)) + 4 * (j16 & 1);
        }
    }
    __device__ __forceinline__ bf16x8 row(const bf16* t, int rb, int kc) const {
        return *(const bf16x8*)(t + row_off[kc] + 32 * D * rb);
    }
    // Transposed operand of 16-row chunk q, dim block db (its k index runs
    // over the rows in accumulator order: 16 q + 4 half + 0..3, then + 8).
    __device__ __forceinline__ bf16x8 tr(const bf16* t, int q, int db) const {
        const i16x4 r1 = lds_read_tr(t + tr_off0[db] + 16 * q * D);
        const i16x4 r2 = lds_read_tr(t + tr_off1[db] + 16 * q * D);
        return __builtin_bit_cast(bf16x8, __builtin_shufflevector(r1, r2, 0, 1, 2, 3, 4, 5, 6, 7));
    }
};

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Accumulator register order -> bf16 B operand pair (16-row chunks 2 h, 2 h + 1).
__device__ __forceinline__ void acc_to_b(const f32x16& acc, bf16x8& b0, bf16x8& b1) {
#pragma unroll
    for (int i = 0; i < 8; i++) {
        b0[i] = (bf16)acc[i];
        b1[i] = (bf16)acc[8 + i];
    }
}

// ---- D = rowsum(dout * out) ----
// d / 8 lanes per (token, head) row, 8 elements each, reduced by shuffles.
__global__ void bwd_prep_kernel(const BwdArgs a) {
    const int lanes = a.d / 8;
    const int64_t n = (int64_t)a.T * a.Hq;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t x0 = (int64_t)blockIdx.x * blockDim.x; x0 < n * lanes; x0 += stride) {
        const int64_t x = x0 + threadIdx.x;
        const int64_t row = x / lanes;
        const int c = (int)(x % lanes);
        float s = 0.f;
        if (row < n) {
            const int64_t t = row / a.Hq, h = row % a.Hq;
            const bf16x8 gv = *(const bf16x8*)((const bf16*)a.dout + t * a.do_st + h * a.do_sh + 8 * c);
            const int64_t oe = t * a.out_st + h * a.out_sh + 8 * c;
            if (a.out_bf16) {
                const bf16x8 ov = *(const bf16x8*)((const bf16*)a.out + oe);
#pragma unroll
                for (int e = 0; e < 8; e++) s = fmaf((float)ov[e], (float)gv[e], s);
            } else {
                const f32x4 o0 = *(const f32x4*)((const float*)a.out + oe);
                const f32x4 o1 = *(const f32x4*)((const float*)a.out + oe + 4);
#pragma unroll
                for (int e = 0; e < 4; e++) s = fmaf(o0[e], (float)gv[e], s);
#pragma unroll
                for (int e = 0; e < 4; e++) s = fmaf(o1[e], (float)gv[4 + e], s);
            }
        }
        for (int w = 1; w < lanes; w <<= 1) s += __shfl_xor(s, w, 64);
        if (row < n && c == 0) a.Dsum[(row % a.Hq) * a.T + row / a.Hq] = s;
    }
}

// ---- dq ----
template <int D>
__global__ __launch_bounds__(BW_THREADS, 2) void bwd_dq_kernel(const BwdArgs a) {
    __shared__ __attribute__((aligned(16))) bf16 k_t[BW_T * D];
    __shared__ __attribute__((aligned(16))) bf16 v_t[BW_T * D];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int half = lane >> 5, col = lane & 31;
    const int qt = blockIdx.x % a.n_qtiles;
    const int head = (blockIdx.x / a.n_qtiles) % a.Hq;
    const int widx = blockIdx.x / (a.n_qtiles * a.Hq);
    const int kvh = head / a.group;
    const BwdWork w = a.works[widx];
    const int64_t B = a.B, ps = a.pos_stride;
    const int64_t u = (int64_t)qt * BW_TQ + wave * 32 + col;  // this lane's query row (local)
    const bool row_ok = u < B;
    const int64_t t_row = w.pos0 + (row_ok ? u : B - 1) * ps;  // its global position = token row
    const float lse_row = a.lse[head * a.T + t_row];
    const float lse2 = (row_ok && lse_row != -INFINITY) ? lse_row * 1.4426950408889634f : INFINITY;
    const float drow = row_ok ? a.Dsum[head * a.T + t_row] : 0.f;
    const int64_t ds_row = a.mask == kMaskDoc ? doc_start(a.cu, a.n_docs, t_row) : 0;

    // This wave's query and dout rows as B operands (row u, dims 16 kc + 8 half .. + 7).
    bf16x8 qf[D / 16], gf[D / 16];
    {
        const bf16* qp = (const bf16*)a.q + t_row * a.q_st + head * a.q_sh + 8 * half;
        const bf16* gp = (const bf16*)a.dout + t_row * a.do_st + head * a.do_sh + 8 * half;
#pragma unroll
        for (int kc = 0; kc < D / 16; kc++) {
            qf[kc] = *(const bf16x8*)(qp + 16 * kc);
            gf[kc] = *(const bf16x8*)(gp + 16 * kc);
        }
    }
    const TileOps<D> ops(lane);
    f32x16 dq[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; db++) dq[db] = f32x16{};

    const int64_t u0 = (int64_t)qt * BW_TQ, u_last = (B < u0 + BW_TQ ? B : u0 + BW_TQ) - 1;
    const int64_t t_min = w.pos0 + u0 * ps, t_max = w.pos0 + u_last * ps;
    const int64_t ds_min = a.mask == kMaskDoc ? doc_start(a.cu, a.n_docs, t_min) : 0;
    const int64_t ds_max = a.mask == kMaskDoc ? doc_start(a.cu, a.n_docs, t_max) : 0;
    const int nkt = (int)((B + BW_T - 1) / BW_T);

    for (int e = 0; e < w.count; e++) {
        const int64_t kp = a.partners[w.first + e];  // position of the key block's row 0
        // This row's allowed keys of the block: local indices [w_lo, w_hi).
        int64_t w_lo = 0, w_hi = row_ok ? B : 0;
        if (a.mask != kMaskNone) {
            const int64_t lim = t_row - kp;
            const int64_t last = lim < 0 ? -1 : lim / ps;
            if (last + 1 < w_hi) w_hi = last + 1;
            if (a.mask == kMaskDoc && ds_row - kp > 0) w_lo = ds_row - kp;
        }
        const bf16* kb = (const bf16*)a.k + kp * a.k_st + kvh * a.k_sh;
        const bf16* vb = (const bf16*)a.v + kp * a.v_st + kvh * a.v_sh;
        for (int kt = 0; kt < nkt; kt++) {
            const int64_t w0 = (int64_t)kt * BW_T, w1 = (B < w0 + BW_T ? B : w0 + BW_T) - 1;
            const Cls cls = classify(a.mask, t_min, t_max, ds_min, ds_max, kp + w0 * ps, kp + w1 * ps);
            if (cls == kSkip) continue;
            __syncthreads();
            load_tile<D>(k_t, kb, ps * a.k_st, w0, B);
            load_tile<D>(v_t, vb, ps * a.v_st, w0, B);
            __syncthreads();
            // S^T and dP^T: the tile's 32 keys (rows) x this wave's 32 query rows (columns).
            f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
            for (int kc = 0; kc < D / 16; kc++) {
                s = mfma(ops.row(k_t, 0, kc), qf[kc], s);
                dp = mfma(ops.row(v_t, 0, kc), gf[kc], dp);
            }
            // dS^T = P^T (dP^T - D); register i holds key w0 + 8 (i/4) + 4 half + i%4.
            const bool full = cls == kFull && w1 - w0 + 1 == BW_T;
            const int64_t x_lo = w_lo - w0 - 4 * half, x_hi = w_hi - w0 - 4 * half;
            f32x16 dsv;
#pragma unroll
            for (int i = 0; i < 16; i++) {
                const int x = 8 * (i / 4) + (i % 4);
                float p = __builtin_amdgcn_exp2f(fmaf(s[i], a.c2, -lse2));
                if (!full && (x < x_lo || x >= x_hi)) p = 0.f;
                dsv[i] = p * (dp[i] - drow);
            }
            bf16x8 b0, b1;
            acc_to_b(dsv, b0, b1);
            // dq^T += K^T dS^T over the tile's two 16-key chunks.
#pragma unroll
            for (int db = 0; db < D / 32; db++) {
                dq[db] = mfma(ops.tr(k_t, 0, db), b0, dq[db]);
                dq[db] = mfma(ops.tr(k_t, 1, db), b1, dq[db]);
            }
        }
    }
    if (!row_ok) return;
    char* ob = (char*)a.dq;
    const int64_t oe = (t_row * a.Hq + head) * D + 4 * half;
#pragma unroll
    for (int db = 0; db < D / 32; db++)
#pragma unroll
        for (int g = 0; g < 4; g++) {
            const int64_t e = oe + 32 * db + 8 * g;
            const float x0 = dq[db][4 * g] * a.scale, x1 = dq[db][4 * g + 1] * a.scale;
            const float x2 = dq[db][4 * g + 2] * a.scale, x3 = dq[db][4 * g + 3] * a.scale;
            if (a.grad_bf16) *(bf16x4*)(ob + 2 * e) = bf16x4{(bf16)x0, (bf16)x1, (bf16)x2, (bf16)x3};
            else *(f32x4*)(ob + 4 * e) = f32x4{x0, x1, x2, x3};
        }
}

// ---- dk, dv ----
template <int D>
__global__ __launch_bounds__(BW_THREADS, 1) void bwd_dkdv_kernel(const BwdArgs a) {
    // This workgroup's keys and values (one swizzled 32-row tile per wave),
    // and the current query tile: q, dout, and per row lse * log2(e) and D.
    __shared__ __attribute__((aligned(16))) bf16 k_all[BW_TK * D];
    __shared__ __attribute__((aligned(16))) bf16 v_all[BW_TK * D];
    __shared__ __attribute__((aligned(16))) bf16 q_t[BW_T * D];
    __shared__ __attribute__((aligned(16))) bf16 g_t[BW_T * D];
    __shared__ __attribute__((aligned(16))) float lse_t[BW_T];
    __shared__ __attribute__((aligned(16))) float d_t[BW_T];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int half = lane >> 5, col = lane & 31;
    const int kt = blockIdx.x % a.n_ktiles;
    const int kvh = (blockIdx.x / a.n_ktiles) % a.Hkv;
    const int ridx = blockIdx.x / (a.n_ktiles * a.Hkv);
    const BwdWork w = a.rworks[ridx];
    const int64_t B = a.B, ps = a.pos_stride;
    const int64_t wk0 = (int64_t)kt * BW_TK;
    const int64_t wk = wk0 + wave * 32 + col;  // this lane's key (local)
    const bool key_ok = wk < B;
    const int64_t p_key = w.pos0 + (key_ok ? wk : B - 1) * ps;  // its global position = token row
    const int64_t de_key = a.mask == kMaskDoc ? doc_end(a.cu, a.n_docs, p_key) : 0;

    {
        const bf16* kb = (const bf16*)a.k + w.pos0 * a.k_st + kvh * a.k_sh;
        const bf16* vb = (const bf16*)a.v + w.pos0 * a.v_st + kvh * a.v_sh;
        for (int ti = 0; ti < BW_WAVES; ti++) {
            load_tile<D>(k_all + ti * BW_T * D, kb, ps * a.k_st, wk0 + ti * BW_T, B);
            load_tile<D>(v_all + ti * BW_T * D, vb, ps * a.v_st, wk0 + ti * BW_T, B);
        }
    }
    const TileOps<D> ops(lane);
    const bf16* k_w = k_all + wave * BW_T * D;
    const bf16* v_w = v_all + wave * BW_T * D;
    f32x16 dk[D / 32], dv[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; db++) dk[db] = dv[db] = f32x16{};

    const int64_t wl = (B < wk0 + BW_TK ? B : wk0 + BW_TK) - 1;  // last key of the workgroup
    const int64_t tk_min = w.pos0 + wk0 * ps, tk_max = w.pos0 + wl * ps;
    const int nqt = (int)((B + BW_T - 1) / BW_T);
    for (int e = 0; e < w.count; e++) {
        const int64_t qp = a.rpartners[w.first + e];  // position of the query block's row 0
        // This key's allowed query rows of the block: local indices [u_lo, u_hi).
        int64_t u_lo = 0, u_hi = key_ok ? B : 0;
        if (a.mask != kMaskNone) {
            const int64_t rel = p_key - qp;  // a query must not precede the key
            const int64_t first = rel <= 0 ? 0 : (rel + ps - 1) / ps;
            u_lo = first;
            if (a.mask == kMaskDoc && de_key - qp < u_hi) u_hi = de_key - qp;
        }
        for (int hq = kvh * a.group; hq < (kvh + 1) * a.group; hq++) {
            const bf16* qb = (const bf16*)a.q + qp * a.q_st + hq * a.q_sh;
            const bf16* gb = (const bf16*)a.dout + qp * a.do_st + hq * a.do_sh;
            for (int qt = 0; qt < nqt; qt++) {
                const int64_t u0 = (int64_t)qt * BW_T, u1 = (B < u0 + BW_T ? B : u0 + BW_T) - 1;
                const int64_t t0 = qp + u0 * ps, t1 = qp + u1 * ps;
                const int64_t ds0 = a.mask == kMaskDoc ? doc_start(a.cu, a.n_docs, t0) : 0;
                const int64_t ds1 = a.mask == kMaskDoc ? doc_start(a.cu, a.n_docs, t1) : 0;
                const Cls cls = classify(a.mask, t0, t1, ds0, ds1, tk_min, tk_max);
                if (cls == kSkip) continue;
                __syncthreads();
                load_tile<D>(q_t, qb, ps * a.q_st, u0, B);
                load_tile<D>(g_t, gb, ps * a.do_st, u0, B);
                if (threadIdx.x < BW_T) {
                    const int64_t uu = u0 + threadIdx.x;
                    const int64_t tt = qp + (uu < B ? uu : B - 1) * ps;
                    const float l = a.lse[hq * a.T + tt];
                    lse_t[threadIdx.x] = l == -INFINITY ? INFINITY : l * 1.4426950408889634f;
                    d_t[threadIdx.x] = a.Dsum[hq * a.T + tt];
                }
                __syncthreads();
                // S and dP: the tile's 32 query rows (rows) x this wave's 32 keys (columns).
                f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
                for (int kc = 0; kc < D / 16; kc++) {
                    s = mfma(ops.row(q_t, 0, kc), ops.row(k_w, 0, kc), s);
                    dp = mfma(ops.row(g_t, 0, kc), ops.row(v_w, 0, kc), dp);
                }
                // Register i holds query row u0 + 8 (i/4) + 4 half + i%4.
                const bool full = cls == kFull && u1 - u0 + 1 == BW_T;
                const int64_t x_lo = u_lo - u0 - 4 * half, x_hi = u_hi - u0 - 4 * half;
                f32x16 pv, dsv;
#pragma unroll
                for (int g4 = 0; g4 < 4; g4++) {
                    const f32x4 l4 = *(const f32x4*)(lse_t + 8 * g4 + 4 * half);
                    const f32x4 d4 = *(const f32x4*)(d_t + 8 * g4 + 4 * half);
#pragma unroll
                    for (int r = 0; r < 4; r++) {
                        const int i = 4 * g4 + r, x = 8 * g4 + r;
                        float p = __builtin_amdgcn_exp2f(fmaf(s[i], a.c2, -l4[r]));
                        if (!full && (x < x_lo || x >= x_hi)) p = 0.f;
                        pv[i] = p;
                        dsv[i] = p * (dp[i] - d4[r]);
                    }
                }
                bf16x8 p0, p1, s0, s1;
                acc_to_b(pv, p0, p1);
                acc_to_b(dsv, s0, s1);
                // dv^T += dout^T P and dk^T += q^T dS over the tile's two 16-row chunks.
#pragma unroll
                for (int db = 0; db < D / 32; db++) {
                    dv[db] = mfma(ops.tr(g_t, 0, db), p0, dv[db]);
                    dv[db] = mfma(ops.tr(g_t, 1, db), p1, dv[db]);
                    dk[db] = mfma(ops.tr(q_t, 0, db), s0, dk[db]);
                    dk[db] = mfma(ops.tr(q_t, 1, db), s1, dk[db]);
                }
            }
        }
    }
    if (!key_ok) return;
    char* kb = (char*)a.dk;
    char* vb = (char*)a.dv;
    const int64_t oe = (p_key * a.Hkv + kvh) * D + 4 * half;
#pragma unroll
    for (int db = 0; db < D / 32; db++)
#pragma unroll
        for (int g = 0; g < 4; g++) {
            const int64_t e = oe + 32 * db + 8 * g;
            const float k0 = dk[db][4 * g] * a.scale, k1 = dk[db][4 * g + 1] * a.scale;
            const float k2 = dk[db][4 * g + 2] * a.scale, k3 = dk[db][4 * g + 3] * a.scale;
            const float v0 = dv[db][4 * g], v1 = dv[db][4 * g + 1], v2 = dv[db][4 * g + 2], v3 = dv[db][4 * g + 3];
            if (a.grad_bf16) {
                *(bf16x4*)(kb + 2 * e) = bf16x4{(bf16)k0, (bf16)k1, (bf16)k2, (bf16)k3};
                *(bf16x4*)(vb + 2 * e) = bf16x4{(bf16)v0, (bf16)v1, (bf16)v2, (bf16)v3};
            } else {
                *(f32x4*)(kb + 4 * e) = f32x4{k0, k1, k2, k3};
                *(f32x4*)(vb + 4 * e) = f32x4{v0, v1, v2, v3};
            }
        }
}

}  // namespace

int bwd_tile_q() { return BW_TQ; }
int bwd_tile_k() { return BW_TK; }

hipError_t launch_backward(const BwdArgs& a, hipStream_t stream) {
    if (a.T > 0) {
        const int64_t threads = (int64_t)a.T * a.Hq * (a.d / 8);
        const int blocks = (int)((threads + 255) / 256 < 8192 ? (threads + 255) / 256 : 8192);
        bwd_prep_kernel<<<blocks, 256, 0, stream>>>(a);
    }
    const int64_t ndq = (int64_t)a.n_works * a.Hq * a.n_qtiles;
    const int64_t ndk = (int64_t)a.n_rworks * a.Hkv * a.n_ktiles;
    if (ndq > 0) {
        if (a.d == 128) bwd_dq_kernel<128><<<(unsigned)ndq, BW_THREADS, 0, stream>>>(a);
        else if (a.d == 64) bwd_dq_kernel<64><<<(unsigned)ndq, BW_THREADS, 0, stream>>>(a);
        else return hipErrorInvalidValue;
    }
    if (ndk > 0) {
        if (a.d == 128) bwd_dkdv_kernel<128><<<(unsigned)ndk, BW_THREADS, 0, stream>>>(a);
        else if (a.d == 64) bwd_dkdv_kernel<64><<<(unsigned)ndk, BW_THREADS, 0, stream>>>(a);
        else return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace ra
