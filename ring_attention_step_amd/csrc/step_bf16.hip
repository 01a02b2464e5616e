// One ring step on the gfx950 matrix cores: bf16 Q, K, V; fp32 accumulation.
//
// A workgroup owns tile_q = 128 query rows of one head of one (query block,
// key/value block) pair; its four waves hold 32 rows each.  The key/value
// block streams through LDS in tiles of 64 keys (double-buffered: the next
// tile's global loads are in flight while the current one is computed).
//
// Per key tile and wave:
//   S^T = K Q^T      2 x 8 MFMA 32x32x16 (keys x queries), K from LDS, Q in
//                    registers.  Working on S^T puts one query row in each
//                    lane (lanes l and l+32 hold the two halves of its keys),
//                    so row max and row sum need one cross-half exchange.
//   online softmax   the running-max recurrence of the "Ring Attention
//                    simulation" gist applied to a whole tile at once (Zhihu
//                    article on local vs. global softmax): tile max, rescale
//                    of the state when the max grows, P = exp2(S*c - m*c)
//                    with c = scale*log2(e), row sums in fp32.
//   O^T += V^T P^T   4 x 4 MFMA 32x32x16 (dims x queries), P converted to bf16
//                    straight from the S^T accumulators (its lane layout is
//                    already the B operand), V^T read from a row-major LDS
//                    tile with the transposing ds_read_b64_tr_b16.
// The O rescale is lazy: it is applied only when some row's maximum grows by
// more than 8 in log2 units (P stays <= 256, far from fp32/bf16 range limits),
// and one final rescale to the true maximum runs before the state is written,
// so the stored (m, l, O) is exactly the state relative to the running max.
#include <cmath>

#include "kernels.h"
#include "plan.h"

namespace ra {
namespace {

typedef __bf16 bf16;
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int BQ = kBf16TileQ;   // 128 query rows per workgroup
constexpr int BK = kBf16TileK;   // 64 keys per tile
constexpr int THREADS = 256;     // 4 waves of 64
constexpr float kLazyRescale = 8.0f;

template <int D>
struct Smem {
    // K rows are skewed by 16 bytes so the 32 rows an MFMA operand read
    // touches fall in distinct banks; V rows by 64 bytes for the transposing
    // reads, which take 4 rows x 64 bytes per half-wave.
    static constexpr int KP = D + 8;
    static constexpr int VP = D + 32;
    bf16 k[2][BK * KP];
    bf16 v[2][BK * VP];
};

template <int D>
struct Stage {
    static constexpr int N = BK * D / 8 / THREADS;  // 16-byte chunks per thread per tensor
    u32x4 k[N], v[N];
};

template <int D>
__device__ __forceinline__ void load_tile(Stage<D>& st, const bf16* kb, const bf16* vb, int64_t k_rs,
                                          int64_t v_rs, int64_t w0, int64_t Bk) {
#pragma unroll
    for (int r = 0; r < Stage<D>::N; r++) {
        const int c = threadIdx.x + r * THREADS;
        const int key = c / (D / 8), col = (c % (D / 8)) * 8;
        const int64_t w = w0 + key;
        if (w < Bk) {
            st.k[r] = *(const u32x4*)(kb + w * k_rs + col);
            st.v[r] = *(const u32x4*)(vb + w * v_rs + col);
        } else {
            st.k[r] = u32x4{0, 0, 0, 0};
            st.v[r] = u32x4{0, 0, 0, 0};
        }
    }
}

template <int D>
__device__ __forceinline__ void store_tile(Smem<D>& sm, int buf, const Stage<D>& st) {
#pragma unroll
    for (int r = 0; r < Stage<D>::N; r++) {
        const int c = threadIdx.x + r * THREADS;
        const int key = c / (D / 8), col = (c % (D / 8)) * 8;
        *(u32x4*)&sm.k[buf][key * Smem<D>::KP + col] = st.k[r];
        *(u32x4*)&sm.v[buf][key * Smem<D>::VP + col] = st.v[r];
    }
}

__device__ __forceinline__ i16x4 lds_read_tr(const bf16* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(p));
}

template <int D>
__global__ __launch_bounds__(THREADS, 2) void step_bf16_kernel(const StepArgs a) {
    __shared__ Smem<D> sm;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int half = lane >> 5, col = lane & 31;

    // Workgroup -> (pair, head, q-tile).  Consecutive workgroup ids go to
    // different XCDs; the remap gives each XCD a contiguous range of
    // (pair, head) so that its L2 sees few distinct key/value heads.  Within
    // a range the q-tiles with the most key tiles (causal) start first.
    const int nwg = gridDim.x, b = blockIdx.x;
    const int logical = (nwg % 8 == 0) ? (b % 8) * (nwg / 8) + b / 8 : b;
    const int qt = a.n_qtiles - 1 - logical % a.n_qtiles;
    const int rest = logical / a.n_qtiles;
    const int head = rest % a.Hq;
    const PairDesc& pd = a.pairs[rest / a.Hq];
    const int kvh = head / a.group;

    const int64_t u0 = (int64_t)qt * BQ;
    const int64_t u_last = (a.Bq < u0 + BQ ? a.Bq : u0 + BQ) - 1;
    const int64_t t_min = pd.q_pos0 + u0 * a.pos_stride, t_max = pd.q_pos0 + u_last * a.pos_stride;
    int64_t ds_min = 0, ds_max = 0;
    if (a.mask == kMaskDoc) {
        ds_min = doc_start(a.cu, a.n_docs, t_min);
        ds_max = doc_start(a.cu, a.n_docs, t_max);
    }
    const int nkt = (int)((a.Bk + BK - 1) / BK);
    auto tile_cls = [&](int kt) {
        const int64_t w0 = (int64_t)kt * BK, w1 = (a.Bk < w0 + BK ? a.Bk : w0 + BK) - 1;
        return classify(a.mask, t_min, t_max, ds_min, ds_max, pd.k_pos0 + w0 * a.pos_stride,
                        pd.k_pos0 + w1 * a.pos_stride);
    };
    // Non-skipped key tiles form one contiguous range (skips are a prefix
    // under doc-causal and a suffix under causal masks).
    int kt_lo = 0, kt_hi = nkt - 1;
    while (kt_lo <= kt_hi && tile_cls(kt_lo) == kSkip) kt_lo++;
    while (kt_hi >= kt_lo && tile_cls(kt_hi) == kSkip) kt_hi--;

    // This lane's query row.
    const int64_t u = u0 + wave * 32 + col;
    const bool row_ok = u < a.Bq;
    const int64_t t = pd.q_pos0 + u * a.pos_stride;
    const int64_t ds = (a.mask == kMaskDoc && row_ok) ? doc_start(a.cu, a.n_docs, t) : 0;

    // Q^T as the B operand: lane holds q[row][16*kc + 8*half .. +7].
    bf16x8 qf[D / 16];
    {
        const bf16* qp = (const bf16*)a.q + pd.q_off + head * a.q_head_stride + u * a.q_row_stride + 8 * half;
#pragma unroll
        for (int kc = 0; kc < D / 16; kc++) {
            if (row_ok) qf[kc] = *(const bf16x8*)(qp + 16 * kc);
            else qf[kc] = bf16x8{};
        }
    }

    // Running state.  o[db][i] is O^T[32*db + 8*(i/4) + 4*half + i%4][row].
    f32x16 o[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; db++) o[db] = f32x16{};
    float mx = -INFINITY;   // max of the raw dot products q.k seen so far
    float mrc = -INFINITY;  // reference (log2 units) the accumulators are relative to
    float lsum = 0.f;       // this lane's share of the denominator
    const int64_t srow = (int64_t)head * a.Bq + u;
    if (pd.load_state && row_ok) {
        const float m_in = pd.m[srow];
        if (m_in != -INFINITY) {
            mx = m_in / a.scale;
            mrc = m_in * 1.4426950408889634f;
            lsum = half == 0 ? pd.l[srow] : 0.f;
            const float* Op = pd.O + srow * D + 4 * half;
#pragma unroll
            for (int db = 0; db < D / 32; db++)
#pragma unroll
                for (int g = 0; g < 4; g++) {
                    const f32x4 x = *(const f32x4*)(Op + 32 * db + 8 * g);
                    o[db][4 * g + 0] = x[0];
                    o[db][4 * g + 1] = x[1];
                    o[db][4 * g + 2] = x[2];
                    o[db][4 * g + 3] = x[3];
                }
        }
    }

    const bf16* kbase = (const bf16*)a.k + pd.k_off + kvh * a.k_head_stride;
    const bf16* vbase = (const bf16*)a.v + pd.v_off + kvh * a.v_head_stride;
    const int j16 = lane & 15, g16 = (lane >> 4) & 1;
    const int tr_row = 4 * half + (j16 >> 2), tr_col = 16 * g16 + 4 * (j16 & 3);
    unsigned n_full = 0, n_part = 0;

    if (kt_lo <= kt_hi) {
        Stage<D> st;
        load_tile<D>(st, kbase, vbase, a.k_row_stride, a.v_row_stride, (int64_t)kt_lo * BK, a.Bk);
        store_tile<D>(sm, 0, st);
        __syncthreads();
        for (int kt = kt_lo; kt <= kt_hi; kt++) {
            const int buf = (kt - kt_lo) & 1;
            const bool has_next = kt < kt_hi;
            if (has_next)
                load_tile<D>(st, kbase, vbase, a.k_row_stride, a.v_row_stride, (int64_t)(kt + 1) * BK, a.Bk);
            const Cls c = tile_cls(kt);
            n_full += c == kFull;
            n_part += c == kPartial;
            const bool ragged = (int64_t)(kt + 1) * BK > a.Bk;

            // S^T = K Q^T
            f32x16 s[2];
            const bf16* kl = &sm.k[buf][col * Smem<D>::KP + 8 * half];
#pragma unroll
            for (int kb = 0; kb < 2; kb++) {
                s[kb] = f32x16{};
#pragma unroll
                for (int kc = 0; kc < D / 16; kc++) {
                    const bf16x8 ka = *(const bf16x8*)(kl + 32 * kb * Smem<D>::KP + 16 * kc);
                    s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[kc], s[kb], 0, 0, 0);
                }
            }

            if (c == kPartial || ragged) {
                // Key x of the tile (0..BK-1) sits at position tk0 + x * pos_stride; turn the
                // row's bounds into bounds on x once, then compare small integers.
                const int64_t w0 = (int64_t)kt * BK;
                const int64_t tk0 = pd.k_pos0 + w0 * a.pos_stride;
                int x_end = (int)(a.Bk - w0 < BK ? a.Bk - w0 : BK);  // keys x < x_end exist
                int x_lo = 0;
                if (a.mask != kMaskNone) {
                    // tk <= t  <=>  x <= floor((t - tk0) / pos_stride)
                    const int64_t lim = t - tk0;
                    const int64_t xm = lim < 0 ? -1 : lim / a.pos_stride;
                    if (xm + 1 < x_end) x_end = (int)(xm + 1);
                }
                if (a.mask == kMaskDoc) {
                    const int64_t lo = ds - tk0;  // pos_stride is 1 here
                    x_lo = lo <= 0 ? 0 : (lo > BK ? BK : (int)lo);
                }
#pragma unroll
                for (int kb = 0; kb < 2; kb++)
#pragma unroll
                    for (int i = 0; i < 16; i++) {
                        const int x = 32 * kb + 8 * (i / 4) + 4 * half + (i % 4);
                        if (x < x_lo || x >= x_end) s[kb][i] = -INFINITY;
                    }
            }

            float mt = -INFINITY;
#pragma unroll
            for (int kb = 0; kb < 2; kb++)
#pragma unroll
                for (int i = 0; i < 16; i++) mt = fmaxf(mt, s[kb][i]);
            mt = fmaxf(mt, __shfl_xor(mt, 32));
            const float mnew = fmaxf(mx, mt);
            const float mnc = mnew * a.c2;
            const bool need = mnc > mrc + kLazyRescale;  // false while the row has no key
            if (__ballot(need)) {
                const float alpha = need ? __builtin_amdgcn_exp2f(mrc - mnc) : 1.f;
                if (need) mrc = mnc;
                lsum *= alpha;
#pragma unroll
                for (int db = 0; db < D / 32; db++) o[db] *= alpha;
            }
            mx = mnew;
            const float mref = mrc == -INFINITY ? 0.f : mrc;

            bf16x8 pb[2][2];
#pragma unroll
            for (int kb = 0; kb < 2; kb++)
#pragma unroll
                for (int i = 0; i < 16; i++) {
                    const float p = __builtin_amdgcn_exp2f(fmaf(s[kb][i], a.c2, -mref));
                    lsum += p;
                    pb[kb][i / 8][i % 8] = (bf16)p;
                }

            // O^T += V^T P^T
            const bf16* vl = &sm.v[buf][tr_row * Smem<D>::VP + tr_col];
#pragma unroll
            for (int db = 0; db < D / 32; db++)
#pragma unroll
                for (int kb = 0; kb < 2; kb++)
#pragma unroll
                    for (int cp = 0; cp < 2; cp++) {
                        const bf16* p1 = vl + (32 * kb + 16 * cp) * Smem<D>::VP + 32 * db;
                        const i16x4 r1 = lds_read_tr(p1);
                        const i16x4 r2 = lds_read_tr(p1 + 8 * Smem<D>::VP);
                        const i16x8 r = __builtin_shufflevector(r1, r2, 0, 1, 2, 3, 4, 5, 6, 7);
                        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, r),
                                                                         pb[kb][cp], o[db], 0, 0, 0);
                    }

            if (has_next) store_tile<D>(sm, buf ^ 1, st);
            __syncthreads();
        }
    }

    if (a.stats && head == 0 && threadIdx.x == 0) {
        atomicAdd(&a.stats[0], (unsigned long long)(nkt - (kt_hi - kt_lo + 1)));
        atomicAdd(&a.stats[1], (unsigned long long)n_full);
        atomicAdd(&a.stats[2], (unsigned long long)n_part);
    }

    // Both halves of a row combine their denominators; then rescale to the
    // true maximum.
    float ltot = lsum + __shfl_xor(lsum, 32);
    if (mx != -INFINITY) {
        const float beta = __builtin_amdgcn_exp2f(mrc - mx * a.c2);
        ltot *= beta;
#pragma unroll
        for (int db = 0; db < D / 32; db++) o[db] *= beta;
    }
    if (!row_ok) return;

    if (pd.finalize) {
        const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
        char* ob = (char*)a.out;
        const int64_t oe = pd.out_off + u * a.out_row_stride + head * a.out_head_stride + 4 * half;
#pragma unroll
        for (int db = 0; db < D / 32; db++)
#pragma unroll
            for (int g = 0; g < 4; g++) {
                const int64_t e = oe + 32 * db + 8 * g;
                const float x0 = o[db][4 * g] * inv, x1 = o[db][4 * g + 1] * inv;
                const float x2 = o[db][4 * g + 2] * inv, x3 = o[db][4 * g + 3] * inv;
                if (a.out_bf16) *(bf16x4*)(ob + 2 * e) = bf16x4{(bf16)x0, (bf16)x1, (bf16)x2, (bf16)x3};
                else *(f32x4*)(ob + 4 * e) = f32x4{x0, x1, x2, x3};
            }
        if (half == 0 && a.lse)
            a.lse[pd.lse_off + head * a.lse_head_stride + u * a.lse_row_stride] =
                ltot > 0.f ? mx * a.scale + logf(ltot) : -INFINITY;
    } else if (!pd.load_state || kt_lo <= kt_hi) {
        float* Op = pd.O + srow * D + 4 * half;
#pragma unroll
        for (int db = 0; db < D / 32; db++)
#pragma unroll
            for (int g = 0; g < 4; g++)
                *(f32x4*)(Op + 32 * db + 8 * g) =
                    f32x4{o[db][4 * g], o[db][4 * g + 1], o[db][4 * g + 2], o[db][4 * g + 3]};
        if (half == 0) {
            pd.m[srow] = ltot > 0.f ? mx * a.scale : -INFINITY;
            pd.l[srow] = ltot;
        }
    }
}

}  // namespace

hipError_t launch_step_bf16(const StepArgs& a, hipStream_t stream) {
    const int64_t nwg = (int64_t)a.n_qtiles * a.Hq * a.n_pairs;
    if (nwg == 0) return hipSuccess;
    if (a.d == 128) step_bf16_kernel<128><<<dim3((unsigned)nwg), dim3(THREADS), 0, stream>>>(a);
    else if (a.d == 64) step_bf16_kernel<64><<<dim3((unsigned)nwg), dim3(THREADS), 0, stream>>>(a);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace ra
