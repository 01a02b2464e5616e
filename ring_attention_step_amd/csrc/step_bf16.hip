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
#include <type_traits>

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

// LDS tiles hold 64 keys x D dims, row-major, 16-byte chunks XOR-swizzled
// per row (no padding): logical chunk c of key row r sits in slot
// c ^ swz(r).  The K swizzle spreads the 16 rows an MFMA operand read takes
// in one pass over distinct banks; the V swizzle does the same for the
// transposing reads, which take 4 rows x 2-4 chunks per pass.
template <int D>
struct Tiles {
    static constexpr int CH = D / 8;                      // 16-byte chunks per row
    static constexpr int ELEMS = BK * D;                  // one tile, elements
    static constexpr int LOADS = BK * CH / 64 / (THREADS / 64);  // 1 KB loads per wave per tensor
    __device__ static constexpr int swz_k(int r) { return r & (CH - 1); }
    __device__ static constexpr int swz_v(int r) { return (4 * (r & 3) + 2 * ((r >> 1) & 1)) & (CH - 1); }
};


typedef __attribute__((address_space(3))) void lds_void;

// Direct global -> LDS copy of one key tile (rows w0 .. w0 + 63 of K and V)
// into k_dst / v_dst: every lane moves one 16-byte chunk per load and the
// hardware writes lane l's chunk to lds + 16 l, so each lane picks the global
// chunk that belongs in its slot.  Addresses are a uniform tile base plus a
// 32-bit per-lane byte offset.  Rows past the end of the block (last_row <
// 63) re-read the last row: their scores are masked to -inf, so they only
// ever meet a zero weight.
template <int D>
__device__ __forceinline__ void issue_tile(bf16* k_dst, bf16* v_dst, const bf16* k_tile, const bf16* v_tile,
                                           uint32_t k_rs_bytes, uint32_t v_rs_bytes, int last_row, int wave) {
    using T = Tiles<D>;
    constexpr int RPI = 64 / T::CH;  // rows per load instruction
    const int lane = threadIdx.x & 63;
    const int slot = lane % T::CH;
#pragma unroll
    for (int i = 0; i < T::LOADS; i++) {
        const int n = wave * T::LOADS + i;  // wave-uniform
        const int r = RPI * n + lane / T::CH;
        const uint32_t row = (uint32_t)(r < last_row ? r : last_row);
        const uint32_t ko = row * k_rs_bytes + 16u * (uint32_t)(slot ^ T::swz_k(r));
        const uint32_t vo = row * v_rs_bytes + 16u * (uint32_t)(slot ^ T::swz_v(r));
        __builtin_amdgcn_global_load_lds((const char*)k_tile + ko, (lds_void*)(k_dst + 512 * n), 16, 0, 0);
        __builtin_amdgcn_global_load_lds((const char*)v_tile + vo, (lds_void*)(v_dst + 512 * n), 16, 0, 0);
    }
}

__device__ __forceinline__ void wait_tile_loads() { __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

__device__ __forceinline__ i16x4 lds_read_tr(const bf16* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(p));
}

// Value of x in lane l ^ 32, through the half-swapping permute.
__device__ __forceinline__ float other_half(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float((threadIdx.x & 32) ? r[0] : r[1]);
}

template <int D>
__global__ __launch_bounds__(THREADS, 2) void step_bf16_kernel(const StepArgs a) {
    // Two K and two V tile buffers as four distinct arrays: the compiler can
    // then tell the direct-to-LDS loads into one buffer from the reads of the
    // other and does not wait for the former before the latter.
    __shared__ bf16 k_buf0[Tiles<D>::ELEMS], k_buf1[Tiles<D>::ELEMS];
    __shared__ bf16 v_buf0[Tiles<D>::ELEMS], v_buf1[Tiles<D>::ELEMS];
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
    using TL = Tiles<D>;
    // Per-lane LDS element offsets of the MFMA operands (buffer 0).
    //  K (A operand of S^T): key row col (+32 kb), logical chunk 2 kc + half.
    //  (2 kc + half) ^ swz = 2 (kc ^ kx) + half_x with kx = swz >> 1, half_x = half ^ (swz & 1).
    const int kx = TL::swz_k(col) >> 1, half_x = half ^ (TL::swz_k(col) & 1);
    //  V (A operand of O^T, transposing read): key row 4 half + j/4 (+ 32 kb + 16 cp + 8 second),
    //  dims 32 db + 16 g + 4 (j % 4) .. +3, i.e. chunk 4 db + 2 g + (j % 4) / 2, half-chunk j % 2.
    const int j16 = lane & 15, g16 = (lane >> 4) & 1;
    const int vrow = 4 * half + (j16 >> 2);
    int v_off[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; db++)
        v_off[db] = vrow * D + 8 * ((4 * db + 2 * g16 + ((j16 & 3) >> 1)) ^ TL::swz_v(vrow)) + 4 * (j16 & 1);
    unsigned n_full = 0, n_part = 0;

    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    const uint32_t k_rs_bytes = (uint32_t)(a.k_row_stride * 2), v_rs_bytes = (uint32_t)(a.v_row_stride * 2);
    auto issue_next = [&](int kt, bf16* kd, bf16* vd) {
        const int64_t w0 = (int64_t)kt * BK;
        const int64_t rem = a.Bk - 1 - w0;
        issue_tile<D>(kd, vd, kbase + w0 * a.k_row_stride, vbase + w0 * a.v_row_stride, k_rs_bytes, v_rs_bytes,
                      rem < BK ? (int)rem : BK, wave_u);
    };
    // One key tile: compute on buffer B while the next tile streams into the other.
    auto tile = [&](int kt, auto bufc) {
            constexpr int B = decltype(bufc)::value;
            const bf16* ks = B ? k_buf1 : k_buf0;
            const bf16* vs = B ? v_buf1 : v_buf0;
            // The other buffer was last read in the previous iteration, which
            // every wave has left (barrier at its end): refill it now.
            if (kt < kt_hi) issue_next(kt + 1, B ? k_buf0 : k_buf1, B ? v_buf0 : v_buf1);
            const Cls c = tile_cls(kt);
            n_full += c == kFull;
            n_part += c == kPartial;
            const bool ragged = (int64_t)(kt + 1) * BK > a.Bk;

            // S^T = K Q^T: 2 x D/16 MFMAs alternating between the two key
            // blocks, operands read 8 ahead.
            constexpr int NS = 2 * (D / 16);
            f32x16 s[2] = {f32x16{}, f32x16{}};
            constexpr int KA = 4;  // K operands in flight
            bf16x8 ka[KA];
            auto k_frag = [&](int n) {  // n = 2 kc + kb
                const int kc = n >> 1;
                const int off = col * D + 8 * half_x + 16 * (kc ^ kx);
                return *(const bf16x8*)(ks + 32 * D * (n & 1) + off);
            };
#pragma unroll
            for (int i = 0; i < KA; i++) ka[i] = k_frag(i);
#pragma unroll
            for (int i = 0; i < NS; i++) {
                s[i & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[i % KA], qf[i >> 1], s[i & 1], 0, 0, 0);
                if (i + KA < NS) ka[i % KA] = k_frag(i + KA);
            }

            // First V operands: they do not depend on P, so their latency hides
            // behind the softmax arithmetic.
            // PV order: pair q = (kb, cp) outer, db inner (consecutive MFMAs use
            // different accumulators).
            constexpr int NP = 4 * (D / 32);
            bf16x8 va[4];
            auto v_frag = [&](int n) {
                const int q = n / (D / 32), db = n % (D / 32);
                const bf16* p1 = vs + (32 * (q >> 1) + 16 * (q & 1)) * D + v_off[db];
                const i16x4 r1 = lds_read_tr(p1);
                const i16x4 r2 = lds_read_tr(p1 + 8 * D);
                return __builtin_bit_cast(bf16x8, __builtin_shufflevector(r1, r2, 0, 1, 2, 3, 4, 5, 6, 7));
            };
#pragma unroll
            for (int i = 0; i < 4; i++) va[i] = v_frag(i);

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
            mt = fmaxf(mt, other_half(mt));
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
#pragma unroll
            for (int n = 0; n < NP; n++) {
                const int q = n / (D / 32), db = n % (D / 32);
                o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[n & 3], pb[q >> 1][q & 1], o[db], 0, 0, 0);
                if (n + 4 < NP) va[n & 3] = v_frag(n + 4);
            }

            // Next tile landed (own loads) and everyone is done with this one.
            wait_tile_loads();
            __syncthreads();
    };
    if (kt_lo <= kt_hi) {
        issue_next(kt_lo, k_buf0, v_buf0);
        wait_tile_loads();
        __syncthreads();
        for (int kt = kt_lo; kt <= kt_hi; kt += 2) {
            tile(kt, std::integral_constant<int, 0>{});
            if (kt + 1 <= kt_hi) tile(kt + 1, std::integral_constant<int, 1>{});
        }
    }

    if (a.stats && head == 0 && threadIdx.x == 0) {
        atomicAdd(&a.stats[0], (unsigned long long)(nkt - (kt_hi - kt_lo + 1)));
        atomicAdd(&a.stats[1], (unsigned long long)n_full);
        atomicAdd(&a.stats[2], (unsigned long long)n_part);
    }

    // Both halves of a row combine their denominators; then rescale to the
    // true maximum.
    float ltot = lsum + other_half(lsum);
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
