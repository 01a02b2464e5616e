// One ring step on the gfx950 matrix cores: bf16 Q, K, V; fp32 accumulation.
//
// A workgroup owns tile_q = 256 query rows of one head of one (query block,
// key/value block) pair: 8 waves of 32 rows.  Waves w and w + 4 share a SIMD
// and belong to the two groups G0 = waves 0-3 and G1 = waves 4-7, which run
// in opposite phases separated by workgroup barriers:
//
//   M phase (matrix cores):  O^T += V^T P^T for the previous key tile and
//                            S^T = K Q^T for the current one, interleaved;
//   V phase (vector ALUs):   mask, row max, online-softmax update, P = exp2.
//
// While one group of a SIMD runs its M phase the other runs its V phase, so
// the matrix-core and vector work of the two overlap by construction.
//
// Per key tile and wave (64 keys):
//   S^T = K Q^T      2 x 8 MFMA 32x32x16 (keys x queries), K from LDS, Q in
//                    registers.  Working on S^T puts one query row in each
//                    lane (lanes l and l+32 hold the two halves of its keys),
//                    so row max and row sum need one half-swap permute.
//   online softmax   the running-max recurrence of the "Ring Attention
//                    simulation" gist applied to a whole tile (Zhihu article,
//                    local vs. global softmax): tile max, rescale of the state
//                    when the max grows, P = exp2(S*c - m*c), c = scale*log2 e.
//   O^T += V^T P^T   4 x 4 MFMA 32x32x16 (dims x queries); P converted to bf16
//                    straight from the S^T accumulators (its lane layout is
//                    already the B operand), V^T read from a row-major LDS
//                    tile with the transposing ds_read_b64_tr_b16.
// The O rescale is lazy: it is applied only when some row's maximum grows by
// more than 8 in log2 units (P stays <= 256), and one final rescale to the
// true maximum runs before the state is written, so the stored (m, l, O) is
// exactly the state relative to the running maximum.
//
// LDS stages: stage j holds K of key tile j and V of key tile j - 1 (the two
// operands one M phase reads); the two groups read a stage in two
// consecutive phases while the next stage streams into the other buffer with
// direct global -> LDS loads.
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
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int BQ = kBf16TileQ;   // 256 query rows per workgroup
constexpr int BK = kBf16TileK;   // 64 keys per tile
constexpr int WAVES = 8;
constexpr int THREADS = 64 * WAVES;
constexpr float kLazyRescale = 8.0f;

template <int I>
using ic = std::integral_constant<int, I>;

// LDS tiles hold 64 keys x D dims, row-major, 16-byte chunks XOR-swizzled per
// row (no padding): logical chunk c of key row r sits in slot c ^ swz(r).  The
// K swizzle spreads the 16 rows an MFMA operand read takes in one pass over
// distinct banks; the V swizzle does the same for the transposing reads,
// which take 4 rows x 2-4 chunks per pass.
template <int D>
struct Tiles {
    static constexpr int CH = D / 8;                 // 16-byte chunks per row
    static constexpr int ELEMS = BK * D;             // one tile, elements
    static constexpr int LOADS = BK * CH / 64 / (WAVES / 2);  // 1 KB loads per issuing wave per tile
    __device__ static constexpr int swz_k(int r) { return r & (CH - 1); }
    __device__ static constexpr int swz_v(int r) { return (4 * (r & 3) + 2 * ((r >> 1) & 1)) & (CH - 1); }
};

typedef __attribute__((address_space(3))) void lds_void;

// Direct global -> LDS copy of one 64-row tile of K (SWZ_V = false) or V into
// dst, by the four waves of one group (gwave = 0..3 within the group): every
// lane moves one 16-byte chunk per load and the hardware writes
// lane l's chunk to dst + 16 l, so each lane picks the global chunk that
// belongs in its slot.  Addresses are a uniform tile base plus a 32-bit
// per-lane byte offset.  Rows past the end of the block (last_row < 63)
// re-read the last row: their scores are masked to -inf, so they only ever
// meet a zero weight.
template <int D, bool SWZ_V>
__device__ __forceinline__ void issue_tile(bf16* dst, const bf16* tile, uint32_t rs_bytes, int last_row, int gwave) {
    using T = Tiles<D>;
    constexpr int RPI = 64 / T::CH;  // rows per load instruction
    const int lane = threadIdx.x & 63;
    const int slot = lane % T::CH;
#pragma unroll
    for (int i = 0; i < T::LOADS; i++) {
        const int n = gwave * T::LOADS + i;  // wave-uniform
        const int r = RPI * n + lane / T::CH;
        const uint32_t row = (uint32_t)(r < last_row ? r : last_row);
        const int swz = SWZ_V ? T::swz_v(r) : T::swz_k(r);
        const uint32_t off = row * rs_bytes + 16u * (uint32_t)(slot ^ swz);
        __builtin_amdgcn_global_load_lds((const char*)tile + off, (lds_void*)(dst + 512 * n), 16, 0, 0);
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
__global__ __launch_bounds__(THREADS, 1) void step_bf16_kernel(const StepArgs a) {
    using TL = Tiles<D>;
    // Two stage buffers as four distinct arrays: the compiler can then tell
    // the direct-to-LDS loads into one stage from the reads of the other and
    // does not wait for the former before the latter.
    __shared__ bf16 k_buf0[TL::ELEMS], k_buf1[TL::ELEMS];
    __shared__ bf16 v_buf0[TL::ELEMS], v_buf1[TL::ELEMS];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int grp = wave >> 2;
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
    auto tile_cls = [&](int kt) __attribute__((always_inline)) {
        const int64_t w0 = (int64_t)kt * BK, w1 = (a.Bk < w0 + BK ? a.Bk : w0 + BK) - 1;
        return classify(a.mask, t_min, t_max, ds_min, ds_max, pd.k_pos0 + w0 * a.pos_stride,
                        pd.k_pos0 + w1 * a.pos_stride);
    };
    // Non-skipped key tiles form one contiguous range (skips are a prefix
    // under doc-causal and a suffix under causal masks).
    int kt_lo = 0, kt_hi = nkt - 1;
    while (kt_lo <= kt_hi && tile_cls(kt_lo) == kSkip) kt_lo++;
    while (kt_hi >= kt_lo && tile_cls(kt_hi) == kSkip) kt_hi--;
    const int nT = kt_hi - kt_lo + 1;

    if (a.stats && head == 0 && threadIdx.x == 0) {
        unsigned n_full = 0, n_part = 0;
        for (int kt = kt_lo; kt <= kt_hi; kt++) {
            const Cls c = tile_cls(kt);
            n_full += c == kFull;
            n_part += c == kPartial;
        }
        atomicAdd(&a.stats[0], (unsigned long long)(nkt - nT));
        atomicAdd(&a.stats[1], (unsigned long long)n_full);
        atomicAdd(&a.stats[2], (unsigned long long)n_part);
    }

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
    const uint32_t k_rs_bytes = (uint32_t)(a.k_row_stride * 2), v_rs_bytes = (uint32_t)(a.v_row_stride * 2);
    auto last_row = [&](int kt) __attribute__((always_inline)) {
        const int64_t rem = a.Bk - 1 - (int64_t)kt * BK;
        return rem < BK ? (int)rem : BK;
    };
    auto issue_k = [&](int kt, bf16* dst) __attribute__((always_inline)) {
        issue_tile<D, false>(dst, kbase + (int64_t)kt * BK * a.k_row_stride, k_rs_bytes, last_row(kt), wave & 3);
    };
    auto issue_v = [&](int kt, bf16* dst) __attribute__((always_inline)) {
        issue_tile<D, true>(dst, vbase + (int64_t)kt * BK * a.v_row_stride, v_rs_bytes, last_row(kt), wave & 3);
    };

    // Per-lane LDS element offsets of the MFMA operands.
    //  K (A operand of S^T): key row col (+32 kb), logical chunk 2 kc + half
    //  = 2 (kc ^ kx) + half_x in swizzled slots.
    const int kx = TL::swz_k(col) >> 1, half_x = half ^ (TL::swz_k(col) & 1);
    //  V (A operand of O^T, transposing read): key row 4 half + j/4 (+ 32 kb + 16 cp + 8 second),
    //  dims 32 db + 16 g + 4 (j % 4) .. +3, i.e. chunk 4 db + 2 g + (j % 4) / 2, half-chunk j % 2.
    const int j16 = lane & 15, g16 = (lane >> 4) & 1;
    const int vrow = 4 * half + (j16 >> 2);
    int v_off[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; db++)
        v_off[db] = vrow * D + 8 * ((4 * db + 2 * g16 + ((j16 & 3) >> 1)) ^ TL::swz_v(vrow)) + 4 * (j16 & 1);

    f32x16 s[2];        // S^T of the current tile (M phase -> V phase)
    bf16x8 pb[2][2];    // P of the previous tile  (V phase -> next M phase)
#pragma unroll
    for (int kb = 0; kb < 2; kb++) pb[kb][0] = pb[kb][1] = bf16x8{};

    // ---- M phase: O^T += V^T P^T (previous tile) and S^T = K Q^T (this tile) ----
    // One PV and one S MFMA per step, on independent accumulators, operands
    // read AHEAD steps early.
    constexpr int NS = 2 * (D / 16);  // S MFMAs: n = 2 kc + kb
    constexpr int AHEAD = 3;
    static_assert(NS == 4 * (D / 32), "one PV MFMA per S MFMA");
    auto m_phase = [&](const bf16* ks, const bf16* vs) __attribute__((always_inline)) {
        auto k_frag = [&](int n) __attribute__((always_inline)) {
            const int kc = n >> 1;
            return *(const bf16x8*)(ks + 32 * D * (n & 1) + col * D + 8 * half_x + 16 * (kc ^ kx));
        };
        auto v_frag = [&](int n) __attribute__((always_inline)) {  // n = (D/32) q + db, q = 2 kb + cp
            const int q = n / (D / 32), db = n % (D / 32);
            const bf16* p1 = vs + (32 * (q >> 1) + 16 * (q & 1)) * D + v_off[db];
            const i16x4 r1 = lds_read_tr(p1);
            const i16x4 r2 = lds_read_tr(p1 + 8 * D);
            return __builtin_bit_cast(bf16x8, __builtin_shufflevector(r1, r2, 0, 1, 2, 3, 4, 5, 6, 7));
        };
        bf16x8 ka[AHEAD], va[AHEAD];
#pragma unroll
        for (int i = 0; i < AHEAD; i++) {
            va[i] = v_frag(i);
            ka[i] = k_frag(i);
        }
        s[0] = f32x16{};
        s[1] = f32x16{};
#pragma unroll
        for (int i = 0; i < NS; i++) {
            const int q = i / (D / 32), db = i % (D / 32);
            o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[i % AHEAD], pb[q >> 1][q & 1], o[db], 0, 0, 0);
            if (i + AHEAD < NS) va[i % AHEAD] = v_frag(i + AHEAD);
            s[i & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[i % AHEAD], qf[i >> 1], s[i & 1], 0, 0, 0);
            if (i + AHEAD < NS) ka[i % AHEAD] = k_frag(i + AHEAD);
        }
    };

    // ---- V phase: mask, max, online-softmax update, P ----
    auto v_phase = [&](int kt) __attribute__((always_inline)) {
        const Cls c = tile_cls(kt);
        const bool ragged = (int64_t)(kt + 1) * BK > a.Bk;
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
                const int64_t xm = lim < 0 ? -1 : (a.pos_stride == 1 ? lim : lim / a.pos_stride);
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
#pragma unroll
        for (int kb = 0; kb < 2; kb++)
#pragma unroll
            for (int i = 0; i < 16; i++) {
                const float p = __builtin_amdgcn_exp2f(fmaf(s[kb][i], a.c2, -mref));
                lsum += p;
                pb[kb][i / 8][i % 8] = (bf16)p;
            }
    };

    // ---- phase schedule ----
    // Every wave runs the same sequence: for j = 0 .. nT, M_j (PV of tile j-1,
    // S of tile j, both read from stage buffer j % 2) then V_j (softmax of tile
    // j), with a barrier after each.  Group G1 runs one phase behind G0 (one
    // extra barrier at the start, G0 one at the end), so on every SIMD one
    // wave is in an M phase while the other is in a V phase.  Workgroup phase
    // 2j is G0's M_j and G1's V_{j-1}; phase 2j+1 is G0's V_j and G1's M_j.
    // Stage j is read during phases 2j and 2j+1.  Stage j+1 is loaded by G1
    // alone, issued at the start of phase 2j (G1's V phase, so no wave ever
    // stalls on the memory queue at the start of an M phase) into the buffer
    // stage j-1 used (read last in phase 2j-1), and G1 waits for it at the end
    // of phase 2j+1.  M_0 multiplies P = 0 by a zeroed V buffer and M_nT
    // computes an S that is discarded, so every M phase has the same shape.
    auto iteration = [&](int j, auto parity) __attribute__((always_inline)) {
        constexpr int P = decltype(parity)::value;
        bf16* const kc = P ? k_buf1 : k_buf0;  // stage j's buffers
        bf16* const vc = P ? v_buf1 : v_buf0;
        m_phase(kc, vc);
        if (grp == 1) wait_tile_loads();
        __syncthreads();
        if (grp == 1) {  // stage j + 2 -> this buffer (G0 finished reading it one barrier ago)
            if (j + 2 < nT) issue_k(kt_lo + j + 2, kc);
            if (j + 1 < nT) issue_v(kt_lo + j + 1, vc);
        }
        if (j < nT) v_phase(kt_lo + j);
        __syncthreads();
    };

    if (nT > 0) {
        // Stage 0 (K of the first tile) and a zero V buffer for M_0.
        if (grp == 1) issue_k(kt_lo, k_buf0);
        for (int i = threadIdx.x; i < TL::ELEMS / 8; i += THREADS) ((bf16x8*)v_buf0)[i] = bf16x8{};
        wait_tile_loads();
        __syncthreads();
        if (grp == 1) {  // stage 1, then G1's one-phase offset
            if (1 < nT) issue_k(kt_lo + 1, k_buf1);
            issue_v(kt_lo, v_buf1);
            __syncthreads();
        }
        for (int j = 0; j <= nT; j += 2) {
            iteration(j, ic<0>{});
            if (j + 1 <= nT) iteration(j + 1, ic<1>{});
        }
        if (grp == 0) __syncthreads();
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
    } else if (!pd.load_state || nT > 0) {
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
