// One ring step on the gfx950 matrix cores: 16-bit Q, K, V (bf16 or fp16,
// the kernel's E); fp32 accumulation.  Operands are held as raw 16-bit values
// (the bf16 vector type is only their container); E picks the MFMA and the
// rounding of P and of a 16-bit output.
//
// A workgroup owns tile_q = 256 query rows of one head of one (query block,
// key/value block) pair: 8 waves of 32 rows.  Waves w and w + 4 share a SIMD
// and belong to the two groups G0 = waves 0-3 and G1 = waves 4-7, which run
// in opposite phases separated by workgroup barriers:
//
//   M phase (matrix cores):  O^T += V^T P^T for the previous key tile and
//                            S^T = K Q^T for the current one, interleaved,
//                            operands read from LDS a few MFMAs ahead;
//   V phase (vector ALUs):   mask, row max, online-softmax update, P = exp2.
//
// While one group of a SIMD runs its M phase the other runs its V phase, so
// the matrix-core and vector work of the two overlap by construction.
//
// Per key tile and wave (64 keys):
//   S^T = K Q^T      2 x D/16 MFMA 32x32x16 (keys x queries), K from LDS, Q
//                    in registers.  Working on S^T puts one query row in each
//                    lane (lanes l and l+32 hold the two halves of its keys),
//                    so row max and row sum need one half-swap permute.
//   online softmax   the running-max recurrence of the "Ring Attention
//                    simulation" gist applied to a whole tile (Zhihu article,
//                    local vs. global softmax): tile max, rescale of the state
//                    when the max grows, P = exp2(S*c - m*c), c = scale*log2 e.
//                    Row sums add up P in fp32, before its 16-bit rounding.
//   O^T += V^T P^T   4 x D/32 MFMA 32x32x16 (dims x queries); P converted to
//                    E straight from the S^T accumulators (its lane layout
//                    is already the B operand).
// The O rescale is lazy: it is applied only when some row's maximum grows by
// more than 8 in log2 units (P stays <= 256), and one final rescale to the
// true maximum runs before the state is written, so the stored (m, l, O) is
// exactly the state relative to the running maximum.
//
// V operands come either from a row-major V tile through the transposing
// ds_read_b64_tr_b16 (VT = false: the step entry point), or -- for the ring
// forward, which packs V^T once per call -- from a V^T tile with plain 16-byte
// reads (VT = true).  The plain reads cost the LDS a fifth of the transposing
// ones, and, unlike them, let the compiler see that they do not touch the
// buffer the next stage is streaming into, so it does not wait for that
// stream before them.
//
// A workgroup runs a chain of (query block, key/value block) pairs: one
// pair for the step entry point, or, for the ring forward in one launch, a
// virtual device's visited blocks in ring order, the state staying in
// registers from the first block to the fused finalize.  The tile pipeline
// below runs straight across block boundaries.
//
// LDS stages: stage j holds K of key tile j and V of key tile j - 1 (the two
// operands one M phase reads); the two groups read a stage in two
// consecutive phases while the next two stages stream into the other two
// buffers with direct global -> LDS loads.
#include <cmath>
#include <type_traits>

#include "kernels.h"
#include "plan.h"

namespace ra {
namespace {

typedef __bf16 bf16;
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16;
typedef f16 f16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int BQ = kBf16TileQ;   // 256 query rows per workgroup
constexpr int BK = kBf16TileK;   // 64 keys per tile
constexpr int WAVES = 8;
constexpr int THREADS = 64 * WAVES;
constexpr float kLazyRescale = 8.0f;
constexpr float kTileSumMax = 16384.0f;  // 2^(kLazyRescale + 6)
static_assert(BK == 64, "the lane layouts below assume 64-key tiles");

template <int I>
using ic = std::integral_constant<int, I>;

// C += A B on the 32x32x16 matrix core for element type E (operands as 16-bit
// containers, reinterpreted without conversion).
template <typename E>
__device__ __forceinline__ f32x16 mma(bf16x8 a, bf16x8 b, f32x16 c) {
    if constexpr (std::is_same<E, f16>::value)
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c,
                                                      0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// x rounded to E (nearest even), in the 16-bit container.
template <typename E>
__device__ __forceinline__ bf16 to16(float x) {
    return __builtin_bit_cast(bf16, (E)x);
}

typedef __attribute__((address_space(3))) void lds_void;

// LDS tiles, 16-byte chunks XOR-swizzled per row (no padding): logical chunk
// c of row r sits in slot c ^ swz(r).
//  K tile   [64 keys][D]:  swz = r & (D/8 - 1); the 16 rows one MFMA operand
//           read takes per pass land in distinct banks.
//  V tile   [64 keys][D] (transposing reads): swz = 4(r&3) + 2((r>>1)&1),
//           the same for the 4 rows x 2-4 chunks such a read takes per pass.
//  V^T tile [D][64 keys] (128-byte rows): swz = (r >> 1) & 7.
template <int D>
struct Tiles {
    static constexpr int CH = D / 8;                    // 16-byte chunks per K / V row
    static constexpr int ELEMS = BK * D;                // one tile, elements (any layout)
    static constexpr int LOADS = ELEMS * 2 / 1024 / 4;  // 1 KB loads per issuing wave per tile
    __device__ static constexpr int swz_k(int r) { return r & (CH - 1); }
    __device__ static constexpr int swz_v(int r) { return (4 * (r & 3) + 2 * ((r >> 1) & 1)) & (CH - 1); }
    __device__ static constexpr int swz_vt(int r) { return (r >> 1) & 7; }
};

// Lane-dependent values that the loop re-derives on every use: an empty asm
// statement hides where the value came from, so the compiler cannot hoist
// the (cheap) address arithmetic built on it out of the loop and keep one
// register per address alive across the whole loop.
__device__ __forceinline__ int fresh_lane() {
    int l = threadIdx.x & 63;
    __asm__ volatile("" : "+v"(l));
    return l;
}

// Marks a register value as produced here: the compiler can no longer sink
// its computation past this point (into a later phase, next to its use).
template <typename T>
__device__ __forceinline__ void pin(T& x) {
    __asm__ volatile("" : "+v"(x));
}

// Direct global -> LDS copy of one tile into dst by the four waves of one
// group (gwave = 0..3): every lane moves one 16-byte chunk per load and the
// hardware writes lane l's chunk to dst + 16 l, so each lane picks the global
// chunk that belongs in its slot.  Addresses are a uniform tile base plus a
// 32-bit per-lane byte offset; tile_chunk_offset is that offset for load n.
//  K, V (KIND 0, 1): rows are keys, D/8 chunks each, row r at r * rs_bytes;
//    rows past last_row re-read last_row (their scores are masked to -inf).
//  V^T (KIND 2): rows are dims (D of them), 8 chunks of 8 keys each, row r at
//    r * rs_bytes (the packed V^T is zero beyond the block: no clamp needed).
template <int D, int KIND>
__device__ __forceinline__ uint32_t tile_chunk_offset(int lane, int n, uint32_t rs_bytes, int last_row) {
    using T = Tiles<D>;
    constexpr int CPR = KIND == 2 ? 8 : T::CH;  // chunks per row
    constexpr int RPI = 64 / CPR;               // rows per load instruction
    const int r = RPI * n + lane / CPR;
    const int swz = KIND == 0 ? T::swz_k(r) : (KIND == 1 ? T::swz_v(r) : T::swz_vt(r));
    const uint32_t row = (uint32_t)(KIND == 2 ? r : (r < last_row ? r : last_row));
    return row * rs_bytes + 16u * (uint32_t)((lane % CPR) ^ swz);
}

template <int D>
__device__ __forceinline__ void issue_tile(bf16* dst, const char* tile, const uint32_t (&off)[Tiles<D>::LOADS],
                                           int gwave) {
    // This wave's part of the tile starts gofs elements into dst.  Derived
    // afresh at every call (the empty asm hides its origin), each load's LDS
    // address is one scalar add, rather than a value the compiler keeps in a
    // register of its own for every buffer and load.
    int gofs = gwave * (512 * Tiles<D>::LOADS);
    __asm__ volatile("" : "+s"(gofs));
#pragma unroll
    for (int i = 0; i < Tiles<D>::LOADS; i++) {
        uint32_t o = off[i];
        __asm__ volatile("" : "+v"(o));  // keeps the 32-bit offset form (uniform base + lane offset)
        __builtin_amdgcn_global_load_lds(tile + o, (lds_void*)(dst + gofs + 512 * i), 16, 0, 0);
    }
}

// s_waitcnt vmcnt(N): all but this wave's N most recent vector-memory loads
// have landed (lgkmcnt and expcnt left at their maxima).  Issued through the
// builtin so that the compiler's own wait bookkeeping sees it: it then knows
// which stage loads are done and adds no wait of its own before later reads.
template <int N>
__device__ __forceinline__ void wait_loads_but() {
    static_assert(N >= 0 && N < 16, "vmcnt field");
    __builtin_amdgcn_s_waitcnt(0x0F70 | N);
}

// Workgroup barrier between phases.  It waits for this wave's LDS traffic
// only: the direct-to-LDS stage loads stay in flight across it (they are
// waited for explicitly, with wait_loads_but, before the barrier that hands
// their buffer to the readers), which a fenced barrier would not allow.  The
// scheduling barriers keep every instruction in the phase it is written in.
__device__ __forceinline__ void phase_barrier() {
    __builtin_amdgcn_sched_barrier(0);
    __asm__ volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

__device__ __forceinline__ i16x4 lds_read_tr(const bf16* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(p));
}

// Value of x in lane l ^ 32, through the half-swapping permute.
__device__ __forceinline__ float other_half(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float((threadIdx.x & 32) ? r[0] : r[1]);
}

template <typename E, int D, bool VT, bool RING, bool KP>
__global__ __launch_bounds__(THREADS, 1) void step_bf16_kernel(const StepArgs a) {
    using TL = Tiles<D>;
    // Three stage buffers as six distinct arrays: the compiler can then tell
    // the direct-to-LDS loads into one stage from the reads of another.
    __shared__ bf16 k_buf0[TL::ELEMS], k_buf1[TL::ELEMS], k_buf2[TL::ELEMS];
    __shared__ bf16 v_buf0[TL::ELEMS], v_buf1[TL::ELEMS], v_buf2[TL::ELEMS];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int grp = wave >> 2, gwave = wave & 3;
    const int half = lane >> 5, col = lane & 31;

    // Workgroup -> (work, head, q-tile).  A work is one (query block,
    // key/value block) pair of a ring step, or, for the ring forward in one
    // launch, one query block with the chain of key/value blocks its ring
    // visits (works come heaviest first).  Consecutive workgroup ids go to
    // the 8 XCDs in turn; (work, head) groups are dealt to the XCDs round
    // robin, each group's q-tiles staying on one XCD (its L2 then serves
    // the group's key/value tiles to all of them), so every XCD gets a like
    // share of heavy and light groups, heavy ones first.  Within a group the
    // q-tiles with the most key tiles (causal) start first.
    const int nwg = gridDim.x, b = blockIdx.x;
    const int n_groups = nwg / a.n_qtiles;
    int grp_id, qt;
    if (n_groups % 8 == 0) {
        const int r = b / 8;
        grp_id = b % 8 + 8 * (r / a.n_qtiles);
        qt = a.n_qtiles - 1 - r % a.n_qtiles;
    } else {
        grp_id = b / a.n_qtiles;
        qt = a.n_qtiles - 1 - b % a.n_qtiles;
    }
    const int head = grp_id % a.Hq;
    const int widx = grp_id / a.Hq;
    const int kvh = head / a.group;
    constexpr bool ring = RING;  // chains from the ring tables (always finalized), else one pair each

    // This work: its query block, state and chain of key/value blocks.
    int64_t q_off, q_pos0, out_off, lse_off;
    float *st_O = nullptr, *st_m = nullptr, *st_l = nullptr;
    bool load_state = false, finalize = true;
    int e_first = 0, n_ent = 1;
    if (ring) {
        const RingWork& w = a.works[widx];
        q_off = w.q_off;
        q_pos0 = w.q_pos0;
        out_off = w.out_off;
        lse_off = w.lse_off;
        e_first = w.first;
        n_ent = w.count;
    } else {
        const PairDesc& pd = a.pairs[widx];
        q_off = pd.q_off;
        q_pos0 = pd.q_pos0;
        out_off = pd.out_off;
        lse_off = pd.lse_off;
        st_O = pd.O;
        st_m = pd.m;
        st_l = pd.l;
        load_state = pd.load_state;
        finalize = pd.finalize;
    }
    // Key/value block e of the chain: element offsets of its rows in k and
    // v (or the packed V^T), and the global position of its row 0.
    struct Blk {
        int64_t k_off, v_off, k_pos0, kb_off;
    };
    auto blk = [&](int e) __attribute__((always_inline)) {
        if (ring) {
            const RingEntry& r = a.entries[e_first + e];
            return Blk{r.k_off, r.vt_off, r.k_pos0, r.kb_off};
        }
        const PairDesc& pd = a.pairs[widx];
        return Blk{pd.k_off, VT ? pd.vt_off : pd.v_off, pd.k_pos0, pd.kb_off};
    };

    const int64_t u0 = (int64_t)qt * BQ;
    const int64_t u_last = (a.Bq < u0 + BQ ? a.Bq : u0 + BQ) - 1;
    const int64_t t_min = q_pos0 + u0 * a.pos_stride, t_max = q_pos0 + u_last * a.pos_stride;
    int64_t ds_min = 0, ds_max = 0;
    if (a.mask == kMaskDoc) {
        ds_min = doc_start(a.cu, a.n_docs, t_min);
        ds_max = doc_start(a.cu, a.n_docs, t_max);
    }
    const int nkt = (int)((a.Bk + BK - 1) / BK);
    auto tile_cls = [&](int kt, int64_t k_pos0) __attribute__((always_inline)) {
        const int64_t w0 = (int64_t)kt * BK, w1 = (a.Bk < w0 + BK ? a.Bk : w0 + BK) - 1;
        return classify(a.mask, t_min, t_max, ds_min, ds_max, k_pos0 + w0 * a.pos_stride,
                        k_pos0 + w1 * a.pos_stride);
    };
    // The chain table, one block per lane (lane e < n_ent holds block e):
    // its non-skipped key tiles [lo, hi] (one contiguous range: skips are a
    // prefix under doc-causal and a suffix under causal masks), the fully
    // visible ones [flo, fhi] (contiguous too, between the partial tiles at
    // a document start and at the diagonal), offsets and first key position.
    // A cursor reads a block's entry with readlane when it moves on to it.
    int cb_lo = 0, cb_hi = -1, cb_flo = 0, cb_fhi = -1, cb_kb = 0;
    int64_t cb_koff = 0, cb_voff = 0, cb_kpos = 0;
    unsigned cb_nfull = 0, cb_npart = 0;
    if (lane < n_ent) {
        const Blk bl = blk(lane);
        cb_koff = bl.k_off;
        cb_voff = bl.v_off;
        cb_kpos = bl.k_pos0;
        if (KP) cb_kb = (int)bl.kb_off;
        cb_lo = 0;
        cb_hi = nkt - 1;
        while (cb_lo <= cb_hi && tile_cls(cb_lo, cb_kpos) == kSkip) cb_lo++;
        while (cb_hi >= cb_lo && tile_cls(cb_hi, cb_kpos) == kSkip) cb_hi--;
        cb_flo = cb_lo;
        cb_fhi = cb_hi;
        while (cb_flo <= cb_fhi && tile_cls(cb_flo, cb_kpos) != kFull) cb_flo++;
        while (cb_fhi >= cb_flo && tile_cls(cb_fhi, cb_kpos) != kFull) cb_fhi--;
        if (a.stats && head == 0)
            for (int kt = cb_lo; kt <= cb_hi; kt++) {
                const Cls c = tile_cls(kt, cb_kpos);
                cb_nfull += c == kFull;
                cb_npart += c == kPartial;
            }
    }
    auto rl32 = [&](int x, int e) __attribute__((always_inline)) { return __builtin_amdgcn_readlane(x, e); };
    auto rl64 = [&](int64_t x, int e) __attribute__((always_inline)) {
        const uint32_t lo32 = __builtin_amdgcn_readlane((int)(uint32_t)x, e);
        const uint32_t hi32 = __builtin_amdgcn_readlane((int)(uint32_t)((uint64_t)x >> 32), e);
        return (int64_t)(((uint64_t)hi32 << 32) | lo32);
    };
    // Tiles of the whole chain, and the tallies (counted once per q-tile).
    int nT = 0;
    {
        unsigned n_skip = 0, n_full = 0, n_part = 0;
        for (int e = 0; e < n_ent; e++) {
            const int cnt = rl32(cb_hi, e) - rl32(cb_lo, e) + 1;
            nT += cnt;
            n_skip += nkt - cnt;
            n_full += rl32((int)cb_nfull, e);
            n_part += rl32((int)cb_npart, e);
        }
        if (a.stats && head == 0 && threadIdx.x == 0) {
            atomicAdd(&a.stats[0], (unsigned long long)n_skip);
            atomicAdd(&a.stats[1], (unsigned long long)n_full);
            atomicAdd(&a.stats[2], (unsigned long long)n_part);
        }
    }
    const bool ragged_block = a.Bk % BK != 0;
    const int ragged_kt = ragged_block ? nkt - 1 : -1;  // a block's part-filled last tile, if any

    // This lane's query row, and the keys of the current block it may see as
    // one index range [w_lo, w_hi) (keys sit at k_pos0 + w * pos_stride):
    //  causal: w * pos_stride <= t - k_pos0;  doc-causal (pos_stride 1) also
    //  w >= doc_start(t) - k_pos0;  and always w < Bk.
    const int64_t u = u0 + wave * 32 + col;
    const bool row_ok = u < a.Bq;
    const int64_t t_row = q_pos0 + u * a.pos_stride;
    const int64_t ds_row = (row_ok && a.mask == kMaskDoc) ? doc_start(a.cu, a.n_docs, t_row) : 0;
    int w_lo = 0, w_hi = (int)a.Bk;
    auto row_bounds = [&](int64_t k_pos0) __attribute__((always_inline)) {
        w_lo = 0;
        w_hi = (int)a.Bk;
        if (row_ok && a.mask != kMaskNone) {
            const int64_t lim = t_row - k_pos0;
            const int64_t last = lim < 0 ? -1 : (a.pos_stride == 1 ? lim : lim / a.pos_stride);
            if (last + 1 < w_hi) w_hi = (int)(last + 1);
            if (a.mask == kMaskDoc) {
                const int64_t lo = ds_row - k_pos0;
                if (lo > 0) w_lo = lo > a.Bk ? (int)a.Bk : (int)lo;
            }
        }
    };

    // Q^T as the B operand: lane holds q[row][16*kc + 8*half .. +7].
    bf16x8 qf[D / 16];
    {
        const bf16* qp = (const bf16*)a.q + q_off + head * a.q_head_stride + u * a.q_row_stride + 8 * half;
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
    if (load_state && row_ok) {
        const float m_in = st_m[srow];
        if (m_in != -INFINITY) {
            mx = m_in / a.scale;
            mrc = m_in * 1.4426950408889634f;
            lsum = half == 0 ? st_l[srow] : 0.f;
            const float* Op = st_O + srow * D + 4 * half;
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

    // ---- stage loads ----
    // Two cursors walk the chain's tiles in order: the load cursor two tiles
    // ahead of the compute cursor.  Both are wave-uniform; moving on to the
    // next block finds its tile range (and, for the compute cursor, the
    // rows' key bounds in it).
    const bf16* const k_all = (const bf16*)a.k + kvh * a.k_head_stride;
    const bf16* const v_all = VT ? (const bf16*)a.vt + kvh * a.vt_head_stride
                                 : (const bf16*)a.v + kvh * a.v_head_stride;
    struct Cursor {
        int e, kt, hi;  // block of the chain, tile in it, last tile of the block
    };
    auto cur_next = [&](Cursor& c) __attribute__((always_inline)) {  // to the next tile, if any
        int e = c.e, kt = c.kt + 1, hi = c.hi;
        while (kt > hi && e + 1 < n_ent) {
            e++;
            kt = rl32(cb_lo, e);
            hi = rl32(cb_hi, e);
        }
        if (kt <= hi) c = Cursor{e, kt, hi};
    };
    Cursor cl{-1, 0, -1};  // load cursor
    cur_next(cl);
    Cursor cc = cl;        // compute cursor
    const int e0 = cc.e < 0 ? 0 : cc.e;
    int cc_flo = rl32(cb_flo, e0), cc_fhi = rl32(cb_fhi, e0);
    row_bounds(rl64(cb_kpos, e0));
    // Key-padding mask: kw is the validity word of the compute cursor's tile
    // (all ones without a mask), read with a scalar load one tile ahead.
    auto key_word = [&](const Cursor& c) __attribute__((always_inline)) {
        typedef const __attribute__((address_space(4))) uint64_t* cwp;
        return *(cwp)(a.kbits + rl32(cb_kb, c.e) + 2 * c.kt);
    };
    uint64_t kw = ~0ull;
    if (KP && nT > 0) kw = key_word(cc);
    const uint32_t k_rs_bytes = (uint32_t)(a.k_row_stride * 2);
    const uint32_t v_rs_bytes = (uint32_t)((VT ? a.vt_row_stride : a.v_row_stride) * 2);
    // This wave's chunk offsets within a stage tile (G0 loads K tiles, G1 V
    // tiles), kept in registers: issuing a load then takes no vector
    // arithmetic.  A ragged last tile of a block recomputes them with its rows
    // clamped to the block's last row.
    uint32_t ld_off[TL::LOADS];
    {
        const int lane0 = threadIdx.x & 63;
#pragma unroll
        for (int i = 0; i < TL::LOADS; i++) {
            const int n = gwave * TL::LOADS + i;
            ld_off[i] = grp == 0 ? tile_chunk_offset<D, 0>(lane0, n, k_rs_bytes, BK)
                                 : tile_chunk_offset<D, VT ? 2 : 1>(lane0, n, v_rs_bytes, BK);
        }
    }
    const int lr_ragged = (int)((a.Bk - 1) % BK);
    // Address of a tile of this wave's group's tensor; the load cursor keeps
    // the address of its tile and moves it by one tile stride within a block.
    const char* const ld_all = (const char*)(grp == 0 ? k_all : v_all);
    const int64_t ld_tab = grp == 0 ? cb_koff : cb_voff;  // lane-distributed block offsets
    const int64_t ld_stride = grp == 0 ? (int64_t)BK * a.k_row_stride * 2
                                       : (VT ? (int64_t)BK * 2 : (int64_t)BK * a.v_row_stride * 2);
    auto ld_addr = [&](const Cursor& c) __attribute__((always_inline)) {
        return ld_all + rl64(ld_tab, c.e) * 2 + (int64_t)c.kt * ld_stride;
    };
    const char* ld_base = ld_addr(cl);
    auto ld_next = [&]() __attribute__((always_inline)) {  // the load cursor to the next tile (there is one)
        const int e_was = cl.e;
        cur_next(cl);
        if (cl.e != e_was) ld_base = ld_addr(cl);
        else ld_base += ld_stride;
    };
    auto issue_stage = [&](bf16* dst, const char* base, int kt) __attribute__((always_inline)) {
        if (!(VT && grp == 1) && kt == ragged_kt) {
            uint32_t o[TL::LOADS];
            const int lane1 = fresh_lane();
#pragma unroll
            for (int i = 0; i < TL::LOADS; i++) {
                const int n = gwave * TL::LOADS + i;
                o[i] = grp == 0 ? tile_chunk_offset<D, 0>(lane1, n, k_rs_bytes, lr_ragged)
                                : tile_chunk_offset<D, 1>(lane1, n, v_rs_bytes, lr_ragged);
            }
            issue_tile<D>(dst, base, o, gwave);
            __asm__ volatile("; ragged tile issued" ::: "memory");
        } else {
            issue_tile<D>(dst, base, ld_off, gwave);
            __asm__ volatile("; tile issued" ::: "memory");
        }
    };

    f32x16 s[2];        // S^T of the current tile, 32 keys each (M phase -> V phase)
    bf16x8 pb[2][2];    // P of the previous tile, one bf16x8 per 16-key chunk (V phase -> next M phase)
#pragma unroll
    for (int kb = 0; kb < 2; kb++) pb[kb][0] = pb[kb][1] = bf16x8{};

    // ---- M phase: O^T += V^T P^T (previous tile) and S^T = K Q^T (this tile) ----
    // One PV and one S MFMA per step, on independent accumulators, operands
    // read AHEAD steps early.
    //  K operand n = 2 kc + kb: key row 32 kb + col, logical chunk 2 kc + half
    //    = 2 (kc ^ kx) + half_x in swizzled slots.
    //  V operand n = (D/32) q + db (16-key chunk q, dims 32 db + col):
    //    V^T tile: row 32 db + col, logical chunk 2 q + half (the packed V^T
    //    stores each 16-key group in S^T register order), slot ^ swz_vt(col).
    //    V tile: transposing reads at key rows 16 q + 4 half + j/4 (+8), dims
    //    32 db + 16 g + 4 (j % 4) (chunk 4 db + 2 g + (j%4)/2, half-chunk j%2).
    constexpr int NS = 2 * (D / 16);  // S MFMAs
    constexpr int AHEAD = 3;
    static_assert(NS == 4 * (D / 32), "one PV MFMA per S MFMA");
    // Lane offsets (elements) of the operand reads; the 32-key half kb of K
    // and the 32-dim block db of V^T are constant offsets on top.
    int k_off[D / 16];
    {
        const int kx = TL::swz_k(col) >> 1, half_x = half ^ (TL::swz_k(col) & 1);
#pragma unroll
        for (int kc = 0; kc < D / 16; kc++) k_off[kc] = col * D + 8 * half_x + 16 * (kc ^ kx);
    }
    int v_off[4];
    if (VT) {
#pragma unroll
        for (int q = 0; q < 4; q++) v_off[q] = col * BK + 8 * ((2 * q + half) ^ TL::swz_vt(col));
    } else {
        const int j16 = lane & 15, g16 = (lane >> 4) & 1, vrow = 4 * half + (j16 >> 2);
#pragma unroll
        for (int db = 0; db < D / 32; db++)
            v_off[db] = vrow * D + 8 * ((4 * db + 2 * g16 + ((j16 & 3) >> 1)) ^ TL::swz_v(vrow)) + 4 * (j16 & 1);
    }
    // Key-padding mask on the matrix core: S^T of a 32-key block starts from
    // one extra 16-deep product whose A operand holds, for key row r (lane r,
    // k = 0), 0 if the key is real and -inf if it is padded, and whose B
    // operand holds 1 at k = 0 for every query: every score of a padded key
    // becomes exactly -inf, every other score gains exactly 0.  Position-full
    // tiles keep their mask-free softmax.
    bf16x8 q_one = bf16x8{};
    if (KP && half == 0) q_one[0] = to16<E>(1.0f);
    auto s_init = [&](int kb) __attribute__((always_inline)) {
        if (!KP) return f32x16{};
        const uint32_t word = kb ? (uint32_t)(kw >> 32) : (uint32_t)kw;
        const bool pad = half == 0 && !((word >> col) & 1u);
        bf16x8 bias = bf16x8{};
        bias[0] = pad ? to16<E>(-INFINITY) : to16<E>(0.0f);
        return mma<E>(bias, q_one, f32x16{});
    };
    auto k_frag = [&](const bf16* ks, int n) __attribute__((always_inline)) {
        return *(const bf16x8*)(ks + k_off[n >> 1] + 32 * D * (n & 1));
    };
    auto m_phase = [&](const bf16* ks, const bf16* vs) __attribute__((always_inline)) {
        auto v_frag = [&](int n) __attribute__((always_inline)) {
            const int q = n / (D / 32), db = n % (D / 32);
            if (VT) {
                return *(const bf16x8*)(vs + v_off[q] + 32 * db * BK);
            } else {
                const bf16* p1 = vs + v_off[db] + 16 * q * D;
                const i16x4 r1 = lds_read_tr(p1);
                const i16x4 r2 = lds_read_tr(p1 + 8 * D);
                return __builtin_bit_cast(bf16x8, __builtin_shufflevector(r1, r2, 0, 1, 2, 3, 4, 5, 6, 7));
            }
        };
        bf16x8 ka[AHEAD], va[AHEAD];
#pragma unroll
        for (int i = 0; i < AHEAD; i++) {
            va[i] = v_frag(i);
            ka[i] = k_frag(ks, i);
        }
        s[0] = s_init(0);
        s[1] = s_init(1);
#pragma unroll
        for (int i = 0; i < NS; i++) {
            const int q = i / (D / 32), db = i % (D / 32);
            o[db] = mma<E>(va[i % AHEAD], pb[q >> 1][q & 1], o[db]);
            if (i + AHEAD < NS) va[i % AHEAD] = v_frag(i + AHEAD);
            s[i & 1] = mma<E>(ka[i % AHEAD], qf[i >> 1], s[i & 1]);
            if (i + AHEAD < NS) ka[i % AHEAD] = k_frag(ks, i + AHEAD);
        }
    };

    // ---- V phase: mask, max, online-softmax update, P ----
    // ks is the tile's K stage buffer, intact through this phase (the next
    // load into it is issued two phases later).
    auto v_phase = [&](int kt, const bf16* ks) __attribute__((always_inline)) {
        const bool full = kt >= cc_flo && kt <= cc_fhi && kt != ragged_kt;
        auto mask = [&]() __attribute__((always_inline)) {
            if (!full) {
                // Register i of s[kb] holds tile key 32 kb + 8 (i/4) + 4 half + i%4;
                // the allowed keys shifted by -4 half leave a constant to compare.
                const int x_lo = w_lo - kt * BK - 4 * half, x_hi = w_hi - kt * BK - 4 * half;
#pragma unroll
                for (int kb = 0; kb < 2; kb++)
#pragma unroll
                    for (int i = 0; i < 16; i++) {
                        const int x = 32 * kb + 8 * (i / 4) + (i % 4);
                        if (x < x_lo || x >= x_hi) s[kb][i] = -INFINITY;
                    }
            }
        };
        mask();
        // Row maximum (four independent chains of three-way maxima) and the
        // lazy re-reference: the accumulators move to a new reference only
        // when the maximum has grown by more than kLazyRescale (log2 units).
        auto rebase = [&]() __attribute__((always_inline)) {
            float m4[4];
#pragma unroll
            for (int c = 0; c < 4; c++) {
                const f32x16& sv = s[c / 2];
                const int i = 8 * (c % 2);
                float t = fmaxf(fmaxf(sv[i], sv[i + 1]), sv[i + 2]);
                t = fmaxf(fmaxf(t, sv[i + 3]), sv[i + 4]);
                t = fmaxf(fmaxf(t, sv[i + 5]), sv[i + 6]);
                m4[c] = fmaxf(t, sv[i + 7]);
            }
            float mt = fmaxf(fmaxf(fmaxf(m4[0], m4[1]), m4[2]), m4[3]);
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
        };
        // P = 2^(c2 s - reference) in bf16 for the next PV, and this lane's
        // (fp32) sum of it.
        auto probs = [&]() __attribute__((always_inline)) {
            const float mref = mrc == -INFINITY ? 0.f : mrc;
            float ps[4];
#pragma unroll
            for (int kb = 0; kb < 2; kb++)
#pragma unroll
                for (int i = 0; i < 16; i++) {
                    const float p = __builtin_amdgcn_exp2f(fmaf(s[kb][i], a.c2, -mref));
                    ps[i % 4] = (kb == 0 && i < 4) ? p : ps[i % 4] + p;
                    pb[kb][i / 8][i % 8] = to16<E>(p);
                }
            return (ps[0] + ps[1]) + (ps[2] + ps[3]);
        };
        // A state written back for a later step holds the exact row maximum,
        // so every tile of a step takes the maximum.  The ring chains end in a
        // fused finalize, which needs only a reference that keeps P bounded:
        // P is taken against the current one, and the tile goes back through
        // the maximum only if a row has no reference yet or its sum of P
        // exceeds 2^(kLazyRescale + 6) (which bounds every P of the tile; NaN
        // sums go back as well).  P overwrites S, so going back recomputes S
        // from the K tile (same MFMA order, same values).
        if (!RING) rebase();
        float lt = probs();
        if (RING && __ballot(!(lt <= kTileSumMax) || mrc == -INFINITY)) {
            s[0] = s_init(0);
            s[1] = s_init(1);
#pragma unroll
            for (int i = 0; i < NS; i++)
                s[i & 1] = mma<E>(k_frag(ks, i), qf[i >> 1], s[i & 1]);
            mask();
            rebase();
            lt = probs();
        }
        lsum += lt;
#pragma unroll
        for (int kb = 0; kb < 2; kb++) {
            pin(pb[kb][0]);
            pin(pb[kb][1]);
        }
        pin(lsum);
    };

    // ---- phase schedule ----
    // Every wave runs the same sequence: for j = 0 .. nT, M_j (PV of tile j-1,
    // S of tile j, both read from stage buffer j % 3) then V_j (softmax of tile
    // j), with a barrier after each.  Group G1 runs one phase behind G0 (one
    // extra barrier at the start, G0 one at the end), so on every SIMD one
    // wave is in an M phase while the other is in a V phase.  Workgroup phase
    // 2j is G0's M_j and G1's V_{j-1}; phase 2j+1 is G0's V_j and G1's M_j.
    // Stage j is read in phases 2j and 2j+1.  Loads are issued at the start
    // of V phases, so that no wave queues behind them in an M phase, and the
    // two groups share them:
    //   G0 issues K_{j+2} in V_j (phase 2j+1, into the buffer stage j-1 left
    //      at phase 2j-1) and waits for it at the end of V_{j+1} (phase 2j+3);
    //   G1 issues V_{j+2} (stage j+3) in V_j (phase 2j+2, into the buffer
    //      stage j left at phase 2j+1) and waits for it at the end of V_{j+1}
    //      (phase 2j+4);
    // so every load has two phases to land.  M_0 multiplies P = 0 by
    // a zeroed V buffer and M_nT computes an S that is discarded, so every M
    // phase has the same shape.
    constexpr int NL = TL::LOADS;
    auto iteration = [&](int j, auto slot) __attribute__((always_inline)) {
        constexpr int B = decltype(slot)::value;  // j % 3
        bf16* const kc = B == 0 ? k_buf0 : (B == 1 ? k_buf1 : k_buf2);  // stage j
        bf16* const vc = B == 0 ? v_buf0 : (B == 1 ? v_buf1 : v_buf2);
        bf16* const k_next2 = B == 0 ? k_buf2 : (B == 1 ? k_buf0 : k_buf1);  // stage j+2 (= j-1)
        __builtin_amdgcn_s_setprio(2);
        m_phase(kc, vc);
        phase_barrier();
        __builtin_amdgcn_s_setprio(0);
        // Past the last tile the batch re-reads the last tile into a buffer
        // no later phase reads: every V phase issues exactly one batch.
        if (j + 2 < nT) ld_next();  // tile j + 2 (past the end: the last tile again)
        // (The two distinct empty asm statements stop the compiler from
        // merging the last load of both branches into one whose LDS target
        // it can no longer tell apart from the buffers read later, which
        // would make it wait for that load before every LDS read.)
        if (grp == 0) {
            issue_stage(k_next2, ld_base, cl.kt);
            __asm__ volatile("; K stage issued" ::: "memory");
        } else {
            issue_stage(vc, ld_base, cl.kt);
            __asm__ volatile("; V stage issued" ::: "memory");
        }
        if (j < nT) {
            // With a key mask, tile j + 1's word is read now, its latency
            // hidden behind this V phase.
            uint64_t kw_next = ~0ull;
            if (KP && j + 1 < nT) {
                Cursor cn = cc;
                cur_next(cn);
                kw_next = key_word(cn);
            }
            v_phase(cc.kt, kc);
            if (j + 1 < nT) {  // the compute cursor moves on to tile j + 1
                const int e_was = cc.e;
                cur_next(cc);
                if (cc.e != e_was) {
                    cc_flo = rl32(cb_flo, cc.e);
                    cc_fhi = rl32(cb_fhi, cc.e);
                    row_bounds(rl64(cb_kpos, cc.e));
                }
            }
            kw = kw_next;
        }
        // Everything but this phase's batch has landed: for G0 that is
        // K_{j+1} (stage j+1, read from phase 2j+2 on), for G1 V_{j+1}
        // (stage j+2, read from phase 2j+4 on).  Both groups run the same
        // wait on the same number of loads, which keeps the compiler's
        // (path-blind) bookkeeping of outstanding loads exact as well.
        wait_loads_but<NL>();
        phase_barrier();
    };

    if (nT > 0) {
        // Q and the state are in registers before any stage load is issued
        // (the waits below then count stage loads only).
        wait_loads_but<0>();
        // Stages 0-2: K_0, K_1 by G0; V_0, V_1 by G1; stage 0's V (tile -1)
        // is a zeroed buffer.
        const Cursor c0 = cl;
        const char* const base0 = ld_base;
        if (nT > 1) ld_next();  // tile 1 (or tile 0 again)
        if (grp == 0) {
            issue_stage(k_buf0, base0, c0.kt);
            issue_stage(k_buf1, ld_base, cl.kt);
            __asm__ volatile("; K stages issued" ::: "memory");
        } else {
            issue_stage(v_buf1, base0, c0.kt);
            issue_stage(v_buf2, ld_base, cl.kt);
            __asm__ volatile("; V stages issued" ::: "memory");
        }
        for (int i = threadIdx.x; i < TL::ELEMS / 8; i += THREADS) ((bf16x8*)v_buf0)[i] = bf16x8{};
        wait_loads_but<NL>();  // K_0 (G0), V_0 (G1)
        phase_barrier();
        if (grp == 1) phase_barrier();  // G1's one-phase offset
        for (int j = 0; j <= nT; j += 3) {
            iteration(j, ic<0>{});
            if (j + 1 <= nT) iteration(j + 1, ic<1>{});
            if (j + 2 <= nT) iteration(j + 2, ic<2>{});
        }
        if (grp == 0) phase_barrier();
        wait_loads_but<0>();  // no load may land in LDS after the workgroup ends
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

    if (finalize) {
        const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
        char* ob = (char*)a.out;
        const int64_t oe = out_off + u * a.out_row_stride + head * a.out_head_stride + 4 * half;
#pragma unroll
        for (int db = 0; db < D / 32; db++)
#pragma unroll
            for (int g = 0; g < 4; g++) {
                const int64_t e = oe + 32 * db + 8 * g;
                const float x0 = o[db][4 * g] * inv, x1 = o[db][4 * g + 1] * inv;
                const float x2 = o[db][4 * g + 2] * inv, x3 = o[db][4 * g + 3] * inv;
                if (a.out16) *(bf16x4*)(ob + 2 * e) = bf16x4{to16<E>(x0), to16<E>(x1), to16<E>(x2), to16<E>(x3)};
                else *(f32x4*)(ob + 4 * e) = f32x4{x0, x1, x2, x3};
            }
        if (half == 0 && a.lse)
            a.lse[lse_off + head * a.lse_head_stride + u * a.lse_row_stride] =
                ltot > 0.f ? mx * a.scale + logf(ltot) : -INFINITY;
    } else if (!load_state || nT > 0) {
        float* Op = st_O + srow * D + 4 * half;
#pragma unroll
        for (int db = 0; db < D / 32; db++)
#pragma unroll
            for (int g = 0; g < 4; g++)
                *(f32x4*)(Op + 32 * db + 8 * g) =
                    f32x4{o[db][4 * g], o[db][4 * g + 1], o[db][4 * g + 2], o[db][4 * g + 3]};
        if (half == 0) {
            st_m[srow] = ltot > 0.f ? mx * a.scale : -INFINITY;
            st_l[srow] = ltot;
        }
    }
}

template <typename E, bool KP>
hipError_t launch_step16(const StepArgs& a, hipStream_t stream) {
    const int64_t nwg = (int64_t)a.n_qtiles * a.Hq * a.n_pairs;
    if (nwg == 0) return hipSuccess;
    const dim3 grid((unsigned)nwg), block(THREADS);
    if (a.works) {  // the one-launch ring reads the packed V^T
        if (!a.vt) return hipErrorInvalidValue;
        if (a.d == 128) step_bf16_kernel<E, 128, true, true, KP><<<grid, block, 0, stream>>>(a);
        else if (a.d == 64) step_bf16_kernel<E, 64, true, true, KP><<<grid, block, 0, stream>>>(a);
        else return hipErrorInvalidValue;
    } else if (a.vt) {
        if (a.d == 128) step_bf16_kernel<E, 128, true, false, KP><<<grid, block, 0, stream>>>(a);
        else if (a.d == 64) step_bf16_kernel<E, 64, true, false, KP><<<grid, block, 0, stream>>>(a);
        else return hipErrorInvalidValue;
    } else {
        if (a.d == 128) step_bf16_kernel<E, 128, false, false, KP><<<grid, block, 0, stream>>>(a);
        else if (a.d == 64) step_bf16_kernel<E, 64, false, false, KP><<<grid, block, 0, stream>>>(a);
        else return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_step_bf16(const StepArgs& a, hipStream_t stream) {
    if (a.works) return launch_ring_fwd(a, stream);
    // KP: with a key-padding mask (the unmasked kernels carry none of its code)
    if (a.kbits) return a.f16 ? launch_step16<f16, true>(a, stream) : launch_step16<bf16, true>(a, stream);
    return a.f16 ? launch_step16<f16, false>(a, stream) : launch_step16<bf16, false>(a, stream);
}

}  // namespace ra
