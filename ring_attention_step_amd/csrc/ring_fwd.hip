// The ring forward in one launch on the gfx950 matrix cores: 16-bit Q, K, V
// (bf16 or fp16, the kernel's E), fp32 accumulation.
//
// A work item is 256 query rows of one virtual device: 256 rows of one head,
// or, when several query heads share a kv head (grouped-query attention),
// 256 / h rows of each of h heads of one group, so that the key/value tiles
// it streams serve them all.  It walks the device's visited key/value blocks
// ("Ring Attention" glossary page, worked example: device i holds key/value
// block i - s at step s) in the order the host's chain table gives: ring
// order with the device's own block last, or ascending block order for
// striped layouts (the merged sum is the same in any order).  The
// online-softmax state (running reference, denominator, unnormalised output)
// stays in registers from the first block to the fused finalize.  Eight waves of 32 query rows, two per
// SIMD.
//
// Every wave runs the whole pipeline by itself -- no phases shared with the
// other wave of its SIMD -- so that the two waves of a SIMD issue LDS reads,
// matrix and vector instructions at the same time and each covers the
// other's stalls: a wave alone cannot read a 1 KB matrix operand from LDS per
// 32x32x16 instruction fast enough to keep the matrix core busy (about 1 KB
// per 43 cycles against 32 cycles per instruction), two waves can.
//
// Software pipeline over 32-key units (half a 64-key tile).  In step u a wave
//   - turns S of unit u into P (online softmax, vector ALU),
//   - computes S of unit u+1 (8 MFMAs for d = 128, K from LDS, Q in VGPRs),
//   - accumulates O += V^T P of unit u-1 (8 MFMAs, V^T from LDS),
// so every step has the same mix of matrix, LDS and vector instructions.  The
// LDS operands are read four slots ahead into a ring of registers, across
// step boundaries.
//
// Work per unit and wave: S^T = K Q^T puts one query row in each lane (lanes
// l and l+32 hold the two 16-key halves of its 32 keys), so a row's sums need
// one half-swap permute; P is converted to 16 bits straight from the S^T
// accumulators, whose lane layout is already the B operand of O^T += V^T P^T.
//
// Softmax (the running-max recurrence of the "Ring Attention simulation"
// gist, applied per unit; Zhihu article "Attention的分块计算", local vs. global
// softmax): P = exp2(c2 s - ref) against the row's current reference, c2 =
// scale log2 e.  The fused finalize only needs a reference that keeps P
// bounded, so a unit goes through the row maximum only when a row has no
// reference yet or a lane's sum of P over the unit exceeds 2^14 (a bound on
// every P of the unit; NaN sums too).  The maximum path moves the reference
// only when the maximum grew by more than 8 in log2 units (lazy rescale of O).
//
// Key/value tiles stream into four LDS buffers each for K and the packed V^T
// with direct global -> LDS loads: during tile iteration j the workgroup
// loads V^T of tile j+2 and K of tile j+3, and at its start it waits for the
// loads issued two iterations earlier; one barrier per tile.
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
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

constexpr int BQ = kBf16TileQ;  // 256 query rows per workgroup
constexpr int BK = kBf16TileK;  // 64 keys per tile
constexpr int WAVES = 8;
constexpr int THREADS = 64 * WAVES;
constexpr int NBUF = 4;              // LDS buffers per operand
constexpr int LA = 4;                // LDS operand read-ahead (slots)
constexpr float kLazyRescale = 8.0f;
constexpr float kUnitSumMax = 16384.0f;  // 2^(kLazyRescale + 6)
constexpr int kCuLds = 4096;             // document starts kept in LDS (more: searched in global memory)
static_assert(BQ == 32 * WAVES && BK == 64, "lane layouts assume 32 rows per wave and 64-key tiles");

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

// LDS tiles are stored fragment-major: a tile is 16 (d = 128) or 8 (d = 64)
// fragments of 1 KB, each exactly the 32 x 16 operand one matrix
// instruction reads, lane l's 16 bytes at 16 l.  An operand read is then one
// contiguous 1 KB read (no bank conflicts) at 16 l plus a constant, and one
// direct-to-LDS load fills one fragment.
//  K fragment (kh, kc), index kh * D/16 + kc: lane l holds K[32 kh + l % 32]
//    [16 kc + 8 (l / 32) .. +7] (keys of half kh, dims of chunk kc).
//  V^T fragment (c, db), index c * D/32 + db: lane l holds V^T[32 db + l % 32]
//    [16 c + 8 (l / 32) .. +7] (dims of block db, packed keys of 16-key chunk c).
template <int D>
struct Tiles {
    static constexpr int ELEMS = BK * D;             // one tile, elements
    static constexpr int FRAGS = ELEMS / 512;        // 1 KB fragments per tile
    static constexpr int LPW = FRAGS / WAVES;        // loads per wave per tile and operand
    static constexpr int KC = D / 16;                // K fragments per key half
    static constexpr int DB = D / 32;                // V^T fragments per 16-key chunk
    static constexpr int NSLOT = D / 8;              // operand slots per step (half S, half PV)
    static constexpr int SPS = 16 / NSLOT;           // softmax scores per slot and lane
};

// One fragment by a direct-to-LDS buffer load: lane l's 16 bytes at
// base + voff land at LDS byte address lds + 16 l.  The resource is a raw
// buffer at base (no stride, no bound; the offsets are checked on the host).
// Written in asm: the compiler then does not pair its LDS reads with these
// loads (it cannot tell the buffers apart and would wait for every load
// before the reads); their order is explicit (wait_loads_but, barriers).
// M0 holds the LDS address; one wait state separates its write from the load.
__device__ __forceinline__ void dma_frag(uint32_t lds, const char* base, uint32_t voff) {
    const uint64_t b = (uint64_t)base;
    i32x4 r;
    r[0] = (int)(uint32_t)b;
    r[1] = (int)(uint32_t)(b >> 32);
    r[2] = -1;
    r[3] = 0x00020000;
    __asm__ volatile("s_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds" ::"{m0}"(lds), "v"(voff), "s"(r) : "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) { return (uint32_t)(uintptr_t)(lds_void*)p; }

// s_waitcnt vmcnt(N): all but this wave's N most recent vector-memory loads
// have landed (the tile loads above are the only vector loads in flight).
template <int N>
__device__ __forceinline__ void wait_loads_but() {
    static_assert(N >= 0 && N < 64, "vmcnt field");
    __asm__ volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Workgroup barrier that waits for this wave's LDS traffic only: the
// direct-to-LDS loads stay in flight across it (they are waited for with
// wait_loads_but before the barrier that hands their buffer to the readers).
__device__ __forceinline__ void tile_barrier() {
    __builtin_amdgcn_sched_barrier(0);
    __asm__ volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

// Value of x in lane l ^ 32, through the half-swapping permute.
__device__ __forceinline__ float other_half(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float((threadIdx.x & 32) ? r[0] : r[1]);
}

template <typename E, int D, bool KP, bool QM>
__global__ __launch_bounds__(THREADS, 1) void ring_fwd_kernel(const StepArgs a) {
    using TL = Tiles<D>;
    constexpr int LPW = TL::LPW, NSLOT = TL::NSLOT, SPS = TL::SPS;
    static_assert(NSLOT % LA == 0, "the operand ring carries across steps: slot n uses ring[n % LA]");
    static_assert(NSLOT * SPS == 16, "a step turns 16 scores per lane into P");
    // NBUF tile buffers per operand; tile j sits in buffer j % NBUF.
    __shared__ bf16 k_lds[NBUF * TL::ELEMS];
    __shared__ bf16 v_lds[NBUF * TL::ELEMS];
    auto kbuf = [&](int j) __attribute__((always_inline)) { return k_lds + (j & (NBUF - 1)) * TL::ELEMS; };
    auto vbuf = [&](int j) __attribute__((always_inline)) { return v_lds + (j & (NBUF - 1)) * TL::ELEMS; };
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int half = lane >> 5, col = lane & 31;
    // The chain table of the current item (see below) and the item number.
    __shared__ int tab_i[5][kMaxRingChain];
    __shared__ int64_t tab_l[3][kMaxRingChain];
    __shared__ int item_s;
    // The document starts (cu_seqlens) of a doc-causal launch, copied once
    // per workgroup: every item searches them, and a binary search in LDS
    // takes a fraction of the time of one through dependent global loads.
    __shared__ int32_t cu_s[kCuLds];
    const bool cu_lds = a.mask == kMaskDoc && a.n_docs + 1 <= kCuLds;
    if (cu_lds)
        for (int i = threadIdx.x; i <= a.n_docs; i += THREADS) cu_s[i] = a.cu[i];
    // (the item loop's first barrier publishes the copy)
    auto doc_of = [&](int64_t t) __attribute__((always_inline)) {
        if (!cu_lds) return doc_start(a.cu, a.n_docs, t);
        int lo = 0, hi = a.n_docs - 1;  // the last cu[x] <= t, as doc_start
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (cu_s[mid] <= t) lo = mid;
            else hi = mid - 1;
        }
        return (int64_t)cu_s[lo];
    };

    // Items are (work, head block, q-tile) triples, numbered so that
    // consecutive numbers go to the 8 XCDs in turn; (work, head block) groups are dealt to the
    // XCDs round robin, each group's q-tiles on one XCD (its L2 serves the
    // group's key/value tiles), heavy works first; within a group the q-tiles
    // with the most key tiles (causal) come first.  With QM (qt_major) the XCD
    // instead runs one q-tile of all its groups before the next q-tile: where
    // every block of a chain is cut by the mask alike (striped blocks), items
    // with equal q-tiles and one chain order walk the same key tiles in step,
    // while items of one group but different q-tiles would drift apart by
    // whole blocks.  The launch holds one
    // workgroup per compute unit; workgroup w (on XCD w mod 8 under the
    // round-robin dispatch) takes the items of queue w mod 8 (numbers = that
    // queue index mod 8, in order), and when its queue is empty takes the
    // next item of another queue: XCDs that run faster (clocks differ between
    // them under a power cap) or whose items are shorter take more work, and
    // the launch ends when the work ends.
    const int n_items = a.n_qtiles * (a.Hq / a.hpi) * a.n_pairs;
    const int own_q = blockIdx.x & 7;
    unsigned q_done = 0;  // thread 0: queues found empty
    auto run_item = [&](const int b) __attribute__((always_inline)) {
    const int nwg = n_items;
    const int n_groups = nwg / a.n_qtiles;
    int grp_id, qt;
    if (n_groups % 8 == 0) {  // rank r = b / 8 on the item's XCD
        const int r = b / 8;
        if (QM) {
            const int per_xcd = n_groups / 8;
            grp_id = b % 8 + 8 * (r % per_xcd);
            qt = a.n_qtiles - 1 - r / per_xcd;
        } else {
            grp_id = b % 8 + 8 * (r / a.n_qtiles);
            qt = a.n_qtiles - 1 - r % a.n_qtiles;
        }
    } else if (QM) {
        grp_id = b % n_groups;
        qt = a.n_qtiles - 1 - b / n_groups;
    } else {
        grp_id = b / a.n_qtiles;
        qt = a.n_qtiles - 1 - b % a.n_qtiles;
    }
    // An item covers hpi query heads of one kv head (hpi divides the group),
    // 256 / hpi rows of each: wave w takes head w / (8 / hpi) of the item and
    // its row block w mod (8 / hpi), so that every key/value tile loaded into
    // LDS serves all hpi heads.
    const int hpi = a.hpi, wph = WAVES / hpi, rpi = 32 * wph;
    const int head_blk = grp_id % (a.Hq / hpi);
    const int widx = grp_id / (a.Hq / hpi);
    const int head = head_blk * hpi + wave / wph;
    const int kvh = head_blk * hpi / a.group;

    const RingWork& wk = a.works[widx];
    const int64_t q_off = wk.q_off, q_pos0 = wk.q_pos0, out_off = wk.out_off, lse_off = wk.lse_off;
    const int e_first = wk.first, n_ent = wk.count;

    const int64_t u0 = (int64_t)qt * rpi;
    const int64_t u_last = (a.Bq < u0 + rpi ? a.Bq : u0 + rpi) - 1;
    const int64_t t_min = q_pos0 + u0 * a.pos_stride, t_max = q_pos0 + u_last * a.pos_stride;

    // This lane's query row.  Its Q and its document start are fetched first,
    // so that their latency overlaps the chain table's loads below.
    const int64_t urow = u0 + (wave % wph) * 32 + col;
    const bool row_ok = urow < a.Bq;
    const int64_t t_row = q_pos0 + urow * a.pos_stride;
    // Q^T as the B operand: lane holds q[row][16 kc + 8 half .. +7].
    bf16x8 qf[D / 16];
    {
        const bf16* qp = (const bf16*)a.q + q_off + head * a.q_head_stride + urow * a.q_row_stride + 8 * half;
#pragma unroll
        for (int kc = 0; kc < D / 16; kc++) qf[kc] = row_ok ? *(const bf16x8*)(qp + 16 * kc) : bf16x8{};
    }
    const int64_t ds_row = (row_ok && a.mask == kMaskDoc) ? doc_of(t_row) : 0;
    int64_t ds_min = 0, ds_max = 0;
    if (a.mask == kMaskDoc) {
        ds_min = doc_of(t_min);
        ds_max = doc_of(t_max);
    }
    const int nkt = (int)((a.Bk + BK - 1) / BK);
    // The chain table: per block of the chain its non-skipped key tiles
    // [lo, hi] (skips are a prefix under doc-causal and a suffix under causal
    // masks), the fully visible ones [flo, fhi], the key-padding word offset,
    // its offsets and first key position.  Computed one block per lane, then
    // kept in LDS, where the cursors read it when they move on to a block.
    int nT = 0;  // tiles of the whole chain; tallies counted once per q-tile
    {
        int lo = 0, hi = -1, flo = 0, fhi = -1;
        unsigned nfull = 0, npart = 0;
        int64_t koff = 0, voff = 0, kpos = 0;
        int kboff = 0;
        if (lane < n_ent) {
            const RingEntry& re = a.entries[e_first + lane];
            kboff = (int)re.kb_off;
            koff = re.k_off;
            voff = re.vt_off;
            kpos = re.k_pos0;
            // Each condition of classify() on a key tile is monotone in the
            // tile index (key positions grow with it): the skipped tiles are
            // a prefix (keys before the first row's document) and a suffix
            // (keys after the last row), the full ones a range.  Bisection on
            // the same conditions replaces a tile-by-tile scan.
            auto tk_first = [&](int kt) { return kpos + (int64_t)kt * BK * a.pos_stride; };
            auto tk_last = [&](int kt) {
                const int64_t w1 = (a.Bk < (int64_t)kt * BK + BK ? a.Bk : (int64_t)kt * BK + BK) - 1;
                return kpos + w1 * a.pos_stride;
            };
            // first kt in [0, nkt) where the monotone (false, then true) predicate holds, else nkt
            auto first_true = [&](auto&& pred) {
                int l = 0, h = nkt;
                while (l < h) {
                    const int m = (l + h) >> 1;
                    if (pred(m)) h = m; else l = m + 1;
                }
                return l;
            };
            if (a.mask == kMaskNone) {
                hi = nkt - 1;
                flo = 0;
                fhi = nkt - 1;
            } else {
                if (a.mask == kMaskDoc) lo = first_true([&](int kt) { return tk_last(kt) >= ds_min; });
                hi = first_true([&](int kt) { return tk_first(kt) > t_max; }) - 1;
                flo = a.mask == kMaskDoc ? first_true([&](int kt) { return tk_first(kt) >= ds_max; }) : 0;
                fhi = first_true([&](int kt) { return tk_last(kt) > t_min; }) - 1;
                if (flo < lo) flo = lo;
                if (fhi > hi) fhi = hi;
            }
            if (lo > hi) {  // nothing visible
                lo = 0;
                hi = -1;
            }
            if (flo > fhi) {  // no full tile: an empty range
                flo = hi + 1;
                fhi = hi;
            }
            if (a.stats && head_blk == 0) {
                nfull = (unsigned)(fhi - flo + 1);
                npart = (unsigned)(hi - lo + 1) - nfull;
            }
            if (wave == 0) {
                tab_i[0][lane] = lo;
                tab_i[1][lane] = hi;
                tab_i[2][lane] = flo;
                tab_i[3][lane] = fhi;
                tab_i[4][lane] = kboff;
                tab_l[0][lane] = koff;
                tab_l[1][lane] = voff;
                tab_l[2][lane] = kpos;
            }
        }
        unsigned n_skip = 0, n_full = 0, n_part = 0;
        for (int e = 0; e < n_ent; e++) {
            const int cnt = __builtin_amdgcn_readlane(hi, e) - __builtin_amdgcn_readlane(lo, e) + 1;
            nT += cnt;
            n_skip += nkt - cnt;
            n_full += __builtin_amdgcn_readlane((int)nfull, e);
            n_part += __builtin_amdgcn_readlane((int)npart, e);
        }
        if (a.stats && head_blk == 0 && threadIdx.x == 0) {
            atomicAdd(&a.stats[0], (unsigned long long)n_skip);
            atomicAdd(&a.stats[1], (unsigned long long)n_full);
            atomicAdd(&a.stats[2], (unsigned long long)n_part);
        }
    }
    __syncthreads();  // the table in LDS
    auto tab32 = [&](int f, int e) __attribute__((always_inline)) { return __builtin_amdgcn_readfirstlane(tab_i[f][e]); };
    auto tab64 = [&](int f, int e) __attribute__((always_inline)) {
        const int64_t x = tab_l[f][e];
        const uint32_t lo32 = __builtin_amdgcn_readfirstlane((int)(uint32_t)x);
        const uint32_t hi32 = __builtin_amdgcn_readfirstlane((int)(uint32_t)((uint64_t)x >> 32));
        return (int64_t)(((uint64_t)hi32 << 32) | lo32);
    };
    const bool ragged_block = a.Bk % BK != 0;
    const int ragged_kt = ragged_block ? nkt - 1 : -1;

    // This lane's query row (wave row col) and the keys of the current block
    // it may see, as an index range [w_lo, w_hi) (keys at k_pos0 + w *
    // pos_stride): causal: w * pos_stride <= t - k_pos0;  doc-causal
    // (pos_stride 1) also w >= doc_start(t) - k_pos0;  and always w < Bk.
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

    // A chain with no tile for this q-tile: its rows see no key (empty rows:
    // out = 0, lse = -inf).
    if (nT == 0) {
        wait_loads_but<0>();  // the Q loads
        if (!row_ok) return;
        char* ob = (char*)a.out;
        const int64_t oe = out_off + urow * a.out_row_stride + head * a.out_head_stride + 4 * half;
#pragma unroll
        for (int db = 0; db < D / 32; db++)
#pragma unroll
            for (int g = 0; g < 4; g++) {
                const int64_t e = oe + 32 * db + 8 * g;
                if (a.out16) *(bf16x4*)(ob + 2 * e) = bf16x4{};
                else *(f32x4*)(ob + 4 * e) = f32x4{};
            }
        if (half == 0 && a.lse) a.lse[lse_off + head * a.lse_head_stride + urow * a.lse_row_stride] = -INFINITY;
        return;
    }


    // ---- cursors and loads ----
    const bf16* const k_all = (const bf16*)a.k + kvh * a.k_head_stride;
    const bf16* const v_all = (const bf16*)a.vt + kvh * a.vt_head_stride;
    struct Cursor {
        int e, kt, hi;  // block of the chain, tile in it, last tile of the block
    };
    auto cur_next = [&](Cursor& c) __attribute__((always_inline)) {  // to the next tile, if any
        int e = c.e, kt = c.kt + 1, hi = c.hi;
        while (kt > hi && e + 1 < n_ent) {
            e++;
            kt = tab32(0, e);
            hi = tab32(1, e);
        }
        if (kt <= hi) c = Cursor{e, kt, hi};
    };
    const uint32_t k_rs_bytes = (uint32_t)(a.k_row_stride * 2);
    // Lane offsets of the fragment loads.  A wave's K fragments all lie in
    // one key half (kh = wave * LPW / (D/16)): the lane offset holds row
    // 32 kh + col of the tile, or, for a ragged last tile of a block, that
    // row clamped to the block's last row (rows past it are masked), and
    // chunk half of the fragment's 32 bytes; the uniform part goes to the
    // base.  V^T is packed in this fragment order (64-key tiles of D / 8
    // fragments, lane l's 16 bytes at 16 l), so a V^T fragment load reads
    // 1 KB of contiguous memory at 16 l.
    const int kh_w = wave * LPW / TL::KC;
    const int lr_ragged = (int)((a.Bk - 1) % BK);
    const uint32_t ld_k = (uint32_t)(32 * kh_w + col) * k_rs_bytes + 16u * (uint32_t)half;
    const uint32_t ld_k_rag =
        (uint32_t)(32 * kh_w + col < lr_ragged ? 32 * kh_w + col : lr_ragged) * k_rs_bytes + 16u * (uint32_t)half;
    const uint32_t ld_v = 16u * (uint32_t)lane;
    const int64_t k_tile_bytes = (int64_t)BK * a.k_row_stride * 2;
    auto k_addr = [&](const Cursor& c) __attribute__((always_inline)) {
        return (const char*)k_all + tab64(0, c.e) * 2 + (int64_t)c.kt * k_tile_bytes;
    };
    auto v_addr = [&](const Cursor& c) __attribute__((always_inline)) {
        return (const char*)v_all + tab64(1, c.e) * 2 + (int64_t)c.kt * (TL::ELEMS * 2);
    };
    // The load cursor also carries the K and V^T addresses of its tile,
    // stepped by one tile inside a block: it reads the chain table only when
    // it enters a new block, not at every tile (a table read right after the
    // tile barrier would stall both waves of the SIMD on its LDS latency).
    struct LCursor {
        Cursor c;
        const char* kp;
        const char* vp;
    };
    auto lc_next = [&](LCursor& l) __attribute__((always_inline)) {
        if (l.c.kt < l.c.hi) {
            l.c.kt++;
            l.kp += k_tile_bytes;
            l.vp += TL::ELEMS * 2;
            return;
        }
        const int e_was = l.c.e;
        cur_next(l.c);  // past the chain's end it stays on the last tile
        if (l.c.e != e_was) {
            l.kp = k_addr(l.c);
            l.vp = v_addr(l.c);
        }
    };
    // Fragment wave * LPW + i of a K or V^T tile (load i of this wave).
    auto issue_k1 = [&](bf16* dst, const char* base, int kt, int i) __attribute__((always_inline)) {
        const int f = wave * LPW + i, kc = f % TL::KC;
        dma_frag(lds_addr(dst) + 1024u * f, base + 32 * kc, kt == ragged_kt ? ld_k_rag : ld_k);
    };
    auto issue_v1 = [&](bf16* dst, const char* base, int i) __attribute__((always_inline)) {
        const int f = wave * LPW + i;
        dma_frag(lds_addr(dst) + 1024u * f, base + 1024 * f, ld_v);
    };
    auto issue_k = [&](bf16* dst, const char* base, int kt) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < LPW; i++) issue_k1(dst, base, kt, i);
    };
    auto issue_v = [&](bf16* dst, const char* base) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < LPW; i++) issue_v1(dst, base, i);
    };

    // Key-padding mask: the validity word of tile kt of the block whose
    // words start at kb (bit w: key row w is real; all ones without a
    // mask), a scalar load.
    auto key_word_at = [&](int kb, int kt) __attribute__((always_inline)) -> uint64_t {
        if (!KP) return ~0ull;
        typedef const __attribute__((address_space(4))) uint64_t* cwp;
        return *(cwp)(a.kbits + kb + 2 * kt);
    };
    auto key_word = [&](const Cursor& c) __attribute__((always_inline)) -> uint64_t {
        return KP ? key_word_at(tab32(4, c.e), c.kt) : ~0ull;
    };
    // With a key-padding mask, S^T of a unit starts from one extra 16-deep
    // product whose A operand holds, for key row r (lane r, k = 0), 0 if the
    // key is real and -inf if it is padded, and whose B operand holds 1 at
    // k = 0 for every query: every score of a padded key becomes exactly
    // -inf, every other score gains exactly 0, and position-full tiles keep
    // the mask-free softmax.
    bf16x8 q_one = bf16x8{};
    if (KP && half == 0) q_one[0] = to16<E>(1.0f);
    auto s_init = [&](uint32_t word) __attribute__((always_inline)) {
        if (!KP) return f32x16{};
        const bool pad = half == 0 && !((word >> col) & 1u);
        bf16x8 bias = bf16x8{};
        bias[0] = pad ? to16<E>(-INFINITY) : to16<E>(0.0f);
        return mma<E>(bias, q_one, f32x16{});
    };

    // Operand reads.  Slot n of a step: even -> S, K fragment (kh, n / 2);
    // odd -> PV, m = n / 2, q = m / (D/32) (16-key chunk of the half vh),
    // db = m % (D/32), V^T fragment (2 vh + q, db).
    auto frag = [&](const bf16* kb, int kh, const bf16* vb, int vh, int n) __attribute__((always_inline)) {
        if (n % 2 == 0) return *(const bf16x8*)(kb + 512 * (kh * TL::KC + n / 2) + 8 * lane);
        const int m = n / 2, q = m / TL::DB, db = m % TL::DB;
        return *(const bf16x8*)(vb + 512 * ((2 * vh + q) * TL::DB + db) + 8 * lane);
    };

    // ---- softmax pieces ----
    // Unit info: the tile's key range relative to this lane's registers, and
    // whether it needs the element mask.
    struct Unit {
        bool masked;
        int x_lo, x_hi;
    };
    auto unit_of = [&](int kt, int kh, bool full) __attribute__((always_inline)) {
        const int base = kt * BK + 32 * kh + 4 * half;
        return Unit{!full, w_lo - base, w_hi - base};
    };
    // Register i of s holds key 8 (i/4) + 4 half + i%4 of the unit.
    auto apply_mask = [&](f32x16& s, const Unit& un) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < 16; i++) {
            const int x = 8 * (i / 4) + (i % 4);
            s[i] = (x < un.x_lo || x >= un.x_hi) ? -INFINITY : s[i];
        }
    };
    // Running state of the row.  o[db][i] = O^T[32 db + 8 (i/4) + 4 half + i%4][row].
    f32x16 o[D / 32];
    float mx = -INFINITY;   // raw q.k maximum at the last move of the reference
    float mrc = -INFINITY;  // reference (log2 units) the accumulators are relative to
    // The fast path's FMA term: minus the reference, or +inf while the row
    // has none, which turns every P of the fast path into inf or NaN and so
    // sends the unit to the slow path through the same sum test.
    float nref = INFINITY;
    float lsum = 0.f;       // this lane's share of the denominator
    // P of one unit against the current reference, and this lane's sum.
    auto probs_all = [&](const f32x16& s, bf16x8 (&p)[2]) __attribute__((always_inline)) {
        const float mref = mrc == -INFINITY ? 0.f : mrc;
        float ps[4];
#pragma unroll
        for (int i = 0; i < 16; i++) {
            const float pv = __builtin_amdgcn_exp2f(fmaf(s[i], a.c2, -mref));
            ps[i % 4] = i < 4 ? pv : ps[i % 4] + pv;
            p[i / 8][i % 8] = to16<E>(pv);
        }
        return (ps[0] + ps[1]) + (ps[2] + ps[3]);
    };
    // The slow path: row maximum over the unit (both lane halves) and the lazy
    // move of the reference, then P again.
    auto rebase = [&](const f32x16& s) __attribute__((always_inline)) {
        float m4[2];
#pragma unroll
        for (int c = 0; c < 2; c++) {
            const int i = 8 * c;
            float t = fmaxf(fmaxf(s[i], s[i + 1]), s[i + 2]);
            t = fmaxf(fmaxf(t, s[i + 3]), s[i + 4]);
            t = fmaxf(fmaxf(t, s[i + 5]), s[i + 6]);
            m4[c] = fmaxf(t, s[i + 7]);
        }
        float mt = fmaxf(m4[0], m4[1]);
        mt = fmaxf(mt, other_half(mt));
        const float mnew = fmaxf(mx, mt);
        const float mnc = mnew * a.c2;
        const bool need = mnc > mrc + kLazyRescale;  // false while the row has no key
        if (__ballot(need)) {
            const float alpha = need ? __builtin_amdgcn_exp2f(mrc - mnc) : 1.f;
            if (need) {
                mrc = mnc;
                nref = -mnc;
            }
            lsum *= alpha;
#pragma unroll
            for (int db = 0; db < D / 32; db++) o[db] *= alpha;
        }
        mx = mnew;
    };

    bf16x8 ring[LA];
    f32x16 sA, sB;  // S of the even / odd unit
    bf16x8 pA[2], pB[2];
    pB[0] = pB[1] = bf16x8{};

    // Step: softmax of s_cur (unit u, mask un) -> p_cur; S of unit u+1 from
    // (kb, kh) -> s_next; O += V^T (vb, vh) p_prev (unit u-1).  The operand
    // ring holds this step's first LA fragments on entry and leaves the next
    // step's (nkb, nkh, nvb, nvh); load(i) issues this wave's i-th tile load
    // of the step, spread over its slots.
    auto step = [&](f32x16& s_cur, bf16x8 (&p_cur)[2], const Unit& un, f32x16& s_next, const bf16* kb, int kh,
                    const bf16* vb, int vh, const bf16x8 (&p_prev)[2], const bf16* nkb, int nkh, const bf16* nvb,
                    int nvh, uint32_t word_next, auto&& load) __attribute__((always_inline)) {
        if (un.masked) apply_mask(s_cur, un);
        f32x16 sn = s_init(word_next);
        float ps[4];
#pragma unroll
        for (int n = 0; n < NSLOT; n++) {
            const bf16x8 fr = ring[n % LA];
            if (n % 2 == 0) {
                sn = mma<E>(fr, qf[n / 2], sn);
            } else {
                const int m = n / 2, q = m / TL::DB, db = m % TL::DB;
                o[db] = mma<E>(fr, p_prev[q], o[db]);
            }
            ring[n % LA] = n + LA < NSLOT ? frag(kb, kh, vb, vh, n + LA) : frag(nkb, nkh, nvb, nvh, n + LA - NSLOT);
            if (n % (NSLOT / LPW) == 0) load(n / (NSLOT / LPW));
#pragma unroll
            for (int v = 0; v < SPS; v++) {
                const int i = n * SPS + v;
                const float pv = __builtin_amdgcn_exp2f(fmaf(s_cur[i], a.c2, nref));
                ps[i % 4] = i < 4 ? pv : ps[i % 4] + pv;
                p_cur[i / 8][i % 8] = to16<E>(pv);
            }
        }
        // P is packed here, among the matrix instructions, not after the
        // slow-path branch (the slow path recomputes it).
        __asm__ volatile("" : "+v"(p_cur[0]), "+v"(p_cur[1]));
        float lt = (ps[0] + ps[1]) + (ps[2] + ps[3]);
        if (__builtin_expect(__ballot(!(lt <= kUnitSumMax)) != 0, 0)) {
            rebase(s_cur);
            lt = probs_all(s_cur, p_cur);
        }
        lsum += lt;
        s_next = sn;
    };

    // ---- tile iterations ----
    // Iteration j (K_j in kbuf(j), V_j in vbuf(j)): step 2j takes unit
    // (j, 0): S of (j, 1) from K_j, PV of (j-1, 1) from V_{j-1}; step 2j+1
    // takes unit (j, 1): S of (j+1, 0) from K_{j+1}, PV of (j, 0) from V_j.
    // At its start the workgroup waits for the load batch issued two
    // iterations earlier; during step 2j it loads V_{j+2} into the buffer of
    // V_{j-2}, during step 2j+1 K_{j+3} into that of K_{j-1}; past the chain's
    // end the last tile is re-read, so that every iteration issues one batch.
    LCursor ck{Cursor{-1, 0, -1}, nullptr, nullptr};  // K load cursor
    lc_next(ck);
    Cursor cc = ck.c;      // compute cursor (tile j)
    int cc_flo = tab32(2, cc.e), cc_fhi = tab32(3, cc.e);
    int cc_kb = KP ? tab32(4, cc.e) : 0;  // key-padding words of the compute cursor's block
    row_bounds(tab64(2, cc.e));
    const char* v_pend = nullptr;  // V^T address of the tile the K cursor loaded last
    uint64_t kw = ~0ull;           // key-padding word of the compute cursor's tile

    // jm = j mod NBUF as a compile-time constant: every LDS buffer address
    // of the iteration is then a constant offset (no address arithmetic in
    // the steps).
    auto iteration = [&](int j, auto jm) __attribute__((always_inline)) {
        constexpr int J = decltype(jm)::value;
        wait_loads_but<2 * LPW>();
        tile_barrier();
        const char* const v_base = v_pend;
        lc_next(ck);  // past the chain's end it stays on the last tile
        const char* const k_base = ck.kp;
        const int k_kt = ck.c.kt;
        v_pend = ck.vp;
        bf16* const v_dst = vbuf(J + 2);
        bf16* const k_dst = kbuf(J + 3);
        const int kt = cc.kt;
        const bool full = kt >= cc_flo && kt <= cc_fhi && kt != ragged_kt;
        // with a key mask: tile j+1's word, its latency hidden behind step 2j
        // (the chain table is read only when tile j+1 opens a new block)
        uint64_t kw_next = ~0ull;
        if (KP && j + 1 < nT) {
            if (cc.kt < cc.hi) {
                kw_next = key_word_at(cc_kb, cc.kt + 1);
            } else {
                Cursor cn = cc;
                cur_next(cn);
                kw_next = key_word(cn);
            }
        }
        step(sA, pA, unit_of(kt, 0, full), sB, kbuf(J), 1, vbuf(J + 3), 1, pB, kbuf(J + 1), 0, vbuf(J), 0,
             (uint32_t)(kw >> 32), [&](int i) __attribute__((always_inline)) { issue_v1(v_dst, v_base, i); });
        step(sB, pB, unit_of(kt, 1, full), sA, kbuf(J + 1), 0, vbuf(J), 0, pA, kbuf(J + 1), 1, vbuf(J), 1,
             (uint32_t)kw_next, [&](int i) __attribute__((always_inline)) { issue_k1(k_dst, k_base, k_kt, i); });
        kw = kw_next;
        if (j + 1 < nT) {  // the compute cursor moves on to tile j + 1
            const int e_was = cc.e;
            cur_next(cc);
            if (cc.e != e_was) {
                cc_flo = tab32(2, cc.e);
                cc_fhi = tab32(3, cc.e);
                if (KP) cc_kb = tab32(4, cc.e);
                row_bounds(tab64(2, cc.e));
            }
        }
    };

#pragma unroll
    for (int db = 0; db < D / 32; db++) o[db] = f32x16{};
    // The Q loads were issued before any tile load: the wait for batch A below
    // covers them too (vector-memory loads complete in issue order).
    // Batch A: K_0, V_0, K_1; batch B: K_2, V_1.  V buffer 3 stands for
    // V_{-1} (P_{-1} = 0 multiplies it): zeroed.
    issue_k(kbuf(0), ck.kp, ck.c.kt);
    issue_v(vbuf(0), ck.vp);
    lc_next(ck);
    issue_k(kbuf(1), ck.kp, ck.c.kt);
    v_pend = ck.vp;
    lc_next(ck);
    issue_k(kbuf(2), ck.kp, ck.c.kt);
    issue_v(vbuf(1), v_pend);
    v_pend = ck.vp;
    for (int i = threadIdx.x; i < TL::ELEMS / 8; i += THREADS) ((bf16x8*)vbuf(3))[i] = bf16x8{};
    wait_loads_but<2 * LPW>();  // batch A
    tile_barrier();
    // S of unit (0, 0) and the operand ring of step 0 (K_0 half 1, V_{-1} half 1).
    kw = key_word(cc);
    {
        f32x16 s0 = s_init((uint32_t)kw);
#pragma unroll
        for (int kc = 0; kc < D / 16; kc++) s0 = mma<E>(*(const bf16x8*)(kbuf(0) + 512 * kc + 8 * lane), qf[kc], s0);
        sA = s0;
    }
#pragma unroll
    for (int n = 0; n < LA; n++) ring[n] = frag(kbuf(0), 1, vbuf(3), 1, n);
    // Whole groups of NBUF iterations, then the 0 to NBUF - 1 left over (j
    // is a multiple of NBUF after the loop).
    static_assert(NBUF == 4, "the unrolled tile loop below");
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    using I3 = std::integral_constant<int, 3>;
    int j = 0;
    for (; j + NBUF <= nT; j += NBUF) {
        iteration(j, I0{});
        iteration(j + 1, I1{});
        iteration(j + 2, I2{});
        iteration(j + 3, I3{});
    }
    if (j < nT) iteration(j, I0{});
    if (j + 1 < nT) iteration(j + 1, I1{});
    if (j + 2 < nT) iteration(j + 2, I2{});
    // PV of the last unit (nT-1, 1) from V_{nT-1}; the ring holds its first
    // operands (the S slots' fragments are unused).
#pragma unroll
    for (int n = 1; n < NSLOT; n += 2) {
        const int m = n / 2, q = m / TL::DB, db = m % TL::DB;
        const bf16x8 fr = n < LA ? ring[n % LA] : frag(kbuf(0), 0, vbuf(nT - 1), 1, n);
        o[db] = mma<E>(fr, pB[q], o[db]);
    }
    wait_loads_but<0>();  // no load may land in LDS after the workgroup ends

    // Both halves of a row combine their denominators; then rescale to the
    // reference's maximum.
    float ltot = lsum + other_half(lsum);
    if (mx != -INFINITY) {
        const float beta = __builtin_amdgcn_exp2f(mrc - mx * a.c2);
        ltot *= beta;
#pragma unroll
        for (int db = 0; db < D / 32; db++) o[db] *= beta;
    }
    if (!row_ok) return;
    const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
    char* ob = (char*)a.out;
    const int64_t oe = out_off + urow * a.out_row_stride + head * a.out_head_stride + 4 * half;
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
        a.lse[lse_off + head * a.lse_head_stride + urow * a.lse_row_stride] =
            ltot > 0.f ? mx * a.scale + logf(ltot) : -INFINITY;
    };  // run_item

    // Every fetch tries each queue at most once, and a queue once found empty
    // is not tried again: the loop ends for every workgroup once all queues
    // are drained.  The barriers keep the item number and the LDS (tables,
    // tile buffers) of one item apart from the next.
    for (;;) {
        __syncthreads();
        if (threadIdx.x == 0) {
            int it = -1;
            for (int k = 0; k < 8 && it < 0; k++) {
                const int y = (own_q + k) & 7;
                if ((q_done >> y) & 1u) continue;
                const int len = y < n_items ? (n_items - y + 7) / 8 : 0;
                const unsigned i = atomicAdd(&a.wq[y], 1u);
                if ((int)i < len) it = 8 * (int)i + y;
                else q_done |= 1u << y;
            }
            item_s = it;
        }
        __syncthreads();
        const int b = __builtin_amdgcn_readfirstlane(item_s);
        if (b < 0) break;
        run_item(b);
    }
}

template <typename E, bool KP>
hipError_t launch16(const StepArgs& a, hipStream_t stream) {
    if (a.hpi < 1 || a.hpi > WAVES || (a.hpi & (a.hpi - 1)) || a.group % a.hpi) return hipErrorInvalidValue;
    const int64_t n_items = (int64_t)a.n_qtiles * (a.Hq / a.hpi) * a.n_pairs;
    if (n_items == 0) return hipSuccess;
    if (!a.wq || n_items > INT32_MAX) return hipErrorInvalidValue;
    int n_cu = 0;  // one workgroup per compute unit
    const hipError_t e = cu_count(&n_cu);
    if (e != hipSuccess) return e;
    const dim3 grid((unsigned)(n_items < n_cu ? n_items : n_cu)), block(THREADS);
    if (a.d == 128) {
        if (a.qt_major) ring_fwd_kernel<E, 128, KP, true><<<grid, block, 0, stream>>>(a);
        else ring_fwd_kernel<E, 128, KP, false><<<grid, block, 0, stream>>>(a);
    } else if (a.d == 64) {
        if (a.qt_major) ring_fwd_kernel<E, 64, KP, true><<<grid, block, 0, stream>>>(a);
        else ring_fwd_kernel<E, 64, KP, false><<<grid, block, 0, stream>>>(a);
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_ring_fwd(const StepArgs& a, hipStream_t stream) {
    if (!a.works || !a.vt) return hipErrorInvalidValue;
    // KP: with a key-padding mask (the unmasked kernels carry none of its code)
    if (a.kbits) return a.f16 ? launch16<f16, true>(a, stream) : launch16<bf16, true>(a, stream);
    return a.f16 ? launch16<f16, false>(a, stream) : launch16<bf16, false>(a, stream);
}

}  // namespace ra
