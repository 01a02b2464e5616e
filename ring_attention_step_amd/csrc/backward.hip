// Backward of the ring forward on the matrix cores (16-bit inputs, bf16 or
// fp16 -- the kernels' E --, fp32 accumulation): the gradients dq, dk, dv of out = ring attention(q, k, v)
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
//  * bwd_prep: D_t and lse_t log2(e) for every (head, row), stored in
//    block-local row order (block b's rows at b B .. b B + B - 1), so that
//    the rows of any tile of a block are contiguous in both layouts.
//  * bwd_dq: one workgroup (8 waves x 32 query rows) per (virtual device,
//    head, 256-row query tile), its q and dout rows held in registers,
//    walking the device's visited key/value blocks in ring order in 64-key
//    tiles streamed through LDS.  Per wave, with S^T = K Q^T so that one
//    query row sits in each lane:
//      S^T = K Q^T, dP^T = V dout^T, dS^T = P^T (dP^T - D), dq^T += K^T dS^T,
//    the last through transposing LDS reads of the K tile.
//  * bwd_dkdv: one workgroup (8 waves) per (key/value block, KV head,
//    128-key tile), walking the query blocks that visit the block, every
//    query head of the KV head's group, in 64-row query tiles streamed
//    through LDS.  Each 32 keys have two waves on one SIMD, the dV wave
//    holding their keys and the dK wave their values in registers, with
//    S = Q K^T so that one key sits in each lane:
//      dV wave:  S = Q K^T, P (handed to the dK wave through LDS), dv^T += dout^T P;
//      dK wave:  dP = dout V^T, dS = P (dP - D), dk^T += q^T dS,
//    the last products through transposing reads of the dout and q tiles;
//    the dK wave runs one query tile behind the dV wave, so P crosses a
//    barrier instead of being waited for.  Each wave holds one set of
//    32 x d accumulators, so two waves fit per SIMD.
// dq streams its tiles through a three-stage LDS ring filled by direct
// global -> LDS loads issued two tiles ahead; dk/dv through three stages
// loaded one tile ahead (two are read per iteration).  Tiles that the mask skips entirely are never loaded:
// per block the non-skipped tiles form one contiguous range (causal: a
// skipped prefix or suffix; doc-causal: both), found before the walk.
//
// The lane layouts of the 32x32x16 bf16 MFMA are those of the forward
// kernel: accumulator register i of lane l holds row 8 (i/4) + 4 (l/32) + i%4
// and column l % 32; an A operand holds row l % 32 and k = 8 (l/32) .. + 7;
// a B operand k = 8 (l/32) .. + 7 and column l % 32.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <type_traits>

#include "bwd_kernels.h"
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
typedef __attribute__((address_space(3))) void lds_void;
typedef int i32x4 __attribute__((ext_vector_type(4)));

template <int I>
using ic = std::integral_constant<int, I>;

constexpr int DQ_WAVES = 8;                // dq: two waves per SIMD
constexpr int DQ_THREADS = 64 * DQ_WAVES;
constexpr int KV_WAVES = 8;                // dk/dv: two waves per 32 keys (dV, dK), two per SIMD
constexpr int KV_THREADS = 64 * KV_WAVES;
constexpr int BW_TQ = 32 * DQ_WAVES;       // query rows per dq workgroup
constexpr int BW_TK = 32 * (KV_WAVES / 2); // keys per dk/dv workgroup
constexpr int BW_T = 64;                   // rows of a streamed tile (keys for dq, queries for dk/dv)
// The LDS operands of a run of matrix instructions are read kla() instructions
// ahead into a ring of registers, each step of the run fenced by a
// scheduling barrier: read next to its use, every operand would stall its
// instruction for the whole LDS latency (the compiler's own schedule does
// that to save registers).
template <int D>
constexpr int kla() { return D == 128 ? 4 : 2; }
constexpr float kLog2e = 1.4426950408889634f;
static_assert(kBwdPad >= 64, "a 64-row tile may read 63 rows past the last block");

// A [64 rows][D] bf16 tile in LDS, 16-byte chunks XOR-swizzled per row:
// logical chunk c of row r at slot c ^ swz(r).  Both kinds of operand read
// are free of bank conflicts (measured with the LDS bank-conflict counter):
//  row reads: 16 lanes read one chunk column of 16 consecutive rows, which
//    swz spreads over 16 distinct slots;
//  transposing reads: 32 lanes read 64 bytes (4 chunks) of each of 4 rows
//    4j .. 4j + 3, which swz moves to 4 different 64-byte quarters of the
//    256-byte bank window (D = 128: by 4 (r & 3); D = 64, where two
//    rows share the window, by 4 ((r >> 1) & 1) and the row's half).
// (r & (D/8 - 1), the plain choice, costs the transposing reads 6 conflict
// cycles each.)  Rows r and r + 8 (r < 8) differ by XOR 2.
template <int D>
__device__ __forceinline__ constexpr int swz(int r) {
    return D == 128 ? ((4 * (r & 3)) ^ ((r >> 2) & 3)) & 15 : ((4 * ((r >> 1) & 1)) ^ ((r >> 2) & 3)) & 7;
}

__device__ __forceinline__ i16x4 lds_read_tr(const bf16* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(p));
}

// s_waitcnt vmcnt(N): all but this wave's N most recent vector-memory loads
// have landed; through the builtin so the compiler's own bookkeeping sees it.
template <int N>
__device__ __forceinline__ void wait_loads_but() {
    static_assert(N >= 0 && N < 16, "vmcnt field");
    __builtin_amdgcn_s_waitcnt(0x0F70 | N);
}

// Workgroup barrier that waits for this wave's LDS traffic only: the direct
// stage loads stay in flight across it (each is waited for explicitly
// before the barrier that hands its buffer to the readers).
__device__ __forceinline__ void phase_barrier() {
    __builtin_amdgcn_sched_barrier(0);
    __asm__ volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
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

// Byte offset, from the tile's first row, of the global 16-byte chunk that
// lands in LDS slot s = 64 n + lane of a [64][D] tile (row s / (D/8), slot
// column s % (D/8), logical chunk slot ^ swz(row)); rows past last_row
// re-read last_row (callers mask them).
template <int D>
__device__ __forceinline__ uint32_t chunk_offset(int lane, int n, uint32_t rs_bytes, int last_row) {
    constexpr int CH = D / 8;
    const int s = 64 * n + lane;
    const int r = s / CH;
    const uint32_t row = (uint32_t)(r < last_row ? r : last_row);
    return row * rs_bytes + 16u * (uint32_t)((s % CH) ^ swz<D>(r));
}

// One 1 KB block by a direct-to-LDS buffer load: lane l's 16 bytes at
// base + voff land at LDS byte address lds + 16 l.  The resource is a raw
// buffer at base (no stride, no bound; every offset lies inside the tensor or
// its padding).  Written in asm, so that the compiler does not pair LDS reads
// with these loads: once a wave picks its stage at run time it cannot tell
// the stages apart and would wait for every load before each read; the
// waits are explicit (wait_loads_but, barriers).  M0 holds the LDS address;
// one wait state separates its write from the load.
__device__ __forceinline__ void dma16(uint32_t lds, const char* base, uint32_t voff) {
    const uint64_t b = (uint64_t)base;
    i32x4 r;
    r[0] = (int)(uint32_t)b;
    r[1] = (int)(uint32_t)(b >> 32);
    r[2] = -1;
    r[3] = 0x00020000;
    __asm__ volatile("s_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds" ::"{m0}"(lds), "v"(voff), "s"(r) : "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) { return (uint32_t)(uintptr_t)(lds_void*)p; }

// MFMA operand offsets (elements) into a swizzled [rows][D] tile:
//  row operand (A or B) of row 32 rb + col, dims 16 kc + 8 half .. + 7;
//  transposing pair for rows 16 q + vrow (+8), dims 32 db + 16 g + 4 (j % 4),
//  which gives lane l dim 32 db + l % 32 and, as its 8 k values, the rows
//  16 q + 4 half + 0..3 and 16 q + 8 + 4 half + 0..3 (accumulator order).
template <int D>
struct TileOps {
    int row_off[D / 16];
    int tr_off[D / 32];
    int tr_d8;  // rows vrow + 8 relative to rows vrow (the same for every db)
    __device__ TileOps(int lane) {
        const int col = lane & 31, half = lane >> 5;
#pragma unroll
        for (int kc = 0; kc < D / 16; kc++) row_off[kc] = col * D + 8 * ((2 * kc + half) ^ swz<D>(col));
        const int j16 = lane & 15, g16 = (lane >> 4) & 1, vrow = 4 * half + (j16 >> 2);
#pragma unroll
        for (int db = 0; db < D / 32; db++) {
            const int chunk = 4 * db + 2 * g16 + ((j16 & 3) >> 1);
            tr_off[db] = vrow * D + 8 * (chunk ^ swz<D>(vrow)) + 4 * (j16 & 1);
        }
        // swz(vrow + 8) = swz(vrow) ^ 2 with bit 1 of swz(vrow) clear, so
        // the chunk moves by 2 slots, down when bit 1 of the chunk (g16) is set.
        tr_d8 = 8 * D + (g16 ? -16 : 16);
    }
    __device__ __forceinline__ bf16x8 row(const bf16* t, int rb, int kc) const {
        return *(const bf16x8*)(t + row_off[kc] + 32 * D * rb);
    }
    __device__ __forceinline__ bf16x8 tr(const bf16* t, int q, int db) const {
        const i16x4 r1 = lds_read_tr(t + tr_off[db] + 16 * q * D);
        const i16x4 r2 = lds_read_tr(t + tr_off[db] + tr_d8 + 16 * q * D);
        return __builtin_bit_cast(bf16x8, __builtin_shufflevector(r1, r2, 0, 1, 2, 3, 4, 5, 6, 7));
    }
};

// 16-bit operands are held as raw values in the bf16 vector type; E (bf16 or
// fp16) picks the matrix-core instruction and the conversions.
template <typename E>
__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
    if constexpr (std::is_same<E, f16>::value)
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c,
                                                      0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

template <typename E>
__device__ __forceinline__ bf16 to16(float x) {  // round to E (nearest even)
    return __builtin_bit_cast(bf16, (E)x);
}

template <typename E>
__device__ __forceinline__ float from16(bf16 x) {
    return (float)__builtin_bit_cast(E, x);
}

// Accumulator register order -> 16-bit operand pair (16-row chunks 2 h, 2 h + 1).
template <typename E>
__device__ __forceinline__ void acc_to_b(const f32x16& acc, bf16x8& b0, bf16x8& b1) {
#pragma unroll
    for (int i = 0; i < 8; i++) {
        b0[i] = to16<E>(acc[i]);
        b1[i] = to16<E>(acc[8 + i]);
    }
}

// ---- D = rowsum(dout * out), lse log2(e) ----
// d / 8 lanes per (token, head) row, 8 elements each, reduced by shuffles.
// Outputs in block-local order: row u of block b (token pos(b, u)) at
// h T + b B + u; lse = -inf (a row with no key) becomes +inf, so that every
// P of the row is exp2(-inf) = 0.
template <typename E>
__global__ void bwd_prep_kernel(const BwdArgs a) {
    const int lanes = a.d / 8;
    const int64_t n = (int64_t)a.T * a.Hq;
    // The padding after both arrays (tiles of a block's last rows read up to
    // 63 rows past it): finite values.
    if (blockIdx.x == 0 && threadIdx.x < kBwdPad) {
        a.Dsum[n + threadIdx.x] = 0.f;
        a.Lse2[n + threadIdx.x] = INFINITY;
    }
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t x0 = (int64_t)blockIdx.x * blockDim.x; x0 < n * lanes; x0 += stride) {
        const int64_t x = x0 + threadIdx.x;
        const int64_t row = x / lanes;
        const int c = (int)(x % lanes);
        float s = 0.f;
        int64_t t = 0, h = 0;
        if (row < n) {
            t = row / a.Hq;
            h = row % a.Hq;
            const bf16x8 gv = *(const bf16x8*)((const bf16*)a.dout + t * a.do_st + h * a.do_sh + 8 * c);
            const int64_t oe = t * a.out_st + h * a.out_sh + 8 * c;
            if (a.out16) {
                const bf16x8 ov = *(const bf16x8*)((const bf16*)a.out + oe);
#pragma unroll
                for (int e = 0; e < 8; e++) s = fmaf(from16<E>(ov[e]), from16<E>(gv[e]), s);
            } else {
                const f32x4 o0 = *(const f32x4*)((const float*)a.out + oe);
                const f32x4 o1 = *(const f32x4*)((const float*)a.out + oe + 4);
#pragma unroll
                for (int e = 0; e < 4; e++) s = fmaf(o0[e], from16<E>(gv[e]), s);
#pragma unroll
                for (int e = 0; e < 4; e++) s = fmaf(o1[e], from16<E>(gv[4 + e]), s);
            }
        }
        for (int w = 1; w < lanes; w <<= 1) s += __shfl_xor(s, w, 64);
        if (row < n && c == 0) {
            const int64_t loc = a.pos_stride == 1 ? t : (t % a.pos_stride) * a.B + t / a.pos_stride;
            const float l = a.lse[h * a.T + t];
            a.Dsum[h * a.T + loc] = s;
            a.Lse2[h * a.T + loc] = l == -INFINITY ? INFINITY : l * kLog2e;
        }
    }
}

// Workgroup b of a grid of groups x per_group workgroups -> (group, index in
// group).  Consecutive workgroup ids are dispatched to the 8 XCDs in turn;
// when the group count is a multiple of 8 every group is kept on one XCD
// (XCD b % 8 takes groups b % 8, b % 8 + 8, ...), else plain row order.
__device__ __forceinline__ void xcd_map(int b, int nwg, int per_group, int& group, int& idx) {
    const int n_groups = nwg / per_group;
    if (n_groups % 8 == 0) {
        const int r = b / 8;
        group = b % 8 + 8 * (r / per_group);
        idx = r % per_group;
    } else {
        group = b / per_group;
        idx = b % per_group;
    }
}

// The tile-index-major numbering of striped layouts (QM): XCD b % 8 runs
// one tile index of all its groups before the next (rank r = b / 8: index
// r / per, group b % 8 + 8 (r % per)), so that the items running together
// stream the same tiles; else plain index-major order.  Every pair of a
// striped chain is cut by the causal diagonal alike, so items of one tile
// index and one chain order read the same tiles in step, while items of
// one group but different indices drift apart by whole blocks.
__device__ __forceinline__ void xcd_map_qm(int b, int nwg, int per_group, int& group, int& idx) {
    const int n_groups = nwg / per_group;
    if (n_groups % 8 == 0) {
        const int r = b / 8, per = n_groups / 8;
        group = b % 8 + 8 * (r % per);
        idx = r / per;
    } else {
        group = b % n_groups;
        idx = b / n_groups;
    }
}

// Group -> (head, block index) for H heads: under QM with H a multiple of 8
// (and the groups dealt evenly), XCD y = group % 8 takes heads y H/8 ..
// y H/8 + H/8 - 1, whole kv-head groups of a grouped-query layout when H/8
// is a multiple of the group, so that one L2 serves their shared tiles;
// else head = group % H.
template <bool QM>
__device__ __forceinline__ void group_head(int group, int n_groups, int H, int& head, int& blk) {
    if (QM && H % 8 == 0 && n_groups % 8 == 0) {
        const int g = group / 8, hx = H / 8;
        head = (group % 8) * hx + g % hx;
        blk = g / hx;
    } else {
        head = group % H;
        blk = group / H;
    }
}

// First index in [0, n) where a predicate that is false, then true, holds
// (n when it never does).  Every condition of classify() on a streamed tile
// is monotone in the tile index (positions grow with it; document starts
// too), so the skipped prefix and suffix and the fully visible range of a
// block are found by bisection on those conditions.
template <typename Pred>
__device__ __forceinline__ int first_true(int n, Pred pred) {
    int l = 0, h = n;
    while (l < h) {
        const int m = (l + h) >> 1;
        if (pred(m)) h = m;
        else l = m + 1;
    }
    return l;
}

// The non-skipped range [lo, hi] and the fully visible one [flo, fhi] of a
// block, normalised: (0, -1) when nothing is visible, (hi + 1, hi) when no
// tile is full.
__device__ __forceinline__ void tile_bounds_fix(int& lo, int& hi, int& flo, int& fhi) {
    if (flo < lo) flo = lo;
    if (fhi > hi) fhi = hi;
    if (lo > hi) {
        lo = 0;
        hi = -1;
    }
    if (flo > fhi) {
        flo = hi + 1;
        fhi = hi;
    }
}

// ---- dq ----
template <typename E, int D, bool KP, bool QM>
__global__ __launch_bounds__(DQ_THREADS, 1) void bwd_dq_kernel(const BwdArgs a) {
    constexpr int TE = BW_T * D;              // elements of one [64][D] tile
    constexpr int NL = 2 * (TE / 512 / DQ_WAVES);  // loads per wave per stage: K tile, then V tile
    // Three stages, one array each (K tile, then V tile).
    __shared__ bf16 st0[2 * TE], st1[2 * TE], st2[2 * TE];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int half = lane >> 5, col = lane & 31;
    __shared__ int item_s;
    const int n_items = a.n_works * a.Hq * a.n_qtiles;
    const int own_q = blockIdx.x & 7;
    unsigned q_done = 0;  // thread 0: queues found empty
    auto run_item = [&](const int b) __attribute__((always_inline)) {
    // Workgroup -> (device, head, q-tile): the q-tiles of one (device, head)
    // group share every K/V tile they stream, so they run on one XCD (whose
    // L2 then serves the re-reads); consecutive workgroup ids go to the 8
    // XCDs in turn, so groups are dealt to the XCDs round robin.  Within a
    // group the q-tiles run last first (under causal masks they have the
    // most keys).
    int grp_id, qi, head, widx;
    if (QM) xcd_map_qm(b, n_items, a.n_qtiles, grp_id, qi);
    else xcd_map(b, n_items, a.n_qtiles, grp_id, qi);
    group_head<QM>(grp_id, n_items / a.n_qtiles, a.Hq, head, widx);
    const int qt = a.n_qtiles - 1 - qi;
    const int kvh = head / a.group;
    const BwdWork w = a.works[widx];
    const int64_t B = a.B, ps = a.pos_stride;
    // Per-lane mask state in 32 bits (positions and indices stay below 2^31).
    const int u = qt * BW_TQ + wave * 32 + col;  // this lane's query row (local)
    const bool row_ok = u < B;
    const int64_t ur = row_ok ? u : B - 1;
    const int64_t t_row = w.pos0 + ur * ps;  // its global position = token row
    const float lse2 = row_ok ? a.Lse2[head * a.T + w.loc0 + ur] : INFINITY;
    const float drow = row_ok ? a.Dsum[head * a.T + w.loc0 + ur] : 0.f;
    const int ds_row = a.mask == kMaskDoc ? (int)doc_start(a.cu, a.n_docs, t_row) : 0;

    // This wave's q and dout rows as B operands (row u, dims 16 kc + 8 half .. + 7).
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
    // The chain table, one visited block per lane (lane e < count holds
    // block e): its first position, non-skipped key tiles [lo, hi] and fully
    // visible ones [flo, fhi] (contiguous, between the partial tiles).  The
    // loop reads it with readlane and so issues no memory loads besides the
    // stage loads (a load waited for inside the loop would also wait for
    // every stage load issued before it).
    // (Positions fit 32 bits; the fully visible range is packed as two
    // 16-bit fields, fhi + 1 above flo: tile indices stay below 2^15.)
    int tb_lo = 0, tb_hi = -1, tb_full = 0;
    int tb_kp = 0;
    if (lane < w.count) {
        const int64_t kp = a.partners[w.first + lane];
        tb_kp = (int)kp;
        // classify()'s conditions on key tile x of this block (rows [t_min, t_max])
        auto tk_first = [&](int x) { return kp + (int64_t)x * BW_T * ps; };
        auto tk_last = [&](int x) { return kp + ((B < (int64_t)x * BW_T + BW_T ? B : (int64_t)x * BW_T + BW_T) - 1) * ps; };
        int flo = 0, fhi = nkt - 1;
        tb_hi = nkt - 1;
        if (a.mask != kMaskNone) {
            if (a.mask == kMaskDoc) {
                tb_lo = first_true(nkt, [&](int x) { return tk_last(x) >= ds_min; });
                flo = first_true(nkt, [&](int x) { return tk_first(x) >= ds_max; });
            }
            tb_hi = first_true(nkt, [&](int x) { return tk_first(x) > t_max; }) - 1;
            fhi = first_true(nkt, [&](int x) { return tk_last(x) > t_min; }) - 1;
        }
        tile_bounds_fix(tb_lo, tb_hi, flo, fhi);
        tb_full = flo | ((fhi + 1) << 16);
    }
    auto rl32 = [&](int x, int e) __attribute__((always_inline)) { return __builtin_amdgcn_readlane(x, e); };
    // Streamed tiles: every non-skipped key tile of every visited block.
    struct Cursor {
        int e, kt, hi;
        int64_t kp;  // position of the block's row 0
    };
    auto cur_next = [&](Cursor& c) __attribute__((always_inline)) {
        int e = c.e, kt = c.kt + 1, hi = c.hi;
        while (kt > hi && e + 1 < w.count) {
            e++;
            kt = rl32(tb_lo, e);
            hi = rl32(tb_hi, e);
        }
        if (kt <= hi) c = Cursor{e, kt, hi, (int64_t)rl32(tb_kp, e)};
    };
    int nT = 0;
    for (int e = 0; e < w.count; e++) nT += rl32(tb_hi, e) - rl32(tb_lo, e) + 1;

    // This row's allowed keys of the block at kp: local indices [w_lo, w_hi).
    // A key must not follow the row: w ps + kp <= u ps + pos0, that is
    // w <= u + floor((pos0 - kp) / ps), the last term per block (both row-0
    // positions lie below ps when striped) and computed in scalar code.
    int w_lo = 0, w_hi = 0;
    auto row_bounds = [&](int64_t kp) __attribute__((always_inline)) {
        w_lo = 0;
        w_hi = row_ok ? (int)B : 0;
        if (a.mask != kMaskNone) {
            const int dd = (int)(w.pos0 - kp);
            const int shift = ps == 1 ? dd : (dd >= 0 ? 0 : -1);  // floor(dd / ps), |dd| < ps when striped
            const int last = u + shift;
            if (last + 1 < w_hi) w_hi = last + 1 < 0 ? 0 : last + 1;
            if (a.mask == kMaskDoc && ds_row - (int)kp > 0) w_lo = ds_row - (int)kp;
        }
    };

    // Chunk offsets of this wave's loads (K: loads 0 .. NL/2-1 of the tile's
    // K part, V likewise), recomputed for a ragged last tile.
    const uint32_t k_rs = (uint32_t)(ps * a.k_st * 2), v_rs = (uint32_t)(ps * a.v_st * 2);
    const int last_full = BW_T - 1, last_ragged = (int)((B - 1) % BW_T);
    const int ragged_kt = B % BW_T ? nkt - 1 : -1;
    // Offsets of a full tile stay in registers; a ragged tile's are computed
    // when it is issued, and selected without a branch around the loads.
    uint32_t off_k[NL / 2], off_v[NL / 2];
#pragma unroll
    for (int i = 0; i < NL / 2; i++) {
        off_k[i] = chunk_offset<D>(lane, wave * (NL / 2) + i, k_rs, last_full);
        off_v[i] = chunk_offset<D>(lane, wave * (NL / 2) + i, v_rs, last_full);
    }
    const char* const k_head = (const char*)((const bf16*)a.k + kvh * a.k_sh);
    const char* const v_head = (const char*)((const bf16*)a.v + kvh * a.v_sh);
    auto issue = [&](bf16* ks, bf16* vs, const Cursor& c) __attribute__((always_inline)) {
        const int64_t row0 = c.kp + (int64_t)c.kt * BW_T * ps;  // token of the tile's first key
        const bool rag = c.kt == ragged_kt;
        uint32_t ok[NL / 2], ov[NL / 2];
#pragma unroll
        for (int i = 0; i < NL / 2; i++) {
            ok[i] = rag ? chunk_offset<D>(lane, wave * (NL / 2) + i, k_rs, last_ragged) : off_k[i];
            ov[i] = rag ? chunk_offset<D>(lane, wave * (NL / 2) + i, v_rs, last_ragged) : off_v[i];
        }
        const uint32_t lk = lds_addr(ks) + 1024u * (uint32_t)(wave * (NL / 2));
        const uint32_t lv = lds_addr(vs) + 1024u * (uint32_t)(wave * (NL / 2));
#pragma unroll
        for (int i = 0; i < NL / 2; i++) dma16(lk + 1024u * i, k_head + row0 * a.k_st * 2, ok[i]);
#pragma unroll
        for (int i = 0; i < NL / 2; i++) dma16(lv + 1024u * i, v_head + row0 * a.v_st * 2, ov[i]);
    };

    int cc_flo = 0, cc_fhi = -1;  // fully visible tiles of the compute cursor's block
    // Key-padding mask: the compute cursor's block's first bit word, and the
    // validity word of its tile (all ones without a mask).
    int kb_cur = 0;
    uint64_t kw = ~0ull;

    auto key_word = [&](const Cursor& c) __attribute__((always_inline)) {
        typedef const __attribute__((address_space(4))) uint64_t* cwp;
        return *(cwp)(a.kbits + kb_cur + 2 * c.kt);
    };
    auto compute = [&](const bf16* ks, const bf16* vs, const Cursor& c) __attribute__((always_inline)) {
        const int64_t w0 = (int64_t)c.kt * BW_T;
        const bool full = c.kt != ragged_kt && c.kt >= cc_flo && c.kt <= cc_fhi;
        // Allowed keys shifted by -4 half, relative to the tile (|x| <= B + 4).
        const int x_lo = w_lo - (int)w0 - 4 * half, x_hi = w_hi - (int)w0 - 4 * half;
#pragma unroll
        for (int kb = 0; kb < 2; kb++) {
            // S^T and dP^T: keys 32 kb .. + 31 of the tile (rows) x this wave's rows.
            f32x16 s = f32x16{}, dp = f32x16{};
            if (KP) {
                // Key-padding mask on the matrix core: one extra 16-deep product
                // adds -inf (padded key, A row = lane r at k = 0) or 0 to every
                // score of key 32 kb + r (B = 1 at k = 0 for every query).
                // Both operands are rebuilt here from a lane id the compiler cannot
                // trace (an empty asm), so it keeps no loop-invariant copy of them.
                int l = threadIdx.x & 63;
                __asm__ volatile("" : "+v"(l));
                const bool lo_half = l < 32;
                const uint32_t word = kb ? (uint32_t)(kw >> 32) : (uint32_t)kw;
                bf16x8 bias = bf16x8{}, one = bf16x8{};
                bias[0] = (lo_half && !((word >> (l & 31)) & 1u)) ? to16<E>(-INFINITY) : to16<E>(0.0f);
                one[0] = lo_half ? to16<E>(1.0f) : to16<E>(0.0f);
                s = mfma<E>(bias, one, s);
            }
            {
                // K rows (even n) and V rows (odd n), read KLA instructions
                // ahead into a ring of registers (next to its use, each read
                // would stall its instruction for the whole LDS latency).
                constexpr int NR = 2 * (D / 16), KLA = kla<D>();
                auto rd = [&](int n) __attribute__((always_inline)) { return ops.row(n % 2 ? vs : ks, kb, n / 2); };
                bf16x8 ring[KLA];
#pragma unroll
                for (int n = 0; n < KLA; n++) ring[n] = rd(n);
#pragma unroll
                for (int n = 0; n < NR; n++) {
                    const bf16x8 fr = ring[n % KLA];
                    if (n + KLA < NR) ring[n % KLA] = rd(n + KLA);
                    if (n % 2 == 0) s = mfma<E>(fr, qf[n / 2], s);
                    else dp = mfma<E>(fr, gf[n / 2], dp);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
            // dS^T = P^T (dP^T - D); register i holds key 32 kb + 8 (i/4) + 4 half + i%4.
            // A masked key's exponent becomes -inf (P = 0, dS = 0): selects,
            // so that no per-element branch is formed around the exp2.  Fully
            // visible tiles take a copy without the mask (the branch holds
            // vector work only, so the accumulators stay in place).
            bf16x8 b0, b1;
            auto softmax = [&](auto full_t) __attribute__((always_inline)) {
                constexpr bool FULL = decltype(full_t)::value;
                f32x16 dsv;
#pragma unroll
                for (int i = 0; i < 16; i++) {
                    const int x = 32 * kb + 8 * (i / 4) + (i % 4);
                    float arg = fmaf(s[i], a.c2, -lse2);
                    if (!FULL) arg = ((x >= x_lo) & (x < x_hi)) ? arg : -INFINITY;
                    dsv[i] = __builtin_amdgcn_exp2f(arg) * (dp[i] - drow);
                }
                acc_to_b<E>(dsv, b0, b1);
            };
            if (__builtin_amdgcn_readfirstlane((int)full)) softmax(std::true_type{});
            else softmax(std::false_type{});
            // dq^T += K^T dS^T over the two 16-key chunks of this half
            // (instruction n: block db = n / 2, chunk n % 2), operands read ahead.
            {
                constexpr int NR = 2 * (D / 32);
                constexpr int LA = kla<D>() < NR ? kla<D>() : NR;
                auto rd = [&](int n) __attribute__((always_inline)) { return ops.tr(ks, 2 * kb + n % 2, n / 2); };
                bf16x8 ring[LA];
#pragma unroll
                for (int n = 0; n < LA; n++) ring[n] = rd(n);
#pragma unroll
                for (int n = 0; n < NR; n++) {
                    const bf16x8 fr = ring[n % LA];
                    if (n + LA < NR) ring[n % LA] = rd(n + LA);
                    dq[n / 2] = mfma<E>(fr, n % 2 ? b1 : b0, dq[n / 2]);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        }
    };

    // ---- pipeline: tile j in stage j % 3, issued two tiles ahead ----
    Cursor cl{-1, 0, -1, 0};
    cur_next(cl);
    Cursor cc = cl;
    auto enter_block = [&](const Cursor& c) __attribute__((always_inline)) {
        row_bounds(c.kp);
        const int f = rl32(tb_full, c.e);
        cc_flo = f & 0xffff;
        cc_fhi = (f >> 16) - 1;
        // block index: position of row 0 over B (contiguous) or itself (striped)
        if (KP) kb_cur = (ps == 1 ? (int)((uint32_t)c.kp / (uint32_t)B) : (int)c.kp) * a.kb_words;
    };
    if (nT > 0) {
        enter_block(cc);
        if (KP) kw = key_word(cc);
    }
    auto iteration = [&](int j, auto slot) __attribute__((always_inline)) {
        constexpr int S = decltype(slot)::value;  // j % 3
        bf16* const kc = S == 0 ? st0 : (S == 1 ? st1 : st2);
        bf16* const vc = kc + TE;
        bf16* const kn = S == 0 ? st2 : (S == 1 ? st0 : st1);  // stage j + 2 (= j - 1)
        bf16* const vn = kn + TE;
        // Tile j + 2 (past the end: the last tile again, into a stage no
        // later iteration reads), so that every iteration issues NL loads.
        if (j + 2 < nT) cur_next(cl);
        issue(kn, vn, cl);
        compute(kc, vc, cc);
        if (j + 1 < nT) {
            const int e_was = cc.e;
            cur_next(cc);
            if (cc.e != e_was) enter_block(cc);
            if (KP) kw = key_word(cc);  // scalar load, complete at the barrier below
        }
        wait_loads_but<NL>();  // tile j + 1 has landed
        phase_barrier();
    };
    if (nT > 0) {
        wait_loads_but<0>();  // q / dout rows in registers: the waits below count stage loads only
        const Cursor c0 = cl;
        if (nT > 1) cur_next(cl);
        issue(st0, st0 + TE, c0);
        issue(st1, st1 + TE, cl);
        wait_loads_but<NL>();
        phase_barrier();
        // Whole triples of tiles in the loop, the rest after it, so that
        // every stage is a fixed array in the loop body.
        int j = 0;
        for (; j + 3 <= nT; j += 3) {
            iteration(j, ic<0>{});
            iteration(j + 1, ic<1>{});
            iteration(j + 2, ic<2>{});
        }
        if (j < nT) iteration(j, ic<0>{});
        if (j + 1 < nT) iteration(j + 1, ic<1>{});
        wait_loads_but<0>();  // no load may land in LDS after the workgroup ends
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
            if (a.grad16) *(bf16x4*)(ob + 2 * e) = bf16x4{to16<E>(x0), to16<E>(x1), to16<E>(x2), to16<E>(x3)};
            else *(f32x4*)(ob + 4 * e) = f32x4{x0, x1, x2, x3};
        }
    };  // run_item

    // One workgroup per compute unit takes items from the queue of its XCD
    // (numbers = that queue index mod 8, in order), then from the other
    // queues: see the forward's ring kernel.  Each fetch tries every queue at
    // most once, and an empty queue is not tried again, so the loop ends for
    // every workgroup once all queues are drained.
    for (;;) {
        __syncthreads();
        if (threadIdx.x == 0) {
            int it = -1;
            for (int k = 0; k < 8 && it < 0; k++) {
                const int y = (own_q + k) & 7;
                if ((q_done >> y) & 1u) continue;
                const int len = y < n_items ? (n_items - y + 7) / 8 : 0;
                const unsigned i = atomicAdd(&a.wq[0 + y], 1u);
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

// ---- dk, dv ----
template <typename E, int D, bool QM>
__global__ __launch_bounds__(KV_THREADS, 1) void bwd_dkdv_kernel(const BwdArgs a) {
    constexpr int TE = BW_T * D;
    constexpr int NQ = TE / 512 / KV_WAVES;  // loads per wave per stage for each of q and dout
    // Three stages in one array, each the q tile, the dout tile, then lse2 of
    // the tile's 64 rows and their D (1 KB, the upper half a duplicate
    // written by lanes 32..63).  Every wave loads that last KB (the same
    // bytes), so that each wave issues the same 2 NQ + 1 loads per stage.
    constexpr int SE = 2 * TE + 512;  // elements of one stage
    __shared__ __attribute__((aligned(16))) bf16 st[3 * SE];
    // P of a tile, handed from each dV wave to its dK partner one iteration
    // later, double-buffered by tile parity: [parity][32-key group][half sb]
    // [operand h][lane] 8 16-bit values (accumulator registers 8 h .. 8 h + 7),
    // so that each 16-byte access of a wave is contiguous.
    __shared__ bf16x8 p_lds[2][KV_WAVES / 2][2][2][64];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int role = wave >> 2;  // 0: dV, 1: dK
    const int kw = wave & 3;     // which 32 keys of the workgroup
    const int half = lane >> 5, col = lane & 31;
    __shared__ int item_s;
    const int n_items = a.n_rworks * a.Hkv * a.n_ktiles;
    const int own_q = blockIdx.x & 7;
    unsigned q_done = 0;  // thread 0: queues found empty
    auto run_item = [&](const int b) __attribute__((always_inline)) {
    // Workgroup -> (key block, kv head, key tile), the key tiles of one
    // (block, kv head) group on one XCD, as for dq; they run first to last
    // (under causal masks the first keys have the most queries).
    int grp_id, kt, kvh, ridx;
    if (QM) xcd_map_qm(b, n_items, a.n_ktiles, grp_id, kt);
    else xcd_map(b, n_items, a.n_ktiles, grp_id, kt);
    group_head<QM>(grp_id, n_items / a.n_ktiles, a.Hkv, kvh, ridx);
    const BwdWork w = a.rworks[ridx];
    const int64_t B = a.B, ps = a.pos_stride;
    const int64_t wk0 = (int64_t)kt * BW_TK;
    // Per-lane mask state in 32 bits (positions and indices stay below 2^31).
    const int wk = (int)wk0 + kw * 32 + col;  // this lane's key (local)
    const bool key_ok = wk < B;
    const int64_t p_key = w.pos0 + (key_ok ? wk : B - 1) * ps;  // its global position = token row
    const int de_key = a.mask == kMaskDoc ? (int)doc_end(a.cu, a.n_docs, p_key) : 0;

    // This wave's B operand rows (key wk, dims 16 kc + 8 half .. + 7): keys
    // for the dV wave (S = q K^T), values for the dK wave (dP = dout V^T).
    bf16x8 opf[D / 16];
    {
        const bf16* op = role ? (const bf16*)a.v + p_key * a.v_st + kvh * a.v_sh
                              : (const bf16*)a.k + p_key * a.k_st + kvh * a.k_sh;
#pragma unroll
        for (int kc = 0; kc < D / 16; kc++) opf[kc] = *(const bf16x8*)(op + 8 * half + 16 * kc);
    }
    const TileOps<D> ops(lane);
    f32x16 acc[D / 32];  // dV^T (dV wave) or dK^T / scale (dK wave)
#pragma unroll
    for (int db = 0; db < D / 32; db++) acc[db] = f32x16{};

    const int64_t wl = (B < wk0 + BW_TK ? B : wk0 + BW_TK) - 1;  // last key of the workgroup
    const int64_t tk_min = w.pos0 + wk0 * ps, tk_max = w.pos0 + wl * ps;
    const int nqt = (int)((B + BW_T - 1) / BW_T);
    // The table of visiting query blocks, one per lane (lane e < count
    // holds block e): its first position, non-skipped query tiles [lo, hi]
    // and fully visible ones [flo, fhi]; read with readlane in the loop,
    // which then issues no memory loads besides the stage loads.
    int tb_lo = 0, tb_hi = -1, tb_flo = 0, tb_fhi = -1;
    int64_t tb_qp = 0;
    if (lane < w.count) {
        tb_qp = a.rpartners[w.first + lane];
        // classify()'s conditions on query tile x of this block (keys [tk_min, tk_max])
        auto t_first = [&](int x) { return tb_qp + (int64_t)x * BW_T * ps; };
        auto t_last = [&](int x) { return tb_qp + ((B < (int64_t)x * BW_T + BW_T ? B : (int64_t)x * BW_T + BW_T) - 1) * ps; };
        tb_hi = nqt - 1;
        tb_flo = 0;
        tb_fhi = nqt - 1;
        if (a.mask != kMaskNone) {
            tb_lo = first_true(nqt, [&](int x) { return t_last(x) >= tk_min; });
            tb_flo = first_true(nqt, [&](int x) { return t_first(x) >= tk_max; });
            if (a.mask == kMaskDoc) {
                tb_hi = first_true(nqt, [&](int x) { return tk_max < doc_start(a.cu, a.n_docs, t_first(x)); }) - 1;
                tb_fhi = first_true(nqt, [&](int x) { return doc_start(a.cu, a.n_docs, t_last(x)) > tk_min; }) - 1;
            }
        }
        tile_bounds_fix(tb_lo, tb_hi, tb_flo, tb_fhi);
    }
    auto rl32 = [&](int x, int e) __attribute__((always_inline)) { return __builtin_amdgcn_readlane(x, e); };
    auto rl64 = [&](int64_t x, int e) __attribute__((always_inline)) {
        const uint32_t lo32 = __builtin_amdgcn_readlane((int)(uint32_t)x, e);
        const uint32_t hi32 = __builtin_amdgcn_readlane((int)(uint32_t)((uint64_t)x >> 32), e);
        return (int64_t)(((uint64_t)hi32 << 32) | lo32);
    };
    // Streamed tiles: for every visiting query block, every query head of
    // the group, its non-skipped query tiles.
    struct Cursor {
        int e, h, qt, lo, hi;
        int64_t qp;  // position of the query block's row 0
        // Byte addresses of the tile's first q row, dout row and lse2 entry;
        // moved by a constant per tile within a (block, head) run.
        const char *qb, *gb, *lb;
    };
    const int hq0 = kvh * a.group;
    auto set_ptrs = [&](Cursor& c) __attribute__((always_inline)) {
        const int hq = hq0 + c.h;
        const int64_t u0 = (int64_t)c.qt * BW_T;
        const int64_t row0 = c.qp + u0 * ps;  // token of the tile's first row
        c.qb = (const char*)((const bf16*)a.q + row0 * a.q_st + hq * a.q_sh);
        c.gb = (const char*)((const bf16*)a.dout + row0 * a.do_st + hq * a.do_sh);
        const int64_t qloc = ps == 1 ? c.qp : c.qp * B;  // block-local index of row 0 (striped: block = qp)
        c.lb = (const char*)(a.Lse2 + hq * a.T + qloc + u0);
    };
    const int64_t q_ts = BW_T * ps * a.q_st * 2, g_ts = BW_T * ps * a.do_st * 2, l_ts = BW_T * 4;
    auto enter = [&](Cursor& c, int e) __attribute__((always_inline)) {
        c.e = e;
        c.h = 0;
        c.qp = rl64(tb_qp, e);
        c.lo = rl32(tb_lo, e);
        c.hi = rl32(tb_hi, e);
        c.qt = c.lo;
    };
    // The next tile after c (c unchanged when there is none).
    auto cur_next = [&](Cursor& c) __attribute__((always_inline)) {
        Cursor n = c;
        n.qt++;
        if (n.qt <= n.hi) {  // the next tile of the same block and head
            n.qb += q_ts;
            n.gb += g_ts;
            n.lb += l_ts;
            c = n;
            return;
        }
        while (n.qt > n.hi) {
            if (n.h + 1 < a.group && n.lo <= n.hi) {
                n.h++;
                n.qt = n.lo;
            } else if (n.e + 1 < w.count) {
                enter(n, n.e + 1);
            } else {
                return;
            }
        }
        set_ptrs(n);
        c = n;
    };
    int nT = 0;
    for (int e = 0; e < w.count; e++) {
        const int lo = rl32(tb_lo, e), hi = rl32(tb_hi, e);
        if (hi >= lo) nT += a.group * (hi - lo + 1);
    }

    // This key's allowed query rows of the block at qp: local indices [u_lo, u_hi).
    // A query must not precede the key: u ps + qp >= wk ps + pos0, that is
    // u >= wk + ceil((pos0 - qp) / ps), where the last term is per block (both
    // row-0 positions lie below ps when striped) and computed in scalar code.
    int u_lo = 0, u_hi = 0;
    auto key_bounds = [&](int64_t qp) __attribute__((always_inline)) {
        u_lo = 0;
        u_hi = key_ok ? (int)B : 0;
        if (a.mask != kMaskNone) {
            const int dd = (int)(w.pos0 - qp);
            const int shift = ps == 1 ? dd : (dd > 0 ? 1 : 0);  // ceil(dd / ps), |dd| < ps when striped
            const int lo = wk + shift;
            u_lo = lo < 0 ? 0 : lo;
            if (a.mask == kMaskDoc && de_key - (int)qp < u_hi) u_hi = de_key - (int)qp;
        }
    };

    // Load offsets: q / dout chunks (NQ loads each), and the lse2 / D rows
    // (lanes 0..15: lse2 rows 4 l .. 4 l + 3; lanes 16..31: D rows; lanes
    // 32..63 repeat lanes 0..31), the same for every wave.
    const uint32_t q_rs = (uint32_t)(ps * a.q_st * 2), g_rs = (uint32_t)(ps * a.do_st * 2);
    const int last_full = BW_T - 1, last_ragged = (int)((B - 1) % BW_T);
    const int ragged_qt = B % BW_T ? nqt - 1 : -1;
    // Offsets of a full tile stay in registers; a ragged tile's are computed
    // when it is issued, and selected without a branch around the loads.
    uint32_t off_q[NQ], off_g[NQ], off_l[1];
#pragma unroll
    for (int i = 0; i < NQ; i++) {
        off_q[i] = chunk_offset<D>(lane, wave * NQ + i, q_rs, last_full);
        off_g[i] = chunk_offset<D>(lane, wave * NQ + i, g_rs, last_full);
    }
    {
        const int l32 = lane & 31;
        // Lse2 and Dsum sit in one allocation, Dsum a fixed number of floats after Lse2.
        const int64_t dd = a.Dsum - a.Lse2;
        off_l[0] = (uint32_t)(4 * (l32 < 16 ? 4 * l32 : dd + 4 * (l32 - 16)));
    }
    // Loads of one tile into stage sx: q, dout, then the lse2 / D block.
    auto issue = [&](int sx, const Cursor& c) __attribute__((always_inline)) {
        const char *qb = c.qb, *gb = c.gb, *lb = c.lb;
        const bool rag = c.qt == ragged_qt;
        const uint32_t l_st = lds_addr(st) + (uint32_t)(2 * SE) * (uint32_t)sx;
#pragma unroll
        for (int i = 0; i < NQ; i++) {
            const uint32_t oq = rag ? chunk_offset<D>(lane, wave * NQ + i, q_rs, last_ragged) : off_q[i];
            dma16(l_st + 1024u * (uint32_t)(wave * NQ + i), qb, oq);
        }
#pragma unroll
        for (int i = 0; i < NQ; i++) {
            const uint32_t og = rag ? chunk_offset<D>(lane, wave * NQ + i, g_rs, last_ragged) : off_g[i];
            dma16(l_st + 2u * TE + 1024u * (uint32_t)(wave * NQ + i), gb, og);
        }
        dma16(l_st + 4u * TE, lb, off_l[0]);
    };

    int cc_flo = 0, cc_fhi = -1;  // fully visible tiles of the dV wave's current block
    // Software pipeline with one workgroup barrier per iteration.  Iteration
    // j (j = 0 .. nT) reads query tiles j and j - 1 from two of the three
    // stages while the third receives tile j + 1:
    //   dV wave:  dv^T += dout_{j-1}^T P_{j-1};  S_j = q_j K^T;  P_j (to LDS, kept as bf16)
    //   dK wave:  dP_{j-1} = dout_{j-1} V^T;  dS = P_{j-1} (dP - D), P from LDS;  dk^T += q_{j-1}^T dS
    // The two waves of a 32-key group share a SIMD and order their matrix
    // and vector work oppositely, so that one's exp (or dS) arithmetic runs
    // beside the other's matrix products; P crosses the barrier between
    // them, never inside an iteration.  Register i of S / dP / P holds tile
    // row 32 sb + 8 (i/4) + 4 half + i%4.  x[sb] holds S or dP of half sb,
    // then P or dS as bf16 operands (first 8 registers).
    f32x16 x[2];
    auto b16 = [&](int sb, int h) __attribute__((always_inline)) {
        return __builtin_bit_cast(bf16x8, f32x4{x[sb][4 * h], x[sb][4 * h + 1], x[sb][4 * h + 2], x[sb][4 * h + 3]});
    };
    auto set_b16 = [&](int sb, int h, bf16x8 v) __attribute__((always_inline)) {
        const f32x4 y = __builtin_bit_cast(f32x4, v);
#pragma unroll
        for (int e = 0; e < 4; e++) x[sb][4 * h + e] = y[e];
    };
    const bool is_dv = __builtin_amdgcn_readfirstlane(role) == 0;
    constexpr int NR = 2 * (D / 16), KLA = kla<D>();  // instructions per run (both halves), operands read KLA ahead
    // S = q K^T (dV wave, t = q tile) or dP = dout V^T (dK wave, t = dout tile), both halves.
    auto row_set = [&](const bf16* t) __attribute__((always_inline)) {
        bf16x8 ring[KLA];
#pragma unroll
        for (int n = 0; n < KLA; n++) ring[n] = ops.row(t, n / (D / 16), n % (D / 16));
        x[0] = x[1] = f32x16{};
#pragma unroll
        for (int n = 0; n < NR; n++) {
            const bf16x8 fr = ring[n % KLA];
            if (n + KLA < NR) ring[n % KLA] = ops.row(t, (n + KLA) / (D / 16), (n + KLA) % (D / 16));
            x[n / (D / 16)] = mfma<E>(fr, opf[n % (D / 16)], x[n / (D / 16)]);
            __builtin_amdgcn_sched_barrier(0);  // keeps each read KLA instructions ahead of its use
        }
    };
    // dv^T += dout^T P (dV wave, t = dout tile) or dk^T += q^T dS (dK wave, t = q tile).
    // Instruction n: half sb = n / (D/16), block db = (n / 2) % (D/32), 16-row chunk h = n % 2.
    auto tr_set = [&](const bf16* t) __attribute__((always_inline)) {
        auto rd = [&](int n) __attribute__((always_inline)) {
            return ops.tr(t, 2 * (n / (D / 16)) + n % 2, (n / 2) % (D / 32));
        };
        bf16x8 ring[KLA];
#pragma unroll
        for (int n = 0; n < KLA; n++) ring[n] = rd(n);
#pragma unroll
        for (int n = 0; n < NR; n++) {
            const bf16x8 fr = ring[n % KLA];
            if (n + KLA < NR) ring[n % KLA] = rd(n + KLA);
            const int db = (n / 2) % (D / 32);
            acc[db] = mfma<E>(fr, b16(n / (D / 16), n % 2), acc[db]);
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    // P of the dV wave's tile (a masked row's exponent becomes -inf), to LDS
    // at pw and kept as bf16 operands.
    auto p_step = [&](const float* lw, int64_t u0, bf16x8* pw, auto full_t) __attribute__((always_inline)) {
        constexpr bool FULL = decltype(full_t)::value;
        const int x_lo = u_lo - (int)u0 - 4 * half, x_hi = u_hi - (int)u0 - 4 * half;
        // every LDS input first, in one batch (read one by one next to their
        // uses, each would wait out the whole LDS latency in turn)
        f32x4 lr[2][4];
#pragma unroll
        for (int sb = 0; sb < 2; sb++)
#pragma unroll
            for (int g4 = 0; g4 < 4; g4++) lr[sb][g4] = *(const f32x4*)(lw + 32 * sb + 8 * g4 + 4 * half);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int sb = 0; sb < 2; sb++) {
            f32x16 pv;
#pragma unroll
            for (int g4 = 0; g4 < 4; g4++) {
                const f32x4 l4 = lr[sb][g4];
#pragma unroll
                for (int r = 0; r < 4; r++) {
                    const int i = 4 * g4 + r, xr = 32 * sb + 8 * g4 + r;
                    float arg = fmaf(x[sb][i], a.c2, -l4[r]);
                    if (!FULL) arg = ((xr >= x_lo) & (xr < x_hi)) ? arg : -INFINITY;
                    pv[i] = __builtin_amdgcn_exp2f(arg);
                }
            }
            bf16x8 b0, b1;
            acc_to_b<E>(pv, b0, b1);
            pw[(2 * sb) * 64 + lane] = b0;
            pw[(2 * sb + 1) * 64 + lane] = b1;
            set_b16(sb, 0, b0);
            set_b16(sb, 1, b1);
        }
    };
    // dS = P (dP - D) of the dK wave's tile, P from pr; a masked row has
    // P = 0 and a finite D (rows past a block read the next rows or zeroed
    // padding).
    auto ds_step = [&](const float* lw, const bf16x8* pr) __attribute__((always_inline)) {
        // every LDS input first, in one batch (as in p_step)
        bf16x8 pp[2][2];
        f32x4 dr[2][4];
#pragma unroll
        for (int sb = 0; sb < 2; sb++) {
#pragma unroll
            for (int h = 0; h < 2; h++) pp[sb][h] = pr[(2 * sb + h) * 64 + lane];
#pragma unroll
            for (int g4 = 0; g4 < 4; g4++) dr[sb][g4] = *(const f32x4*)(lw + 64 + 32 * sb + 8 * g4 + 4 * half);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int sb = 0; sb < 2; sb++) {
            const bf16x8 p0 = pp[sb][0], p1 = pp[sb][1];
            f32x16 dsv;
#pragma unroll
            for (int g4 = 0; g4 < 4; g4++) {
                const f32x4 d4 = dr[sb][g4];
#pragma unroll
                for (int r = 0; r < 4; r++) {
                    const int i = 4 * g4 + r;
                    const float pi = from16<E>(i < 8 ? p0[i] : p1[i - 8]);
                    dsv[i] = pi * (x[sb][i] - d4[r]);
                }
            }
            bf16x8 e0, e1;
            acc_to_b<E>(dsv, e0, e1);
            set_b16(sb, 0, e0);
            set_b16(sb, 1, e1);
        }
    };

    Cursor cl{0, 0, 0, 0, -1, 0};
    if (w.count > 0) {
        enter(cl, 0);
        if (cl.hi < cl.lo) cur_next(cl);  // empty first block: step onto the first real tile
        set_ptrs(cl);
    }
    Cursor cc = cl;  // the dV wave's tile
    auto enter_block = [&](const Cursor& c) __attribute__((always_inline)) {
        key_bounds(c.qp);
        cc_flo = rl32(tb_flo, c.e);
        cc_fhi = rl32(tb_fhi, c.e);
    };
    if (nT > 0) {
        enter_block(cc);
        issue(0, cl);
        wait_loads_but<0>();
        phase_barrier();
        int s_cur = 0;  // stage of tile j
        for (int j = 0; j <= nT; j++) {
            const int s_prv = s_cur == 0 ? 2 : s_cur - 1, s_nxt = s_cur == 2 ? 0 : s_cur + 1;
            if (j + 1 < nT) {
                cur_next(cl);
                issue(s_nxt, cl);
            }
            const bf16* const t_cur = st + s_cur * SE;
            const bf16* const t_prv = st + s_prv * SE;
            if (is_dv && j >= 1) tr_set(t_prv + TE);  // dv += dout_{j-1}^T P_{j-1}
            if (is_dv ? j < nT : j >= 1) {
                row_set(is_dv ? t_cur : t_prv + TE);
                if (is_dv) {
                    const int64_t u0 = (int64_t)cc.qt * BW_T;
                    const bool full = cc.qt != ragged_qt && cc.qt >= cc_flo && cc.qt <= cc_fhi;
                    bf16x8* const pw = &p_lds[j & 1][kw][0][0][0];
                    const float* const lw = (const float*)(t_cur + 2 * TE);
                    if (__builtin_amdgcn_readfirstlane((int)full)) p_step(lw, u0, pw, std::true_type{});
                    else p_step(lw, u0, pw, std::false_type{});
                } else {
                    ds_step((const float*)(t_prv + 2 * TE), &p_lds[(j - 1) & 1][kw][0][0][0]);
                }
            }
            if (!is_dv && j >= 1) tr_set(t_prv);  // dk += q_{j-1}^T dS
            if (j + 1 < nT) {
                const int e_was = cc.e;
                cur_next(cc);
                if (cc.e != e_was) enter_block(cc);
            }
            wait_loads_but<0>();  // this wave's loads of tile j + 1
            phase_barrier();      // ... and every wave's; P_j is in LDS
            s_cur = s_nxt;
        }
    }

    if (!key_ok) return;
    // A padded key gets exact zeros.  Every other key's sums above never
    // involve a padded key (P comes from the forward's lse, D from its out).
    const bool padded = a.key_valid && !a.key_valid[p_key];
    const float mul = role ? a.scale : 1.f;
    char* ob = (char*)(role ? a.dk : a.dv);
    const int64_t oe = (p_key * a.Hkv + kvh) * D + 4 * half;
#pragma unroll
    for (int db = 0; db < D / 32; db++)
#pragma unroll
        for (int g = 0; g < 4; g++) {
            const int64_t e = oe + 32 * db + 8 * g;
            float x0 = acc[db][4 * g] * mul, x1 = acc[db][4 * g + 1] * mul;
            float x2 = acc[db][4 * g + 2] * mul, x3 = acc[db][4 * g + 3] * mul;
            if (padded) x0 = x1 = x2 = x3 = 0.f;
            if (a.grad16) *(bf16x4*)(ob + 2 * e) = bf16x4{to16<E>(x0), to16<E>(x1), to16<E>(x2), to16<E>(x3)};
            else *(f32x4*)(ob + 4 * e) = f32x4{x0, x1, x2, x3};
        }
    };  // run_item

    // One workgroup per compute unit takes items from the queue of its XCD
    // (numbers = that queue index mod 8, in order), then from the other
    // queues: see the forward's ring kernel.  Each fetch tries every queue at
    // most once, and an empty queue is not tried again, so the loop ends for
    // every workgroup once all queues are drained.
    for (;;) {
        __syncthreads();
        if (threadIdx.x == 0) {
            int it = -1;
            for (int k = 0; k < 8 && it < 0; k++) {
                const int y = (own_q + k) & 7;
                if ((q_done >> y) & 1u) continue;
                const int len = y < n_items ? (n_items - y + 7) / 8 : 0;
                const unsigned i = atomicAdd(&a.wq[8 + y], 1u);
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

template <typename E>
hipError_t launch_backward16(const BwdArgs& a, hipStream_t stream) {
    if (a.T > 0) {
        const int64_t threads = (int64_t)a.T * a.Hq * (a.d / 8);
        const int blocks = (int)((threads + 255) / 256 < 8192 ? (threads + 255) / 256 : 8192);
        bwd_prep_kernel<E><<<blocks, 256, 0, stream>>>(a);
    }
    // one workgroup per compute unit (fewer when there are fewer items)
    const int64_t ndq_items = (int64_t)a.n_works * a.Hq * a.n_qtiles;
    const int64_t ndk_items = (int64_t)a.n_rworks * a.Hkv * a.n_ktiles;
    if ((ndq_items > 0 || ndk_items > 0) && !a.wq) return hipErrorInvalidValue;
    if (ndq_items > INT32_MAX || ndk_items > INT32_MAX) return hipErrorInvalidValue;
    int n_cu = 0;
    hipError_t e = cu_count(&n_cu);
    if (e != hipSuccess) return e;
    const int64_t ndq = ndq_items < n_cu ? ndq_items : n_cu;
    const int64_t ndk = ndk_items < n_cu ? ndk_items : n_cu;
    if (a.d != 128 && a.d != 64) return hipErrorInvalidValue;
    if (ndq > 0) {
        // KP: with a key-padding mask (the unmasked kernel carries none of its code);
        // QM: the tile-major item order of striped layouts
        const int v = (a.kbits ? 2 : 0) + (a.qt_major ? 1 : 0);
        auto dq = [&](auto d_t) {
            constexpr int Dc = decltype(d_t)::value;
            switch (v) {
                case 0: bwd_dq_kernel<E, Dc, false, false><<<(unsigned)ndq, DQ_THREADS, 0, stream>>>(a); break;
                case 1: bwd_dq_kernel<E, Dc, false, true><<<(unsigned)ndq, DQ_THREADS, 0, stream>>>(a); break;
                case 2: bwd_dq_kernel<E, Dc, true, false><<<(unsigned)ndq, DQ_THREADS, 0, stream>>>(a); break;
                default: bwd_dq_kernel<E, Dc, true, true><<<(unsigned)ndq, DQ_THREADS, 0, stream>>>(a); break;
            }
        };
        if (a.d == 128) dq(ic<128>{});
        else dq(ic<64>{});
    }
    if (ndk > 0) {
        auto dkdv = [&](auto d_t) {
            constexpr int Dc = decltype(d_t)::value;
            if (a.qt_major) bwd_dkdv_kernel<E, Dc, true><<<(unsigned)ndk, KV_THREADS, 0, stream>>>(a);
            else bwd_dkdv_kernel<E, Dc, false><<<(unsigned)ndk, KV_THREADS, 0, stream>>>(a);
        };
        if (a.d == 128) dkdv(ic<128>{});
        else dkdv(ic<64>{});
    }
    return hipGetLastError();
}

}  // namespace

int bwd_tile_q() { return BW_TQ; }
int bwd_tile_k() { return BW_TK; }

hipError_t launch_backward(const BwdArgs& a, hipStream_t stream) {
    return a.f16 ? launch_backward16<f16>(a, stream) : launch_backward16<bf16>(a, stream);
}

}  // namespace ra
