// C ABI entry points: argument checks, the one-GPU ring driver, optional
// side-stream prefetch of the next key/value blocks, and tallies.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstring>
#include <memory>
#include <mutex>
#include <vector>

#include "bwd_kernels.h"
#include "kernels.h"
#include "plan.h"
#include "ring_attn.h"

namespace ra {
namespace {

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// 16-bit element types (bf16, fp16) run on the matrix-core kernels.
bool is16(int t) { return t == RA_BF16 || t == RA_F16; }

size_t elem_size(ra_dtype t) { return is16(t) ? 2 : 4; }

bool valid_dtype(int t) { return t == RA_F32 || is16(t); }

bool tensor_ok(const ra_tensor* x) {
    return x && (x->data || x->n_tok == 0) && valid_dtype(x->dtype) && x->n_tok >= 0 && x->n_head >= 1 && x->head_dim >= 1 &&
           x->stride_tok >= 0 && x->stride_head >= 0;
}

// Which kernel serves (dtype, head_dim); RA_OK when one does.
ra_status kernel_for(ra_dtype dt, int64_t d, int* tq, int* tk) {
    if (is16(dt)) {
        if (d != 64 && d != 128) return RA_E_UNSUPPORTED;
        *tq = kBf16TileQ;
        *tk = kBf16TileK;
        return RA_OK;
    }
    if (dt == RA_F32) {
        if (d < 1 || d > 128) return RA_E_UNSUPPORTED;
        *tq = kF32TileQ;
        *tk = kF32TileK;
        return RA_OK;
    }
    return RA_E_ARG;
}

// The matrix-core kernel reads 16-byte vectors: base pointers and strides
// must keep every row of 8 16-bit elements aligned.
bool bf16_aligned(const ra_tensor* x) {
    return ((uintptr_t)x->data % 16 == 0) && x->stride_tok % 8 == 0 && x->stride_head % 8 == 0;
}

// The matrix-core kernel addresses a 64-row key tile with 32-bit byte offsets
// from the tile's first row.
bool bf16_tile_addressable(int64_t row_stride_elems) {
    return row_stride_elems >= 0 && row_stride_elems * 2 * kBf16TileK < ((int64_t)1 << 31);
}

bool scale_ok(float s) { return std::isfinite(s) && s > 0.f; }

// 32-bit words of a block's key-padding bits: whole 64-key tiles.
int64_t key_words(int64_t B) { return 2 * ((B + 63) / 64); }

hipError_t launch(const StepArgs& a, ra_dtype dt, hipStream_t st) {
    return is16(dt) ? launch_step_bf16(a, st) : launch_step_f32(a, st);
}

// Side stream + events used by the prefetch path, created once per device.
// A prefetch forward holds `enqueue` while it records and waits on them, so
// that calls from several host threads cannot interleave their event pairs.
struct PrefetchCtx {
    hipStream_t copy = nullptr;
    hipEvent_t copied[2] = {nullptr, nullptr};
    hipEvent_t consumed[2] = {nullptr, nullptr};
    std::mutex enqueue;
};

// Test hook of the prefetch path (0 = off): a bounded wait enqueued before
// every step's copies on the copy stream, and before every step's compute
// on the caller's stream, so that a test can make either side run late.
std::atomic<uint32_t> g_copy_delay_us{0}, g_compute_delay_us{0};
constexpr uint32_t kMaxDelayUs = 100000;

hipError_t prefetch_ctx(PrefetchCtx** out) {
    static std::mutex mu;
    static std::vector<std::unique_ptr<PrefetchCtx>> ctx;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    std::lock_guard<std::mutex> g(mu);
    if ((int)ctx.size() <= dev) ctx.resize(dev + 1);
    if (!ctx[dev]) ctx[dev].reset(new PrefetchCtx);
    PrefetchCtx& c = *ctx[dev];
    if (!c.copy) {
        if ((e = hipStreamCreateWithFlags(&c.copy, hipStreamNonBlocking)) != hipSuccess) return e;
        for (int b = 0; b < 2; b++) {
            if ((e = hipEventCreateWithFlags(&c.copied[b], hipEventDisableTiming)) != hipSuccess) return e;
            if ((e = hipEventCreateWithFlags(&c.consumed[b], hipEventDisableTiming)) != hipSuccess) return e;
        }
    }
    *out = &c;
    return hipSuccess;
}

// Host-to-device copies of the per-call tables (chain tables, document
// boundaries).  They are gathered into one pinned host buffer, taken from a
// per-device ring of kStageSlots, and copied with plain DMA transfers on the
// caller's stream; a slot is refilled only after the event recorded behind
// its last copies has completed.  The host thus hands the copies to the
// stream without the runtime's pageable staging, and may run up to
// kStageSlots calls ahead of the GPU.  With pinned = false (callers that must
// not allocate) the same copies go straight from the callers' host memory.
constexpr int kStageSlots = 8;

struct StageDev {
    std::mutex mu;
    char* buf[kStageSlots] = {};
    size_t cap[kStageSlots] = {};
    hipEvent_t done[kStageSlots] = {};
    bool recorded[kStageSlots] = {};
    unsigned next = 0;
};

class HostStager {
  public:
    explicit HostStager(bool pinned) : pinned_(pinned) {}
    // Queues n bytes at src for dst; src must stay valid until flush().
    void add(void* dst, const void* src, size_t n) {
        if (n == 0) return;
        recs_.push_back({dst, src, n, bytes_});
        bytes_ += align_up(n);
    }
    hipError_t flush(hipStream_t st) {
        if (recs_.empty()) return hipSuccess;
        hipError_t e;
        if (!pinned_) {
            for (const Rec& r : recs_)
                if ((e = hipMemcpyAsync(r.dst, r.src, r.n, hipMemcpyHostToDevice, st)) != hipSuccess) return e;
            recs_.clear();
            return hipSuccess;
        }
        StageDev* sd = nullptr;
        if ((e = stage_dev(&sd)) != hipSuccess) return e;
        std::lock_guard<std::mutex> g(sd->mu);
        const int slot = (int)(sd->next++ % kStageSlots);
        if (!sd->done[slot] && (e = hipEventCreateWithFlags(&sd->done[slot], hipEventDisableTiming)) != hipSuccess)
            return e;
        if (sd->recorded[slot] && (e = hipEventSynchronize(sd->done[slot])) != hipSuccess)
            return e;  // the slot's last copies have landed
        if (sd->cap[slot] < bytes_) {
            if (sd->buf[slot] && (e = hipHostFree(sd->buf[slot])) != hipSuccess) return e;
            sd->buf[slot] = nullptr;
            sd->cap[slot] = 0;
            const size_t cap = std::max<size_t>(bytes_, (size_t)64 << 10);
            if ((e = hipHostMalloc((void**)&sd->buf[slot], cap, hipHostMallocDefault)) != hipSuccess) return e;
            sd->cap[slot] = cap;
        }
        for (const Rec& r : recs_) std::memcpy(sd->buf[slot] + r.off, r.src, r.n);
        for (const Rec& r : recs_)
            if ((e = hipMemcpyAsync(r.dst, sd->buf[slot] + r.off, r.n, hipMemcpyHostToDevice, st)) != hipSuccess)
                return e;
        recs_.clear();
        if ((e = hipEventRecord(sd->done[slot], st)) != hipSuccess) return e;
        sd->recorded[slot] = true;
        return hipSuccess;
    }

  private:
    struct Rec {
        void* dst;
        const void* src;
        size_t n, off;
    };
    static hipError_t stage_dev(StageDev** out) {
        static std::mutex mu;
        static std::vector<std::unique_ptr<StageDev>> devs;  // kept until the process ends
        int dev = 0;
        hipError_t e = hipGetDevice(&dev);
        if (e != hipSuccess) return e;
        std::lock_guard<std::mutex> g(mu);
        if ((int)devs.size() <= dev) devs.resize(dev + 1);
        if (!devs[dev]) devs[dev].reset(new StageDev);
        *out = devs[dev].get();
        return hipSuccess;
    }
    bool pinned_;
    std::vector<Rec> recs_;
    size_t bytes_ = 0;
};

// Workspace of ring_attn_forward_noalloc: a fixed array in device memory,
// one copy per GPU, held until the process ends.  Host code never passes the
// array's name to a kernel or copy (on the host it is only a stand-in): each
// device's address comes from hipGetSymbolAddress, taken once per device with
// that device current.
constexpr size_t kScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) char scratch[kScratchBytes];

hipError_t scratch_address(void** out) {
    static std::mutex mu;
    static std::vector<void*> addr;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    std::lock_guard<std::mutex> g(mu);
    if ((int)addr.size() <= dev) addr.resize(dev + 1, nullptr);
    if (!addr[dev]) {
        void* p = nullptr;
        if ((e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch))) != hipSuccess) return e;
        addr[dev] = p;
    }
    *out = addr[dev];
    return hipSuccess;
}

struct Workspace {
    unsigned long long* counters = nullptr;  // 4 x u64
    int32_t* cu = nullptr;
    float* O = nullptr;
    float* m = nullptr;
    float* l = nullptr;
    char* vt = nullptr;     // packed V^T of all blocks (16-bit path): [N][Hkv][d][Bp]
    RingWork* works = nullptr;    // one-launch ring forward (16-bit): N works
    unsigned* wq = nullptr;       //   its 8 work-queue counters
    RingEntry* entries = nullptr; //   and up to N x N chain entries
    uint32_t* kbits = nullptr;    // key-padding bits of every block: [N][key_words(B)]
    char* kv = nullptr;     // prefetch double buffers: K [2][N][B][Hkv][d], then V (f32) or V^T (16-bit)
    size_t k_half = 0;      // bytes of the K double buffer
    size_t total = 0;
};

// Whether a forward with these shapes may take the per-step path, whose
// state (unnormalised O, m, l of every row) lives in the workspace between
// steps: fp32 inputs, the side-stream prefetch, or a ring the one-launch
// kernel cannot hold (longer chains than its table, too many workgroups).
// Otherwise the one-launch ring runs and keeps the state in registers.
bool fwd_needs_state(int64_t T, int64_t N, int64_t Hq, int64_t d, ra_dtype dt, bool prefetch) {
    if (!is16(dt) || prefetch || N > kMaxRingChain) return true;
    int tq = 0, tk = 0;
    if (kernel_for(dt, d, &tq, &tk) != RA_OK || tq <= 0) return true;
    const int64_t n_qtiles = (T / N + tq - 1) / tq;
    return n_qtiles * Hq * N > INT32_MAX;
}

Workspace carve(void* base, int64_t T, int64_t N, int64_t Hq, int64_t Hkv, int64_t d, int64_t n_docs, ra_dtype dt,
                bool prefetch) {
    Workspace w;
    size_t off = 0;
    char* b = (char*)base;
    auto take = [&](size_t bytes) {
        char* p = b ? b + off : nullptr;
        off += align_up(bytes);
        return p;
    };
    const int64_t B = N > 0 ? T / N : 0;
    const size_t es = elem_size(dt);
    const size_t vt_bytes = is16(dt) ? (size_t)N * Hkv * d * vt_padded_keys(B) * 2 : 0;
    w.counters = (unsigned long long*)take(4 * sizeof(unsigned long long));
    w.cu = (int32_t*)take(sizeof(int32_t) * (size_t)(n_docs + 1));
    if (N > 0 && fwd_needs_state(T, N, Hq, d, dt, prefetch)) {
        w.O = (float*)take(sizeof(float) * (size_t)(T * Hq * d));
        w.m = (float*)take(sizeof(float) * (size_t)(T * Hq));
        w.l = (float*)take(sizeof(float) * (size_t)(T * Hq));
    }
    w.kbits = (uint32_t*)take(sizeof(uint32_t) * (size_t)(N * key_words(B)));
    if (is16(dt)) {
        w.vt = take(vt_bytes);
        w.works = (RingWork*)take(sizeof(RingWork) * (size_t)N);
        w.wq = (unsigned*)take(8 * sizeof(unsigned));
        w.entries = (RingEntry*)take(sizeof(RingEntry) * (size_t)N * (size_t)N);
    }
    if (prefetch) {
        w.k_half = 2 * (size_t)T * Hkv * d * es;
        const size_t v_half = is16(dt) ? 2 * vt_bytes : w.k_half;
        w.kv = take(w.k_half + v_half);
    }
    w.total = off;
    return w;
}

struct BwdWorkspace {
    float* Lse2 = nullptr;          // [Hq, T] + kBwdPad floats of padding (tiles may read past a block)
    float* Dsum = nullptr;          // [Hq, T] + kBwdPad, right after Lse2 in the same allocation
    int32_t* cu = nullptr;
    BwdWork* works = nullptr;       // N
    int64_t* partners = nullptr;    // N x N
    BwdWork* rworks = nullptr;      // N
    int64_t* rpartners = nullptr;   // N x N
    uint32_t* kbits = nullptr;      // key-padding bits: [N][key_words(B)]
    unsigned* wq = nullptr;         // 16 work-queue counters of the dq and dk/dv kernels
    size_t total = 0;
};

BwdWorkspace carve_bwd(void* base, int64_t T, int64_t N, int64_t Hq, int64_t n_docs) {
    BwdWorkspace w;
    size_t off = 0;
    char* b = (char*)base;
    auto take = [&](size_t bytes) {
        char* p = b ? b + off : nullptr;
        off += align_up(bytes);
        return p;
    };
    const size_t plane = align_up(sizeof(float) * (size_t)(T * Hq + kBwdPad));
    w.Lse2 = (float*)take(2 * plane);
    w.Dsum = w.Lse2 ? (float*)((char*)w.Lse2 + plane) : nullptr;
    w.cu = (int32_t*)take(sizeof(int32_t) * (size_t)(n_docs + 1));
    w.works = (BwdWork*)take(sizeof(BwdWork) * (size_t)N);
    w.partners = (int64_t*)take(sizeof(int64_t) * (size_t)(N * N));
    w.rworks = (BwdWork*)take(sizeof(BwdWork) * (size_t)N);
    w.rpartners = (int64_t*)take(sizeof(int64_t) * (size_t)(N * N));
    w.kbits = (uint32_t*)take(sizeof(uint32_t) * (size_t)(N * key_words(N > 0 ? T / N : 0)));
    w.wq = (unsigned*)take(16 * sizeof(unsigned));
    w.total = off;
    return w;
}

}  // namespace
}  // namespace ra

using namespace ra;

extern "C" {

const char* ring_attn_status_string(ra_status s) {
    switch (s) {
        case RA_OK: return "ok";
        case RA_E_ARG: return "invalid argument";
        case RA_E_UNSUPPORTED: return "unsupported dtype / head_dim / mask combination";
        case RA_E_HIP: return "HIP runtime error";
        case RA_E_WORKSPACE: return "workspace missing or too small";
        case RA_E_TOO_LARGE: return "shapes need more than the fixed scratch of ring_attn_forward_noalloc";
    }
    return "unknown status";
}

ra_status ring_attn_pack_key_mask(const uint8_t* key_valid, int64_t n_keys, int64_t stride, uint32_t* key_bits,
                                  void* stream) {
    if (!key_valid || !key_bits || n_keys < 0 || stride < 1 || (uintptr_t)key_bits % 8) return RA_E_ARG;
    if (launch_pack_key_bits(key_valid, stride, 1, n_keys, 0, key_words(n_keys), key_bits, (hipStream_t)stream) !=
        hipSuccess)
        return RA_E_HIP;
    return RA_OK;
}

ra_status ring_attn_tile_shape(ra_dtype dtype, int64_t head_dim, int32_t* tile_q, int32_t* tile_k) {
    if (!tile_q || !tile_k) return RA_E_ARG;
    int tq = 0, tk = 0;
    ra_status s = kernel_for(dtype, head_dim, &tq, &tk);
    if (s != RA_OK) return s;
    *tile_q = tq;
    *tile_k = tk;
    return RA_OK;
}

ra_status ring_attn_step(const ra_tensor* q_blk, const ra_tensor* k_blk, const ra_tensor* v_blk, float* O, float* m,
                         float* l, int first_step, float scale, ra_mask mask_mode, int64_t q_offset,
                         int64_t kv_offset, int64_t pos_stride, const int32_t* cu_seqlens, int32_t n_docs,
                         const uint32_t* key_bits, int64_t* stats_dev, void* stream) {
    if (!tensor_ok(q_blk) || !tensor_ok(k_blk) || !tensor_ok(v_blk)) return RA_E_ARG;
    if (q_blk->dtype != k_blk->dtype || q_blk->dtype != v_blk->dtype) return RA_E_ARG;
    const int64_t d = q_blk->head_dim;
    if (k_blk->head_dim != d || v_blk->head_dim != d) return RA_E_ARG;
    if (k_blk->n_tok != v_blk->n_tok || k_blk->n_head != v_blk->n_head) return RA_E_ARG;
    if (q_blk->n_head % k_blk->n_head) return RA_E_ARG;
    if ((!O || !m || !l) && q_blk->n_tok > 0) return RA_E_ARG;  // no state for an empty block
    if (!scale_ok(scale) || pos_stride < 1) return RA_E_ARG;
    if (mask_mode < RA_MASK_NONE || mask_mode > RA_MASK_DOC_CAUSAL) return RA_E_ARG;
    if (mask_mode == RA_MASK_DOC_CAUSAL && (!cu_seqlens || n_docs < 1)) return RA_E_ARG;
    if (mask_mode == RA_MASK_DOC_CAUSAL && pos_stride != 1) return RA_E_UNSUPPORTED;
    if ((uintptr_t)key_bits % 8) return RA_E_ARG;
    int tq = 0, tk = 0;
    ra_status ks = kernel_for(q_blk->dtype, d, &tq, &tk);
    if (ks != RA_OK) return ks;
    if (is16(q_blk->dtype) && (!bf16_aligned(q_blk) || !bf16_aligned(k_blk) || !bf16_aligned(v_blk) ||
                                    !bf16_tile_addressable(k_blk->stride_tok) ||
                                    !bf16_tile_addressable(v_blk->stride_tok)))
        return RA_E_UNSUPPORTED;
    const int64_t Bq = q_blk->n_tok, Hq = q_blk->n_head;
    const int64_t n_qtiles = (Bq + tq - 1) / tq;
    if (n_qtiles * Hq > INT32_MAX) return RA_E_UNSUPPORTED;
    if (Bq == 0) return RA_OK;

    StepArgs a;
    std::memset(&a, 0, sizeof a);
    a.q = q_blk->data;
    a.k = k_blk->data;
    a.v = v_blk->data;
    a.q_row_stride = q_blk->stride_tok;
    a.q_head_stride = q_blk->stride_head;
    a.k_row_stride = k_blk->stride_tok;
    a.k_head_stride = k_blk->stride_head;
    a.v_row_stride = v_blk->stride_tok;
    a.v_head_stride = v_blk->stride_head;
    a.Bq = Bq;
    a.Bk = k_blk->n_tok;
    a.pos_stride = pos_stride;
    a.Hq = (int32_t)Hq;
    a.group = (int32_t)(Hq / k_blk->n_head);
    a.d = (int32_t)d;
    a.f16 = q_blk->dtype == RA_F16;
    a.kbits = key_bits;
    a.mask = mask_mode;
    a.scale = scale;
    a.c2 = scale * 1.4426950408889634f;
    a.cu = cu_seqlens;
    a.n_docs = n_docs;
    a.stats = (unsigned long long*)stats_dev;
    a.n_qtiles = (int32_t)n_qtiles;
    a.n_pairs = 1;
    PairDesc& p = a.pairs[0];
    p.q_pos0 = q_offset;
    p.k_pos0 = kv_offset;
    p.O = O;
    p.m = m;
    p.l = l;
    p.load_state = first_step ? 0 : 1;
    p.finalize = 0;
    if (launch(a, q_blk->dtype, (hipStream_t)stream) != hipSuccess) return RA_E_HIP;
    return RA_OK;
}

ra_status ring_attn_finalize(const float* O, const float* m, const float* l, int64_t Hq, int64_t Bq, int64_t d,
                             void* out, ra_dtype out_dtype, int64_t out_stride_tok, int64_t out_stride_head,
                             float* lse, void* stream) {
    if (Hq < 1 || Bq < 0 || d < 1 || !valid_dtype(out_dtype)) return RA_E_ARG;
    if (out_stride_tok < 0 || out_stride_head < 0) return RA_E_ARG;
    if (Bq == 0) return RA_OK;  // an empty block: its pointers may be NULL
    if (!O || !m || !l || !out) return RA_E_ARG;
    if (launch_finalize(O, m, l, Hq, Bq, d, out, (int)out_dtype, out_stride_tok, out_stride_head, lse,
                        (hipStream_t)stream) != hipSuccess)
        return RA_E_HIP;
    return RA_OK;
}

ra_status ring_attn_merge(void* out_acc, float* lse_acc, const void* out_blk, const float* lse_blk,
                          ra_dtype dtype, int64_t Hq, int64_t rows, int64_t d, void* stream) {
    if (!valid_dtype(dtype) || Hq < 1 || rows < 0 || d < 1) return RA_E_ARG;
    if (rows == 0) return RA_OK;  // nothing to merge: the pointers may be NULL
    if (!out_acc || !lse_acc || !out_blk || !lse_blk) return RA_E_ARG;
    if (launch_merge(out_acc, lse_acc, out_blk, lse_blk, (int)dtype, Hq, rows, d, (hipStream_t)stream) !=
        hipSuccess)
        return RA_E_HIP;
    return RA_OK;
}

size_t ring_attn_forward_workspace_size(const ra_tensor* q, const ra_tensor* k, int32_t n_blocks, int32_t n_docs,
                                        int prefetch) {
    if (!q || !k || n_blocks < 1 || n_docs < 0 || !valid_dtype(q->dtype)) return 0;
    if (q->n_tok % n_blocks) return 0;
    return carve(nullptr, q->n_tok, n_blocks, q->n_head, k->n_head, q->head_dim, n_docs, q->dtype, prefetch != 0).total;
}

ra_status ring_attn_plan(int64_t T, int32_t n_blocks, ra_layout layout, ra_mask mask_mode, int32_t max_ring_passes,
                         const int32_t* cu_seqlens_host, int32_t n_docs, ra_dtype dtype, int64_t head_dim,
                         ra_stats* stats) {
    if (!stats || T < 0 || n_blocks < 1 || T % n_blocks || max_ring_passes < 1) return RA_E_ARG;
    if (layout != RA_LAYOUT_CONTIGUOUS && layout != RA_LAYOUT_STRIPED) return RA_E_ARG;
    if (mask_mode < RA_MASK_NONE || mask_mode > RA_MASK_DOC_CAUSAL) return RA_E_ARG;
    if (mask_mode == RA_MASK_DOC_CAUSAL) {
        if (!cu_seqlens_host || n_docs < 1 || cu_seqlens_host[0] != 0 || cu_seqlens_host[n_docs] != T)
            return RA_E_ARG;
        for (int32_t i = 0; i < n_docs; i++)
            if (cu_seqlens_host[i + 1] < cu_seqlens_host[i]) return RA_E_ARG;
        if (layout == RA_LAYOUT_STRIPED) return RA_E_UNSUPPORTED;
    }
    int tq = 0, tk = 0;
    ra_status ks = kernel_for(dtype, head_dim, &tq, &tk);
    if (ks != RA_OK) return ks;
    Ring r;
    r.T = T;
    r.N = n_blocks;
    r.B = T / n_blocks;
    r.layout = layout;
    r.mask = mask_mode;
    r.passes = std::min<int64_t>(max_ring_passes, n_blocks);
    r.cu = cu_seqlens_host;
    r.n_docs = n_docs;
    Plan p = make_plan(r, tq, tk);
    int64_t c[3];
    tile_tallies(r, tq, tk, c);
    stats->block_pairs_visited = p.visited;
    stats->block_pairs_skipped = p.skipped;
    stats->block_pairs_full = p.full;
    stats->block_pairs_partial = p.partial;
    stats->tiles_skipped = c[0];
    stats->tiles_full = c[1];
    stats->tiles_partial = c[2];
    stats->allowed_pairs = allowed_pairs(r);
    stats->tile_q = tq;
    stats->tile_k = tk;
    return RA_OK;
}

// The forward behind both entry points; pinned selects how the per-call
// tables travel to the device (see HostStager).
static ra_status forward_impl(const ra_tensor* q, const ra_tensor* k, const ra_tensor* v, void* out,
                              ra_dtype out_dtype, float* lse, int32_t n_blocks, ra_layout layout, ra_mask mask_mode,
                              int32_t max_ring_passes, const int32_t* cu_seqlens_host, int32_t n_docs,
                              const uint8_t* key_valid, float scale, int prefetch, void* workspace,
                              size_t workspace_bytes, ra_stats* stats, void* stream, bool pinned) {
    // ---- arguments ----
    if (!tensor_ok(q) || !tensor_ok(k) || !tensor_ok(v) || (!out && q->n_tok > 0)) return RA_E_ARG;
    if (q->dtype != k->dtype || q->dtype != v->dtype || !valid_dtype(out_dtype)) return RA_E_ARG;
    const int64_t T = q->n_tok, Hq = q->n_head, Hkv = k->n_head, d = q->head_dim;
    if (k->n_tok != T || v->n_tok != T || v->n_head != Hkv || k->head_dim != d || v->head_dim != d) return RA_E_ARG;
    if (Hq % Hkv) return RA_E_ARG;
    if (n_blocks < 1 || T % n_blocks || max_ring_passes < 1 || !scale_ok(scale)) return RA_E_ARG;
    if (layout != RA_LAYOUT_CONTIGUOUS && layout != RA_LAYOUT_STRIPED) return RA_E_ARG;
    if (mask_mode < RA_MASK_NONE || mask_mode > RA_MASK_DOC_CAUSAL) return RA_E_ARG;
    if (mask_mode == RA_MASK_DOC_CAUSAL) {
        if (!cu_seqlens_host || n_docs < 1 || cu_seqlens_host[0] != 0 || cu_seqlens_host[n_docs] != T)
            return RA_E_ARG;
        for (int32_t i = 0; i < n_docs; i++)
            if (cu_seqlens_host[i + 1] < cu_seqlens_host[i]) return RA_E_ARG;
        if (layout == RA_LAYOUT_STRIPED) return RA_E_UNSUPPORTED;
    } else {
        n_docs = 0;
    }
    if (is16(out_dtype) && out_dtype != q->dtype) return RA_E_UNSUPPORTED;
    int tq = 0, tk = 0;
    ra_status ks = kernel_for(q->dtype, d, &tq, &tk);
    if (ks != RA_OK) return ks;
    const int64_t row_mult = layout == RA_LAYOUT_STRIPED ? n_blocks : 1;
    if (is16(q->dtype) && (!bf16_aligned(q) || !bf16_aligned(k) || !bf16_aligned(v) ||
                                !bf16_tile_addressable(row_mult * k->stride_tok) ||
                                !bf16_tile_addressable(row_mult * v->stride_tok) ||
                                vt_padded_keys(T / n_blocks) * 2 * d >= ((int64_t)1 << 31)))  // V^T tile rows
        return RA_E_UNSUPPORTED;
    if (prefetch && (k->stride_head != d || v->stride_head != d)) return RA_E_UNSUPPORTED;
    if (is16(q->dtype) && (uintptr_t)out % 16) return RA_E_UNSUPPORTED;
    const int64_t N = n_blocks, B = T / N;
    const int64_t n_qtiles = (B + tq - 1) / tq;
    if (n_qtiles * Hq * kMaxPairs > INT32_MAX) return RA_E_UNSUPPORTED;
    if (T == 0) {  // an empty sequence: nothing to launch, no workspace needed
        if (stats) {
            std::memset(stats, 0, sizeof *stats);
            stats->tile_q = tq;
            stats->tile_k = tk;
        }
        return RA_OK;
    }
    Workspace ws = carve(workspace, T, n_blocks, Hq, Hkv, d, n_docs, q->dtype, prefetch != 0);
    if (!workspace || workspace_bytes < ws.total) return RA_E_WORKSPACE;
    if ((uintptr_t)workspace % kAlign) return RA_E_WORKSPACE;

    hipStream_t st = (hipStream_t)stream;
    Ring r;
    r.T = T;
    r.N = N;
    r.B = B;
    r.layout = layout;
    r.mask = mask_mode;
    r.passes = std::min<int64_t>(max_ring_passes, N);
    r.cu = cu_seqlens_host;
    r.n_docs = n_docs;
    const Plan plan = make_plan(r, tq, tk);
    // The one-launch ring serves hpi query heads of a kv head per work item
    // (the largest power of two <= 8 dividing the group), tq / hpi rows each;
    // its tiles, and so its tallies, are tq / hpi rows tall.
    int hpi = 1;
    if (is16(q->dtype))
        while (hpi < 8 && (Hq / Hkv) % (2 * hpi) == 0) hpi *= 2;
    const int tq_ring = tq / hpi;
    const int64_t n_qtiles_ring = (B + tq_ring - 1) / tq_ring;
    const Plan plan_ring = hpi > 1 ? make_plan(r, tq_ring, tk) : Plan{};
    const bool striped = layout == RA_LAYOUT_STRIPED;
    const int64_t out_tok = Hq * d;  // out is [T, Hq, d] contiguous

    PrefetchCtx* pf = nullptr;
    std::unique_lock<std::mutex> pf_lock;
    if (prefetch && r.passes > 1) {
        if (prefetch_ctx(&pf) != hipSuccess) return RA_E_HIP;
        pf_lock = std::unique_lock<std::mutex>(pf->enqueue);
    }

    // ---- enqueue ----
    if (stats && launch_fill_u64(ws.counters, 4, st) != hipSuccess) return RA_E_HIP;
    HostStager stage(pinned);  // flushed before the first kernel that reads a table
    if (n_docs > 0) stage.add(ws.cu, cu_seqlens_host, sizeof(int32_t) * (size_t)(n_docs + 1));
    const int64_t kbw = key_words(B);  // key-padding words per block; block j's at j * kbw
    if (key_valid && launch_pack_key_bits(key_valid, 1, N, B, striped, kbw, ws.kbits, st) != hipSuccess)
        return RA_E_HIP;

    StepArgs base;
    std::memset(&base, 0, sizeof base);
    base.Bq = B;
    base.Bk = B;
    base.pos_stride = striped ? N : 1;
    base.Hq = (int32_t)Hq;
    base.group = (int32_t)(Hq / Hkv);
    base.d = (int32_t)d;
    base.mask = mask_mode;
    base.scale = scale;
    base.c2 = scale * 1.4426950408889634f;
    base.cu = ws.cu;
    base.n_docs = n_docs;
    base.f16 = q->dtype == RA_F16;
    base.kbits = key_valid ? ws.kbits : nullptr;
    base.out16 = is16(out_dtype);
    base.out = out;
    base.out_row_stride = (striped ? N : 1) * out_tok;
    base.out_head_stride = d;
    base.lse = lse;
    base.lse_row_stride = striped ? N : 1;
    base.lse_head_stride = T;
    base.stats = stats ? ws.counters : nullptr;
    base.n_qtiles = (int32_t)n_qtiles;
    base.q = q->data;
    base.q_row_stride = (striped ? N : 1) * q->stride_tok;
    base.q_head_stride = q->stride_head;

    const size_t es = elem_size(q->dtype);
    const bool use_vt = is16(q->dtype);
    const int64_t Bp = vt_padded_keys(B);
    const int64_t vt_blk = Hkv * d * Bp;    // elements of one packed V^T block
    const int64_t blk_elems = B * Hkv * d;  // one contiguous prefetched K (or V) block
    auto k_slot = [&](int slot, int64_t i) { return ws.kv + ((size_t)slot * N + i) * blk_elems * es; };
    auto v_slot = [&](int slot, int64_t i) {
        return ws.kv + ws.k_half + ((size_t)slot * N + i) * (use_vt ? vt_blk * 2 : blk_elems * es);
    };
    auto row_off = [&](int64_t blk, int64_t stride_tok) { return striped ? blk * stride_tok : blk * B * stride_tok; };

    // ---- bf16 without the side-stream prefetch: the whole ring in one launch ----
    // Each device's visited (non-skipped) blocks in ring order form its
    // chain; one workgroup per (device, head, q-tile) runs the chain with
    // the state in registers and finalises at its end.
    std::vector<std::vector<int32_t>> chain;
    size_t longest = 0;
    if (use_vt && !pf) {
        chain.resize((size_t)N);
        for (int64_t s = 0; s < r.passes; s++)
            for (const StepPair& sp : plan.steps[s]) chain[sp.i].push_back(sp.j);
        for (const auto& c : chain) longest = std::max(longest, c.size());
    }
    const bool one_launch =
        use_vt && !pf && longest <= (size_t)kMaxRingChain && n_qtiles_ring * (Hq / hpi) * N <= INT32_MAX;
    // V^T in matrix-fragment order for the one-launch kernel, in rows for
    // the per-step kernel
    if (use_vt && launch_pack_vt(v->data, v->stride_tok, v->stride_head, N, B, striped, Hkv, d, one_launch, ws.vt,
                                 st) != hipSuccess)
        return RA_E_HIP;

    bool ring_done = false;
    if (one_launch) {
        // Every block of a chain is resident, and the online-softmax merge
        // gives the same sum in any order, so the chain takes the device's
        // own block last: under a causal mask that block is the partly
        // visible one, whose tile count differs between the query tiles of a
        // group, and with it first those tiles would read every later block
        // out of step (and miss the XCD's L2).
        // Striped blocks are the exception: there every pair is cut by the
        // causal diagonal alike, so the chains all take ascending block order
        // and the items run q-tile first (the same key tiles at the same time
        // on an XCD, whatever the device).
        for (int64_t i = 0; i < N; i++) {
            if (striped) std::sort(chain[i].begin(), chain[i].end());
            else if (chain[i].size() > 1 && chain[i].front() == i)
                std::rotate(chain[i].begin(), chain[i].begin() + 1, chain[i].end());
        }
        {
            std::vector<int32_t> order;
            for (int64_t i = 0; i < N; i++)
                if (!chain[i].empty()) order.push_back((int32_t)i);
            // heaviest first: longest chains, then later devices (more keys under causal masks)
            std::stable_sort(order.begin(), order.end(), [&](int32_t x, int32_t y) {
                return chain[x].size() != chain[y].size() ? chain[x].size() > chain[y].size() : x > y;
            });
            std::vector<RingWork> works;
            std::vector<RingEntry> entries;
            for (int32_t i : order) {
                RingWork w;
                w.q_off = row_off(i, q->stride_tok);
                w.q_pos0 = striped ? i : i * B;
                w.out_off = striped ? i * out_tok : i * B * out_tok;
                w.lse_off = striped ? i : i * B;
                w.first = (int32_t)entries.size();
                w.count = (int32_t)chain[i].size();
                works.push_back(w);
                for (int32_t j : chain[i]) {
                    RingEntry e;
                    e.k_off = row_off(j, k->stride_tok);
                    e.vt_off = (int64_t)j * vt_blk;
                    e.k_pos0 = striped ? j : j * B;
                    e.kb_off = j * kbw;
                    entries.push_back(e);
                }
            }
            if (!works.empty()) {
                stage.add(ws.works, works.data(), sizeof(RingWork) * works.size());
                stage.add(ws.entries, entries.data(), sizeof(RingEntry) * entries.size());
                if (stage.flush(st) != hipSuccess) return RA_E_HIP;
                StepArgs a = base;
                a.k = k->data;
                a.k_row_stride = (striped ? N : 1) * k->stride_tok;
                a.k_head_stride = k->stride_head;
                a.vt = ws.vt;
                a.vt_row_stride = Bp;
                a.vt_head_stride = d * Bp;
                a.works = ws.works;
                a.entries = ws.entries;
                a.wq = ws.wq;
                a.hpi = hpi;
                a.qt_major = striped;
                a.n_qtiles = (int32_t)n_qtiles_ring;
                // the work queues start at zero (a fill kernel, no memset node under graph capture)
                if (launch_fill_u64((unsigned long long*)ws.wq, 4, st) != hipSuccess) return RA_E_HIP;
                a.n_pairs = (int32_t)works.size();
                if (launch(a, q->dtype, st) != hipSuccess) return RA_E_HIP;
            }
            ring_done = true;
        }
    }

    // (the workspace holds the per-step state whenever this path can run)
    if (!ring_done && !fwd_needs_state(T, N, Hq, d, q->dtype, prefetch != 0)) return RA_E_UNSUPPORTED;
    if (stage.flush(st) != hipSuccess) return RA_E_HIP;
    for (int64_t s = 0; s < (ring_done ? 0 : r.passes); s++) {
        const std::vector<StepPair>& pairs = plan.steps[s];
        const bool use_buf = pf && s > 0;
        const int slot = (int)(s & 1);
        if (pf && s == 0) {
            // Step 1's copies must not start before the caller's earlier work
            // (which produced k and v) and the V^T pack are done.
            if (hipEventRecord(pf->consumed[1], st) != hipSuccess) return RA_E_HIP;
            if (hipStreamWaitEvent(pf->copy, pf->consumed[1], 0) != hipSuccess) return RA_E_HIP;
        }
        if (use_buf) {
            // The copy engine may overwrite this slot once step s-2 has read it.
            if (s >= 2 && hipStreamWaitEvent(pf->copy, pf->consumed[slot], 0) != hipSuccess) return RA_E_HIP;
            if (const uint32_t us = g_copy_delay_us.load())
                if (launch_spin(us, pf->copy) != hipSuccess) return RA_E_HIP;
            for (const StepPair& sp : pairs) {
                const char* kb = (const char*)k->data + row_off(sp.j, k->stride_tok) * es;
                const size_t kpitch = (size_t)(striped ? N : 1) * k->stride_tok * es;
                if (hipMemcpy2DAsync(k_slot(slot, sp.i), (size_t)Hkv * d * es, kb, kpitch, (size_t)Hkv * d * es,
                                     (size_t)B, hipMemcpyDeviceToDevice, pf->copy) != hipSuccess)
                    return RA_E_HIP;
                if (use_vt) {
                    if (hipMemcpyAsync(v_slot(slot, sp.i), ws.vt + (size_t)sp.j * vt_blk * 2, (size_t)vt_blk * 2,
                                       hipMemcpyDeviceToDevice, pf->copy) != hipSuccess)
                        return RA_E_HIP;
                } else {
                    const char* vb = (const char*)v->data + row_off(sp.j, v->stride_tok) * es;
                    const size_t vpitch = (size_t)(striped ? N : 1) * v->stride_tok * es;
                    if (hipMemcpy2DAsync(v_slot(slot, sp.i), (size_t)Hkv * d * es, vb, vpitch, (size_t)Hkv * d * es,
                                         (size_t)B, hipMemcpyDeviceToDevice, pf->copy) != hipSuccess)
                        return RA_E_HIP;
                }
            }
            if (hipEventRecord(pf->copied[slot], pf->copy) != hipSuccess) return RA_E_HIP;
            if (hipStreamWaitEvent(st, pf->copied[slot], 0) != hipSuccess) return RA_E_HIP;
        }
        if (pf) {
            if (const uint32_t us = g_compute_delay_us.load())
                if (launch_spin(us, st) != hipSuccess) return RA_E_HIP;
        }
        for (size_t c0 = 0; c0 < pairs.size(); c0 += kMaxPairs) {
            StepArgs a = base;
            a.n_pairs = (int32_t)std::min<size_t>(kMaxPairs, pairs.size() - c0);
            if (use_buf) {
                a.k = ws.kv;
                a.k_row_stride = Hkv * d;
                a.k_head_stride = d;
                if (use_vt) {
                    a.vt = ws.kv + ws.k_half;
                } else {
                    a.v = ws.kv + ws.k_half;
                    a.v_row_stride = Hkv * d;
                    a.v_head_stride = d;
                }
            } else {
                a.k = k->data;
                a.k_row_stride = (striped ? N : 1) * k->stride_tok;
                a.k_head_stride = k->stride_head;
                if (use_vt) {
                    a.vt = ws.vt;
                } else {
                    a.v = v->data;
                    a.v_row_stride = (striped ? N : 1) * v->stride_tok;
                    a.v_head_stride = v->stride_head;
                }
            }
            if (use_vt) {
                a.vt_row_stride = Bp;
                a.vt_head_stride = d * Bp;
            }
            for (int32_t x = 0; x < a.n_pairs; x++) {
                const StepPair& sp = pairs[c0 + x];
                PairDesc& p = a.pairs[x];
                p.q_off = row_off(sp.i, q->stride_tok);
                if (use_buf) {
                    p.k_off = ((int64_t)slot * N + sp.i) * blk_elems;
                    p.v_off = p.k_off;
                    p.vt_off = ((int64_t)slot * N + sp.i) * vt_blk;
                } else {
                    p.k_off = row_off(sp.j, k->stride_tok);
                    p.v_off = row_off(sp.j, v->stride_tok);
                    p.vt_off = (int64_t)sp.j * vt_blk;
                }
                p.q_pos0 = striped ? sp.i : sp.i * B;
                p.k_pos0 = striped ? sp.j : sp.j * B;
                p.kb_off = sp.j * kbw;
                p.O = ws.O + (size_t)sp.i * Hq * B * d;
                p.m = ws.m + (size_t)sp.i * Hq * B;
                p.l = ws.l + (size_t)sp.i * Hq * B;
                p.out_off = striped ? sp.i * out_tok : sp.i * B * out_tok;
                p.lse_off = striped ? sp.i : sp.i * B;
                p.load_state = sp.load_state;
                p.finalize = sp.finalize;
            }
            if (launch(a, q->dtype, st) != hipSuccess) return RA_E_HIP;
        }
        if (use_buf && hipEventRecord(pf->consumed[slot], st) != hipSuccess) return RA_E_HIP;
    }
    for (int32_t i : plan.empty_devices) {
        const int64_t o_off = striped ? i * out_tok : i * B * out_tok;
        if (launch_empty_rows(out, (int)out_dtype, o_off, base.out_row_stride, d, lse, striped ? i : i * B,
                              base.lse_row_stride, T, B, Hq, d, st) != hipSuccess)
            return RA_E_HIP;
    }

    if (stats) {
        unsigned long long c[4] = {0, 0, 0, 0};
        if (hipMemcpyAsync(c, ws.counters, sizeof c, hipMemcpyDeviceToHost, st) != hipSuccess) return RA_E_HIP;
        if (hipStreamSynchronize(st) != hipSuccess) return RA_E_HIP;
        stats->block_pairs_visited = plan.visited;
        stats->block_pairs_skipped = plan.skipped;
        stats->block_pairs_full = plan.full;
        stats->block_pairs_partial = plan.partial;
        // the one-launch ring counted tiles of its own height
        const bool ring_tiles = ring_done && hpi > 1;
        stats->tiles_skipped = (int64_t)c[0] + (ring_tiles ? plan_ring : plan).tiles_in_skipped_pairs;
        stats->tiles_full = (int64_t)c[1];
        stats->tiles_partial = (int64_t)c[2];
        stats->allowed_pairs = allowed_pairs(r);
        stats->tile_q = ring_tiles ? tq_ring : tq;
        stats->tile_k = tk;
    }
    return RA_OK;
}

ra_status ring_attn_forward(const ra_tensor* q, const ra_tensor* k, const ra_tensor* v, void* out,
                            ra_dtype out_dtype, float* lse, int32_t n_blocks, ra_layout layout, ra_mask mask_mode,
                            int32_t max_ring_passes, const int32_t* cu_seqlens_host, int32_t n_docs,
                            const uint8_t* key_valid, float scale, int prefetch, void* workspace,
                            size_t workspace_bytes, ra_stats* stats, void* stream) {
    return forward_impl(q, k, v, out, out_dtype, lse, n_blocks, layout, mask_mode, max_ring_passes, cu_seqlens_host,
                        n_docs, key_valid, scale, prefetch, workspace, workspace_bytes, stats, stream, true);
}

ra_status ring_attn_forward_noalloc(const ra_tensor* q, const ra_tensor* k, const ra_tensor* v, void* out,
                                    ra_dtype out_dtype, float* lse, int32_t n_blocks, ra_layout layout,
                                    ra_mask mask_mode, int32_t max_ring_passes, const int32_t* cu_seqlens_host,
                                    int32_t n_docs, const uint8_t* key_valid, float scale, ra_stats* stats,
                                    void* stream) {
    // Invalid shapes size to 0 here and are refused by ring_attn_forward.
    if (q && k) {
        const int32_t docs = mask_mode == RA_MASK_DOC_CAUSAL ? n_docs : 0;
        if (ring_attn_forward_workspace_size(q, k, n_blocks, docs, 0) > kScratchBytes) return RA_E_TOO_LARGE;
    }
    void* ws = nullptr;
    if (scratch_address(&ws) != hipSuccess) return RA_E_HIP;
    // (its tables go to the device straight from host memory: no pinned staging buffer is allocated)
    return forward_impl(q, k, v, out, out_dtype, lse, n_blocks, layout, mask_mode, max_ring_passes, cu_seqlens_host,
                        n_docs, key_valid, scale, 0, ws, kScratchBytes, stats, stream, false);
}

size_t ring_attn_forward_noalloc_scratch_bytes(void) { return kScratchBytes; }

ra_status ring_attn_test_prefetch_delays(uint32_t copy_delay_us, uint32_t compute_delay_us) {
    if (copy_delay_us > kMaxDelayUs || compute_delay_us > kMaxDelayUs) return RA_E_ARG;
    g_copy_delay_us.store(copy_delay_us);
    g_compute_delay_us.store(compute_delay_us);
    return RA_OK;
}

size_t ring_attn_backward_workspace_size(const ra_tensor* q, int32_t n_blocks, int32_t n_docs) {
    if (!q || n_blocks < 1 || n_docs < 0 || q->n_tok < 0 || q->n_head < 1) return 0;
    if (q->n_tok % n_blocks) return 0;
    return carve_bwd(nullptr, q->n_tok, n_blocks, q->n_head, n_docs).total;
}

ra_status ring_attn_backward(const ra_tensor* q, const ra_tensor* k, const ra_tensor* v, const ra_tensor* out,
                             const ra_tensor* dout, const float* lse, void* dq, void* dk, void* dv,
                             ra_dtype grad_dtype, int32_t n_blocks, ra_layout layout, ra_mask mask_mode,
                             int32_t max_ring_passes, const int32_t* cu_seqlens_host, int32_t n_docs,
                             const uint8_t* key_valid, float scale, void* workspace, size_t workspace_bytes,
                             void* stream) {
    // ---- arguments ----
    if (!tensor_ok(q) || !tensor_ok(k) || !tensor_ok(v) || !tensor_ok(out) || !tensor_ok(dout)) return RA_E_ARG;
    if ((!lse || !dq || !dk || !dv) && q->n_tok > 0) return RA_E_ARG;  // an empty sequence needs no buffers
    if (!valid_dtype(grad_dtype)) return RA_E_ARG;
    if (q->dtype != k->dtype || q->dtype != v->dtype || dout->dtype != q->dtype) return RA_E_ARG;
    const int64_t T = q->n_tok, Hq = q->n_head, Hkv = k->n_head, d = q->head_dim;
    if (k->n_tok != T || v->n_tok != T || v->n_head != Hkv || k->head_dim != d || v->head_dim != d) return RA_E_ARG;
    if (out->n_tok != T || out->n_head != Hq || out->head_dim != d) return RA_E_ARG;
    if (dout->n_tok != T || dout->n_head != Hq || dout->head_dim != d) return RA_E_ARG;
    if (Hq % Hkv) return RA_E_ARG;
    if (n_blocks < 1 || T % n_blocks || max_ring_passes < 1 || !scale_ok(scale)) return RA_E_ARG;
    if (layout != RA_LAYOUT_CONTIGUOUS && layout != RA_LAYOUT_STRIPED) return RA_E_ARG;
    if (mask_mode < RA_MASK_NONE || mask_mode > RA_MASK_DOC_CAUSAL) return RA_E_ARG;
    if (mask_mode == RA_MASK_DOC_CAUSAL) {
        if (!cu_seqlens_host || n_docs < 1 || cu_seqlens_host[0] != 0 || cu_seqlens_host[n_docs] != T)
            return RA_E_ARG;
        for (int32_t i = 0; i < n_docs; i++)
            if (cu_seqlens_host[i + 1] < cu_seqlens_host[i]) return RA_E_ARG;
        if (layout == RA_LAYOUT_STRIPED) return RA_E_UNSUPPORTED;
    } else {
        n_docs = 0;
    }
    // Matrix-core backward only: 16-bit inputs, head_dim 64 or 128, 16-byte
    // rows, at most one ring block per lane of a wave (the per-block tables);
    // a 16-bit out or gradient has the inputs' type.
    if (!is16(q->dtype) || (d != 64 && d != 128)) return RA_E_UNSUPPORTED;
    if ((is16(out->dtype) && out->dtype != q->dtype) || (is16(grad_dtype) && grad_dtype != q->dtype))
        return RA_E_UNSUPPORTED;
    if (n_blocks > kMaxRingChain) return RA_E_UNSUPPORTED;
    if (T >= ((int64_t)1 << 31)) return RA_E_UNSUPPORTED;  // per-lane positions are 32-bit
    if (T / n_blocks >= ((int64_t)1 << 21)) return RA_E_UNSUPPORTED;  // 64-row tile indices fit 15 bits
    if (!bf16_aligned(q) || !bf16_aligned(k) || !bf16_aligned(v) || !bf16_aligned(dout)) return RA_E_UNSUPPORTED;
    if ((uintptr_t)out->data % 16 || out->stride_tok % (is16(out->dtype) ? 8 : 4) ||
        out->stride_head % (is16(out->dtype) ? 8 : 4))
        return RA_E_UNSUPPORTED;
    if ((uintptr_t)dq % 16 || (uintptr_t)dk % 16 || (uintptr_t)dv % 16) return RA_E_UNSUPPORTED;
    {
        // 64-row tiles are addressed with 32-bit byte offsets from their first row.
        const int64_t rm = layout == RA_LAYOUT_STRIPED ? n_blocks : 1;
        if (!bf16_tile_addressable(rm * q->stride_tok) || !bf16_tile_addressable(rm * k->stride_tok) ||
            !bf16_tile_addressable(rm * v->stride_tok) || !bf16_tile_addressable(rm * dout->stride_tok))
            return RA_E_UNSUPPORTED;
    }
    const int64_t N = n_blocks, B = T / N;
    const int64_t n_qtiles = (B + bwd_tile_q() - 1) / bwd_tile_q();
    const int64_t n_ktiles = (B + bwd_tile_k() - 1) / bwd_tile_k();
    if (N * Hq * n_qtiles * 256 > INT32_MAX || N * Hkv * n_ktiles * 256 > INT32_MAX) return RA_E_UNSUPPORTED;
    if (T == 0) return RA_OK;  // an empty sequence needs no workspace
    BwdWorkspace ws = carve_bwd(workspace, T, N, Hq, n_docs);
    if (!workspace || workspace_bytes < ws.total) return RA_E_WORKSPACE;
    if ((uintptr_t)workspace % kAlign) return RA_E_WORKSPACE;

    // ---- ring visits: device i's key blocks (ring order) and block j's visitors ----
    Ring r;
    r.T = T;
    r.N = N;
    r.B = B;
    r.layout = layout;
    r.mask = mask_mode;
    r.passes = std::min<int64_t>(max_ring_passes, N);
    r.cu = cu_seqlens_host;
    r.n_docs = n_docs;
    const Plan plan = make_plan(r, bwd_tile_q(), bwd_tile_k());
    const bool striped = layout == RA_LAYOUT_STRIPED;
    auto pos0 = [&](int64_t blk) { return striped ? blk : blk * B; };
    std::vector<std::vector<int64_t>> fwd((size_t)N), rev((size_t)N);
    // Visiting order: the gradients are sums with no required order, so each
    // chain takes the diagonal pair (step 0: a block with itself, where the
    // tiles of one group stop at different points under causal masks) last;
    // the group's tiles then walk every other block in step, and its L2
    // serves their shared K/V (or q/dout) tiles.
    for (int64_t s = r.passes - 1; s >= 0; s--)
        for (const StepPair& sp : plan.steps[s]) {
            fwd[sp.i].push_back(pos0(sp.j));
            rev[sp.j].push_back(pos0(sp.i));
        }
    // Striped blocks are cut by the causal diagonal alike in every pair: all
    // chains take ascending block order there, and the kernels number their
    // items tile index first, so that the items running together on an XCD
    // stream the same tiles at the same time.
    if (striped)
        for (int64_t i = 0; i < N; i++) {
            std::sort(fwd[i].begin(), fwd[i].end());
            std::sort(rev[i].begin(), rev[i].end());
        }
    std::vector<BwdWork> works, rworks;
    std::vector<int64_t> partners, rpartners;
    auto flatten = [&](std::vector<std::vector<int64_t>>& lists, std::vector<BwdWork>& wv, std::vector<int64_t>& pv) {
        // Blocks with the most partners first (the longest workgroups start early).
        std::vector<int64_t> order((size_t)N);
        for (int64_t i = 0; i < N; i++) order[i] = i;
        std::stable_sort(order.begin(), order.end(),
                         [&](int64_t x, int64_t y) { return lists[x].size() > lists[y].size(); });
        for (int64_t i : order) {
            BwdWork w;
            w.pos0 = pos0(i);
            w.loc0 = i * B;
            w.first = (int32_t)pv.size();
            w.count = (int32_t)lists[i].size();
            wv.push_back(w);
            pv.insert(pv.end(), lists[i].begin(), lists[i].end());
        }
    };
    flatten(fwd, works, partners);
    flatten(rev, rworks, rpartners);

    hipStream_t st = (hipStream_t)stream;
    HostStager stage(true);
    if (n_docs > 0) stage.add(ws.cu, cu_seqlens_host, sizeof(int32_t) * (size_t)(n_docs + 1));
    stage.add(ws.works, works.data(), sizeof(BwdWork) * works.size());
    stage.add(ws.rworks, rworks.data(), sizeof(BwdWork) * rworks.size());
    stage.add(ws.partners, partners.data(), sizeof(int64_t) * partners.size());
    stage.add(ws.rpartners, rpartners.data(), sizeof(int64_t) * rpartners.size());
    if (stage.flush(st) != hipSuccess) return RA_E_HIP;
    if (key_valid && launch_pack_key_bits(key_valid, 1, N, B, striped, key_words(B), ws.kbits, st) != hipSuccess)
        return RA_E_HIP;

    BwdArgs a;
    std::memset(&a, 0, sizeof a);
    a.key_valid = key_valid;
    a.kbits = key_valid ? ws.kbits : nullptr;
    a.kb_words = (int32_t)key_words(B);
    a.q = q->data;
    a.k = k->data;
    a.v = v->data;
    a.out = out->data;
    a.dout = dout->data;
    a.q_st = q->stride_tok;
    a.q_sh = q->stride_head;
    a.k_st = k->stride_tok;
    a.k_sh = k->stride_head;
    a.v_st = v->stride_tok;
    a.v_sh = v->stride_head;
    a.out_st = out->stride_tok;
    a.out_sh = out->stride_head;
    a.do_st = dout->stride_tok;
    a.do_sh = dout->stride_head;
    a.lse = lse;
    a.Lse2 = ws.Lse2;
    a.Dsum = ws.Dsum;
    a.dq = dq;
    a.dk = dk;
    a.dv = dv;
    a.f16 = q->dtype == RA_F16;
    a.out16 = is16(out->dtype);
    a.grad16 = is16(grad_dtype);
    a.T = T;
    a.B = B;
    a.pos_stride = striped ? N : 1;
    a.Hq = (int32_t)Hq;
    a.Hkv = (int32_t)Hkv;
    a.group = (int32_t)(Hq / Hkv);
    a.d = (int32_t)d;
    a.mask = mask_mode;
    a.scale = scale;
    a.c2 = scale * 1.4426950408889634f;
    a.cu = ws.cu;
    a.n_docs = n_docs;
    a.n_qtiles = (int32_t)n_qtiles;
    a.n_ktiles = (int32_t)n_ktiles;
    a.n_works = (int32_t)works.size();
    a.n_rworks = (int32_t)rworks.size();
    a.works = ws.works;
    a.partners = ws.partners;
    a.rworks = ws.rworks;
    a.rpartners = ws.rpartners;
    // the kernels' work queues start at zero (a fill kernel, no memset node under graph capture)
    a.qt_major = striped;
    a.wq = ws.wq;
    if (launch_fill_u64((unsigned long long*)ws.wq, 8, st) != hipSuccess) return RA_E_HIP;
    if (launch_backward(a, st) != hipSuccess) return RA_E_HIP;
    return RA_OK;
}

}  // extern "C"
