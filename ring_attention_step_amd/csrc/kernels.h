// Launch descriptors shared by the C ABI driver and the HIP kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <cstdint>

namespace ra {

// One (query block, key/value block) pair of a ring step.
struct PairDesc {
    int64_t q_off, k_off, v_off;   // element offset of local row 0 in q / k / v
    int64_t q_pos0, k_pos0;        // global position of local row 0 (mask coordinates)
    float* O;                      // running state of the query block: [Hq, Bq, d]
    float* m;                      //   [Hq, Bq]
    float* l;                      //   [Hq, Bq]
    int64_t out_off;               // element offset of local row 0 in out (finalize)
    int64_t lse_off;               // offset of (head 0, local row 0) in lse (finalize)
    int64_t vt_off;                // element offset of this key block in the packed V^T
    int32_t load_state;            // state holds earlier steps' keys
    int32_t finalize;              // write out / lse instead of the state
    int64_t kb_off;                // offset (32-bit words) of the key block's validity bits in kbits
};

constexpr int kMaxPairs = 16;

// Ring forward in one launch (bf16 path): a workgroup takes one query tile of
// one head of virtual device i through every key/value block device i visits,
// in ring order, with the online-softmax state kept in registers throughout.
struct RingWork {                  // one virtual device (query block)
    int64_t q_off, q_pos0;         // as in PairDesc
    int64_t out_off, lse_off;      // finalize targets
    int32_t first, count;          // its key/value blocks: entries [first, first + count)
};
constexpr int kMaxRingChain = 64;  // chain blocks a workgroup can hold (one per lane)
struct RingEntry {                 // one key/value block of a device's ring, in visiting order
    int64_t k_off, vt_off;         // element offsets of the block in k and in the packed V^T
    int64_t k_pos0;                // global position of its local row 0
    int64_t kb_off;                // offset (32-bit words) of its validity bits in kbits
};

struct StepArgs {
    const void* q;
    const void* k;
    const void* v;
    int64_t q_row_stride, q_head_stride;   // elements, per local row / head
    int64_t k_row_stride, k_head_stride;
    int64_t v_row_stride, v_head_stride;
    const void* vt;                        // packed V^T (16-bit matrix-core path) or null
    int64_t vt_row_stride, vt_head_stride; // elements per dim row / per head of a packed block
    int64_t Bq, Bk;                        // rows in the query block / key block
    int64_t pos_stride;                    // position step between local rows
    int32_t Hq, group;                     // query heads; query heads per kv head
    int32_t d;
    int32_t mask;
    float scale;                           // scores are scale * q.k
    float c2;                              // scale * log2(e)
    const int32_t* cu;                     // device cu_seqlens (doc-causal)
    int32_t n_docs;
    int32_t out16;                         // out in the inputs' 16-bit type (else fp32)
    void* out;
    int64_t out_row_stride, out_head_stride;
    float* lse;                            // nullable
    int64_t lse_row_stride, lse_head_stride;
    unsigned long long* stats;             // nullable, 3 counters
    int32_t n_qtiles, n_pairs;
    PairDesc pairs[kMaxPairs];
    // Ring forward in one launch: when works is set, the grid covers n_pairs
    // RingWork entries (pairs[] is unused), each finalised at its end.
    const RingWork* works;
    const RingEntry* entries;
    unsigned* wq;                          // its 8 work-queue counters, zero at the launch
    int32_t hpi;                           // query heads per work item (a power of two dividing the
                                           // group, <= 8); rows per item 256 / hpi; n_qtiles counts those
    int32_t qt_major;                      // items numbered q-tile first (else (work, head block) first)
    // Key-padding mask (nullable): bit w % 32 of word kb_off + w / 32 is set
    // when key row w of a block takes part; a block's bits are whole 64-key
    // tiles (2 words each, 8-byte aligned), zero past its last row.
    const uint32_t* kbits;
    int32_t f16;                           // 16-bit inputs are fp16, else bf16 (picks the kernel)
};

// Kernel tile shapes (query rows x key columns per workgroup tile).
constexpr int kBf16TileQ = 256, kBf16TileK = 64;
constexpr int kF32TileQ = 64, kF32TileK = 64;

hipError_t launch_step_bf16(const StepArgs& a, hipStream_t stream);
// The one-launch ring forward (works set, packed V^T): eight waves of 32
// query rows each per workgroup, each wave its own software pipeline.
hipError_t launch_ring_fwd(const StepArgs& a, hipStream_t stream);
hipError_t launch_step_f32(const StepArgs& a, hipStream_t stream);
hipError_t launch_finalize(const float* O, const float* m, const float* l, int64_t Hq, int64_t Bq,
                           int64_t d, void* out, int out_kind, int64_t out_stride_tok,
                           int64_t out_stride_head, float* lse, hipStream_t stream);
hipError_t launch_merge(void* out_acc, float* lse_acc, const void* out_blk, const float* lse_blk,
                        int kind, int64_t Hq, int64_t rows, int64_t d, hipStream_t stream);
// out_kind / kind: element type of out (0 fp32, 1 bf16, 2 fp16).
hipError_t launch_fill_u64(unsigned long long* p, int64_t n, hipStream_t stream);
// Compute units of the current device (queried once per device).
hipError_t cu_count(int* n);
// A bounded wait of `us` microseconds on `stream` (one wave).
hipError_t launch_spin(uint32_t us, hipStream_t stream);

// Key-padding bits of ring blocks: for block j < n_blocks and row w < B,
// bit w % 32 of bits[j * words_per_block + w / 32] = (key_valid[pos] != 0),
// pos = j + w * n_blocks (striped) or j * B + w; every other bit of the
// block's words_per_block words is 0.  n_blocks = 1, B = n, striped = 0 and
// a row stride packs one block given by its own rows.
hipError_t launch_pack_key_bits(const uint8_t* key_valid, int64_t row_stride, int64_t n_blocks, int64_t B,
                                int striped, int64_t words_per_block, uint32_t* bits, hipStream_t stream);

// Packed V^T of the ring blocks: vt[j][g][c][p] (p < Bp = B rounded up to the
// key tile) holds V of key w of block j, kv head g, dim c, where p is w with
// bits 2 and 3 swapped inside each 16-key group (the order in which the S^T
// accumulators hold their keys); zero for w >= B.  frag: the same values in
// the one-launch ring kernel's fragment order (its LDS tile layout): in the
// region of (j, g), tile kt of 64 keys at kt * 64 * d, fragment f at 512 f,
// lane l's eight positions 16 (f / (d/32)) + 8 (l / 32) .. +7 of dim row
// 32 (f % (d/32)) + l % 32 at 8 l.
int64_t vt_padded_keys(int64_t B);
hipError_t launch_pack_vt(const void* v, int64_t v_stride_tok, int64_t v_stride_head, int64_t N, int64_t B,
                          int striped, int64_t Hkv, int64_t d, bool frag, void* vt, hipStream_t stream);
hipError_t launch_empty_rows(void* out, int out_kind, int64_t out_off, int64_t out_row_stride,
                             int64_t out_head_stride, float* lse, int64_t lse_off,
                             int64_t lse_row_stride, int64_t lse_head_stride, int64_t rows,
                             int64_t Hq, int64_t d, hipStream_t stream);

}  // namespace ra
