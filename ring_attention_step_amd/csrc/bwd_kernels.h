// Launch descriptors of the ring backward, shared by the C ABI driver and the
// backward kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <cstdint>

namespace ra {

// Backward of the ring (16-bit inputs, bf16 or fp16; matrix cores).  Rows of every tensor are
// global token positions (striped blocks are strided views).
struct BwdWork {                   // one ring block and the blocks paired with it
    int64_t pos0;                  // global position of its local row 0
    int64_t loc0;                  // block index * rows per block (block-local row order)
    int32_t first, count;          // partner positions: partners[first .. first + count)
};
struct BwdArgs {
    const void* q;                 // 16-bit [T, Hq, d] view
    const void* k;                 // 16-bit [T, Hkv, d] view
    const void* v;
    const void* out;               // forward output [T, Hq, d], 16-bit or f32 (out16)
    const void* dout;              // 16-bit [T, Hq, d] view
    int64_t q_st, q_sh, k_st, k_sh, v_st, v_sh, out_st, out_sh, do_st, do_sh;  // element strides
    const float* lse;              // [Hq, T], natural log
    float* Lse2;                   // workspace [Hq, T] (+ pad): lse * log2(e) in block-local row order
    float* Dsum;                   // workspace [Hq, T] (+ pad), same order: dout . out; Dsum - Lse2 < 2^30
    void* dq;                      // [T, Hq, d] contiguous, f32 or 16-bit (grad16)
    void* dk;                      // [T, Hkv, d] contiguous
    void* dv;
    int32_t out16, grad16;
    int64_t T, B, pos_stride;      // tokens; rows per block; position step between local rows
    int32_t Hq, Hkv, group, d, mask;
    float scale, c2;               // scale and scale * log2(e)
    const int32_t* cu;             // device cu_seqlens (doc-causal)
    int32_t n_docs;
    int32_t n_qtiles, n_ktiles;    // 128-row tiles of a block, query side / key side
    int32_t n_works, n_rworks;
    const BwdWork* works;          // per query block: the key blocks it visits (positions)
    const int64_t* partners;
    const BwdWork* rworks;         // per key block: the query blocks that visit it
    const int64_t* rpartners;
    // Key-padding mask (both null without one): key_valid[t] != 0 when key
    // token t takes part; kbits holds the same as bits of whole 64-key tiles,
    // block j's kb_words words at j * kb_words (block-local rows).
    const uint8_t* key_valid;
    const uint32_t* kbits;
    int32_t kb_words;
    int32_t f16;                   // 16-bit values are fp16, else bf16 (picks the kernels)
    unsigned* wq;                  // 16 work-queue counters (dq 0..7, dk/dv 8..15), zero at the launch
    int32_t qt_major;              // items numbered tile index first (striped blocks), else group first
};
constexpr int kBwdPad = 256;       // floats of padding after Lse2 and after Dsum
int bwd_tile_q();
int bwd_tile_k();
hipError_t launch_backward(const BwdArgs& a, hipStream_t stream);

}  // namespace ra
