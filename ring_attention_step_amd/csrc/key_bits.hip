// Packs a key-padding mask (one byte per key, nonzero = the key takes part)
// into the bit words the matrix-core kernels test: one 64-bit word per
// 64-key tile of a ring block, so a kernel reads a tile's mask with one
// scalar load and takes its mask-free path when the word is all ones.
// HBM-bound and tiny: T bytes read, T / 8 bytes written.
#include "kernels.h"

namespace ra {
namespace {

__global__ __launch_bounds__(256) void pack_key_bits_kernel(const uint8_t* key_valid, int64_t row_stride,
                                                            int64_t n_blocks, int64_t B, int striped,
                                                            int64_t words_per_block, uint32_t* bits) {
    const int64_t n_words = n_blocks * words_per_block;
    for (int64_t x = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; x < n_words;
         x += (int64_t)gridDim.x * blockDim.x) {
        const int64_t j = x / words_per_block, w0 = (x % words_per_block) * 32;
        uint32_t word = 0;
        for (int b = 0; b < 32; b++) {
            const int64_t w = w0 + b;
            if (w >= B) break;
            const int64_t pos = striped ? j + w * n_blocks : j * B + w;
            word |= (uint32_t)(key_valid[pos * row_stride] != 0) << b;
        }
        bits[x] = word;
    }
}

}  // namespace

hipError_t launch_pack_key_bits(const uint8_t* key_valid, int64_t row_stride, int64_t n_blocks, int64_t B,
                                int striped, int64_t words_per_block, uint32_t* bits, hipStream_t stream) {
    const int64_t n_words = n_blocks * words_per_block;
    if (n_words == 0) return hipSuccess;
    const int64_t blocks = (n_words + 255) / 256 < 4096 ? (n_words + 255) / 256 : 4096;
    pack_key_bits_kernel<<<(unsigned)blocks, 256, 0, stream>>>(key_valid, row_stride, n_blocks, B, striped,
                                                               words_per_block, bits);
    return hipGetLastError();
}

}  // namespace ra
