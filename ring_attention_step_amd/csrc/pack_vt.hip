// Packs V of every ring block as V^T once per forward call, so the matrix-core
// step reads the V operand of O^T += V^T P^T with plain 16-byte LDS reads
// instead of transposing reads.  HBM-bound: one read and one write of V.
//
// Output vt[j][g][c][p], p < Bp: key position p of block j holds key
// w = swap_bits_2_3(p mod 16) + 16 floor(p / 16), i.e. inside every 16-key
// group the keys are stored as 0-3, 8-11, 4-7, 12-15 -- the order in which a
// lane half of the S^T accumulator holds them -- so each lane half's eight
// keys of a 16-key chunk are contiguous.  Keys w >= B are zero.
//
// FRAG: the same values in the order of the one-launch ring kernel's LDS
// tiles, so that each of its 1 KB tile loads reads 1 KB of contiguous memory
// (with rows of V^T, a load gathers 32 B from each of 32 rows): the region of
// (j, g) holds its 64-key tiles one after the other, tile kt as D / 8
// fragments of 512 elements, fragment f = c16 * (D / 32) + db holding, for
// lane l, positions 16 c16 + 8 (l / 32) .. +7 of dim row 32 db + l % 32.
#include "kernels.h"

namespace ra {
namespace {

typedef __bf16 bf16;
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));

constexpr int KEYS = 64;  // keys per workgroup

__device__ __forceinline__ int swap_bits_2_3(int p) { return (p & ~12) | ((p & 4) << 1) | ((p & 8) >> 1); }

template <int D, bool FRAG>
__global__ __launch_bounds__(256) void pack_vt_kernel(const bf16* v, int64_t st_tok, int64_t st_head, int64_t N,
                                                      int64_t B, int striped, int64_t Bp, bf16* vt) {
    __shared__ unsigned short tile[KEYS][D + 8];  // +8: spread the column reads over banks
    const int64_t w0 = (int64_t)blockIdx.x * KEYS;
    const int64_t g = blockIdx.y, j = blockIdx.z, Hkv = gridDim.y;
    // load 64 keys x D dims, 16 bytes per thread per step
    for (int c = threadIdx.x; c < KEYS * D / 8; c += 256) {
        const int key = c / (D / 8), col = (c % (D / 8)) * 8;
        const int64_t w = w0 + key;
        u32x4 x = {0u, 0u, 0u, 0u};
        if (w < B) {
            const int64_t tok = striped ? w * N + j : j * B + w;
            x = *(const u32x4*)(v + tok * st_tok + g * st_head + col);
        }
        *(u32x4*)&tile[key][col] = x;
    }
    __syncthreads();
    if (FRAG) {
        // 16 bytes per lane of a fragment, consecutive threads consecutive
        // 16-byte pieces (Bp is a multiple of the 64-key tile)
        bf16* out = vt + ((j * Hkv + g) * D) * Bp + w0 * D;
        for (int c = threadIdx.x; c < D * KEYS / 8; c += 256) {
            const int f = c / 64, l = c % 64;
            const int dim = 32 * (f % (D / 32)) + l % 32, p0 = 16 * (f / (D / 32)) + 8 * (l / 32);
            u16x8 x;
#pragma unroll
            for (int e = 0; e < 8; e++) x[e] = tile[swap_bits_2_3(p0 + e)][dim];
            *(u16x8*)(out + 8 * c) = x;
        }
        return;
    }
    // write D rows x 64 positions, 8 positions (16 bytes) per thread per step
    bf16* out = vt + ((j * Hkv + g) * D) * Bp;
    for (int c = threadIdx.x; c < D * KEYS / 8; c += 256) {
        const int dim = c / (KEYS / 8), p0 = (c % (KEYS / 8)) * 8;
        if (w0 + p0 >= Bp) continue;  // Bp is a multiple of 8
        u16x8 x;
#pragma unroll
        for (int e = 0; e < 8; e++) x[e] = tile[swap_bits_2_3(p0 + e)][dim];
        *(u16x8*)(out + dim * Bp + w0 + p0) = x;
    }
}

}  // namespace

int64_t vt_padded_keys(int64_t B) { return (B + kBf16TileK - 1) / kBf16TileK * kBf16TileK; }

hipError_t launch_pack_vt(const void* v, int64_t st_tok, int64_t st_head, int64_t N, int64_t B, int striped,
                          int64_t Hkv, int64_t d, bool frag, void* vt, hipStream_t stream) {
    static_assert(KEYS == kBf16TileK, "one workgroup per key tile of the fragment order");
    const int64_t Bp = vt_padded_keys(B);
    if (Bp == 0 || Hkv == 0 || N == 0) return hipSuccess;
    const dim3 grid((unsigned)((Bp + KEYS - 1) / KEYS), (unsigned)Hkv, (unsigned)N);
    const bf16* vb = (const bf16*)v;
    bf16* o = (bf16*)vt;
    if (d == 128 && frag)
        pack_vt_kernel<128, true><<<grid, 256, 0, stream>>>(vb, st_tok, st_head, N, B, striped, Bp, o);
    else if (d == 128)
        pack_vt_kernel<128, false><<<grid, 256, 0, stream>>>(vb, st_tok, st_head, N, B, striped, Bp, o);
    else if (d == 64 && frag)
        pack_vt_kernel<64, true><<<grid, 256, 0, stream>>>(vb, st_tok, st_head, N, B, striped, Bp, o);
    else if (d == 64)
        pack_vt_kernel<64, false><<<grid, 256, 0, stream>>>(vb, st_tok, st_head, N, B, striped, Bp, o);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace ra
