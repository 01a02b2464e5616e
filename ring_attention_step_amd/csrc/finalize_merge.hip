// Element-wise kernels around the ring step (HBM-bound, no data reuse):
//  finalize: out = O / l, lse = m + ln l (the glossary page's worked example
//            divides the accumulated weighted values by the accumulated
//            weights once the ring is done);
//  merge:    two normalised partials combined through their log-sum-exp
//            (GitHub issue: the returned lse is what makes blockwise results
//            combinable; shift invariance of softmax lets the larger lse be
//            factored out first);
//  fill / empty rows: counters to zero and rows that saw no key.
// Each row is handled by one wave: lanes stride over head_dim (coalesced) and
// lane 0 writes the row's lse after every lane has read the old one.
#include <cmath>

#include "kernels.h"

namespace ra {
namespace {

typedef __bf16 bf16;
typedef _Float16 f16;

// Element kinds: 0 fp32, 1 bf16, 2 fp16 (16-bit stores round to nearest even).
__device__ __forceinline__ float load_val(const void* p, int kind, int64_t i) {
    if (kind == 1) return (float)((const bf16*)p)[i];
    if (kind == 2) return (float)((const f16*)p)[i];
    return ((const float*)p)[i];
}
__device__ __forceinline__ void store_val(void* p, int kind, int64_t i, float x) {
    if (kind == 1) ((bf16*)p)[i] = (bf16)x;
    else if (kind == 2) ((f16*)p)[i] = (f16)x;
    else ((float*)p)[i] = x;
}

__global__ __launch_bounds__(256) void finalize_kernel(const float* O, const float* m, const float* l,
                                                        int64_t Hq, int64_t Bq, int64_t d, void* out,
                                                        int out_kind, int64_t ost, int64_t osh, float* lse) {
    const int lane = threadIdx.x & 63;
    const int64_t rows = Hq * Bq;
    for (int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); r < rows; r += (int64_t)gridDim.x * 4) {
        const int64_t h = r / Bq, u = r % Bq;
        const float lr = l[r];
        const float inv = lr > 0.f ? 1.f / lr : 0.f;
        for (int64_t c = lane; c < d; c += 64) store_val(out, out_kind, u * ost + h * osh + c, O[r * d + c] * inv);
        if (lane == 0 && lse) lse[r] = lr > 0.f ? m[r] + logf(lr) : -INFINITY;
    }
}

__global__ __launch_bounds__(256) void merge_kernel(void* out_acc, float* lse_acc, const void* out_blk,
                                                     const float* lse_blk, int kind, int64_t Hq, int64_t rows,
                                                     int64_t d) {
    const int lane = threadIdx.x & 63;
    const int64_t n = Hq * rows;
    for (int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); r < n; r += (int64_t)gridDim.x * 4) {
        const int64_t h = r / rows, u = r % rows;
        const float la = lse_acc[r], lb = lse_blk[r];
        const float big = fmaxf(la, lb);
        float wa = 0.f, wb = 0.f, lse = -INFINITY;
        if (big != -INFINITY) {
            wa = expf(la - big);
            wb = expf(lb - big);
            const float tot = wa + wb;
            lse = big + logf(tot);
            wa /= tot;
            wb /= tot;
        }
        const int64_t base = (u * Hq + h) * d;
        for (int64_t c = lane; c < d; c += 64) {
            const float x = wa * load_val(out_acc, kind, base + c) + wb * load_val(out_blk, kind, base + c);
            store_val(out_acc, kind, base + c, big == -INFINITY ? 0.f : x);
        }
        if (lane == 0) lse_acc[r] = lse;
    }
}

__global__ void fill_u64_kernel(unsigned long long* p, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        p[i] = 0ull;
}

__global__ __launch_bounds__(256) void empty_rows_kernel(void* out, int out_kind, int64_t out_off, int64_t ors,
                                                          int64_t ohs, float* lse, int64_t lse_off, int64_t lrs,
                                                          int64_t lhs, int64_t rows, int64_t Hq, int64_t d) {
    const int64_t n = rows * Hq * d;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t c = i % d, h = (i / d) % Hq, u = i / (d * Hq);
        store_val(out, out_kind, out_off + u * ors + h * ohs + c, 0.f);
        if (c == 0 && lse) lse[lse_off + h * lhs + u * lrs] = -INFINITY;
    }
}

unsigned grid_for(int64_t work, int64_t per_block) {
    int64_t g = (work + per_block - 1) / per_block;
    if (g < 1) g = 1;
    if (g > 65536) g = 65536;
    return (unsigned)g;
}

}  // namespace

hipError_t launch_finalize(const float* O, const float* m, const float* l, int64_t Hq, int64_t Bq, int64_t d,
                           void* out, int out_kind, int64_t ost, int64_t osh, float* lse, hipStream_t stream) {
    if (Hq * Bq == 0) return hipSuccess;
    finalize_kernel<<<grid_for(Hq * Bq, 4), 256, 0, stream>>>(O, m, l, Hq, Bq, d, out, out_kind, ost, osh, lse);
    return hipGetLastError();
}

hipError_t launch_merge(void* out_acc, float* lse_acc, const void* out_blk, const float* lse_blk, int kind,
                        int64_t Hq, int64_t rows, int64_t d, hipStream_t stream) {
    if (Hq * rows == 0) return hipSuccess;
    merge_kernel<<<grid_for(Hq * rows, 4), 256, 0, stream>>>(out_acc, lse_acc, out_blk, lse_blk, kind, Hq, rows, d);
    return hipGetLastError();
}

hipError_t cu_count(int* n) {
    static int cache[64] = {0};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    if (!cache[dev]) {
        int c = 0;
        if ((e = hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return e;
        cache[dev] = c > 0 ? c : 1;
    }
    *n = cache[dev];
    return hipSuccess;
}

// One wave that waits `ticks` of the constant-rate wall clock, then exits
// (a bounded delay on a stream; used only by the prefetch ordering test hook).
__global__ void spin_kernel(uint64_t ticks) {
    const uint64_t t0 = wall_clock64();
    while (wall_clock64() - t0 < ticks) __builtin_amdgcn_s_sleep(8);
}

hipError_t launch_spin(uint32_t us, hipStream_t stream) {
    static int khz = 0;  // wall-clock rate of device 0's kind (the only GPU model this library targets)
    if (!khz) {
        int dev = 0;
        hipError_t e = hipGetDevice(&dev);
        if (e == hipSuccess) e = hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev);
        if (e != hipSuccess) return e;
        if (khz <= 0) khz = 100000;
    }
    spin_kernel<<<1, 64, 0, stream>>>((uint64_t)us * (uint64_t)khz / 1000u);
    return hipGetLastError();
}

hipError_t launch_fill_u64(unsigned long long* p, int64_t n, hipStream_t stream) {
    if (n == 0) return hipSuccess;
    fill_u64_kernel<<<grid_for(n, 256), 256, 0, stream>>>(p, n);
    return hipGetLastError();
}

hipError_t launch_empty_rows(void* out, int out_kind, int64_t out_off, int64_t ors, int64_t ohs, float* lse,
                             int64_t lse_off, int64_t lrs, int64_t lhs, int64_t rows, int64_t Hq, int64_t d,
                             hipStream_t stream) {
    if (rows * Hq * d == 0) return hipSuccess;
    empty_rows_kernel<<<grid_for(rows * Hq * d, 256), 256, 0, stream>>>(out, out_kind, out_off, ors, ohs, lse,
                                                                         lse_off, lrs, lhs, rows, Hq, d);
    return hipGetLastError();
}

}  // namespace ra
