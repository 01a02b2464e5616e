// One ring step in true fp32 (no bf16 or reduced-precision matrix ops), for
// fp32 inputs with head_dim up to 128.  One wave per workgroup, one query row
// per lane; the key/value block streams through LDS in tiles of 64 keys.  Per
// tile and row: scores s = scale * q.k in fp32, tile maximum, rescale of the
// state by exp(m_old - m_new), p = exp(s - m_new), l += p, O += p v -- the
// running-max recurrence of the "Ring Attention simulation" gist applied one
// tile at a time, with m kept in the natural units of the scaled score.
#include <cmath>

#include "kernels.h"
#include "plan.h"

namespace ra {
namespace {

constexpr int TQ = kF32TileQ;  // 64 rows = one wave
constexpr int TK = kF32TileK;  // 64 keys per tile
static_assert(TK == 64, "one 64-bit key-validity word per key tile");

template <int DP>
__global__ __launch_bounds__(64) void step_f32_kernel(const StepArgs a) {
    __shared__ float ks[TK][DP];
    __shared__ float vs[TK][DP];
    const int lane = threadIdx.x;

    const int nwg = gridDim.x, b = blockIdx.x;
    const int logical = (nwg % 8 == 0) ? (b % 8) * (nwg / 8) + b / 8 : b;
    const int qt = a.n_qtiles - 1 - logical % a.n_qtiles;
    const int rest = logical / a.n_qtiles;
    const int head = rest % a.Hq;
    const PairDesc& pd = a.pairs[rest / a.Hq];
    const int kvh = head / a.group;
    const int d = a.d;

    const int64_t u0 = (int64_t)qt * TQ;
    const int64_t u_last = (a.Bq < u0 + TQ ? a.Bq : u0 + TQ) - 1;
    const int64_t t_min = pd.q_pos0 + u0 * a.pos_stride, t_max = pd.q_pos0 + u_last * a.pos_stride;
    int64_t ds_min = 0, ds_max = 0;
    if (a.mask == kMaskDoc) {
        ds_min = doc_start(a.cu, a.n_docs, t_min);
        ds_max = doc_start(a.cu, a.n_docs, t_max);
    }
    const int nkt = (int)((a.Bk + TK - 1) / TK);
    auto tile_cls = [&](int kt) {
        const int64_t w0 = (int64_t)kt * TK, w1 = (a.Bk < w0 + TK ? a.Bk : w0 + TK) - 1;
        return classify(a.mask, t_min, t_max, ds_min, ds_max, pd.k_pos0 + w0 * a.pos_stride,
                        pd.k_pos0 + w1 * a.pos_stride);
    };
    int kt_lo = 0, kt_hi = nkt - 1;
    while (kt_lo <= kt_hi && tile_cls(kt_lo) == kSkip) kt_lo++;
    while (kt_hi >= kt_lo && tile_cls(kt_hi) == kSkip) kt_hi--;

    const int64_t u = u0 + lane;
    const bool row_ok = u < a.Bq;
    const int64_t t = pd.q_pos0 + u * a.pos_stride;
    const int64_t ds = (a.mask == kMaskDoc && row_ok) ? doc_start(a.cu, a.n_docs, t) : 0;

    float q[DP], o[DP];
    const float* qp = (const float*)a.q + pd.q_off + head * a.q_head_stride + u * a.q_row_stride;
#pragma unroll
    for (int c = 0; c < DP; c++) {
        q[c] = (row_ok && c < d) ? qp[c] : 0.f;
        o[c] = 0.f;
    }
    float m = -INFINITY, l = 0.f;
    const int64_t srow = (int64_t)head * a.Bq + u;
    if (pd.load_state && row_ok) {
        m = pd.m[srow];
        l = pd.l[srow];
        const float* Op = pd.O + srow * d;
#pragma unroll
        for (int c = 0; c < DP; c++)
            if (c < d) o[c] = Op[c];
    }

    const float* kbase = (const float*)a.k + pd.k_off + kvh * a.k_head_stride;
    const float* vbase = (const float*)a.v + pd.v_off + kvh * a.v_head_stride;
    unsigned n_full = 0, n_part = 0;
    for (int kt = kt_lo; kt <= kt_hi; kt++) {
        const Cls cls = tile_cls(kt);
        n_full += cls == kFull;
        n_part += cls == kPartial;
        for (int idx = lane; idx < TK * DP; idx += 64) {
            const int key = idx / DP, c = idx % DP;
            const int64_t w = (int64_t)kt * TK + key;
            const bool in = w < a.Bk && c < d;
            ks[key][c] = in ? kbase[w * a.k_row_stride + c] : 0.f;
            vs[key][c] = in ? vbase[w * a.v_row_stride + c] : 0.f;
        }
        __syncthreads();
        float s[TK];
        float mt = -INFINITY;
        // Key-padding mask: bit j of the tile's validity word (TK = 64 keys).
        const uint64_t kw = a.kbits ? *(const uint64_t*)(a.kbits + pd.kb_off + 2 * kt) : ~0ull;
#pragma unroll
        for (int j = 0; j < TK; j++) {
            float acc = 0.f;
#pragma unroll
            for (int c = 0; c < DP; c++) acc = fmaf(q[c], ks[j][c], acc);
            acc *= a.scale;
            const int64_t w = (int64_t)kt * TK + j;
            const int64_t tk = pd.k_pos0 + w * a.pos_stride;
            bool ok = w < a.Bk && ((kw >> j) & 1);
            if (a.mask != kMaskNone) ok = ok && tk <= t;
            if (a.mask == kMaskDoc) ok = ok && tk >= ds;
            s[j] = ok ? acc : -INFINITY;
            mt = fmaxf(mt, s[j]);
        }
        const float mnew = fmaxf(m, mt);
        if (mnew != -INFINITY) {
            const float alpha = m == -INFINITY ? 0.f : expf(m - mnew);
            l *= alpha;
#pragma unroll
            for (int c = 0; c < DP; c++) o[c] *= alpha;
#pragma unroll
            for (int j = 0; j < TK; j++) {
                const float p = expf(s[j] - mnew);
                l += p;
#pragma unroll
                for (int c = 0; c < DP; c++) o[c] = fmaf(p, vs[j][c], o[c]);
            }
            m = mnew;
        }
        __syncthreads();
    }

    if (a.stats && head == 0 && lane == 0) {
        atomicAdd(&a.stats[0], (unsigned long long)(nkt - (kt_hi - kt_lo + 1)));
        atomicAdd(&a.stats[1], (unsigned long long)n_full);
        atomicAdd(&a.stats[2], (unsigned long long)n_part);
    }
    if (!row_ok) return;
    if (pd.finalize) {
        const float inv = l > 0.f ? 1.f / l : 0.f;
        float* op = (float*)a.out + pd.out_off + u * a.out_row_stride + head * a.out_head_stride;
#pragma unroll
        for (int c = 0; c < DP; c++)
            if (c < d) op[c] = o[c] * inv;
        if (a.lse)
            a.lse[pd.lse_off + head * a.lse_head_stride + u * a.lse_row_stride] =
                l > 0.f ? m + logf(l) : -INFINITY;
    } else if (!pd.load_state || kt_lo <= kt_hi) {
        float* Op = pd.O + srow * d;
#pragma unroll
        for (int c = 0; c < DP; c++)
            if (c < d) Op[c] = o[c];
        pd.m[srow] = m;
        pd.l[srow] = l;
    }
}

}  // namespace

hipError_t launch_step_f32(const StepArgs& a, hipStream_t stream) {
    const int64_t nwg = (int64_t)a.n_qtiles * a.Hq * a.n_pairs;
    if (nwg == 0) return hipSuccess;
    const dim3 grid((unsigned)nwg), block(64);
    if (a.d <= 4) step_f32_kernel<4><<<grid, block, 0, stream>>>(a);
    else if (a.d <= 16) step_f32_kernel<16><<<grid, block, 0, stream>>>(a);
    else if (a.d <= 32) step_f32_kernel<32><<<grid, block, 0, stream>>>(a);
    else if (a.d <= 64) step_f32_kernel<64><<<grid, block, 0, stream>>>(a);
    else if (a.d <= 128) step_f32_kernel<128><<<grid, block, 0, stream>>>(a);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace ra
