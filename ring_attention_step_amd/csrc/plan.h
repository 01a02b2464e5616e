// Ring planning: the ring schedule, exact mask classification of rectangles
// of (query, key) pairs, the per-step list of active block pairs, tallies and
// allowed-pair counts.  Plain C++ (no HIP).  doc_start and classify are
// constexpr, which HIP compiles for both host and device, so the kernels
// classify their tiles with the very same code the host plans with.
#pragma once
#include <cstdint>
#include <vector>

namespace ra {

enum Cls : int { kSkip = 0, kFull = 1, kPartial = 2 };
enum { kMaskNone = 0, kMaskCausal = 1, kMaskDoc = 2 };
enum { kLayoutContiguous = 0, kLayoutStriped = 1 };

// Start position of the document holding global position t (cu: n_docs + 1
// cumulative lengths from 0).  Binary search for the last cu[a] <= t.
constexpr int64_t doc_start(const int32_t* cu, int64_t n_docs, int64_t t) {
    int64_t lo = 0, hi = n_docs - 1;
    while (lo < hi) {
        int64_t mid = (lo + hi + 1) >> 1;
        if (cu[mid] <= t) lo = mid; else hi = mid - 1;
    }
    return cu[lo];
}

// Classification of every (query, key) pair with query positions in
// [t_min, t_max] and key positions in [tk_min, tk_max], both sides increasing
// with the local row index.  ds_min / ds_max are the document starts of t_min
// and t_max (doc-causal only; contiguous positions there).
//  causal: nothing allowed iff the smallest key is after the largest query;
//          everything allowed iff the largest key is not after the smallest query.
//  doc-causal: the keys allowed for some query form [doc_start(t_min), t_max]
//          (each key in it is allowed at least by the query at its own position
//          or by t_min), so nothing is allowed iff the key range misses it;
//          everything is allowed iff every key is <= t_min and >= the latest
//          document start, doc_start(t_max).
constexpr Cls classify(int mask, int64_t t_min, int64_t t_max, int64_t ds_min, int64_t ds_max,
                    int64_t tk_min, int64_t tk_max) {
    if (mask == kMaskNone) return kFull;
    if (mask == kMaskCausal) {
        if (tk_min > t_max) return kSkip;
        return tk_max <= t_min ? kFull : kPartial;
    }
    if (tk_max < ds_min || tk_min > t_max) return kSkip;
    return (ds_max <= tk_min && tk_max <= t_min) ? kFull : kPartial;
}

struct Ring {
    int64_t T = 0, N = 1, B = 0;
    int layout = kLayoutContiguous, mask = kMaskNone;
    int64_t passes = 1;            // min(max_ring_passes, N)
    const int32_t* cu = nullptr;   // host
    int64_t n_docs = 0;

    int64_t pos(int64_t blk, int64_t u) const { return layout == kLayoutStriped ? u * N + blk : blk * B + u; }
    int64_t ds(int64_t t) const { return mask == kMaskDoc ? doc_start(cu, n_docs, t) : 0; }
    // Rows [u0, u1] of block i against keys [w0, w1] of block j.
    Cls classify_rect(int64_t i, int64_t u0, int64_t u1, int64_t j, int64_t w0, int64_t w1) const {
        int64_t t0 = pos(i, u0), t1 = pos(i, u1);
        return classify(mask, t0, t1, ds(t0), ds(t1), pos(j, w0), pos(j, w1));
    }
};

struct StepPair {
    int32_t i = 0, j = 0;      // query block (virtual device) and key/value block
    bool load_state = false;   // an earlier step of device i already wrote state
    bool finalize = false;     // last active step of device i: write out / lse
};

struct Plan {
    std::vector<std::vector<StepPair>> steps;  // active (non-skipped) pairs per step
    std::vector<int32_t> empty_devices;        // devices with no active step (B == 0 only)
    int64_t visited = 0, skipped = 0, full = 0, partial = 0;
    int64_t tiles_in_skipped_pairs = 0;
};

// Ring schedule (device i holds block (i - s) mod N at step s), block-pair
// classification and the state hand-off flags.
Plan make_plan(const Ring& r, int tile_q, int tile_k);

// Tile classification counts {skipped, full, partial} over every visited
// block pair (host prediction of what the kernels count).
void tile_tallies(const Ring& r, int tile_q, int tile_k, int64_t counts[3]);

// (query, key) pairs per head that pass both the mask and the ring.
int64_t allowed_pairs(const Ring& r);

}  // namespace ra
