#include "plan.h"

#include <algorithm>

namespace ra {

Plan make_plan(const Ring& r, int tile_q, int tile_k) {
    Plan p;
    p.steps.assign(r.passes, {});
    const int64_t nqt = (r.B + tile_q - 1) / tile_q, nkt = (r.B + tile_k - 1) / tile_k;
    std::vector<int> first(r.N, -1), last(r.N, -1);
    std::vector<std::vector<Cls>> cls(r.passes, std::vector<Cls>(r.N, kSkip));
    for (int64_t s = 0; s < r.passes; s++) {
        for (int64_t i = 0; i < r.N; i++) {
            int64_t j = ((i - s) % r.N + r.N) % r.N;
            Cls c = r.B > 0 ? r.classify_rect(i, 0, r.B - 1, j, 0, r.B - 1) : kSkip;
            cls[s][i] = c;
            p.visited++;
            if (c == kSkip) {
                p.skipped++;
                p.tiles_in_skipped_pairs += nqt * nkt;
                continue;
            }
            (c == kFull ? p.full : p.partial)++;
            if (first[i] < 0) first[i] = (int)s;
            last[i] = (int)s;
        }
    }
    for (int64_t s = 0; s < r.passes; s++) {
        for (int64_t i = 0; i < r.N; i++) {
            if (cls[s][i] == kSkip) continue;
            StepPair sp;
            sp.i = (int32_t)i;
            sp.j = (int32_t)(((i - s) % r.N + r.N) % r.N);
            sp.load_state = first[i] != (int)s;
            sp.finalize = last[i] == (int)s;
            p.steps[s].push_back(sp);
        }
    }
    for (int64_t i = 0; i < r.N; i++)
        if (first[i] < 0) p.empty_devices.push_back((int32_t)i);
    return p;
}

void tile_tallies(const Ring& r, int tile_q, int tile_k, int64_t counts[3]) {
    counts[0] = counts[1] = counts[2] = 0;
    const int64_t nqt = (r.B + tile_q - 1) / tile_q, nkt = (r.B + tile_k - 1) / tile_k;
    for (int64_t s = 0; s < r.passes; s++) {
        for (int64_t i = 0; i < r.N; i++) {
            int64_t j = ((i - s) % r.N + r.N) % r.N;
            for (int64_t a = 0; a < nqt; a++) {
                int64_t u0 = a * tile_q, u1 = std::min(r.B, u0 + tile_q) - 1;
                for (int64_t b = 0; b < nkt; b++) {
                    int64_t w0 = b * tile_k, w1 = std::min(r.B, w0 + tile_k) - 1;
                    counts[r.classify_rect(i, u0, u1, j, w0, w1)]++;
                }
            }
        }
    }
}

int64_t allowed_pairs(const Ring& r) {
    int64_t total = 0;
    for (int64_t i = 0; i < r.N; i++) {
        for (int64_t u = 0; u < r.B; u++) {
            const int64_t t = r.pos(i, u);
            // keys allowed by the mask form the interval [lo, hi] of positions
            int64_t lo = 0, hi = r.T - 1;
            if (r.mask != kMaskNone) hi = t;
            if (r.mask == kMaskDoc) lo = r.ds(t);
            for (int64_t s = 0; s < r.passes; s++) {
                int64_t j = ((i - s) % r.N + r.N) % r.N;
                // keys of block j inside [lo, hi]: local indices w with lo <= pos(j, w) <= hi
                int64_t w_lo, w_hi;
                if (r.layout == kLayoutStriped) {
                    // pos = w * N + j
                    w_lo = lo - j <= 0 ? 0 : (lo - j + r.N - 1) / r.N;
                    w_hi = hi - j < 0 ? -1 : (hi - j) / r.N;
                } else {
                    w_lo = lo - j * r.B;
                    w_hi = hi - j * r.B;
                }
                w_lo = std::max<int64_t>(w_lo, 0);
                w_hi = std::min<int64_t>(w_hi, r.B - 1);
                if (w_hi >= w_lo) total += w_hi - w_lo + 1;
            }
        }
    }
    return total;
}

}  // namespace ra
