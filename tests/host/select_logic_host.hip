// Host build of the selection kernels' per-thread logic (select_logic.hpp), driven the way the
// kernels drive it: a 512-thread workgroup emulated with sequential prefix sums.  Used only by
// tests/test_select_logic.py; compiled for the host, no device code runs.
#include <stdint.h>
#include <string.h>

#include <vector>

#include "select_logic.hpp"

namespace {
constexpr int kThreads = 512;
constexpr int kSlice = 8192;

// The threshold search of a workgroup over nbins = BPT * 512 bins: returns how many threads
// claimed the threshold (exactly one when 1 <= need <= total), with its bin and count above.
template <int BPT>
int threshold(const uint32_t *hist, uint32_t need, int *T, uint32_t *above) {
    uint32_t mine[kThreads];
    for (int t = 0; t < kThreads; t++) {
        mine[t] = 0;
        for (int i = 0; i < BPT; i++) mine[t] += hist[BPT * t + i];
    }
    int claims = 0;
    *T = -1;
    *above = 0;
    for (int t = 0; t < kThreads; t++) {
        uint32_t over = 0;  // held by threads above t
        for (int u = t + 1; u < kThreads; u++) over += mine[u];
        uint32_t c[BPT];
        for (int i = 0; i < BPT; i++) c[i] = hist[BPT * t + i];
        int b;
        uint32_t ab;
        if (v4a::sel_threshold_in_run<BPT>(c, over, need, &b, &ab)) {
            claims++;
            *T = BPT * t + b;
            *above = ab;
        }
    }
    return claims;
}
}  // namespace

extern "C" {

// Threshold of a 4096-bin histogram (8 bins per thread) or a 1024-bin one (2 per thread).
int sel_threshold_host(const uint32_t *hist, int nbins, uint32_t need, int *T, uint32_t *above) {
    if (nbins == 4096) return threshold<8>(hist, need, T, above);
    if (nbins == 1024) return threshold<2>(hist, need, T, above);
    return -1;
}

int sel_meta_consistent_host(int T, uint32_t above, uint32_t k_eff) { return v4a::sel_meta_consistent(T, above, k_eff); }

uint32_t sel_clamp_count_host(uint32_t c) { return v4a::sel_clamp_count(c, kSlice); }

// The whole selection of the k best of n 32-bit score keys, as the two kernels compose the
// steps: 12-bit bin threshold, the list of keys at or above it in index order, two 10-bit
// digit passes inside the bin, then the ordered compaction with each thread owning a
// contiguous run.  out[k] gets the ascending selection, -1 padded.  Returns 0, or -1 when a
// step found an inconsistency (the kernels then select nothing).
int sel_select_host(const uint32_t *keys, int64_t n, int k, int32_t *out) {
    for (int j = 0; j < k; j++) out[j] = -1;
    const uint32_t k_eff = (uint32_t)(n < k ? n : k);
    if (k_eff == 0) return 0;
    std::vector<uint32_t> h(4096, 0);
    for (int64_t i = 0; i < n; i++) h[keys[i] >> 20]++;
    int T;
    uint32_t above;
    if (threshold<8>(h.data(), k_eff, &T, &above) != 1) return -1;
    if (!v4a::sel_meta_consistent(T, above, k_eff)) return -1;
    std::vector<uint32_t> lidx, lkey;
    for (int64_t i = 0; i < n; i++)
        if ((int)(keys[i] >> 20) >= T) {
            lidx.push_back((uint32_t)i);
            lkey.push_back(keys[i]);
        }
    const uint32_t L = (uint32_t)lkey.size();
    uint32_t rem = k_eff - above, sub = 0, sub_mask = 0;
    for (int p = 0; p < 2; p++) {
        const int shift = p == 0 ? 10 : 0;
        std::vector<uint32_t> hs(1024, 0);
        for (uint32_t j = 0; j < L; j++)
            if ((int)(lkey[j] >> 20) == T && (lkey[j] & sub_mask) == sub) hs[(lkey[j] >> shift) & 1023u]++;
        int d;
        uint32_t ab;
        if (threshold<2>(hs.data(), rem, &d, &ab) != 1) return -1;
        rem -= ab;
        sub |= (uint32_t)d << shift;
        sub_mask |= 1023u << shift;
    }
    const uint32_t tkey = ((uint32_t)T << 20) | sub;
    const uint32_t per = (L + kThreads - 1) / kThreads;
    // exclusive prefix counts of keys above / equal to tkey over the threads' runs
    uint32_t gt_run = 0, eq_run = 0;
    for (int t = 0; t < kThreads; t++) {
        const uint32_t j0 = per * (uint32_t)t, j1 = j0 + per < L ? j0 + per : L;
        uint32_t gt_before = gt_run, eq_before = eq_run;
        for (uint32_t j = j0; j < j1; j++) {
            gt_run += lkey[j] > tkey;
            eq_run += lkey[j] == tkey;
        }
        for (uint32_t j = j0; j < j1; j++) {
            const int q = v4a::sel_place(lkey[j], tkey, rem, k_eff, &gt_before, &eq_before);
            if (q >= 0) out[q] = (int32_t)lidx[j];
        }
    }
    return 0;
}

}  // extern "C"
