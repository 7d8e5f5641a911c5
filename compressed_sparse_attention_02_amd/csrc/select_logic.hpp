// select_logic.hpp -- the per-thread steps of the radix top-k selection: the threshold search
// inside one thread's histogram bins, the consistency checks the final selection applies to
// what the scan left, and the ordered compaction's placement rule.  The selection kernels
// (topk.hip) call these; a host build of the same header drives them in a unit test that
// emulates a workgroup with sequential prefix sums.
//
// Order: larger score key first, then lower index ("DeepSeek-V4 technical report walkthrough"
// (cyqw.cn), section 2.2: each query keeps its top-k entries; the tie rule is this library's).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace v4a {

// Threshold search of one thread owning bins BPT*t .. BPT*t+BPT-1 (counts c[], ascending bin
// order), with `over` keys in the bins of all higher threads.  Walking down from the top bin,
// the threshold bin is the one where the running count first reaches `need`.  Returns true,
// with the bin's index inside this thread's run (*b) and the count strictly above it (*above),
// iff that bin is one of this thread's.  Exactly one thread returns true when
// 1 <= need <= total, none otherwise.
template <int BPT>
__host__ __device__ __forceinline__ bool sel_threshold_in_run(const uint32_t (&c)[BPT], uint32_t over, uint32_t need,
                                                             int *b, uint32_t *above) {
    uint32_t mine = 0;
#pragma unroll
    for (int i = 0; i < BPT; i++) mine += c[i];
    if (!(over < need && need <= over + mine)) return false;
    uint32_t run = over;
    bool found = false;
#pragma unroll
    for (int i = BPT - 1; i >= 0; i--) {
        if (!found && run < need && need <= run + c[i]) {
            *b = i;
            *above = run;
            found = true;
        }
        run += c[i];
    }
    return found;
}

// The scan's result as the final selection reads it back: threshold bin T and the count of
// keys strictly above it.  Consistent iff a bin was found and fewer than k_eff keys lie above
// it (so at least one key of bin T is still needed).  An inconsistent result selects nothing.
__host__ __device__ __forceinline__ bool sel_meta_consistent(int T, uint32_t above, uint32_t k_eff) {
    return T >= 0 && above < k_eff;
}

// A slice's listed-key count as the final selection trusts it: never more than the slice's list
// region holds, so no read leaves it.
__host__ __device__ __forceinline__ uint32_t sel_clamp_count(uint32_t c, uint32_t slice_cap) {
    return c < slice_cap ? c : slice_cap;
}

// Ordered compaction: walking the listed keys in index order with gt_before keys above the
// threshold key tkey and eq_before keys equal to it already seen, returns the output slot of a
// key (keys above tkey are all kept; keys equal to it while fewer than rem have been kept,
// lowest index first), or -1 if it is not kept; advances the counts.  Both counts are read
// and written back unconditionally: a store through a pointer chosen by the comparison would
// keep them in memory (scratch on the GPU) instead of registers.
__host__ __device__ __forceinline__ int sel_place(uint32_t key, uint32_t tkey, uint32_t rem, uint32_t k_eff,
                                                  uint32_t *gt_before, uint32_t *eq_before) {
    const uint32_t g = *gt_before, e = *eq_before;
    const bool gt = key > tkey, eq = key == tkey;
    int p = -1;
    if (gt) {
        const uint32_t q = g + (e < rem ? e : rem);
        if (q < k_eff) p = (int)q;
    } else if (eq) {
        const uint32_t q = g + e;
        if (e < rem && q < k_eff) p = (int)q;
    }
    *gt_before = g + (gt ? 1u : 0u);
    *eq_before = e + (eq ? 1u : 0u);
    return p;
}

}  // namespace v4a
