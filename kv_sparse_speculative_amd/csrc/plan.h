// Launch planning of the attention and SnapKV passes: how a (sequence, KV head)'s key range is
// split over workgroups. Host code, shared by the entry points that size workspaces and launch.

#ifndef KVSS_PLAN_H
#define KVSS_PLAN_H

#include "kvss.h"

namespace kvss_plan {

inline long ceil_div(long a, long b) { return (a + b - 1) / b; }

// Workgroups a launch should offer: 256 compute units, a few resident workgroups each.
constexpr long kTargetWorkgroups = 1024;
// Draft launches: one round of resident workgroups (two per CU).
constexpr long kDraftTargetWorkgroups = 2 * 256;
// The SnapKV row-statistics pass keeps two (eight row tiles) or three (fewer) workgroups per
// CU resident: 3072 workgroups are whole rounds either way (six or four).
constexpr long kSnapTargetWorkgroups = 3 * 256 * 4;
constexpr int kMfmaUnit = 128;     // keys one bf16 attention workgroup consumes per round
constexpr int kSimpleUnit = 32;    // keys one fp32 attention workgroup consumes per round

struct Plan {
    int nsplit;
    int split_len;
};

// Split a virtual key range of up to max_total keys per (sequence, KV head) so that the
// launch offers about `target` workgroups, each doing at least eight rounds (a shorter split
// would not pay for the extra merge launch and partial traffic); a range shorter than
// `unsplit_below` keys is not split at all.
inline Plan plan_splits(long pairs, long max_total, int unit, long max_len = 1L << 30,
                 long target = kTargetWorkgroups, long unsplit_below = 0) {
    Plan p{1, unit};
    if (max_total <= 0 || pairs <= 0) return p;
    const long want = ceil_div(target, pairs);
    const long useful = max_total < unsplit_below ? 1 : ceil_div(max_total, 8L * unit);
    long ns = want < useful ? want : useful;
    if (ns < 1) ns = 1;
    if (ceil_div(max_total, ns) > max_len) ns = ceil_div(max_total, max_len);
    long len = ceil_div(ceil_div(max_total, ns), unit) * unit;
    if (len > max_len) len = max_len / unit * unit;
    p.split_len = (int)len;
    p.nsplit = (int)ceil_div(max_total, len);
    return p;
}

// bf16 verify: contexts under 16k keys are not split. Measured on the Llama-shaped layer (B
// 32-128, gamma 3-4): an 8k context runs fastest unsplit (no merge launch; whole-sequence
// workgroups already saturate HBM), while longer contexts gain from the regular plan.
constexpr long kVerifyUnsplitBelow = 16384;

inline Plan verify_plan(const kvss_kv* kv) {
    return kv->dtype == KVSS_BF16
               ? plan_splits((long)kv->batch * kv->num_kv_heads, kv->max_kv_len, kMfmaUnit,
                             1L << 30, kTargetWorkgroups, kVerifyUnsplitBelow)
               : plan_splits((long)kv->batch * kv->num_kv_heads, kv->max_kv_len, kSimpleUnit);
}

}  // namespace kvss_plan

#endif  // KVSS_PLAN_H
