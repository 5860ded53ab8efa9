// Prints the launch plans of the library's host planner for the queries read from stdin, so
// that tests can check the planner's invariants without a GPU.
//   input lines:  split <pairs> <max_total> <unit> <max_len> <target> <unsplit_below>
//                 verify <dtype> <batch> <num_kv_heads> <max_kv_len>
//   output lines: <nsplit> <split_len>
#include <cstdio>
#include <cstring>

#include "plan.h"

int main() {
    char kind[16];
    while (std::scanf("%15s", kind) == 1) {
        kvss_plan::Plan p{};
        if (std::strcmp(kind, "split") == 0) {
            long pairs, total, max_len, target, unsplit;
            int unit;
            if (std::scanf("%ld %ld %d %ld %ld %ld", &pairs, &total, &unit, &max_len, &target,
                           &unsplit) != 6)
                return 2;
            p = kvss_plan::plan_splits(pairs, total, unit, max_len, target, unsplit);
        } else if (std::strcmp(kind, "verify") == 0) {
            kvss_kv kv{};
            if (std::scanf("%d %d %d %d", &kv.dtype, &kv.batch, &kv.num_kv_heads,
                           &kv.max_kv_len) != 4)
                return 2;
            p = kvss_plan::verify_plan(&kv);
        } else {
            return 2;
        }
        std::printf("%d %d\n", p.nsplit, p.split_len);
    }
    return 0;
}
