/* Plain C consumer of include/kvss.h: compiles the header as C99, links libkvss.so and calls
 * entry points that return before any HIP call (version, workspace queries, argument
 * validation). Prints one line per check; exit status 0 when all pass. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "kvss.h"

static int failures = 0;

static void check(int cond, const char* what) {
    printf("%s %s\n", cond ? "ok" : "FAIL", what);
    if (!cond) ++failures;
}

int main(void) {
    static char fake[256];
    kvss_kv kv;
    memset(&kv, 0, sizeof(kv));
    kv.k = fake;
    kv.v = fake;
    kv.block_table = (const int32_t*)fake;
    kv.kv_lens = (const int32_t*)fake;
    kv.batch = 2;
    kv.num_kv_heads = 2;
    kv.head_dim = 128;
    kv.block_size = 16;
    kv.max_blocks = 4;
    kv.num_blocks = 8;
    kv.max_kv_len = 64;
    kv.dtype = KVSS_BF16;

    check(kvss_version() == 1, "kvss_version");
    check(kvss_verify_workspace_bytes(&kv, 8, 5) < ((size_t)1 << 30), "verify workspace query");
    check(kvss_snapkv_workspace_bytes(&kv, 8, 16, 64) > 0, "snapkv workspace query");
    check(kvss_accept_workspace_bytes(4, 3, 100) > 0, "accept workspace query");
    check(kvss_sample_workspace_bytes(4, 1000) > 0, "sample workspace query");

    kv.head_dim = 96;
    check(verify_attn_full(&kv, fake, 8, 5, 0.1f, (float*)fake, NULL, NULL, 0, NULL) ==
              KVSS_EUNSUPPORTED, "head_dim 96 is refused");
    check(strlen(kvss_last_error()) > 0, "error message is set");
    kv.head_dim = 128;
    check(verify_attn_full(&kv, fake, 7, 5, 0.1f, (float*)fake, NULL, NULL, 0, NULL) ==
              KVSS_EINVAL, "num_q_heads not a multiple of num_kv_heads");
    check(spec_accept(NULL, NULL, NULL, 4, 3, 100, 1.0f, 1, 0, NULL, NULL, NULL, NULL, 0, NULL) ==
              KVSS_EINVAL, "spec_accept with NULL logits");
    check(draft_sample((const float*)fake, 2, 10, -1.0f, 1, 2, 0, (int32_t*)fake, NULL, fake,
                       1 << 20, NULL) == KVSS_EINVAL, "negative temperature");
    kv.batch = 0;
    check(verify_attn_full(&kv, NULL, 8, 5, 0.1f, NULL, NULL, NULL, 0, NULL) == KVSS_OK,
          "empty batch is a no-op");
    return failures == 0 ? 0 : 1;
}
