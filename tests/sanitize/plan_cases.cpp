// Host-only driver of the attention planning code (attn_plan.cpp), built with
// the address and undefined-behaviour sanitizers by tests/test_host_sanitizers.py.
// Reads one case per line on stdin and prints one result line per case:
//   V B H N M d scale dtype splits causal kv_len bias sb sh sn q k v o lse
//       -> "rc nothing kernel split splits tiles_per_split workspace_bytes"
//          (osa::plan_attn; pointers are numbers, never dereferenced)
//   P B H N M d dtype splits  -> "name splits"   (attn_fwd_plan; name "-" for NULL)
//   E code                    -> attn_strerror(code)
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "attn_plan.h"

static void *ptr(unsigned long long a) { return reinterpret_cast<void *>(static_cast<uintptr_t>(a)); }

int main() {
    char kind[4];
    while (scanf("%3s", kind) == 1) {
        if (strcmp(kind, "V") == 0) {
            long long B, H, N, M, sb, sh, sn;
            int d, dtype, splits, causal;
            float scale;
            unsigned long long kv, bias, q, k, v, o, lse;
            if (scanf("%lld %lld %lld %lld %d %f %d %d %d %llu %llu %lld %lld %lld %llu %llu %llu %llu %llu", &B, &H,
                      &N, &M, &d, &scale, &dtype, &splits, &causal, &kv, &bias, &sb, &sh, &sn, &q, &k, &v, &o,
                      &lse) != 19)
                return 2;
            attn_mask mask{causal, static_cast<const int32_t *>(ptr(kv)), static_cast<const float *>(ptr(bias)), sb,
                           sh, sn};
            osa::PlannedCall plan{};
            bool nothing = false;
            const int rc = osa::plan_attn(ptr(q), ptr(k), ptr(v), ptr(o), static_cast<float *>(ptr(lse)), B, H, N, M,
                                          d, scale, &mask, dtype, splits, &plan, &nothing);
            if (rc == ATTN_OK && !nothing)
                printf("%d 0 %s %d %d %d %zu\n", rc, osa::main_kernel_name(plan.kernel), plan.split ? 1 : 0,
                       plan.p.splits, plan.p.tiles_per_split, plan.workspace_bytes);
            else
                printf("%d %d - 0 0 0 0\n", rc, nothing ? 1 : 0);
        } else if (strcmp(kind, "P") == 0) {
            long long B, H, N, M;
            int d, dtype, splits;
            if (scanf("%lld %lld %lld %lld %d %d %d", &B, &H, &N, &M, &d, &dtype, &splits) != 7) return 2;
            int s = -1;
            const char *name = attn_fwd_plan(B, H, N, M, d, dtype, splits, &s);
            printf("%s %d\n", name ? name : "-", s);
        } else if (strcmp(kind, "E") == 0) {
            int code;
            if (scanf("%d", &code) != 1) return 2;
            printf("%s\n", attn_strerror(code));
        } else {
            return 2;
        }
    }
    return 0;
}
