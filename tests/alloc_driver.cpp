// Test driver (not part of the library): runs an allocator operation script read from
// stdin through the C ABI and prints every result, for the sanitizer build in
// tests/test_lib_host.py.
//   create N BS perm...      add S      append S n      batch k S1 n1 ... Sk nk
//   fork P C                 free S     table S max     dump
//   host NH                  swapout k S1 ... Sk        swapin k S1 ... Sk
//   prompt S k t1 ... tk     appendt S k t1 ... tk
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "pagedkv.h"

int main() {
    pa_allocator* a = nullptr;
    char op[32];
    while (std::scanf("%31s", op) == 1) {
        std::string o(op);
        int rc = 0;
        if (o == "create") {
            int n, bs;
            std::scanf("%d %d", &n, &bs);
            std::vector<int32_t> perm(n);
            for (int i = 0; i < n; ++i) std::scanf("%d", &perm[i]);
            rc = pa_alloc_create(n, bs, perm.data(), &a);
            std::printf("create %d\n", rc);
        } else if (o == "add") {
            long long s;
            std::scanf("%lld", &s);
            std::printf("add %d\n", pa_seq_add(a, s));
        } else if (o == "append") {
            long long s;
            int n;
            std::scanf("%lld %d", &s, &n);
            std::vector<int64_t> slots(n + 1);
            int64_t cow[2];
            int32_t ncow = 0;
            rc = pa_seq_append(a, s, n, slots.data(), cow, &ncow);
            std::printf("append %d", rc);
            if (rc == 0) {
                for (int i = 0; i < n; ++i) std::printf(" %lld", (long long)slots[i]);
                if (ncow) std::printf(" cow %lld %lld", (long long)cow[0], (long long)cow[1]);
            }
            std::printf("\n");
        } else if (o == "batch") {
            int k;
            std::scanf("%d", &k);
            std::vector<int64_t> ids(k);
            std::vector<int32_t> ns(k);
            int total = 0;
            for (int i = 0; i < k; ++i) {
                long long s;
                std::scanf("%lld %d", &s, &ns[i]);
                ids[i] = s;
                total += ns[i];
            }
            std::vector<int64_t> slots(total + 1), cow(2 * k + 2);
            int32_t ncow = 0;
            rc = pa_batch_append(a, ids.data(), ns.data(), k, slots.data(), cow.data(), &ncow);
            std::printf("batch %d", rc);
            if (rc == 0) {
                for (int i = 0; i < total; ++i) std::printf(" %lld", (long long)slots[i]);
                for (int i = 0; i < ncow; ++i) std::printf(" cow %lld %lld", (long long)cow[2 * i], (long long)cow[2 * i + 1]);
            }
            std::printf("\n");
        } else if (o == "fork") {
            long long p, c;
            std::scanf("%lld %lld", &p, &c);
            std::printf("fork %d\n", pa_seq_fork(a, p, c));
        } else if (o == "free") {
            long long s;
            std::scanf("%lld", &s);
            std::printf("free %d\n", pa_seq_free(a, s));
        } else if (o == "table") {
            long long s;
            int mb;
            std::scanf("%lld %d", &s, &mb);
            std::vector<int32_t> t(mb + 1);
            int32_t len = 0;
            int64_t id = s;
            rc = pa_block_tables(a, &id, 1, mb, t.data(), &len);
            std::printf("table %d", rc);
            if (rc == 0) {
                std::printf(" len %d", len);
                for (int i = 0; i < mb; ++i) std::printf(" %d", t[i]);
            }
            std::printf("\n");
        } else if (o == "host") {
            int nh;
            std::scanf("%d", &nh);
            std::printf("host %d\n", pa_alloc_set_host_blocks(a, nh));
        } else if (o == "swapout" || o == "swapin") {
            int k;
            std::scanf("%d", &k);
            std::vector<int64_t> ids(k);
            for (int i = 0; i < k; ++i) {
                long long s;
                std::scanf("%lld", &s);
                ids[i] = s;
            }
            const int maxp = 64;
            std::vector<int64_t> pairs(2 * maxp);
            int32_t np = 0;
            rc = (o == "swapout" ? pa_swap_out : pa_swap_in)(a, ids.data(), k, pairs.data(), maxp, &np);
            std::printf("%s %d", op, rc);
            if (rc == 0)
                for (int i = 0; i < np; ++i) std::printf(" %lld:%lld", (long long)pairs[2 * i], (long long)pairs[2 * i + 1]);
            std::printf("\n");
        } else if (o == "prompt" || o == "appendt") {
            long long s;
            int k;
            std::scanf("%lld %d", &s, &k);
            std::vector<int32_t> toks(k + 1);
            for (int i = 0; i < k; ++i) std::scanf("%d", &toks[i]);
            std::vector<int64_t> slots(k + 1);
            int32_t nc = 0, ncow = 0;
            int64_t cow[2];
            if (o == "prompt") rc = pa_seq_add_prompt(a, s, toks.data(), k, &nc, slots.data());
            else rc = pa_seq_append_tokens(a, s, toks.data(), k, slots.data(), cow, &ncow);
            std::printf("%s %d", op, rc);
            if (rc == 0) {
                const int ns = o == "prompt" ? k - nc : k;
                std::printf(" cached %d", nc);
                for (int i = 0; i < ns; ++i) std::printf(" %lld", (long long)slots[i]);
            }
            std::printf("\n");
        } else if (o == "dump") {
            pa_alloc_stats_t st;
            pa_alloc_stats(a, &st);
            std::printf("stats %lld %lld %lld %lld %lld %lld %lld %lld %lld %lld %lld %lld\n", (long long)st.free_blocks,
                        (long long)st.used_blocks, (long long)st.total_refs, (long long)st.exhaustion_events,
                        (long long)st.waste_slots, (long long)st.num_seqs, (long long)st.host_free_blocks,
                        (long long)st.host_used_blocks, (long long)st.swapped_seqs, (long long)st.cached_blocks,
                        (long long)st.cache_hit_blocks, (long long)st.cache_evictions);
        }
    }
    pa_alloc_destroy(a);
    return 0;
}
