// Host block allocator of the paged KV cache (CPU only; never touches the device).
//
// Rules ("KV Cache Management", "The Solution: PagedAttention (vLLM)" and "The Bonus:
// Zero-Copy Sharing"; "PagedAttention: Optimizing KV Cache Utilization in Large Language
// Models", "The Mechanics of PagedAttention" and "Conclusion"; "KV Cache Optimization and
// PagedAttention", prose on paging and copy-on-write):
//  - the pool is a FIFO queue of free physical blocks; a grant pops the head, a release
//    pushes to the tail, so allocation order is deterministic given the initial order;
//  - a sequence takes a new block only when its last block is full (on-demand);
//  - fork shares every block of the parent (reference count + 1);
//  - appending into a shared, partially filled last block first moves the sequence to a
//    fresh block (copy-on-write) and reports the pair for the device copy;
//  - every operation is all-or-nothing: on failure no state changes.
//
// Storage: refcounts and the free queue are flat int32 arrays of num_blocks entries (the
// queue is a ring: it never holds more than num_blocks ids); each sequence keeps its block
// list in a vector, so a table export is a memcpy per sequence.

#include <algorithm>
#include <cstdint>
#include <cstring>
#include <new>
#include <unordered_map>
#include <vector>

#include "pa_error.h"
#include "../../include/pagedkv.h"

using pagedkv::fail;

namespace {

struct Seq {
    std::vector<int32_t> blocks;
    int64_t n = 0;  // tokens held
};

}  // namespace

struct pa_allocator {
    int32_t num_blocks = 0;
    int32_t block_size = 0;
    std::vector<int32_t> refcount;
    std::vector<int32_t> ring;   // free queue storage
    int64_t head = 0;            // index of the queue head in `ring`
    int64_t count = 0;           // ids in the queue
    std::unordered_map<int64_t, Seq> seqs;
    int64_t exhaustion_events = 0;

    int32_t pop() {
        int32_t b = ring[head];
        head = (head + 1) % num_blocks;
        --count;
        return b;
    }
    void push(int32_t b) {
        ring[(head + count) % num_blocks] = b;
        ++count;
    }
    // Blocks one append of n tokens to `s` would take, given `extra_drop` references that
    // earlier appends in the same batch already moved off s's last block.
    int64_t blocks_needed(const Seq& s, int64_t n, int32_t extra_drop) const {
        if (n <= 0) return 0;
        const int64_t bs = block_size;
        int64_t need = 0;
        if (s.n % bs != 0 && refcount[s.blocks.back()] - extra_drop > 1) need += 1;  // COW
        // tokens at positions s.n .. s.n+n-1 that start a block
        int64_t first = (s.n + bs - 1) / bs;         // first block index starting at >= s.n
        int64_t last = (s.n + n - 1) / bs;           // block index of the last token
        if (last >= first) need += last - first + 1;
        return need;
    }
    // Performs an append already known to fit.  Returns the number of COW pairs (0 or 1).
    int append_fit(Seq& s, int64_t n, int64_t* slots, int64_t* cow) {
        const int64_t bs = block_size;
        int ncow = 0;
        for (int64_t t = 0; t < n; ++t) {
            if (s.n % bs == 0) {
                int32_t b = pop();
                refcount[b] = 1;
                s.blocks.push_back(b);
            } else if (refcount[s.blocks.back()] > 1) {
                int32_t old = s.blocks.back();
                int32_t fresh = pop();
                refcount[old] -= 1;
                refcount[fresh] = 1;
                s.blocks.back() = fresh;
                cow[0] = old;
                cow[1] = fresh;
                ncow = 1;
            }
            slots[t] = static_cast<int64_t>(s.blocks.back()) * bs + s.n % bs;
            s.n += 1;
        }
        return ncow;
    }
};

extern "C" {

int pa_alloc_create(int32_t num_blocks, int32_t block_size, const int32_t* initial_free_order,
                    pa_allocator** out) {
    pagedkv::clear_error();
    if (!out) return fail(PA_ERR_INVALID, "pa_alloc_create: out is NULL");
    *out = nullptr;
    if (num_blocks <= 0 || block_size <= 0)
        return fail(PA_ERR_INVALID, "pa_alloc_create: num_blocks=%d block_size=%d must be > 0",
                    num_blocks, block_size);
    pa_allocator* a = new (std::nothrow) pa_allocator();
    if (!a) return fail(PA_ERR_INVALID, "pa_alloc_create: out of host memory");
    a->num_blocks = num_blocks;
    a->block_size = block_size;
    a->refcount.assign(num_blocks, 0);
    a->ring.resize(num_blocks);
    if (initial_free_order) {
        std::vector<char> seen(num_blocks, 0);
        for (int32_t i = 0; i < num_blocks; ++i) {
            int32_t b = initial_free_order[i];
            if (b < 0 || b >= num_blocks || seen[b]) {
                delete a;
                return fail(PA_ERR_INVALID,
                            "pa_alloc_create: initial_free_order is not a permutation (entry %d = %d)",
                            i, b);
            }
            seen[b] = 1;
            a->ring[i] = b;
        }
    } else {
        for (int32_t i = 0; i < num_blocks; ++i) a->ring[i] = i;
    }
    a->head = 0;
    a->count = num_blocks;
    *out = a;
    return PA_OK;
}

void pa_alloc_destroy(pa_allocator* a) { delete a; }

int pa_seq_add(pa_allocator* a, int64_t seq_id) {
    pagedkv::clear_error();
    if (!a) return fail(PA_ERR_INVALID, "pa_seq_add: NULL allocator");
    if (a->seqs.count(seq_id)) return fail(PA_ERR_INVALID, "pa_seq_add: sequence %lld exists", (long long)seq_id);
    a->seqs.emplace(seq_id, Seq());
    return PA_OK;
}

int pa_seq_append(pa_allocator* a, int64_t seq_id, int32_t n_tokens, int64_t* slots_out,
                  int64_t* cow_out, int32_t* n_cow_out) {
    pagedkv::clear_error();
    if (!a) return fail(PA_ERR_INVALID, "pa_seq_append: NULL allocator");
    if (n_tokens < 0) return fail(PA_ERR_INVALID, "pa_seq_append: n_tokens=%d < 0", n_tokens);
    if (n_tokens > 0 && !slots_out) return fail(PA_ERR_INVALID, "pa_seq_append: slots_out is NULL");
    if (!cow_out || !n_cow_out) return fail(PA_ERR_INVALID, "pa_seq_append: cow_out/n_cow_out is NULL");
    auto it = a->seqs.find(seq_id);
    if (it == a->seqs.end()) return fail(PA_ERR_INVALID, "pa_seq_append: unknown sequence %lld", (long long)seq_id);
    Seq& s = it->second;
    int64_t need = a->blocks_needed(s, n_tokens, 0);
    if (need > a->count) {
        a->exhaustion_events += 1;
        return fail(PA_ERR_NO_BLOCKS, "pa_seq_append: sequence %lld needs %lld blocks, %lld free",
                    (long long)seq_id, (long long)need, (long long)a->count);
    }
    *n_cow_out = a->append_fit(s, n_tokens, slots_out, cow_out);
    return PA_OK;
}

int pa_batch_append(pa_allocator* a, const int64_t* seq_ids, const int32_t* n_tokens,
                    int32_t n_seqs, int64_t* slots_out, int64_t* cow_out, int32_t* n_cow_out) {
    pagedkv::clear_error();
    if (!a) return fail(PA_ERR_INVALID, "pa_batch_append: NULL allocator");
    if (n_seqs < 0) return fail(PA_ERR_INVALID, "pa_batch_append: n_seqs=%d < 0", n_seqs);
    if (n_seqs > 0 && (!seq_ids || !n_tokens || !slots_out || !cow_out))
        return fail(PA_ERR_INVALID, "pa_batch_append: NULL array");
    if (!n_cow_out) return fail(PA_ERR_INVALID, "pa_batch_append: n_cow_out is NULL");
    // validate ids, distinctness and counts; find the blocks the whole batch needs, taking
    // into account that a copy-on-write by an earlier sequence drops a reference that a
    // later sequence sharing the same last block would otherwise have counted
    std::vector<Seq*> ss(n_seqs);
    std::unordered_map<int32_t, int32_t> dropped;  // last-block id -> references moved off
    std::unordered_map<int64_t, char> ids;
    int64_t need = 0;
    for (int32_t i = 0; i < n_seqs; ++i) {
        if (n_tokens[i] < 0) return fail(PA_ERR_INVALID, "pa_batch_append: n_tokens[%d] < 0", i);
        auto it = a->seqs.find(seq_ids[i]);
        if (it == a->seqs.end())
            return fail(PA_ERR_INVALID, "pa_batch_append: unknown sequence %lld", (long long)seq_ids[i]);
        if (!ids.emplace(seq_ids[i], 1).second)
            return fail(PA_ERR_INVALID, "pa_batch_append: sequence %lld listed twice", (long long)seq_ids[i]);
        Seq& s = it->second;
        ss[i] = &s;
        int32_t drop = 0;
        if (n_tokens[i] > 0 && s.n % a->block_size != 0) {
            auto d = dropped.find(s.blocks.back());
            drop = d == dropped.end() ? 0 : d->second;
            if (a->refcount[s.blocks.back()] - drop > 1) dropped[s.blocks.back()] = drop + 1;
        }
        need += a->blocks_needed(s, n_tokens[i], drop);
    }
    if (need > a->count) {
        a->exhaustion_events += 1;
        return fail(PA_ERR_NO_BLOCKS, "pa_batch_append: batch needs %lld blocks, %lld free",
                    (long long)need, (long long)a->count);
    }
    int64_t off = 0;
    int32_t ncow = 0;
    for (int32_t i = 0; i < n_seqs; ++i) {
        ncow += a->append_fit(*ss[i], n_tokens[i], slots_out + off, cow_out + 2 * ncow);
        off += n_tokens[i];
    }
    *n_cow_out = ncow;
    return PA_OK;
}

int pa_seq_fork(pa_allocator* a, int64_t parent, int64_t child) {
    pagedkv::clear_error();
    if (!a) return fail(PA_ERR_INVALID, "pa_seq_fork: NULL allocator");
    auto it = a->seqs.find(parent);
    if (it == a->seqs.end()) return fail(PA_ERR_INVALID, "pa_seq_fork: unknown parent %lld", (long long)parent);
    if (a->seqs.count(child)) return fail(PA_ERR_INVALID, "pa_seq_fork: child %lld exists", (long long)child);
    Seq c = it->second;  // copy of the block list and token count
    for (int32_t b : c.blocks) a->refcount[b] += 1;
    a->seqs.emplace(child, std::move(c));
    return PA_OK;
}

int pa_seq_free(pa_allocator* a, int64_t seq_id) {
    pagedkv::clear_error();
    if (!a) return fail(PA_ERR_INVALID, "pa_seq_free: NULL allocator");
    auto it = a->seqs.find(seq_id);
    if (it == a->seqs.end()) return fail(PA_ERR_INVALID, "pa_seq_free: unknown sequence %lld", (long long)seq_id);
    for (int32_t b : it->second.blocks) {
        if (--a->refcount[b] == 0) a->push(b);
    }
    a->seqs.erase(it);
    return PA_OK;
}

int pa_block_tables(const pa_allocator* a, const int64_t* seq_ids, int32_t n_seqs,
                    int32_t max_blocks, int32_t* tables_out, int32_t* seq_lens_out) {
    pagedkv::clear_error();
    if (!a) return fail(PA_ERR_INVALID, "pa_block_tables: NULL allocator");
    if (n_seqs < 0 || max_blocks < 0) return fail(PA_ERR_INVALID, "pa_block_tables: negative size");
    if (n_seqs > 0 && (!seq_ids || !seq_lens_out || (max_blocks > 0 && !tables_out)))
        return fail(PA_ERR_INVALID, "pa_block_tables: NULL array");
    std::vector<const Seq*> ss(n_seqs);
    for (int32_t i = 0; i < n_seqs; ++i) {
        auto it = a->seqs.find(seq_ids[i]);
        if (it == a->seqs.end())
            return fail(PA_ERR_INVALID, "pa_block_tables: unknown sequence %lld", (long long)seq_ids[i]);
        if ((int64_t)it->second.blocks.size() > max_blocks)
            return fail(PA_ERR_INVALID, "pa_block_tables: sequence %lld holds %zu blocks > max_blocks %d",
                        (long long)seq_ids[i], it->second.blocks.size(), max_blocks);
        if (it->second.n > INT32_MAX)
            return fail(PA_ERR_INVALID, "pa_block_tables: sequence %lld length exceeds int32", (long long)seq_ids[i]);
        ss[i] = &it->second;
    }
    for (int32_t i = 0; i < n_seqs; ++i) {
        int32_t* row = tables_out + (int64_t)i * max_blocks;
        const auto& bl = ss[i]->blocks;
        if (!bl.empty()) std::memcpy(row, bl.data(), bl.size() * sizeof(int32_t));
        std::fill(row + bl.size(), row + max_blocks, -1);
        seq_lens_out[i] = static_cast<int32_t>(ss[i]->n);
    }
    return PA_OK;
}

int pa_alloc_stats(const pa_allocator* a, pa_alloc_stats_t* out) {
    pagedkv::clear_error();
    if (!a || !out) return fail(PA_ERR_INVALID, "pa_alloc_stats: NULL argument");
    int64_t used = 0, refs = 0;
    for (int32_t r : a->refcount) {
        used += r > 0;
        refs += r;
    }
    int64_t waste = 0;
    const int64_t bs = a->block_size;
    for (const auto& kv : a->seqs) waste += (kv.second.n + bs - 1) / bs * bs - kv.second.n;
    out->free_blocks = a->count;
    out->used_blocks = used;
    out->total_refs = refs;
    out->exhaustion_events = a->exhaustion_events;
    out->waste_slots = waste;
    out->num_seqs = static_cast<int64_t>(a->seqs.size());
    return PA_OK;
}

int pa_alloc_dump(const pa_allocator* a, int32_t* refcounts, int32_t* free_order, int32_t* n_free) {
    pagedkv::clear_error();
    if (!a || !refcounts || !free_order || !n_free) return fail(PA_ERR_INVALID, "pa_alloc_dump: NULL argument");
    std::memcpy(refcounts, a->refcount.data(), a->refcount.size() * sizeof(int32_t));
    for (int64_t i = 0; i < a->count; ++i) free_order[i] = a->ring[(a->head + i) % a->num_blocks];
    *n_free = static_cast<int32_t>(a->count);
    return PA_OK;
}

}  // extern "C"
