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
//  - every operation is all-or-nothing: on failure no state changes;
//  - preemption by swapping ("PagedAttention: Optimizing KV Cache Utilization in Large
//    Language Models", "Conclusion": a request may be preempted and its KV cache swapped):
//    a second pool of host blocks (its own FIFO queue and refcounts) receives the blocks of
//    swapped-out sequences.  Swap-out walks the listed sequences' blocks in logical order,
//    gives each distinct device block one host block (pair reported for the copy), moves every
//    reference to the host block and releases the device references as a free would; swap-in
//    is the mirror image.  A device block also held by a sequence that stays resident keeps
//    that holder and is copied, so the swapped set and the resident one stop sharing it;
//  - prefix caching ("KV Cache Management", "The Bonus: Zero-Copy Sharing": a system prompt
//    shared by many users is computed and stored once and every user's table points at that
//    block; "KV Cache Optimization and PagedAttention", first paragraph: prefix caching):
//    a full block whose token ids are known is registered under its content, the whole token
//    prefix up to its end.  A new sequence added with its prompt takes, from block 0 on, every
//    registered block whose content equals its own prefix and stops at the first miss; the
//    caller computes and writes K/V only from there.  A registered block whose refcount drops
//    to 0 stays registered in the free queue until the queue hands it out again (then its
//    registration is dropped: eviction in release order); a hit takes it out of the queue.
//
// Storage: refcounts are a flat int32 array; the device free queue is an intrusive doubly
// linked list over block ids (FIFO, and a hit removes a block from its middle in O(1)); the
// host pool's queue is a ring.  Each sequence keeps its block list in a vector, so a table
// export is a memcpy per sequence.  Block contents are interned: a node stands for a token
// prefix ending at a block boundary, keyed exactly by (node of the prefix one block shorter,
// the block's token ids) in a hash table; nodes live while a block, a longer prefix or a
// sequence refers to them.

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
    std::vector<int32_t> blocks;  // device block ids, or host block ids while swapped out
    int64_t n = 0;                // tokens held
    bool swapped = false;
    bool tracked = true;          // the token id of every token held is known
    int64_t chain = -1;           // content node of the last full block (-1: none)
    std::vector<int32_t> partial; // token ids in the partially filled last block (tracked only)
};

// The device pool's FIFO free queue with O(1) removal of any member: an intrusive doubly
// linked list over block ids.
struct FreeList {
    std::vector<int32_t> nxt, prv;
    int32_t head = -1, tail = -1;
    int64_t count = 0;
    void init(int32_t n) {
        nxt.assign(n, -1);
        prv.assign(n, -1);
        head = tail = -1;
        count = 0;
    }
    void push(int32_t b) {
        prv[b] = tail;
        nxt[b] = -1;
        if (tail >= 0) nxt[tail] = b; else head = b;
        tail = b;
        ++count;
    }
    void remove(int32_t b) {
        const int32_t p = prv[b], q = nxt[b];
        if (p >= 0) nxt[p] = q; else head = q;
        if (q >= 0) prv[q] = p; else tail = p;
        --count;
    }
    int32_t pop() {
        const int32_t b = head;
        remove(b);
        return b;
    }
};

// Content of a full block: the node of the token prefix one block shorter (-1 for the first
// block) and the block's own token ids.  Compared exactly; the hash (FNV-1a, 64 bit, over the
// parent id's 8 bytes and each token id's 4 bytes, little end first) only indexes the table.
struct BlockKey {
    int64_t parent;
    std::vector<int32_t> tokens;
    bool operator==(const BlockKey& o) const { return parent == o.parent && tokens == o.tokens; }
};

struct BlockKeyHash {
    size_t operator()(const BlockKey& k) const {
        uint64_t h = 14695981039346656037ull;
        auto mix = [&h](uint64_t v, int bytes) {
            for (int i = 0; i < bytes; ++i) {
                h ^= (v >> (8 * i)) & 0xffu;
                h *= 1099511628211ull;
            }
        };
        mix(static_cast<uint64_t>(k.parent), 8);
        for (int32_t t : k.tokens) mix(static_cast<uint32_t>(t), 4);
        return static_cast<size_t>(h);
    }
};

struct Node {
    BlockKey key;
    int32_t block = -1;   // the registered device block holding this content, or -1
    int64_t refs = 0;     // longer prefixes + sequences ending a full block here + (block >= 0)
};

// A FIFO queue of free block ids over a ring of capacity `cap` (it never holds more).
struct FreeQueue {
    std::vector<int32_t> ring;
    int64_t head = 0, count = 0;
    void reset(int32_t cap) {
        ring.resize(cap);
        for (int32_t i = 0; i < cap; ++i) ring[i] = i;
        head = 0;
        count = cap;
    }
    int32_t pop() {
        const int32_t b = ring[head];
        head = (head + 1) % static_cast<int64_t>(ring.size());
        --count;
        return b;
    }
    void push(int32_t b) {
        ring[(head + count) % static_cast<int64_t>(ring.size())] = b;
        ++count;
    }
};

}  // namespace

struct pa_allocator {
    int32_t num_blocks = 0;
    int32_t block_size = 0;
    std::vector<int32_t> refcount;
    FreeList freeq;
    std::unordered_map<int64_t, Seq> seqs;
    int64_t exhaustion_events = 0;
    std::vector<int32_t> host_refcount;   // host pool (empty until pa_alloc_set_host_blocks)
    FreeQueue host_free;
    int64_t swapped_seqs = 0;
    // prefix cache
    std::unordered_map<BlockKey, int64_t, BlockKeyHash> node_of_key;
    std::unordered_map<int64_t, Node> nodes;
    std::vector<int64_t> node_of_block;   // device block -> the node it is registered under, or -1
    int64_t next_node = 0;
    int64_t cached_blocks = 0, cache_hit_blocks = 0, cache_evictions = 0;

    // Drops one reference of a node; a node left without references is deleted, which drops
    // its reference on the prefix one block shorter, and so on.
    void unref(int64_t id) {
        while (id >= 0) {
            auto it = nodes.find(id);
            if (--it->second.refs > 0) return;
            const int64_t parent = it->second.key.parent;
            node_of_key.erase(it->second.key);
            nodes.erase(it);
            id = parent;
        }
    }
    // The node of (parent, tokens), created without references if new.
    int64_t intern(int64_t parent, const std::vector<int32_t>& tokens) {
        BlockKey k{parent, tokens};
        auto it = node_of_key.find(k);
        if (it != node_of_key.end()) return it->second;
        const int64_t id = next_node++;
        nodes.emplace(id, Node{k, -1, 0});
        node_of_key.emplace(std::move(k), id);
        if (parent >= 0) nodes.find(parent)->second.refs += 1;
        return id;
    }
    // Hands out the free queue's head; a registered block loses its registration.
    int32_t pop() {
        const int32_t b = freeq.pop();
        const int64_t id = node_of_block[b];
        if (id >= 0) {
            node_of_block[b] = -1;
            nodes.find(id)->second.block = -1;
            cached_blocks -= 1;
            cache_evictions += 1;
            unref(id);
        }
        return b;
    }
    void push(int32_t b) { freeq.push(b); }
    // The sequence's token ids stop being known: it leaves the content chain.
    void untrack(Seq& s) {
        if (!s.tracked) return;
        if (s.chain >= 0) unref(s.chain);
        s.chain = -1;
        s.partial.clear();
        s.tracked = false;
    }
    // A tracked sequence has just filled block b (its tokens are s.partial): the sequence's
    // chain moves to that content, and b is registered under it unless another block is.
    void complete_block(Seq& s, int32_t b) {
        const int64_t id = intern(s.chain, s.partial);
        Node& nd = nodes.find(id)->second;
        nd.refs += 1;                         // the sequence's reference
        if (s.chain >= 0) unref(s.chain);     // still held by the new node
        s.chain = id;
        s.partial.clear();
        if (nd.block < 0) {
            nd.block = b;
            nd.refs += 1;
            node_of_block[b] = id;
            cached_blocks += 1;
        }
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
    // Performs an append already known to fit, registering the blocks it fills when the
    // tokens' ids are given and the sequence is tracked.  Returns the number of COW pairs (0
    // or 1).
    int append_fit(Seq& s, int64_t n, int64_t* slots, int64_t* cow, const int32_t* tokens = nullptr) {
        const int64_t bs = block_size;
        if (!tokens && n > 0) untrack(s);
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
            if (s.tracked) {
                s.partial.push_back(tokens[t]);
                if (s.n % bs == 0) complete_block(s, s.blocks.back());
            }
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
    a->node_of_block.assign(num_blocks, -1);
    a->freeq.init(num_blocks);
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
        }
        for (int32_t i = 0; i < num_blocks; ++i) a->freeq.push(initial_free_order[i]);
    } else {
        for (int32_t i = 0; i < num_blocks; ++i) a->freeq.push(i);
    }
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
    if (s.swapped) return fail(PA_ERR_INVALID, "pa_seq_append: sequence %lld is swapped out", (long long)seq_id);
    int64_t need = a->blocks_needed(s, n_tokens, 0);
    if (need > a->freeq.count) {
        a->exhaustion_events += 1;
        return fail(PA_ERR_NO_BLOCKS, "pa_seq_append: sequence %lld needs %lld blocks, %lld free",
                    (long long)seq_id, (long long)need, (long long)a->freeq.count);
    }
    *n_cow_out = a->append_fit(s, n_tokens, slots_out, cow_out);
    return PA_OK;
}

int pa_seq_append_tokens(pa_allocator* a, int64_t seq_id, const int32_t* tokens, int32_t n_tokens,
                         int64_t* slots_out, int64_t* cow_out, int32_t* n_cow_out) {
    pagedkv::clear_error();
    if (!a) return fail(PA_ERR_INVALID, "pa_seq_append_tokens: NULL allocator");
    if (n_tokens < 0) return fail(PA_ERR_INVALID, "pa_seq_append_tokens: n_tokens=%d < 0", n_tokens);
    if (n_tokens > 0 && (!slots_out || !tokens)) return fail(PA_ERR_INVALID, "pa_seq_append_tokens: NULL array");
    if (!cow_out || !n_cow_out) return fail(PA_ERR_INVALID, "pa_seq_append_tokens: cow_out/n_cow_out is NULL");
    auto it = a->seqs.find(seq_id);
    if (it == a->seqs.end())
        return fail(PA_ERR_INVALID, "pa_seq_append_tokens: unknown sequence %lld", (long long)seq_id);
    Seq& s = it->second;
    if (s.swapped)
        return fail(PA_ERR_INVALID, "pa_seq_append_tokens: sequence %lld is swapped out", (long long)seq_id);
    const int64_t need = a->blocks_needed(s, n_tokens, 0);
    if (need > a->freeq.count) {
        a->exhaustion_events += 1;
        return fail(PA_ERR_NO_BLOCKS, "pa_seq_append_tokens: sequence %lld needs %lld blocks, %lld free",
                    (long long)seq_id, (long long)need, (long long)a->freeq.count);
    }
    *n_cow_out = a->append_fit(s, n_tokens, slots_out, cow_out, tokens);
    return PA_OK;
}

int pa_seq_add_prompt(pa_allocator* a, int64_t seq_id, const int32_t* tokens, int32_t n_tokens,
                      int32_t* n_cached_out, int64_t* slots_out) {
    pagedkv::clear_error();
    if (!a) return fail(PA_ERR_INVALID, "pa_seq_add_prompt: NULL allocator");
    if (n_tokens < 0) return fail(PA_ERR_INVALID, "pa_seq_add_prompt: n_tokens=%d < 0", n_tokens);
    if (!n_cached_out || (n_tokens > 0 && !tokens))
        return fail(PA_ERR_INVALID, "pa_seq_add_prompt: NULL argument");
    if (a->seqs.count(seq_id)) return fail(PA_ERR_INVALID, "pa_seq_add_prompt: sequence %lld exists", (long long)seq_id);
    const int64_t bs = a->block_size;
    // the longest run of registered blocks from block 0 whose content is this prompt's prefix
    std::vector<int32_t> hits;
    int64_t chain = -1, hit_free = 0;
    std::vector<int32_t> blk(bs);
    for (int64_t k = 0; (k + 1) * bs <= n_tokens; ++k) {
        blk.assign(tokens + k * bs, tokens + (k + 1) * bs);
        auto it = a->node_of_key.find(BlockKey{chain, blk});
        if (it == a->node_of_key.end()) break;
        const int32_t b = a->nodes.find(it->second)->second.block;
        if (b < 0) break;
        hits.push_back(b);
        hit_free += a->refcount[b] == 0;
        chain = it->second;
    }
    const int64_t n_cached = static_cast<int64_t>(hits.size()) * bs;
    const int64_t need = (n_tokens - n_cached + bs - 1) / bs;   // fresh blocks for the rest
    if (n_tokens - n_cached > 0 && !slots_out) return fail(PA_ERR_INVALID, "pa_seq_add_prompt: slots_out is NULL");
    if (need > a->freeq.count - hit_free) {
        a->exhaustion_events += 1;
        return fail(PA_ERR_NO_BLOCKS, "pa_seq_add_prompt: sequence %lld needs %lld blocks, %lld free",
                    (long long)seq_id, (long long)need, (long long)(a->freeq.count - hit_free));
    }
    Seq s;
    for (int32_t b : hits) {
        if (a->refcount[b] == 0) a->freeq.remove(b);   // a cached block back in use
        a->refcount[b] += 1;
        s.blocks.push_back(b);
    }
    s.n = n_cached;
    s.chain = chain;
    if (chain >= 0) a->nodes.find(chain)->second.refs += 1;
    a->cache_hit_blocks += static_cast<int64_t>(hits.size());
    int64_t cow[2];
    a->append_fit(s, n_tokens - n_cached, slots_out, cow, tokens + n_cached);   // starts a fresh block: no copy
    a->seqs.emplace(seq_id, std::move(s));
    *n_cached_out = static_cast<int32_t>(n_cached);
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
        if (s.swapped)
            return fail(PA_ERR_INVALID, "pa_batch_append: sequence %lld is swapped out", (long long)seq_ids[i]);
        ss[i] = &s;
        int32_t drop = 0;
        if (n_tokens[i] > 0 && s.n % a->block_size != 0) {
            auto d = dropped.find(s.blocks.back());
            drop = d == dropped.end() ? 0 : d->second;
            if (a->refcount[s.blocks.back()] - drop > 1) dropped[s.blocks.back()] = drop + 1;
        }
        need += a->blocks_needed(s, n_tokens[i], drop);
    }
    if (need > a->freeq.count) {
        a->exhaustion_events += 1;
        return fail(PA_ERR_NO_BLOCKS, "pa_batch_append: batch needs %lld blocks, %lld free",
                    (long long)need, (long long)a->freeq.count);
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
    if (it->second.swapped) return fail(PA_ERR_INVALID, "pa_seq_fork: parent %lld is swapped out", (long long)parent);
    Seq c = it->second;  // copy of the block list, token count and content chain
    for (int32_t b : c.blocks) a->refcount[b] += 1;
    if (c.chain >= 0) a->nodes.find(c.chain)->second.refs += 1;
    a->seqs.emplace(child, std::move(c));
    return PA_OK;
}

int pa_seq_free(pa_allocator* a, int64_t seq_id) {
    pagedkv::clear_error();
    if (!a) return fail(PA_ERR_INVALID, "pa_seq_free: NULL allocator");
    auto it = a->seqs.find(seq_id);
    if (it == a->seqs.end()) return fail(PA_ERR_INVALID, "pa_seq_free: unknown sequence %lld", (long long)seq_id);
    if (it->second.swapped) {   // its references are host blocks
        for (int32_t b : it->second.blocks)
            if (--a->host_refcount[b] == 0) a->host_free.push(b);
        a->swapped_seqs -= 1;
    } else {
        for (int32_t b : it->second.blocks)
            if (--a->refcount[b] == 0) a->push(b);
    }
    a->untrack(it->second);
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
        if (it->second.swapped)
            return fail(PA_ERR_INVALID, "pa_block_tables: sequence %lld is swapped out", (long long)seq_ids[i]);
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
    for (const auto& kv : a->seqs)
        if (!kv.second.swapped) waste += (kv.second.n + bs - 1) / bs * bs - kv.second.n;
    out->free_blocks = a->freeq.count;
    out->used_blocks = used;
    out->total_refs = refs;
    out->exhaustion_events = a->exhaustion_events;
    out->waste_slots = waste;
    out->num_seqs = static_cast<int64_t>(a->seqs.size());
    int64_t host_used = 0;
    for (int32_t r : a->host_refcount) host_used += r > 0;
    out->host_free_blocks = a->host_free.count;
    out->host_used_blocks = host_used;
    out->swapped_seqs = a->swapped_seqs;
    out->cached_blocks = a->cached_blocks;
    out->cache_hit_blocks = a->cache_hit_blocks;
    out->cache_evictions = a->cache_evictions;
    return PA_OK;
}

int pa_alloc_dump_cached(const pa_allocator* a, int32_t* registered) {
    pagedkv::clear_error();
    if (!a || !registered) return fail(PA_ERR_INVALID, "pa_alloc_dump_cached: NULL argument");
    for (int32_t b = 0; b < a->num_blocks; ++b) registered[b] = a->node_of_block[b] >= 0 ? 1 : 0;
    return PA_OK;
}

int pa_alloc_dump(const pa_allocator* a, int32_t* refcounts, int32_t* free_order, int32_t* n_free) {
    pagedkv::clear_error();
    if (!a || !refcounts || !free_order || !n_free) return fail(PA_ERR_INVALID, "pa_alloc_dump: NULL argument");
    std::memcpy(refcounts, a->refcount.data(), a->refcount.size() * sizeof(int32_t));
    int64_t i = 0;
    for (int32_t b = a->freeq.head; b >= 0; b = a->freeq.nxt[b]) free_order[i++] = b;
    *n_free = static_cast<int32_t>(a->freeq.count);
    return PA_OK;
}

int pa_alloc_set_host_blocks(pa_allocator* a, int32_t num_host_blocks) {
    pagedkv::clear_error();
    if (!a) return fail(PA_ERR_INVALID, "pa_alloc_set_host_blocks: NULL allocator");
    if (num_host_blocks < 0) return fail(PA_ERR_INVALID, "pa_alloc_set_host_blocks: %d < 0", num_host_blocks);
    if (a->swapped_seqs > 0)
        return fail(PA_ERR_INVALID, "pa_alloc_set_host_blocks: %lld sequences are swapped out",
                    (long long)a->swapped_seqs);
    a->host_refcount.assign(num_host_blocks, 0);
    a->host_free.reset(num_host_blocks);
    return PA_OK;
}

}  // extern "C"

namespace {

// Moves the listed sequences' references from one pool to the other.  `from_ref` / `to_ref`
// are the refcounts of the pools, `release` returns a block whose count reaches 0 to its
// pool's free queue and `grant` pops the other pool's free head.  Validation (ids, state,
// room, buffer size) has been done by the caller.
template <class Release, class Grant>
int32_t move_refs(const std::vector<Seq*>& ss, std::vector<int32_t>& from_ref,
                  std::vector<int32_t>& to_ref, Release release, Grant grant, int64_t* pairs_out) {
    std::unordered_map<int32_t, int32_t> map;   // block in the old pool -> block in the new
    int32_t np = 0;
    for (Seq* s : ss) {
        for (int32_t& b : s->blocks) {
            auto it = map.find(b);
            int32_t nb;
            if (it == map.end()) {
                nb = grant();
                to_ref[nb] = 0;
                map.emplace(b, nb);
                pairs_out[2 * np] = b;
                pairs_out[2 * np + 1] = nb;
                ++np;
            } else {
                nb = it->second;
            }
            to_ref[nb] += 1;
            if (--from_ref[b] == 0) release(b);
            b = nb;
        }
        s->swapped = !s->swapped;
    }
    return np;
}

// Checks the listed sequences (known, distinct, all in state `swapped`) and counts the
// distinct blocks they hold.
int collect(pa_allocator* a, const char* fn, const int64_t* seq_ids, int32_t n_seqs, bool swapped,
            std::vector<Seq*>& ss, int64_t& distinct) {
    if (n_seqs < 0) return fail(PA_ERR_INVALID, "%s: n_seqs=%d < 0", fn, n_seqs);
    if (n_seqs > 0 && !seq_ids) return fail(PA_ERR_INVALID, "%s: seq_ids is NULL", fn);
    std::unordered_map<int64_t, char> ids;
    std::unordered_map<int32_t, char> blocks;
    ss.resize(n_seqs);
    for (int32_t i = 0; i < n_seqs; ++i) {
        auto it = a->seqs.find(seq_ids[i]);
        if (it == a->seqs.end()) return fail(PA_ERR_INVALID, "%s: unknown sequence %lld", fn, (long long)seq_ids[i]);
        if (!ids.emplace(seq_ids[i], 1).second)
            return fail(PA_ERR_INVALID, "%s: sequence %lld listed twice", fn, (long long)seq_ids[i]);
        if (it->second.swapped != swapped)
            return fail(PA_ERR_INVALID, "%s: sequence %lld is %s", fn, (long long)seq_ids[i],
                        swapped ? "not swapped out" : "already swapped out");
        ss[i] = &it->second;
        for (int32_t b : it->second.blocks) blocks.emplace(b, 1);
    }
    distinct = static_cast<int64_t>(blocks.size());
    return PA_OK;
}

}  // namespace

extern "C" {

int pa_swap_out(pa_allocator* a, const int64_t* seq_ids, int32_t n_seqs, int64_t* pairs_out,
                int32_t max_pairs, int32_t* n_pairs_out) {
    pagedkv::clear_error();
    if (!a) return fail(PA_ERR_INVALID, "pa_swap_out: NULL allocator");
    if (!n_pairs_out) return fail(PA_ERR_INVALID, "pa_swap_out: n_pairs_out is NULL");
    std::vector<Seq*> ss;
    int64_t distinct = 0;
    if (int rc = collect(a, "pa_swap_out", seq_ids, n_seqs, false, ss, distinct)) return rc;
    if (distinct > max_pairs || (distinct > 0 && !pairs_out))
        return fail(PA_ERR_INVALID, "pa_swap_out: %lld pairs do not fit the buffer of %d", (long long)distinct, max_pairs);
    if (distinct > a->host_free.count)
        return fail(PA_ERR_NO_BLOCKS, "pa_swap_out: %lld host blocks needed, %lld free", (long long)distinct,
                    (long long)a->host_free.count);
    *n_pairs_out = move_refs(
        ss, a->refcount, a->host_refcount, [a](int32_t b) { a->push(b); },
        [a]() { return a->host_free.pop(); }, pairs_out);
    a->swapped_seqs += n_seqs;
    return PA_OK;
}

int pa_swap_in(pa_allocator* a, const int64_t* seq_ids, int32_t n_seqs, int64_t* pairs_out,
               int32_t max_pairs, int32_t* n_pairs_out) {
    pagedkv::clear_error();
    if (!a) return fail(PA_ERR_INVALID, "pa_swap_in: NULL allocator");
    if (!n_pairs_out) return fail(PA_ERR_INVALID, "pa_swap_in: n_pairs_out is NULL");
    std::vector<Seq*> ss;
    int64_t distinct = 0;
    if (int rc = collect(a, "pa_swap_in", seq_ids, n_seqs, true, ss, distinct)) return rc;
    if (distinct > max_pairs || (distinct > 0 && !pairs_out))
        return fail(PA_ERR_INVALID, "pa_swap_in: %lld pairs do not fit the buffer of %d", (long long)distinct, max_pairs);
    if (distinct > a->freeq.count) {
        a->exhaustion_events += 1;
        return fail(PA_ERR_NO_BLOCKS, "pa_swap_in: %lld blocks needed, %lld free", (long long)distinct,
                    (long long)a->freeq.count);
    }
    *n_pairs_out = move_refs(
        ss, a->host_refcount, a->refcount, [a](int32_t b) { a->host_free.push(b); },
        [a]() { return a->pop(); }, pairs_out);
    a->swapped_seqs -= n_seqs;
    return PA_OK;
}

int pa_seq_is_swapped(const pa_allocator* a, int64_t seq_id) {
    pagedkv::clear_error();
    if (!a) return fail(PA_ERR_INVALID, "pa_seq_is_swapped: NULL allocator");
    auto it = a->seqs.find(seq_id);
    if (it == a->seqs.end()) return fail(PA_ERR_INVALID, "pa_seq_is_swapped: unknown sequence %lld", (long long)seq_id);
    return it->second.swapped ? 1 : 0;
}

int pa_alloc_dump_host(const pa_allocator* a, int32_t* refcounts, int32_t* free_order, int32_t* n_free) {
    pagedkv::clear_error();
    if (!a || !n_free) return fail(PA_ERR_INVALID, "pa_alloc_dump_host: NULL argument");
    const int64_t nh = static_cast<int64_t>(a->host_refcount.size());
    if (nh > 0 && (!refcounts || !free_order)) return fail(PA_ERR_INVALID, "pa_alloc_dump_host: NULL argument");
    if (nh > 0) std::memcpy(refcounts, a->host_refcount.data(), nh * sizeof(int32_t));
    for (int64_t i = 0; i < a->host_free.count; ++i) free_order[i] = a->host_free.ring[(a->host_free.head + i) % nh];
    *n_free = static_cast<int32_t>(a->host_free.count);
    return PA_OK;
}

}  // extern "C"
