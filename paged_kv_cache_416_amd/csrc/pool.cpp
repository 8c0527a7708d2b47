// Host block-pool allocator: the scheduler-side half of the paged KV cache.
//
// "vLLM and PagedAttention" slides 10-16 and the "Week 22 Day 2" lesson note,
// sections 2-4: one pool of fixed-size blocks shared by all requests, a
// per-sequence block table, allocation only once the last block has no free slot,
// reference-counted sharing (fork), copy-on-write of a shared, partly filled
// last block, immediate release of a finished sequence's blocks, and
// all-or-nothing admission when the pool runs short.
//
// Choices the pages leave open: free blocks form a LIFO stack (free_order[0]
// is handed out first; a freed block is the next one handed out); a freed
// sequence returns its blocks in logical order; a batched append serves its
// sequences in the order given.
//
// Prefix cache (the lesson note, section 3.1: prompt blocks are looked up by a cryptographic
// digest; a new request whose prompt block has the digest of a held block maps that block and
// increments its count). Readings: the digest of full prompt block j is SHA-256 of (the digest of block j-1,
// or 32 zero bytes for j = 0) followed by the block's token ids as little-endian int32, so equal
// digests mean equal prefixes, which is what a block's keys and values depend on; only full
// prompt blocks are hashed, and hits are taken as a prefix of the prompt. A hashed block that
// falls free keeps its digest and contents until the pool needs it: free blocks without a
// digest are handed out first (the LIFO stack), then hashed free blocks, least recently freed
// first, each dropping its digest.
#include <algorithm>
#include <array>
#include <cstring>
#include <iterator>
#include <list>
#include <unordered_map>
#include <unordered_set>
#include <vector>

#include "common.h"

using pkv::fail;

namespace pkv {
void sha256(const uint8_t *data, size_t n, uint8_t out[32]);
}

namespace {
typedef std::array<uint8_t, 32> Digest;
struct DigestHash {
    size_t operator()(const Digest &d) const {
        size_t h;
        std::memcpy(&h, d.data(), sizeof h);
        return h;
    }
};

// Chained digests of the full blocks of a token stream (see above).
void prompt_digests(const int32_t *tokens, int64_t n_full, int32_t block_size, Digest *out) {
    std::vector<uint8_t> buf(32 + static_cast<size_t>(block_size) * 4);
    Digest prev{};
    for (int64_t j = 0; j < n_full; ++j) {
        std::memcpy(buf.data(), prev.data(), 32);
        for (int32_t t = 0; t < block_size; ++t) {
            const uint32_t v = static_cast<uint32_t>(tokens[j * block_size + t]);
            for (int b = 0; b < 4; ++b) buf[32 + 4 * t + b] = static_cast<uint8_t>(v >> (8 * b));
        }
        pkv::sha256(buf.data(), buf.size(), out[j].data());
        prev = out[j];
    }
}
}  // namespace

struct pkv_pool {
    struct Seq {
        std::vector<int32_t> blocks;  // logical block j -> physical block
        int64_t len = 0;              // tokens written
        uint64_t stamp = 0;           // the last batched append that named it
    };
    int32_t num_blocks = 0;
    int32_t block_size = 0;
    std::vector<int32_t> free_stack;  // free blocks without a digest; back() is handed out next
    std::list<int32_t> cached_free;   // free blocks that keep a digest, least recently freed first
    std::vector<std::list<int32_t>::iterator> lru_pos;
    std::vector<int32_t> ref;  // sequences mapping each block
    std::vector<Digest> digest;
    std::vector<char> has_digest;
    std::unordered_map<Digest, int32_t, DigestHash> by_digest;
    std::unordered_map<int64_t, Seq> seqs;
    // batched-append scratch, kept between calls so that a decode step allocates nothing
    uint64_t append_stamp = 0;
    std::vector<Seq *> batch;
    std::vector<int32_t> pending_drop;  // per block: shared last blocks given up earlier in the batch
    std::vector<int32_t> touched;       // blocks whose pending_drop is non-zero

    int64_t available() const { return static_cast<int64_t>(free_stack.size() + cached_free.size()); }

    int32_t take() {
        int32_t b;
        if (!free_stack.empty()) {
            b = free_stack.back();
            free_stack.pop_back();
        } else {  // evict the least recently freed hashed block
            b = cached_free.front();
            cached_free.pop_front();
            by_digest.erase(digest[b]);
            has_digest[b] = 0;
        }
        ref[b] = 1;
        return b;
    }

    // b's count just reached zero
    void release(int32_t b) {
        if (has_digest[b]) {
            cached_free.push_back(b);
            lru_pos[b] = std::prev(cached_free.end());
        } else {
            free_stack.push_back(b);
        }
    }
};

extern "C" {

int pkv_pool_create(int32_t num_blocks, int32_t block_size, const int32_t *free_order, pkv_pool **out) {
    if (!out) return fail(PKV_EINVAL, "pkv_pool_create: out is NULL");
    *out = nullptr;
    if (num_blocks <= 0 || block_size <= 0)
        return fail(PKV_EINVAL, "pkv_pool_create: num_blocks=%d block_size=%d must be positive", num_blocks,
                    block_size);
    auto *p = new pkv_pool;
    p->num_blocks = num_blocks;
    p->block_size = block_size;
    p->ref.assign(num_blocks, 0);
    p->digest.resize(num_blocks);
    p->has_digest.assign(num_blocks, 0);
    p->lru_pos.resize(num_blocks);
    p->free_stack.resize(num_blocks);
    if (free_order) {
        std::vector<char> seen(num_blocks, 0);
        for (int32_t i = 0; i < num_blocks; ++i) {
            int32_t b = free_order[i];
            if (b < 0 || b >= num_blocks || seen[b]) {
                delete p;
                return fail(PKV_EINVAL, "pkv_pool_create: free_order is not a permutation (entry %d = %d)", i, b);
            }
            seen[b] = 1;
            p->free_stack[num_blocks - 1 - i] = b;
        }
    } else {
        for (int32_t i = 0; i < num_blocks; ++i) p->free_stack[num_blocks - 1 - i] = i;
    }
    *out = p;
    return PKV_OK;
}

void pkv_pool_destroy(pkv_pool *pool) { delete pool; }

int32_t pkv_pool_num_blocks(const pkv_pool *pool) { return pool ? pool->num_blocks : PKV_EINVAL; }
int32_t pkv_pool_block_size(const pkv_pool *pool) { return pool ? pool->block_size : PKV_EINVAL; }
int32_t pkv_pool_num_free(const pkv_pool *pool) {
    return pool ? static_cast<int32_t>(pool->available()) : PKV_EINVAL;
}

int32_t pkv_pool_num_cached(const pkv_pool *pool) {
    return pool ? static_cast<int32_t>(pool->by_digest.size()) : PKV_EINVAL;
}

int32_t pkv_block_ref_count(const pkv_pool *pool, int32_t block) {
    if (!pool || block < 0 || block >= pool->num_blocks) return -1;
    return pool->ref[block];
}

int pkv_seq_add(pkv_pool *pool, int64_t seq_id) {
    if (!pool) return fail(PKV_EINVAL, "pkv_seq_add: pool is NULL");
    if (pool->seqs.count(seq_id)) return fail(PKV_EEXIST, "pkv_seq_add: sequence %lld exists", (long long)seq_id);
    pool->seqs.emplace(seq_id, pkv_pool::Seq{});
    return PKV_OK;
}

int pkv_seq_free(pkv_pool *pool, int64_t seq_id) {
    if (!pool) return fail(PKV_EINVAL, "pkv_seq_free: pool is NULL");
    auto it = pool->seqs.find(seq_id);
    if (it == pool->seqs.end()) return fail(PKV_ENOSEQ, "pkv_seq_free: unknown sequence %lld", (long long)seq_id);
    for (int32_t b : it->second.blocks)
        if (--pool->ref[b] == 0) pool->release(b);
    pool->seqs.erase(it);
    return PKV_OK;
}

int pkv_seq_fork(pkv_pool *pool, int64_t parent, int64_t child) {
    if (!pool) return fail(PKV_EINVAL, "pkv_seq_fork: pool is NULL");
    auto it = pool->seqs.find(parent);
    if (it == pool->seqs.end()) return fail(PKV_ENOSEQ, "pkv_seq_fork: unknown parent %lld", (long long)parent);
    if (pool->seqs.count(child)) return fail(PKV_EEXIST, "pkv_seq_fork: sequence %lld exists", (long long)child);
    pkv_pool::Seq copy = it->second;
    for (int32_t b : copy.blocks) ++pool->ref[b];
    pool->seqs.emplace(child, std::move(copy));
    return PKV_OK;
}

int64_t pkv_seq_len(const pkv_pool *pool, int64_t seq_id) {
    if (!pool) return fail(PKV_EINVAL, "pkv_seq_len: pool is NULL");
    auto it = pool->seqs.find(seq_id);
    if (it == pool->seqs.end()) return fail(PKV_ENOSEQ, "pkv_seq_len: unknown sequence %lld", (long long)seq_id);
    return it->second.len;
}

int32_t pkv_seq_num_blocks(const pkv_pool *pool, int64_t seq_id) {
    if (!pool) return fail(PKV_EINVAL, "pkv_seq_num_blocks: pool is NULL");
    auto it = pool->seqs.find(seq_id);
    if (it == pool->seqs.end())
        return fail(PKV_ENOSEQ, "pkv_seq_num_blocks: unknown sequence %lld", (long long)seq_id);
    return static_cast<int32_t>(it->second.blocks.size());
}

int32_t pkv_seq_blocks(const pkv_pool *pool, int64_t seq_id, int32_t *out, int32_t cap) {
    if (!pool || (!out && cap > 0)) return fail(PKV_EINVAL, "pkv_seq_blocks: NULL argument");
    auto it = pool->seqs.find(seq_id);
    if (it == pool->seqs.end()) return fail(PKV_ENOSEQ, "pkv_seq_blocks: unknown sequence %lld", (long long)seq_id);
    const auto &b = it->second.blocks;
    if (static_cast<int64_t>(b.size()) > cap)
        return fail(PKV_EINVAL, "pkv_seq_blocks: %zu blocks, room for %d", b.size(), cap);
    for (size_t j = 0; j < b.size(); ++j) out[j] = b[j];
    return static_cast<int32_t>(b.size());
}

int pkv_seq_append(pkv_pool *pool, const int64_t *seq_ids, const int32_t *n_tokens, int32_t n_seqs,
                   int64_t *slots_out, int32_t *cow_pairs_out, int32_t max_pairs, int32_t *n_pairs_out) {
    if (!pool || n_seqs < 0 || (n_seqs > 0 && (!seq_ids || !n_tokens)) || max_pairs < 0 ||
        (max_pairs > 0 && !cow_pairs_out))
        return fail(PKV_EINVAL, "pkv_seq_append: bad arguments");
    const int64_t B = pool->block_size;
    // Validation and a dry run that counts the blocks the whole batch needs, so that a
    // batch the pool cannot serve changes nothing (slide 15: all or nothing). A sequence named
    // twice is caught by its stamp; pending_drop counts, per block, the sharers that already
    // gave up a shared partial last block earlier in the batch (cleared again on every exit).
    const uint64_t stamp = ++pool->append_stamp;
    if (pool->pending_drop.size() != static_cast<size_t>(pool->num_blocks)) pool->pending_drop.assign(pool->num_blocks, 0);
    auto &pending = pool->pending_drop;
    auto &touched = pool->touched;
    auto clear_pending = [&]() {
        for (const int32_t b : touched) pending[b] = 0;
        touched.clear();
    };
    int64_t need = 0, total_tokens = 0;
    int32_t pairs = 0;
    auto &seqv = pool->batch;
    seqv.resize(n_seqs);
    for (int32_t i = 0; i < n_seqs; ++i) {
        auto it = pool->seqs.find(seq_ids[i]);
        if (it == pool->seqs.end()) {
            clear_pending();
            return fail(PKV_ENOSEQ, "pkv_seq_append: unknown sequence %lld", (long long)seq_ids[i]);
        }
        pkv_pool::Seq &q = it->second;
        if (q.stamp == stamp) {
            clear_pending();
            return fail(PKV_EINVAL, "pkv_seq_append: sequence %lld appears twice", (long long)seq_ids[i]);
        }
        q.stamp = stamp;
        if (n_tokens[i] < 0) {
            clear_pending();
            return fail(PKV_EINVAL, "pkv_seq_append: n_tokens[%d] = %d < 0", i, n_tokens[i]);
        }
        seqv[i] = &q;
        const int64_t n = n_tokens[i];
        if (n == 0) continue;
        if (q.len % B) {
            const int32_t last = q.blocks.back();
            if (pool->ref[last] - pending[last] > 1) {
                if (pending[last]++ == 0) touched.push_back(last);
                ++need;
                ++pairs;
            }
        }
        const int64_t blocks_after = pkv::ceil_div(q.len + n, B);
        if (blocks_after > INT32_MAX) {
            clear_pending();
            return fail(PKV_EINVAL, "pkv_seq_append: sequence %lld too long", (long long)seq_ids[i]);
        }
        need += blocks_after - static_cast<int64_t>(q.blocks.size());
        total_tokens += n;
    }
    clear_pending();
    if (total_tokens > 0 && !slots_out) return fail(PKV_EINVAL, "pkv_seq_append: slots_out is NULL");
    if (pairs > max_pairs)
        return fail(PKV_EINVAL, "pkv_seq_append: %d copy-on-write pairs, room for %d", pairs, max_pairs);
    if (need > pool->available())
        return fail(PKV_ENOMEM, "pkv_seq_append: batch needs %lld blocks, %lld free", (long long)need,
                    (long long)pool->available());
    // Apply.
    int64_t k = 0;
    int32_t np = 0;
    for (int32_t i = 0; i < n_seqs; ++i) {
        pkv_pool::Seq &q = *seqv[i];
        const int64_t n = n_tokens[i];
        if (n == 0) continue;
        if (q.len % B && pool->ref[q.blocks.back()] > 1) {
            const int32_t src = q.blocks.back();
            const int32_t dst = pool->take();
            --pool->ref[src];
            q.blocks.back() = dst;
            cow_pairs_out[2 * np] = src;
            cow_pairs_out[2 * np + 1] = dst;
            ++np;
        }
        while (static_cast<int64_t>(q.blocks.size()) * B < q.len + n) q.blocks.push_back(pool->take());
        for (int64_t t = q.len; t < q.len + n; ++t) slots_out[k++] = static_cast<int64_t>(q.blocks[t / B]) * B + t % B;
        q.len += n;
    }
    if (n_pairs_out) *n_pairs_out = np;
    return PKV_OK;
}

int pkv_shared_prefix_lens(const pkv_pool *pool, const int64_t *seq_ids, int32_t n, int32_t *out) {
    if (!pool || n < 0 || (n > 0 && (!seq_ids || !out))) return fail(PKV_EINVAL, "pkv_shared_prefix_lens: bad arguments");
    for (int32_t i = 0; i < n; ++i)
        if (!pool->seqs.count(seq_ids[i]))
            return fail(PKV_ENOSEQ, "pkv_shared_prefix_lens: unknown sequence %lld", (long long)seq_ids[i]);
    for (int32_t i = 0; i < n; ++i) {
        const auto &q = pool->seqs.find(seq_ids[i])->second;
        int64_t j = 0;
        while (j < static_cast<int64_t>(q.blocks.size()) && pool->ref[q.blocks[j]] > 1) ++j;
        out[i] = static_cast<int32_t>(std::min<int64_t>({q.len, j * pool->block_size, INT32_MAX}));
    }
    return PKV_OK;
}

int pkv_build_block_tables(const pkv_pool *pool, const int64_t *seq_ids, int32_t n, int32_t max_blocks,
                           int32_t pad_value, int32_t *tables_out, int32_t *ctx_out) {
    if (!pool || n < 0 || max_blocks < 0 || (n > 0 && (!seq_ids || !tables_out || !ctx_out)))
        return fail(PKV_EINVAL, "pkv_build_block_tables: bad arguments");
    for (int32_t i = 0; i < n; ++i) {
        auto it = pool->seqs.find(seq_ids[i]);
        if (it == pool->seqs.end())
            return fail(PKV_ENOSEQ, "pkv_build_block_tables: unknown sequence %lld", (long long)seq_ids[i]);
        if (static_cast<int64_t>(it->second.blocks.size()) > max_blocks)
            return fail(PKV_EINVAL, "pkv_build_block_tables: sequence %lld has %zu blocks > max_blocks %d",
                        (long long)seq_ids[i], it->second.blocks.size(), max_blocks);
        if (it->second.len > INT32_MAX)
            return fail(PKV_EINVAL, "pkv_build_block_tables: sequence %lld too long", (long long)seq_ids[i]);
    }
    for (int32_t i = 0; i < n; ++i) {
        const auto &q = pool->seqs.find(seq_ids[i])->second;
        int32_t *row = tables_out + static_cast<int64_t>(i) * max_blocks;
        size_t j = 0;
        for (; j < q.blocks.size(); ++j) row[j] = q.blocks[j];
        for (; j < static_cast<size_t>(max_blocks); ++j) row[j] = pad_value;
        ctx_out[i] = static_cast<int32_t>(q.len);
    }
    return PKV_OK;
}

int pkv_prompt_digests(const int32_t *tokens, int64_t n_tokens, int32_t block_size, uint8_t *digests_out,
                       int64_t max_blocks) {
    if (n_tokens < 0 || block_size <= 0 || (n_tokens > 0 && !tokens) || max_blocks < 0)
        return fail(PKV_EINVAL, "pkv_prompt_digests: bad arguments");
    const int64_t n_full = n_tokens / block_size;
    if (n_full > max_blocks || (n_full > 0 && !digests_out))
        return fail(PKV_EINVAL, "pkv_prompt_digests: %lld full blocks, room for %lld", (long long)n_full,
                    (long long)max_blocks);
    if (n_full > INT32_MAX) return fail(PKV_EINVAL, "pkv_prompt_digests: too many blocks");
    std::vector<Digest> d(n_full);
    prompt_digests(tokens, n_full, block_size, d.data());
    for (int64_t j = 0; j < n_full; ++j) std::memcpy(digests_out + 32 * j, d[j].data(), 32);
    return static_cast<int32_t>(n_full);
}

int pkv_seq_add_prompt(pkv_pool *pool, int64_t seq_id, const int32_t *tokens, int32_t n_tokens, int64_t *slots_out,
                       int32_t *n_cached_out) {
    if (n_cached_out) *n_cached_out = 0;
    if (!pool || n_tokens < 0 || (n_tokens > 0 && (!tokens || !slots_out)))
        return fail(PKV_EINVAL, "pkv_seq_add_prompt: bad arguments");
    if (pool->seqs.count(seq_id))
        return fail(PKV_EEXIST, "pkv_seq_add_prompt: sequence %lld exists", (long long)seq_id);
    const int32_t B = pool->block_size;
    const int32_t n_full = n_tokens / B;
    std::vector<Digest> d(n_full);
    prompt_digests(tokens, n_full, B, d.data());
    // cached prefix: leading full blocks whose digests the pool holds
    std::vector<int32_t> hit;
    int64_t revive = 0;  // hits on free (cached) blocks: they leave the free lists
    for (int32_t j = 0; j < n_full; ++j) {
        auto f = pool->by_digest.find(d[j]);
        if (f == pool->by_digest.end()) break;
        hit.push_back(f->second);
        if (pool->ref[f->second] == 0) ++revive;
    }
    const int32_t n_hit = static_cast<int32_t>(hit.size());
    const int64_t fresh = (n_full - n_hit) + (n_tokens % B ? 1 : 0);
    if (revive + fresh > pool->available())
        return fail(PKV_ENOMEM, "pkv_seq_add_prompt: %lld blocks needed, %lld free", (long long)(revive + fresh),
                    (long long)pool->available());
    pkv_pool::Seq q;
    q.len = n_tokens;
    for (int32_t b : hit) {
        if (pool->ref[b] == 0) pool->cached_free.erase(pool->lru_pos[b]);
        ++pool->ref[b];
        q.blocks.push_back(b);
    }
    for (int32_t j = n_hit; j < n_full; ++j) {
        const int32_t b = pool->take();
        auto f = pool->by_digest.find(d[j]);
        if (f != pool->by_digest.end()) {
            // a later block of a chain whose earlier block was evicted: the new block takes the
            // digest over and the old one becomes an ordinary block (free, if unused)
            const int32_t old = f->second;
            pool->has_digest[old] = 0;
            if (pool->ref[old] == 0) {
                pool->cached_free.erase(pool->lru_pos[old]);
                pool->free_stack.push_back(old);
            }
        }
        pool->digest[b] = d[j];
        pool->has_digest[b] = 1;
        pool->by_digest[d[j]] = b;
        q.blocks.push_back(b);
    }
    if (n_tokens % B) q.blocks.push_back(pool->take());
    const int64_t cached = static_cast<int64_t>(n_hit) * B;
    for (int64_t t = 0; t < n_tokens; ++t)
        slots_out[t] = t < cached ? -1 : static_cast<int64_t>(q.blocks[t / B]) * B + t % B;
    pool->seqs.emplace(seq_id, std::move(q));
    if (n_cached_out) *n_cached_out = static_cast<int32_t>(cached);
    return PKV_OK;
}

// Moves whole sequences to another pool, all or nothing (slide 15: a preempted request leaves
// at once and comes back by swap). Every distinct block the sequences map gets one block of
// dst, in first-use order (sequence order, then logical order), carrying the sequences' own
// reference counts; in src the sequences are then freed in the order given, as
// pkv_seq_free would, so a block still mapped by a sequence left behind stays there.
int pkv_seq_migrate(pkv_pool *src, pkv_pool *dst, const int64_t *seq_ids, int32_t n, int32_t *pairs_out,
                    int32_t max_pairs, int32_t *n_pairs_out) {
    if (n_pairs_out) *n_pairs_out = 0;
    if (!src || !dst || src == dst || n < 0 || (n > 0 && !seq_ids) || max_pairs < 0 ||
        (max_pairs > 0 && !pairs_out))
        return fail(PKV_EINVAL, "pkv_seq_migrate: bad arguments");
    if (src->block_size != dst->block_size)
        return fail(PKV_EINVAL, "pkv_seq_migrate: block sizes differ (%d, %d)", src->block_size, dst->block_size);
    std::unordered_set<int64_t> seen;
    std::unordered_map<int32_t, int32_t> uses;  // src block -> references among the moved sequences
    std::vector<int32_t> order;                 // distinct src blocks, first use first
    for (int32_t i = 0; i < n; ++i) {
        const int64_t id = seq_ids[i];
        if (!seen.insert(id).second)
            return fail(PKV_EINVAL, "pkv_seq_migrate: sequence %lld given twice", (long long)id);
        auto it = src->seqs.find(id);
        if (it == src->seqs.end())
            return fail(PKV_ENOSEQ, "pkv_seq_migrate: unknown sequence %lld", (long long)id);
        if (dst->seqs.count(id)) return fail(PKV_EEXIST, "pkv_seq_migrate: sequence %lld exists in dst", (long long)id);
        for (int32_t b : it->second.blocks)
            if (uses[b]++ == 0) order.push_back(b);
    }
    const int32_t need = static_cast<int32_t>(order.size());
    if (need > max_pairs)
        return fail(PKV_EINVAL, "pkv_seq_migrate: %d blocks to move, room for %d pairs", need, max_pairs);
    if (need > dst->available())
        return fail(PKV_ENOMEM, "pkv_seq_migrate: %d blocks needed, %lld free", need, (long long)dst->available());
    std::unordered_map<int32_t, int32_t> to;
    for (int32_t k = 0; k < need; ++k) {
        const int32_t b = order[k], d = dst->take();
        dst->ref[d] = uses[b];
        to[b] = d;
        pairs_out[2 * k] = b;
        pairs_out[2 * k + 1] = d;
    }
    for (int32_t i = 0; i < n; ++i) {
        auto it = src->seqs.find(seq_ids[i]);
        pkv_pool::Seq moved;
        moved.len = it->second.len;
        moved.blocks.reserve(it->second.blocks.size());
        for (int32_t b : it->second.blocks) {
            moved.blocks.push_back(to[b]);
            if (--src->ref[b] == 0) src->release(b);
        }
        dst->seqs.emplace(seq_ids[i], std::move(moved));
        src->seqs.erase(it);
    }
    if (n_pairs_out) *n_pairs_out = need;
    return PKV_OK;
}

}  // extern "C"
