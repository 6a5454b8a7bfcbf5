// Host-side KV-cache block manager (C ABI in include/pa_block_manager.h).
//
// Free list, reference counts, copy-on-write trigger, prefix caching and
// swap bookkeeping, as the PagedAttention digest's "Method" (core
// components, flowchart), the continuous-batching page's sections 2 and 4,
// and the KV-cache page's prefix-caching note describe them; the policies
// the pages leave open are listed in the header.
//
// Prefix identity.  A full block is identified by the whole token prefix up
// to its end.  Prefixes are interned as nodes of a trie: node = (parent
// node, the block's B tokens), parent 0 = the empty prefix.  Two blocks have
// the same identity exactly when they map to the same node, so lookups
// compare whole prefixes without storing them.  Nodes are reference counted
// (by the sequences whose full blocks they identify, by the cache entry that
// names a block for them, and by their child nodes) and freed at zero.
#include <algorithm>
#include <cstring>
#include <deque>
#include <list>
#include <new>
#include <string>
#include <unordered_map>
#include <vector>

#include "../../include/pa.h"
#include "../../include/pa_block_manager.h"

namespace {

struct Seq {
    std::vector<int32_t> table;  // physical block of each logical block
    int64_t len = 0;             // tokens
    std::vector<int32_t> tail;   // tokens of the partly filled last block (prefix caching)
    std::vector<int64_t> keys;   // prefix node of each full block (prefix caching)
};

struct Node {
    int64_t parent = 0;
    int64_t refs = 0;
    std::string key;  // parent id + tokens, the interning key
};

class Manager {
public:
    Manager(int64_t n, int32_t b, bool prefix) : num_blocks_(n), B_(b), prefix_(prefix), ref_(n, 0), key_of_(n, 0),
                                                   lru_pos_(n) {}

    std::deque<int32_t> free_;

    int64_t num_blocks() const { return num_blocks_; }
    int32_t block_size() const { return B_; }
    bool prefix() const { return prefix_; }
    int64_t num_free() const { return static_cast<int64_t>(free_.size() + lru_.size()); }
    int64_t num_cached() const { return static_cast<int64_t>(cache_.size()); }
    int32_t ref(int32_t b) const { return ref_[b]; }
    Seq* find(int64_t s) {
        auto it = seqs_.find(s);
        return it == seqs_.end() ? nullptr : &it->second;
    }
    const Seq* find(int64_t s) const {
        auto it = seqs_.find(s);
        return it == seqs_.end() ? nullptr : &it->second;
    }

    int32_t blocks_needed(const Seq& q, int64_t n) const {
        const int64_t held = (q.len + B_ - 1) / B_;
        int64_t need = (q.len + n + B_ - 1) / B_ - held;
        if (n > 0 && q.len % B_ && ref_[q.table.back()] > 1) need += 1;
        return static_cast<int32_t>(need);
    }

    int32_t allocate() {
        int32_t b;
        if (!free_.empty()) {
            b = free_.front();
            free_.pop_front();
        } else {
            b = lru_.front();
            lru_.pop_front();
            uncache(b);
        }
        ref_[b] = 1;
        return b;
    }

    void release(int32_t b) {
        if (--ref_[b] == 0) {
            if (key_of_[b]) {
                lru_.push_back(b);
                lru_pos_[b] = std::prev(lru_.end());
            } else {
                free_.push_back(b);
            }
        }
    }

    void share(int32_t b) {
        if (ref_[b]++ == 0) lru_.erase(lru_pos_[b]);  // a released cached block taken back
    }

    // ---- prefix nodes
    std::string node_key(int64_t parent, const int32_t* toks) const {
        std::string k(sizeof(int64_t) + sizeof(int32_t) * B_, '\0');
        std::memcpy(&k[0], &parent, sizeof(int64_t));
        std::memcpy(&k[sizeof(int64_t)], toks, sizeof(int32_t) * B_);
        return k;
    }
    int64_t lookup(int64_t parent, const int32_t* toks) const {
        auto it = intern_.find(node_key(parent, toks));
        return it == intern_.end() ? 0 : it->second;
    }
    // Node for (parent, toks), created if new; one more holder.
    int64_t acquire(int64_t parent, const int32_t* toks) {
        std::string k = node_key(parent, toks);
        auto it = intern_.find(k);
        if (it != intern_.end()) {
            ++nodes_[it->second].refs;
            return it->second;
        }
        const int64_t id = next_node_++;
        Node& nd = nodes_[id];
        nd.parent = parent;
        nd.refs = 1;
        nd.key = k;
        if (parent) ++nodes_[parent].refs;
        intern_.emplace(std::move(k), id);
        return id;
    }
    void hold(int64_t id) { ++nodes_[id].refs; }
    void drop(int64_t id) {
        while (id) {
            auto it = nodes_.find(id);
            if (--it->second.refs > 0) return;
            const int64_t parent = it->second.parent;
            intern_.erase(it->second.key);
            nodes_.erase(it);
            id = parent;
        }
    }
    // Tokens of a node (its own block), for re-interning in another manager.
    const int32_t* node_tokens(int64_t id) const {
        return reinterpret_cast<const int32_t*>(nodes_.at(id).key.data() + sizeof(int64_t));
    }

    // ---- cache
    int32_t cached_block(int64_t node) const {
        auto it = cache_.find(node);
        return it == cache_.end() ? -1 : it->second;
    }
    void cache_block(int64_t node, int32_t b) {
        cache_.emplace(node, b);
        key_of_[b] = node;
        hold(node);
    }
    void uncache(int32_t b) {
        const int64_t node = key_of_[b];
        cache_.erase(node);
        key_of_[b] = 0;
        drop(node);
    }

    std::unordered_map<int64_t, Seq> seqs_;

private:
    int64_t num_blocks_;
    int32_t B_;
    bool prefix_;
    std::vector<int32_t> ref_;
    std::vector<int64_t> key_of_;  // cached node of each block (0 = none)
    std::list<int32_t> lru_;       // released cached blocks, least recently released first
    std::vector<std::list<int32_t>::iterator> lru_pos_;
    std::unordered_map<int64_t, int32_t> cache_;  // node -> block
    std::unordered_map<int64_t, Node> nodes_;
    std::unordered_map<std::string, int64_t> intern_;
    int64_t next_node_ = 1;
};

// Append n tokens to q (capacity already checked).
void append_tokens(Manager& m, Seq& q, int32_t n, const int32_t* tokens, int64_t* slots, int64_t* pair,
                   int32_t* num_pairs) {
    const int32_t B = m.block_size();
    int32_t np = 0;
    for (int32_t i = 0; i < n; ++i) {
        const int64_t pos = q.len;
        const size_t j = static_cast<size_t>(pos / B);
        const int32_t off = static_cast<int32_t>(pos % B);
        if (j == q.table.size()) {
            q.table.push_back(m.allocate());
        } else if (m.ref(q.table[j]) > 1) {
            const int32_t nb = m.allocate();
            if (pair) {
                pair[0] = q.table[j];
                pair[1] = nb;
            }
            ++np;
            m.release(q.table[j]);
            q.table[j] = nb;
        }
        if (slots) slots[i] = static_cast<int64_t>(q.table[j]) * B + off;
        ++q.len;
        if (m.prefix()) {
            q.tail.push_back(tokens[i]);
            if (off == B - 1) {
                const int64_t parent = q.keys.empty() ? 0 : q.keys.back();
                const int64_t node = m.acquire(parent, q.tail.data());
                q.keys.push_back(node);
                q.tail.clear();
                if (m.cached_block(node) < 0) m.cache_block(node, q.table[j]);
            }
        }
    }
    if (num_pairs) *num_pairs = np;
}

void release_seq(Manager& m, Seq& q) {
    for (int32_t b : q.table) m.release(b);
    for (int64_t k : q.keys) m.drop(k);
}

// Re-express q's prefix nodes (from `from`) in `to`.
std::vector<int64_t> move_keys(const Manager& from, Manager& to, const std::vector<int64_t>& keys) {
    std::vector<int64_t> out;
    out.reserve(keys.size());
    int64_t parent = 0;
    for (int64_t k : keys) {
        parent = to.acquire(parent, from.node_tokens(k));
        out.push_back(parent);
    }
    return out;  // one hold per node for the moved sequence, as append gives it
}

// Move `seq` from src to dst onto freshly allocated dst blocks; pairs
// receives (src block, dst block) in table order.
int move_seq(Manager& src, Manager& dst, int64_t seq, int64_t* pairs, int32_t capacity, int32_t* num_pairs) {
    Seq* q = src.find(seq);
    if (!q || dst.find(seq) || src.block_size() != dst.block_size()) return PA_ERR_INVALID;
    const int64_t n = static_cast<int64_t>(q->table.size());
    if (n > capacity || (n && !pairs)) return PA_ERR_INVALID;
    if (dst.num_free() < n) return PA_ERR_OUT_OF_BLOCKS;
    Seq moved;
    moved.len = q->len;
    moved.tail = q->tail;
    moved.keys = move_keys(src, dst, q->keys);
    for (int64_t i = 0; i < n; ++i) {
        const int32_t b = dst.allocate();
        moved.table.push_back(b);
        pairs[2 * i] = q->table[i];
        pairs[2 * i + 1] = b;
    }
    release_seq(src, *q);
    src.seqs_.erase(seq);
    dst.seqs_.emplace(seq, std::move(moved));
    if (num_pairs) *num_pairs = static_cast<int32_t>(n);
    return PA_OK;
}

}  // namespace

struct pa_bm {
    Manager m;
};

extern "C" {

pa_bm* pa_bm_create(int64_t num_blocks, int32_t block_size, const int32_t* free_order, int32_t prefix_cache) {
    if (num_blocks < 1 || num_blocks >= (int64_t{1} << 31) || block_size < 1 || block_size > 65536) return nullptr;
    pa_bm* bm = new (std::nothrow) pa_bm{Manager(num_blocks, block_size, prefix_cache != 0)};
    if (!bm) return nullptr;
    if (free_order) {
        std::vector<char> seen(static_cast<size_t>(num_blocks), 0);
        for (int64_t i = 0; i < num_blocks; ++i) {
            const int32_t b = free_order[i];
            if (b < 0 || b >= num_blocks || seen[b]) {
                delete bm;
                return nullptr;
            }
            seen[b] = 1;
            bm->m.free_.push_back(b);
        }
    } else {
        for (int64_t i = 0; i < num_blocks; ++i) bm->m.free_.push_back(static_cast<int32_t>(i));
    }
    return bm;
}

void pa_bm_destroy(pa_bm* bm) { delete bm; }

int pa_bm_add_seq(pa_bm* bm, int64_t seq, const int32_t* prompt, int32_t prompt_len, int32_t* cached_tokens) {
    if (!bm) return PA_ERR_NULL;
    if (prompt_len < 0 || (prompt_len > 0 && !prompt)) return PA_ERR_INVALID;
    Manager& m = bm->m;
    if (m.find(seq)) return PA_ERR_INVALID;
    Seq q;
    if (m.prefix() && prompt_len > 0) {
        const int32_t B = m.block_size();
        int64_t parent = 0;
        std::vector<int32_t> hit;
        std::vector<int64_t> nodes;
        for (int32_t j = 0; j < (prompt_len - 1) / B; ++j) {
            const int64_t node = m.lookup(parent, prompt + static_cast<int64_t>(j) * B);
            const int32_t b = node ? m.cached_block(node) : -1;
            if (b < 0) break;
            hit.push_back(b);
            nodes.push_back(node);
            parent = node;
        }
        for (size_t i = 0; i < hit.size(); ++i) {
            m.share(hit[i]);
            m.hold(nodes[i]);
        }
        q.table = hit;
        q.keys = nodes;
        q.len = static_cast<int64_t>(hit.size()) * B;
    }
    if (cached_tokens) *cached_tokens = static_cast<int32_t>(q.len);
    m.seqs_.emplace(seq, std::move(q));
    return PA_OK;
}

int pa_bm_append(pa_bm* bm, int64_t seq, int32_t n, const int32_t* tokens, int64_t* slots, int64_t* pair,
                 int32_t* num_pairs) {
    if (!bm) return PA_ERR_NULL;
    Manager& m = bm->m;
    Seq* q = m.find(seq);
    if (!q || n < 0) return PA_ERR_INVALID;
    if (n > 0 && (!slots || (m.prefix() && !tokens))) return PA_ERR_NULL;
    if (m.blocks_needed(*q, n) > m.num_free()) return PA_ERR_OUT_OF_BLOCKS;
    append_tokens(m, *q, n, tokens, slots, pair, num_pairs);
    return PA_OK;
}

int pa_bm_append_batch(pa_bm* bm, const int64_t* seqs, int32_t n_seqs, const int32_t* tokens, int64_t* slots,
                       int64_t* pairs, int32_t* num_pairs, int32_t* done) {
    if (!bm) return PA_ERR_NULL;
    Manager& m = bm->m;
    if (n_seqs < 0) return PA_ERR_INVALID;
    if (n_seqs > 0 && (!seqs || !slots || !pairs || (m.prefix() && !tokens))) return PA_ERR_NULL;
    int32_t np = 0, i = 0;
    int status = PA_OK;
    for (; i < n_seqs; ++i) {
        Seq* q = m.find(seqs[i]);
        if (!q) {
            status = PA_ERR_INVALID;
            break;
        }
        if (m.blocks_needed(*q, 1) > m.num_free()) {
            status = PA_ERR_OUT_OF_BLOCKS;
            break;
        }
        int32_t k = 0;
        append_tokens(m, *q, 1, tokens ? tokens + i : nullptr, slots + i, pairs + 2 * np, &k);
        np += k;
    }
    if (num_pairs) *num_pairs = np;
    if (done) *done = i;
    return status;
}

int pa_bm_fork(pa_bm* bm, int64_t parent, int64_t child) {
    if (!bm) return PA_ERR_NULL;
    Manager& m = bm->m;
    const Seq* p = m.find(parent);
    if (!p || m.find(child)) return PA_ERR_INVALID;
    Seq c = *p;
    for (int32_t b : c.table) m.share(b);
    for (int64_t k : c.keys) m.hold(k);
    m.seqs_.emplace(child, std::move(c));
    return PA_OK;
}

int pa_bm_free_seq(pa_bm* bm, int64_t seq) {
    if (!bm) return PA_ERR_NULL;
    Manager& m = bm->m;
    Seq* q = m.find(seq);
    if (!q) return PA_ERR_INVALID;
    release_seq(m, *q);
    m.seqs_.erase(seq);
    return PA_OK;
}

int pa_bm_swap_out(pa_bm* bm, pa_bm* host, int64_t seq, int64_t* pairs, int32_t capacity, int32_t* num_pairs) {
    if (!bm || !host) return PA_ERR_NULL;
    if (bm == host) return PA_ERR_INVALID;
    return move_seq(bm->m, host->m, seq, pairs, capacity, num_pairs);
}

int pa_bm_swap_in(pa_bm* bm, pa_bm* host, int64_t seq, int64_t* pairs, int32_t capacity, int32_t* num_pairs) {
    if (!bm || !host) return PA_ERR_NULL;
    if (bm == host) return PA_ERR_INVALID;
    return move_seq(host->m, bm->m, seq, pairs, capacity, num_pairs);
}

int pa_bm_block_tables(const pa_bm* bm, const int64_t* seqs, int32_t n_seqs, int32_t width, int32_t* tables,
                       int32_t* lens) {
    if (!bm) return PA_ERR_NULL;
    if (n_seqs < 0 || width < 0) return PA_ERR_INVALID;
    if (n_seqs > 0 && (!seqs || (width > 0 && !tables))) return PA_ERR_NULL;
    const Manager& m = bm->m;
    for (int32_t i = 0; i < n_seqs; ++i) {
        const Seq* q = m.find(seqs[i]);
        if (!q || static_cast<int64_t>(q->table.size()) > width) return PA_ERR_INVALID;
    }
    for (int32_t i = 0; i < n_seqs; ++i) {
        const Seq* q = m.find(seqs[i]);
        int32_t* row = tables + static_cast<int64_t>(i) * width;
        std::copy(q->table.begin(), q->table.end(), row);
        std::fill(row + q->table.size(), row + width, -1);
        if (lens) lens[i] = static_cast<int32_t>(q->len);
    }
    return PA_OK;
}

int64_t pa_bm_num_free(const pa_bm* bm) { return bm ? bm->m.num_free() : -1; }

int64_t pa_bm_seq_len(const pa_bm* bm, int64_t seq) {
    const Seq* q = bm ? bm->m.find(seq) : nullptr;
    return q ? q->len : -1;
}

int32_t pa_bm_num_blocks_held(const pa_bm* bm, int64_t seq) {
    const Seq* q = bm ? bm->m.find(seq) : nullptr;
    return q ? static_cast<int32_t>(q->table.size()) : -1;
}

int32_t pa_bm_blocks_needed(const pa_bm* bm, int64_t seq, int32_t n) {
    const Seq* q = bm ? bm->m.find(seq) : nullptr;
    return (q && n >= 0) ? bm->m.blocks_needed(*q, n) : -1;
}

int32_t pa_bm_ref_count(const pa_bm* bm, int32_t block) {
    if (!bm || block < 0 || block >= bm->m.num_blocks()) return -1;
    return bm->m.ref(block);
}

int64_t pa_bm_num_cached(const pa_bm* bm) { return bm ? bm->m.num_cached() : -1; }

}  // extern "C"
