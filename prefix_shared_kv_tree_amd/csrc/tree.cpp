// Host prefix tree: arrival, decode append, departure (ChunkAttention digest,
// Knowl 1).  See tree.h for the readings of the page.
#include "tree.h"

#include <algorithm>
#include <cstring>

#include "pkvt.h"

namespace pkvt {

Tree::Tree(int32_t h, int32_t d, int32_t c, int32_t pool_chunks)
    : H(h), D(d), C(c), N(pool_chunks), nodes_(static_cast<size_t>(pool_chunks) + 1) {
    free_.reserve(pool_chunks);
    for (int32_t i = pool_chunks - 1; i >= 0; --i) free_.push_back(i);   // pops 0, 1, 2, ...
    nodes_[N].live = true;                                               // the root
}

uint64_t Tree::hash_tokens(const int32_t* t) const {
    uint64_t h = 1469598103934665603ull;                 // FNV-1a over the c token ids
    for (int32_t i = 0; i < C; ++i) {
        uint32_t v = static_cast<uint32_t>(t[i]);
        for (int b = 0; b < 4; ++b) {
            h ^= (v >> (8 * b)) & 0xffu;
            h *= 1099511628211ull;
        }
    }
    return h;
}

int32_t Tree::find_full_child(int32_t parent, const int32_t* t) const {
    const Node& p = nodes_[parent];
    auto it = p.full_children.find(hash_tokens(t));
    if (it == p.full_children.end()) return -1;
    for (int32_t ch : it->second)                        // creation order: earliest first
        if (std::memcmp(nodes_[ch].tokens.data(), t, sizeof(int32_t) * C) == 0) return ch;
    return -1;
}

void Tree::index_full(int32_t id) {
    Node& n = nodes_[id];
    n.key_hash = hash_tokens(n.tokens.data());
    auto& bucket = nodes_[n.parent].full_children[n.key_hash];
    auto pos = std::upper_bound(bucket.begin(), bucket.end(), n.created,
                                [this](int64_t c, int32_t x) { return c < nodes_[x].created; });
    bucket.insert(pos, id);
}

void Tree::unindex_full(int32_t id) {
    Node& n = nodes_[id];
    auto& map = nodes_[n.parent].full_children;
    auto it = map.find(n.key_hash);
    if (it == map.end()) return;
    auto& bucket = it->second;
    bucket.erase(std::remove(bucket.begin(), bucket.end(), id), bucket.end());
    if (bucket.empty()) map.erase(it);
}

int32_t Tree::alloc_node(int32_t parent, const int32_t* t, int32_t n) {
    int32_t id = free_.back();
    free_.pop_back();
    Node& x = nodes_[id];
    x.parent = parent;
    x.fill = n;
    x.refs = 0;
    x.created = next_created_++;
    x.live = true;
    x.children.clear();
    x.full_children.clear();
    x.tokens.assign(t, t + n);
    nodes_[parent].children.push_back(id);
    if (n == C) index_full(id);
    return id;
}

void Tree::free_node(int32_t id) {
    Node& x = nodes_[id];
    if (x.fill == C) unindex_full(id);
    auto& sib = nodes_[x.parent].children;
    sib.erase(std::remove(sib.begin(), sib.end(), id), sib.end());
    x.live = false;
    x.refs = 0;
    x.fill = 0;
    x.tokens.clear();
    x.children.clear();
    x.full_children.clear();
    free_.push_back(id);
}

int32_t Tree::shared_chunks() const {
    int32_t s = 0;
    for (int32_t i = 0; i < N; ++i)
        if (nodes_[i].live && nodes_[i].refs >= 2) ++s;
    return s;
}

const Seq* Tree::find_seq(int32_t id) const {
    auto it = seqs_.find(id);
    return it == seqs_.end() ? nullptr : &it->second;
}

int Tree::build(int32_t n_seqs, const int32_t* tokens, const int64_t* offsets,
                int32_t* seq_ids, int64_t* slots, std::string& err) {
    if (n_seqs < 0 || (n_seqs > 0 && (!tokens || !offsets || !seq_ids || !slots))) {
        err = "tree_build: null pointer or negative n_seqs";
        return PKVT_ERR_INVALID_ARG;
    }
    if (n_seqs > 0 && offsets[0] != 0) {
        err = "tree_build: offsets[0] must be 0";
        return PKVT_ERR_INVALID_ARG;
    }
    for (int32_t s = 0; s < n_seqs; ++s) {
        if (offsets[s + 1] < offsets[s]) {
            err = "tree_build: offsets must be non-decreasing";
            return PKVT_ERR_INVALID_ARG;
        }
        if (offsets[s + 1] == offsets[s]) {
            err = "tree_build: sequence " + std::to_string(s) + " is empty";
            return PKVT_ERR_EMPTY_SEQ;
        }
    }
    // Everything below is undone on NO_CHUNKS.
    std::vector<int32_t> created;
    std::vector<int32_t> added;
    const int32_t seq_mark = next_seq_;
    const int64_t created_mark = next_created_;
    auto rollback = [&]() {
        for (int32_t id : added) {
            for (int32_t x : seqs_[id].path) nodes_[x].refs--;
            seqs_.erase(id);
        }
        for (auto it = created.rbegin(); it != created.rend(); ++it) free_node(*it);
        next_seq_ = seq_mark;
        next_created_ = created_mark;
    };
    for (int32_t s = 0; s < n_seqs; ++s) {
        const int64_t beg = offsets[s], L = offsets[s + 1] - offsets[s];
        const int32_t* t = tokens + beg;
        Seq seq;
        seq.len = L;
        int32_t at = root();
        bool matching = true;
        for (int64_t pos = 0; pos < L;) {
            const int32_t n = static_cast<int32_t>(std::min<int64_t>(C, L - pos));
            int32_t id = (matching && n == C) ? find_full_child(at, t + pos) : -1;
            if (id >= 0) {
                for (int32_t k = 0; k < n; ++k) slots[beg + pos + k] = -1;
            } else {
                matching = false;
                if (free_.empty()) {
                    rollback();
                    err = "tree_build: chunk pool exhausted (" + std::to_string(N) + " chunks)";
                    return PKVT_ERR_NO_CHUNKS;
                }
                id = alloc_node(at, t + pos, n);
                created.push_back(id);
                for (int32_t k = 0; k < n; ++k)
                    slots[beg + pos + k] = static_cast<int64_t>(id) * C + k;
            }
            seq.path.push_back(id);
            at = id;
            pos += n;
        }
        for (int32_t x : seq.path) nodes_[x].refs++;
        const int32_t sid = next_seq_++;
        seqs_.emplace(sid, std::move(seq));
        added.push_back(sid);
        seq_ids[s] = sid;
    }
    if (n_seqs > 0) ++struct_version_;
    return PKVT_OK;
}

int Tree::append(int32_t n, const int32_t* seq_ids, const int32_t* tokens, int64_t* slots,
                 std::string& err) {
    if (n < 0 || (n > 0 && (!seq_ids || !tokens || !slots))) {
        err = "tree_append: null pointer or negative n";
        return PKVT_ERR_INVALID_ARG;
    }
    struct Step { int32_t sid; int32_t node; bool created; bool filled; };
    std::vector<Step> log;
    log.reserve(n);
    auto rollback = [&]() {
        for (auto it = log.rbegin(); it != log.rend(); ++it) {
            Seq& s = seqs_[it->sid];
            s.len--;
            if (it->created) {
                s.path.pop_back();
                free_node(it->node);
                next_created_--;
            } else {
                Node& x = nodes_[it->node];
                if (it->filled) unindex_full(it->node);
                x.tokens.pop_back();
                x.fill--;
            }
        }
    };
    bool structural = false;
    for (int32_t i = 0; i < n; ++i) {
        auto it = seqs_.find(seq_ids[i]);
        if (it == seqs_.end()) {
            rollback();
            err = "tree_append: unknown sequence id " + std::to_string(seq_ids[i]);
            return PKVT_ERR_UNKNOWN_SEQ;
        }
        Seq& s = it->second;
        const int32_t leaf = s.path.back();
        Node& x = nodes_[leaf];
        if (x.fill < C) {
            // a partial leaf is always private to its sequence
            x.tokens.push_back(tokens[i]);
            x.fill++;
            const bool filled = (x.fill == C);
            if (filled) index_full(leaf);
            slots[i] = static_cast<int64_t>(leaf) * C + (x.fill - 1);
            log.push_back({it->first, leaf, false, filled});
        } else {
            if (free_.empty()) {
                rollback();
                err = "tree_append: chunk pool exhausted (" + std::to_string(N) + " chunks)";
                return PKVT_ERR_NO_CHUNKS;
            }
            const int32_t id = alloc_node(leaf, tokens + i, 1);
            nodes_[id].refs = 1;
            s.path.push_back(id);
            slots[i] = static_cast<int64_t>(id) * C;
            log.push_back({it->first, id, true, false});
            structural = true;
        }
        s.len++;
    }
    if (n > 0) ++len_version_;
    if (structural) ++struct_version_;
    return PKVT_OK;
}

int Tree::remove(int32_t seq_id, std::string& err) {
    auto it = seqs_.find(seq_id);
    if (it == seqs_.end()) {
        err = "tree_remove: unknown sequence id " + std::to_string(seq_id);
        return PKVT_ERR_UNKNOWN_SEQ;
    }
    const std::vector<int32_t> path = it->second.path;
    seqs_.erase(it);
    for (auto p = path.rbegin(); p != path.rend(); ++p) {
        Node& x = nodes_[*p];
        if (--x.refs == 0) free_node(*p);               // leaf first: children already gone
    }
    ++struct_version_;
    return PKVT_OK;
}

}  // namespace pkvt
