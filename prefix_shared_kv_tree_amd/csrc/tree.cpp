// Host prefix tree: arrival, decode append, departure (ChunkAttention digest,
// Knowl 1).  See tree.h for the readings of the page.
#include "tree.h"

#include <algorithm>
#include <cstring>
#include <memory>

#include "pkvt.h"

namespace pkvt {

Tree::Tree(int32_t h, int32_t d, int32_t c, int32_t pool_chunks, Match m)
    : H(h), D(d), C(c), N(pool_chunks), match(m), nodes_(static_cast<size_t>(pool_chunks) + 1) {
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
    if (match != Match::kChunks) return;                 // token matching compares prefixes
    Node& n = nodes_[id];
    n.key_hash = hash_tokens(n.tokens.data());
    auto& bucket = nodes_[n.parent].full_children[n.key_hash];
    auto pos = std::upper_bound(bucket.begin(), bucket.end(), n.created,
                                [this](int64_t c, int32_t x) { return c < nodes_[x].created; });
    bucket.insert(pos, id);
}

void Tree::unindex_full(int32_t id) {
    if (match != Match::kChunks) return;
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
    moves_.clear();
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
    if (match == Match::kTokens) return build_tokens(n_seqs, tokens, offsets, seq_ids, slots, err);
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
    if (n_seqs > 0) reshaped();
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
        if (x.fill < C && x.refs == 1 && x.children.empty()) {
            // a partial, private, childless leaf (with whole-chunk matching
            // every partial leaf is one)
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
    if (structural) {
        ++struct_version_;
        if (grown_.size() + log.size() > kMaxGrown) {
            reshaped();                                 // too many to patch: plan afresh
        } else {
            for (const Step& st : log)
                if (st.created) grown_.emplace_back(struct_version_, st.sid);
        }
    }
    return PKVT_OK;
}

// Token-granular arrival (see tree.h).  Slots are assigned once all prompts
// are in, from the final paths, because a later prompt of the same call may
// split a node an earlier one created.  A split's new node records where its
// tokens' K/V physically are (src); nodes created by this call that are not
// in src hold only tokens the caller has yet to write.
int Tree::build_tokens(int32_t n_seqs, const int32_t* tokens, const int64_t* offsets,
                       int32_t* seq_ids, int64_t* slots, std::string& err) {
    // At most one split and ceil(L / c) new chunks per prompt: with that many
    // free chunks the call cannot fail, otherwise keep a copy to roll back to.
    int64_t bound = 0;
    for (int32_t s = 0; s < n_seqs; ++s) bound += (offsets[s + 1] - offsets[s] + C - 1) / C + 1;
    struct Snapshot {
        std::vector<Node> nodes;
        std::vector<int32_t> free;
        std::unordered_map<int32_t, Seq> seqs;
        int32_t next_seq;
        int64_t next_created;
    };
    std::unique_ptr<Snapshot> snap;
    if (bound > static_cast<int64_t>(free_.size()))
        snap.reset(new Snapshot{nodes_, free_, seqs_, next_seq_, next_created_});
    auto out_of_chunks = [&]() {
        nodes_ = std::move(snap->nodes);
        free_ = std::move(snap->free);
        seqs_ = std::move(snap->seqs);
        next_seq_ = snap->next_seq;
        next_created_ = snap->next_created;
        moves_.clear();
        err = "tree_build: chunk pool exhausted (" + std::to_string(N) + " chunks)";
        return PKVT_ERR_NO_CHUNKS;
    };
    const int64_t created_mark = next_created_;
    std::unordered_map<int32_t, std::vector<int64_t>> src;
    auto src_of = [&](int32_t id, int32_t k) -> int64_t {
        auto it = src.find(id);
        if (it != src.end()) return it->second[k];
        return nodes_[id].created >= created_mark ? -1 : static_cast<int64_t>(id) * C + k;
    };
    auto split = [&](int32_t y, int32_t t) {
        const int32_t id = free_.back();
        free_.pop_back();
        Node& x = nodes_[id];
        Node& old = nodes_[y];
        x.parent = y;
        x.fill = old.fill - t;
        x.refs = old.refs;
        x.created = next_created_++;
        x.live = true;
        x.full_children.clear();
        x.tokens.assign(old.tokens.begin() + t, old.tokens.end());
        x.children = std::move(old.children);
        for (int32_t ch : x.children) nodes_[ch].parent = id;
        std::vector<int64_t> from(x.fill);
        bool any = false;
        for (int32_t k = 0; k < x.fill; ++k) any |= (from[k] = src_of(y, t + k)) >= 0;
        if (any) src[id] = std::move(from);
        auto it = src.find(y);
        if (it != src.end()) it->second.resize(t);
        old.children.assign(1, id);
        old.tokens.resize(t);
        old.fill = t;
        for (auto& kv : seqs_) {
            std::vector<int32_t>& path = kv.second.path;
            auto at = std::find(path.begin(), path.end(), y);
            if (at != path.end()) path.insert(at + 1, id);
        }
    };
    std::vector<int64_t> matched(n_seqs);
    for (int32_t s = 0; s < n_seqs; ++s) {
        const int64_t beg = offsets[s], L = offsets[s + 1] - offsets[s];
        const int32_t* t = tokens + beg;
        Seq seq;
        seq.len = L;
        int32_t at = root();
        int64_t pos = 0;
        while (pos < L) {
            int32_t best = -1, best_len = 0;
            for (int32_t ch : nodes_[at].children) {          // creation order
                const Node& x = nodes_[ch];
                const int32_t lim = static_cast<int32_t>(std::min<int64_t>(x.fill, L - pos));
                int32_t k = 0;
                while (k < lim && x.tokens[k] == t[pos + k]) ++k;
                if (k > best_len) {
                    best = ch;
                    best_len = k;
                }
            }
            if (best < 0) break;
            if (best_len < nodes_[best].fill) {
                if (free_.empty()) return out_of_chunks();
                split(best, best_len);
            }
            seq.path.push_back(best);
            at = best;
            pos += best_len;
        }
        matched[s] = pos;
        while (pos < L) {
            if (free_.empty()) return out_of_chunks();
            const int32_t n = static_cast<int32_t>(std::min<int64_t>(C, L - pos));
            at = alloc_node(at, t + pos, n);
            seq.path.push_back(at);
            pos += n;
        }
        for (int32_t x : seq.path) nodes_[x].refs++;
        const int32_t sid = next_seq_++;
        seqs_.emplace(sid, std::move(seq));
        seq_ids[s] = sid;
    }
    // slots from the final paths: tokens a prompt did not match are its own
    for (int32_t s = 0; s < n_seqs; ++s) {
        int64_t p = 0;
        int64_t* out = slots + offsets[s];
        for (int32_t x : seqs_[seq_ids[s]].path)
            for (int32_t k = 0; k < nodes_[x].fill; ++k, ++p)
                out[p] = p >= matched[s] ? static_cast<int64_t>(x) * C + k : -1;
    }
    for (const auto& kv : src)
        for (int32_t k = 0; k < nodes_[kv.first].fill; ++k)
            if (kv.second[k] >= 0) moves_.emplace_back(kv.second[k], static_cast<int64_t>(kv.first) * C + k);
    std::sort(moves_.begin(), moves_.end());
    if (n_seqs > 0) reshaped();
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
    reshaped();
    return PKVT_OK;
}

}  // namespace pkvt
