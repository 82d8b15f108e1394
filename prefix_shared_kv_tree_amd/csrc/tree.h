// Host prefix tree over a fixed pool of KV chunks.
//
// Follows "ChunkAttention: Efficient Self-Attention with Prefix-Aware KV Cache
// and Two-Phase Partition" (chapterpal digest), Knowl 1: the KV cache is cut
// along the sequence axis into chunks of c tokens; chunks are nodes of a
// prefix tree (a forest: every distinct first chunk is a root child); every
// root-to-leaf path is one sequence; a pool allocator hands out fixed-size
// chunks and takes freed ones back without releasing memory.
//
// Readings of the page (it leaves them open):
//   * whole-chunk matching from token 0: only FULL chunks are shared, a
//     partial tail chunk is private, decode never writes into a shared chunk;
//   * a chunk filled by decode appends becomes matchable; nodes are never
//     merged; among live full children with equal tokens a lookup takes the
//     earliest created one.
//
// Token-granular matching (Match::kTokens), a variant the page does not
// describe (its nodes are whole chunks): a node holds 1..c tokens at the
// start of its chunk.  An arrival descends into the child sharing the
// longest common prefix with the rest of its prompt (ties: earliest created)
// and splits a child it matches only in part: the child keeps the matched
// tokens, a new node below it takes the rest and the old children, and the
// rest's K/V must move to the new node's chunk (moves()).  A decode append
// writes into the leaf only while it is partial, private and childless.
// Shared prefixes that end inside a chunk are then stored once, at the cost
// of partial chunks inside the tree.
#pragma once

#include <cstdint>
#include <string>
#include <unordered_map>
#include <vector>

namespace pkvt {

struct Node {
    int32_t parent = -1;                 // node id of the parent (the root is id N)
    int32_t fill = 0;                    // tokens stored in the chunk
    int32_t refs = 0;                    // live sequences whose path holds this node
    int64_t created = 0;                 // creation counter (lookup tie-break)
    bool live = false;
    uint64_t key_hash = 0;               // hash of the c tokens, valid when full
    std::vector<int32_t> children;       // creation order
    std::vector<int32_t> tokens;         // the fill tokens
    // full live children keyed by token hash, each bucket in creation order
    std::unordered_map<uint64_t, std::vector<int32_t>> full_children;
};

struct Seq {
    std::vector<int32_t> path;           // node (= chunk) ids, root to leaf
    int64_t len = 0;
};

enum class Match : int32_t { kChunks = 0, kTokens = 1 };

class Tree {
public:
    Tree(int32_t h, int32_t d, int32_t c, int32_t pool_chunks, Match match = Match::kChunks);

    int32_t H, D, C, N;
    Match match;
    int32_t root() const { return N; }

    // Return codes are the PKVT_* status values; err receives a message.
    int build(int32_t n_seqs, const int32_t* tokens, const int64_t* offsets,
              int32_t* seq_ids, int64_t* slots, std::string& err);
    int append(int32_t n, const int32_t* seq_ids, const int32_t* tokens,
               int64_t* slots, std::string& err);
    int remove(int32_t seq_id, std::string& err);

    const Seq* find_seq(int32_t id) const;
    const Node& node(int32_t id) const { return nodes_[id]; }
    int32_t used_chunks() const { return N - (int32_t)free_.size(); }
    int32_t shared_chunks() const;
    int32_t live_seqs() const { return (int32_t)seqs_.size(); }

    // K/V that the last build moved between slots (token matching): the
    // token at slot first now belongs at slot second.  Sources lie in chunks
    // that existed before that build, destinations in chunks it allocated.
    const std::vector<std::pair<int64_t, int64_t>>& moves() const { return moves_; }

    // Bumped on every change of which chunks form which paths.
    int64_t structure_version() const { return struct_version_; }
    // The structure version of the last change other than decode appends
    // that opened a new leaf chunk at the end of a sequence (arrival,
    // departure): a plan at or after it can follow the appends since by
    // extending the sequences' last work items (grown()).
    int64_t reshape_version() const { return reshape_version_; }
    // (structure version, sequence id) of every append that opened a new
    // leaf chunk since reshape_version(), in order.
    const std::vector<std::pair<int64_t, int32_t>>& grown() const { return grown_; }
    static constexpr size_t kMaxGrown = 1 << 16;
    // Bumped on every decode append (sequence lengths change).
    int64_t length_version() const { return len_version_; }

private:
    std::vector<Node> nodes_;            // N chunk nodes + the root at index N
    std::vector<int32_t> free_;          // stack of free chunk ids
    std::unordered_map<int32_t, Seq> seqs_;
    int32_t next_seq_ = 0;
    int64_t next_created_ = 0;
    int64_t struct_version_ = 0;
    int64_t len_version_ = 0;
    int64_t reshape_version_ = 0;
    std::vector<std::pair<int64_t, int32_t>> grown_;
    std::vector<std::pair<int64_t, int64_t>> moves_;

    // a structural change that is not an append opening a leaf chunk
    void reshaped() {
        ++struct_version_;
        reshape_version_ = struct_version_;
        grown_.clear();
    }

    int build_tokens(int32_t n_seqs, const int32_t* tokens, const int64_t* offsets,
                     int32_t* seq_ids, int64_t* slots, std::string& err);

    uint64_t hash_tokens(const int32_t* t) const;
    int32_t find_full_child(int32_t parent, const int32_t* t) const;
    void index_full(int32_t id);
    void unindex_full(int32_t id);
    int32_t alloc_node(int32_t parent, const int32_t* t, int32_t n);
    void free_node(int32_t id);
};

}  // namespace pkvt
