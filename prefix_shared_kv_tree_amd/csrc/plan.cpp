// Context generation (ChunkAttention chapterpal digest, Knowl 2 and Knowl 5).
//
// 1. Renumber the batch's sequences in depth-first leaf order, children in
//    creation order, so the batch sequences under any node are one
//    contiguous range [i, j) (Knowl 1's contiguity invariant).
// 2. Phase 1 (chunk-first): nodes covering >= min_share batch sequences;
//    chains of such nodes with the same [i, j) form one segment, cut into
//    items of at most phase1_chunks chunks.  Each item is a context tuple
//    (chunk list, i, j) and yields one partial (o, m, n) per covered row.
// 3. Phase 2 (sequence-first): the rest of each sequence's path -- always a
//    suffix, since coverage can only shrink towards the leaves -- cut into
//    items of at most phase2_chunks chunks.
//    Under token-granular matching a node may hold fewer than C tokens
//    anywhere on a path.  A kernel item addresses key k at chunk k / C, so an
//    item may end with a partial chunk but hold none before that: segments
//    and phase-2 runs are cut after every partial node, and an item that
//    ends in one carries the keys it lacks (tail).
// 4. A sequence with exactly one item, a phase-2 one, is finalised by that
//    item; every other sequence's partials are merged afterwards.
// 5. The attention kernel runs G persistent workgroups of 4 waves.  Work is
//    handed out longest first.  A phase-1 item's rows are cut into blocks
//    of up to 64; a block of more than 16 rows is a workgroup unit per head,
//    whose 4 waves split the loads of every step and share them through
//    LDS; it goes to the workgroup whose busiest wave is least loaded.  Every other (item, head)
//    -- phase 2, and phase-1 blocks of <= 16 rows -- is a single-wave task
//    that goes to the least loaded wave.  Items are cut so that no task is
//    longer than the mean per-wave load.
#include "plan.h"

#include <algorithm>
#include <queue>
#include <unordered_map>

#include "pkvt.h"

namespace pkvt {

namespace {

int64_t steps_of(int64_t keys) { return (keys + kKeysPerStep - 1) / kKeysPerStep; }

// Cost in quarter steps of a single-wave task: 4 per 64-key step plus a
// start-up share.  A workgroup-unit step costs each of the unit's 4 waves
// kUnitStepCost quarter steps: its waves issue a quarter of the loads each
// (measured under load: a unit step takes ~0.4 of a single-wave step).
int64_t task_cost(int64_t keys) { return 4 * steps_of(keys) + 1; }
int64_t unit_cost(int64_t keys) { return kUnitStepCost * steps_of(keys) + 1; }

int32_t steps_to_chunks(int64_t steps, int32_t C) {
    const int64_t ch = steps * kKeysPerStep / C;
    return static_cast<int32_t>(std::max<int64_t>(1, std::min<int64_t>(ch, 1 << 30)));
}

struct Range { int32_t i = 0, j = 0; };

// Row blocks of a phase-1 item with n_rows rows: blocks of kRowsPerUnit and
// the remainder, except that a remainder too small for a workgroup unit is
// avoided by cutting the rows into equal blocks when those are all large
// enough (80 rows: 40 + 40 rather than 64 + a 16-row single-wave task).
std::vector<int32_t> row_blocks(int32_t n_rows, int32_t unit_rows) {
    std::vector<int32_t> out;
    const int32_t k = (n_rows + kRowsPerUnit - 1) / kRowsPerUnit;
    const int32_t rem = n_rows % kRowsPerUnit;
    if (k > 1 && rem != 0 && rem < unit_rows && n_rows / k >= unit_rows) {
        for (int32_t i = 0; i < k; ++i) out.push_back(n_rows / k + (i < n_rows % k ? 1 : 0));
        return out;
    }
    for (int32_t r0 = 0; r0 < n_rows; r0 += kRowsPerUnit) out.push_back(std::min(kRowsPerUnit, n_rows - r0));
    return out;
}

// The lanes of one speed class, ordered by (load, lane).  The balancer only
// ever takes the first lane and puts it back with a larger load, so the
// class minimum never decreases: lanes sit in a ring of buckets, one per
// load value, each a bitset over the class's lanes.  When the loads span
// too many values for that, a 4-ary heap of (load << lane_bits | lane) keys
// does the same job.
class LaneQueue {
public:
    void init(int32_t lo, int32_t n, const std::vector<int64_t>& load, int64_t max_cost) {
        lo_ = lo;
        n_ = n;
        if (n <= 0) return;
        int64_t mn = load[lo], mx = load[lo];
        for (int32_t l = lo; l < lo + n; ++l) {
            mn = std::min(mn, load[l]);
            mx = std::max(mx, load[l]);
        }
        words_ = (static_cast<size_t>(n) + 63) / 64;
        size_t ring = 1;
        while (ring <= static_cast<size_t>(mx - mn + max_cost)) ring <<= 1;
        bucket_mode_ = ring * words_ <= (size_t{1} << 22);
        if (bucket_mode_) {
            mask_ = ring - 1;
            bits_.assign(ring * words_, 0);
            cnt_.assign(ring, 0);
            cur_ = mn;
            wc_ = 0;
            for (int32_t l = lo; l < lo + n; ++l) add(l, load[l]);
        } else {
            lane_bits_ = 1;
            while ((int64_t{1} << lane_bits_) < lo + n) ++lane_bits_;
            heap_.clear();
            heap_.reserve(n);
            for (int32_t l = lo; l < lo + n; ++l) heap_push((static_cast<uint64_t>(load[l]) << lane_bits_) | l);
        }
    }
    bool empty() const { return n_ <= 0; }
    int64_t min_load() {
        if (!bucket_mode_) return static_cast<int64_t>(heap_[0] >> lane_bits_);
        while (cnt_[cur_ & mask_] == 0) {
            ++cur_;
            wc_ = 0;
        }
        return cur_;
    }
    // Take the first lane, give it load min_load() + cost, return it.
    int32_t take(int64_t cost) {
        const int64_t l0 = min_load();
        if (!bucket_mode_) {
            const int32_t lane = static_cast<int32_t>(heap_[0] & ((uint64_t{1} << lane_bits_) - 1));
            heap_replace_top((static_cast<uint64_t>(l0 + cost) << lane_bits_) | lane);
            return lane;
        }
        uint64_t* w = &bits_[(l0 & mask_) * words_];
        while (w[wc_] == 0) ++wc_;
        const int bit = __builtin_ctzll(w[wc_]);
        w[wc_] &= w[wc_] - 1;
        cnt_[l0 & mask_]--;
        const int32_t lane = lo_ + static_cast<int32_t>(wc_ * 64) + bit;
        add(lane, l0 + cost);
        return lane;
    }

private:
    void add(int32_t lane, int64_t load) {
        const size_t k = static_cast<size_t>(lane - lo_);
        bits_[(load & mask_) * words_ + k / 64] |= uint64_t{1} << (k % 64);
        cnt_[load & mask_]++;
    }
    void heap_push(uint64_t k) {
        size_t i = heap_.size();
        heap_.push_back(k);
        while (i > 0) {
            const size_t p = (i - 1) / 4;
            if (heap_[p] <= k) break;
            heap_[i] = heap_[p];
            i = p;
        }
        heap_[i] = k;
    }
    void heap_replace_top(uint64_t k) {
        const size_t n = heap_.size();
        size_t i = 0;
        for (;;) {
            const size_t c = 4 * i + 1;
            if (c >= n) break;
            size_t m = c;
            const size_t e = std::min(c + 4, n);
            for (size_t j = c + 1; j < e; ++j) m = heap_[j] < heap_[m] ? j : m;
            if (heap_[m] >= k) break;
            heap_[i] = heap_[m];
            i = m;
        }
        heap_[i] = k;
    }

    int32_t lo_ = 0, n_ = 0;
    bool bucket_mode_ = true;
    size_t words_ = 0, mask_ = 0, wc_ = 0;
    int64_t cur_ = 0;
    std::vector<uint64_t> bits_;
    std::vector<int32_t> cnt_;
    int lane_bits_ = 1;
    std::vector<uint64_t> heap_;
};

struct Item {
    std::vector<int32_t> chunks;
    int32_t k0 = -1;             // path index of the first chunk (a row's own items)
    int32_t key_base = 0;
    int32_t len_row = -1;
    int32_t tail = 0;            // keys missing from the last chunk when len_row < 0
    int32_t row_lo = 0;
    int32_t n_rows = 0;
    int32_t out = -1;
};

// Workgroup units, longest first (equal costs in index order), each to the
// workgroup that would finish it first, where the younger workgroups
// (g >= G/2) run at young_pct % of the older ones' speed: the younger of the
// two workgroups that share a compute unit in decode, the second round of
// prefill workgroups (whose share of the load it then sets).  Ties go to the
// older class, then to the lower workgroup index.
// add: keep the lists and loads already in wg_units / wg_load and append to them.
void assign_units(const std::vector<int64_t>& cost, int32_t G,
                  std::vector<std::vector<int32_t>>& wg_units, std::vector<int64_t>& wg_load,
                  int32_t young_pct = kYoungSpeedPct, bool add = false) {
    if (!add || static_cast<int32_t>(wg_units.size()) != G) {
        wg_units.assign(G, {});
        wg_load.assign(G, 0);
    }
    std::vector<int32_t> order(cost.size());
    for (size_t i = 0; i < order.size(); ++i) order[i] = static_cast<int32_t>(i);
    std::stable_sort(order.begin(), order.end(), [&](int32_t a, int32_t c) { return cost[a] > cost[c]; });
    int64_t max_cost = 1;
    for (int64_t c : cost) max_cost = std::max(max_cost, c);
    const int32_t n_old = G > 1 ? G / 2 : G;
    LaneQueue q[2];
    q[0].init(0, n_old, wg_load, max_cost);
    q[1].init(n_old, G - n_old, wg_load, max_cost);
    for (int32_t ui : order) {
        int cls = -1;
        int64_t best = 0;
        for (int c = 0; c < 2; ++c) {
            if (q[c].empty()) continue;
            const int64_t fin = (q[c].min_load() + cost[ui]) * 100 / (c ? young_pct : 100);
            if (cls < 0 || fin < best) {
                cls = c;
                best = fin;
            }
        }
        const int32_t g = q[cls].take(cost[ui]);
        wg_load[g] += cost[ui];
        wg_units[g].push_back(ui);
    }
}

// Depth-first order over the paths of the batch sequences, children in
// creation order (Knowl 1's contiguity invariant: the sequences under any
// node are one range of depth-first positions).  Fills sc.node[x] = {i, j}
// for every node on a batch path (and the root), with seg = -1; returns the
// depth-first position -> batch index order and the visited nodes, parents
// first.  False if a row was lost (cannot happen for a consistent tree).
bool batch_dfs(const Tree& t, const std::vector<const Seq*>& seqs, PlanScratch& sc,
               std::vector<int32_t>& dfs_row, std::vector<int32_t>& preorder) {
    const int32_t b = static_cast<int32_t>(seqs.size());
    const int32_t root = t.root();
    const size_t n_nodes = static_cast<size_t>(t.N) + 1;
    if (sc.mark.size() != n_nodes) {
        sc.mark.assign(n_nodes, 0);
        sc.node.resize(n_nodes);
        sc.epoch = 0;
    }
    if (++sc.epoch == 0) {
        std::fill(sc.mark.begin(), sc.mark.end(), 0u);
        sc.epoch = 1;
    }
    const uint32_t epoch = sc.epoch;
    auto on_path = [&](int32_t x) { return sc.mark[x] == epoch; };
    PlanScratch::NodeInfo* info = sc.node.data();
    auto touch = [&](int32_t x) {
        if (!on_path(x)) {
            sc.mark[x] = epoch;
            info[x] = PlanScratch::NodeInfo{0, 0, -1, -1};
        }
    };
    touch(root);
    for (int32_t r = 0; r < b; ++r)
        for (int32_t x : seqs[r]->path) touch(x);
    // rows ending at each leaf, as lists threaded through next_row (ascending)
    std::vector<int32_t> next_row(b, -1);
    for (int32_t r = b - 1; r >= 0; --r) {
        const int32_t leaf = seqs[r]->path.back();
        next_row[r] = info[leaf].first_row;
        info[leaf].first_row = r;
    }
    dfs_row.clear();
    preorder.clear();
    dfs_row.reserve(b);
    struct Frame { int32_t node; size_t next; };
    std::vector<Frame> stack{{root, 0}};
    while (!stack.empty()) {
        Frame& f = stack.back();
        const Node& n = t.node(f.node);
        if (f.next < n.children.size()) {
            const int32_t ch = n.children[f.next++];
            if (!on_path(ch)) continue;                       // not on a batch path
            info[ch].i = static_cast<int32_t>(dfs_row.size());
            preorder.push_back(ch);
            for (int32_t r = info[ch].first_row; r >= 0; r = next_row[r]) dfs_row.push_back(r);
            stack.push_back({ch, 0});
        } else {
            info[f.node].j = static_cast<int32_t>(dfs_row.size());
            stack.pop_back();
        }
    }
    return static_cast<int32_t>(dfs_row.size()) == b;
}

}  // namespace

static void write_seqlen(const Tree& t, Plan& plan) {
    const int32_t off = plan.blob[kOffSeqlen];
    int64_t logical = 0;
    for (int32_t p = 0; p < plan.b; ++p) {
        const Seq* s = t.find_seq(plan.dfs_seq[p]);
        plan.blob[off + p] = static_cast<int32_t>(s->len);
        logical += s->len;
    }
    plan.logical_tokens = logical;
}

// Follow the decode appends since the plan was built (the tree was changed
// by nothing else): each row whose sequence opened new leaf chunks gets them
// at the end of its last work item, in the room reserved after that item's
// chunk ids.  Only the item's chunk count and ids change: the new chunks are
// private (phase 2) and every other node keeps its coverage, so the depth-first
// order, the items, the partial slots and the merge lists stay valid.  The
// balance of the task lists drifts by at most kAppendSlack steps per task.
// False (and nothing changed) when some row cannot be patched: its path ends
// in phase-1 chunks, its room is used up, or its old last chunk is partial.
static bool patch_appends(const Tree& t, Plan& plan) {
    std::vector<int32_t> rows;
    for (const auto& g : t.grown()) {
        if (g.first <= plan.struct_version) continue;
        const auto it = plan.pos_of_seq.find(g.second);
        if (it != plan.pos_of_seq.end()) rows.push_back(it->second);
    }
    std::sort(rows.begin(), rows.end());
    rows.erase(std::unique(rows.begin(), rows.end()), rows.end());
    std::vector<int32_t>& blob = plan.blob;
    const int32_t wbase = blob[kOffWaves], cbase = blob[kOffChunks];
    for (const int32_t p : rows) {                           // check every row first
        const int32_t w = plan.last_wave[p];
        if (w < 0) return false;
        const std::vector<int32_t>& path = t.find_seq(plan.dfs_seq[p])->path;
        const int32_t n = static_cast<int32_t>(path.size());
        const int32_t k0 = plan.last_k0[p];
        const int32_t old_n = blob[wbase + 8 * w + 1];
        if (n - k0 > plan.wave_cap[w] || n - k0 <= old_n) return false;
        for (int32_t k = k0 + old_n - 1; k < n; ++k) {
            const Node& x = t.node(path[k]);
            if (k + 1 < n && x.fill != t.C) return false;         // key k must lie in chunk k / C
            if (k >= k0 + old_n && x.refs != 1) return false;     // new chunks are private
        }
    }
    for (const int32_t p : rows) {
        const int32_t w = plan.last_wave[p];
        const std::vector<int32_t>& path = t.find_seq(plan.dfs_seq[p])->path;
        const int32_t n = static_cast<int32_t>(path.size());
        const int32_t k0 = plan.last_k0[p];
        int32_t* wd = &blob[wbase + 8 * w];
        for (int32_t k = k0 + wd[1]; k < n; ++k) blob[cbase + wd[0] + (k - k0)] = path[k];
        wd[1] = n - k0;
    }
    plan.serial += 1;
    blob[kSerial] = static_cast<int32_t>(plan.serial & 0x7fffffff);
    plan.struct_version = t.structure_version();
    plan.patches += 1;
    return true;
}

int make_plan(const Tree& t, int32_t b, const int32_t* q_order, const PlanOpts& in_opts,
              Plan& plan, std::string& err) {
    if (b < 1 || !q_order) {
        err = "plan: need b >= 1 and a q_order array";
        return PKVT_ERR_INVALID_ARG;
    }
    PlanOpts opts = in_opts;
    if (opts.min_share == 0) opts.min_share = 2;
    if (opts.unit_rows == 0) opts.unit_rows = kRowsPerWave + 1;
    if (opts.min_share < 2 || opts.phase1_chunks < 0 || opts.phase2_chunks < 0 ||
        opts.unit_rows <= kRowsPerWave) {
        err = "plan: min_share must be >= 2 (or 0 for the default); chunk limits >= 0; "
              "unit_rows > 16 (or 0 for the default)";
        return PKVT_ERR_INVALID_ARG;
    }
    const int32_t G = opts.workgroups > 0 ? opts.workgroups : kDefaultWorkgroups;
    const int32_t lanes = G * kWavesPerWg;

    // ---- validate the batch --------------------------------------------------
    std::vector<const Seq*> seqs(b);
    {
        std::unordered_map<int32_t, int32_t> seen;
        for (int32_t r = 0; r < b; ++r) {
            const Seq* s = t.find_seq(q_order[r]);
            if (!s) {
                err = "plan: unknown sequence id " + std::to_string(q_order[r]);
                return PKVT_ERR_UNKNOWN_SEQ;
            }
            if (s->len < 1) {
                err = "plan: sequence " + std::to_string(q_order[r]) + " is empty";
                return PKVT_ERR_EMPTY_SEQ;
            }
            if (!seen.emplace(q_order[r], r).second) {
                err = "plan: sequence id " + std::to_string(q_order[r]) + " listed twice";
                return PKVT_ERR_INVALID_ARG;
            }
            seqs[r] = s;
        }
    }

    // ---- same structure as the current plan: refresh lengths only ------------
    const bool same_batch = plan.valid && plan.b == b && plan.opts == opts &&
                            std::equal(q_order, q_order + b, plan.q_order.begin());
    if (same_batch && plan.struct_version == t.structure_version()) {
        write_seqlen(t, plan);
        plan.len_version = t.length_version();
        plan.last_update = 0;
        return PKVT_OK;
    }
    // ---- only appends that opened leaf chunks since: patch the last items -----
    if (same_batch && t.reshape_version() <= plan.struct_version && plan.patches < kMaxPatches &&
        patch_appends(t, plan)) {
        write_seqlen(t, plan);
        plan.len_version = t.length_version();
        plan.last_update = 1;
        return PKVT_OK;
    }

    // ---- 1. depth-first order over the batch's paths --------------------------
    const int32_t root = t.root();
    std::vector<int32_t> dfs_row;             // depth-first position -> query row
    std::vector<int32_t> preorder;            // visited nodes, parents first
    if (!batch_dfs(t, seqs, plan.scratch, dfs_row, preorder)) {
        err = "plan: internal error, depth-first order lost rows";
        return PKVT_ERR_INVALID_ARG;
    }
    PlanScratch::NodeInfo* info = plan.scratch.node.data();
    auto cov = [&](int32_t x) { return info[x].j - info[x].i; };

    // ---- 2. phase-1 segments ----------------------------------------------------
    std::vector<std::vector<int32_t>> segs;
    std::vector<Range> seg_range;
    for (int32_t x : preorder) {
        if (cov(x) < opts.min_share) continue;
        const int32_t p = t.node(x).parent;
        if (p != root && info[p].seg >= 0 && info[p].i == info[x].i && info[p].j == info[x].j &&
            t.node(p).fill == t.C) {
            segs[info[p].seg].push_back(x);
            info[x].seg = info[p].seg;
        } else {
            info[x].seg = static_cast<int32_t>(segs.size());
            segs.push_back({x});
            seg_range.push_back(Range{info[x].i, info[x].j});
        }
    }
    // private suffix of every sequence: path[k0[p] ..), starting at token pos0[p]
    std::vector<int32_t> k0(b);
    std::vector<int64_t> pos0(b);
    for (int32_t p = 0; p < b; ++p) {
        const Seq* sq = seqs[dfs_row[p]];
        const std::vector<int32_t>& path = sq->path;
        int32_t k = static_cast<int32_t>(path.size());
        int64_t pos = sq->len;
        while (k > 0 && cov(path[k - 1]) < opts.min_share) pos -= t.node(path[--k]).fill;
        k0[p] = k;
        pos0[p] = pos;
    }
    std::vector<int64_t> seg_keys(segs.size(), 0);
    for (size_t s = 0; s < segs.size(); ++s)
        for (int32_t x : segs[s]) seg_keys[s] += t.node(x).fill;

    // ---- units-only plans -----------------------------------------------------------
    // When every row's whole context is shared by at least unit_rows rows (no
    // sequence-first work and no single-wave phase-1 groups) and head_dim >=
    // 128, the plan runs on the units-only kernel: one workgroup of 8 waves
    // per compute unit (G / 2 of them), each unit computed by two phases of 4
    // waves that take alternate steps.  Items are then cut so that there are
    // about as many units as workgroups (subject to the partial-cost floor).
    bool units_only = t.D >= 128 && G >= 2 && !segs.empty();
    for (int32_t p = 0; p < b && units_only; ++p)
        units_only = k0[p] == static_cast<int32_t>(seqs[dfs_row[p]]->path.size());
    for (size_t s = 0; s < segs.size() && units_only; ++s)
        for (const int32_t rb : row_blocks(seg_range[s].j - seg_range[s].i, opts.unit_rows))
            units_only = units_only && rb >= opts.unit_rows;
    const int32_t Gk = units_only ? G / 2 : G;        // workgroups of the kernel that runs the plan

    // ---- item size ----------------------------------------------------------------
    // T = the mean per-wave load in 64-key steps with nothing cut (a unit
    // step counted at its cost relative to a single-wave step).  Phase-1
    // items read by single-wave tasks are cut at T, those read by workgroup
    // units at 5T / kUnitStepCost steps, which a unit takes 5/4 of T to run
    // (fewer, longer units: fewer partials to write and merge; measured on
    // the 1K-, 4K-prefix and two-level-tree batches).  Phase-2 items are cut at T when nothing is shared
    // (all tasks then tend to be alike and need no merge); with a shared
    // prefix the phase-1 units make the per-wave loads uneven and finer
    // phase-2 pieces (T/4, but at least 4 steps) fill the gaps better.  The
    // floor holds also when T is below it: a small batch cut into 1- or
    // 2-step pieces spends more on the extra partials and their merge than
    // the finer balance wins back.
    int32_t s1 = opts.phase1_chunks, s2 = opts.phase2_chunks;
    int32_t s1_unit = s1;                 // phase-1 items whose rows form workgroup units
    if (s1 == 0 || s2 == 0) {
        int64_t quarters = 0;
        for (size_t s = 0; s < segs.size(); ++s) {
            const int64_t st = steps_of(seg_keys[s]);
            const int32_t rows = seg_range[s].j - seg_range[s].i;
            for (const int32_t rb : row_blocks(rows, opts.unit_rows)) {
                if (rb >= opts.unit_rows)
                    quarters += kWavesPerWg * kUnitStepCost * st;
                else
                    quarters += 4 * st * ((rb + kRowsPerWave - 1) / kRowsPerWave);
            }
        }
        for (int32_t p = 0; p < b; ++p)
            quarters += 4 * steps_of(seqs[dfs_row[p]]->len - pos0[p]);
        const int64_t mean = std::max<int64_t>(1, (quarters * t.H + 4 * lanes - 1) / (4 * lanes));
        if (s1 == 0) {
            s1 = steps_to_chunks(mean, t.C);
            // a unit step takes a wave kUnitStepCost / 4 of a task step: units
            // of up to 5/4 T * 4 / kUnitStepCost steps last at most 5/4 of a
            // mean wave load
            s1_unit = steps_to_chunks(mean * 5 / kUnitStepCost, t.C);
        }
        if (s2 == 0) {
            const int64_t fine = std::max<int64_t>(4, (mean + 3) / 4);
            s2 = steps_to_chunks(segs.empty() ? mean : fine, t.C);
        }
    }
    // the kernel holds a task's chunk ids one per lane of a 64-lane wave
    s1 = std::min(s1, kMaxItemChunks);
    s2 = std::min(s2, kMaxItemChunks);
    // units-only: unit steps spread evenly over the Gk workgroups
    int32_t s1_units_only = kMaxItemChunks;
    if (units_only) {
        int64_t unit_steps = 0;
        for (size_t s = 0; s < segs.size(); ++s)
            unit_steps += steps_of(seg_keys[s]) *
                          static_cast<int64_t>(row_blocks(seg_range[s].j - seg_range[s].i, opts.unit_rows).size());
        unit_steps *= t.H;
        s1_units_only = std::min(kMaxItemChunks, steps_to_chunks((unit_steps + Gk - 1) / Gk, t.C));
    }

    // ---- 3. items ------------------------------------------------------------------
    std::vector<Item> items1;
    std::vector<int32_t> src_count(b, 0);
    int32_t shared_chunks = 0;
    // a run of n chunks is cut into ceil(n / limit) items of near-equal size
    auto cuts = [](int32_t n, int32_t limit) {
        std::vector<int32_t> at{0};
        const int32_t k = (n + limit - 1) / limit;
        for (int32_t i = 0; i < k; ++i) at.push_back(at.back() + n / k + (i < n % k ? 1 : 0));
        return at;
    };
    for (size_t s = 0; s < segs.size(); ++s) {
        shared_chunks += static_cast<int32_t>(segs[s].size());
        // Every phase-1 item writes one partial (o, m, n) per row and head,
        // read back by the merge: 8 R (d+2) bytes against 4 c d KV bytes
        // per chunk.  Unless the caller fixed the size, an item is long
        // enough that its partials cost at most a quarter of its KV bytes --
        // except in units-only plans, which are cut into about one unit per
        // workgroup even below that floor: there the launch is short and a
        // grid left partly idle costs more than the extra partials (32 rows
        // over a fully shared 1K context: 256 units of 2 chunks 14.3 us per
        // layer, the floor's 128 units of 4 chunks 15.0-15.9 us).
        int32_t limit = s1;
        if (opts.phase1_chunks == 0) {
            const int64_t rows = seg_range[s].j - seg_range[s].i;
            if (rows >= opts.unit_rows) limit = units_only ? s1_units_only : s1_unit;
            const int64_t need = (8 * rows * (t.D + 2) * 4 + 4LL * t.C * t.D - 1) / (4LL * t.C * t.D);
            limit = static_cast<int32_t>(
                std::min<int64_t>(kMaxItemChunks, units_only ? limit : std::max<int64_t>(limit, need)));
        }
        const std::vector<int32_t> at = cuts(static_cast<int32_t>(segs[s].size()), limit);
        for (size_t q = 0; q + 1 < at.size(); ++q) {
            Item it;
            it.chunks.assign(segs[s].begin() + at[q], segs[s].begin() + at[q + 1]);
            it.tail = t.C - t.node(it.chunks.back()).fill;     // only a segment's last node is partial
            it.row_lo = seg_range[s].i;
            it.n_rows = seg_range[s].j - seg_range[s].i;
            for (int32_t p = seg_range[s].i; p < seg_range[s].j; ++p) src_count[p]++;
            items1.push_back(std::move(it));
        }
    }
    std::vector<Item> items2;
    for (int32_t p = 0; p < b; ++p) {
        const std::vector<int32_t>& path = seqs[dfs_row[p]]->path;
        const int32_t n = static_cast<int32_t>(path.size());
        int64_t pos = pos0[p];
        // runs of full chunks ending at a partial node or at the leaf
        for (int32_t r0 = k0[p]; r0 < n;) {
            int32_t r1 = r0;
            while (r1 < n - 1 && t.node(path[r1]).fill == t.C) ++r1;
            ++r1;
            const std::vector<int32_t> at = cuts(r1 - r0, s2);
            for (size_t q = 0; q + 1 < at.size(); ++q) {
                Item it;
                const int32_t a = r0 + at[q];
                const int32_t e = r0 + at[q + 1];
                it.chunks.assign(path.begin() + a, path.begin() + e);
                it.k0 = a;
                it.key_base = static_cast<int32_t>(pos + static_cast<int64_t>(at[q]) * t.C);
                it.len_row = (e == n) ? p : -1;
                if (e < n) it.tail = t.C - t.node(path[e - 1]).fill;
                it.row_lo = p;
                it.n_rows = 1;
                src_count[p]++;
                items2.push_back(std::move(it));
            }
            for (int32_t k = r0; k < r1; ++k) pos += t.node(path[k]).fill;
            r0 = r1;
        }
    }

    // ---- 4. partial slots and merge lists -------------------------------------------
    int32_t n_slots = 0;
    std::vector<std::vector<int32_t>> mslots(b);
    for (Item& it : items1) {
        it.out = n_slots;
        for (int32_t r = 0; r < it.n_rows; ++r) mslots[it.row_lo + r].push_back(n_slots + r);
        n_slots += it.n_rows;
    }
    for (Item& it : items2) {
        const int32_t p = it.row_lo;
        if (src_count[p] == 1) {
            it.out = -1;                                    // finalised by the item itself
        } else {
            it.out = n_slots++;
            mslots[p].push_back(it.out);
        }
    }

    // ---- 5. wave descriptors, workgroup units and per-lane task lists -----------------
    std::vector<WaveDesc> waves;
    std::vector<const std::vector<int32_t>*> wave_chunks;
    std::vector<int64_t> wave_cost;
    auto item_keys = [&](const Item& it) {
        int64_t keys = static_cast<int64_t>(it.chunks.size()) * t.C - it.tail;
        if (it.len_row >= 0)
            keys = std::min<int64_t>(keys, seqs[dfs_row[it.len_row]]->len - it.key_base);
        return keys;
    };
    auto add_wave = [&](const Item& it, int32_t row_off) {
        WaveDesc w{};
        w.n_chunks = static_cast<int32_t>(it.chunks.size());
        w.key_base = it.key_base;
        w.len_row = it.len_row;
        w.tail = it.tail;
        w.row_lo = it.row_lo + row_off;
        w.n_rows = std::min(kRowsPerWave, it.n_rows - row_off);
        w.out = it.out < 0 ? -1 : it.out + row_off;
        waves.push_back(w);
        wave_chunks.push_back(&it.chunks);
        wave_cost.push_back(task_cost(item_keys(it)));
        return static_cast<int32_t>(waves.size()) - 1;
    };
    // Phase-1 rows are cut into blocks of up to kRowsPerUnit.  A block of at least
    // unit_rows rows (default: more than one row group) becomes one workgroup
    // unit per head, in which the 4 waves split every step's loads and share
    // the data through LDS.  Smaller blocks are cut into single-wave tasks of
    // up to 16 rows, like phase 2.
    struct Unit { const Item* it; int32_t r0, rows, head, keys; int64_t cost; };
    std::vector<Unit> units;
    std::vector<int32_t> singles;            // single-wave tasks (x heads)
    for (const Item& it : items1) {
        const int32_t keys = static_cast<int32_t>(item_keys(it));
        int32_t r0 = 0;
        for (const int32_t rb : row_blocks(it.n_rows, opts.unit_rows)) {
            if (rb < opts.unit_rows) {
                for (int32_t r = r0; r < r0 + rb; r += kRowsPerWave) singles.push_back(add_wave(it, r));
            } else {
                for (int32_t h = 0; h < t.H; ++h) units.push_back({&it, r0, rb, h, keys, unit_cost(keys)});
            }
            r0 += rb;
        }
    }
    for (const Item& it : items2) singles.push_back(add_wave(it, 0));

    std::vector<std::vector<int32_t>> wg_units(G);
    std::vector<int32_t> task_lane;                                      // lane of each task
    std::vector<std::pair<int32_t, int32_t>> task_entry;                  // (wave, head)
    std::vector<int64_t> load(lanes, 0);
    {
        // Workgroups g and g + G/2 share a compute unit and the hardware
        // favours the older one (g < G/2): while both run, the younger one's
        // waves progress at about kYoungSpeedPct % of the older one's speed.
        // Work goes, longest first, to whichever wave (or workgroup, for
        // units) would finish it first at its speed.
        {
            std::vector<int64_t> cost(units.size());
            for (size_t i = 0; i < units.size(); ++i) cost[i] = units[i].cost;
            std::vector<int64_t> wg_load;
            // units-only: one workgroup per compute unit, all at the same speed
            assign_units(cost, Gk, wg_units, wg_load, units_only ? 100 : kYoungSpeedPct);
            wg_units.resize(G);
            for (int32_t g = 0; g < Gk; ++g)
                for (int32_t k = 0; k < kWavesPerWg; ++k) load[g * kWavesPerWg + k] = wg_load[g];
        }
        // single-wave tasks x heads, longest first; equal costs keep the
        // (task, head) order.  The lane heaps hold load << lane_bits | lane,
        // which orders like the pair (load, lane).
        std::vector<int32_t> sorder(singles.size());
        for (size_t i = 0; i < sorder.size(); ++i) sorder[i] = static_cast<int32_t>(i);
        std::stable_sort(sorder.begin(), sorder.end(), [&](int32_t a, int32_t c) {
            return wave_cost[singles[a]] > wave_cost[singles[c]];
        });
        int64_t max_cost = 1;
        for (int32_t w : singles) max_cost = std::max(max_cost, wave_cost[w]);
        const int32_t n_old = G > 1 ? kWavesPerWg * (G / 2) : lanes;     // lanes of older workgroups
        LaneQueue lq[2];
        lq[0].init(0, n_old, load, max_cost);
        lq[1].init(n_old, lanes - n_old, load, max_cost);
        task_lane.reserve(singles.size() * t.H);
        task_entry.reserve(singles.size() * t.H);
        for (int32_t i : sorder) {
            const int64_t cost = wave_cost[singles[i]];
            for (int32_t h = 0; h < t.H; ++h) {
                int cls = -1;
                int64_t best = 0;
                for (int c = 0; c < 2; ++c) {
                    if (lq[c].empty()) continue;
                    const int64_t fin = (lq[c].min_load() + cost) * 100 / (c ? kYoungSpeedPct : 100);
                    if (cls < 0 || fin < best) {
                        cls = c;
                        best = fin;
                    }
                }
                const int32_t l = lq[cls].take(cost);
                load[l] += cost;
                task_lane.push_back(l);
                task_entry.push_back({singles[i], h});
            }
        }
    }
    // per-lane lists in assignment order (CSR over lanes)
    std::vector<int32_t> lane_start(lanes + 1, 0);
    for (int32_t l : task_lane) lane_start[l + 1]++;
    for (int32_t l = 0; l < lanes; ++l) lane_start[l + 1] += lane_start[l];
    std::vector<std::pair<int32_t, int32_t>> lane_tasks(task_lane.size());   // (wave, head)
    {
        std::vector<int32_t> fill(lane_start.begin(), lane_start.end() - 1);
        for (size_t k = 0; k < task_lane.size(); ++k) lane_tasks[fill[task_lane[k]]++] = task_entry[k];
    }

    // ---- 6. emit the blob -------------------------------------------------------------
    const int32_t n_waves = static_cast<int32_t>(waves.size());
    const int32_t n_units = static_cast<int32_t>(units.size());
    const int32_t n_tasks = static_cast<int32_t>(lane_tasks.size());
    // a row's last item keeps room for kAppendSlack more chunk ids (patch_appends)
    std::vector<int32_t> wave_cap(n_waves);
    std::vector<int32_t> last_wave(b, -1), last_k0(b, -1);
    for (int32_t w = 0; w < n_waves; ++w) {
        const int32_t n = static_cast<int32_t>(wave_chunks[w]->size());
        wave_cap[w] = waves[w].len_row >= 0 ? std::max(n, std::min(kMaxItemChunks, n + kAppendSlack)) : n;
    }
    for (const Item& it : items2)
        if (it.len_row >= 0) last_k0[it.len_row] = it.k0;
    for (int32_t w = 0; w < n_waves; ++w)
        if (waves[w].len_row >= 0) last_wave[waves[w].len_row] = w;
    int32_t total_chunks = 0;
    for (int32_t w = 0; w < n_waves; ++w) total_chunks += wave_cap[w];
    for (const Unit& u : units) total_chunks += static_cast<int32_t>(u.it->chunks.size());
    std::vector<int32_t> merge_rows;
    for (int32_t p = 0; p < b; ++p)
        if (!mslots[p].empty()) merge_rows.push_back(p);
    int32_t n_mslots = 0;
    for (auto& m : mslots) n_mslots += static_cast<int32_t>(m.size());

    std::vector<int32_t> blob(kHeaderWords, 0);
    auto section = [&](HeaderField f, size_t words) {
        while (blob.size() % 4) blob.push_back(0);             // 16-byte aligned sections
        blob[f] = static_cast<int32_t>(blob.size());
        blob.resize(blob.size() + words, 0);
    };
    section(kOffLists, static_cast<size_t>(lanes) * 2);
    section(kOffTasks, static_cast<size_t>(n_tasks) * 2);
    section(kOffWaves, static_cast<size_t>(n_waves) * 8);
    section(kOffWgUnits, static_cast<size_t>(G) * 2);
    section(kOffUnits, static_cast<size_t>(n_units) * 8);
    section(kOffChunks, total_chunks);
    section(kOffRows, b);
    section(kOffMerge, merge_rows.size());
    section(kOffMptr, b + 1);
    section(kOffMslots, n_mslots);
    section(kOffSeqlen, b);
    while (blob.size() % 4) blob.push_back(0);

    {
        for (int32_t l = 0; l < lanes; ++l) {
            blob[blob[kOffLists] + 2 * l] = lane_start[l];
            blob[blob[kOffLists] + 2 * l + 1] = lane_start[l + 1] - lane_start[l];
        }
        for (int32_t k = 0; k < n_tasks; ++k) {
            blob[blob[kOffTasks] + 2 * k] = lane_tasks[k].first;
            blob[blob[kOffTasks] + 2 * k + 1] = lane_tasks[k].second;
        }
        int32_t coff = 0;
        for (int32_t w = 0; w < n_waves; ++w) {
            WaveDesc d = waves[w];
            d.chunk_off = coff;
            for (int32_t id : *wave_chunks[w]) blob[blob[kOffChunks] + coff++] = id;
            coff += wave_cap[w] - static_cast<int32_t>(wave_chunks[w]->size());
            std::copy(reinterpret_cast<const int32_t*>(&d),
                      reinterpret_cast<const int32_t*>(&d) + 8, &blob[blob[kOffWaves] + w * 8]);
        }
        int32_t ua = 0;
        for (int32_t g = 0; g < G; ++g) {
            blob[blob[kOffWgUnits] + 2 * g] = ua;
            blob[blob[kOffWgUnits] + 2 * g + 1] = static_cast<int32_t>(wg_units[g].size());
            for (int32_t ui : wg_units[g]) {
                const Unit& u = units[ui];
                UnitDesc d{};
                d.n_keys = u.keys;
                d.chunk_off = coff;
                d.n_chunks = static_cast<int32_t>(u.it->chunks.size());
                for (int32_t id : u.it->chunks) blob[blob[kOffChunks] + coff++] = id;
                d.head = u.head;
                d.row_lo = u.it->row_lo + u.r0;
                d.n_rows = u.rows;
                d.out = u.it->out + u.r0;
                std::copy(reinterpret_cast<const int32_t*>(&d),
                          reinterpret_cast<const int32_t*>(&d) + 8, &blob[blob[kOffUnits] + ua * 8]);
                ++ua;
            }
        }
    }
    for (int32_t p = 0; p < b; ++p) blob[blob[kOffRows] + p] = dfs_row[p];
    for (size_t m = 0; m < merge_rows.size(); ++m) blob[blob[kOffMerge] + m] = merge_rows[m];
    {
        int32_t at = 0;
        for (int32_t p = 0; p < b; ++p) {
            blob[blob[kOffMptr] + p] = at;
            for (int32_t sl : mslots[p]) blob[blob[kOffMslots] + at++] = sl;
        }
        blob[blob[kOffMptr] + b] = at;
    }
    blob[kMagic] = kPlanMagic;
    blob[kB] = b;
    blob[kNWaves] = n_waves;
    blob[kNWg] = Gk;
    blob[kKernel] = units_only ? 1 : 0;
    blob[kNTasks] = n_tasks;
    blob[kNUnits] = n_units;
    blob[kNSlots] = n_slots;
    blob[kNMerge] = static_cast<int32_t>(merge_rows.size());
    blob[kTotalWords] = static_cast<int32_t>(blob.size());

    // unique (stored) tokens of the batch: every distinct node once
    int64_t unique = 0;
    for (int32_t x : preorder) unique += t.node(x).fill;

    plan.serial += 1;
    blob[kSerial] = static_cast<int32_t>(plan.serial & 0x7fffffff);
    plan.blob = std::move(blob);
    plan.valid = true;
    plan.struct_version = t.structure_version();
    plan.len_version = t.length_version();
    plan.b = b;
    plan.q_order.assign(q_order, q_order + b);
    plan.opts = opts;
    plan.phase1_items = static_cast<int32_t>(items1.size());
    plan.phase2_items = static_cast<int32_t>(items2.size());
    plan.n_waves = n_waves;
    plan.n_wg = Gk;
    plan.kernel = units_only ? 1 : 0;
    plan.n_tasks = n_tasks;
    plan.n_units = n_units;
    plan.n_slots = n_slots;
    plan.n_merge = static_cast<int32_t>(merge_rows.size());
    plan.split1_chunks = s1;
    plan.split2_chunks = s2;
    plan.shared_chunks = shared_chunks;
    plan.unique_tokens = unique;
    plan.dfs_seq.resize(b);
    for (int32_t p = 0; p < b; ++p) plan.dfs_seq[p] = q_order[dfs_row[p]];
    plan.last_wave = std::move(last_wave);
    plan.last_k0 = std::move(last_k0);
    plan.wave_cap = std::move(wave_cap);
    plan.pos_of_seq.clear();
    for (int32_t p = 0; p < b; ++p) plan.pos_of_seq[plan.dfs_seq[p]] = p;
    plan.patches = 0;
    plan.last_update = 2;
    write_seqlen(t, plan);
    return PKVT_OK;
}

int make_prefill_plan(const Tree& t, int32_t n, const int32_t* seq_ids, const int64_t* q_from,
                      const PlanOpts& in_opts, Plan& plan, std::string& err) {
    if (n < 1 || !seq_ids || !q_from) {
        err = "prefill_plan: need n >= 1, seq_ids and q_from";
        return PKVT_ERR_INVALID_ARG;
    }
    if (in_opts.phase1_chunks < 0 || in_opts.workgroups < 0) {
        err = "prefill_plan: chunk limit and workgroups must be >= 0";
        return PKVT_ERR_INVALID_ARG;
    }
    const int32_t G = in_opts.workgroups > 0 ? in_opts.workgroups : kDefaultWorkgroups;
    const int32_t lanes = G * kWavesPerWg;
    const int32_t S = in_opts.phase1_chunks > 0 ? std::min(in_opts.phase1_chunks, kPrefillMaxChunks)
                                                : kPrefillMaxChunks;
    const int32_t C = t.C;
    const int32_t kRows = 16 * prefill_waves(t.D) * prefill_row_tiles(t.D);   // rows per work unit

    // ---- validate; rows per sequence ------------------------------------------
    std::vector<const Seq*> seqs(n);
    std::vector<int64_t> nrows(n);
    int64_t R = 0;
    {
        std::unordered_map<int32_t, int32_t> seen;
        for (int32_t s = 0; s < n; ++s) {
            const Seq* sq = t.find_seq(seq_ids[s]);
            if (!sq) {
                err = "prefill_plan: unknown sequence id " + std::to_string(seq_ids[s]);
                return PKVT_ERR_UNKNOWN_SEQ;
            }
            if (!seen.emplace(seq_ids[s], s).second) {
                err = "prefill_plan: sequence id " + std::to_string(seq_ids[s]) + " listed twice";
                return PKVT_ERR_INVALID_ARG;
            }
            if (q_from[s] < 0 || q_from[s] >= sq->len) {
                err = "prefill_plan: q_from of sequence " + std::to_string(seq_ids[s]) +
                      " must lie in [0, length)";
                return PKVT_ERR_INVALID_ARG;
            }
            seqs[s] = sq;
            nrows[s] = sq->len - q_from[s];
            R += nrows[s];
        }
        if (R > (int64_t{1} << 30)) {
            err = "prefill_plan: too many query rows";
            return PKVT_ERR_INVALID_ARG;
        }
    }

    // ---- depth-first order; row numbering -------------------------------------
    std::vector<int32_t> dfs_seq, preorder;
    if (!batch_dfs(t, seqs, plan.scratch, dfs_seq, preorder)) {
        err = "prefill_plan: internal error, depth-first order lost rows";
        return PKVT_ERR_INVALID_ARG;
    }
    PlanScratch::NodeInfo* info = plan.scratch.node.data();
    std::vector<int64_t> caller_start(n + 1, 0), dfs_start(n + 1, 0);
    for (int32_t s = 0; s < n; ++s) caller_start[s + 1] = caller_start[s] + nrows[s];
    for (int32_t p = 0; p < n; ++p) dfs_start[p + 1] = dfs_start[p] + nrows[dfs_seq[p]];
    std::vector<int32_t> row_of(R), qpos(R);
    for (int32_t p = 0; p < n; ++p) {
        const int32_t s = dfs_seq[p];
        for (int64_t k = 0; k < nrows[s]; ++k) {
            row_of[dfs_start[p] + k] = static_cast<int32_t>(caller_start[s] + k);
            qpos[dfs_start[p] + k] = static_cast<int32_t>(q_from[s] + k);
        }
    }

    // ---- row blocks: depth-first rows, up to kRows per block ------------------------
    // Each sequence's rows are cut into near-equal pieces of at most kRows rows;
    // consecutive pieces (of neighbouring sequences, which share the longest
    // prefixes in depth-first order) are packed into one block while it
    // holds at most kRows rows.  A block reads, once for all its rows, the
    // chunks common to all its sequences (the chunk-first batching of Knowl
    // 2, over query rows), and each of its sequences reads its own chunks
    // beyond those for its rows.  A unit reads at most S chunks; the rows of
    // a block with a single sequence and a single unit get O directly.
    struct Piece { int32_t p; int64_t r0, r1; };
    std::vector<Piece> pieces;
    for (int32_t p = 0; p < n; ++p) {
        const int64_t len = nrows[dfs_seq[p]];
        const int64_t k = (len + kRows - 1) / kRows;
        int64_t r0 = dfs_start[p];
        for (int64_t i = 0; i < k; ++i) {
            const int64_t rows = len / k + (i < len % k ? 1 : 0);
            pieces.push_back({p, r0, r0 + rows});
            r0 += rows;
        }
    }
    struct Block { size_t first, last; };          // pieces [first, last]
    std::vector<Block> blks;
    for (size_t i = 0; i < pieces.size(); ++i) {
        if (!blks.empty() &&
            pieces[i].r1 - pieces[blks.back().first].r0 <= kRows)
            blks.back().last = i;
        else
            blks.push_back({i, i});
    }
    // chunks: every batch sequence's path, once; pstart[p][k] = sequence
    // position of the first token of chunk k (chunks may be partial anywhere
    // under token-granular matching)
    std::vector<int32_t> path_off(n + 1, 0);
    std::vector<std::vector<int64_t>> pstart(n);
    for (int32_t p = 0; p < n; ++p) {
        const std::vector<int32_t>& path = seqs[dfs_seq[p]]->path;
        path_off[p + 1] = path_off[p] + static_cast<int32_t>(path.size());
        pstart[p].assign(path.size() + 1, 0);
        for (size_t k = 0; k < path.size(); ++k) pstart[p][k + 1] = pstart[p][k] + t.node(path[k]).fill;
    }
    // chunks of sequence p holding a position <= pos
    auto chunks_upto = [&](int32_t p, int64_t pos) {
        const std::vector<int64_t>& ps = pstart[p];
        return static_cast<int32_t>(std::upper_bound(ps.begin(), ps.end() - 1, pos) - ps.begin());
    };

    struct PUnit { int32_t keys, chunk_off, n_chunks, row_lo, n_rows, out, key_base; int64_t cost; };
    std::vector<PUnit> blocks;                      // work units (x heads below)
    std::vector<int32_t> n_units_of(R, 0);          // units per row
    struct Pending { int64_t r0, r1; int32_t p, k0, k1; int64_t max_pos; };
    std::vector<Pending> pend;
    for (const Block& bk : blks) {
        const int32_t pa = pieces[bk.first].p, pb_ = pieces[bk.last].p;
        const std::vector<int32_t>& path_a = seqs[dfs_seq[pa]]->path;
        const std::vector<int32_t>& path_b = seqs[dfs_seq[pb_]]->path;
        const int64_t r0 = pieces[bk.first].r0, r1 = pieces[bk.last].r1;
        if (pa == pb_) {
            int32_t max_pos = 0;
            for (int64_t r = r0; r < r1; ++r) max_pos = std::max(max_pos, qpos[r]);
            pend.push_back({r0, r1, pa, 0, chunks_upto(pa, max_pos), max_pos});
            continue;
        }
        int32_t lcp = 0;                            // chunks common to every sequence of the block
        while (lcp < static_cast<int32_t>(std::min(path_a.size(), path_b.size())) &&
               path_a[lcp] == path_b[lcp])
            ++lcp;
        if (lcp > 0) {
            int32_t max_pos = 0;
            for (int64_t r = r0; r < r1; ++r) max_pos = std::max(max_pos, qpos[r]);
            const int32_t k1 = std::min(lcp, chunks_upto(pa, max_pos));
            pend.push_back({r0, r1, pa, 0, k1, max_pos});
        }
        for (size_t i = bk.first; i <= bk.last; ++i) {
            const Piece& pc = pieces[i];
            int32_t max_pos = 0;
            for (int64_t r = pc.r0; r < pc.r1; ++r) max_pos = std::max(max_pos, qpos[r]);
            const int32_t k1 = chunks_upto(pc.p, max_pos);
            if (k1 <= lcp) continue;                // every key it sees is common
            // rows before the first private key see nothing of it
            int64_t q0 = pc.r0;
            while (q0 < pc.r1 && qpos[q0] < pstart[pc.p][lcp]) ++q0;
            pend.push_back({q0, pc.r1, pc.p, lcp, k1, max_pos});
        }
    }
    // cut into units of at most S chunks, each holding full chunks but its
    // last (a unit addresses key k at chunk k / C); count units per row
    struct Cut { int64_t r0, r1; int32_t p, k0, k1; };
    std::vector<Cut> cuts_v;
    for (const Pending& pd : pend) {
        const std::vector<int32_t>& path = seqs[dfs_seq[pd.p]]->path;
        for (int32_t g0 = pd.k0; g0 < pd.k1;) {
            int32_t g1 = g0;
            while (g1 < pd.k1 - 1 && t.node(path[g1]).fill == C) ++g1;
            ++g1;                                   // [g0, g1): full chunks, then any
            const int32_t m = g1 - g0;
            const int32_t k_items = (m + S - 1) / S;
            int32_t a2 = g0;
            for (int32_t q = 0; q < k_items; ++q) {
                const int32_t e = a2 + m / k_items + (q < m % k_items ? 1 : 0);
                // runs of rows that see at least the first key of this cut (a
                // block of several sequences has no order of positions)
                const int64_t first = pstart[pd.p][a2];
                int64_t q0 = pd.r0;
                while (q0 < pd.r1) {
                    while (q0 < pd.r1 && qpos[q0] < first) ++q0;
                    int64_t q1 = q0;
                    while (q1 < pd.r1 && qpos[q1] >= first) ++q1;
                    if (q1 > q0) {
                        cuts_v.push_back({q0, q1, pd.p, a2, e});
                        for (int64_t r = q0; r < q1; ++r) n_units_of[r]++;
                    }
                    q0 = q1;
                }
                a2 = e;
            }
            g0 = g1;
        }
    }
    std::vector<std::vector<int32_t>> mslots(R);
    int32_t n_slots = 0;
    for (const Cut& ct : cuts_v) {
        const Seq* sq = seqs[dfs_seq[ct.p]];
        const int64_t kb = pstart[ct.p][ct.k0];
        int64_t n_keys = 0;
        for (int32_t k = ct.k0; k < ct.k1; ++k) n_keys += t.node(sq->path[k]).fill;
        int32_t max_pos = 0;
        bool direct = true;
        for (int64_t r = ct.r0; r < ct.r1; ++r) {
            max_pos = std::max(max_pos, qpos[r]);
            direct = direct && n_units_of[r] == 1;
        }
        const int64_t keys = std::min<int64_t>(n_keys, max_pos - kb + 1);
        PUnit u;
        u.keys = static_cast<int32_t>(keys);
        u.chunk_off = path_off[ct.p] + ct.k0;
        u.n_chunks = static_cast<int32_t>((keys + C - 1) / C);
        u.row_lo = static_cast<int32_t>(ct.r0);
        u.n_rows = static_cast<int32_t>(ct.r1 - ct.r0);
        u.key_base = static_cast<int32_t>(kb);
        u.cost = unit_cost(keys);
        if (direct) {
            u.out = -1;
        } else {
            u.out = n_slots;
            for (int64_t r = ct.r0; r < ct.r1; ++r)
                mslots[r].push_back(n_slots + static_cast<int32_t>(r - ct.r0));
            n_slots += u.n_rows;
        }
        blocks.push_back(u);
    }
    for (int64_t r = 0; r < R; ++r) {
        if (n_units_of[r] == 0) {
            err = "prefill_plan: internal error, a row reads no key";
            return PKVT_ERR_INVALID_ARG;
        }
    }
    const int32_t H = t.H;
    const int64_t n_units64 = static_cast<int64_t>(blocks.size()) * H;
    if (n_units64 > (int64_t{1} << 28)) {
        err = "prefill_plan: too many work units";
        return PKVT_ERR_INVALID_ARG;
    }
    // Workgroups are spread round-robin over the 8 accelerator dies (XCDs),
    // each with its own L2.  With heads a multiple of 8, the units of head h
    // go to workgroups g = h (mod 8), so the blocks that re-read a head's K/V
    // find it in one die's L2.  A die serves several heads; when the chunks
    // that many of its blocks re-read (read by at least a quarter of the
    // blocks: the shared prefixes) do not fit its L2 for all of those heads
    // together, the die's workgroups take their units head by
    // head instead (each head's units balanced over all of them, longest
    // first, on top of the loads already given), so that at any time the die
    // mostly reads one head's shared chunks; the second round of workgroups
    // (the younger half, which start as the first finish) take the heads in
    // reverse order, starting with the one still in L2.  Otherwise every
    // workgroup's units are balanced together, whatever their head.
    std::vector<std::vector<int32_t>> wg_units(G);
    {
        constexpr int32_t kDies = 8;
        constexpr int64_t kDieL2Bytes = int64_t{4} << 20;
        const bool by_die = H % kDies == 0 && G % (2 * kDies) == 0;
        const int32_t groups = by_die ? kDies : 1;
        const int32_t per = G / groups;
        std::unordered_map<int32_t, int32_t> readers;          // chunk -> blocks reading it
        for (const PUnit& u : blocks) {
            int32_t p = static_cast<int32_t>(std::upper_bound(path_off.begin(), path_off.end(), u.chunk_off) -
                                             path_off.begin()) - 1;
            const std::vector<int32_t>& path = seqs[dfs_seq[p]]->path;
            for (int32_t k = 0; k < u.n_chunks; ++k) readers[path[u.chunk_off - path_off[p] + k]]++;
        }
        const int32_t many = std::max<int32_t>(2, static_cast<int32_t>(blocks.size() / 4));
        int64_t reread_chunks = 0;
        for (const auto& kv : readers) reread_chunks += kv.second >= many;
        const int64_t reread_bytes = reread_chunks * C * t.D * 4 * (H / groups);   // K and V, fp16
        const bool head_by_head = by_die && reread_bytes > kDieL2Bytes;
        for (int32_t x = 0; x < groups && !head_by_head; ++x) {
            std::vector<int64_t> cost;
            std::vector<int32_t> ids;
            for (size_t bi = 0; bi < blocks.size(); ++bi)
                for (int32_t h = x; h < H; h += groups) {
                    cost.push_back(blocks[bi].cost);
                    ids.push_back(static_cast<int32_t>(bi * H + h));
                }
            std::vector<std::vector<int32_t>> wu;
            std::vector<int64_t> wl;
            assign_units(cost, per, wu, wl, kPrefillSecondRoundPct);
            for (int32_t i = 0; i < per; ++i)
                for (int32_t k : wu[i]) wg_units[i * groups + x].push_back(ids[k]);
        }
        for (int32_t x = 0; x < groups && head_by_head; ++x) {
            std::vector<std::vector<int32_t>> wu;
            std::vector<int64_t> wl;
            std::vector<std::vector<int32_t>> ids_of(per);    // unit ids per workgroup, head by head
            std::vector<std::vector<int32_t>> head_of(per);
            for (int32_t h = x; h < H; h += groups) {
                std::vector<int64_t> cost;
                for (size_t bi = 0; bi < blocks.size(); ++bi) cost.push_back(blocks[bi].cost);
                std::vector<size_t> before(per);
                for (int32_t i = 0; i < static_cast<int32_t>(wu.size()); ++i) before[i] = wu[i].size();
                assign_units(cost, per, wu, wl, kPrefillSecondRoundPct, /*add=*/true);
                for (int32_t i = 0; i < per; ++i)
                    for (size_t k = before[i]; k < wu[i].size(); ++k) {
                        ids_of[i].push_back(static_cast<int32_t>(wu[i][k] * H + h));
                        head_of[i].push_back(h);
                    }
            }
            for (int32_t i = 0; i < per; ++i) {
                std::vector<int32_t>& dst = wg_units[i * groups + x];
                if (i < per / 2) {
                    dst = ids_of[i];
                } else {                                   // younger: heads in reverse order
                    const int32_t last_h = H - groups + x;
                    for (int32_t h = last_h; h >= x; h -= groups)
                        for (size_t k = 0; k < ids_of[i].size(); ++k)
                            if (head_of[i][k] == h) dst.push_back(ids_of[i][k]);
                }
            }
        }
    }
    std::vector<int32_t> merge_rows;
    for (int64_t r = 0; r < R; ++r)
        if (!mslots[r].empty()) merge_rows.push_back(static_cast<int32_t>(r));

    // ---- emit the blob ------------------------------------------------------------
    const int32_t Ri = static_cast<int32_t>(R);
    const int32_t n_units = static_cast<int32_t>(n_units64);
    const int64_t total_chunks = path_off[n];
    int64_t n_mslots = 0;
    for (const auto& m : mslots) n_mslots += static_cast<int64_t>(m.size());
    std::vector<int32_t> blob(kHeaderWords, 0);
    auto section = [&](HeaderField f, size_t words) {
        while (blob.size() % 4) blob.push_back(0);
        blob[f] = static_cast<int32_t>(blob.size());
        blob.resize(blob.size() + words, 0);
    };
    section(kOffLists, static_cast<size_t>(lanes) * 2);
    section(kOffTasks, 0);
    section(kOffWaves, 0);
    section(kOffWgUnits, static_cast<size_t>(G) * 2);
    section(kOffUnits, static_cast<size_t>(n_units) * 8);
    section(kOffChunks, static_cast<size_t>(total_chunks));
    section(kOffRows, R);
    section(kOffMerge, merge_rows.size());
    section(kOffMptr, R + 1);
    section(kOffMslots, static_cast<size_t>(n_mslots));
    section(kOffSeqlen, R);
    section(kOffQpos, R);
    while (blob.size() % 4) blob.push_back(0);
    if (blob.size() > (size_t{1} << 31) - 1) {
        err = "prefill_plan: metadata too large";
        return PKVT_ERR_INVALID_ARG;
    }
    {
        for (int32_t p = 0; p < n; ++p) {
            const std::vector<int32_t>& path = seqs[dfs_seq[p]]->path;
            std::copy(path.begin(), path.end(), &blob[blob[kOffChunks] + path_off[p]]);
        }
        int32_t ua = 0;
        for (int32_t g = 0; g < G; ++g) {
            blob[blob[kOffWgUnits] + 2 * g] = ua;
            blob[blob[kOffWgUnits] + 2 * g + 1] = static_cast<int32_t>(wg_units[g].size());
            for (int32_t ui : wg_units[g]) {
                const PUnit& u = blocks[ui / H];
                UnitDesc d{};
                d.n_keys = u.keys;
                d.chunk_off = u.chunk_off;
                d.n_chunks = u.n_chunks;
                d.head = ui % H;
                d.row_lo = u.row_lo;
                d.n_rows = u.n_rows;
                d.out = u.out;
                d.key_base = u.key_base;
                std::copy(reinterpret_cast<const int32_t*>(&d),
                          reinterpret_cast<const int32_t*>(&d) + 8, &blob[blob[kOffUnits] + ua * 8]);
                ++ua;
            }
        }
    }
    {
        int32_t at = 0;
        for (size_t m = 0; m < merge_rows.size(); ++m) blob[blob[kOffMerge] + m] = merge_rows[m];
        for (int32_t r = 0; r < Ri; ++r) {
            blob[blob[kOffRows] + r] = row_of[r];
            blob[blob[kOffQpos] + r] = qpos[r];
            blob[blob[kOffMptr] + r] = at;
            for (int32_t sl : mslots[r]) blob[blob[kOffMslots] + at++] = sl;
        }
        blob[blob[kOffMptr] + Ri] = at;
    }
    blob[kMagic] = kPlanMagic;
    blob[kB] = Ri;
    blob[kNWaves] = 0;
    blob[kNWg] = G;
    blob[kNTasks] = 0;
    blob[kNUnits] = n_units;
    blob[kNSlots] = n_slots;
    blob[kNMerge] = static_cast<int32_t>(merge_rows.size());
    blob[kTotalWords] = static_cast<int32_t>(blob.size());

    int64_t unique = 0, logical = 0;
    for (int32_t x : preorder) unique += t.node(x).fill;
    for (int32_t s = 0; s < n; ++s) logical += seqs[s]->len;
    plan.serial += 1;
    blob[kSerial] = static_cast<int32_t>(plan.serial & 0x7fffffff);
    plan.blob = std::move(blob);
    plan.valid = true;
    plan.struct_version = t.structure_version();
    plan.len_version = t.length_version();
    plan.b = Ri;
    plan.q_order.assign(seq_ids, seq_ids + n);
    plan.opts = in_opts;
    plan.phase1_items = static_cast<int32_t>(blocks.size());
    plan.phase2_items = 0;
    plan.n_waves = 0;
    plan.n_wg = G;
    plan.n_tasks = 0;
    plan.n_units = n_units;
    plan.n_slots = n_slots;
    plan.n_merge = static_cast<int32_t>(merge_rows.size());
    plan.split1_chunks = S;
    plan.split2_chunks = 0;
    int32_t shared = 0;
    for (int32_t x : preorder)
        if (info[x].j - info[x].i >= 2) ++shared;
    plan.shared_chunks = shared;
    plan.unique_tokens = unique;
    plan.logical_tokens = logical;
    plan.dfs_seq.resize(n);
    for (int32_t p = 0; p < n; ++p) plan.dfs_seq[p] = seq_ids[dfs_seq[p]];
    return PKVT_OK;
}

}  // namespace pkvt
