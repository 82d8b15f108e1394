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
// 4. A sequence with exactly one item, a phase-2 one, is finalised by that
//    item; every other sequence's partials are merged afterwards.
#include "plan.h"

#include <algorithm>
#include <unordered_map>

#include "pkvt.h"

namespace pkvt {

namespace {

constexpr int32_t kDefaultPhase1Steps = 8;   // 64-key steps per phase-1 item
constexpr int32_t kDefaultPhase2Steps = 4;   // 64-key steps per phase-2 item

struct Range { int32_t i = 0, j = 0; };

struct Item {
    std::vector<int32_t> chunks;
    int32_t key_base = 0;
    int32_t len_row = -1;
    int32_t row_lo = 0;
    int32_t n_rows = 0;
    int32_t out = -1;
};

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

int make_plan(const Tree& t, int32_t b, const int32_t* q_order, const PlanOpts& in_opts,
              Plan& plan, std::string& err) {
    if (b < 1 || !q_order) {
        err = "plan: need b >= 1 and a q_order array";
        return PKVT_ERR_INVALID_ARG;
    }
    PlanOpts opts = in_opts;
    if (opts.min_share == 0) opts.min_share = 2;
    if (opts.min_share < 2 || opts.phase1_chunks < 0 || opts.phase2_chunks < 0) {
        err = "plan: min_share must be >= 2 (or 0 for the default); chunk limits >= 0";
        return PKVT_ERR_INVALID_ARG;
    }
    const int32_t steps_to_chunks = std::max(1, kKeysPerStep / t.C);
    const int32_t s1 = opts.phase1_chunks ? opts.phase1_chunks
                                          : std::max(1, kDefaultPhase1Steps * kKeysPerStep / t.C);
    const int32_t s2 = opts.phase2_chunks ? opts.phase2_chunks
                                          : std::max(1, kDefaultPhase2Steps * kKeysPerStep / t.C);
    (void)steps_to_chunks;

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
    if (plan.valid && plan.struct_version == t.structure_version() && plan.b == b &&
        plan.opts == opts && std::equal(q_order, q_order + b, plan.q_order.begin())) {
        write_seqlen(t, plan);
        plan.len_version = t.length_version();
        return PKVT_OK;
    }

    // ---- 1. depth-first order over the batch's paths --------------------------
    const int32_t root = t.root();
    std::unordered_map<int32_t, std::vector<int32_t>> ends;      // leaf node -> rows
    std::unordered_map<int32_t, Range> range;                    // node -> [i, j)
    for (int32_t r = 0; r < b; ++r) {
        for (int32_t x : seqs[r]->path) range.emplace(x, Range{});
        ends[seqs[r]->path.back()].push_back(r);
    }
    std::vector<int32_t> dfs_row;             // depth-first position -> query row
    std::vector<int32_t> preorder;            // visited nodes, parents first
    dfs_row.reserve(b);
    {
        struct Frame { int32_t node; size_t next; };
        std::vector<Frame> stack{{root, 0}};
        range[root] = Range{0, 0};
        while (!stack.empty()) {
            Frame& f = stack.back();
            const Node& n = t.node(f.node);
            if (f.next < n.children.size()) {
                const int32_t ch = n.children[f.next++];
                auto it = range.find(ch);
                if (it == range.end()) continue;                  // not on a batch path
                it->second.i = static_cast<int32_t>(dfs_row.size());
                preorder.push_back(ch);
                auto e = ends.find(ch);
                if (e != ends.end())
                    for (int32_t r : e->second) dfs_row.push_back(r);
                stack.push_back({ch, 0});
            } else {
                range[f.node].j = static_cast<int32_t>(dfs_row.size());
                stack.pop_back();
            }
        }
    }
    if (static_cast<int32_t>(dfs_row.size()) != b) {
        err = "plan: internal error, depth-first order lost rows";
        return PKVT_ERR_INVALID_ARG;
    }
    std::vector<int32_t> pos_of_row(b);
    for (int32_t p = 0; p < b; ++p) pos_of_row[dfs_row[p]] = p;
    auto cov = [&](int32_t x) { const Range& r = range[x]; return r.j - r.i; };

    // ---- 2. phase-1 segments and items ------------------------------------------
    std::vector<Item> items1;
    std::vector<int32_t> src_count(b, 0);
    int32_t shared_chunks = 0;
    {
        std::vector<std::vector<int32_t>> segs;
        std::vector<Range> seg_range;
        std::unordered_map<int32_t, int32_t> seg_of;
        for (int32_t x : preorder) {
            if (cov(x) < opts.min_share) continue;
            const int32_t p = t.node(x).parent;
            auto it = seg_of.find(p);
            if (p != root && it != seg_of.end() && range[p].i == range[x].i &&
                range[p].j == range[x].j) {
                segs[it->second].push_back(x);
                seg_of[x] = it->second;
            } else {
                seg_of[x] = static_cast<int32_t>(segs.size());
                segs.push_back({x});
                seg_range.push_back(range[x]);
            }
        }
        for (size_t s = 0; s < segs.size(); ++s) {
            shared_chunks += static_cast<int32_t>(segs[s].size());
            for (size_t a = 0; a < segs[s].size(); a += s1) {
                Item it;
                it.chunks.assign(segs[s].begin() + a,
                                 segs[s].begin() + std::min(segs[s].size(), a + s1));
                it.row_lo = seg_range[s].i;
                it.n_rows = seg_range[s].j - seg_range[s].i;
                for (int32_t p = seg_range[s].i; p < seg_range[s].j; ++p) src_count[p]++;
                items1.push_back(std::move(it));
            }
        }
    }

    // ---- 3. phase-2 items --------------------------------------------------------
    std::vector<Item> items2;
    for (int32_t p = 0; p < b; ++p) {
        const std::vector<int32_t>& path = seqs[dfs_row[p]]->path;
        int32_t k0 = static_cast<int32_t>(path.size());
        while (k0 > 0 && cov(path[k0 - 1]) < opts.min_share) --k0;
        for (int32_t a = k0; a < static_cast<int32_t>(path.size()); a += s2) {
            Item it;
            const int32_t e = std::min<int32_t>(static_cast<int32_t>(path.size()), a + s2);
            it.chunks.assign(path.begin() + a, path.begin() + e);
            it.key_base = a * t.C;
            it.len_row = (e == static_cast<int32_t>(path.size())) ? p : -1;
            it.row_lo = p;
            it.n_rows = 1;
            src_count[p]++;
            items2.push_back(std::move(it));
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

    // ---- 5. waves and workgroups (longest first) -------------------------------------
    std::vector<WaveDesc> waves;
    std::vector<std::vector<int32_t>> chunk_lists;
    struct Unit { std::vector<int32_t> waves; int32_t cost; };
    std::vector<Unit> units1;
    std::vector<int32_t> waves2;
    auto add_wave = [&](const Item& it, int32_t row_off) {
        WaveDesc w{};
        w.chunk_off = 0;                                   // filled at emission
        w.n_chunks = static_cast<int32_t>(it.chunks.size());
        w.key_base = it.key_base;
        w.len_row = it.len_row;
        w.row_lo = it.row_lo + row_off;
        w.n_rows = std::min(kRowsPerWave, it.n_rows - row_off);
        w.out = it.out < 0 ? -1 : it.out + row_off;
        waves.push_back(w);
        chunk_lists.push_back(it.chunks);
        return static_cast<int32_t>(waves.size()) - 1;
    };
    for (const Item& it : items1) {
        for (int32_t r0 = 0; r0 < it.n_rows; r0 += kRowsPerWave * kWavesPerWg) {
            Unit u;
            u.cost = static_cast<int32_t>(it.chunks.size());
            for (int32_t r = r0; r < std::min(it.n_rows, r0 + kRowsPerWave * kWavesPerWg);
                 r += kRowsPerWave)
                u.waves.push_back(add_wave(it, r));
            units1.push_back(std::move(u));
        }
    }
    for (const Item& it : items2) waves2.push_back(add_wave(it, 0));
    std::stable_sort(units1.begin(), units1.end(),
                     [](const Unit& a, const Unit& c) { return a.cost > c.cost; });
    std::stable_sort(waves2.begin(), waves2.end(), [&](int32_t a, int32_t c) {
        return waves[a].n_chunks > waves[c].n_chunks;
    });
    std::vector<Unit> wgs;
    size_t next2 = 0;
    for (Unit& u : units1) {
        while (u.waves.size() < static_cast<size_t>(kWavesPerWg) && next2 < waves2.size()) {
            u.cost = std::max(u.cost, waves[waves2[next2]].n_chunks);
            u.waves.push_back(waves2[next2++]);
        }
        wgs.push_back(std::move(u));
    }
    while (next2 < waves2.size()) {
        Unit u;
        u.cost = 0;
        while (u.waves.size() < static_cast<size_t>(kWavesPerWg) && next2 < waves2.size()) {
            u.cost = std::max(u.cost, waves[waves2[next2]].n_chunks);
            u.waves.push_back(waves2[next2++]);
        }
        wgs.push_back(std::move(u));
    }
    std::stable_sort(wgs.begin(), wgs.end(),
                     [](const Unit& a, const Unit& c) { return a.cost > c.cost; });

    // ---- 6. emit the blob -------------------------------------------------------------
    const int32_t n_wg = static_cast<int32_t>(wgs.size());
    const int32_t n_waves = static_cast<int32_t>(waves.size());
    int32_t total_chunks = 0;
    for (auto& l : chunk_lists) total_chunks += static_cast<int32_t>(l.size());
    std::vector<int32_t> merge_rows;
    for (int32_t p = 0; p < b; ++p)
        if (!mslots[p].empty()) merge_rows.push_back(p);
    int32_t n_mslots = 0;
    for (auto& m : mslots) n_mslots += static_cast<int32_t>(m.size());

    std::vector<int32_t> blob(kHeaderWords, 0);
    auto section = [&](HeaderField f, size_t words) {
        // keep every section 16-byte aligned
        while (blob.size() % 4) blob.push_back(0);
        blob[f] = static_cast<int32_t>(blob.size());
        blob.resize(blob.size() + words, 0);
    };
    section(kOffWg, static_cast<size_t>(n_wg) * kWavesPerWg);
    section(kOffWaves, static_cast<size_t>(n_waves) * 8);
    section(kOffChunks, total_chunks);
    section(kOffRows, b);
    section(kOffMerge, merge_rows.size());
    section(kOffMptr, b + 1);
    section(kOffMslots, n_mslots);
    section(kOffSeqlen, b);
    while (blob.size() % 4) blob.push_back(0);

    // waves are renumbered in workgroup order so neighbours read neighbours
    int32_t wslot = 0, coff = 0;
    for (int32_t g = 0; g < n_wg; ++g) {
        for (int32_t k = 0; k < kWavesPerWg; ++k) {
            int32_t* wg = &blob[blob[kOffWg] + g * kWavesPerWg + k];
            if (k >= static_cast<int32_t>(wgs[g].waves.size())) {
                *wg = -1;
                continue;
            }
            const int32_t src = wgs[g].waves[k];
            WaveDesc w = waves[src];
            w.chunk_off = coff;
            for (int32_t id : chunk_lists[src]) blob[blob[kOffChunks] + coff++] = id;
            std::copy(reinterpret_cast<const int32_t*>(&w),
                      reinterpret_cast<const int32_t*>(&w) + 8,
                      &blob[blob[kOffWaves] + wslot * 8]);
            *wg = wslot++;
        }
    }
    for (int32_t p = 0; p < b; ++p) blob[blob[kOffRows] + p] = dfs_row[p];
    for (size_t m = 0; m < merge_rows.size(); ++m) blob[blob[kOffMerge] + m] = merge_rows[m];
    {
        int32_t at = 0;
        for (int32_t p = 0; p < b; ++p) {
            blob[blob[kOffMptr] + p] = at;
            for (int32_t s : mslots[p]) blob[blob[kOffMslots] + at++] = s;
        }
        blob[blob[kOffMptr] + b] = at;
    }
    blob[kMagic] = kPlanMagic;
    blob[kB] = b;
    blob[kNWaves] = n_waves;
    blob[kNWg] = n_wg;
    blob[kNSlots] = n_slots;
    blob[kNMerge] = static_cast<int32_t>(merge_rows.size());
    blob[kTotalWords] = static_cast<int32_t>(blob.size());

    // unique (stored) tokens of the batch: every distinct node once
    int64_t unique = 0;
    for (auto& kv : range)
        if (kv.first != root) unique += t.node(kv.first).fill;

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
    plan.n_wg = n_wg;
    plan.n_slots = n_slots;
    plan.n_merge = static_cast<int32_t>(merge_rows.size());
    plan.shared_chunks = shared_chunks;
    plan.unique_tokens = unique;
    plan.dfs_seq.resize(b);
    for (int32_t p = 0; p < b; ++p) plan.dfs_seq[p] = q_order[dfs_row[p]];
    write_seqlen(t, plan);
    return PKVT_OK;
}

}  // namespace pkvt
