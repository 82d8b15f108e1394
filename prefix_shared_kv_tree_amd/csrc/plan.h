// Context generation for one decode batch: the host side of the two-phase
// partition ("ChunkAttention ..." chapterpal digest, Knowl 2 and Knowl 5).
//
// The plan is a flat int32 blob that is copied to device memory once and
// re-used for every layer and every decode step until the tree structure
// changes (lazy context copy, Knowl 5).  Layout (word offsets in the header):
//
//   header   [kHeaderWords]
//   lists    [4*G][2]          per wave lane of the G persistent workgroups:
//                              (first entry in tasks, number of tasks)
//   tasks    [n_tasks][2]      (wave descriptor index, head), in lane order
//   waves    [n_waves][8]      WaveDesc (head-independent)
//   wgunits  [G][2]            per workgroup: (first entry in units, count)
//   units    [n_units][8]      UnitDesc, in workgroup order
//   chunks   [...]             chunk ids referenced by the waves and units
//   rows     [b]               depth-first position -> query row of Q / O
//   merge    [n_merge]         depth-first positions whose partials are merged
//   mptr     [b+1]             CSR over depth-first positions ...
//   mslots   [...]             ... of partial slot indices
//   seqlen   [b]               tokens stored per depth-first position (last,
//                              so that a length-only update copies one range)
#pragma once

#include <cstdint>
#include <string>
#include <unordered_map>
#include <vector>

#include "shapes.h"
#include "tree.h"

namespace pkvt {

// One 64-lane unit of work of the attention kernel: up to 16 query rows
// against a list of chunks of one head (the head comes from the task list).
// Every chunk but the last is full; key k lies in chunk k / C.
struct WaveDesc {
    int32_t chunk_off;   // first entry in the chunks section
    int32_t n_chunks;
    int32_t key_base;    // index, within its sequence, of the first key (len_row >= 0)
    int32_t len_row;     // depth-first row whose length bounds the keys, -1 = tail bounds them
    int32_t row_lo;      // depth-first position of query row 0
    int32_t n_rows;      // 1..16
    int32_t out;         // partial slot of row 0, or -1: write O directly (n_rows == 1)
    int32_t tail;        // keys missing from the last chunk (len_row < 0): C minus its fill
};
static_assert(sizeof(WaveDesc) == 32, "WaveDesc is 8 int32");

// A workgroup unit: query rows [row_lo, row_lo + n_rows) (17..64 rows in
// decode, up to 64 per row tile count in prefill) of one head against a list
// of chunks, every one but the last full.  All 4 waves of one workgroup run
// it in lock step: each loads a quarter of every 64-key step into LDS and
// computes its rows from there.
struct UnitDesc {
    int32_t n_keys;      // keys read: (n_chunks - 1) * C plus what the last chunk holds (or less)
    int32_t chunk_off;   // first entry in the chunks section
    int32_t n_chunks;
    int32_t head;
    int32_t row_lo;      // depth-first position of row 0
    int32_t n_rows;
    int32_t out;         // partial slot of row 0
    int32_t key_base;    // prefill: sequence position of the first key (causal mask); decode: 0
};
static_assert(sizeof(UnitDesc) == 32, "UnitDesc is 8 int32");

enum HeaderField {
    kMagic = 0, kSerial, kB, kNWaves, kNWg, kNTasks, kNSlots, kNMerge,
    kOffLists, kOffTasks, kOffWaves, kOffChunks, kOffRows, kOffMerge, kOffMptr, kOffMslots,
    kOffSeqlen, kTotalWords, kNUnits, kOffWgUnits, kOffUnits, kOffQpos, kKernel,
    kHeaderWords = 24
};
constexpr int32_t kPlanMagic = 0x504b5657;   // "PKVW": lane lists + workgroup units
constexpr int32_t kRowsPerUnit = 64;         // query rows of one workgroup-unit block
constexpr int32_t kWavesPerWg = 4;
constexpr int32_t kRowsPerWave = 16;
constexpr int32_t kKeysPerStep = 64;
constexpr int32_t kDefaultWorkgroups = 512;  // 256 CUs x 2 resident workgroups
constexpr int32_t kMaxItemChunks = 64;       // chunks per work item (one per wave lane)
constexpr int32_t kUnitStepCost = 2;         // quarter steps per wave of a unit step (4 = a task step)
constexpr int32_t kYoungSpeedPct = 70;       // speed of a compute unit's younger workgroup, % of the older
// Prefill workgroups (one resident per compute unit) run in two rounds, the
// second starting as the first finish: the second round's load, % of the first's.
constexpr int32_t kPrefillSecondRoundPct = 60;
constexpr int32_t kAppendSlack = 2;          // chunk ids reserved after a row's last item for appends
constexpr int32_t kMaxPatches = 256;         // incremental patches before a plan is rebuilt anyway

struct PlanOpts {
    int32_t phase1_chunks = 0;   // 0 = derived from the balanced per-lane load
    int32_t phase2_chunks = 0;
    int32_t min_share = 2;
    int32_t workgroups = 0;      // persistent workgroups; 0 = kDefaultWorkgroups
    int32_t unit_rows = 0;       // smallest row block run as a workgroup unit; 0 = 17
    bool operator==(const PlanOpts& o) const {
        return phase1_chunks == o.phase1_chunks && phase2_chunks == o.phase2_chunks &&
               min_share == o.min_share && workgroups == o.workgroups && unit_rows == o.unit_rows;
    }
};

// Per-node working state of the planner, kept between calls so that a
// re-plan allocates nothing proportional to the pool.  An entry is valid when
// its mark equals the current epoch.
struct PlanScratch {
    struct NodeInfo { int32_t i, j, seg, first_row; };
    std::vector<uint32_t> mark;
    std::vector<NodeInfo> node;
    uint32_t epoch = 0;
};

struct Plan {
    bool valid = false;
    int64_t serial = 0;               // identifies the structure part of the blob
    int64_t struct_version = -1;      // tree versions the plan was built from
    int64_t len_version = -1;
    int32_t b = 0;
    std::vector<int32_t> q_order;
    PlanOpts opts;
    std::vector<int32_t> blob;
    // summary
    int32_t phase1_items = 0, phase2_items = 0, n_waves = 0, n_wg = 0, n_tasks = 0, n_units = 0;
    int32_t kernel = 0;               // 0: attn_kernel; 1: unit_kernel (units-only decode plans)
    int32_t n_slots = 0, n_merge = 0;
    int32_t split1_chunks = 0, split2_chunks = 0;   // the item sizes actually used
    int32_t shared_chunks = 0;
    int64_t unique_tokens = 0, logical_tokens = 0;
    std::vector<int32_t> dfs_seq;     // depth-first position -> sequence id (tests)
    PlanScratch scratch;
    // Incremental patching: a decode append that opens a new leaf chunk adds
    // that chunk to the end of its row's last work item, in room reserved
    // after the item's chunk ids, instead of rebuilding the plan.
    std::vector<int32_t> last_wave;   // depth-first position -> wave of its last item, -1 if none
    std::vector<int32_t> last_k0;     // ... and the path index of that item's first chunk
    std::vector<int32_t> wave_cap;    // chunk ids reserved per wave
    std::unordered_map<int32_t, int32_t> pos_of_seq;   // sequence id -> depth-first position
    int32_t patches = 0;              // patches since the plan was last built
    int32_t last_update = 0;          // last make_plan: 0 lengths only, 1 patched, 2 rebuilt

    int32_t off(HeaderField f) const { return blob[f]; }
};

// Build (or refresh) the plan.  Returns a PKVT_* status.
int make_plan(const Tree& tree, int32_t b, const int32_t* q_order, const PlanOpts& opts,
              Plan& plan, std::string& err);

// Prefill plan: the query rows are positions q_from[s] .. len - 1 of each of
// the n sequences seq_ids[s] (in that order, positions ascending), and a row
// at position p attends to its sequence's tokens 0 .. p.  Rows are cut into
// blocks of up to 16 * prefill_waves(d) * prefill_row_tiles(d) depth-first rows; a block reads
// the chunks common to its sequences once for all its rows and each
// sequence's own chunks for that sequence's rows, with the causal mask
// applied per row in the kernel.  The blob has the decode layout with no
// single-wave tasks, plus qpos [R] (position of every depth-first row); b is
// the row count R; rows read by one unit only get O from it directly, the
// others are merged from their partials.  Options used: phase1_chunks
// (chunks per unit, 0 = kPrefillMaxChunks) and workgroups.
int make_prefill_plan(const Tree& tree, int32_t n, const int32_t* seq_ids, const int64_t* q_from,
                      const PlanOpts& opts, Plan& plan, std::string& err);

}  // namespace pkvt
