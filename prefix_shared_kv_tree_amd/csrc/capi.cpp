// C ABI of libpkvt (declared in include/pkvt.h): argument checking, the
// lazy metadata upload and kernel launches.  No device memory is allocated
// here; the only HIP allocation is the pinned host staging buffer of the
// metadata upload, made on the first upload.
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <new>
#include <string>

#include "kernels.h"
#include "pkvt.h"
#include "plan.h"
#include "tree.h"

// Pinned host buffer that the metadata upload kernel reads through its
// device mapping, with the event that marks the end of that read.
struct Staging {
    int32_t* host = nullptr;
    const int32_t* dev = nullptr;
    size_t words = 0;
    hipEvent_t done = nullptr;
    bool in_flight = false;
};
constexpr int kStagingRing = 4;

// What the last upload of a plan put where.
struct Uploaded {
    const void* ptr = nullptr;
    int64_t serial = -1;
    int64_t len_version = -1;
};

struct pkvt_tree {
    pkvt::Tree tree;
    pkvt::Plan plan;          // decode
    pkvt::Plan prefill;       // prefill
    Uploaded up_plan, up_prefill;
    Staging staging[kStagingRing];
    int next_staging = 0;

    pkvt_tree(int32_t h, int32_t d, int32_t c, int32_t n, pkvt::Match m) : tree(h, d, c, n, m) {}
    ~pkvt_tree() {
        for (Staging& st : staging) {
            if (st.in_flight) (void)hipEventSynchronize(st.done);
            if (st.host) (void)hipHostFree(st.host);
            if (st.done) (void)hipEventDestroy(st.done);
        }
    }
};

namespace {

thread_local std::string g_last_error;

pkvt_status fail(pkvt_status code, const std::string& msg) {
    g_last_error = msg;
    return code;
}

pkvt_status hip_fail(hipError_t e, const std::string& what) {
    return fail(PKVT_ERR_HIP, what + ": " + hipGetErrorString(e));
}

bool shape_ok(int32_t d, int32_t c) {
    return (d == 64 || d == 128 || d == 256) && (c == 16 || c == 32 || c == 64 || c == 128);
}

// Two resident workgroups of 4 waves per compute unit: the attention kernel
// is built for 2 waves per SIMD.  Falls back to a 256-CU device when no GPU
// is visible (host-only use of the planner).
int32_t default_workgroups() {
    static int32_t cached = -1;
    if (cached > 0) return cached;
    int n = 0, dev = 0, cus = 0;
    if (hipGetDeviceCount(&n) == hipSuccess && n > 0 && hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
        cus > 0) {
        cached = 2 * cus;
    } else {
        (void)hipGetLastError();
        cached = pkvt::kDefaultWorkgroups;
    }
    return cached;
}

bool current(const pkvt_tree* t, const pkvt::Plan& p) {
    return p.valid && p.struct_version == t->tree.structure_version() &&
           p.len_version == t->tree.length_version();
}
bool plan_current(const pkvt_tree* t) { return current(t, t->plan); }

// Copy plan p into d_meta (lazily: nothing when d_meta already holds it;
// with len_refresh, only the length table when only lengths changed) through
// the next staging buffer of the ring and the word-copy kernel.  other: the
// upload record of the tree's other plan, forgotten if d_meta held it.
pkvt_status upload(pkvt_tree* t, const pkvt::Plan& p, Uploaded& up, Uploaded& other,
                   void* d_meta, size_t meta_bytes, void* stream, bool len_refresh,
                   const std::string& who) {
    const size_t words = p.blob.size();
    if (meta_bytes < words * sizeof(int32_t))
        return fail(PKVT_ERR_BUFFER_TOO_SMALL, who + ": meta buffer smaller than the plan");
    size_t first = 0, count = words;
    if (up.ptr == d_meta && up.serial == p.serial) {
        if (up.len_version == p.len_version) return PKVT_OK;             // already there
        if (len_refresh) {
            first = static_cast<size_t>(p.blob[pkvt::kOffSeqlen]);       // lengths only
            count = static_cast<size_t>(p.b);
        }
    }
    if (count % 4) count += 4 - count % 4;            // sections are padded to 16 bytes
    count = std::min(count, words - first);
    hipError_t e;
    Staging& st = t->staging[t->next_staging];
    if (st.in_flight) {
        if ((e = hipEventSynchronize(st.done)) != hipSuccess) return hip_fail(e, who);
        st.in_flight = false;
    }
    if (!st.done && (e = hipEventCreateWithFlags(&st.done, hipEventDisableTiming)) != hipSuccess)
        return hip_fail(e, who + ": event");
    if (st.words < words) {
        if (st.host) (void)hipHostFree(st.host);
        st.host = nullptr;
        st.dev = nullptr;
        st.words = 0;
        const size_t want = words + words / 2;        // room for the plan to grow
        if ((e = hipHostMalloc(reinterpret_cast<void**>(&st.host), want * sizeof(int32_t),
                               hipHostMallocMapped | hipHostMallocCoherent)) != hipSuccess)
            return hip_fail(e, who + ": pinned staging");
        void* dev = nullptr;
        if ((e = hipHostGetDevicePointer(&dev, st.host, 0)) != hipSuccess) {
            (void)hipHostFree(st.host);
            st.host = nullptr;
            return hip_fail(e, who + ": staging mapping");
        }
        st.dev = static_cast<const int32_t*>(dev);
        st.words = want;
    }
    std::memcpy(st.host + first, p.blob.data() + first, count * sizeof(int32_t));
    auto s = static_cast<hipStream_t>(stream);
    if ((e = pkvt::launch_copy_words(st.dev + first, static_cast<int32_t*>(d_meta) + first,
                                     static_cast<int64_t>(count), s)) != hipSuccess)
        return hip_fail(e, who + ": copy kernel");
    if ((e = hipEventRecord(st.done, s)) != hipSuccess) return hip_fail(e, who + ": record");
    st.in_flight = true;
    t->next_staging = (t->next_staging + 1) % kStagingRing;
    up.ptr = d_meta;
    up.serial = p.serial;
    up.len_version = p.len_version;
    if (other.ptr == d_meta) other = Uploaded{};
    return PKVT_OK;
}

void fill_info(const pkvt::Plan& p, pkvt_plan_info* out) {
    std::memset(out, 0, sizeof(*out));
    out->b = p.b;
    out->phase1_items = p.phase1_items;
    out->phase2_items = p.phase2_items;
    out->waves = p.n_waves;
    out->workgroups = p.n_wg;
    out->slots = p.n_slots;
    out->merge_rows = p.n_merge;
    out->shared_chunks = p.shared_chunks;
    out->unique_tokens = p.unique_tokens;
    out->logical_tokens = p.logical_tokens;
    out->structure_version = static_cast<int32_t>(p.serial & 0x7fffffff);
    out->tasks = p.n_tasks;
    out->phase1_split = p.split1_chunks;
    out->phase2_split = p.split2_chunks;
    out->wg_units = p.n_units;
    out->last_update = p.last_update;
    out->patches = p.patches;
    out->kernel = p.kernel;
}

}  // namespace

extern "C" {

const char* pkvt_last_error(void) { return g_last_error.c_str(); }

pkvt_status pkvt_pool_bytes(int32_t n_heads, int32_t head_dim, int32_t chunk_size,
                            int32_t pool_chunks, size_t* bytes) {
    if (!bytes || n_heads < 1 || pool_chunks < 1)
        return fail(PKVT_ERR_INVALID_ARG, "pool_bytes: bad arguments");
    if (!shape_ok(head_dim, chunk_size))
        return fail(PKVT_ERR_UNSUPPORTED_SHAPE, "pool_bytes: head_dim must be 64, 128 or 256 and "
                                                "chunk_size one of 16, 32, 64, 128");
    *bytes = static_cast<size_t>(pool_chunks) * n_heads * chunk_size * head_dim * 2;
    return PKVT_OK;
}

pkvt_status pkvt_tree_create_ex(int32_t n_heads, int32_t head_dim, int32_t chunk_size,
                                int32_t pool_chunks, int32_t match, pkvt_tree** out) {
    if (!out) return fail(PKVT_ERR_INVALID_ARG, "tree_create: out is NULL");
    *out = nullptr;
    if (n_heads < 1 || head_dim < 1 || chunk_size < 1 || chunk_size > 4096 || pool_chunks < 1)
        return fail(PKVT_ERR_INVALID_ARG, "tree_create: need n_heads, head_dim, pool_chunks >= 1 "
                                          "and chunk_size in [1, 4096]");
    if (match != PKVT_MATCH_CHUNKS && match != PKVT_MATCH_TOKENS)
        return fail(PKVT_ERR_INVALID_ARG, "tree_create: match must be PKVT_MATCH_CHUNKS or PKVT_MATCH_TOKENS");
    try {
        *out = new pkvt_tree(n_heads, head_dim, chunk_size, pool_chunks,
                             match == PKVT_MATCH_TOKENS ? pkvt::Match::kTokens : pkvt::Match::kChunks);
    } catch (const std::bad_alloc&) {
        return fail(PKVT_ERR_HOST_MEMORY, "tree_create: out of host memory");
    }
    return PKVT_OK;
}

pkvt_status pkvt_tree_create(int32_t n_heads, int32_t head_dim, int32_t chunk_size,
                             int32_t pool_chunks, pkvt_tree** out) {
    return pkvt_tree_create_ex(n_heads, head_dim, chunk_size, pool_chunks, PKVT_MATCH_CHUNKS, out);
}

void pkvt_tree_destroy(pkvt_tree* tree) { delete tree; }

#define PKVT_GUARD(expr)                                                         \
    try {                                                                        \
        expr;                                                                    \
    } catch (const std::bad_alloc&) {                                            \
        return fail(PKVT_ERR_HOST_MEMORY, "out of host memory");                 \
    } catch (const std::exception& e) {                                          \
        return fail(PKVT_ERR_INVALID_ARG, e.what());                             \
    }

pkvt_status pkvt_tree_build(pkvt_tree* t, int32_t n_seqs, const int32_t* tokens,
                            const int64_t* offsets, int32_t* seq_ids, int64_t* slots) {
    if (!t) return fail(PKVT_ERR_INVALID_ARG, "tree_build: tree is NULL");
    std::string err;
    int rc = 0;
    PKVT_GUARD(rc = t->tree.build(n_seqs, tokens, offsets, seq_ids, slots, err));
    return rc ? fail(rc, err) : PKVT_OK;
}

pkvt_status pkvt_tree_append(pkvt_tree* t, int32_t n, const int32_t* seq_ids,
                             const int32_t* tokens, int64_t* slots) {
    if (!t) return fail(PKVT_ERR_INVALID_ARG, "tree_append: tree is NULL");
    std::string err;
    int rc = 0;
    PKVT_GUARD(rc = t->tree.append(n, seq_ids, tokens, slots, err));
    return rc ? fail(rc, err) : PKVT_OK;
}

pkvt_status pkvt_tree_remove(pkvt_tree* t, int32_t seq_id) {
    if (!t) return fail(PKVT_ERR_INVALID_ARG, "tree_remove: tree is NULL");
    std::string err;
    int rc = 0;
    PKVT_GUARD(rc = t->tree.remove(seq_id, err));
    return rc ? fail(rc, err) : PKVT_OK;
}

pkvt_status pkvt_tree_stats(const pkvt_tree* t, pkvt_stats* out) {
    if (!t || !out) return fail(PKVT_ERR_INVALID_ARG, "tree_stats: NULL argument");
    std::memset(out, 0, sizeof(*out));
    out->capacity = t->tree.N;
    out->used_chunks = t->tree.used_chunks();
    out->free_chunks = t->tree.N - out->used_chunks;
    out->shared_chunks = t->tree.shared_chunks();
    out->live_seqs = t->tree.live_seqs();
    return PKVT_OK;
}

pkvt_status pkvt_tree_chunk_path(const pkvt_tree* t, int32_t seq_id, int32_t* ids, int32_t cap,
                                 int32_t* n) {
    if (!t || !n || (cap > 0 && !ids)) return fail(PKVT_ERR_INVALID_ARG, "chunk_path: NULL argument");
    const pkvt::Seq* s = t->tree.find_seq(seq_id);
    if (!s) return fail(PKVT_ERR_UNKNOWN_SEQ, "chunk_path: unknown sequence id " + std::to_string(seq_id));
    *n = static_cast<int32_t>(s->path.size());
    if (cap < *n) return fail(PKVT_ERR_BUFFER_TOO_SMALL, "chunk_path: cap smaller than the path");
    std::memcpy(ids, s->path.data(), sizeof(int32_t) * s->path.size());
    return PKVT_OK;
}

pkvt_status pkvt_tree_seq_len(const pkvt_tree* t, int32_t seq_id, int64_t* len) {
    if (!t || !len) return fail(PKVT_ERR_INVALID_ARG, "seq_len: NULL argument");
    const pkvt::Seq* s = t->tree.find_seq(seq_id);
    if (!s) return fail(PKVT_ERR_UNKNOWN_SEQ, "seq_len: unknown sequence id " + std::to_string(seq_id));
    *len = s->len;
    return PKVT_OK;
}

pkvt_status pkvt_tree_chunk_refcount(const pkvt_tree* t, int32_t chunk_id, int32_t* refs) {
    if (!t || !refs) return fail(PKVT_ERR_INVALID_ARG, "chunk_refcount: NULL argument");
    if (chunk_id < 0 || chunk_id >= t->tree.N)
        return fail(PKVT_ERR_INVALID_ARG, "chunk_refcount: chunk id out of range");
    const pkvt::Node& x = t->tree.node(chunk_id);
    *refs = x.live ? x.refs : 0;
    return PKVT_OK;
}

pkvt_status pkvt_tree_chunk_fill(const pkvt_tree* t, int32_t chunk_id, int32_t* fill) {
    if (!t || !fill) return fail(PKVT_ERR_INVALID_ARG, "chunk_fill: NULL argument");
    if (chunk_id < 0 || chunk_id >= t->tree.N)
        return fail(PKVT_ERR_INVALID_ARG, "chunk_fill: chunk id out of range");
    const pkvt::Node& x = t->tree.node(chunk_id);
    *fill = x.live ? x.fill : 0;
    return PKVT_OK;
}

pkvt_status pkvt_tree_moves(const pkvt_tree* t, int64_t* src, int64_t* dst, int64_t cap, int64_t* n) {
    if (!t || !n) return fail(PKVT_ERR_INVALID_ARG, "tree_moves: NULL argument");
    const auto& mv = t->tree.moves();
    *n = static_cast<int64_t>(mv.size());
    if (mv.empty()) return PKVT_OK;
    if (cap < *n) return fail(PKVT_ERR_BUFFER_TOO_SMALL, "tree_moves: cap < number of moves");
    if (!src || !dst) return fail(PKVT_ERR_INVALID_ARG, "tree_moves: NULL output array");
    for (size_t i = 0; i < mv.size(); ++i) {
        src[i] = mv[i].first;
        dst[i] = mv[i].second;
    }
    return PKVT_OK;
}

pkvt_status pkvt_plan(pkvt_tree* t, int32_t b, const int32_t* q_order, const pkvt_plan_opts* opts,
                      size_t* meta_bytes, size_t* workspace_bytes) {
    if (!t) return fail(PKVT_ERR_INVALID_ARG, "plan: tree is NULL");
    pkvt::PlanOpts o;
    if (opts) {
        o.phase1_chunks = opts->phase1_chunks;
        o.phase2_chunks = opts->phase2_chunks;
        o.min_share = opts->min_share;
        o.workgroups = opts->workgroups;
        o.unit_rows = opts->unit_rows;
    }
    if (o.workgroups < 0) return fail(PKVT_ERR_INVALID_ARG, "plan: workgroups must be >= 0");
    if (o.workgroups == 0) o.workgroups = default_workgroups();
    std::string err;
    int rc = 0;
    PKVT_GUARD(rc = pkvt::make_plan(t->tree, b, q_order, o, t->plan, err));
    if (rc) return fail(rc, err);
    if (meta_bytes) *meta_bytes = t->plan.blob.size() * sizeof(int32_t);
    if (workspace_bytes)
        *workspace_bytes = static_cast<size_t>(t->plan.n_slots) * t->tree.H * (t->tree.D + 2) *
                           sizeof(float);
    return PKVT_OK;
}

pkvt_status pkvt_plan_info_get(const pkvt_tree* t, pkvt_plan_info* out) {
    if (!t || !out) return fail(PKVT_ERR_INVALID_ARG, "plan_info: NULL argument");
    if (!t->plan.valid) return fail(PKVT_ERR_STALE_PLAN, "plan_info: no plan");
    fill_info(t->plan, out);
    return PKVT_OK;
}

pkvt_status pkvt_plan_blob(const pkvt_tree* t, int32_t* out, int32_t cap, int32_t* n) {
    if (!t || !n || (cap > 0 && !out)) return fail(PKVT_ERR_INVALID_ARG, "plan_blob: NULL argument");
    if (!t->plan.valid) return fail(PKVT_ERR_STALE_PLAN, "plan_blob: no plan");
    *n = static_cast<int32_t>(t->plan.blob.size());
    if (cap < *n) return fail(PKVT_ERR_BUFFER_TOO_SMALL, "plan_blob: cap smaller than the plan");
    std::memcpy(out, t->plan.blob.data(), t->plan.blob.size() * sizeof(int32_t));
    return PKVT_OK;
}

pkvt_status pkvt_plan_upload(pkvt_tree* t, void* d_meta, size_t meta_bytes, void* stream) {
    if (!t || !d_meta) return fail(PKVT_ERR_INVALID_ARG, "plan_upload: NULL argument");
    if (!plan_current(t)) return fail(PKVT_ERR_STALE_PLAN, "plan_upload: no plan for the current tree");
    if (!shape_ok(t->tree.D, t->tree.C))
        return fail(PKVT_ERR_UNSUPPORTED_SHAPE, "plan_upload: the kernels need head_dim 64, 128 or 256 "
                                                "and chunk_size 16, 32, 64 or 128");
    return upload(t, t->plan, t->up_plan, t->up_prefill, d_meta, meta_bytes, stream, true,
                  "plan_upload");
}

pkvt_status pkvt_attn_decode(const pkvt_tree* t, const void* d_meta, const void* q,
                             const void* k_pool, const void* v_pool, void* out, void* workspace,
                             size_t workspace_bytes, float scale, void* stream) {
    return pkvt_attn_decode_ex(t, d_meta, q, k_pool, v_pool, out, workspace, workspace_bytes,
                               scale, stream, nullptr, nullptr);
}

pkvt_status pkvt_attn_decode_ex(const pkvt_tree* t, const void* d_meta, const void* q,
                                const void* k_pool, const void* v_pool, void* out,
                                void* workspace, size_t workspace_bytes, float scale,
                                void* stream, void* attn_start_event, void* attn_end_event) {
    if (!t || !d_meta || !q || !k_pool || !v_pool || !out)
        return fail(PKVT_ERR_INVALID_ARG, "attn_decode: NULL argument");
    if (!std::isfinite(scale)) return fail(PKVT_ERR_INVALID_ARG, "attn_decode: scale is not finite");
    if (!plan_current(t)) return fail(PKVT_ERR_STALE_PLAN, "attn_decode: plan is older than the tree");
    if (!shape_ok(t->tree.D, t->tree.C))
        return fail(PKVT_ERR_UNSUPPORTED_SHAPE, "attn_decode: unsupported head_dim / chunk_size");
    const pkvt::Plan& p = t->plan;
    if (t->up_plan.ptr != d_meta || t->up_plan.serial != p.serial ||
        t->up_plan.len_version != p.len_version)
        return fail(PKVT_ERR_STALE_PLAN, "attn_decode: the current plan is not uploaded to d_meta");
    const int32_t H = t->tree.H, D = t->tree.D, C = t->tree.C;
    const size_t need = static_cast<size_t>(p.n_slots) * H * (D + 2) * sizeof(float);
    if (need > 0 && (!workspace || workspace_bytes < need))
        return fail(PKVT_ERR_BUFFER_TOO_SMALL, "attn_decode: workspace smaller than the plan needs");
    const int32_t* m = static_cast<const int32_t*>(d_meta);
    float* part_o = static_cast<float*>(workspace);
    float* part_ml = part_o ? part_o + static_cast<size_t>(p.n_slots) * H * D : nullptr;
    auto s = static_cast<hipStream_t>(stream);

    pkvt::AttnArgs a{};
    a.lists = m + p.blob[pkvt::kOffLists];
    a.tasks = m + p.blob[pkvt::kOffTasks];
    a.waves = m + p.blob[pkvt::kOffWaves];
    a.wg_units = m + p.blob[pkvt::kOffWgUnits];
    a.units = m + p.blob[pkvt::kOffUnits];
    a.chunks = m + p.blob[pkvt::kOffChunks];
    a.rows = m + p.blob[pkvt::kOffRows];
    a.seqlen = m + p.blob[pkvt::kOffSeqlen];
    a.q = q;
    a.kpool = k_pool;
    a.vpool = v_pool;
    a.out = out;
    a.part_o = part_o;
    a.part_ml = part_ml;
    a.H = H;
    a.n_wg = (p.n_tasks > 0 || p.n_units > 0) ? p.n_wg : 0;
    a.scale_log2e = scale * 1.4426950408889634f;
    hipError_t e;
    if (attn_start_event &&
        (e = hipEventRecord(static_cast<hipEvent_t>(attn_start_event), s)) != hipSuccess)
        return hip_fail(e, "attn_decode: event record");
    e = p.kernel == 1 ? pkvt::launch_units(a, D, C, s) : pkvt::launch_attn(a, D, C, s);
    if (e != hipSuccess) return hip_fail(e, "attn_decode: attention kernel");
    if (attn_end_event && (e = hipEventRecord(static_cast<hipEvent_t>(attn_end_event), s)) != hipSuccess)
        return hip_fail(e, "attn_decode: event record");
    if (p.n_merge > 0) {
        pkvt::MergeArgs mg{};
        mg.merge_rows = m + p.blob[pkvt::kOffMerge];
        mg.mptr = m + p.blob[pkvt::kOffMptr];
        mg.mslots = m + p.blob[pkvt::kOffMslots];
        mg.rows = a.rows;
        mg.part_o = part_o;
        mg.part_ml = part_ml;
        mg.out = out;
        mg.H = H;
        mg.n_merge = p.n_merge;
        e = pkvt::launch_merge(mg, D, s);
        if (e != hipSuccess) return hip_fail(e, "attn_decode: merge kernel");
    }
    return PKVT_OK;
}

pkvt_status pkvt_attn_decode_noalloc(const pkvt_tree* t, const void* d_meta, const void* q,
                                     const void* k_pool, const void* v_pool, void* out,
                                     float scale, void* stream) {
    if (!t) return fail(PKVT_ERR_INVALID_ARG, "attn_decode_noalloc: tree is NULL");
    if (!plan_current(t))
        return fail(PKVT_ERR_STALE_PLAN, "attn_decode_noalloc: plan is older than the tree");
    const size_t need = static_cast<size_t>(t->plan.n_slots) * t->tree.H * (t->tree.D + 2) *
                        sizeof(float);
    if (need > pkvt::kNoAllocScratchBytes)
        return fail(PKVT_ERR_BUFFER_TOO_SMALL,
                    "attn_decode_noalloc: the plan's partials need " + std::to_string(need) +
                        " bytes, more than the library's fixed scratch of " +
                        std::to_string(pkvt::kNoAllocScratchBytes) +
                        " bytes (use pkvt_attn_decode with a workspace)");
    void* ws = nullptr;
    if (need > 0) {
        const hipError_t e = pkvt::noalloc_scratch(&ws);
        if (e != hipSuccess) return hip_fail(e, "attn_decode_noalloc: scratch address");
    }
    return pkvt_attn_decode_ex(t, d_meta, q, k_pool, v_pool, out, ws, need, scale, stream,
                               nullptr, nullptr);
}

pkvt_status pkvt_kv_scatter(const pkvt_tree* t, void* k_pool, void* v_pool, const int64_t* slots,
                            const void* k_new, const void* v_new, int64_t n_tokens, void* stream) {
    if (!t || n_tokens < 0) return fail(PKVT_ERR_INVALID_ARG, "kv_scatter: bad arguments");
    if (!shape_ok(t->tree.D, t->tree.C))
        return fail(PKVT_ERR_UNSUPPORTED_SHAPE, "kv_scatter: unsupported head_dim / chunk_size");
    if (n_tokens == 0) return PKVT_OK;
    if (!k_pool || !v_pool || !slots || !k_new || !v_new)
        return fail(PKVT_ERR_INVALID_ARG, "kv_scatter: NULL argument");
    pkvt::ScatterArgs a{};
    a.kpool = k_pool;
    a.vpool = v_pool;
    a.slots = slots;
    a.knew = k_new;
    a.vnew = v_new;
    a.n_tokens = n_tokens;
    a.slot_limit = static_cast<int64_t>(t->tree.N) * t->tree.C;
    a.H = t->tree.H;
    hipError_t e = pkvt::launch_scatter(a, t->tree.D, t->tree.C, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "kv_scatter");
    return PKVT_OK;
}

pkvt_status pkvt_kv_move(const pkvt_tree* t, void* k_pool, void* v_pool, const int64_t* src,
                         const int64_t* dst, int64_t n, void* stream) {
    if (!t || n < 0) return fail(PKVT_ERR_INVALID_ARG, "kv_move: bad arguments");
    if (!shape_ok(t->tree.D, t->tree.C))
        return fail(PKVT_ERR_UNSUPPORTED_SHAPE, "kv_move: unsupported head_dim / chunk_size");
    if (n == 0) return PKVT_OK;
    if (!k_pool || !v_pool || !src || !dst) return fail(PKVT_ERR_INVALID_ARG, "kv_move: NULL argument");
    pkvt::MoveArgs a{};
    a.kpool = k_pool;
    a.vpool = v_pool;
    a.src = src;
    a.dst = dst;
    a.n = n;
    a.slot_limit = static_cast<int64_t>(t->tree.N) * t->tree.C;
    a.H = t->tree.H;
    hipError_t e = pkvt::launch_move(a, t->tree.D, t->tree.C, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "kv_move");
    return PKVT_OK;
}

pkvt_status pkvt_prefill_plan(pkvt_tree* t, int32_t n, const int32_t* seq_ids, const int64_t* q_from,
                              const pkvt_plan_opts* opts, size_t* meta_bytes, size_t* workspace_bytes) {
    if (!t) return fail(PKVT_ERR_INVALID_ARG, "prefill_plan: tree is NULL");
    pkvt::PlanOpts o;
    if (opts) {
        o.phase1_chunks = opts->phase1_chunks;
        o.workgroups = opts->workgroups;
    }
    if (o.workgroups < 0) return fail(PKVT_ERR_INVALID_ARG, "prefill_plan: workgroups must be >= 0");
    if (o.workgroups == 0) o.workgroups = default_workgroups();
    std::string err;
    int rc = 0;
    PKVT_GUARD(rc = pkvt::make_prefill_plan(t->tree, n, seq_ids, q_from, o, t->prefill, err));
    if (rc) return fail(rc, err);
    if (meta_bytes) *meta_bytes = t->prefill.blob.size() * sizeof(int32_t);
    if (workspace_bytes)
        *workspace_bytes = static_cast<size_t>(t->prefill.n_slots) * t->tree.H * (t->tree.D + 2) *
                           sizeof(float);
    return PKVT_OK;
}

pkvt_status pkvt_prefill_info_get(const pkvt_tree* t, pkvt_plan_info* out) {
    if (!t || !out) return fail(PKVT_ERR_INVALID_ARG, "prefill_info: NULL argument");
    if (!t->prefill.valid) return fail(PKVT_ERR_STALE_PLAN, "prefill_info: no prefill plan");
    fill_info(t->prefill, out);
    return PKVT_OK;
}

pkvt_status pkvt_prefill_blob(const pkvt_tree* t, int32_t* out, int32_t cap, int32_t* n) {
    if (!t || !n || (cap > 0 && !out)) return fail(PKVT_ERR_INVALID_ARG, "prefill_blob: NULL argument");
    if (!t->prefill.valid) return fail(PKVT_ERR_STALE_PLAN, "prefill_blob: no prefill plan");
    *n = static_cast<int32_t>(t->prefill.blob.size());
    if (cap < *n) return fail(PKVT_ERR_BUFFER_TOO_SMALL, "prefill_blob: cap smaller than the plan");
    std::memcpy(out, t->prefill.blob.data(), t->prefill.blob.size() * sizeof(int32_t));
    return PKVT_OK;
}

pkvt_status pkvt_prefill_upload(pkvt_tree* t, void* d_meta, size_t meta_bytes, void* stream) {
    if (!t || !d_meta) return fail(PKVT_ERR_INVALID_ARG, "prefill_upload: NULL argument");
    if (!current(t, t->prefill))
        return fail(PKVT_ERR_STALE_PLAN, "prefill_upload: no prefill plan for the current tree");
    if (!shape_ok(t->tree.D, t->tree.C))
        return fail(PKVT_ERR_UNSUPPORTED_SHAPE, "prefill_upload: unsupported head_dim / chunk_size");
    return upload(t, t->prefill, t->up_prefill, t->up_plan, d_meta, meta_bytes, stream, false,
                  "prefill_upload");
}

pkvt_status pkvt_prefill_attn(const pkvt_tree* t, const void* d_meta, const void* q,
                              const void* k_pool, const void* v_pool, void* out, void* workspace,
                              size_t workspace_bytes, float scale, void* stream) {
    if (!t || !d_meta || !q || !k_pool || !v_pool || !out)
        return fail(PKVT_ERR_INVALID_ARG, "prefill_attn: NULL argument");
    if (!std::isfinite(scale)) return fail(PKVT_ERR_INVALID_ARG, "prefill_attn: scale is not finite");
    const pkvt::Plan& p = t->prefill;
    if (!current(t, p)) return fail(PKVT_ERR_STALE_PLAN, "prefill_attn: prefill plan is older than the tree");
    if (!shape_ok(t->tree.D, t->tree.C))
        return fail(PKVT_ERR_UNSUPPORTED_SHAPE, "prefill_attn: unsupported head_dim / chunk_size");
    if (t->up_prefill.ptr != d_meta || t->up_prefill.serial != p.serial)
        return fail(PKVT_ERR_STALE_PLAN, "prefill_attn: the prefill plan is not uploaded to d_meta");
    const int32_t H = t->tree.H, D = t->tree.D, C = t->tree.C;
    const size_t need = static_cast<size_t>(p.n_slots) * H * (D + 2) * sizeof(float);
    if (need > 0 && (!workspace || workspace_bytes < need))
        return fail(PKVT_ERR_BUFFER_TOO_SMALL, "prefill_attn: workspace smaller than the plan needs");
    const int32_t* m = static_cast<const int32_t*>(d_meta);
    float* part_o = need > 0 ? static_cast<float*>(workspace) : nullptr;
    float* part_ml = part_o ? part_o + static_cast<size_t>(p.n_slots) * H * D : nullptr;
    auto s = static_cast<hipStream_t>(stream);
    pkvt::AttnArgs a{};
    a.lists = m + p.blob[pkvt::kOffLists];
    a.tasks = m + p.blob[pkvt::kOffTasks];
    a.waves = m + p.blob[pkvt::kOffWaves];
    a.wg_units = m + p.blob[pkvt::kOffWgUnits];
    a.units = m + p.blob[pkvt::kOffUnits];
    a.chunks = m + p.blob[pkvt::kOffChunks];
    a.rows = m + p.blob[pkvt::kOffRows];
    a.seqlen = m + p.blob[pkvt::kOffSeqlen];
    a.qpos = m + p.blob[pkvt::kOffQpos];
    a.q = q;
    a.kpool = k_pool;
    a.vpool = v_pool;
    a.out = out;
    a.part_o = part_o;
    a.part_ml = part_ml;
    a.H = H;
    a.n_wg = p.n_units > 0 ? p.n_wg : 0;
    a.scale_log2e = scale * 1.4426950408889634f;
    hipError_t e = pkvt::launch_prefill(a, D, C, s);
    if (e != hipSuccess) return hip_fail(e, "prefill_attn: attention kernel");
    if (p.n_merge == 0) return PKVT_OK;
    pkvt::MergeArgs mg{};
    mg.merge_rows = m + p.blob[pkvt::kOffMerge];
    mg.mptr = m + p.blob[pkvt::kOffMptr];
    mg.mslots = m + p.blob[pkvt::kOffMslots];
    mg.rows = a.rows;
    mg.part_o = part_o;
    mg.part_ml = part_ml;
    mg.out = out;
    mg.H = H;
    mg.n_merge = p.n_merge;
    e = pkvt::launch_merge(mg, D, s);
    if (e != hipSuccess) return hip_fail(e, "prefill_attn: merge kernel");
    return PKVT_OK;
}

pkvt_status pkvt_kv_scatter_host_slots(const pkvt_tree* t, void* k_pool, void* v_pool,
                                       const int64_t* slots, const void* k_new, const void* v_new,
                                       int64_t n_tokens, void* stream) {
    if (!t || n_tokens < 0 || n_tokens > PKVT_INLINE_SLOTS)
        return fail(PKVT_ERR_INVALID_ARG, "kv_scatter_host_slots: need 0 <= n_tokens <= " +
                                              std::to_string(PKVT_INLINE_SLOTS));
    if (!shape_ok(t->tree.D, t->tree.C))
        return fail(PKVT_ERR_UNSUPPORTED_SHAPE,
                    "kv_scatter_host_slots: unsupported head_dim / chunk_size");
    if (n_tokens == 0) return PKVT_OK;
    if (!k_pool || !v_pool || !slots || !k_new || !v_new)
        return fail(PKVT_ERR_INVALID_ARG, "kv_scatter_host_slots: NULL argument");
    static_assert(PKVT_INLINE_SLOTS == pkvt::kInlineSlots, "inline slot capacity");
    pkvt::ScatterArgs a{};
    a.kpool = k_pool;
    a.vpool = v_pool;
    a.slots = nullptr;
    a.knew = k_new;
    a.vnew = v_new;
    a.n_tokens = n_tokens;
    a.slot_limit = static_cast<int64_t>(t->tree.N) * t->tree.C;
    a.H = t->tree.H;
    pkvt::InlineSlots is;
    std::memcpy(is.slot, slots, static_cast<size_t>(n_tokens) * sizeof(int64_t));
    hipError_t e = pkvt::launch_scatter_inline(a, is, t->tree.D, t->tree.C,
                                               static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "kv_scatter_host_slots");
    return PKVT_OK;
}

}  // extern "C"
