// Launch interface between the C ABI (capi.cpp) and the HIP kernels
// (attn.hip).  Plain pointers only; fp16 tensors are passed as void*.
#pragma once

#include <hip/hip_runtime_api.h>

#include <cstddef>
#include <cstdint>

#include "shapes.h"

namespace pkvt {

struct AttnArgs {
    const int32_t* lists;     // [4*n_wg][2] per wave lane: first task, task count
    const int32_t* tasks;     // [n_tasks][2] (wave descriptor, head)
    const int32_t* waves;     // [n_waves][8] WaveDesc
    const int32_t* wg_units;  // [n_wg][2] per workgroup: first unit, unit count
    const int32_t* units;     // [n_units][16] UnitDesc
    const int32_t* chunks;    // chunk ids
    const int32_t* rows;      // [b] depth-first position -> query row
    const int32_t* seqlen;    // [b] tokens per depth-first position
    const void* q;            // fp16 [b][H][D]
    const void* kpool;        // fp16 [N][H][D/8][C][8]
    const void* vpool;        // fp16 [N][H] slices of C x D in the V order of VLay
    void* out;                // fp16 [b][H][D]
    float* part_o;            // [n_slots][H][D]
    float* part_ml;           // [n_slots][H][2]  (m in log2 units, n)
    int32_t H;
    int32_t n_wg;             // persistent workgroups (grid size)
    float scale_log2e;        // score scale * log2(e)
    const int32_t* qpos;      // prefill: [R] sequence position of every depth-first row
};

struct MergeArgs {
    const int32_t* merge_rows;  // [n_merge] depth-first positions
    const int32_t* mptr;        // [b+1]
    const int32_t* mslots;      // partial slots
    const int32_t* rows;        // [b] depth-first position -> query row
    const float* part_o;
    const float* part_ml;
    void* out;
    int32_t H;
    int32_t n_merge;
};

struct ScatterArgs {
    void* kpool;
    void* vpool;
    const int64_t* slots;
    const void* knew;         // fp16 [n][H][D]
    const void* vnew;
    int64_t n_tokens;
    int64_t slot_limit;       // pool_chunks * C
    int32_t H;
};

// Token K/V moves inside the pools: token at slot src[i] -> slot dst[i].
struct MoveArgs {
    void* kpool;
    void* vpool;
    const int64_t* src;
    const int64_t* dst;
    int64_t n;
    int64_t slot_limit;       // pool_chunks * C
    int32_t H;
};

constexpr int kInlineSlots = 256;
struct InlineSlots {
    int64_t slot[kInlineSlots];
};

// Bytes of the library's fixed device scratch (pkvt_attn_decode_noalloc).
constexpr size_t kNoAllocScratchBytes = size_t(64) << 20;
constexpr int kMaxDevices = 64;
// Device address of the current device's scratch (looked up once per device).
hipError_t noalloc_scratch(void** ptr);

hipError_t launch_attn(const AttnArgs& a, int D, int C, hipStream_t s);
// units-only decode plans (head_dim >= 128): 8-wave workgroups, one per CU
hipError_t launch_units(const AttnArgs& a, int D, int C, hipStream_t s);
// units only, each row masked to the keys at positions <= a.qpos[row]
hipError_t launch_prefill(const AttnArgs& a, int D, int C, hipStream_t s);
// slots come from is.slot instead of a.slots (a.n_tokens <= kInlineSlots)
hipError_t launch_scatter_inline(const ScatterArgs& a, const InlineSlots& is, int D, int C,
                                 hipStream_t s);
// dst[i] = src[i] for i < n; src may be a device-mapped host pointer
hipError_t launch_copy_words(const int32_t* src, int32_t* dst, int64_t n, hipStream_t s);
hipError_t launch_merge(const MergeArgs& a, int D, hipStream_t s);
hipError_t launch_scatter(const ScatterArgs& a, int D, int C, hipStream_t s);
// moves with a source or destination outside [0, slot_limit) are skipped;
// sources and destinations must be disjoint slot sets
hipError_t launch_move(const MoveArgs& a, int D, int C, hipStream_t s);

}  // namespace pkvt
