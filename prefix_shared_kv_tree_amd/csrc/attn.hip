// HIP kernels for decode attention over a prefix-shared KV tree, gfx950.
//
// Method: "ChunkAttention: Efficient Self-Attention with Prefix-Aware KV Cache
// and Two-Phase Partition" (chapterpal digest).  Knowl 2 gives the two-phase
// partition: phase 1 batches the queries of all sequences covering a shared
// chunk against that chunk; phase 2 walks each sequence's own chunks and
// folds every partial together.  Knowl 3 gives partial_attn (W = Q K^T,
// m = row max, E = exp(W - m), n = row sum, O = E V unnormalised) and
// attn_reduce (rescale both sides to the larger max and add), and the final
// O = o / n.  The score scale 1/sqrt(d) is the attention definition's
// (CachedAttention digest, "Load-bearing equations").
//
// One kernel serves both phases.  Its unit of work is a wave task: up to 16
// query rows of one head against a list of chunks.  A phase-1 item with R
// rows gives ceil(R/16) tasks per head that the planner places on the waves
// of one workgroup, so the waves reading the same shared chunks share the
// CU's caches; a phase-2 item gives one single-row task per head.  The grid
// is a fixed set of persistent workgroups; every wave walks its own task
// list (filled longest-first by the planner) and streams the tasks' chunks
// 64 keys at a time through the matrix cores:
//
//   S^T (keys x rows)  = K  . Q^T    v_mfma_f32_16x16x32_f16, K as the A operand
//   O^T (dims x rows) += V^T . P^T   v_mfma_f32_16x16x32_f16, V^T as the A operand
//
// The loads of the next step -- or of the next task's first step, with its
// queries -- are issued as soon as the registers they land in are free, so
// a wave keeps about one step (32 KiB of K and V) in flight across task
// boundaries too.  K and V are read once, with non-temporal loads.
//
// With one query row (phase 2) 15 of the 16 MFMA columns idle; that costs
// nothing measurable, because a decode step does ~1 FLOP per byte while the
// matrix cores sustain ~300, and it keeps both phases on one code path with
// the same streaming loads.  The pool layouts are chosen so that the A-operand
// fragments are whole 16-byte (K) and 8-byte (V) pieces and 16 consecutive
// lanes read 256 (K) or 128 (V) consecutive bytes:
//   K slice [d/8][c][8]: the 8 dims a lane needs for one key are contiguous,
//                        and consecutive keys are 16 bytes apart;
//   V slice [c/4][d][4]: 4 consecutive keys of one dim are contiguous, and
//                        consecutive dims are 8 bytes apart.
// The online softmax (max, exp2, rescale) runs in fp32 on the S^T fragments;
// P is rounded to fp16 for the PV product and n sums those rounded weights.
// Scores are scaled by scale*log2(e) in fp32 so exp2 gives exp.
#include <hip/hip_runtime.h>

#include <cmath>

#include "kernels.h"

namespace pkvt {
namespace {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef float f4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;          // waves per workgroup
constexpr int kStep = 64;          // keys per step of the streaming loop

__device__ __forceinline__ int wave_uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Wave-uniform description of one task.
struct Task {
    const int32_t* chunks;   // the task's chunk ids
    int n_valid;             // keys to attend over
    int n_steps;             // ceil(n_valid / 64)
    int row_lo;              // depth-first position of query row 0
    int n_rows;
    int out;                 // partial slot of row 0, or -1: write O
    int head;
};

// The plan metadata is read-only for the whole launch.  Reading it through
// the constant address space lets the compiler use scalar loads: task fields
// and chunk ids then live in SGPRs, and fetching the next chunk id never
// waits on the vector loads in flight (a vector load would, since vmcnt
// retires in order).
typedef const __attribute__((address_space(4))) int32_t cint;
__device__ __forceinline__ cint* meta(const int32_t* p) { return (cint*)(p); }

template <int C>
__device__ __forceinline__ Task fetch_task(const AttnArgs& a, int idx) {
    cint* tk = meta(a.tasks) + 2 * idx;
    const int wave_id = tk[0];
    Task t;
    t.head = tk[1];
    cint* wd = meta(a.waves) + 8 * wave_id;
    const int n_chunks = wd[1];
    const int key_base = wd[2];
    const int len_row = wd[3];
    t.chunks = a.chunks + wd[0];
    t.row_lo = wd[4];
    t.n_rows = wd[5];
    t.out = wd[6];
    int n_valid = n_chunks * C;
    if (len_row >= 0) n_valid = min(n_valid, meta(a.seqlen)[len_row] - key_base);
    t.n_valid = n_valid;
    t.n_steps = (n_valid + kStep - 1) / kStep;
    return t;
}

template <int D, int C>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 8)))
void attn_kernel(AttnArgs a) {
    static_assert(D % 32 == 0 && C % 16 == 0, "tile shape");
    constexpr int KS = D / 32;     // 32-dim k-steps of Q K^T
    constexpr int DT = D / 16;     // 16-dim output tiles of P V
    const int H = a.H;
    const int wave = wave_uniform(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int col = lane & 15;     // MFMA row/column index held by this lane
    const int grp = lane >> 4;     // which 8-element k slice of the fragment
    const int lane_id = blockIdx.x * kWaves + wave;
    const int first = meta(a.lists)[2 * lane_id];
    const int count = meta(a.lists)[2 * lane_id + 1];
    if (count == 0) return;

    const _Float16* __restrict__ kpool = static_cast<const _Float16*>(a.kpool);
    const _Float16* __restrict__ vpool = static_cast<const _Float16*>(a.vpool);
    const size_t slice = static_cast<size_t>(C) * D;          // halves per (chunk, head)

    h8 qb[KS];        // Q^T (B operand): row col, dims 32*ks + 8*grp .. +7
    h8 kr[4][KS];     // K of one step: tile t = keys 16t .. 16t+15
    h4 vr[DT][2][2];  // V of one step: [dim tile][key half][4-key piece]

    auto query_row = [&](const Task& t) { return col < t.n_rows ? a.rows[t.row_lo + col] : -1; };
    auto load_q = [&](const Task& t, int qrow) {
        const _Float16* qp = static_cast<const _Float16*>(a.q) +
                             (static_cast<size_t>(qrow < 0 ? 0 : qrow) * H + t.head) * D + 8 * grp;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            qb[ks] = qrow >= 0 ? *reinterpret_cast<const h8*>(qp + 32 * ks) : h8{};
    };
    // Byte offsets: a uniform part (chunk slice, key tile, k-step / dim tile)
    // plus one per-lane constant, so every load is SGPR base + VGPR offset.
    const uint32_t k_lane = static_cast<uint32_t>(col + grp * C) * 16u;   // key col, dims 8*grp..
    const uint32_t v_lane = static_cast<uint32_t>(grp * D + col) * 8u;    // keys 4*grp.., dim col
    auto slice_of = [&](const _Float16* pool, int chunk, int head) {
        return reinterpret_cast<const char*>(pool + (static_cast<size_t>(chunk) * H + head) * slice);
    };
    // Loads are unconditional so the compiler can count them exactly and wait
    // for just the step it needs (a branch around a load makes it wait for
    // everything).  A tile past the end of the keys re-reads the last tile
    // that has valid keys -- same addresses, so no extra HBM traffic -- and
    // its scores are forced to -inf and its V entries zeroed below.
    auto tile_key = [&](const Task& t, int step, int tt) {
        const int key = step * kStep + 16 * tt;
        const int last = (t.n_valid - 1) & ~15;
        return key < last ? key : last;
    };
    auto load_k = [&](const Task& t, int step) {
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
            const int key = tile_key(t, step, tt);
            const char* base = slice_of(kpool, meta(t.chunks)[key / C], t.head) + (key % C) * 16;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                kr[tt][ks] = __builtin_nontemporal_load(
                    reinterpret_cast<const h8*>(base + ks * (C * 64) + k_lane));
        }
    };
    auto load_v = [&](const Task& t, int step) {
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
            const int key = tile_key(t, step, tt);
            const char* base = slice_of(vpool, meta(t.chunks)[key / C], t.head) +
                               ((key % C) / 4) * (D * 8);
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
                vr[dt][tt >> 1][tt & 1] =
                    __builtin_nontemporal_load(reinterpret_cast<const h4*>(base + dt * 128 + v_lane));
        }
    };

    Task cur = fetch_task<C>(a, first);
    int cur_qrow = query_row(cur);
    load_q(cur, cur_qrow);
    load_k(cur, 0);
    load_v(cur, 0);
    int ti = 0;
    bool has_next = count > 1;
    Task nxt = cur;
    int nxt_qrow = -1;
    if (has_next) {
        nxt = fetch_task<C>(a, first + 1);
        nxt_qrow = query_row(nxt);
    }

    f4 o[DT];
    float m_run, l_run;
    f4 s[4];

    // S^T = K Q^T for the 64 keys of a step
    auto qk = [&]() {
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
            s[tt] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                s[tt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kr[tt][ks], qb[ks], s[tt], 0, 0, 0);
        }
    };
    // online softmax of the step (partial_attn) folded into the run
    // (attn_reduce), then O^T += V^T P^T
    auto softmax_pv = [&](int step, int n_valid) {
        const int key0 = step * kStep;
        const bool tail = key0 + kStep > n_valid;
        float mx = -INFINITY;
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float x = s[tt][i] * a.scale_log2e;
                if (tail && key0 + 16 * tt + 4 * grp + i >= n_valid) x = -INFINITY;
                s[tt][i] = x;
                mx = fmaxf(mx, x);
            }
        }
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_new = fmaxf(m_run, mx);        // finite: every step has a valid key
        const float alpha = fast_exp2(m_run - m_new);
        m_run = m_new;
        h8 pb[2];
        float lsum = 0.f;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const _Float16 p = static_cast<_Float16>(fast_exp2(s[e >> 2][e & 3] - m_new));
            pb[e >> 3][e & 7] = p;
            lsum += static_cast<float>(p);
        }
        l_run = l_run * alpha + lsum;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) o[dt] *= alpha;
        if (tail) {
            // keys past the end hold stale pool contents (possibly NaN bit
            // patterns): zero their V so that 0 * garbage cannot reach the
            // MFMA.  One 64-bit mask per 4-key piece a lane holds.
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) {
                const int nk = n_valid - (key0 + 16 * tt + 4 * grp);
                const unsigned long long mk =
                    nk >= 4 ? ~0ull : (nk <= 0 ? 0ull : (1ull << (16 * nk)) - 1ull);
#pragma unroll
                for (int dt = 0; dt < DT; ++dt)
                    vr[dt][tt >> 1][tt & 1] = __builtin_bit_cast(
                        h4, __builtin_bit_cast(unsigned long long, vr[dt][tt >> 1][tt & 1]) & mk);
            }
        }
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
            for (int hs = 0; hs < 2; ++hs) {
                const h8 va = __builtin_shufflevector(vr[dt][hs][0], vr[dt][hs][1],
                                                      0, 1, 2, 3, 4, 5, 6, 7);
                o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va, pb[hs], o[dt], 0, 0, 0);
            }
        }
    };

    for (;;) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) o[dt] = f4{0.f, 0.f, 0.f, 0.f};
        m_run = -INFINITY;
        l_run = 0.f;
        // all steps but the last: the next step's K and V follow right behind
        const int n_steps = cur.n_steps;
        for (int step = 0; step + 1 < n_steps; ++step) {
            qk();
            load_k(cur, step + 1);
            softmax_pv(step, cur.n_valid);
            load_v(cur, step + 1);
        }
        // last step: the next task's queries and K/V follow instead
        qk();
        if (has_next) {
            load_q(nxt, nxt_qrow);
            load_k(nxt, 0);
        }
        softmax_pv(n_steps - 1, cur.n_valid);

        // ---- task epilogue: n of row col = sum over the four lane groups --------
        float l_tot = l_run + __shfl_xor(l_run, 16);
        l_tot += __shfl_xor(l_tot, 32);
        if (cur_qrow >= 0) {
            if (cur.out < 0) {
                const float inv = 1.0f / l_tot;
                _Float16* op = static_cast<_Float16*>(a.out) +
                               (static_cast<size_t>(cur_qrow) * H + cur.head) * D + 4 * grp;
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) {
                    h4 v;
#pragma unroll
                    for (int i = 0; i < 4; ++i) v[i] = static_cast<_Float16>(o[dt][i] * inv);
                    *reinterpret_cast<h4*>(op + 16 * dt) = v;
                }
            } else {
                const size_t slot = static_cast<size_t>(cur.out + col);
                float* po = a.part_o + (slot * H + cur.head) * D + 4 * grp;
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) *reinterpret_cast<f4*>(po + 16 * dt) = o[dt];
                if (grp == 0) {
                    float* pm = a.part_ml + (slot * H + cur.head) * 2;
                    pm[0] = m_run;
                    pm[1] = l_tot;
                }
            }
        }
        if (!has_next) break;
        load_v(nxt, 0);
        cur = nxt;
        cur_qrow = nxt_qrow;
        ++ti;
        has_next = ti + 1 < count;
        if (has_next) {
            nxt = fetch_task<C>(a, first + ti + 1);
            nxt_qrow = query_row(nxt);
        }
    }
}

// Fold every partial of one (sequence, head) with attn_reduce and divide.
// One wave per (sequence, head): the lanes first read the partials' (m, n)
// in parallel and agree on the common max M; then every partial's o row is
// read with independent loads (each lane owns D/64 dims) and accumulated
// with weight exp2(m - M); finally o / n.
template <int D>
__global__ __launch_bounds__(256) void merge_kernel(MergeArgs a) {
    constexpr int J = D / 64;
    const int wave = wave_uniform(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int idx = blockIdx.x * kWaves + wave;
    if (idx >= a.n_merge * a.H) return;
    const int mr = idx / a.H;
    const int head = idx - mr * a.H;
    const int p = a.merge_rows[mr];
    const int s0 = a.mptr[p];
    const int n = a.mptr[p + 1] - s0;
    float M = -INFINITY;
    for (int base = 0; base < n; base += 64) {
        const int s = base + lane;
        if (s < n) {
            const size_t slot = static_cast<size_t>(a.mslots[s0 + s]);
            M = fmaxf(M, a.part_ml[(slot * a.H + head) * 2]);
        }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
    float acc[J];
#pragma unroll
    for (int j = 0; j < J; ++j) acc[j] = 0.f;
    float L = 0.f;
    for (int base = 0; base < n; base += 64) {
        const int s = base + lane;
        int my_slot = 0;
        float my_w = 0.f;
        if (s < n) {
            my_slot = a.mslots[s0 + s];
            const float* ml = a.part_ml + (static_cast<size_t>(my_slot) * a.H + head) * 2;
            my_w = fast_exp2(ml[0] - M);
            L += my_w * ml[1];
        }
        const int cnt = min(64, n - base);
        int k = 0;
        for (; k + 4 <= cnt; k += 4) {       // four independent row loads in flight
            float v[4][J], w[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const size_t slot = static_cast<size_t>(__shfl(my_slot, k + u));
                w[u] = __shfl(my_w, k + u);
                const float* po = a.part_o + (slot * a.H + head) * D + J * lane;
#pragma unroll
                for (int j = 0; j < J; ++j) v[u][j] = po[j];
            }
#pragma unroll
            for (int u = 0; u < 4; ++u)
#pragma unroll
                for (int j = 0; j < J; ++j) acc[j] += w[u] * v[u][j];
        }
        for (; k < cnt; ++k) {
            const size_t slot = static_cast<size_t>(__shfl(my_slot, k));
            const float w = __shfl(my_w, k);
            const float* po = a.part_o + (slot * a.H + head) * D + J * lane;
#pragma unroll
            for (int j = 0; j < J; ++j) acc[j] += w * po[j];
        }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) L += __shfl_xor(L, off);
    const float inv = 1.0f / L;
    _Float16* op = static_cast<_Float16*>(a.out) +
                   (static_cast<size_t>(a.rows[p]) * a.H + head) * D + J * lane;
#pragma unroll
    for (int j = 0; j < J; ++j) op[j] = static_cast<_Float16>(acc[j] * inv);
}

// Write tokens' K/V (natural [token][head][dim]) into their pool slots.
template <int D, int C>
__global__ __launch_bounds__(256) void scatter_kernel(ScatterArgs a) {
    constexpr int P = D / 8;
    const int64_t gid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (gid >= a.n_tokens * a.H * P) return;
    const int piece = static_cast<int>(gid % P);
    const int64_t th = gid / P;
    const int head = static_cast<int>(th % a.H);
    const int64_t tok = th / a.H;
    const int64_t slot = a.slots[tok];
    if (slot < 0 || slot >= a.slot_limit) return;
    const int64_t chunk = slot / C;
    const int t = static_cast<int>(slot % C);
    const size_t sbase = (static_cast<size_t>(chunk) * a.H + head) * C * D;
    const size_t src = (static_cast<size_t>(tok) * a.H + head) * D + piece * 8;
    const h8 kv = *reinterpret_cast<const h8*>(static_cast<const _Float16*>(a.knew) + src);
    *reinterpret_cast<h8*>(static_cast<_Float16*>(a.kpool) + sbase +
                           (static_cast<size_t>(piece) * C + t) * 8) = kv;
    const h8 vv = *reinterpret_cast<const h8*>(static_cast<const _Float16*>(a.vnew) + src);
    _Float16* vb = static_cast<_Float16*>(a.vpool) + sbase +
                   (static_cast<size_t>(t / 4) * D + piece * 8) * 4 + (t % 4);
#pragma unroll
    for (int e = 0; e < 8; ++e) vb[e * 4] = vv[e];
}

template <int D, int C>
hipError_t attn_dc(const AttnArgs& a, hipStream_t s) {
    const unsigned grid = static_cast<unsigned>(a.n_wg);
    if (grid == 0) return hipSuccess;
    attn_kernel<D, C><<<dim3(grid), dim3(256), 0, s>>>(a);
    return hipGetLastError();
}

template <int D, int C>
hipError_t scatter_dc(const ScatterArgs& a, hipStream_t s) {
    const int64_t threads = a.n_tokens * a.H * (D / 8);
    if (threads == 0) return hipSuccess;
    scatter_kernel<D, C><<<dim3(static_cast<unsigned>((threads + 255) / 256)), dim3(256), 0, s>>>(a);
    return hipGetLastError();
}

}  // namespace

#define PKVT_DISPATCH(FN, D, C, ...)                                  \
    switch (D * 1000 + C) {                                            \
        case 64016: return FN<64, 16>(__VA_ARGS__);                    \
        case 64032: return FN<64, 32>(__VA_ARGS__);                    \
        case 64064: return FN<64, 64>(__VA_ARGS__);                    \
        case 64128: return FN<64, 128>(__VA_ARGS__);                   \
        case 128016: return FN<128, 16>(__VA_ARGS__);                  \
        case 128032: return FN<128, 32>(__VA_ARGS__);                  \
        case 128064: return FN<128, 64>(__VA_ARGS__);                  \
        case 128128: return FN<128, 128>(__VA_ARGS__);                 \
        default: return hipErrorInvalidValue;                          \
    }

hipError_t launch_attn(const AttnArgs& a, int D, int C, hipStream_t s) {
    PKVT_DISPATCH(attn_dc, D, C, a, s)
}

hipError_t launch_scatter(const ScatterArgs& a, int D, int C, hipStream_t s) {
    PKVT_DISPATCH(scatter_dc, D, C, a, s)
}

hipError_t launch_merge(const MergeArgs& a, int D, hipStream_t s) {
    const int64_t waves = static_cast<int64_t>(a.n_merge) * a.H;
    if (waves == 0) return hipSuccess;
    const dim3 grid(static_cast<unsigned>((waves + kWaves - 1) / kWaves));
    if (D == 64)
        merge_kernel<64><<<grid, dim3(256), 0, s>>>(a);
    else if (D == 128)
        merge_kernel<128><<<grid, dim3(256), 0, s>>>(a);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace pkvt
