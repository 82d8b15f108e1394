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
// rows becomes ceil(R/16) wave tasks placed in one workgroup, so the waves
// that read the same shared chunks share the CU's caches; a phase-2 item is
// one wave task with one query row.  Each wave streams its chunks 64 keys at
// a time through the matrix cores:
//
//   S^T (keys x rows)  = K  . Q^T    v_mfma_f32_16x16x32_f16, K as the A operand
//   O^T (dims x rows) += V^T . P^T   v_mfma_f32_16x16x32_f16, V^T as the A operand
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

template <int D, int C>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 8))) void attn_kernel(AttnArgs a) {
    static_assert(D % 32 == 0 && C % 16 == 0, "tile shape");
    constexpr int KS = D / 32;     // 32-dim k-steps of Q K^T
    constexpr int DT = D / 16;     // 16-dim output tiles of P V
    const int H = a.H;
    const int g = blockIdx.x / H;
    const int head = blockIdx.x - g * H;
    const int wave = wave_uniform(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int col = lane & 15;     // MFMA row/column index held by this lane
    const int grp = lane >> 4;     // which 8-element k slice of the fragment

    const int task = a.wg[g * kWaves + wave];
    if (task < 0) return;
    const int32_t* wd = a.waves + task * 8;
    const int n_chunks = wd[1];
    const int key_base = wd[2];
    const int len_row = wd[3];
    const int row_lo = wd[4];
    const int n_rows = wd[5];
    const int out_slot = wd[6];
    const int32_t* chunks = a.chunks + wd[0];
    int n_valid = n_chunks * C;
    if (len_row >= 0) n_valid = min(n_valid, a.seqlen[len_row] - key_base);
    const int n_steps = (n_valid + kStep - 1) / kStep;

    const _Float16* __restrict__ kpool = static_cast<const _Float16*>(a.kpool);
    const _Float16* __restrict__ vpool = static_cast<const _Float16*>(a.vpool);
    const size_t slice = static_cast<size_t>(C) * D;          // halves per (chunk, head)

    // Q^T as the B operand: lane (grp, col) holds row col, dims 32*ks + 8*grp .. +7.
    const bool row_ok = col < n_rows;
    const int qrow = row_ok ? a.rows[row_lo + col] : 0;
    h8 qb[KS];
    {
        const _Float16* qp = static_cast<const _Float16*>(a.q) +
                             (static_cast<size_t>(qrow) * H + head) * D + 8 * grp;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            qb[ks] = row_ok ? *reinterpret_cast<const h8*>(qp + 32 * ks) : h8{};
    }

    // K fragments of one step: tile t holds keys 16t .. 16t+15 of the step.
    h8 kr[4][KS];
    // V fragments: [dim tile][key half-step][4-key piece]
    h4 vr[DT][2][2];

    auto load_k = [&](int step) {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int key = step * kStep + 16 * t;
            if (key < n_valid) {
                const int chunk = chunks[key / C];
                const _Float16* base = kpool + (static_cast<size_t>(chunk) * H + head) * slice +
                                       static_cast<size_t>(key % C + col) * 8;
#pragma unroll
                for (int ks = 0; ks < KS; ++ks)
                    kr[t][ks] = *reinterpret_cast<const h8*>(
                        base + static_cast<size_t>(4 * ks + grp) * C * 8);
            } else {
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) kr[t][ks] = h8{};
            }
        }
    };
    auto load_v = [&](int step) {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int key = step * kStep + 16 * t;
            if (key < n_valid) {
                const int chunk = chunks[key / C];
                const _Float16* base = vpool + (static_cast<size_t>(chunk) * H + head) * slice +
                                       static_cast<size_t>(((key % C) / 4 + grp) * D + col) * 4;
#pragma unroll
                for (int dt = 0; dt < DT; ++dt)
                    vr[dt][t >> 1][t & 1] = *reinterpret_cast<const h4*>(base + 64 * dt);
            } else {
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) vr[dt][t >> 1][t & 1] = h4{};
            }
        }
    };

    f4 o[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[dt] = f4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY;
    float l_run = 0.f;

    load_k(0);
    load_v(0);
    for (int step = 0; step < n_steps; ++step) {
        // ---- S^T = K Q^T for the 64 keys of this step --------------------------
        f4 s[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            s[t] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                s[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kr[t][ks], qb[ks], s[t], 0, 0, 0);
        }
        if (step + 1 < n_steps) load_k(step + 1);

        // ---- online softmax (partial_attn per step, attn_reduce into the run) ----
        const int key0 = step * kStep;
        const bool tail = key0 + kStep > n_valid;
        float mx = -INFINITY;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float x = s[t][i] * a.scale_log2e;
                if (tail && key0 + 16 * t + 4 * grp + i >= n_valid) x = -INFINITY;
                s[t][i] = x;
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
            // keys past the end hold stale pool contents: zero them so that
            // 0 * garbage cannot produce a NaN inside the MFMA
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (key0 + 16 * t + 4 * grp + i >= n_valid)
#pragma unroll
                        for (int dt = 0; dt < DT; ++dt) vr[dt][t >> 1][t & 1][i] = 0;
        }

        // ---- O^T += V^T P^T ------------------------------------------------------
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
            for (int hs = 0; hs < 2; ++hs) {
                const h8 va = __builtin_shufflevector(vr[dt][hs][0], vr[dt][hs][1],
                                                      0, 1, 2, 3, 4, 5, 6, 7);
                o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va, pb[hs], o[dt], 0, 0, 0);
            }
        }
        if (step + 1 < n_steps) load_v(step + 1);
    }

    // n of row col = sum over the four lane groups
    float l_tot = l_run + __shfl_xor(l_run, 16);
    l_tot += __shfl_xor(l_tot, 32);
    if (!row_ok) return;
    if (out_slot < 0) {
        const float inv = 1.0f / l_tot;
        _Float16* op = static_cast<_Float16*>(a.out) +
                       (static_cast<size_t>(qrow) * H + head) * D + 4 * grp;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            h4 v;
#pragma unroll
            for (int i = 0; i < 4; ++i) v[i] = static_cast<_Float16>(o[dt][i] * inv);
            *reinterpret_cast<h4*>(op + 16 * dt) = v;
        }
    } else {
        const size_t slot = static_cast<size_t>(out_slot + col);
        float* po = a.part_o + (slot * H + head) * D + 4 * grp;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) *reinterpret_cast<f4*>(po + 16 * dt) = o[dt];
        if (grp == 0) {
            float* pm = a.part_ml + (slot * H + head) * 2;
            pm[0] = m_run;
            pm[1] = l_tot;
        }
    }
}

// Fold every partial of one (sequence, head) with attn_reduce and divide.
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
    const int s0 = a.mptr[p], s1 = a.mptr[p + 1];
    float M = -INFINITY;
    for (int s = s0; s < s1; ++s)
        M = fmaxf(M, a.part_ml[(static_cast<size_t>(a.mslots[s]) * a.H + head) * 2]);
    float acc[J];
#pragma unroll
    for (int j = 0; j < J; ++j) acc[j] = 0.f;
    float L = 0.f;
    for (int s = s0; s < s1; ++s) {
        const size_t base = static_cast<size_t>(a.mslots[s]) * a.H + head;
        const float w = fast_exp2(a.part_ml[base * 2] - M);
        L += w * a.part_ml[base * 2 + 1];
#pragma unroll
        for (int j = 0; j < J; ++j) acc[j] += w * a.part_o[base * D + lane + 64 * j];
    }
    const float inv = 1.0f / L;
    _Float16* op = static_cast<_Float16*>(a.out) +
                   (static_cast<size_t>(a.rows[p]) * a.H + head) * D;
#pragma unroll
    for (int j = 0; j < J; ++j) op[lane + 64 * j] = static_cast<_Float16>(acc[j] * inv);
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
    const unsigned grid = static_cast<unsigned>(a.n_wg) * static_cast<unsigned>(a.H);
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
