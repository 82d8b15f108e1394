// HIP kernels for attention over a prefix-shared KV tree, gfx950: decode
// (both phases), prefill of arriving sequences, the partial merge, and the
// K/V scatter / move / metadata-copy helpers.
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
// One kernel serves both phases.  The grid is a fixed set of persistent
// workgroups of 4 waves.  Every step of the streaming loop takes 64 keys of
// one head through the matrix cores (16 keys at head_dim 256):
//
//   S^T (keys x rows)  = K  . Q^T    v_mfma_f32_16x16x32_f16, K as the A operand
//   O^T (dims x rows) += V^T . P^T   v_mfma_f32_16x16x32_f16, V^T as the A operand
//
// so one wave covers up to 16 query rows.  Work comes in two forms:
//
//  * Workgroup units (phase-1 row blocks of 17..64 rows).  The unit's waves
//    split the loads of every step (each loads a quarter of the step's K and
//    V into LDS -- straight from memory into two images used in turn from
//    head_dim 128 on, through registers at head_dim 64), meet at a barrier,
//    and each wave computes 16 of the rows from the LDS copy.  Every stored
//    byte of a shared chunk is thus fetched once per row block, however many
//    rows read it.  Each workgroup runs its units first, all 4 waves in lock
//    step.  Prefill runs wider units of the same kind (run_unit_wide: eight
//    waves, up to two 16-row tiles per wave, a causal limit per row; at
//    head_dim 128 the two waves of each SIMD take turns, one issuing matrix
//    products while the other runs its softmax; at head_dim 256 four 16-key
//    steps and at head_dim 64 two steps share a barrier).
//  * Single-wave tasks (phase-2 items, and phase-1 row blocks of <= 16
//    rows): every wave then walks its own list of tasks, keeping the next
//    step's K/V -- or the next task's queries and first K/V -- in flight
//    while it computes the current step.
//
// The planner fills both lists longest first.  With one query row (phase 2)
// 15 of the 16 MFMA columns idle; that costs nothing measurable, because a
// decode step does ~1 FLOP per byte while the matrix cores sustain ~300, and
// it keeps both phases on the same streaming loop.  The pool layouts are
// chosen so that the A-operand fragments are whole 16-byte pieces and 16
// consecutive lanes read 256 consecutive bytes:
//   K slice [d/8][c][8]: the 8 dims a lane needs for one key are contiguous,
//                        and consecutive keys are 16 bytes apart;
//   V slice, per 32-key block (16 at head_dim 256 or chunk 16):
//                        [d/16][4 groups][16][8]: 8 keys of one dim are
//                        contiguous, consecutive dims 16 bytes apart, and
//                        the keys of a group are those of one lane group of
//                        the P V instruction (VLay below).
// The online softmax (max, exp2, rescale) runs in fp32 on the S^T fragments;
// P is rounded to fp16 for the PV product and n sums those rounded weights.
// Scores are scaled by scale*log2(e) in fp32 (inside the exponent's FMA) so
// exp2 gives exp.  K and V are
// read with non-temporal loads.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <type_traits>
#include <mutex>

#include "kernels.h"

// Fixed device scratch for callers that cannot allocate (the partials of
// pkvt_attn_decode_noalloc): kNoAllocScratchBytes bytes on every device the
// library runs on, held until the process ends.  In host code the name
// `scratch` is only a stand-in for the symbol: its device address comes from
// hipGetSymbolAddress, once per device (pkvt::noalloc_scratch below).
static __device__ __align__(256) unsigned char scratch[pkvt::kNoAllocScratchBytes];

namespace pkvt {
namespace {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef float f4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;          // waves per workgroup

// Keys per step of the streaming loop: 4 tiles of 16 keys up to head_dim
// 128; one tile at head_dim 256, where a step of K and V in registers next
// to the 64 accumulator registers of O^T would not fit otherwise (16 KiB of
// K and V per wave per step).  With one tile the P V product takes the
// 16-key form of the matrix instruction.
template <int D>
struct Step {
    static constexpr int kTiles = D <= 128 ? 4 : 1;
    static constexpr int kKeys = 16 * kTiles;
};

__device__ __forceinline__ int wave_uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

// The SIMD of its compute unit that the calling wave runs on: field SIMD_ID
// (bits 5:4) of the HW_ID hardware register (register 4), read with
// s_getreg_b32 (operand: register id | offset << 6 | (size - 1) << 11).
__device__ __forceinline__ int simd_id() { return __builtin_amdgcn_s_getreg(4 | (4 << 6) | (1 << 11)); }

// A compile-time flag passed to generic lambdas (two instantiations of a
// loop body chosen by a wave-uniform branch).
template <bool B>
struct Flag {
    static constexpr bool value = B;
};

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Lazy running max of the prefill softmax (softmax_step): moved only when a
// row's step max exceeds it by more than this many log2 units.
constexpr int kLazyLog2 = 8;

// Max / sum over the four 16-lane rows of a wave (lanes l, l^16, l^32, l^48),
// left in every lane: two register swaps between rows (gfx950 permlane
// swaps, plain VALU work) instead of two round trips through the LDS
// crossbar.  A swap of x with itself puts x of lane l^32 (then l^16) beside
// x of lane l.
__device__ __forceinline__ float rows_max(float x) {
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float rows_sum(float x) {
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// The plan metadata is read-only for the whole launch.  Reading it through
// the constant address space lets the compiler use scalar loads: task fields
// and chunk ids then live in SGPRs, and fetching the next chunk id never
// waits on the vector loads in flight (a vector load would, since vmcnt
// retires in order).
typedef const __attribute__((address_space(4))) int32_t cint;
__device__ __forceinline__ cint* meta(const int32_t* p) { return (cint*)(p); }

// Start of the 16-key tile tt of a step, clamped to the last tile that holds
// a valid key.  Loads are issued unconditionally so that the compiler can
// count them and wait for exactly the step it needs (a branch around a load
// makes it wait for everything); a tile past the end re-reads the last valid
// tile -- same addresses, so no extra HBM traffic -- and its scores are
// forced to -inf and its V entries zeroed by softmax_pv.
template <int D>
__device__ __forceinline__ int tile_start(int step, int tt, int n_valid) {
    const int key = step * Step<D>::kKeys + 16 * tt;
    const int last = (n_valid - 1) & ~15;
    return key < last ? key : last;
}

// A task's chunk ids are held one per lane in a VGPR (the planner cuts every
// task to at most 64 chunks), loaded once when the task is fetched.  The id
// of the chunk holding a 16-key tile is then a readlane -- no memory access
// and no wait inside the streaming loop.  (A scalar load per step would
// force a wait for every scalar load in flight, as they complete out of
// order.)  The tile's chunk is that of its first key, clamped to the chunk
// of the last valid key, i.e. the chunk of tile_start(step, tt, n_valid).
__device__ __forceinline__ int lane_ids(cint* chunks, int n_chunks, int lane) {
    return lane < n_chunks ? chunks[lane] : 0;
}

template <int D, int C>
__device__ __forceinline__ int tile_id(int ids, int step, int tt, int n_valid) {
    return __builtin_amdgcn_readlane(ids, min((step * Step<D>::kKeys + 16 * tt) / C, (n_valid - 1) / C));
}

// V pool order.  A (chunk, head) slice of V is a run of fragments, 32 keys
// each (paired) or 16, stored one after the other.  Inside a fragment the
// keys are split into 8-key groups (4 or 2), and the fragment is
// [D/16 dim tiles][group][16 dims][8 keys]: a 16-byte piece holds 8 keys of
// one dim, and the pieces that one P V instruction takes for one dim tile
// (every group, 16 dims) are one contiguous run of 1 KiB (512 B unpaired).
// Paired (steps of 4 tiles, chunks of at least 32 keys): group g of a block
// holds keys 4g .. 4g+3 of its first 16-key tile and then keys 4g .. 4g+3
// of its second -- the 8 keys whose weights lane group g holds for the
// 32-key P V instruction -- so that operand is one 16-byte load and needs
// no register shuffles.  Otherwise (head_dim 256, whose steps are one tile;
// chunks of 16, where a block would span two chunks) a fragment is one
// 16-key tile in key order, and P V goes tile by tile through the 16-key
// instruction, whose operand is half a piece.
template <int D, int C>
struct VLay {
    static constexpr int NT = Step<D>::kTiles;
    static constexpr bool kPaired = NT > 1 && C >= 32;
    static constexpr int kFrags = kPaired ? NT / 2 : NT;      // per 16-dim tile and step
    static constexpr int kFragKeys = kPaired ? 32 : 16;
    static constexpr int kGroups = kFragKeys / 8;             // 8-key groups per fragment
    using Frag = std::conditional_t<kPaired, h8, h4>;
    // element offset (halves) of key t, dim x in a slice
    __host__ __device__ static constexpr int elem(int t, int x) {
        const int w = t % kFragKeys;
        const int g = kPaired ? (w & 15) >> 2 : w >> 3;
        const int e = kPaired ? (w >> 4) * 4 + (w & 3) : w & 7;
        return (t - w) * D + (((x >> 4) * kGroups + g) * 16 + (x & 15)) * 8 + e;
    }
    // Where the V of key tile tt of a step is read from, as a key: the V of
    // keys p .. p+15 (p a multiple of 16) is the contiguous 32 D bytes from
    // p * 2 D -- a whole fragment, or the first or second half of a paired
    // one.  Fragments are clamped like tile_start, to the last one that
    // holds a valid key.
    __device__ static int tile_src(int step, int tt, int n_valid) {
        if constexpr (kPaired) {
            const int key = step * Step<D>::kKeys + 32 * (tt >> 1);
            const int last = (n_valid - 1) & ~31;
            return (key < last ? key : last) + 16 * (tt & 1);
        } else {
            return tile_start<D>(step, tt, n_valid);
        }
    }
    // a lane's part of a fragment: its 8-position group within the fragment,
    // and the byte offset inside the 16-byte piece
    __device__ static int lane_group(int grp) { return kPaired ? grp : grp >> 1; }
    __device__ static int lane_byte(int grp) { return kPaired ? 0 : (grp & 1) * 8; }
};

// S^T = K Q^T for the keys of a step: tile tt = keys 16tt .. 16tt+15.
template <int NT, int KS>
__device__ __forceinline__ void qk(f4 (&s)[NT], const h8 (&kr)[NT][KS], const h8 (&qb)[KS]) {
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) {
        s[tt] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            s[tt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kr[tt][ks], qb[ks], s[tt], 0, 0, 0);
    }
}

// Online softmax of one step (partial_attn) folded into the running state
// (attn_reduce): lane (col, grp) holds the scores of query row col for keys
// 16tt + 4grp + i.  Returns P^T in fp16, pq[tt] = keys 16tt + 4grp .. +3 of
// row col (the B-operand layout of the P V product), and rescales o to the
// new running max.
// kSkip (workgroup units, whose steps are bound by the instructions a wave
// issues): the key mask and the rescale of o are skipped, wave-wide, on
// steps where no lane needs them (no lane's keys end inside the step; no
// lane's running max moved).
// With a positive scale (the attention scale always is) the scores stay
// unscaled: their max is scaled once and each weight is exp2 of one fused
// multiply-add, s * scale - m.  Other scales scale the scores first.  The
// running sum adds the fp16 weights that the P V product uses, two at a
// time with a packed dot product against (1, 1).
//
// kLazy > 0 (prefill units): the running max m is moved only when a row's
// step max exceeds it by more than kLazy (log2 units), so the weights of
// the other steps are exp2 of at most kLazy (<= 2^kLazy, exact in fp16's
// range) and o and n keep their scale: (o, m, n) still means
// o = sum 2^(s - m) v, n = sum 2^(s - m) for the m it holds, the form that
// attn_reduce and the final o / n take.  Late in a long context a new
// maximum rarely moves by that much, so the rescale of o mostly drops out.
template <int NT, int DT, bool kSkip = false, int kLazy = 0>
__device__ __forceinline__ void softmax_step(f4 (&s)[NT], h4 (&pq)[NT], f4 (&o)[DT], float& m_run,
                                             float& l_run, int step, int n_valid, int grp,
                                             float scale_log2e) {
    const int key0 = step * 16 * NT;
    const bool tail = key0 + 16 * NT > n_valid;
    const bool raw = scale_log2e > 0.f;          // kernel argument: uniform
    const float sc = raw ? scale_log2e : 1.f;
    if (!raw) {
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) s[tt] *= scale_log2e;
    }
    if (!kSkip || __any(tail)) {
#pragma unroll
        for (int tt = 0; tt < NT; ++tt)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (tail && key0 + 16 * tt + 4 * grp + i >= n_valid) s[tt][i] = -INFINITY;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int tt = 0; tt < NT; ++tt)
#pragma unroll
        for (int i = 0; i < 4; ++i) mx = fmaxf(mx, s[tt][i]);
    mx = rows_max(mx);
    float m_new, alpha;
    bool rescale;
    if constexpr (kLazy > 0) {
        // A row's first step always moves m (-inf before); a step whose keys
        // are all masked for the row (mx = -inf) never does.
        const float m_step = mx * sc;
        const bool grow = m_step > m_run + static_cast<float>(kLazy);
        m_new = grow ? m_step : m_run;
        alpha = grow ? fast_exp2(m_run - m_new) : 1.0f;
        rescale = __any(grow);
    } else {
        m_new = fmaxf(m_run, mx * sc);            // finite: every step has a valid key
        alpha = fast_exp2(m_run - m_new);
        rescale = !kSkip || __any(alpha != 1.0f);
    }
    m_run = m_new;
    float lsum = 0.f;
    const h2 one = {static_cast<_Float16>(1.0f), static_cast<_Float16>(1.0f)};
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            pq[tt][i] = static_cast<_Float16>(fast_exp2(__builtin_fmaf(s[tt][i], sc, -m_new)));
        lsum = __builtin_amdgcn_fdot2(__builtin_shufflevector(pq[tt], pq[tt], 0, 1), one, lsum, false);
        lsum = __builtin_amdgcn_fdot2(__builtin_shufflevector(pq[tt], pq[tt], 2, 3), one, lsum, false);
    }
    l_run = l_run * alpha + lsum;
    if (rescale) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) o[dt] *= alpha;
    }
}

// Keys past the end hold stale pool contents (possibly NaN bit patterns):
// zero the V entries of a 4-key piece that lie past n_valid so that
// 0 * garbage cannot reach the MFMA.  key = first key of the piece.
__device__ __forceinline__ h4 mask_v(h4 v, int key, int n_valid) {
    const int nk = n_valid - key;
    const unsigned long long mk = nk >= 4 ? ~0ull : (nk <= 0 ? 0ull : (1ull << (16 * nk)) - 1ull);
    return __builtin_bit_cast(h4, __builtin_bit_cast(unsigned long long, v) & mk);
}

// A paired V piece: positions 0..3 are keys key_a .. key_a+3, positions 4..7
// are keys key_a+16 .. key_a+19.
__device__ __forceinline__ h8 mask_v(h8 v, int key_a, int n_valid) {
    const h4 lo = mask_v(__builtin_shufflevector(v, v, 0, 1, 2, 3), key_a, n_valid);
    const h4 hi = mask_v(__builtin_shufflevector(v, v, 4, 5, 6, 7), key_a + 16, n_valid);
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Zero the V entries of the lane's part of fragment f of a step (first key
// key0) that lie past n_valid.
template <int D, int C>
__device__ __forceinline__ typename VLay<D, C>::Frag mask_frag(typename VLay<D, C>::Frag v, int key0,
                                                               int f, int grp, int n_valid) {
    if constexpr (VLay<D, C>::kPaired)
        return mask_v(v, key0 + 32 * f + 4 * grp, n_valid);
    else
        return mask_v(v, key0 + 16 * f + 4 * grp, n_valid);
}

// O^T += V^T P^T for one 16-dim tile: v[f] is the lane's part of V fragment
// f for dim 16dt + col, pq[tt] the lane's weights for keys 16tt + 4grp ..
// +3.  Paired fragments go through the 32-key instruction (the weights of a
// block's two tiles side by side, in the order of the V piece), single
// tiles through the 16-key one.
template <int D, int C>
__device__ __forceinline__ f4 pv_frags(f4 o, const typename VLay<D, C>::Frag (&v)[VLay<D, C>::kFrags],
                                       const h4 (&pq)[Step<D>::kTiles]) {
#pragma unroll
    for (int f = 0; f < VLay<D, C>::kFrags; ++f) {
        if constexpr (VLay<D, C>::kPaired) {
            const h8 pb = __builtin_shufflevector(pq[2 * f], pq[2 * f + 1], 0, 1, 2, 3, 4, 5, 6, 7);
            o = __builtin_amdgcn_mfma_f32_16x16x32_f16(v[f], pb, o, 0, 0, 0);
        } else {
            o = __builtin_amdgcn_mfma_f32_16x16x16f16(v[f], pq[f], o, 0, 0, 0);
        }
    }
    return o;
}

// softmax_step, then the PV product with a whole step of V in registers.
template <int D, int C>
using VStep = typename VLay<D, C>::Frag[D / 16][VLay<D, C>::kFrags];   // [dim tile][fragment]

template <int D, int C, int NT = Step<D>::kTiles, int DT = D / 16>
__device__ __forceinline__ void softmax_pv(f4 (&s)[NT], VStep<D, C>& vr, f4 (&o)[DT], float& m_run,
                                           float& l_run, int step, int n_valid, int grp, float scale_log2e) {
    h4 pq[NT];
    softmax_step<NT, DT>(s, pq, o, m_run, l_run, step, n_valid, grp, scale_log2e);
    const int key0 = step * 16 * NT;
    if (key0 + 16 * NT > n_valid) {
#pragma unroll
        for (int f = 0; f < VLay<D, C>::kFrags; ++f)
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
                vr[dt][f] = mask_frag<D, C>(vr[dt][f], key0, f, grp, n_valid);
    }
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[dt] = pv_frags<D, C>(o[dt], vr[dt], pq);
}

// End of a task for query row col (lane group grp holds dims 16dt + 4grp ..):
// either the final O = o / n in fp16 (out < 0) or the partial (o, m, n) of
// slot out + col.  qrow < 0 marks a lane without a row.
template <int D, int DT>
__device__ __forceinline__ void finish(const AttnArgs& a, const f4 (&o)[DT], float m_run,
                                       float l_run, int qrow, int out, int head, int col, int grp) {
    const float l_tot = rows_sum(l_run);
    if (qrow < 0) return;
    const int H = a.H;
    if (out < 0) {
        const float inv = 1.0f / l_tot;
        _Float16* op = static_cast<_Float16*>(a.out) + (static_cast<size_t>(qrow) * H + head) * D + 4 * grp;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            h4 v;
#pragma unroll
            for (int i = 0; i < 4; ++i) v[i] = static_cast<_Float16>(o[dt][i] * inv);
            *reinterpret_cast<h4*>(op + 16 * dt) = v;
        }
    } else {
        const size_t slot = static_cast<size_t>(out + col);
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

// Bytes of a workgroup unit's LDS image of one step: K as [tile][d/8][16 keys][8],
// then the V fragments of the step in pool order.  An operand read of V (one
// dim tile of a fragment, every lane) is a contiguous 1 KiB (512 B), free of
// bank conflicts without padding.
template <int D>
struct Img {
    static constexpr int kBytesK = Step<D>::kKeys * D * 2;
    static constexpr int kBytes = 2 * kBytesK;
    static constexpr int kPiecesK = kBytesK / 16;         // 16-byte pieces of K (2D per tile)
    static constexpr int kPieces = 2 * kPiecesK;          // ... of K and V together
};

// LDS of the two-phase unit kernel: four images, also holding at the end
// one phase's running state (o as f4 per dim tile and lane, then m and n)
// for every wave of a phase.
template <int D>
constexpr int unit_lds_bytes() {
    const int x = kWaves * (D / 16) * 64 * 16 + kWaves * 64 * 8;
    return 4 * Img<D>::kBytes > x ? 4 * Img<D>::kBytes : x;
}

// LDS offset of V piece jv of a step's image.  The pieces of key tile tt
// are 2 D tt .. 2 D tt + 2 D - 1, in the order they sit in memory from the
// tile's source (VLay::tile_src).
template <int D>
__device__ __forceinline__ int v_piece_dst(int jv) {
    return Img<D>::kBytesK + jv * 16;
}
// byte offset, inside a fragment, of the lane's part for dims 16dt + col
template <int D, int C>
__device__ __forceinline__ int v_frag_lane(int dt, int col, int grp) {
    using L = VLay<D, C>;
    return ((dt * L::kGroups + L::lane_group(grp)) * 16 + col) * 16 + L::lane_byte(grp);
}
// LDS offset of the lane's part of V fragment f for dims 16dt + col
template <int D, int C>
__device__ __forceinline__ int v_frag_lds(int f, int dt, int col, int grp) {
    return Img<D>::kBytesK + f * (VLay<D, C>::kFragKeys * D * 2) + v_frag_lane<D, C>(dt, col, grp);
}

// One workgroup unit: query rows [row_lo, row_lo + n_rows) of one head.
// Wave w loads pieces [w, w + 1) * kPieces / 4 of every step's image and
// computes rows 16w .. 16w + 15 (if it has any) from the LDS copy.  The trip
// count comes from the unit descriptor that all 4 waves read, so every wave
// passes the same number of barriers.  Decode only (every row sees all of
// the unit's keys); prefill units are run_unit_wide's.
template <int D, int C>
__device__ __forceinline__ void run_unit(const AttnArgs& a, cint* u, int wave, int lane, char* img) {
    constexpr int KS = D / 32, DT = D / 16, NT = Step<D>::kTiles;
    constexpr int kPer = Img<D>::kPieces / kWaves;   // pieces per wave per step
    constexpr int NL = kPer / 64;                    // 16-byte loads per lane per step
    constexpr int KP = Img<D>::kPiecesK;
    constexpr int TPW = kPer >= 2 * D ? kPer / (2 * D) : 1;   // tiles a wave loads per step
    static_assert(kPer % 64 == 0 && (2 * D) % 64 == 0 && (kPer % (2 * D) == 0 || NT == 1) &&
                  NL % TPW == 0, "piece split");
    const int col = lane & 15;
    const int grp = lane >> 4;
    const int H = a.H;
    const int n_keys = u[0];
    const int ids = lane_ids(meta(a.chunks) + u[1], u[2], lane);
    const int head = u[3];
    const int row_lo = u[4];
    const int n_rows = u[5];
    const int out = u[6];
    const int role = wave;
    const bool computes = 16 * role < n_rows;
    const int n_steps = (n_keys + Step<D>::kKeys - 1) / Step<D>::kKeys;
    const size_t slice = static_cast<size_t>(C) * D * 2;      // bytes per (chunk, head)
    const char* kbase = static_cast<const char*>(a.kpool) + static_cast<size_t>(head) * slice;
    const char* vbase = static_cast<const char*>(a.vpool) + static_cast<size_t>(head) * slice;
    const size_t cstride = static_cast<size_t>(H) * slice;    // bytes per chunk

    h8 stg[NL];
    // piece j of the image: K pieces [0, KP) as (tile, d/8 piece, key), then
    // V pieces [KP, 2 KP) as (group, dim)
    // A wave's pieces cover TPW tiles from ta on (of K for waves 0-1, of V
    // for waves 2-3); load i falls in tile ta + i / (NL / TPW).  With one
    // tile per step every wave loads a part of tile 0.
    const int ta = NT == 1 ? 0 : TPW * (role & 1);
    auto stage = [&](int step) {
        int id[TPW];
#pragma unroll
        for (int k = 0; k < TPW; ++k) id[k] = tile_id<D, C>(ids, step, ta + k, n_keys);
#pragma unroll
        for (int i = 0; i < NL; ++i) {
            const int j0 = role * kPer + i * 64;                   // wave-uniform
            const bool is_k = j0 < KP;
            const int jj = is_k ? j0 : j0 - KP;
            const int ts = tile_start<D>(step, jj / (2 * D), n_keys);
            const int tv = VLay<D, C>::tile_src(step, jj / (2 * D), n_keys);
            const int rem = jj % (2 * D) + lane;
            const size_t cbytes = static_cast<size_t>(id[i / (NL / TPW)]) * cstride;
            const char* kp = kbase + cbytes + (static_cast<size_t>(rem >> 4) * C + ts % C + (rem & 15)) * 16;
            const char* vp = vbase + cbytes + static_cast<size_t>(tv % C) * (D * 2) + rem * 16;
            stg[i] = __builtin_nontemporal_load(reinterpret_cast<const h8*>(is_k ? kp : vp));
        }
    };
    auto commit = [&]() {
#pragma unroll
        for (int i = 0; i < NL; ++i) {
            const int j = role * kPer + i * 64 + lane;
            *reinterpret_cast<h8*>(img + (j < KP ? j * 16 : v_piece_dst<D>(j - KP))) = stg[i];
        }
    };

    h8 qb[KS];
    int qrow = -1;
    if (computes) {
        const int r = 16 * role + col;
        qrow = r < n_rows ? a.rows[row_lo + r] : -1;
        const _Float16* qp = static_cast<const _Float16*>(a.q) +
                             (static_cast<size_t>(qrow < 0 ? 0 : qrow) * H + head) * D + 8 * grp;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            qb[ks] = qrow >= 0 ? *reinterpret_cast<const h8*>(qp + 32 * ks) : h8{};
    }
    f4 o[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[dt] = f4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.f;

    stage(0);
    for (int step = 0; step < n_steps; ++step) {
        __syncthreads();                       // every wave is done reading the last image
        commit();
        __syncthreads();                       // this step's image is complete
        if (step + 1 < n_steps) stage(step + 1);
        if (computes) {
            // fragments are read from LDS tile by tile, next to the MFMAs
            // that use them, to keep register pressure low
            f4 s[NT];
#pragma unroll
            for (int tt = 0; tt < NT; ++tt) {
                s[tt] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    const h8 kf = *reinterpret_cast<const h8*>(
                        img + ((tt * (D / 8) + 4 * ks + grp) * 16 + col) * 16);
                    s[tt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf, qb[ks], s[tt], 0, 0, 0);
                }
            }
            h4 pq[NT];
            softmax_step<NT, DT>(s, pq, o, m_run, l_run, step, n_keys, grp, a.scale_log2e);
            // V entries past the last key are zeroed on the last step only
            auto pv = [&](auto masked) {
                using L = VLay<D, C>;
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) {
                    typename L::Frag v[L::kFrags];
#pragma unroll
                    for (int f = 0; f < L::kFrags; ++f) {
                        v[f] = *reinterpret_cast<const typename L::Frag*>(img + v_frag_lds<D, C>(f, dt, col, grp));
                        if constexpr (decltype(masked)::value)
                            v[f] = mask_frag<D, C>(v[f], step * Step<D>::kKeys, f, grp, n_keys);
                    }
                    o[dt] = pv_frags<D, C>(o[dt], v, pq);
                }
            };
            if ((step + 1) * Step<D>::kKeys > n_keys)
                pv(Flag<true>{});
            else
                pv(Flag<false>{});
        }
    }
    if (computes) finish<D, DT>(a, o, m_run, l_run, qrow, out + 16 * role, head, col, grp);
}

// A wide unit: like run_unit (with the causal mask for prefill), but every one
// of the W waves computes RT tiles of 16 query rows (a unit covers up to
// 16 W RT rows), so each K/V fragment read from LDS feeds RT matrix
// instructions, and the unit may read up to 128 chunks (ids in two registers
// per lane).  Each wave loads 1/W of every step's image.  From
// head_dim 128 on, K/V go from memory straight into LDS (global_load_lds,
// 16 bytes per lane, lanes at consecutive 16-byte LDS addresses) into two
// images used in turn: the loads of step s + 1 fly while step s is computed,
// with one barrier per step and no staging registers.  At head_dim 64 a V
// load spans two padded 4-key groups, so the register path is kept.
//
// P = 2 (decode units of the units-only kernel, head_dim >= 128): the
// workgroup has 2 W waves in two phases of W; phase ph computes the unit's
// steps ph, ph + 2, ph + 4, ... from its own pair of images (img0/img1 for
// phase 0, img2/img3 for phase 1), so two steps are in flight and each SIMD
// holds one wave of each phase, which hides the latency of one wave's step.
// Both phases pass the same barriers (one per pair of steps).  At the end
// phase 1 hands its running state (o, m, n) to phase 0 through LDS, which
// folds it in with attn_reduce before writing the unit's partials.
//
// P = 3 (prefill units at head_dim 128, W = 8): a ping-pong schedule over
// three images.  Each SIMD holds one wave of each kind: a leading wave
// (lead) issues the matrix products of a step -- P V of step i - 1, then
// Q K^T of step i -- while its partner runs the softmax of step i, and the
// other way round in the next half of the step.  Two barriers per step
// separate the halves; the matrix cores of a SIMD then work during the
// partner's exponentials instead of both waves of a SIMD issuing the same
// kind of work at the same time.  The image of step i is read from the
// half before the leading waves' Q K^T of step i to the half of their
// P V of step i, so the loads of step i + 2 go into the third image, one
// step ahead.  The softmax moves the running max lazily (kLazy).
template <int D, int C, int RT, bool kCausal, int W = kWaves, int P = 1>
__device__ __forceinline__ void run_unit_wide(const AttnArgs& a, cint* u, int wave, int lane,
                                              char* img0, char* img1, char* img2 = nullptr,
                                              char* img3 = nullptr, bool lead = true) {
    constexpr int KS = D / 32, DT = D / 16, NT = Step<D>::kTiles;
    constexpr int kPer = Img<D>::kPieces / W;
    constexpr int NL = kPer / 64;
    constexpr int KP = Img<D>::kPiecesK;
    constexpr int TPW = kPer >= 2 * D ? kPer / (2 * D) : 1;
    constexpr bool kDirect = D >= 128;
    static_assert(kPer % 64 == 0 && (2 * D) % 64 == 0 && (kPer % (2 * D) == 0 || NT == 1) &&
                  NL % TPW == 0 && (NT == 1 || (W / 2) * TPW == NT), "piece split");
    static_assert(D % 64 == 0, "a load's 64 pieces must stay inside one V group");
    const int col = lane & 15;
    const int grp = lane >> 4;
    const int H = a.H;
    const int n_keys = u[0];
    cint* chunks = meta(a.chunks) + u[1];
    const int n_chunks = u[2];
    const int ids_lo = lane_ids(chunks, n_chunks, lane);
    const int ids_hi = lane + 64 < n_chunks ? chunks[lane + 64] : 0;
    const int head = u[3];
    const int row_lo = u[4];
    const int n_rows = u[5];
    const int out = u[6];
    const int key_base = kCausal ? u[7] : 0;
    static_assert(P == 1 || (P == 2 && RT == 1 && !kCausal) || (P == 3 && kCausal && D == 128),
                  "two phases: decode units only; ping-pong: prefill at head_dim 128");
    const int role = P == 2 ? wave % W : wave;
    const int phase = P == 2 ? wave / W : 0;
    const bool computes = 16 * RT * role < n_rows;
    const int n_steps = (n_keys + Step<D>::kKeys - 1) / Step<D>::kKeys;
    const size_t slice = static_cast<size_t>(C) * D * 2;
    const char* kbase = static_cast<const char*>(a.kpool) + static_cast<size_t>(head) * slice;
    const char* vbase = static_cast<const char*>(a.vpool) + static_cast<size_t>(head) * slice;
    const size_t cstride = static_cast<size_t>(H) * slice;
    auto chunk_of = [&](int step, int tt) {
        const int k = min((step * Step<D>::kKeys + 16 * tt) / C, (n_keys - 1) / C);
        return k < 64 ? __builtin_amdgcn_readlane(ids_lo, k) : __builtin_amdgcn_readlane(ids_hi, k - 64);
    };
    // the first tile this wave loads: K tiles go to waves 0 .. W/2 - 1, V
    // tiles to the others, TPW consecutive tiles each
    const int ta = NT == 1 ? 0 : TPW * (role % (W / 2));
    // memory address of this lane's piece of load i of a step: a wave-uniform
    // base (pool, chunk, key tile) plus the lane's offset inside the tile,
    // which does not change from step to step and is computed once
    uint32_t loff[NL];
#pragma unroll
    for (int i = 0; i < NL; ++i) {
        const int j0 = role * kPer + i * 64;
        const int rem = (j0 < KP ? j0 : j0 - KP) % (2 * D) + lane;
        loff[i] = j0 < KP ? static_cast<uint32_t>(((rem >> 4) * C + (rem & 15)) * 16)
                          : static_cast<uint32_t>(rem * 16);
    }
    auto src = [&](int step, int i, const int (&id)[TPW]) {
        const int j0 = role * kPer + i * 64;
        const bool is_k = j0 < KP;
        const int jj = is_k ? j0 : j0 - KP;
        const int tk = tile_start<D>(step, jj / (2 * D), n_keys);
        const int tv = VLay<D, C>::tile_src(step, jj / (2 * D), n_keys);
        const size_t cbytes = static_cast<size_t>(id[i / (NL / TPW)]) * cstride;
        const char* base = (is_k ? kbase : vbase) + cbytes +
                           (is_k ? static_cast<size_t>(tk % C) * 16 : static_cast<size_t>(tv % C) * (D * 2));
        return reinterpret_cast<const h8*>(base + loff[i]);
    };
    // LDS byte offset of the piece a lane of load i writes (lane offset excluded
    // when lane_part is false)
    auto dst = [&](int i, bool lane_part) {
        const int j = role * kPer + i * 64 + (lane_part ? lane : 0);
        return j < KP ? j * 16 : v_piece_dst<D>(j - KP);
    };

    h8 stg[kDirect ? 1 : NL];
    // a wave loads either K or V pieces (all of its pieces are of one kind)
    const bool kwave = role * kPer < KP;
    int ldso[NL];                                 // LDS offset of load i (lane 0)
#pragma unroll
    for (int i = 0; i < NL; ++i) ldso[i] = wave_uniform(dst(i, false));
    // loads staged in registers, for a given set of staging registers
    // (head_dim < 128 takes two steps per barrier, one set per step)
    auto stage_regs = [&](int step, h8 (&st)[kDirect ? 1 : NL]) {
        if constexpr (!kDirect) {
            int id[TPW];
#pragma unroll
            for (int k = 0; k < TPW; ++k) id[k] = chunk_of(step, ta + k);
#pragma unroll
            for (int i = 0; i < NL; ++i) st[i] = __builtin_nontemporal_load(src(step, i, id));
        }
    };
    auto commit_regs = [&](char* img, const h8 (&st)[kDirect ? 1 : NL]) {
        if constexpr (!kDirect) {
#pragma unroll
            for (int i = 0; i < NL; ++i) *reinterpret_cast<h8*>(img + dst(i, true)) = st[i];
        }
    };
    auto stage = [&](int step, char* img) {
        if constexpr (kDirect) {
            // per tile: one wave-uniform base (pool, chunk, key offset), then
            // its loads at the lanes' fixed offsets
#pragma unroll
            for (int k = 0; k < TPW; ++k) {
                const int tt = ta + k;
                const int ts = kwave ? tile_start<D>(step, tt, n_keys) : VLay<D, C>::tile_src(step, tt, n_keys);
                const size_t cb = static_cast<size_t>(chunk_of(step, tt)) * cstride;
                const char* base = kwave ? kbase + cb + static_cast<size_t>(ts % C) * 16
                                         : vbase + cb + static_cast<size_t>(ts % C) * (D * 2);
#pragma unroll
                for (int i = k * (NL / TPW); i < (k + 1) * (NL / TPW); ++i)
                    __builtin_amdgcn_global_load_lds(
                        reinterpret_cast<const h8*>(base + loff[i]),
                        (__attribute__((address_space(3))) void*)(img + ldso[i]), 16, 0, 0);
            }
        } else {
            stage_regs(step, stg);
        }
    };

    h8 qb[RT][KS];
    int qrow[RT];
    int lim[RT];
    f4 o[RT][DT];
    float m_run[RT], l_run[RT];
    // Every lane reads a row entry (lanes past the unit's rows read its last
    // one and discard it), so that the reads of all row tiles go out together
    // instead of one tile's waiting for the previous tile's branch.  (A unit
    // always has rows; one without would read none.)
    int qpos_raw[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        const int ri = row_lo + min(16 * (RT * role + rt) + col, n_rows - 1);
        qrow[rt] = n_rows > 0 ? a.rows[ri] : -1;
        qpos_raw[rt] = kCausal && n_rows > 0 ? a.qpos[ri] : 0;
    }
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        const int r = 16 * (RT * role + rt) + col;
        const bool valid = computes && r < n_rows;
        qrow[rt] = valid ? qrow[rt] : -1;
        lim[rt] = kCausal && valid ? min(n_keys, qpos_raw[rt] + 1 - key_base) : n_keys;
        if constexpr (P != 3) {
            const _Float16* qp = static_cast<const _Float16*>(a.q) +
                                 (static_cast<size_t>(qrow[rt] < 0 ? 0 : qrow[rt]) * H + head) * D + 8 * grp;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                qb[rt][ks] = qrow[rt] >= 0 ? *reinterpret_cast<const h8*>(qp + 32 * ks) : h8{};
        }
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) o[rt][dt] = f4{0.f, 0.f, 0.f, 0.f};
        m_run[rt] = -INFINITY;
        l_run[rt] = 0.f;
    }
    if constexpr (P == 3) {
        // ping-pong: the queries wait in this wave's part of the Q area of LDS
        // (img3), in operand order -- a contiguous 1 KiB per (row tile,
        // k-step) -- instead of 32 registers.  The rows of every tile are
        // read first, then all queries, and the unit's first two steps of K/V
        // are issued while the queries are in flight (the images and the Q
        // area were free at the end of the last unit): two memory round trips
        // before the first product instead of one per dependent read.
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            const _Float16* qp = static_cast<const _Float16*>(a.q) +
                                 (static_cast<size_t>(qrow[rt] < 0 ? 0 : qrow[rt]) * H + head) * D + 8 * grp;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                qb[rt][ks] = qrow[rt] >= 0 ? *reinterpret_cast<const h8*>(qp + 32 * ks) : h8{};
        }
        stage(0, img0);
        if (n_steps > 1) stage(1, img1);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                *reinterpret_cast<h8*>(img3 + ((role * RT + rt) * KS + ks) * 1024 + lane * 16) = qb[rt][ks];
    }

    // One row tile per wave (decode units): every K fragment of the step is
    // read before the first product and every V fragment before the softmax,
    // so that the step waits for LDS twice instead of once per fragment pair
    // (a decode unit's step is bound by its waves' latency, not by registers).
    auto compute1 = [&](const char* img, int step) {
        h8 kf[NT][KS];
#pragma unroll
        for (int tt = 0; tt < NT; ++tt)
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                kf[tt][ks] = *reinterpret_cast<const h8*>(img + ((tt * (D / 8) + 4 * ks + grp) * 16 + col) * 16);
        f4 s[NT];
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) {
            s[tt] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                s[tt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf[tt][ks], qb[0][ks], s[tt], 0, 0, 0);
        }
        using L = VLay<D, C>;
        typename L::Frag vf[DT][L::kFrags];
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int f = 0; f < L::kFrags; ++f)
                vf[dt][f] = *reinterpret_cast<const typename L::Frag*>(img + v_frag_lds<D, C>(f, dt, col, grp));
        h4 pq[NT];
        softmax_step<NT, DT, true>(s, pq, o[0], m_run[0], l_run[0], step, lim[0], grp, a.scale_log2e);
        if ((step + 1) * Step<D>::kKeys > n_keys) {           // V past the last key: zero
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                for (int f = 0; f < L::kFrags; ++f)
                    vf[dt][f] = mask_frag<D, C>(vf[dt][f], step * Step<D>::kKeys, f, grp, n_keys);
        }
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) o[0][dt] = pv_frags<D, C>(o[0][dt], vf[dt], pq);
    };
    // S^T of a step for every row tile
    auto qk_rt = [&](const char* img, f4 (&s)[RT][NT]) {
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) {
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) s[rt][tt] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const h8 kf = *reinterpret_cast<const h8*>(
                    img + ((tt * (D / 8) + 4 * ks + grp) * 16 + col) * 16);
#pragma unroll
                for (int rt = 0; rt < RT; ++rt)
                    s[rt][tt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf, qb[rt][ks], s[rt][tt], 0, 0, 0);
            }
        }
    };
    // the softmax of a step whose S^T is s: its weights P^T in pq
    auto softmax_rt = [&](int step, f4 (&s)[RT][NT], h4 (&pq)[RT][NT]) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            softmax_step<NT, DT, true, P == 3 ? kLazyLog2 : 0>(s[rt], pq[rt], o[rt], m_run[rt], l_run[rt],
                                                               step, lim[rt], grp, a.scale_log2e);
            // ping-pong: one row tile at a time (fewer registers in flight)
            if constexpr (P == 3) __builtin_amdgcn_sched_barrier(0);
        }
    };
    // O^T += V^T P^T for a step; V entries past the last key are zeroed on
    // the last step only
    auto pv_rt = [&](const char* img, int step, const h4 (&pq)[RT][NT]) {
        auto pv = [&](auto masked) {
            using L = VLay<D, C>;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                typename L::Frag v[L::kFrags];
#pragma unroll
                for (int f = 0; f < L::kFrags; ++f) {
                    v[f] = *reinterpret_cast<const typename L::Frag*>(img + v_frag_lds<D, C>(f, dt, col, grp));
                    if constexpr (decltype(masked)::value)
                        v[f] = mask_frag<D, C>(v[f], step * Step<D>::kKeys, f, grp, n_keys);
                }
#pragma unroll
                for (int rt = 0; rt < RT; ++rt) o[rt][dt] = pv_frags<D, C>(o[rt][dt], v, pq[rt]);
            }
        };
        if ((step + 1) * Step<D>::kKeys > n_keys)
            pv(Flag<true>{});
        else
            pv(Flag<false>{});
    };
    auto compute = [&](const char* img, int step) {
        if constexpr (RT == 1) {
            compute1(img, step);
        } else {
            f4 s[RT][NT];
            h4 pq[RT][NT];
            qk_rt(img, s);
            softmax_rt(step, s, pq);
            pv_rt(img, step, pq);
        }
    };

    if constexpr (P == 2) {
        static_assert(kDirect, "two phases need loads straight into LDS");
        // iteration i: phase ph computes step 2i + ph from image (i % 2) of its
        // pair while step 2i + 2 + ph loads into the other image of the pair
        char* mine0 = phase ? img2 : img0;
        char* mine1 = phase ? img3 : img1;
        const int n_iter = (n_steps + 1) / 2;
        if (phase < n_steps) stage(phase, mine0);
        for (int it = 0; it < n_iter; ++it) {
            const int step = 2 * it + phase;
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // this wave's loads (see below)
            __syncthreads();
            char* cur = (it & 1) ? mine1 : mine0;
            char* nxt = (it & 1) ? mine0 : mine1;
            if (step + 2 < n_steps) stage(step + 2, nxt);
            if (step < n_steps && computes) compute(cur, step);
        }
        __syncthreads();                     // every image has been read
        // phase 1's (o, m, n) to phase 0: o as [role][dt][lane] f4, then (m, n)
        constexpr int kOBytes = W * DT * 64 * 16;
        static_assert(W == kWaves && kOBytes + W * 64 * 8 <= unit_lds_bytes<D>(), "state exchange fits");
        f4* xo = reinterpret_cast<f4*>(img0);
        float* xml = reinterpret_cast<float*>(img0 + kOBytes);
        if (phase == 1 && computes) {
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) xo[(role * DT + dt) * 64 + lane] = o[0][dt];
            xml[(role * 64 + lane) * 2] = m_run[0];
            xml[(role * 64 + lane) * 2 + 1] = l_run[0];
        }
        __syncthreads();
        if (phase == 0 && computes) {
            const float mb = xml[(role * 64 + lane) * 2];
            const float lb = xml[(role * 64 + lane) * 2 + 1];
            const float mx = fmaxf(m_run[0], mb);     // finite: phase 0 has step 0
            const float wa = fast_exp2(m_run[0] - mx);
            const float wb = fast_exp2(mb - mx);      // 0 when phase 1 had no step
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) o[0][dt] = wa * o[0][dt] + wb * xo[(role * DT + dt) * 64 + lane];
            l_run[0] = wa * l_run[0] + wb * lb;
            m_run[0] = mx;
            finish<D, DT>(a, o[0], m_run[0], l_run[0], qrow[0], out < 0 ? -1 : out + 16 * role, head,
                          col, grp);
        }
        __syncthreads();                     // the next unit reuses the images
        return;
    } else if constexpr (P == 3) {
        static_assert(kDirect && RT > 1 && NL == 4, "ping-pong: loads straight into LDS, two row tiles");
        // What a wave carries across a barrier is either S^T of a step or its
        // weights P^T; both live in sp (P^T as the bits of sp[rt][tt].xy), so
        // the two kinds of wave need one set of registers.
        f4 sp[RT][NT];
        // One matrix block: O^T += V^T P^T for a step (P^T from sp), then -- if
        // kQK -- S^T = K Q^T of the next step into sp, k-step by k-step (the
        // queries' fragments of a k-step come from the Q area once and meet
        // every key tile).  A lone wave per SIMD issues these, so the reads
        // of the next group of fragments are issued before the products of
        // the current one (one ds_read_b128 per ~30 cycles per wave), in an
        // order pinned by scheduling groups.  kMask zeroes V past the unit's
        // last key (its last step, which is also the one without kQK).
        using VL = VLay<D, C>;
        using VF = typename VL::Frag;
        constexpr int NF = VL::kFrags;
        constexpr int kDsRead = 0x100, kMfma = 0x008;
        auto vread = [&](VF (&v)[NF], const char* img, int dt) {
#pragma unroll
            for (int f = 0; f < NF; ++f)
                v[f] = *reinterpret_cast<const VF*>(img + v_frag_lds<D, C>(f, dt, col, grp));
        };
        auto qkread = [&](h8 (&q)[RT], h8 (&k)[NT], const char* img, int ks) {
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
                q[rt] = *reinterpret_cast<const h8*>(img3 + ((role * RT + rt) * KS + ks) * 1024 + lane * 16);
#pragma unroll
            for (int tt = 0; tt < NT; ++tt)
                k[tt] = *reinterpret_cast<const h8*>(img + ((tt * (D / 8) + 4 * ks + grp) * 16 + col) * 16);
        };
        auto qkmma = [&](const h8 (&q)[RT], const h8 (&k)[NT]) {
#pragma unroll
            for (int tt = 0; tt < NT; ++tt)
#pragma unroll
                for (int rt = 0; rt < RT; ++rt)
                    sp[rt][tt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(k[tt], q[rt], sp[rt][tt], 0, 0, 0);
        };
        auto zero_sp = [&]() {
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int tt = 0; tt < NT; ++tt) sp[rt][tt] = f4{0.f, 0.f, 0.f, 0.f};
        };
        // Q K^T alone (the first step of a unit), pipelined the same way
        auto qk_pp = [&](const char* img) {
            h8 qa[RT], ka[NT], qb2[RT], kb[NT];
            zero_sp();
            qkread(qa, ka, img, 0);
            __builtin_amdgcn_sched_group_barrier(kDsRead, RT + NT, 0);
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                if (ks + 1 < KS) {
                    if (ks & 1)
                        qkread(qa, ka, img, ks + 1);
                    else
                        qkread(qb2, kb, img, ks + 1);
                    __builtin_amdgcn_sched_group_barrier(kDsRead, RT + NT, 0);
                }
                if (ks & 1)
                    qkmma(qb2, kb);
                else
                    qkmma(qa, ka);
                __builtin_amdgcn_sched_group_barrier(kMfma, RT * NT, 0);
            }
        };
        auto block = [&](auto mask, auto with_qk, const char* pv_img, int pv_step, const char* qk_img) {
            constexpr bool kMask = decltype(mask)::value, kQK = decltype(with_qk)::value;
            h4 pq[RT][NT];
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int tt = 0; tt < NT; ++tt)
                    pq[rt][tt] = __builtin_bit_cast(
                        h4, __builtin_shufflevector(sp[rt][tt], sp[rt][tt], 0, 1));
            VF va[NF], vb[NF];
            h8 qa[RT], ka[NT], qb2[RT], kb[NT];
            vread(va, pv_img, 0);
            __builtin_amdgcn_sched_group_barrier(kDsRead, NF, 0);
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                if (dt + 1 < DT) {
                    if (dt & 1)
                        vread(va, pv_img, dt + 1);
                    else
                        vread(vb, pv_img, dt + 1);
                    __builtin_amdgcn_sched_group_barrier(kDsRead, NF, 0);
                } else if constexpr (kQK) {
                    qkread(qa, ka, qk_img, 0);
                    __builtin_amdgcn_sched_group_barrier(kDsRead, RT + NT, 0);
                }
                VF (&v)[NF] = (dt & 1) ? vb : va;
                if constexpr (kMask) {
#pragma unroll
                    for (int f = 0; f < NF; ++f)
                        v[f] = mask_frag<D, C>(v[f], pv_step * Step<D>::kKeys, f, grp, n_keys);
                }
#pragma unroll
                for (int rt = 0; rt < RT; ++rt) o[rt][dt] = pv_frags<D, C>(o[rt][dt], v, pq[rt]);
                __builtin_amdgcn_sched_group_barrier(kMfma, RT * NF, 0);
            }
            zero_sp();
            if constexpr (kQK) {
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    if (ks + 1 < KS) {
                        if (ks & 1)
                            qkread(qa, ka, qk_img, ks + 1);
                        else
                            qkread(qb2, kb, qk_img, ks + 1);
                        __builtin_amdgcn_sched_group_barrier(kDsRead, RT + NT, 0);
                    }
                    if (ks & 1)
                        qkmma(qb2, kb);
                    else
                        qkmma(qa, ka);
                    __builtin_amdgcn_sched_group_barrier(kMfma, RT * NT, 0);
                }
            }
        };
        auto softmax_pp = [&](int step) {
            h4 pq[RT][NT];
            softmax_rt(step, sp, pq);
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int tt = 0; tt < NT; ++tt) {
                    const auto w = __builtin_bit_cast(float __attribute__((ext_vector_type(2))), pq[rt][tt]);
                    sp[rt][tt][0] = w[0];
                    sp[rt][tt][1] = w[1];
                }
        };
        // Step i (i + 1 < n_steps) is: wait for this wave's loads of step
        // i + 1, a workgroup barrier (step i + 1 is complete, step i - 1 is
        // read), the second half (lead: softmax of i; partner: P V of i and
        // Q K^T of i + 1), a plain barrier, and the first half of step i + 1
        // (lead: P V of i and Q K^T of i + 1; partner: softmax of i + 1).
        // Every wave loads its part of step i + 2 into the image of step
        // i - 1 at the start of its softmax half: a lead right after the
        // workgroup barrier, a partner after the plain one, not in front of
        // its matrix block (a wave that issues loads stalls while the compute
        // unit's earlier loads drain; spreading them over the half, or one
        // wave of a pair issuing both parts, measured slower).  The
        // plain barrier only keeps the two kinds of wave in step: the next
        // half reads the same images, and the loads in flight go to the
        // third (__syncthreads() would wait for them: its release fence
        // covers writes to LDS).  Each kind of wave runs its own loop, the
        // steps unrolled by three so that every image is known at compile
        // time (the compiler then waits for loads into LDS only where an
        // image is read), and the last step is peeled off.
        // (Both barriers are fenced with sched_barrier: a barrier orders
        // memory operations, and the compiler would otherwise move the last
        // matrix instructions of a block into the next half.)
        auto half2 = [&](int i, char* ld) {
            __builtin_amdgcn_sched_barrier(0);
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();
            __builtin_amdgcn_sched_barrier(0);
            if (ld && i + 2 < n_steps) stage(i + 2, ld);
        };
        auto mid = [&]() {
            __builtin_amdgcn_sched_barrier(0);
            __builtin_amdgcn_s_barrier();
            __builtin_amdgcn_sched_barrier(0);
        };
        auto steps = [&](auto body) {
            int i = 0;
            for (; i + 3 < n_steps; i += 3) {
                body(i, img0, img1, img2);
                body(i + 1, img1, img2, img0);
                body(i + 2, img2, img0, img1);
            }
            if (i + 1 < n_steps) body(i, img0, img1, img2);
            if (i + 2 < n_steps) body(i + 1, img1, img2, img0);
            return (n_steps - 1) % 3;            // the image of the last step
        };
        // Every wave waits for its loads of steps 0 and 1 (issued with the
        // queries above): step 0 and the Q area are complete when all have
        // passed the plain barrier that follows.  Then the partner computes
        // S^T of step 0 ahead.
        auto prologue = [&]() {
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            mid();
        };
        int last;
        if (!computes) {
            prologue();
            mid();
            last = steps([&](int i, char*, char*, char* ld) {
                half2(i, ld);
                mid();
            });
            half2(n_steps - 1, nullptr);
            mid();
        } else if (lead) {
            prologue();
            mid();
            qk_pp(img0);
            last = steps([&](int i, char* cur, char* nxt, char* ld) {
                half2(i, ld);
                softmax_pp(i);
                mid();
                block(Flag<false>{}, Flag<true>{}, cur, i, nxt);
            });
            char* cur = last == 0 ? img0 : last == 1 ? img1 : img2;
            half2(n_steps - 1, nullptr);
            softmax_pp(n_steps - 1);
            mid();
            block(Flag<true>{}, Flag<false>{}, cur, n_steps - 1, nullptr);
        } else {
            prologue();
            qk_pp(img0);
            mid();
            softmax_pp(0);
            last = steps([&](int i, char* cur, char* nxt, char* ld) {
                half2(i, nullptr);
                block(Flag<false>{}, Flag<true>{}, cur, i, nxt);
                mid();
                if (i + 2 < n_steps) stage(i + 2, ld);
                softmax_pp(i + 1);
            });
            char* cur = last == 0 ? img0 : last == 1 ? img1 : img2;
            half2(n_steps - 1, nullptr);
            block(Flag<true>{}, Flag<false>{}, cur, n_steps - 1, nullptr);
            mid();
        }
        __syncthreads();                     // the next unit reuses the images
    } else if constexpr (kDirect && kCausal && D == 256) {
        // Prefill at head_dim 256, whose steps are 16 keys: four steps per
        // workgroup barrier.  Each of the four images holds two steps (one
        // at its start, one Img<D>::kBytes in); steps s .. s + 3 are computed
        // from one pair of images (img0, img1 or img2, img3) while s + 4 ..
        // s + 7 load into the other pair.
        constexpr int kB = Img<D>::kBytes;
        auto at = [&](char* a, char* b, int j) { return (j < 2 ? a : b) + (j & 1) * kB; };
        auto stage4 = [&](int s, char* a, char* b) {
#pragma unroll
            for (int j = 0; j < 4; ++j)
                if (s + j < n_steps) stage(s + j, at(a, b, j));
        };
        auto body4 = [&](char* ca, char* cb, char* na, char* nb, int s) {
            // this wave's loads of steps s .. s + 3 are in, then every
            // wave's; nobody reads steps s - 4 .. s - 1 any more
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();
            stage4(s + 4, na, nb);
            if (computes) {
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    if (s + j < n_steps) compute(at(ca, cb, j), s + j);
            }
        };
        stage4(0, img0, img1);
        for (int s = 0; s < n_steps; s += 8) {
            body4(img0, img1, img2, img3, s);
            if (s + 4 < n_steps) body4(img2, img3, img0, img1, s + 4);
        }
        __syncthreads();                     // the next unit reuses the images
    } else if constexpr (kDirect) {
        // step s is computed from image s % 2 while step s + 1 loads into the other
        auto body = [&](char* cur, char* nxt, int step) {
            // The loads into LDS count as vector-memory operations: wait for this
            // wave's own (the workgroup barrier alone does not), then for every
            // wave -- the image of step is complete and nobody reads step - 1's.
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();
            if (step + 1 < n_steps) stage(step + 1, nxt);
            if (computes) compute(cur, step);
        };
        stage(0, img0);
        for (int step = 0; step < n_steps; step += 2) {
            body(img0, img1, step);
            if (step + 1 < n_steps) body(img1, img0, step + 1);
        }
        __syncthreads();                     // the next unit reuses the images
    } else {
        // loads staged in registers (head_dim < 128): two steps per barrier.
        // Steps s, s + 1 go from their registers into one image (img0 or
        // img1 in turn; each holds two steps, the second Img<D>::kBytes in)
        // and are computed there while s + 2, s + 3 load into the registers.
        // A wave that writes an image has passed the previous barrier, which
        // every wave reached only after computing the steps it held before.
        constexpr int kB = Img<D>::kBytes;
        h8 stg_b[kDirect ? 1 : NL];
        auto body2 = [&](char* img, int s) {
            commit_regs(img, stg);
            if (s + 1 < n_steps) commit_regs(img + kB, stg_b);
            __syncthreads();
            if (s + 2 < n_steps) stage_regs(s + 2, stg);
            if (s + 3 < n_steps) stage_regs(s + 3, stg_b);
            if (computes) {
                compute(img, s);
                if (s + 1 < n_steps) compute(img + kB, s + 1);
            }
        };
        stage_regs(0, stg);
        if (n_steps > 1) stage_regs(1, stg_b);
        for (int s = 0; s < n_steps; s += 4) {
            body2(img0, s);
            if (s + 2 < n_steps) body2(img1, s + 2);
        }
        __syncthreads();                     // the next unit reuses the images
    }
    if (computes) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
            finish<D, DT>(a, o[rt], m_run[rt], l_run[rt], qrow[rt],
                          out < 0 ? -1 : out + 16 * (RT * role + rt), head, col, grp);
    }
}

// Wave-uniform description of one single-wave task.
struct Task {
    int ids;                 // the task's chunk ids, one per lane (lane_ids)
    int n_valid;             // keys to attend over
    int n_steps;             // ceil(n_valid / keys per step)
    int row_lo;              // depth-first position of query row 0
    int n_rows;
    int out;                 // partial slot of row 0, or -1: write O
    int head;
};

template <int D, int C>
__device__ __forceinline__ Task fetch_task(const AttnArgs& a, int idx) {
    cint* tk = meta(a.tasks) + 2 * idx;
    const int wave_id = tk[0];
    Task t;
    t.head = tk[1];
    cint* wd = meta(a.waves) + 8 * wave_id;
    const int n_chunks = wd[1];
    const int key_base = wd[2];
    const int len_row = wd[3];
    t.ids = lane_ids(meta(a.chunks) + wd[0], n_chunks, static_cast<int>(threadIdx.x & 63));
    t.row_lo = wd[4];
    t.n_rows = wd[5];
    t.out = wd[6];
    int n_valid = n_chunks * C - wd[7];          // wd[7]: keys the last chunk lacks
    if (len_row >= 0) n_valid = min(n_valid, meta(a.seqlen)[len_row] - key_base);
    t.n_valid = n_valid;
    t.n_steps = (n_valid + Step<D>::kKeys - 1) / Step<D>::kKeys;
    return t;
}

template <int D, int C>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 8)))
void attn_kernel(AttnArgs a) {
    static_assert(D % 32 == 0 && C % 16 == 0, "tile shape");
    constexpr int KS = D / 32;     // 32-dim k-steps of Q K^T
    constexpr int DT = D / 16;     // 16-dim output tiles of P V
    constexpr int NT = Step<D>::kTiles;
    // units: two LDS images, filled in turn straight from memory (D >= 128)
    __shared__ __attribute__((aligned(16))) char lds[Img<D>::kBytes];
    __shared__ __attribute__((aligned(16))) char lds1[D >= 128 ? Img<D>::kBytes : 16];
    const int H = a.H;
    const int wave = wave_uniform(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int col = lane & 15;     // MFMA row/column index held by this lane
    const int grp = lane >> 4;     // which 8-element k slice of the fragment

    // ---- this workgroup's units, all 4 waves together ---------------------------
    {
        const int ufirst = meta(a.wg_units)[2 * blockIdx.x];
        const int ucount = meta(a.wg_units)[2 * blockIdx.x + 1];
        for (int k = 0; k < ucount; ++k) {
            if constexpr (D >= 128)
                run_unit_wide<D, C, 1, false>(a, meta(a.units) + 8 * (ufirst + k), wave, lane, lds, lds1);
            else
                run_unit<D, C>(a, meta(a.units) + 8 * (ufirst + k), wave, lane, lds);
        }
    }

    // ---- this wave's single-wave tasks ------------------------------------------
    const int lane_id = blockIdx.x * kWaves + wave;
    const int first = meta(a.lists)[2 * lane_id];
    const int count = meta(a.lists)[2 * lane_id + 1];
    if (count == 0) return;

    const size_t slice = static_cast<size_t>(C) * D;          // halves per (chunk, head)
    const _Float16* __restrict__ kpool = static_cast<const _Float16*>(a.kpool);
    const _Float16* __restrict__ vpool = static_cast<const _Float16*>(a.vpool);

    h8 qb[KS];            // Q^T (B operand): row col, dims 32*ks + 8*grp .. +7
    h8 kr[NT][KS];        // K of one step: tile t = keys 16t .. 16t+15
    using VL = VLay<D, C>;
    typename VL::Frag vr[DT][VL::kFrags];   // V of one step: [dim tile][fragment]

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
    const uint32_t v_lane = static_cast<uint32_t>(v_frag_lane<D, C>(0, col, grp));   // the lane's keys, dim col
    auto slice_of = [&](const _Float16* pool, int chunk, int head) {
        return reinterpret_cast<const char*>(pool + (static_cast<size_t>(chunk) * H + head) * slice);
    };
    auto load_k = [&](const Task& t, int step) {
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) {
            const int key = tile_start<D>(step, tt, t.n_valid);
            const char* base = slice_of(kpool, tile_id<D, C>(t.ids, step, tt, t.n_valid), t.head) + (key % C) * 16;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                kr[tt][ks] = __builtin_nontemporal_load(
                    reinterpret_cast<const h8*>(base + ks * (C * 64) + k_lane));
        }
    };
    auto load_v = [&](const Task& t, int step) {
        constexpr int TPF = NT / VL::kFrags;       // key tiles per fragment
        const char* base[VL::kFrags];
#pragma unroll
        for (int f = 0; f < VL::kFrags; ++f) {
            const int key = VL::tile_src(step, TPF * f, t.n_valid);
            base[f] = slice_of(vpool, tile_id<D, C>(t.ids, step, TPF * f, t.n_valid), t.head) + (key % C) * (D * 2);
        }
        // dim tile by dim tile across the fragments: the P V product of a dim
        // tile waits only for its own loads (measured faster than fragment by
        // fragment when every wave streams one long context)
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int f = 0; f < VL::kFrags; ++f)
                vr[dt][f] = __builtin_nontemporal_load(
                    reinterpret_cast<const typename VL::Frag*>(base[f] + dt * (VL::kGroups * 256) + v_lane));
    };

    Task cur = fetch_task<D, C>(a, first);
    int cur_qrow = query_row(cur);
    load_q(cur, cur_qrow);
    load_k(cur, 0);
    load_v(cur, 0);
    int ti = 0;
    bool has_next = count > 1;
    Task nxt = cur;
    int nxt_qrow = -1;
    if (has_next) {
        nxt = fetch_task<D, C>(a, first + 1);
        nxt_qrow = query_row(nxt);
    }

    f4 o[DT];
    float m_run, l_run;
    f4 s[NT];
    for (;;) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) o[dt] = f4{0.f, 0.f, 0.f, 0.f};
        m_run = -INFINITY;
        l_run = 0.f;
        // all steps but the last: the next step's K and V follow right behind
        const int n_steps = cur.n_steps;
        for (int step = 0; step + 1 < n_steps; ++step) {
            qk<NT, KS>(s, kr, qb);
            load_k(cur, step + 1);
            softmax_pv<D, C>(s, vr, o, m_run, l_run, step, cur.n_valid, grp, a.scale_log2e);
            load_v(cur, step + 1);
        }
        // last step: the next task's queries and K/V follow instead
        qk<NT, KS>(s, kr, qb);
        if (has_next) {
            load_q(nxt, nxt_qrow);
            load_k(nxt, 0);
        }
        softmax_pv<D, C>(s, vr, o, m_run, l_run, n_steps - 1, cur.n_valid, grp, a.scale_log2e);
        finish<D, DT>(a, o, m_run, l_run, cur_qrow, cur.out, cur.head, col, grp);
        if (!has_next) break;
        load_v(nxt, 0);
        cur = nxt;
        cur_qrow = nxt_qrow;
        ++ti;
        has_next = ti + 1 < count;
        if (has_next) {
            nxt = fetch_task<D, C>(a, first + ti + 1);
            nxt_qrow = query_row(nxt);
        }
    }
}

// Prefill: the workgroup's units with the causal mask per row; nothing else.
template <int D, int C>
__global__ __launch_bounds__(64 * prefill_waves(D)) __attribute__((amdgpu_waves_per_eu(2, 8)))
void prefill_kernel(AttnArgs a) {
    constexpr bool kPingPong = D == 128;
    // head_dim 256: four 16-key steps per barrier, from four images of two
    // steps each; head_dim 64: two steps per barrier, two images of two steps
    constexpr bool kFourStep = D == 256;
    constexpr int kImg = (kFourStep || D < 128 ? 2 : 1) * Img<D>::kBytes;
    __shared__ __attribute__((aligned(16))) char img0[kImg];
    __shared__ __attribute__((aligned(16))) char img1[kImg];
    __shared__ __attribute__((aligned(16))) char img2[kPingPong || kFourStep ? kImg : 16];
    // the units' queries (ping-pong): 16 rows x D halves per row tile of every
    // wave; the fourth image at head_dim 256
    __shared__ __attribute__((aligned(16)))
    char qlds[kPingPong ? prefill_waves(D) * prefill_row_tiles(D) * 16 * D * 2 : kFourStep ? kImg : 16];
    const int wave = wave_uniform(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int ufirst = meta(a.wg_units)[2 * blockIdx.x];
    const int ucount = meta(a.wg_units)[2 * blockIdx.x + 1];
    if constexpr (kPingPong) {
        // Pair the waves by the SIMD they run on: of the waves of this
        // workgroup on a SIMD, in index order, every other one leads.  (The
        // SIMD numbers pass through the Q area before any query does.)
        int* simd_of = reinterpret_cast<int*>(qlds);
        const int simd = wave_uniform(simd_id());
        if (lane == 0) simd_of[wave] = simd;
        __syncthreads();
        int below = 0;
        for (int w = 0; w < wave; ++w) below += simd_of[w] == simd;
        const bool lead = (below & 1) == 0;
        __syncthreads();
        for (int k = 0; k < ucount; ++k)
            run_unit_wide<D, C, prefill_row_tiles(D), true, prefill_waves(D), 3>(
                a, meta(a.units) + 8 * (ufirst + k), wave, lane, img0, img1, img2, qlds, lead);
    } else {
        for (int k = 0; k < ucount; ++k)
            run_unit_wide<D, C, prefill_row_tiles(D), true, prefill_waves(D)>(
                a, meta(a.units) + 8 * (ufirst + k), wave, lane, img0, img1, img2, qlds);
    }
}

// Decode plans whose work is all workgroup units (every batch row's context
// lies in chunks shared by at least unit_rows rows, head_dim >= 128): one
// workgroup of 8 waves per compute unit runs its units in two phases of 4
// waves (run_unit_wide, P = 2) from four LDS images.
template <int D, int C>
__global__ __launch_bounds__(64 * 2 * kWaves) __attribute__((amdgpu_waves_per_eu(2, 8)))
void unit_kernel(AttnArgs a) {
    static_assert(D >= 128, "two-phase units load straight into LDS");
    __shared__ __attribute__((aligned(16))) char lds[unit_lds_bytes<D>()];
    const int wave = wave_uniform(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int ufirst = meta(a.wg_units)[2 * blockIdx.x];
    const int ucount = meta(a.wg_units)[2 * blockIdx.x + 1];
    for (int k = 0; k < ucount; ++k)
        run_unit_wide<D, C, 1, false, kWaves, 2>(a, meta(a.units) + 8 * (ufirst + k), wave, lane, lds,
                                                 lds + Img<D>::kBytes, lds + 2 * Img<D>::kBytes,
                                                 lds + 3 * Img<D>::kBytes);
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
// One thread moves 8 dims of one (token, head): a 16-byte K piece and the
// same dims of V.
template <int D, int C>
__device__ __forceinline__ void scatter_piece(const ScatterArgs& a, int64_t gid, int64_t slot_of_tok,
                                              int64_t tok) {
    constexpr int P = D / 8;
    const int piece = static_cast<int>(gid % P);
    const int head = static_cast<int>((gid / P) % a.H);
    const int64_t slot = slot_of_tok;
    if (slot < 0 || slot >= a.slot_limit) return;
    const int64_t chunk = slot / C;
    const int t = static_cast<int>(slot % C);
    const size_t sbase = (static_cast<size_t>(chunk) * a.H + head) * C * D;
    const size_t src = (static_cast<size_t>(tok) * a.H + head) * D + piece * 8;
    const h8 kv = *reinterpret_cast<const h8*>(static_cast<const _Float16*>(a.knew) + src);
    *reinterpret_cast<h8*>(static_cast<_Float16*>(a.kpool) + sbase +
                           (static_cast<size_t>(piece) * C + t) * 8) = kv;
    const h8 vv = *reinterpret_cast<const h8*>(static_cast<const _Float16*>(a.vnew) + src);
    _Float16* vb = static_cast<_Float16*>(a.vpool) + sbase + VLay<D, C>::elem(t, piece * 8);
#pragma unroll
    for (int e = 0; e < 8; ++e) vb[e * 8] = vv[e];
}

template <int D, int C>
__global__ __launch_bounds__(256) void scatter_kernel(ScatterArgs a) {
    const int64_t gid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (gid >= a.n_tokens * a.H * (D / 8)) return;
    const int64_t tok = gid / (static_cast<int64_t>(a.H) * (D / 8));
    scatter_piece<D, C>(a, gid, a.slots[tok], tok);
}

// Same, with the slots in the launch arguments (n_tokens <= kInlineSlots).
template <int D, int C>
__global__ __launch_bounds__(256) void scatter_inline_kernel(ScatterArgs a, InlineSlots is) {
    const int64_t gid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (gid >= a.n_tokens * a.H * (D / 8)) return;
    const int64_t tok = gid / (static_cast<int64_t>(a.H) * (D / 8));
    scatter_piece<D, C>(a, gid, is.slot[tok], tok);
}

// Move tokens' K/V between pool slots (the split of a node under token
// matching).  One thread per (move, head, 8 dims): a 16-byte K piece and the
// same 8 dims of V, which sit 8 halves apart in the V layout.
template <int D, int C>
__global__ __launch_bounds__(256) void move_kernel(MoveArgs a) {
    constexpr int P = D / 8;
    const int64_t gid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (gid >= a.n * a.H * P) return;
    const int64_t i = gid / (static_cast<int64_t>(a.H) * P);
    const int piece = static_cast<int>(gid % P);
    const int head = static_cast<int>((gid / P) % a.H);
    const int64_t from = a.src[i], to = a.dst[i];
    if (from < 0 || from >= a.slot_limit || to < 0 || to >= a.slot_limit) return;
    const size_t fb = (static_cast<size_t>(from / C) * a.H + head) * C * D;
    const size_t tb = (static_cast<size_t>(to / C) * a.H + head) * C * D;
    const int ft = static_cast<int>(from % C), tt = static_cast<int>(to % C);
    _Float16* kp = static_cast<_Float16*>(a.kpool);
    *reinterpret_cast<h8*>(kp + tb + (static_cast<size_t>(piece) * C + tt) * 8) =
        *reinterpret_cast<const h8*>(kp + fb + (static_cast<size_t>(piece) * C + ft) * 8);
    _Float16* vp = static_cast<_Float16*>(a.vpool);
    const _Float16* vf = vp + fb + VLay<D, C>::elem(ft, piece * 8);
    _Float16* vt = vp + tb + VLay<D, C>::elem(tt, piece * 8);
#pragma unroll
    for (int e = 0; e < 8; ++e) vt[e * 8] = vf[e * 8];
}

__global__ __launch_bounds__(256) void copy_words_kernel(const int32_t* __restrict__ src,
                                                         int32_t* __restrict__ dst, int64_t n) {
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
         i += static_cast<int64_t>(gridDim.x) * blockDim.x)
        dst[i] = src[i];
}

template <int D, int C>
hipError_t attn_dc(const AttnArgs& a, hipStream_t s) {
    const unsigned grid = static_cast<unsigned>(a.n_wg);
    if (grid == 0) return hipSuccess;
    attn_kernel<D, C><<<dim3(grid), dim3(256), 0, s>>>(a);
    return hipGetLastError();
}

template <int D, int C>
hipError_t units_dc(const AttnArgs& a, hipStream_t s) {
    const unsigned grid = static_cast<unsigned>(a.n_wg);
    if (grid == 0) return hipSuccess;
    if constexpr (D >= 128) {
        unit_kernel<D, C><<<dim3(grid), dim3(64 * 2 * kWaves), 0, s>>>(a);
        return hipGetLastError();
    } else {
        return hipErrorInvalidValue;
    }
}

template <int D, int C>
hipError_t prefill_dc(const AttnArgs& a, hipStream_t s) {
    const unsigned grid = static_cast<unsigned>(a.n_wg);
    if (grid == 0) return hipSuccess;
    prefill_kernel<D, C><<<dim3(grid), dim3(64 * prefill_waves(D)), 0, s>>>(a);
    return hipGetLastError();
}

template <int D, int C>
hipError_t scatter_dc(const ScatterArgs& a, hipStream_t s) {
    const int64_t threads = a.n_tokens * a.H * (D / 8);
    if (threads == 0) return hipSuccess;
    scatter_kernel<D, C><<<dim3(static_cast<unsigned>((threads + 255) / 256)), dim3(256), 0, s>>>(a);
    return hipGetLastError();
}

template <int D, int C>
hipError_t scatter_inline_dc(const ScatterArgs& a, const InlineSlots& is, hipStream_t s) {
    const int64_t threads = a.n_tokens * a.H * (D / 8);
    if (threads == 0) return hipSuccess;
    scatter_inline_kernel<D, C><<<dim3(static_cast<unsigned>((threads + 255) / 256)), dim3(256), 0, s>>>(
        a, is);
    return hipGetLastError();
}

template <int D, int C>
hipError_t move_dc(const MoveArgs& a, hipStream_t s) {
    const int64_t threads = a.n * a.H * (D / 8);
    if (threads == 0) return hipSuccess;
    move_kernel<D, C><<<dim3(static_cast<unsigned>((threads + 255) / 256)), dim3(256), 0, s>>>(a);
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
        case 256016: return FN<256, 16>(__VA_ARGS__);                  \
        case 256032: return FN<256, 32>(__VA_ARGS__);                  \
        case 256064: return FN<256, 64>(__VA_ARGS__);                  \
        case 256128: return FN<256, 128>(__VA_ARGS__);                 \
        default: return hipErrorInvalidValue;                          \
    }

hipError_t launch_attn(const AttnArgs& a, int D, int C, hipStream_t s) {
    PKVT_DISPATCH(attn_dc, D, C, a, s)
}

hipError_t launch_units(const AttnArgs& a, int D, int C, hipStream_t s) {
    PKVT_DISPATCH(units_dc, D, C, a, s)
}

hipError_t launch_prefill(const AttnArgs& a, int D, int C, hipStream_t s) {
    PKVT_DISPATCH(prefill_dc, D, C, a, s)
}

hipError_t launch_scatter(const ScatterArgs& a, int D, int C, hipStream_t s) {
    PKVT_DISPATCH(scatter_dc, D, C, a, s)
}

hipError_t launch_scatter_inline(const ScatterArgs& a, const InlineSlots& is, int D, int C,
                                 hipStream_t s) {
    if (a.n_tokens > kInlineSlots) return hipErrorInvalidValue;
    PKVT_DISPATCH(scatter_inline_dc, D, C, a, is, s)
}

hipError_t launch_move(const MoveArgs& a, int D, int C, hipStream_t s) {
    PKVT_DISPATCH(move_dc, D, C, a, s)
}

hipError_t launch_copy_words(const int32_t* src, int32_t* dst, int64_t n, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    const int64_t blocks = std::min<int64_t>((n + 255) / 256, 1024);
    copy_words_kernel<<<dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s>>>(src, dst, n);
    return hipGetLastError();
}

hipError_t noalloc_scratch(void** ptr) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    static std::mutex mu;
    static void* addr[kMaxDevices] = {};
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void* p = nullptr;
        // the device address of this device's copy (dev is current)
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        addr[dev] = p;
    }
    *ptr = addr[dev];
    return hipSuccess;
}

hipError_t launch_merge(const MergeArgs& a, int D, hipStream_t s) {
    const int64_t waves = static_cast<int64_t>(a.n_merge) * a.H;
    if (waves == 0) return hipSuccess;
    const dim3 grid(static_cast<unsigned>((waves + kWaves - 1) / kWaves));
    if (D == 64)
        merge_kernel<64><<<grid, dim3(256), 0, s>>>(a);
    else if (D == 128)
        merge_kernel<128><<<grid, dim3(256), 0, s>>>(a);
    else if (D == 256)
        merge_kernel<256><<<grid, dim3(256), 0, s>>>(a);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace pkvt
