// Work-unit shapes that the prefill planner and the prefill kernel agree on.
#pragma once

namespace pkvt {

// Query-row tiles of 16 rows that one wave of a prefill unit computes: two
// up to head_dim 128, one at head_dim 256.
constexpr int prefill_row_tiles(int head_dim) { return head_dim <= 128 ? 2 : 1; }
// Waves of a prefill workgroup: every wave computes its own row tiles from
// one shared LDS image of each step, so eight waves read a step's K and V
// from memory once for 128 * prefill_row_tiles rows.  Two such waves per SIMD
// make one resident workgroup per CU; a grid of twice that many workgroups
// lets the dispatcher start the second half as the first ones finish.
constexpr int prefill_waves(int) { return 8; }
// Chunks one prefill unit reads (its chunk ids sit in two registers per lane).
constexpr int kPrefillMaxChunks = 128;

}  // namespace pkvt
