// Work-unit shapes that the prefill planner and the prefill kernel agree on.
#pragma once

namespace pkvt {

// Query-row tiles of 16 rows that one wave of a prefill unit computes: two
// up to head_dim 128 (a unit covers 128 rows), one at head_dim 256.
constexpr int prefill_row_tiles(int head_dim) { return head_dim <= 128 ? 2 : 1; }
// Chunks one prefill unit reads (its chunk ids sit in two registers per lane).
constexpr int kPrefillMaxChunks = 128;

}  // namespace pkvt
