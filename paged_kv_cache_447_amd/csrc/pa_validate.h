// Host-side checks of PA_FLAG_VALIDATE (see pa_validate.cpp): each returns
// PA_OK or PA_ERR_BAD_INDEX (PA_ERR_HIP if a copy fails) with the message set.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <vector>

#include "pa.h"

namespace pa {

// PA_ERR_ARG on a stream that is being captured (the checks copy and wait).
pa_status validation_allowed(hipStream_t stream);

// An I32/I64 tensor of rank 1 or 2 (non-negative strides), copied to the host
// after the stream's earlier work, in row-major order.
struct HostInts {
  std::vector<int64_t> v;
  int64_t rows = 0, cols = 0;
  pa_status fetch(const pa_tensor &t, const char *name, hipStream_t stream);
  int64_t at(int64_t r, int64_t c = 0) const { return v[(size_t)(r * cols + c)]; }
};

// Context lengths within [0, table width * block_size], and the table entries
// that cover each context within [0, num_blocks).
pa_status check_tables(const HostInts &block_tables, const HostInts &context_lens, int64_t block_size,
                       int64_t num_blocks);
// A fused step's slots: each written slot is its sequence's position L - 1,
// and no two sequences write one slot.
pa_status check_new_token_slots(const HostInts &slots, const HostInts &block_tables, const HostInts &context_lens,
                                int64_t block_size, int64_t num_slots);
// A cache write's slots inside the pool are distinct.
pa_status check_distinct_slots(const HostInts &slots, int64_t num_slots);
// query_start_loc: 0, non-decreasing, ending at num_rows; no sequence has
// more query rows than context.
pa_status check_query_starts(const HostInts &query_start_loc, const HostInts &context_lens, int64_t num_rows);
// Block pairs: distinct destinations; in one pool no destination is a source.
pa_status check_block_pairs(const HostInts &mapping, int64_t src_blocks, int64_t dst_blocks, bool same_pool);
// Per-kv-head (or per-block) scales (n of each, device or pinned host
// memory): finite and > 0.  The names are those the message gives.
pa_status check_head_scales(const float *k_head_scales, const float *v_head_scales, int64_t n, hipStream_t stream,
                            const char *k_name = "k_head_scales", const char *v_name = "v_head_scales");

}  // namespace pa
