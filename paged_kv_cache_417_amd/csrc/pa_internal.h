// pa_internal.h — shared helpers of libpa's host code (not part of the ABI).
#pragma once

#include <cstdarg>
#include <cstdint>

#include "pa.h"

namespace pa {

// Record a message for pa_last_error() on this thread and return `st`.
pa_status fail(pa_status st, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
// Clear this thread's message and return PA_OK.
pa_status ok();

// The allocator's positions per block.
int32_t block_size(const pa_allocator *a);

// Default decode partition size (pa_decode_default_partition).
int32_t default_partition(int32_t num_seqs, int32_t num_kv_heads, int32_t block_size,
                          int32_t max_context_len);

}  // namespace pa
