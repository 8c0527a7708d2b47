// Shared host-side helpers of the pkv library: status codes, thread-local error text.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdint>

#include "pkv.h"

namespace pkv {

// Record a formatted message as this thread's last error and return `code`.
int fail(int code, const char *fmt, ...) __attribute__((format(printf, 2, 3)));

// PKV_OK if e == hipSuccess, else PKV_EHIP with the runtime's message.
int hip_status(hipError_t e, const char *what);

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

inline bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline int elt_bytes(int32_t dtype) { return dtype == PKV_F32 ? 4 : 2; }

inline bool valid_dtype(int32_t dtype) { return dtype == PKV_F32 || dtype == PKV_F16 || dtype == PKV_BF16; }

// PKV_DEBUG_VALIDATE set (and not "0"): the entry points check the device-side contract on
// host copies before launching.
bool debug_validate();

// Lengths within [0, max_context_len] (and lmax when block_tables is NULL: the contiguous
// layout), at most max_blocks blocks, every used table entry inside [0, num_blocks).
// Synchronises `stream`; PKV_EINVAL with a message on the first violation.
// PKV_DEBUG_VALIDATE: PKV_EINVAL unless dev points into device memory.
int validate_device_array(const char *fn, const char *what, const void *dev);
// PKV_DEBUG_VALIDATE for a decode step with the cache write: each non-negative slot_mapping[s] is
// the slot of position context_lens[s] - 1 through the block table.
int validate_step_slots(const char *fn, const int64_t *slot_mapping, const int32_t *context_lens,
                        const int32_t *block_tables, int32_t num_seqs, int32_t max_blocks, int32_t block_size,
                        hipStream_t stream);
int validate_attention(const char *fn, const int32_t *context_lens, int32_t num_seqs, int32_t max_context_len,
                       const int32_t *block_tables, int32_t max_blocks, int32_t block_size, int64_t num_blocks,
                       int32_t lmax, hipStream_t stream);

// query_start[0] = 0, each sequence's query count in [0, min(max_query_len, its length)] and
// query_start[num_seqs] <= num_tokens. Synchronises `stream`.
int validate_query_start(const char *fn, const int32_t *query_start, const int32_t *context_lens, int32_t num_seqs,
                         int32_t num_tokens, int32_t max_query_len, hipStream_t stream);

// Slots below num_slots and no non-negative slot twice. Synchronises `stream`.
int validate_slots(const char *fn, const int64_t *slot_mapping, int32_t num_tokens, int64_t num_slots,
                   hipStream_t stream);

}  // namespace pkv
