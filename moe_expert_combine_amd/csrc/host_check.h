// Host-only argument validation of the MoE combine library, shared by the
// entry points in moe_combine.hip and the exported moe_combine_check_args.
// Plain C++: no HIP header, no device call, so it builds with any host
// compiler (and under the host sanitizers).
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "moe_combine.h"

namespace moe_host {

constexpr int kMaxTopK = 32;            // slots per token (and dense inputs)
constexpr int kMaxHidden = 1 << 28;     // output rows use 32-bit byte offsets
constexpr int kMaxRmsHidden = 32768;    // one workgroup holds the whole row
constexpr int kDispatchChunk = 256;     // pairs per count chunk of the dispatch
constexpr int kMaxExperts = 4096;       // dispatch: LDS counters per workgroup

// Records a message for moe_combine_last_error() and returns st.
moe_status_t fail(moe_status_t st, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
// Clears the message and returns MOE_OK.
moe_status_t ok();

// Validates one call (sizes, required pointers, alignment, and byte-range
// overlap between what it writes and everything else it touches).
moe_status_t check_call(const moe_call_args_t &c);

// The dispatch's checks for the allocation-free entry point, whose
// workspace is the library's own device array (not checked here).
moe_status_t check_dispatch_own_scratch(const moe_call_args_t &c);

// Size checks of a kind alone (the launch description validates these).
moe_status_t check_sizes(const moe_call_args_t &c);

size_t dispatch_workspace_bytes(int64_t T, int32_t k, int32_t E);

}  // namespace moe_host
