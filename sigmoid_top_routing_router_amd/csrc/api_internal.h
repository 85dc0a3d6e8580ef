// Internal entry points shared by the C ABI's source files.
#pragma once
#include <cstddef>
#include <cstdint>

#include "../../include/moe_mi355x.h"

namespace moe {
// moe_forward's argument checks and launch sequence.  in_order: no side
// stream and no stage timing (nothing but kernel launches and async copies on
// `stream`).
moe_status_t forward_bf16(const moe_problem_t* p, const moe_weights_t* w, const uint16_t* x,
                          const float* beta_in, uint16_t* y, moe_aux_t* aux, void* workspace,
                          size_t workspace_bytes, void* stream, bool in_order);
// Sets the thread's last error message; returns s.
moe_status_t set_error(moe_status_t s, const char* msg);
}  // namespace moe
