// abi_internal.h — library-internal entry points shared by the ABI's
// translation units.
#pragma once

#include <stddef.h>

#include "bdattn.h"

namespace bd {

// Body of bdattn_fwd on a given scratch of `ws_bytes` bytes (bdattn.cpp).
int fwd_impl(const bdattn_problem* problem, const bdattn_share* share, const bdattn_kv* kv,
             bdattn_tensor q_clean, bdattn_tensor q_corr, bdattn_tensor k_clean, bdattn_tensor v_clean,
             bdattn_tensor k_corr, bdattn_tensor v_corr, bdattn_tensor o, int32_t o_dtype, float* lse,
             void* workspace, size_t ws_bytes, void* hip_stream);

// Device address of the static scratch on the current device, looked up on
// the first call per device; nullptr on a HIP error (static_fwd.cpp).
void* static_scratch_ptr();

}  // namespace bd
