// Host-side helpers shared by the C ABI sources of libmsa (internal).
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "msa.h"

namespace msa {

// Every host-side check msa_decode makes except those on the workspace;
// *need gets the workspace bytes the call takes. Launches nothing.
msa_status decode_check(const msa_params* p, int32_t batch, int64_t max_ctx, const void* q, const void* q_idx,
                        const void* k_cache, const void* v_cache, const void* k_idx_cache, const int32_t* ctx_lens,
                        const void* out, const int32_t* sel_out, const float* lse_out, size_t* need);

}  // namespace msa
