// Internal launch interface between the C-ABI layer (api.hip) and the kernel
// translation units.  Arguments reaching these functions are validated.
#pragma once

#include <hip/hip_runtime.h>

#include "../../include/sel_attn.h"

namespace selattn {

// Host-side argument checks of the C ABI (status codes of include/sel_attn.h).
int validate_decode(const sel_attn_decode_args* a);
int validate_combine(const sel_attn_combine_args* a);

// Generic vector-ALU kernels (every dtype, every supported shape).
hipError_t launch_valu_decode(const sel_attn_decode_args& a, hipStream_t st);
hipError_t launch_valu_prefill(const sel_attn_prefill_args& a, hipStream_t st);
hipError_t launch_combine(const sel_attn_combine_args& a, hipStream_t st);

// Matrix-core kernels.  `*_eligible` says whether the MFMA kernel takes the
// validated arguments; the launchers assume it does.
bool mfma_decode_eligible(const sel_attn_decode_args& a);
hipError_t launch_mfma_decode(const sel_attn_decode_args& a, hipStream_t st);
bool mfma_prefill_eligible(const sel_attn_prefill_args& a);
hipError_t launch_mfma_prefill(const sel_attn_prefill_args& a, hipStream_t st);
hipError_t launch_mfma_prefill_sel(const sel_attn_prefill_args& a, hipStream_t st);
hipError_t launch_mfma_prefill_mask(const sel_attn_prefill_args& a, hipStream_t st);

}  // namespace selattn
