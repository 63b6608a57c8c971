// Which calls the matrix-core kernel takes, and the prefill dispatch.
#include "mfma_kernel.h"

namespace selattn {

namespace {
bool dtype_ok(int dt) {
    return dt == SEL_ATTN_BF16 || dt == SEL_ATTN_F16 || dt == SEL_ATTN_I8 || dt == SEL_ATTN_FP8;
}
}  // namespace

bool mfma_decode_eligible(const sel_attn_decode_args& a) {
    return dtype_ok(a.kv_dtype) && (a.head_dim == 128 || a.head_dim == 256);
}

bool mfma_prefill_eligible(const sel_attn_prefill_args& a) {
    const int G = a.n_head_q / a.n_head_kv;
    // selection mode: one work-group per (row, kv head) holds all G heads (up to 4 waves of 16)
    return dtype_ok(a.kv_dtype) && (a.head_dim == 128 || a.head_dim == 256) && (a.mask || G <= 64);
}

hipError_t launch_mfma_prefill(const sel_attn_prefill_args& a, hipStream_t st) {
    return a.sel ? launch_mfma_prefill_sel(a, st) : launch_mfma_prefill_mask(a, st);
}

}  // namespace selattn
