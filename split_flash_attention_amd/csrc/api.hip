// C-ABI layer: argument validation on the host, kernel choice, launch.
//
// Validation runs before any HIP call, so every error return leaves the
// device untouched ("launch only where the grid stays inside the buffers",
// TensorFold PR #2595 review; refusals instead of aborts, strix-llama.cpp
// PR #115 "Additional information" and TensorFold PR #985 "options the host
// cannot honor are refused").
#include <cmath>
#include <cstdint>

#include "common.h"
#include "internal.h"

namespace {

bool head_dim_ok(int d) { return d == 64 || d == 128 || d == 256; }

bool dtype_ok(int dt) {
    return dt == SEL_ATTN_F32 || dt == SEL_ATTN_F16 || dt == SEL_ATTN_BF16 || dt == SEL_ATTN_I8 ||
           dt == SEL_ATTN_FP8;
}

int elem_bytes(int dt) {
    switch (dt) {
    case SEL_ATTN_F32: return 4;
    case SEL_ATTN_I8:
    case SEL_ATTN_FP8: return 1;
    default: return 2;
    }
}

// 1-byte rows that carry one fp32 scale per (cell, kv head) row
bool scaled(int dt) { return dt == SEL_ATTN_I8 || dt == SEL_ATTN_FP8; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool stride16(int64_t s, int dt) { return s > 0 && (s * elem_bytes(dt)) % 16 == 0; }

int check_scores(float scale, float softcap) {
    if (!std::isfinite(scale)) return SEL_ATTN_EUNSUPPORTED;
    if (!std::isfinite(softcap) || softcap < 0.f) return SEL_ATTN_EUNSUPPORTED;
    return SEL_ATTN_OK;
}

}  // namespace

namespace selattn {

int validate_decode(const sel_attn_decode_args* a) {
    if (!a) return SEL_ATTN_EINVAL;
    if (!a->q || !a->k || !a->v || !a->kv_len || !a->part_o || !a->part_ml) return SEL_ATTN_EINVAL;
    if (a->n_stream <= 0 || a->n_row <= 0 || a->n_head_q <= 0 || a->n_head_kv <= 0 ||
        a->head_dim <= 0 || a->cap <= 0 || a->slice_len <= 0 || a->n_slices_max <= 0)
        return SEL_ATTN_EINVAL;
    if (a->n_head_q % a->n_head_kv != 0) return SEL_ATTN_EINVAL;
    if (!dtype_ok(a->kv_dtype)) return SEL_ATTN_EUNSUPPORTED;
    if (scaled(a->kv_dtype) && (!a->k_scale || !a->v_scale)) return SEL_ATTN_EINVAL;
    if (scaled(a->kv_dtype) &&
        (a->sc_stride_stream < 0 || a->sc_stride_cell < 0 || a->sc_stride_head < 0))
        return SEL_ATTN_EINVAL;
    if (!head_dim_ok(a->head_dim)) return SEL_ATTN_EUNSUPPORTED;
    int s = check_scores(a->scale, a->softcap);
    if (s) return s;
    if (!aligned16(a->k) || !aligned16(a->v) || !stride16(a->kv_stride_stream, a->kv_dtype) ||
        !stride16(a->kv_stride_cell, a->kv_dtype) || !stride16(a->kv_stride_head, a->kv_dtype))
        return SEL_ATTN_EUNSUPPORTED;
    if (!aligned16(a->q) || !aligned16(a->part_o)) return SEL_ATTN_EUNSUPPORTED;
    if (static_cast<int64_t>(a->n_slices_max) * a->slice_len < a->cap) return SEL_ATTN_EWORKSPACE;
    if (static_cast<int64_t>(a->n_stream) * a->n_slices_max > 0x7fffffffLL) return SEL_ATTN_EUNSUPPORTED;
    if (a->tree_parent && a->n_row > 64) return SEL_ATTN_EUNSUPPORTED;   // one 64-bit path mask per row
    return SEL_ATTN_OK;
}

int validate_combine(const sel_attn_combine_args* a) {
    if (!a) return SEL_ATTN_EINVAL;
    if (!a->part_o || !a->part_ml || !a->out) return SEL_ATTN_EINVAL;
    if (a->n_stream <= 0 || a->n_row <= 0 || a->n_head_q <= 0 || a->head_dim <= 0 ||
        a->n_slices_max <= 0)
        return SEL_ATTN_EINVAL;
    if (a->kv_len && (a->slice_len <= 0 || a->cap <= 0)) return SEL_ATTN_EINVAL;
    if (!head_dim_ok(a->head_dim)) return SEL_ATTN_EUNSUPPORTED;
    if (!aligned16(a->part_o) || !aligned16(a->out)) return SEL_ATTN_EUNSUPPORTED;
    if ((reinterpret_cast<uintptr_t>(a->part_ml) & 7u) != 0) return SEL_ATTN_EUNSUPPORTED;
    if (static_cast<int64_t>(a->n_stream) * a->n_row * a->n_head_q > 0x7fffffffLL)
        return SEL_ATTN_EUNSUPPORTED;
    return SEL_ATTN_OK;
}

}  // namespace selattn

namespace {

using selattn::validate_combine;
using selattn::validate_decode;

int validate_prefill(const sel_attn_prefill_args* a) {
    if (!a) return SEL_ATTN_EINVAL;
    if (!a->q || !a->k || !a->v) return SEL_ATTN_EINVAL;
    if ((a->sel != nullptr) == (a->mask != nullptr)) return SEL_ATTN_EINVAL;
    if (a->n_row <= 0 || a->n_head_q <= 0 || a->n_head_kv <= 0 || a->head_dim <= 0 ||
        a->n_kv <= 0 || a->n_splits < 1)
        return SEL_ATTN_EINVAL;
    if (a->n_head_q % a->n_head_kv != 0) return SEL_ATTN_EINVAL;
    if (a->n_splits == 1 && !a->out) return SEL_ATTN_EINVAL;
    if (a->n_splits > 1 && (!a->part_o || !a->part_ml)) return SEL_ATTN_EINVAL;
    if (!dtype_ok(a->kv_dtype)) return SEL_ATTN_EUNSUPPORTED;
    if (scaled(a->kv_dtype) && (!a->k_scale || !a->v_scale)) return SEL_ATTN_EINVAL;
    if (scaled(a->kv_dtype) && (a->sc_stride_cell < 0 || a->sc_stride_head < 0))
        return SEL_ATTN_EINVAL;
    if ((a->alibi_slopes || (a->mask && a->causal)) && !a->q_pos) return SEL_ATTN_EINVAL;
    if (a->sel) {
        if (a->n_sel < 1 || a->n_sel > 4096 || a->block_size < 1) return SEL_ATTN_EINVAL;
    } else {
        if (a->mask_stride_row <= 0 || a->mask_stride_head < 0) return SEL_ATTN_EINVAL;
    }
    if (!head_dim_ok(a->head_dim)) return SEL_ATTN_EUNSUPPORTED;
    if (a->n_head_q / a->n_head_kv > 32) return SEL_ATTN_EUNSUPPORTED;
    if (a->n_splits > 65535) return SEL_ATTN_EUNSUPPORTED;
    int s = check_scores(a->scale, a->softcap);
    if (s) return s;
    if (!aligned16(a->k) || !aligned16(a->v) || !stride16(a->kv_stride_cell, a->kv_dtype) ||
        !stride16(a->kv_stride_head, a->kv_dtype))
        return SEL_ATTN_EUNSUPPORTED;
    if (!aligned16(a->q) || !aligned16(a->out) || !aligned16(a->part_o)) return SEL_ATTN_EUNSUPPORTED;
    // Selection mode runs only on the matrix-core kernel (16-bit or int8 K/V,
    // head dim 128 or 256); the generic kernel does not take it.
    if (a->sel && !selattn::mfma_prefill_eligible(*a)) return SEL_ATTN_EUNSUPPORTED;
    return SEL_ATTN_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? SEL_ATTN_OK : SEL_ATTN_EHIP; }

}  // namespace

extern "C" {

int sel_attn_abi_version(void) { return SEL_ATTN_ABI_VERSION; }

size_t sel_attn_args_size(int op) {
    switch (op) {
    case SEL_ATTN_OP_DECODE: return sizeof(sel_attn_decode_args);
    case SEL_ATTN_OP_PREFILL: return sizeof(sel_attn_prefill_args);
    case SEL_ATTN_OP_COMBINE: return sizeof(sel_attn_combine_args);
    default: return 0;
    }
}

const char* sel_attn_strerror(int status) {
    switch (status) {
    case SEL_ATTN_OK: return "ok";
    case SEL_ATTN_EINVAL: return "invalid argument";
    case SEL_ATTN_EUNSUPPORTED: return "unsupported argument combination";
    case SEL_ATTN_EWORKSPACE: return "partial buffer too small for the slices";
    case SEL_ATTN_EHIP: return "HIP runtime error at launch";
    default: return "unknown status";
    }
}

int sel_attn_decode_workspace(const sel_attn_decode_args* a, size_t* part_o_bytes,
                              size_t* part_ml_bytes) {
    if (!a || a->n_stream <= 0 || a->n_row <= 0 || a->n_head_q <= 0 || a->head_dim <= 0 ||
        a->cap <= 0 || a->slice_len <= 0)
        return SEL_ATTN_EINVAL;
    const size_t ns = static_cast<size_t>((a->cap + a->slice_len - 1) / a->slice_len);
    const size_t units = static_cast<size_t>(a->n_stream) * a->n_row * a->n_head_q * ns;
    if (part_o_bytes) *part_o_bytes = units * a->head_dim * sizeof(float);
    if (part_ml_bytes) *part_ml_bytes = units * 2 * sizeof(float);
    return SEL_ATTN_OK;
}

int sel_attn_supports(int op, const void* args) {
    switch (op) {
    case SEL_ATTN_OP_DECODE:
        return validate_decode(static_cast<const sel_attn_decode_args*>(args)) == SEL_ATTN_OK;
    case SEL_ATTN_OP_PREFILL:
        return validate_prefill(static_cast<const sel_attn_prefill_args*>(args)) == SEL_ATTN_OK;
    case SEL_ATTN_OP_COMBINE:
        return validate_combine(static_cast<const sel_attn_combine_args*>(args)) == SEL_ATTN_OK;
    default: return 0;
    }
}

int sel_attn_decode_path(const sel_attn_decode_args* a) {
    int s = validate_decode(a);
    if (s) return s;
    return selattn::mfma_decode_eligible(*a) ? 1 : 0;
}

int sel_attn_prefill_path(const sel_attn_prefill_args* a) {
    int s = validate_prefill(a);
    if (s) return s;
    return selattn::mfma_prefill_eligible(*a) ? 1 : 0;
}

int sel_attn_decode(const sel_attn_decode_args* a, void* hip_stream) {
    int s = validate_decode(a);
    if (s) return s;
    hipStream_t st = static_cast<hipStream_t>(hip_stream);
    if (selattn::mfma_decode_eligible(*a)) return hip_status(selattn::launch_mfma_decode(*a, st));
    return hip_status(selattn::launch_valu_decode(*a, st));
}

int sel_attn_split_combine(const sel_attn_combine_args* a, void* hip_stream) {
    int s = validate_combine(a);
    if (s) return s;
    return hip_status(selattn::launch_combine(*a, static_cast<hipStream_t>(hip_stream)));
}

int sel_attn_prefill(const sel_attn_prefill_args* a, void* hip_stream) {
    int s = validate_prefill(a);
    if (s) return s;
    hipStream_t st = static_cast<hipStream_t>(hip_stream);
    if (selattn::mfma_prefill_eligible(*a)) return hip_status(selattn::launch_mfma_prefill(*a, st));
    return hip_status(selattn::launch_valu_prefill(*a, st));
}

}  // extern "C"
