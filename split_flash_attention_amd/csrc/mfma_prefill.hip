// Prefill on the matrix-core kernel.
//   Selection mode: one work-group per (query row, kv head) holding every query
//   head of the group (strix-llama.cpp PR #115, Vulkan selected-key commit
//   message); the row's list is sorted and de-duplicated in LDS first.
//   Mask mode: one work-group per (block of rows, kv head); rows x heads make up
//   to 64 query vectors, the F32 mask is read per (row, key).
#include "lean_kernel.h"

#include <algorithm>

namespace selattn {
namespace {

mk::MParams common(const sel_attn_prefill_args& a) {
    mk::MParams p{};
    p.Hq = a.n_head_q; p.Hkv = a.n_head_kv; p.G = a.n_head_q / a.n_head_kv; p.D = a.head_dim;
    p.q = a.q; p.k = a.k; p.v = a.v;
    p.kv_sc = a.kv_stride_cell; p.kv_sh = a.kv_stride_head;
    p.ksc = a.k_scale; p.vsc = a.v_scale;
    p.sc_sc = a.sc_stride_cell; p.sc_sh = a.sc_stride_head;
    p.scale = a.scale; p.softcap = a.softcap; p.alibi = a.alibi_slopes;
    p.R = a.n_row; p.n_kv = a.n_kv; p.q_pos = a.q_pos; p.causal = a.causal;
    p.n_splits = a.n_splits;
    p.split_step = (a.n_kv + a.n_splits - 1) / a.n_splits;
    p.out = a.out; p.part_o = a.part_o; p.part_ml = a.part_ml;
    p.dbg_visit = a.dbg_visit; p.dbg_sel = a.dbg_sel;
    p.sinks = a.sinks;
    return p;
}

int next_pow2(int x) {
    int q = 1;
    while (q < x) q <<= 1;
    return q;
}

}  // namespace

hipError_t launch_mfma_prefill_sel(const sel_attn_prefill_args& a, hipStream_t st) {
    using namespace mk;
    MParams p = common(a);
    p.M = p.G;
    p.rows_per_wg = 1;
    const Shape sh = pick_shape(p.M);
    p.qpw = sh.waves * sh.qb * 16;
    p.sel = a.sel; p.n_sel = a.n_sel; p.bs = a.block_size; p.sel_pow2 = next_pow2(a.n_sel);
    const int nqc = (p.M + p.qpw - 1) / p.qpw;
    dim3 grid(a.n_splits, a.n_head_kv * nqc, a.n_row);
    const int64_t span = static_cast<int64_t>(a.n_kv) * a.kv_stride_cell * (a.kv_dtype == SEL_ATTN_I8 || a.kv_dtype == SEL_ATTN_FP8 ? 1 : 2);
    if (span < (int64_t{1} << 31) - 64) {
        p.qpw = 16;
        const int nqc16 = (p.M + 15) / 16;
        return lean_launch<kSel>(a.kv_dtype, p, dim3(a.n_splits, a.n_head_kv * nqc16, a.n_row), st);
    }
    return launch_mode<kSel>(a.kv_dtype, p, grid, sh, st);
}

hipError_t launch_mfma_prefill_mask(const sel_attn_prefill_args& a, hipStream_t st) {
    using namespace mk;
    MParams p = common(a);
    const int rows = std::max(1, std::min(a.n_row, 64 / std::min(p.G, 64)));
    p.rows_per_wg = rows;
    p.M = rows * p.G;
    const Shape sh = pick_shape(p.M);
    p.qpw = sh.waves * sh.qb * 16;
    p.mask = a.mask; p.m_sr = a.mask_stride_row; p.m_sh = a.mask_stride_head;
    const int nqc = (p.M + p.qpw - 1) / p.qpw;
    const int n_rb = (a.n_row + rows - 1) / rows;
    dim3 grid(a.n_splits, a.n_head_kv * nqc, n_rb);
    return launch_mode<kMask>(a.kv_dtype, p, grid, sh, st);
}

}  // namespace selattn
