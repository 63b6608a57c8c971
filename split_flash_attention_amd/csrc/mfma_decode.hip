// Split-K decode and verify windows on the matrix-core kernels: one work-group
// per (stream, kv head, slice[, query chunk]) (TensorFold PR #2595: the
// attn_decode grid of rows, heads and slices), partials merged by the combine.
// Up to 16 query vectors per unit run on the single-wave kernel; int8 units of more
// than 32 on the wide kernel (32-column blocks, one wave per SIMD); the others on
// the group kernel (one wave per 16 query vectors sharing each K/V tile).
#include "group_kernel.h"
#include "lean_kernel.h"
#include "wide_kernel.h"

#include <algorithm>

namespace selattn {

hipError_t launch_mfma_decode(const sel_attn_decode_args& a, hipStream_t st) {
    using namespace mk;
    MParams p{};
    p.Hq = a.n_head_q; p.Hkv = a.n_head_kv; p.G = a.n_head_q / a.n_head_kv; p.D = a.head_dim;
    p.M = a.n_row * p.G;
    p.q = a.q; p.k = a.k; p.v = a.v;
    p.kv_ss = a.kv_stride_stream; p.kv_sc = a.kv_stride_cell; p.kv_sh = a.kv_stride_head;
    p.ksc = a.k_scale; p.vsc = a.v_scale;
    p.sc_ss = a.sc_stride_stream; p.sc_sc = a.sc_stride_cell; p.sc_sh = a.sc_stride_head;
    p.scale = a.scale; p.softcap = a.softcap; p.alibi = a.alibi_slopes;
    p.R = a.n_row; p.cap = a.cap; p.kv_len = a.kv_len; p.causal = a.causal;
    p.slice_len = a.slice_len; p.n_slices_max = a.n_slices_max;
    p.part_o = a.part_o; p.part_ml = a.part_ml; p.dbg_visit = a.dbg_visit;
    p.tree = a.tree_parent;
    const int n_sl = std::min(a.n_slices_max, (a.cap + a.slice_len - 1) / a.slice_len);
    p.n_units_x = n_sl;
    p.n_units_z = a.n_stream;
    // the single-wave and group kernels address a unit's rows with 32-bit buffer offsets
    const int64_t cell_bytes = a.kv_stride_cell * (a.kv_dtype == SEL_ATTN_I8 || a.kv_dtype == SEL_ATTN_FP8 ? 1 : 2);
    const bool off32 = static_cast<int64_t>(a.cap) * cell_bytes < (int64_t{1} << 31) - 64;
    const int nqb = (p.M + 15) / 16;
    if (off32 && nqb <= 1) {
        // one block of 16 query vectors: one wave per unit
        p.qpw = 16;
        p.n_units_y = a.n_head_kv;
        return lean_launch<kDecode>(a.kv_dtype, p, dim3(n_sl, a.n_head_kv, a.n_stream), st);
    }
    const bool sc32 = static_cast<int64_t>(a.cap) * a.sc_stride_cell * 4 < (int64_t{1} << 31) - 64;
    if (off32 && sc32 && wide_eligible(a.kv_dtype, a.head_dim, p.M)) {
        // int8 verify windows: four waves of two 32-column blocks share each tile
        p.qpw = kWQ;
        const int nqc = (p.M + kWQ - 1) / kWQ;
        p.n_units_y = a.n_head_kv * nqc;
        return wide_launch(p, dim3(n_sl, a.n_head_kv * nqc, a.n_stream), st);
    }
    if (off32) {
        // many query vectors: one wave per block, a work-group shares each tile
        const int w = group_waves(nqb);
        p.qpw = 16 * w;
        const int nqc = (nqb + w - 1) / w;
        p.n_units_y = a.n_head_kv * nqc;
        return group_launch(a.kv_dtype, p, dim3(n_sl, a.n_head_kv * nqc, a.n_stream), w, st);
    }
    const Shape sh = pick_shape(p.M);
    p.qpw = sh.waves * sh.qb * 16;
    const int nqc = (p.M + p.qpw - 1) / p.qpw;
    p.n_units_y = a.n_head_kv * nqc;
    return launch_mode<kDecode>(a.kv_dtype, p, dim3(n_sl, a.n_head_kv * nqc, a.n_stream), sh, st);
}

}  // namespace selattn
