// Matrix-core split-K decode kernel for verify windows with int8 K/V: units of
// many query vectors (16 draft rows x 12 heads = 192 per (stream, slice, kv head)
// for the int8 verify workload), on v_mfma_f32_32x32x16_bf16 with one wave per
// SIMD (TensorFold PR #2595: one work-group per (stream, kv head, slice) of the
// attn_decode grid; partials merged by the log-sum-exp combine afterwards).
//
// Four waves share each 32-key tile of K and V^T, widened to bf16 in LDS and
// double-buffered.  Wave w owns the 32-column blocks w and w + 4 of its query
// chunk (up to 64 query vectors; 256 per work-group): their Q^T operands stay in
// registers and their O^T accumulators (256 values a lane) beside them.  Per tile:
//   * S^T[key][qv] = K . Q^T over D / 16 steps of 16 dims.  A lane ends up with 16
//     scores of ONE query vector (lane l & 31 of the block); the tile's other 16
//     keys of that query vector sit in lane l ^ 32.
//   * one online-softmax step with lazy rescaling (TensorFold PR #985, "What this
//     changes": running maximum, correction exp(m_old - m_new) applied to l and o):
//     the exponent reference moves only when a score passes it by kLazy, the true
//     maximum is applied once at the end.
//   * O^T[dim][qv] += V^T . P^T over the tile's two 16-key halves; the lane's own
//     weights (times the V row scale) are its P^T operand, because V^T is stored
//     in that contraction order.
// Register budget (one wave per SIMD: 256 VGPRs and 256 AGPRs): the accumulators
// fill the AGPRs; block 0's Q^T operands live in VGPRs and block 1's in this
// wave's part of LDS.  Operand reads run two steps ahead of their products, each
// step fenced by a scheduling barrier so that the reads of a phase are not all
// issued at once, and the rare rescale of the accumulators goes through a short
// AGPR sequence (read, multiply, write back) so that they never leave the AGPRs.
// K rows are padded by 16 bytes: one base register plus an immediate addresses
// every step, and the 32 rows of an operand read fall on distinct bank groups.
// A key no query vector of the chunk can see is never loaded; keys some query
// vectors see and others don't are excluded per score (int8 V is always finite
// and its row scale joins visible weights only).
#pragma once

#include <type_traits>

#include "mfma_kernel.h"

namespace selattn {
namespace mk {

constexpr int kWT = 32;          // keys per tile
constexpr int kWW = 4;           // waves per work-group
constexpr int kWQ = 64 * kWW;    // query vectors per work-group: two 32-column blocks a wave

typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ f32x16 mfma32x32x16(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                   c, 0, 0, 0);
}

// The score products, with their accumulator pinned to VGPRs: the O^T accumulators
// take all 256 AGPRs, and the compiler would otherwise place every matrix
// accumulator in AGPRs.  Because the compiler does not look inside the asm, the
// asm supplies the wait states it would insert itself: 2 after a vector ALU write
// of an operand (the leading s_nop 1), and, once a chain ends, 16 before anything
// reads the result (wide_mfma_drain; the 8-pass instruction needs 11).  Products
// chained on the same accumulator need none.
__device__ __forceinline__ void mfma_v_first(f32x16& acc, const u32x4& a, const u32x4& b) {
    asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_v(f32x16& acc, const u32x4& a, const u32x4& b) {
    asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void wide_mfma_drain(f32x16& s) {
    asm volatile("s_nop 7\n\ts_nop 7" : "+v"(s));
}

// LDS of one tile buffer: K [32 keys][D] bf16 in rows padded by 16 bytes; V^T
// [4 groups][D dims][8 keys] bf16; the tile's K and V row scales.
template <int D>
constexpr int wide_krow() { return D * 2 + 16; }
template <int D>
constexpr int wide_buf_bytes() { return kWT * wide_krow<D>() + D * kWT * 2 + 2 * kWT * 4; }
// two tile buffers, each wave's block-1 Q^T operands (D / 16 steps x 1 KiB), the
// tree path masks and the visit counters of the 256 query vectors
template <int D>
constexpr int wide_smem() { return 2 * wide_buf_bytes<D>() + kWW * (D / 16) * 1024 + kWQ * 8 + kWQ * 3 * 8; }

// Key of score i (0..15) of a lane in half h of the wave: 8 (i / 4) + 4 h + i % 4.
// Contraction chunk c of P.V takes the lane's scores 8c .. 8c + 7, i.e. the keys of
// V^T group 2c + h in this order.
__device__ __forceinline__ int wide_key(int i, int h) { return 8 * (i >> 2) + 4 * h + (i & 3); }

// byte offset of 16-byte chunk ch (dims 8 ch .. 8 ch + 7) of key row `key` in the K tile
template <int D>
__device__ __forceinline__ int wk_off(int key, int ch) { return key * wide_krow<D>() + (ch << 4); }

// o *= c for an accumulator held in an AGPR: read into a VGPR, multiply, write back
// (keeps the accumulators in the AGPRs through the rare rescale)
__device__ __forceinline__ void agpr_scale(float& o, float c) {
    float t;
    asm volatile("v_accvgpr_read_b32 %1, %0\n\tv_mul_f32 %1, %1, %2\n\tv_accvgpr_write_b32 %0, %1"
                 : "+a"(o), "=&v"(t)
                 : "v"(c));
}
// byte offset of the 8 keys of group g at dim d in the V^T tile
template <int D>
__device__ __forceinline__ int wv_off(int g, int d) { return (g * D + d) << 4; }

// f(integral_constant<int, i>) for i = B .. E - 1, unrolled at compile time
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        static_for<B + 1, E>(f);
    }
}

template <int KT, int D, bool TREE>
__device__ __forceinline__ void wide_unit(const MParams& p, const int t_split, const int gy, const int b,
                                          char* smem) {
    static_assert(KT == SEL_ATTN_I8, "the wide kernel widens int8 rows");
    constexpr int NS = D / 16;                   // S^T contraction steps
    constexpr int NDB = D / 32;                  // O^T dim blocks
    constexpr int NT = 64 * kWW;
    constexpr int K_TASKS = kWT * D / 16;        // 16 int8 of one key row each
    constexpr int V_TASKS = 4 * D / 4;           // (group, 4 dims): 4 bytes of 8 rows each
    constexpr int NKL = (K_TASKS + NT - 1) / NT;
    constexpr int BUF = wide_buf_bytes<D>();
    static_assert(V_TASKS <= NT, "one V task per thread at most");

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: scalar branches
    const int lane = tid & 63;
    const int l32 = lane & 31;
    const int h = lane >> 5;
    const int G = p.G;

    // this wave's block-1 Q^T operands (step st of lane l at st * 1024 + l * 16), then
    // the tree path masks and visit counters of the work-group's query vectors
    char* q1_lds = smem + 2 * BUF + wave * (NS * 1024) + lane * 16;
    unsigned long long* tpath_lds = reinterpret_cast<unsigned long long*>(smem + 2 * BUF + kWW * NS * 1024);   // [256]
    unsigned long long* dbg_lds = tpath_lds + kWQ;                                                          // [256][3]

    // ---- work unit ---------------------------------------------------------
    const int g = gy % p.Hkv;
    const int qchunk = gy / p.Hkv;
    const int kvl = min(max(p.kv_len[b], 0), p.cap);
    const int lo = t_split * p.slice_len;
    if (lo >= kvl) return;                      // uniform over the work-group
    const int hi = min(lo + p.slice_len, kvl);
    const int m_wg = qchunk * kWQ;
    const int m_end = min(p.M, m_wg + kWQ);
    const bool tree = TREE;

    // this wave's blocks: w and w + 4 of the chunk; per block, this lane's query vector
    int m0[2];
    bool live[2];
    int qv_r[2], qv_h[2], qv_lim[2];
    bool qv_ok[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        m0[k] = m_wg + 32 * (wave + 4 * k);
        live[k] = m0[k] < m_end;                 // uniform over the wave
        const int m = m0[k] + l32;
        bool ok = m < m_end;
        int r = m / G, hh = g * G + m % G;
        ok = ok && r < p.R;
        if (!ok) { r = 0; hh = g * G; }
        qv_ok[k] = ok;
        qv_r[k] = r;
        qv_h[k] = hh;
        const int pos = kvl - p.R + r;
        qv_lim[k] = ok ? min((p.causal && !tree) ? min(pos + 1, kvl) : kvl, hi) : -1;
        if constexpr (TREE) {
            // (uniform: every lane of the wave takes part in the exchanges)
            const unsigned long long path = tree_path_mask_wave(p.tree + static_cast<int64_t>(b) * p.R, p.R, r);
            if (h == 0) tpath_lds[32 * (wave + 4 * k) + l32] = path;
        }
    }

    // Q^T operands, scale folded in: step st of lane l holds Q[qv l & 31][16 st + 8 h + j],
    // j = 0..7; block 0's in registers, block 1's in this wave's part of LDS
    u32x4 qop[NS];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const float* qp = p.q + ((static_cast<int64_t>(b) * p.R + qv_r[k]) * p.Hq + qv_h[k]) * D;
#pragma unroll
        for (int st = 0; st < NS; ++st) {
            float x[8];
            if (qv_ok[k]) {
                const float4 a = *reinterpret_cast<const float4*>(qp + 16 * st + 8 * h);
                const float4 c = *reinterpret_cast<const float4*>(qp + 16 * st + 8 * h + 4);
                x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
                x[4] = c.x; x[5] = c.y; x[6] = c.z; x[7] = c.w;
            } else {
#pragma unroll
                for (int j = 0; j < 8; ++j) x[j] = 0.f;
            }
            u32x4 w;
#pragma unroll
            for (int j = 0; j < 4; ++j) w[j] = pack2<false>(x[2 * j] * p.scale, x[2 * j + 1] * p.scale);
            if (k == 0) qop[st] = w;
            else *reinterpret_cast<u32x4*>(q1_lds + st * 1024) = w;
        }
    }
    float slope[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) slope[k] = (p.alibi && qv_ok[k]) ? p.alibi[qv_h[k]] : 0.f;

    // keys no query vector of the chunk can see are never loaded (lim_max); keys
    // below lim_min are seen by every query vector of it
    int lim_max = -1, lim_min = 0x7fffffff;
    for (int rr = m_wg / G; rr <= (m_end - 1) / G && rr < p.R; ++rr) {
        const int l = (p.causal && !tree) ? min(kvl - p.R + rr + 1, kvl) : kvl;
        lim_max = max(lim_max, l);
        lim_min = min(lim_min, tree ? max(kvl - p.R, 0) : l);
    }
    const int n_keys = max(0, min(hi, lim_max) - lo);
    const int n_full = max(0, min(hi, lim_min) - lo);
    const int n_tiles = (n_keys + kWT - 1) / kWT;

    // ---- tile loads ------------------------------------------------------------
    // Buffer loads through a descriptor that starts at the unit's first key row and
    // ends with its last needed row: rows past it read as zeros (the range check
    // covers the scalar offset too, which carries the tile's and the row's part of
    // each offset).  32-bit offsets: cap * cell stride < 2^31 is checked on the host.
    const int cb = static_cast<int>(p.kv_sc);
    const int64_t kv_base = static_cast<int64_t>(b) * p.kv_ss + static_cast<int64_t>(g) * p.kv_sh;
    const int64_t sc_base = static_cast<int64_t>(b) * p.sc_ss + static_cast<int64_t>(g) * p.sc_sh;
    const char* kbase = static_cast<const char*>(p.k) + kv_base + static_cast<int64_t>(lo) * p.kv_sc;
    const char* vbase = static_cast<const char*>(p.v) + kv_base + static_cast<int64_t>(lo) * p.kv_sc;
    const int nrec = n_keys > 0 ? (n_keys - 1) * cb + D : 0;
    const __amdgpu_buffer_rsrc_t krs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(kbase), static_cast<short>(0), nrec, 0x00020000);
    const __amdgpu_buffer_rsrc_t vrs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(vbase), static_cast<short>(0), nrec, 0x00020000);

    // the unit's row scales through a descriptor of the same extent (32-bit offsets:
    // cap * scale cell stride * 4 < 2^31 is checked on the host)
    const int scb = static_cast<int>(p.sc_sc) * 4;
    const int nsc = n_keys > 0 ? (n_keys - 1) * scb + 4 : 0;
    const int64_t sc_first = sc_base + static_cast<int64_t>(lo) * p.sc_sc;
    const __amdgpu_buffer_rsrc_t ksrs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(p.ksc + sc_first), static_cast<short>(0), nsc, 0x00020000);
    const __amdgpu_buffer_rsrc_t vsrs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(p.vsc + sc_first), static_cast<short>(0), nsc, 0x00020000);

    // this thread's tasks: K chunks tid + NT i (key e / (D / 16), 16 dims e % (D / 16));
    // V task tid: group vg, dims 4 vq .. 4 vq + 3, keys 16 (vg >> 1) + 8 (j >> 2) + 4 (vg & 1) + (j & 3);
    // every thread loads the scales of key tid & 31 (threads below 32 store them).
    // The loads are unconditional where the task counts fill the work-group (no
    // masked branch, so no merge point where the compiler must assume an earlier
    // load to the same registers is still in flight); the scales go first.
    constexpr bool K_ALL = K_TASKS % NT == 0;
    constexpr bool V_ALL = V_TASKS >= NT;
    const bool has_v = V_ALL || tid < V_TASKS;
    const int vg = tid / (D / 4), vq = tid % (D / 4);
    static_assert(NT % (D / 16) == 0, "K tasks of a thread are whole rows apart");
    // per-thread parts of the load offsets; the rest is uniform (scalar offsets):
    // vg >> 1 = tid / (D / 2) is the same over a wave for D >= 128
    const int sc_voff = (tid & (kWT - 1)) * scb;
    const int k_voff = (tid / (D / 16)) * cb + (tid % (D / 16)) * 16;
    const int v_voff = 4 * (vg & 1) * cb + 4 * vq;
    const int v_hi = __builtin_amdgcn_readfirstlane(vg >> 1);
    struct Regs {
        u32x4 k[NKL];
        uint32_t v[8];
        float ks, vs;
    };
    auto load_tile = [&](Regs& rg, int t0) __attribute__((always_inline)) {
        rg.ks = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(ksrs, sc_voff, t0 * scb, 0));
        rg.vs = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(vsrs, sc_voff, t0 * scb, 0));
#pragma unroll
        for (int i = 0; i < NKL; ++i) {
            if (K_ALL || tid + i * NT < K_TASKS) {
                // task tid + i NT is task tid shifted by i NT / (D / 16) rows
                rg.k[i] = __builtin_bit_cast(
                    u32x4, __builtin_amdgcn_raw_buffer_load_b128(krs, k_voff, (t0 + i * (NT / (D / 16))) * cb, 0));
            }
        }
        if (has_v) {
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int row = t0 + 16 * v_hi + 8 * (j >> 2) + (j & 3);
                rg.v[j] = __builtin_amdgcn_raw_buffer_load_b32(vrs, v_voff, row * cb, 0);
            }
        }
    };
    // Stores tile data from rg into buffer buf, widened to bf16: part 0 / 1 the K
    // chunks, 2..5 the V^T dims 4 vq + part - 2, 6 the row scales; -1 all of them.
    auto store_tile = [&](const Regs& rg, char* buf, int part) __attribute__((always_inline)) {
        char* k_lds = buf;
        char* vt_lds = buf + kWT * wide_krow<D>();
        float* sc_lds = reinterpret_cast<float*>(vt_lds + D * kWT * 2);
#pragma unroll
        for (int i = 0; i < NKL; ++i) {
            const int e = tid + i * NT;
            if ((part < 0 || part == i) && (K_ALL || e < K_TASKS)) {
                const int key = e / (D / 16), c16 = e % (D / 16);
                const u32x4 w = rg.k[i];
                u32x4 w0, w1;
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    w0[2 * j] = kpair_bf16<KT>(w[j], 0);
                    w0[2 * j + 1] = kpair_bf16<KT>(w[j], 1);
                    w1[2 * j] = kpair_bf16<KT>(w[2 + j], 0);
                    w1[2 * j + 1] = kpair_bf16<KT>(w[2 + j], 1);
                }
                *reinterpret_cast<u32x4*>(k_lds + wk_off<D>(key, 2 * c16)) = w0;
                *reinterpret_cast<u32x4*>(k_lds + wk_off<D>(key, 2 * c16 + 1)) = w1;
            }
        }
        // dim 4 vq + dd: bytes dd of the 8 rows, as 4 bf16 pairs of consecutive keys
#pragma unroll
        for (int dd = 0; dd < 4; ++dd) {
            if ((part < 0 || part == 2 + dd) && has_v) {
                u32x4 o;
#pragma unroll
                for (int j = 0; j < 4; ++j) o[j] = bpair_bf16<KT>(rg.v[2 * j], dd, rg.v[2 * j + 1], dd);
                *reinterpret_cast<u32x4*>(vt_lds + wv_off<D>(vg, 4 * vq + dd)) = o;
            }
        }
        if ((part < 0 || part == 6) && tid < kWT) {
            sc_lds[tid] = rg.ks;
            sc_lds[kWT + tid] = rg.vs;
        }
    };
    static_assert(NKL <= 2, "K staging parts 0 and 1");
    static_assert(2 * NDB == NS, "the O^T and S^T phases have the same step count");

    // ---- running state ---------------------------------------------------------
    float m_use[2], m_true[2], l_run[2];
    f32x16 o_acc[2][NDB];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        m_use[k] = kNegInf;
        m_true[k] = kNegInf;
        l_run[k] = 0.f;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int e = 0; e < 16; ++e) o_acc[k][db][e] = 0.f;
    }
    if (p.dbg_visit && h == 0) {
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            unsigned long long* d = dbg_lds + (32 * (wave + 4 * k) + l32) * 3;
            d[0] = d[1] = d[2] = 0ull;
        }
    }
    // operand read bases: K (key l32, dims 8 h ..), V^T (group h, dim l32)
    const int kread = wk_off<D>(l32, h);
    const int vread = kWT * wide_krow<D>() + wv_off<D>(h, l32);

    // ---- online softmax of one block, in 16 stages --------------------------------
    // Stage q of block k works on the tile's scores s (lane: 16 scores of its query
    // vector, keys wide_key(i, h)); the stages are spread over the matrix products
    // of another block (below) so that the vector ALU work runs while the matrix
    // core is busy.  ksr / vsr: the tile's K and V row scales of the lane's 16 keys,
    // read once per tile for both blocks.
    float4 ksr[4], vsr[4];
    struct Smx {
        float sc[16];
        uint32_t vword;     // visibility of the tile's key slots (partial tiles)
        bool full;          // every key of the tile is seen by every query vector
        float mls;
        u32x4 pop[2];       // P^T operands of the tile's two 16-key halves
    };
    auto smx = [&](int k, auto qc, const f32x16& s, int t0, Smx& x) __attribute__((always_inline)) {
        constexpr int q = decltype(qc)::value;
        const int cell0 = lo + t0;                 // cell of key 0 of the tile
        if constexpr (q == 0) {
            x.full = t0 + kWT <= n_full;
#pragma unroll
            for (int i = 0; i < 8; ++i) x.sc[i] = s[i] * ksr[i >> 2][i & 3];
        } else if constexpr (q == 1) {
#pragma unroll
            for (int i = 8; i < 16; ++i) x.sc[i] = s[i] * ksr[i >> 2][i & 3];
        } else if constexpr (q == 2) {
            if (p.softcap > 0.f) {                  // uniform: softcap before ALiBi
#pragma unroll
                for (int i = 0; i < 16; ++i) x.sc[i] = p.softcap * tanhf(x.sc[i] / p.softcap);
            }
            if (p.alibi) {
                const int pos = kvl - p.R + qv_r[k];
#pragma unroll
                for (int i = 0; i < 16; ++i) x.sc[i] += slope[k] * static_cast<float>(cell0 + wide_key(i, h) - pos);
            }
            // bit j: key slot j of the tile is seen by this lane's query vector
            x.vword = 0xffffffffu;
            if (!x.full) {
                const int vlim = qv_lim[k] - cell0;
                x.vword = vlim >= 32 ? 0xffffffffu : (vlim <= 0 ? 0u : (1u << vlim) - 1u);
                if (tree) {
                    const unsigned long long path = tpath_lds[32 * (wave + 4 * k) + l32];
                    const int w0 = kvl - p.R - cell0;   // slot of the window's first node
                    uint32_t keep;
                    if (w0 >= 32) keep = 0xffffffffu;
                    else if (w0 >= 0) keep = ((1u << w0) - 1u) | static_cast<uint32_t>(path << w0);
                    else keep = w0 <= -64 ? 0u : static_cast<uint32_t>(path >> (-w0));
                    x.vword &= keep;
                }
                // keys not seen: score -inf (no weight, no part in the maximum)
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    if (!((x.vword >> wide_key(i, h)) & 1u)) x.sc[i] = kNegInf;
            }
        } else if constexpr (q == 3) {
            // A NaN score is left out of the maximum (v_max_f32 returns the other
            // operand) and shows up as a NaN weight, hence a NaN running sum: the NaN flag.
            float tmax = kNegInf;
#pragma unroll
            for (int i = 0; i < 16; ++i) tmax = fmaxf(tmax, x.sc[i]);
            x.mls = tmax;                           // (the tile maximum until stage 4)
            if (p.dbg_visit) {
                unsigned long long c = 0, sm = 0, sq = 0;
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    if ((x.vword >> wide_key(i, h)) & 1u) {
                        const unsigned long long cell = cell0 + wide_key(i, h);
                        c += 1;
                        sm += cell;
                        sq += cell * cell;
                    }
                }
                unsigned long long* d = dbg_lds + (32 * (wave + 4 * k) + l32) * 3;
                atomicAdd(d + 0, c);
                atomicAdd(d + 1, sm);
                atomicAdd(d + 2, sq);
            }
        } else if constexpr (q == 4) {
            float tmax = x.mls;
            tmax = fmaxf(tmax, wave_xor(tmax, 32));
            m_true[k] = fmaxf(m_true[k], tmax);
            const bool need = (tmax > m_use[k] + kLazy) || (m_use[k] == kNegInf && tmax != kNegInf);
            if (wave_any(need)) {
                const float c = need ? rescale_factor(m_use[k], tmax) : 1.f;
                if (need) m_use[k] = tmax;
                l_run[k] *= c;
#pragma unroll
                for (int db = 0; db < NDB; ++db)
#pragma unroll
                    for (int e = 0; e < 16; ++e) {
                        float y = o_acc[k][db][e];
                        agpr_scale(y, c);
                        o_acc[k][db][e] = y;
                    }
            }
            // (no key seen yet: any finite reference keeps exp2 of an excluded key's -inf at 0)
            x.mls = m_use[k] == kNegInf ? 0.f : m_use[k] * kLog2e;
        } else if constexpr (q <= 12) {
            // weights exp(s - m_use) (v_exp_f32; below 2^-126 they flush to zero) for
            // two keys; the V row scale joins the seen weights only
            const int i0 = 2 * (q - 5);
#pragma unroll
            for (int i = i0; i < i0 + 2; ++i) {
                const float w = __builtin_amdgcn_exp2f(fmaf(x.sc[i], kLog2e, -x.mls));
                l_run[k] += w;
                x.sc[i] = w * vsr[i >> 2][i & 3];
            }
        } else if constexpr (q == 13) {
            if (!x.full) {
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    if (!((x.vword >> wide_key(i, h)) & 1u)) x.sc[i] = 0.f;
            }
        } else if constexpr (q == 14) {
#pragma unroll
            for (int j = 0; j < 4; ++j) x.pop[0][j] = pack2<false>(x.sc[2 * j], x.sc[2 * j + 1]);
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) x.pop[1][j] = pack2<false>(x.sc[8 + 2 * j], x.sc[8 + 2 * j + 1]);
        }
    };
    // the softmax stages that go with matrix step ST of NS
    auto smx_step = [&](int k, auto stc, const f32x16& s, int t0, Smx& x) __attribute__((always_inline)) {
        constexpr int st = decltype(stc)::value;
        static_for<st * 16 / NS, (st + 1) * 16 / NS>([&](auto qc) { smx(k, qc, s, t0, x); });
    };

    // ---- the key loop: tile t in buffer t & 1; tile t + 1 staged during tile t -----
    Regs rg;
    if (n_tiles > 0) {
        load_tile(rg, 0);
        store_tile(rg, smem, -1);
        if (n_tiles > 1) load_tile(rg, kWT);
    }
    __syncthreads();
    // Per tile, for a wave with two blocks:
    //   P1  S^T of block 0
    //   P2  S^T of block 1, with block 0's softmax
    //   P3  O^T of block 0 += V^T . P^T, with block 1's softmax
    //   P4  O^T of block 1 += V^T . P^T, with the staging of tile t + 1 and the
    //       loads of tile t + 2
    // A wave with one block (its block 1 lies past the chunk's end) runs P1, block
    // 0's softmax, P3 and the staging.  The block count is fixed at compile time per
    // wave.  Consecutive matrix instructions never chain on one accumulator: the
    // S^T products alternate between two partial sums, the O^T products run over the
    // dim blocks first.
    auto key_loop = [&](auto two_c) __attribute__((always_inline)) {
        constexpr bool two = decltype(two_c)::value;
        for (int t = 0; t < n_tiles; ++t) {
            const char* buf = smem + (t & 1) * BUF;
            const int t0 = t * kWT;
            const bool stage_next = t + 1 < n_tiles;
            const bool load_next = t + 2 < n_tiles;
            char* nbuf = smem + ((t + 1) & 1) * BUF;
            const float* sc_lds = reinterpret_cast<const float*>(buf + kWT * wide_krow<D>() + D * kWT * 2);
            // staging part st (0..6: stores of tile t + 1; 7: loads of tile t + 2)
            auto staging = [&](auto stc) __attribute__((always_inline)) {
                constexpr int st = decltype(stc)::value;
                if constexpr (st < 7) {
                    if (stage_next) store_tile(rg, nbuf, st);
                } else if constexpr (st == 7) {
                    if (load_next) load_tile(rg, t0 + 2 * kWT);
                }
            };
            // S^T of one block; with SPLIT the steps alternate between two partial sums
            // (P1, where nothing else hides the matrix core's latency)
            auto s_phase = [&](auto split_c, f32x16& sacc, auto qsrc, auto&& per_step)
                __attribute__((always_inline)) {
                constexpr bool SPLIT = decltype(split_c)::value;
                f32x16 s2;
                u32x4 ka = *reinterpret_cast<const u32x4*>(buf + kread);
                u32x4 kb = *reinterpret_cast<const u32x4*>(buf + kread + 32);
                u32x4 qa = qsrc(0), qb = qsrc(1);
                static_for<0, NS>([&](auto stc) {
                    constexpr int st = decltype(stc)::value;
                    u32x4 kc = kb, qc = qb;
                    if constexpr (st + 2 < NS) {
                        kc = *reinterpret_cast<const u32x4*>(buf + kread + (st + 2) * 32);
                        qc = qsrc(st + 2);
                    }
                    if constexpr (st == 0) mfma_v_first(sacc, ka, qa);
                    else if constexpr (SPLIT && st == 1) mfma_v_first(s2, ka, qa);
                    else if constexpr (!SPLIT || st % 2 == 0) mfma_v(sacc, ka, qa);
                    else mfma_v(s2, ka, qa);
                    ka = kb;
                    kb = kc;
                    qa = qb;
                    qb = qc;
                    per_step(stc);
                    __builtin_amdgcn_sched_barrier(0);
                });
                wide_mfma_drain(sacc);
                if constexpr (SPLIT) {
                    wide_mfma_drain(s2);
#pragma unroll
                    for (int e = 0; e < 16; ++e) sacc[e] += s2[e];
                }
            };
            // the tile's K / V row scales of the lane's 16 keys, read shortly before a
            // block's softmax uses them (first at stage 0 / stage 5)
            auto read_ks = [&]() __attribute__((always_inline)) {
#pragma unroll
                for (int a = 0; a < 4; ++a) ksr[a] = *reinterpret_cast<const float4*>(sc_lds + 8 * a + 4 * h);
            };
            auto read_vs = [&]() __attribute__((always_inline)) {
#pragma unroll
                for (int a = 0; a < 4; ++a) vsr[a] = *reinterpret_cast<const float4*>(sc_lds + kWT + 8 * a + 4 * h);
            };
            constexpr int KS_STEP = NS - 3;       // steps ahead of the next phase
            constexpr int VS_STEP = NS / 8;       // before stage 5 of the softmax
            // O^T of block k: step i is (key half i / NDB, dim block i % NDB)
            auto vrd = [&](int i) -> u32x4 {
                return *reinterpret_cast<const u32x4*>(buf + vread + (i / NDB) * (2 * D * 16) + (i % NDB) * 512);
            };
            auto o_phase = [&](f32x16 (&oacc)[NDB], const u32x4 (&pop)[2], auto&& per_step)
                __attribute__((always_inline)) {
                u32x4 va = vrd(0), vb = vrd(1);
                static_for<0, 2 * NDB>([&](auto ic) {
                    constexpr int i = decltype(ic)::value;
                    u32x4 vc = vb;
                    if constexpr (i + 2 < 2 * NDB) vc = vrd(i + 2);
                    oacc[i % NDB] = mfma32x32x16(va, pop[i / NDB], oacc[i % NDB]);
                    va = vb;
                    vb = vc;
                    per_step(ic);
                    __builtin_amdgcn_sched_barrier(0);
                });
            };

            // P1 (and block 0's K scales)
            f32x16 s0, s1;
            s_phase(std::true_type{}, s0, [&](int st) { return qop[st]; }, [&](auto stc) {
                if constexpr (decltype(stc)::value == KS_STEP) read_ks();
            });
            // P2 (and block 0's V scales, then block 1's K scales)
            Smx x0, x1;
            if constexpr (two) {
                s_phase(std::false_type{}, s1,
                        [&](int st) { return *reinterpret_cast<const u32x4*>(q1_lds + st * 1024); },
                        [&](auto stc) {
                            constexpr int st = decltype(stc)::value;
                            smx_step(0, stc, s0, t0, x0);
                            if constexpr (st == VS_STEP) read_vs();
                            if constexpr (st == KS_STEP) read_ks();
                        });
            } else {
                read_vs();
                static_for<0, 16>([&](auto qc) { smx(0, qc, s0, t0, x0); });
            }
            // P3
            o_phase(o_acc[0], x0.pop, [&](auto ic) {
                if constexpr (two) {
                    smx_step(1, ic, s1, t0, x1);
                    if constexpr (decltype(ic)::value == VS_STEP) read_vs();
                }
            });
            // P4
            if constexpr (two) {
                o_phase(o_acc[1], x1.pop, [&](auto ic) {
                    constexpr int i = decltype(ic)::value;
                    if constexpr (i < 8) staging(ic);
                });
            } else {
                static_for<0, 8>([&](auto stc) { staging(stc); });
            }
            __syncthreads();
        }
    };
    if (live[1]) key_loop(std::true_type{});
    else key_loop(std::false_type{});

    // ---- epilogue: partials of this slice -------------------------------------
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        if (!live[k]) continue;                    // uniform
        float l = l_run[k] + wave_xor(l_run[k], 32);
        int tn = (l_run[k] != l_run[k]) ? 1 : 0;   // a NaN visible score made a running sum NaN
        tn |= wave_xor_i(tn, 32);
        const bool nan_run = tn != 0;
        unsigned long long cnt = 0, sum = 0, sq = 0;
        if (p.dbg_visit) {
            const unsigned long long* d = dbg_lds + (32 * (wave + 4 * k) + l32) * 3;
            cnt = d[0];
            sum = d[1];
            sq = d[2];
        }
        if (!qv_ok[k]) continue;
        const int r = qv_r[k], hh = qv_h[k];
        const bool bad = nan_run || m_true[k] == kPosInf;
        const bool empty = !bad && m_true[k] == kNegInf;
        float f = 1.f;
        if (!bad && !empty && m_use[k] != m_true[k]) f = exp2f((m_use[k] - m_true[k]) * kLog2e);
        l *= f;
        const int64_t pi = ((static_cast<int64_t>(b) * p.R + r) * p.Hq + hh) * p.n_slices_max + t_split;
        // lane l holds dims db * 32 + 8 a + 4 h + q of its query vector
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                float4 o;
                if (empty) o = float4{0.f, 0.f, 0.f, 0.f};
                else o = float4{o_acc[k][db][4 * a] * f, o_acc[k][db][4 * a + 1] * f, o_acc[k][db][4 * a + 2] * f,
                                o_acc[k][db][4 * a + 3] * f};
                *reinterpret_cast<float4*>(p.part_o + pi * D + db * 32 + 8 * a + 4 * h) = o;
            }
        }
        if (h == 0) {
            p.part_ml[pi * 2 + 0] = nan_run ? __builtin_nanf("") : m_true[k];
            p.part_ml[pi * 2 + 1] = bad ? __builtin_nanf("") : (empty ? 0.f : l);
        }
        if (p.dbg_visit && h == 0 && (m0[k] + l32) % G == 0) {
            const int64_t di = ((static_cast<int64_t>(b) * p.R + r) * p.Hkv + g) * p.n_slices_max + t_split;
            p.dbg_visit[di * 3 + 0] = static_cast<int64_t>(cnt);
            p.dbg_visit[di * 3 + 1] = static_cast<int64_t>(sum);
            p.dbg_visit[di * 3 + 2] = static_cast<int64_t>(sq);
        }
    }
}

template <int KT, int D, bool TREE>
__global__ __launch_bounds__(64 * kWW, 1) void wide_decode_kernel(MParams p) {
    extern __shared__ __align__(16) char smem[];
    for_each_decode_item(p, [&](int t, int gy, int bz) {
        wide_unit<KT, D, TREE>(p, t, gy, bz, smem);
        __syncthreads();                                         // LDS is reused by the next item
    });
}

template <int KT, int D, bool TREE>
hipError_t wide_launch_one(const MParams& p, dim3 grid, hipStream_t st) {
    constexpr int smem = wide_smem<D>();
    static DeviceCache cache;
    hipError_t attr = hipSuccess;
    const int resident = cache.get(0, [&attr]() {
        attr = hipFuncSetAttribute(reinterpret_cast<const void*>(&wide_decode_kernel<KT, D, TREE>),
                                   hipFuncAttributeMaxDynamicSharedMemorySize, smem);
        if (attr != hipSuccess) return 0;
        int dev = 0, cus = 0, per_cu = 0;
        if (hipGetDevice(&dev) != hipSuccess) dev = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
            cus = 256;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, wide_decode_kernel<KT, D, TREE>, 64 * kWW, smem) !=
                hipSuccess ||
            per_cu <= 0)
            per_cu = 1;
        return cus * per_cu;
    });
    if (attr != hipSuccess) return attr;
    const long long items = static_cast<long long>(grid.x) * grid.y * grid.z;
    hipLaunchKernelGGL((wide_decode_kernel<KT, D, TREE>), dim3(decode_grid(items, resident)), dim3(64 * kWW), smem,
                       st, p);
    return hipGetLastError();
}

// Decode units the wide kernel takes: int8 K/V, head dim 128 or 256, more than 32
// query vectors per (stream, kv head).
inline bool wide_eligible(int dt, int D, int M) { return dt == SEL_ATTN_I8 && (D == 128 || D == 256) && M > 32; }

// Launches the wide kernel for p (int8 K/V, D 128 or 256); defined in its own
// translation unit.
hipError_t wide_launch(const MParams& p, dim3 grid, hipStream_t st);

}  // namespace mk
}  // namespace selattn
