// Matrix-core (MFMA) flash attention for gfx950: split-K decode / verify
// windows and prefill in selection or mask mode, for bf16, fp16 and int8 K/V.
//
// A query vector is one (row, query head) pair of one kv head.  A wave owns QB
// blocks of 16 query vectors; the W waves of a work-group share each 32-key
// tile of K and V staged in LDS:
//   * K tile  [32 keys][D] 16-bit, 16-byte chunks XOR-swizzled by key;
//   * V tile  transposed [D][32], keys in the contraction order of P^T below.
// Scores are computed transposed, S^T[key][qv] = K . Q^T (one MFMA per 16 keys
// x 32 dims), so each lane ends up holding 8 scores of ONE query vector.  The
// online softmax of TensorFold PR #985 ("What this changes": running max per
// fixed key tile, correction exp(m_old - m_new), l and o rescaled) then needs
// only two cross-lane max exchanges per tile, and the lane's own 8 weights ARE
// its P^T operand for O^T[dim][qv] += V^T . P^T (no data movement).
//
// Key sources: a contiguous slice (decode, TensorFold PR #2595: one
// work-group per (stream, kv head, slice), partials merged afterwards), a
// contiguous range with an F32 mask (HartsyInference PR #910), or the sorted,
// de-duplicated selection list gathered in 32-cell tiles (strix-llama.cpp
// PR #115, Vulkan selected-key commit message: one work-group per query x kv
// head, list sorted in shared memory, invalid and repeated ids skipped).
// Keys a query vector cannot see get weight 0 and are never loaded when no
// query vector of the work-group sees them.
#include "arch.h"
#include "common.h"
#include "internal.h"

#include <algorithm>

namespace selattn {
namespace {

constexpr int kTK = 32;          // keys per tile
constexpr int kMaxSelM = 4096;   // longest selection list

enum Mode : int { kDecode = 0, kMask = 1, kSel = 2 };

struct MParams {
    int mode;
    int Hq, Hkv, G, D;
    int M;               // query vectors per (unit, kv head): R*G (decode), G (sel), rows*G (mask)
    int qpw;             // query vectors per work-group = W * QB * 16
    const float* q;
    const void* k;
    const void* v;
    int64_t kv_ss, kv_sc, kv_sh;
    const float* ksc;
    const float* vsc;
    int64_t sc_ss, sc_sc, sc_sh;
    float scale, softcap;
    const float* alibi;
    // decode
    int R, cap;
    const int32_t* kv_len;
    int causal;
    int slice_len, n_slices_max;
    // prefill
    int n_kv;
    const int32_t* q_pos;
    const int32_t* sel;
    int n_sel, bs, sel_pow2;
    const float* mask;
    int64_t m_sr, m_sh;
    int rows_per_wg, n_splits, split_step;
    // outputs
    float* out;
    float* part_o;
    float* part_ml;
    int64_t* dbg_visit;
    int32_t* dbg_sel;
};

// ---------------------------------------------------------------------------
// 16-bit conversions and LDS addressing
// ---------------------------------------------------------------------------
template <bool F16>
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    uint16_t a, b;
    if constexpr (F16) {
        a = __builtin_bit_cast(uint16_t, static_cast<_Float16>(lo));
        b = __builtin_bit_cast(uint16_t, static_cast<_Float16>(hi));
    } else {
        a = __builtin_bit_cast(uint16_t, static_cast<__bf16>(lo));
        b = __builtin_bit_cast(uint16_t, static_cast<__bf16>(hi));
    }
    return static_cast<uint32_t>(a) | (static_cast<uint32_t>(b) << 16);
}

// int8 -> bf16 bits, exact for |x| <= 127
__device__ __forceinline__ uint32_t i8pair_to_bf16(int32_t word, int byte0) {
    const float f0 = static_cast<float>(static_cast<int8_t>((word >> (8 * byte0)) & 0xff));
    const float f1 = static_cast<float>(static_cast<int8_t>((word >> (8 * byte0 + 8)) & 0xff));
    return (__float_as_uint(f0) >> 16) | (__float_as_uint(f1) & 0xffff0000u);
}

// byte offset of 16-byte chunk `ch` (8 dims) of key row `key` in the K tile
__device__ __forceinline__ int k_off(int key, int ch, int D) {
    return key * D * 2 + ((ch ^ (key & 7)) << 4);
}
// byte offset of contraction chunk `cc` (8 keys) of dim row `d` in the V^T tile
__device__ __forceinline__ int vt_off(int d, int cc) {
    return d * 64 + ((cc ^ ((d >> 1) & 3)) << 4);
}

// ---------------------------------------------------------------------------
// the kernel
// ---------------------------------------------------------------------------
template <int KT, int D, int QB>
__global__ __launch_bounds__(256) void mfma_attn_kernel(MParams p) {
    constexpr bool F16 = (KT == SEL_ATTN_F16);
    constexpr int NKK = D / 32;      // contraction steps for S^T
    constexpr int NDB = D / 16;      // dim blocks of O^T
    constexpr int NCH = D / 8;       // 16-byte chunks per 16-bit K row

    extern __shared__ __align__(16) char smem[];
    char* k_lds = smem;                                   // kTK * D * 2
    char* vt_lds = smem + kTK * D * 2;                    // D * 64
    float* ksc_lds = reinterpret_cast<float*>(vt_lds + D * 64);   // kTK
    float* vsc_lds = ksc_lds + kTK;                                 // kTK
    int* cell_lds = reinterpret_cast<int*>(vsc_lds + kTK);          // kTK
    int* list = cell_lds + kTK;                                     // kMaxSelM (sel mode)

    __shared__ int s_nids;

    const int W = blockDim.x >> 6;
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int ln = lane & 15;        // query vector within a block / key row within a 16-block
    const int lg = lane >> 4;        // lane group 0..3
    const int G = p.G;

    // ---- work unit ---------------------------------------------------------
    const int t_split = blockIdx.x;
    const int g = blockIdx.y % p.Hkv;
    const int qchunk = blockIdx.y / p.Hkv;
    int b = 0, kvl = 0, lo = 0, hi = 0, row0 = 0;
    if (p.mode == kDecode) {
        b = blockIdx.z;
        kvl = min(max(p.kv_len[b], 0), p.cap);
        lo = t_split * p.slice_len;
        if (lo >= kvl) return;
        hi = min(lo + p.slice_len, kvl);
    } else {
        row0 = blockIdx.z * p.rows_per_wg;
        lo = t_split * p.split_step;
        hi = min(lo + p.split_step, p.n_kv);
    }
    const int m_wg = qchunk * p.qpw;                  // first query vector of the work-group
    const int m_wave = m_wg + wave * QB * 16;          // first of this wave

    // query vector -> (row, head, position, causal limit)
    int qv_row[QB], qv_head[QB], qv_pos[QB], qv_lim[QB];
    bool qv_ok[QB];
#pragma unroll
    for (int k = 0; k < QB; ++k) {
        const int m = m_wave + 16 * k + ln;
        qv_ok[k] = m < p.M && m < m_wg + p.qpw;
        const int mm = qv_ok[k] ? m : 0;
        int r, h;
        if (p.mode == kDecode) { r = mm / G; h = g * G + mm % G; }
        else if (p.mode == kSel) { r = row0; h = g * G + mm; }
        else { r = row0 + mm / G; h = g * G + mm % G; }
        if (p.mode != kSel && r >= (p.mode == kDecode ? p.R : min(row0 + p.rows_per_wg, p.R))) qv_ok[k] = false;
        if (!qv_ok[k]) {                  // padding: point at a real row, never used
            r = p.mode == kDecode ? 0 : row0;
            h = g * G;
        }
        qv_row[k] = r;
        qv_head[k] = h;
        if (p.mode == kDecode) {
            qv_pos[k] = kvl - p.R + r;
            qv_lim[k] = p.causal ? min(qv_pos[k] + 1, kvl) : kvl;
        } else {
            qv_pos[k] = p.q_pos ? p.q_pos[r] : 0;
            qv_lim[k] = (p.mode == kMask && p.causal) ? qv_pos[k] + 1 : 0x7fffffff;
        }
        if (!qv_ok[k]) qv_lim[k] = -1;    // sees nothing
    }

    // ---- Q^T operands (scale folded in) ----------------------------------
    u32x4 qop[QB][NKK];
#pragma unroll
    for (int k = 0; k < QB; ++k) {
        const float* qp;
        if (p.mode == kDecode)
            qp = p.q + ((static_cast<int64_t>(b) * p.R + qv_row[k]) * p.Hq + qv_head[k]) * D;
        else
            qp = p.q + (static_cast<int64_t>(qv_row[k]) * p.Hq + qv_head[k]) * D;
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
            float x[8];
            if (qv_ok[k]) {
                const float4 a = *reinterpret_cast<const float4*>(qp + kk * 32 + 8 * lg);
                const float4 c = *reinterpret_cast<const float4*>(qp + kk * 32 + 8 * lg + 4);
                x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
                x[4] = c.x; x[5] = c.y; x[6] = c.z; x[7] = c.w;
            } else {
#pragma unroll
                for (int j = 0; j < 8; ++j) x[j] = 0.f;
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) qop[k][kk][j] = pack2<F16>(x[2 * j] * p.scale, x[2 * j + 1] * p.scale);
        }
    }
    float slope[QB];
#pragma unroll
    for (int k = 0; k < QB; ++k) slope[k] = (p.alibi && qv_ok[k]) ? p.alibi[qv_head[k]] : 0.f;

    // ---- selection list: sort, drop invalid and repeated ids ------------------
    int n_keys = hi - lo;           // key slots to walk
    if (p.mode == kSel) {
        const int P = p.sel_pow2;
        const int32_t* srow = p.sel + static_cast<int64_t>(row0) * p.n_sel;
        for (int e = threadIdx.x; e < P; e += blockDim.x) {
            int id = 0x7fffffff;
            if (e < p.n_sel) {
                const int x = srow[e];
                if (x >= 0 && static_cast<int64_t>(x) * p.bs < p.n_kv) id = x;
            }
            list[e] = id;
        }
        __syncthreads();
        for (int kq = 2; kq <= P; kq <<= 1) {
            for (int j = kq >> 1; j > 0; j >>= 1) {
                for (int e = threadIdx.x; e < P; e += blockDim.x) {
                    const int o = e ^ j;
                    if (o > e) {
                        const int x = list[e], y = list[o];
                        if ((x > y) == ((e & kq) == 0)) { list[e] = y; list[o] = x; }
                    }
                }
                __syncthreads();
            }
        }
        // in-place compaction: a single pass by thread 0 keeps the order stable
        if (threadIdx.x == 0) {
            int w = 0;
            int prev = -1;
            for (int e = 0; e < P; ++e) {
                const int x = list[e];
                if (x == 0x7fffffff) break;
                if (x != prev) list[w++] = x;
                prev = x;
            }
            s_nids = w;
        }
        __syncthreads();
        const int n_ids = s_nids;
        if (p.dbg_sel && t_split == 0) {
            int32_t* dst = p.dbg_sel + (static_cast<int64_t>(row0) * p.Hkv + g) * (1 + p.n_sel);
            if (threadIdx.x == 0) dst[0] = n_ids;
            for (int e = threadIdx.x; e < n_ids; e += blockDim.x) dst[1 + e] = list[e];
        }
        n_keys = n_ids * p.bs;
    }
    // decode / mask: no query vector of this work-group sees keys at or past the largest limit
    if (p.mode != kSel) {
        int lim_max = -1;
        const int m_end = min(p.M, m_wg + p.qpw);
        if (m_end > m_wg) {
            const int r_first = (p.mode == kDecode ? 0 : row0) + m_wg / G;
            const int r_last = (p.mode == kDecode ? 0 : row0) + (m_end - 1) / G;
            for (int r = r_first; r <= r_last && r < p.R; ++r) {
                int l;
                if (p.mode == kDecode) l = p.causal ? min(kvl - p.R + r + 1, kvl) : kvl;
                else l = p.causal ? (p.q_pos[r] + 1) : hi;
                lim_max = max(lim_max, l);
            }
        }
        n_keys = max(0, min(hi, lim_max) - lo);
    }

    // ---- running state ---------------------------------------------------------
    float m_run[QB], l_run[QB];
    bool nan_run[QB];
    f32x4 o_acc[QB][NDB];
    long long dbg_cnt[QB], dbg_sum[QB], dbg_sq[QB];
#pragma unroll
    for (int k = 0; k < QB; ++k) {
        m_run[k] = kNegInf;
        l_run[k] = 0.f;
        nan_run[k] = false;
        dbg_cnt[k] = dbg_sum[k] = dbg_sq[k] = 0;
#pragma unroll
        for (int db = 0; db < NDB; ++db) o_acc[k][db] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    const int64_t kv_base = (p.mode == kDecode ? static_cast<int64_t>(b) * p.kv_ss : 0) +
                            static_cast<int64_t>(g) * p.kv_sh;
    const int64_t sc_base = (p.mode == kDecode ? static_cast<int64_t>(b) * p.sc_ss : 0) +
                            static_cast<int64_t>(g) * p.sc_sh;

    for (int t0 = 0; t0 < n_keys; t0 += kTK) {
        // ---- cells of this tile (-1: nothing there) ----
        if (threadIdx.x < kTK) {
            const int kslot = t0 + threadIdx.x;
            int c = -1;
            if (kslot < n_keys) {
                if (p.mode == kSel) {
                    const int cc = list[kslot / p.bs] * p.bs + kslot % p.bs;
                    c = (cc < p.n_kv && cc >= lo && cc < hi) ? cc : -1;
                } else {
                    c = lo + kslot;
                }
            }
            cell_lds[threadIdx.x] = c;
        }
        __syncthreads();

        // ---- stage K (row-major, swizzled) ----
        if constexpr (KT == SEL_ATTN_I8) {
            // 16 int8 per load -> two 16-byte bf16 chunks
            for (int e = threadIdx.x; e < kTK * (D / 16); e += blockDim.x) {
                const int key = e / (D / 16), c16 = e % (D / 16);
                const int cell = cell_lds[key];
                u32x4 w0 = {0u, 0u, 0u, 0u}, w1 = {0u, 0u, 0u, 0u};
                if (cell >= 0) {
                    const int4 raw = *reinterpret_cast<const int4*>(
                        static_cast<const int8_t*>(p.k) + kv_base + cell * p.kv_sc + c16 * 16);
                    w0 = u32x4{i8pair_to_bf16(raw.x, 0), i8pair_to_bf16(raw.x, 2),
                               i8pair_to_bf16(raw.y, 0), i8pair_to_bf16(raw.y, 2)};
                    w1 = u32x4{i8pair_to_bf16(raw.z, 0), i8pair_to_bf16(raw.z, 2),
                               i8pair_to_bf16(raw.w, 0), i8pair_to_bf16(raw.w, 2)};
                }
                *reinterpret_cast<u32x4*>(k_lds + k_off(key, 2 * c16, D)) = w0;
                *reinterpret_cast<u32x4*>(k_lds + k_off(key, 2 * c16 + 1, D)) = w1;
            }
            if (threadIdx.x < kTK) {
                const int cell = cell_lds[threadIdx.x];
                ksc_lds[threadIdx.x] = cell >= 0 ? p.ksc[sc_base + cell * p.sc_sc] : 0.f;
                vsc_lds[threadIdx.x] = cell >= 0 ? p.vsc[sc_base + cell * p.sc_sc] : 0.f;
            }
        } else {
            for (int e = threadIdx.x; e < kTK * NCH; e += blockDim.x) {
                const int key = e / NCH, ch = e % NCH;
                const int cell = cell_lds[key];
                u32x4 w = {0u, 0u, 0u, 0u};
                if (cell >= 0)
                    w = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(p.k) + kv_base +
                                                        cell * p.kv_sc + ch * 8);
                *reinterpret_cast<u32x4*>(k_lds + k_off(key, ch, D)) = w;
            }
        }
        // ---- stage V transposed: 4 consecutive keys x 8 (or 16) dims per task ----
        if constexpr (KT == SEL_ATTN_I8) {
            for (int e = threadIdx.x; e < 8 * (D / 16); e += blockDim.x) {
                const int kg = e / (D / 16), c16 = e % (D / 16);     // key group of 4, 16-dim chunk
                int4 raw[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int cell = cell_lds[4 * kg + i];
                    raw[i] = cell >= 0 ? *reinterpret_cast<const int4*>(static_cast<const int8_t*>(p.v) +
                                                                        kv_base + cell * p.kv_sc + c16 * 16)
                                       : int4{0, 0, 0, 0};
                }
                const int kb = kg >> 2, gq = kg & 3;      // key = kb*16 + 4*gq + i
#pragma unroll
                for (int dd = 0; dd < 16; ++dd) {
                    uint32_t lohi[2];
#pragma unroll
                    for (int h2 = 0; h2 < 2; ++h2) {
                        int32_t w0 = (&raw[2 * h2].x)[dd >> 2];
                        int32_t w1 = (&raw[2 * h2 + 1].x)[dd >> 2];
                        const float f0 = static_cast<float>(static_cast<int8_t>((w0 >> (8 * (dd & 3))) & 0xff));
                        const float f1 = static_cast<float>(static_cast<int8_t>((w1 >> (8 * (dd & 3))) & 0xff));
                        lohi[h2] = (__float_as_uint(f0) >> 16) | (__float_as_uint(f1) & 0xffff0000u);
                    }
                    const int d = c16 * 16 + dd;
                    *reinterpret_cast<uint2*>(vt_lds + vt_off(d, gq) + 8 * kb) = uint2{lohi[0], lohi[1]};
                }
            }
        } else {
            for (int e = threadIdx.x; e < 8 * NCH; e += blockDim.x) {
                const int kg = e / NCH, ch = e % NCH;
                u32x4 raw[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int cell = cell_lds[4 * kg + i];
                    raw[i] = cell >= 0 ? *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(p.v) +
                                                                         kv_base + cell * p.kv_sc + ch * 8)
                                       : u32x4{0u, 0u, 0u, 0u};
                }
                const int kb = kg >> 2, gq = kg & 3;
#pragma unroll
                for (int dd = 0; dd < 8; ++dd) {
                    const int wsel = dd >> 1;
                    const bool hi16 = dd & 1;
                    uint32_t a0 = raw[0][wsel], a1 = raw[1][wsel], a2 = raw[2][wsel], a3 = raw[3][wsel];
                    uint32_t lo2 = hi16 ? ((a0 >> 16) | (a1 & 0xffff0000u)) : ((a0 & 0xffffu) | (a1 << 16));
                    uint32_t hi2 = hi16 ? ((a2 >> 16) | (a3 & 0xffff0000u)) : ((a2 & 0xffffu) | (a3 << 16));
                    const int d = ch * 8 + dd;
                    *reinterpret_cast<uint2*>(vt_lds + vt_off(d, gq) + 8 * kb) = uint2{lo2, hi2};
                }
            }
        }
        __syncthreads();

        // ---- S^T = K . Q^T ----
        f32x4 s[QB][2];
#pragma unroll
        for (int k = 0; k < QB; ++k) s[k][0] = s[k][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int kk = 0; kk < NKK; ++kk) {
                const u32x4 a = *reinterpret_cast<const u32x4*>(k_lds + k_off(kb * 16 + ln, kk * 4 + lg, D));
#pragma unroll
                for (int k = 0; k < QB; ++k) s[k][kb] = mfma16x16x32<F16>(a, qop[k][kk], s[k][kb]);
            }
        }

        // ---- score pipeline, visibility, online softmax ----
        int cell_of[8];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int i = 0; i < 4; ++i) cell_of[4 * kb + i] = cell_lds[kb * 16 + 4 * lg + i];

        u32x4 pop[QB];
#pragma unroll
        for (int k = 0; k < QB; ++k) {
            float sc[8];
            bool vis[8];
            float tmax = kNegInf;
            bool tnan = false;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int kb = e >> 2, i = e & 3;
                const int cell = cell_of[e];
                bool v = cell >= 0 && cell < qv_lim[k];
                float maskv = 0.f;
                if (v && p.mode == kMask) {
                    maskv = p.mask[static_cast<int64_t>(qv_row[k]) * p.m_sr +
                                   static_cast<int64_t>(qv_head[k]) * p.m_sh + cell];
                    v = maskv != kNegInf;
                }
                float x = s[k][kb][i];
                if constexpr (KT == SEL_ATTN_I8) x *= ksc_lds[kb * 16 + 4 * lg + i];
                if (p.softcap > 0.f) x = p.softcap * tanhf(x / p.softcap);
                x += slope[k] * static_cast<float>(cell - qv_pos[k]);
                x += maskv;
                vis[e] = v;
                sc[e] = x;
                if (v) {
                    if (x != x) tnan = true;
                    else tmax = max_keep(tmax, x);
                }
            }
            // combine over the four lane groups that hold this query vector
            tmax = max_keep(tmax, wave_xor(tmax, 16));
            tmax = max_keep(tmax, wave_xor(tmax, 32));
            int tn = tnan ? 1 : 0;
            tn |= wave_xor_i(tn, 16);
            tn |= wave_xor_i(tn, 32);
            nan_run[k] = nan_run[k] || tn;
            const float m_new = max_keep(m_run[k], tmax);
            const float c = rescale_factor(m_run[k], m_new);
            float pe[8];
            float lsum = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                pe[e] = vis[e] ? exp_diff(sc[e], m_new) : 0.f;
                lsum += pe[e];
            }
            l_run[k] = l_run[k] * c + lsum;
            m_run[k] = m_new;
            if (wave_any(c != 1.f)) {
#pragma unroll
                for (int db = 0; db < NDB; ++db) o_acc[k][db] *= c;
            }
            float pv[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                float w = pe[e];
                if constexpr (KT == SEL_ATTN_I8) w *= vsc_lds[(e >> 2) * 16 + 4 * lg + (e & 3)];
                pv[e] = w;
            }
            pop[k] = u32x4{pack2<F16>(pv[0], pv[1]), pack2<F16>(pv[2], pv[3]),
                           pack2<F16>(pv[4], pv[5]), pack2<F16>(pv[6], pv[7])};
            if (p.dbg_visit) {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    if (vis[e]) {
                        dbg_cnt[k] += 1;
                        dbg_sum[k] += cell_of[e];
                        dbg_sq[k] += static_cast<long long>(cell_of[e]) * cell_of[e];
                    }
                }
            }
        }

        // ---- O^T += V^T . P^T ----
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
            const u32x4 a = *reinterpret_cast<const u32x4*>(vt_lds + vt_off(db * 16 + ln, lg));
#pragma unroll
            for (int k = 0; k < QB; ++k) o_acc[k][db] = mfma16x16x32<F16>(a, pop[k], o_acc[k][db]);
        }
        __syncthreads();
    }

    // ---- epilogue ---------------------------------------------------------------
#pragma unroll
    for (int k = 0; k < QB; ++k) {
        float l = l_run[k];
        l += wave_xor(l, 16);
        l += wave_xor(l, 32);
        long long cnt = 0, sum = 0, sq = 0;
        if (p.dbg_visit) {
            // the four lane groups of a query vector saw disjoint keys: add their counts
            auto xsum = [&](long long v) -> long long {
                long long acc = v;
                for (int msk = 16; msk <= 32; msk <<= 1) {
                    const unsigned lo32 = static_cast<unsigned>(acc & 0xffffffffLL);
                    const int hi32 = static_cast<int>(acc >> 32);
                    const unsigned olo = static_cast<unsigned>(wave_xor_i(static_cast<int>(lo32), msk));
                    const int ohi = wave_xor_i(hi32, msk);
                    acc += static_cast<long long>((static_cast<unsigned long long>(static_cast<unsigned>(ohi)) << 32) | olo);
                }
                return acc;
            };
            cnt = xsum(dbg_cnt[k]);
            sum = xsum(dbg_sum[k]);
            sq = xsum(dbg_sq[k]);
        }
        if (!qv_ok[k]) continue;
        const int r = qv_row[k], h = qv_head[k];
        const float m = m_run[k];
        const bool bad = nan_run[k] || m == kPosInf;
        const bool empty = !bad && m == kNegInf;
        const bool split = p.mode == kDecode || p.n_splits > 1;
        int64_t pi;
        if (p.mode == kDecode)
            pi = ((static_cast<int64_t>(b) * p.R + r) * p.Hq + h) * p.n_slices_max + t_split;
        else
            pi = (static_cast<int64_t>(r) * p.Hq + h) * p.n_splits + t_split;
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
            const int d0 = db * 16 + 4 * lg;
            float4 o;
            if (!split) {
                const float inv = 1.f / l;
                if (bad) o = float4{__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""), __builtin_nanf("")};
                else if (empty) o = float4{0.f, 0.f, 0.f, 0.f};
                else o = float4{o_acc[k][db][0] * inv, o_acc[k][db][1] * inv, o_acc[k][db][2] * inv,
                                o_acc[k][db][3] * inv};
                *reinterpret_cast<float4*>(p.out + (static_cast<int64_t>(r) * p.Hq + h) * D + d0) = o;
            } else {
                if (empty) o = float4{0.f, 0.f, 0.f, 0.f};
                else o = float4{o_acc[k][db][0], o_acc[k][db][1], o_acc[k][db][2], o_acc[k][db][3]};
                *reinterpret_cast<float4*>(p.part_o + pi * D + d0) = o;
            }
        }
        if (split && lg == 0) {
            p.part_ml[pi * 2 + 0] = nan_run[k] ? __builtin_nanf("") : m;
            p.part_ml[pi * 2 + 1] = bad ? __builtin_nanf("") : (empty ? 0.f : l);
        }
        if (p.dbg_visit && lg == 0) {
            const int m_idx = m_wave + 16 * k + ln;
            const bool first_head = m_idx % G == 0;
            if (first_head) {
                int64_t di;
                if (p.mode == kDecode)
                    di = ((static_cast<int64_t>(b) * p.R + r) * p.Hkv + g) * p.n_slices_max + t_split;
                else
                    di = (static_cast<int64_t>(r) * p.Hkv + g) * p.n_splits + t_split;
                p.dbg_visit[di * 3 + 0] = cnt;
                p.dbg_visit[di * 3 + 1] = sum;
                p.dbg_visit[di * 3 + 2] = sq;
            }
        }
    }
}

// LDS bytes of a launch
size_t mfma_smem(int D, bool sel) {
    return static_cast<size_t>(kTK) * D * 2 + static_cast<size_t>(D) * 64 + 3 * kTK * 4 +
           (sel ? kMaxSelM * 4 : 0);
}

struct Shape {
    int qb;      // query blocks per wave
    int waves;   // waves per work-group
};

Shape pick_shape(int M) {
    const int nqb = (M + 15) / 16;
    if (nqb <= 1) return {1, 1};
    if (nqb <= 4) return {1, nqb};
    if (nqb <= 8) return {2, (nqb + 1) / 2};
    return {3, std::min(4, (nqb + 2) / 3)};
}

template <int KT, int D, int QB>
hipError_t launch_t(const MParams& p, dim3 grid, int waves, size_t smem, hipStream_t st) {
    static bool attr = false;
    if (!attr) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&mfma_attn_kernel<KT, D, QB>),
                                           hipFuncAttributeMaxDynamicSharedMemorySize,
                                           static_cast<int>(mfma_smem(256, true)));
        if (e != hipSuccess) return e;
        attr = true;
    }
    hipLaunchKernelGGL((mfma_attn_kernel<KT, D, QB>), grid, dim3(64 * waves), smem, st, p);
    return hipGetLastError();
}

template <int KT, int D>
hipError_t launch_qb(const MParams& p, dim3 grid, Shape sh, size_t smem, hipStream_t st) {
    switch (sh.qb) {
    case 1: return launch_t<KT, D, 1>(p, grid, sh.waves, smem, st);
    case 2: return launch_t<KT, D, 2>(p, grid, sh.waves, smem, st);
    default: return launch_t<KT, D, 3>(p, grid, sh.waves, smem, st);
    }
}

hipError_t dispatch(int dt, const MParams& p, dim3 grid, Shape sh, size_t smem, hipStream_t st) {
    if (dt == SEL_ATTN_BF16)
        return p.D == 256 ? launch_qb<SEL_ATTN_BF16, 256>(p, grid, sh, smem, st)
                          : launch_qb<SEL_ATTN_BF16, 128>(p, grid, sh, smem, st);
    if (dt == SEL_ATTN_F16)
        return p.D == 256 ? launch_qb<SEL_ATTN_F16, 256>(p, grid, sh, smem, st)
                          : launch_qb<SEL_ATTN_F16, 128>(p, grid, sh, smem, st);
    return p.D == 256 ? launch_qb<SEL_ATTN_I8, 256>(p, grid, sh, smem, st)
                      : launch_qb<SEL_ATTN_I8, 128>(p, grid, sh, smem, st);
}

int next_pow2(int x) {
    int q = 1;
    while (q < x) q <<= 1;
    return q;
}

bool dtype_ok(int dt) { return dt == SEL_ATTN_BF16 || dt == SEL_ATTN_F16 || dt == SEL_ATTN_I8; }

}  // namespace

bool mfma_decode_eligible(const sel_attn_decode_args& a) {
    return dtype_ok(a.kv_dtype) && (a.head_dim == 128 || a.head_dim == 256);
}

bool mfma_prefill_eligible(const sel_attn_prefill_args& a) {
    return dtype_ok(a.kv_dtype) && (a.head_dim == 128 || a.head_dim == 256) &&
           a.n_head_q / a.n_head_kv <= 16 * 3 * 4;
}

hipError_t launch_mfma_decode(const sel_attn_decode_args& a, hipStream_t st) {
    MParams p{};
    p.mode = kDecode;
    p.Hq = a.n_head_q; p.Hkv = a.n_head_kv; p.G = a.n_head_q / a.n_head_kv; p.D = a.head_dim;
    p.M = a.n_row * p.G;
    const Shape sh = pick_shape(p.M);
    p.qpw = sh.waves * sh.qb * 16;
    p.q = a.q; p.k = a.k; p.v = a.v;
    p.kv_ss = a.kv_stride_stream; p.kv_sc = a.kv_stride_cell; p.kv_sh = a.kv_stride_head;
    p.ksc = a.k_scale; p.vsc = a.v_scale;
    p.sc_ss = a.sc_stride_stream; p.sc_sc = a.sc_stride_cell; p.sc_sh = a.sc_stride_head;
    p.scale = a.scale; p.softcap = a.softcap; p.alibi = a.alibi_slopes;
    p.R = a.n_row; p.cap = a.cap; p.kv_len = a.kv_len; p.causal = a.causal;
    p.slice_len = a.slice_len; p.n_slices_max = a.n_slices_max;
    p.part_o = a.part_o; p.part_ml = a.part_ml; p.dbg_visit = a.dbg_visit;
    const int nqc = (p.M + p.qpw - 1) / p.qpw;
    const int n_sl = std::min(a.n_slices_max, (a.cap + a.slice_len - 1) / a.slice_len);
    dim3 grid(n_sl, a.n_head_kv * nqc, a.n_stream);
    return dispatch(a.kv_dtype, p, grid, sh, mfma_smem(a.head_dim, false), st);
}

hipError_t launch_mfma_prefill(const sel_attn_prefill_args& a, hipStream_t st) {
    MParams p{};
    const bool sel = a.sel != nullptr;
    p.mode = sel ? kSel : kMask;
    p.Hq = a.n_head_q; p.Hkv = a.n_head_kv; p.G = a.n_head_q / a.n_head_kv; p.D = a.head_dim;
    Shape sh;
    if (sel) {
        p.M = p.G;
        sh = pick_shape(p.M);
        p.rows_per_wg = 1;
    } else {
        // 16-row blocks of query vectors (rows x heads), up to 4 waves
        const int rows = std::max(1, std::min(a.n_row, 64 / p.G));
        p.M = rows * p.G;
        sh = pick_shape(p.M);
        p.rows_per_wg = rows;
    }
    p.qpw = sh.waves * sh.qb * 16;
    p.q = a.q; p.k = a.k; p.v = a.v;
    p.kv_sc = a.kv_stride_cell; p.kv_sh = a.kv_stride_head;
    p.ksc = a.k_scale; p.vsc = a.v_scale;
    p.sc_sc = a.sc_stride_cell; p.sc_sh = a.sc_stride_head;
    p.scale = a.scale; p.softcap = a.softcap; p.alibi = a.alibi_slopes;
    p.R = a.n_row; p.n_kv = a.n_kv; p.q_pos = a.q_pos; p.causal = a.causal;
    p.sel = a.sel; p.n_sel = a.n_sel; p.bs = a.block_size; p.sel_pow2 = sel ? next_pow2(a.n_sel) : 0;
    p.mask = a.mask; p.m_sr = a.mask_stride_row; p.m_sh = a.mask_stride_head;
    p.n_splits = a.n_splits;
    p.split_step = (a.n_kv + a.n_splits - 1) / a.n_splits;
    p.out = a.out; p.part_o = a.part_o; p.part_ml = a.part_ml;
    p.dbg_visit = a.dbg_visit; p.dbg_sel = a.dbg_sel;
    const int nqc = (p.M + p.qpw - 1) / p.qpw;
    const int n_rb = (a.n_row + p.rows_per_wg - 1) / p.rows_per_wg;
    dim3 grid(a.n_splits, a.n_head_kv * nqc, n_rb);
    return dispatch(a.kv_dtype, p, grid, sh, mfma_smem(a.head_dim, sel), st);
}

}  // namespace selattn
