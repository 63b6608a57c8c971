// Matrix-core split-K decode kernel for units with many query vectors: verify
// windows of R draft rows x G query heads of one kv head (16 x 12 = 192 query
// vectors per (stream, slice, kv head) unit for the int8 verify workload).
//
// One work-group per unit (or per chunk of its query vectors), one wave per block
// of 16 query vectors, so every K/V tile is loaded, dequantised and staged in LDS
// once for all query vectors of the unit (TensorFold PR #2595: one work-group per
// (stream, kv head, slice) of the attn_decode grid; partials merged by the
// log-sum-exp combine afterwards):
//   * 32-key tiles: K row-major and V^T in contraction order in LDS (the layouts
//     of mfma_kernel.h);
//   * S^T = K . Q^T and O^T += V^T . P^T both on v_mfma_f32_16x16x32, each lane
//     holding the 8 scores of one query vector that form its P^T operand;
//   * the tile loads are spread over every thread of the work-group (K as 16-byte
//     chunks, V as 4 keys x 8 bytes) and kept two tiles ahead in registers with 4
//     or 8 waves, one tile ahead with 12 (three waves share a SIMD's registers);
//   * lazy rescaling of o and l as in lean_kernel.h: the exponent reference only
//     moves when a score passes it by more than kLazy, the true maximum is applied
//     once at the end (the correction exp(m_old - m_new) of TensorFold PR #985,
//     "What this changes").
#pragma once

#include "mfma_kernel.h"

namespace selattn {
namespace mk {

// LDS: K tile, V^T tile, the tile's int8 scales, each wave's Q^T operands (16
// query vectors x D, bf16/fp16, in operand order), its visit counters, its tree
// path masks, its non-finite-V flag, and (16-bit and e4m3 data) the V^T indicator
// tile of tiles seen in part.
template <int D, int W, int KT>
constexpr int group_smem() {
    return kTK * D * 2 + D * 64 + 2 * kTK * 4 + W * D * 32 + W * 16 * 3 * 8 + W * 16 * 8 + 16 * 4 +
           (KT != SEL_ATTN_I8 ? D * 64 : 0);
}

template <int KT, int D, int W>
__device__ __forceinline__ void group_unit(const MParams& p, const int t_split, const int gy, const int b,
                                           char* smem) {
    constexpr bool F16 = (KT == SEL_ATTN_F16);
    constexpr bool B8 = byte_kv(KT);       // int8 or e4m3 rows with row scales
    constexpr int NKK = D / 32;                  // contraction steps of S^T
    constexpr int NDB = D / 16;                  // dim blocks of O^T
    constexpr int GCH = B8 ? D / 16 : D / 8;     // 16-byte chunks per K/V row in memory
    constexpr int NT = 64 * W;
    constexpr int K_TASKS = kTK * GCH;           // task e < K_TASKS: K row e / GCH, chunk e % GCH
    constexpr int V_TASKS = 8 * 2 * GCH;         // keys 4 * (e' & 7) + 0..3, 8-byte half chunk e' >> 3
    constexpr int TASKS = K_TASKS + V_TASKS;
    constexpr int NSLOT = (TASKS + NT - 1) / NT;
    constexpr int EPH = B8 ? 8 : 4;              // elements per 8-byte half chunk
    constexpr int ROWB = D * (B8 ? 1 : 2);
    static_assert(K_TASKS % 64 == 0 && V_TASKS % 64 == 0, "tasks must fill whole waves");
    static_assert(NDB % 4 == 0, "O^T dim blocks are taken four at a time");
    // Tiles that some query vectors see only in part (the window of a causal or tree
    // verify) are staged with their non-finite V values split off (int8 data is
    // always finite); see split_nonfinite.
    constexpr bool CHK = KT != SEL_ATTN_I8;

    char* k_lds = smem;                                            // kTK * D * 2
    char* vt_lds = smem + kTK * D * 2;                             // D * 64
    float* ksc_lds = reinterpret_cast<float*>(vt_lds + D * 64);    // kTK
    float* vsc_lds = ksc_lds + kTK;                                // kTK
    char* q_lds = reinterpret_cast<char*>(vsc_lds + kTK);          // W * D * 32
    unsigned long long* dbg_lds =                                  // W * 16 * 3
        reinterpret_cast<unsigned long long*>(q_lds + W * D * 32);
    unsigned long long* tpath_lds = dbg_lds + W * 16 * 3;          // W * 16
    uint32_t* wflag = reinterpret_cast<uint32_t*>(tpath_lds + W * 16);   // [16]: wave w staged a non-finite V value
    const int ind_off = static_cast<int>(reinterpret_cast<char*>(wflag + 16) - vt_lds);   // indicator tile - vt_lds

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int ln = lane & 15;
    const int lg = lane >> 4;
    const int G = p.G;

    // ---- work unit ---------------------------------------------------------
    const int g = gy % p.Hkv;
    const int qchunk = gy / p.Hkv;
    const int kvl = min(max(p.kv_len[b], 0), p.cap);
    const int lo = t_split * p.slice_len;
    if (lo >= kvl) return;                      // uniform over the work-group
    const int hi = min(lo + p.slice_len, kvl);
    const int m_wg = qchunk * p.qpw;
    const int m_end = min(p.M, m_wg + p.qpw);
    const int m_wave = m_wg + wave * 16;
    const bool wave_live = m_wave < m_end;      // uniform over the wave

    // this lane's query vector: row r, head h
    const int m = m_wave + ln;
    bool ok = m < m_end;
    int r = m / G, h = g * G + m % G;
    ok = ok && r < p.R;
    if (!ok) { r = 0; h = g * G; }
    const int pos = kvl - p.R + r;
    const bool tree = p.tree != nullptr;
    int lim = min((p.causal && !tree) ? min(pos + 1, kvl) : kvl, hi);
    if (!ok) lim = -1;
    // tree windows: the window nodes this query vector sees, kept in LDS for the
    // partial tiles (read after the first tile's barrier)
    unsigned long long* my_tpath = tpath_lds + wave * 16 + ln;
    if (tree) {                                 // uniform
        const unsigned long long path = tree_path_mask_wave(p.tree + static_cast<int64_t>(b) * p.R, p.R, r);
        if (lg == 0) *my_tpath = path;
    }

    // Q^T operands, scale folded in, kept in this wave's part of LDS (registers go
    // to the O^T accumulators): step kk of lane l at kk * 1024 + l * 16
    char* qw_lds = q_lds + wave * (NKK * 1024) + lane * 16;
    {
        const float* qp = p.q + ((static_cast<int64_t>(b) * p.R + r) * p.Hq + h) * D;
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
            float x[8];
            if (ok) {
                const float4 a = *reinterpret_cast<const float4*>(qp + kk * 32 + 8 * lg);
                const float4 c = *reinterpret_cast<const float4*>(qp + kk * 32 + 8 * lg + 4);
                x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
                x[4] = c.x; x[5] = c.y; x[6] = c.z; x[7] = c.w;
            } else {
#pragma unroll
                for (int j = 0; j < 8; ++j) x[j] = 0.f;
            }
            u32x4 qv;
#pragma unroll
            for (int j = 0; j < 4; ++j) qv[j] = pack2<F16>(x[2 * j] * p.scale, x[2 * j + 1] * p.scale);
            *reinterpret_cast<u32x4*>(qw_lds + kk * 1024) = qv;
        }
    }
    const float slope = (p.alibi && ok) ? p.alibi[h] : 0.f;

    // keys no query vector of the work-group can see are never loaded
    // (lim_max); keys below lim_min are seen by every query vector of it
    int lim_max = -1, lim_min = 0x7fffffff;
    for (int rr = m_wg / G; rr <= (m_end - 1) / G && rr < p.R; ++rr) {
        const int l = (p.causal && !tree) ? min(kvl - p.R + rr + 1, kvl) : kvl;
        lim_max = max(lim_max, l);
        lim_min = min(lim_min, tree ? max(kvl - p.R, 0) : l);
    }
    const int n_keys = max(0, min(hi, lim_max) - lo);
    const int n_full = max(0, min(hi, lim_min) - lo);      // key slots visible to all

    // ---- tile loads ----------------------------------------------------------
    // Buffer loads through a descriptor that starts at the unit's first key row and
    // ends with its last needed row: rows past it (the tail of the last tile) read
    // as zeros.  32-bit offsets: slice_len * cell stride < 2^31 is checked on the host.
    const int cb = static_cast<int>(p.kv_sc * (B8 ? 1 : 2));
    const int64_t kv_base = static_cast<int64_t>(b) * p.kv_ss + static_cast<int64_t>(g) * p.kv_sh;
    const int64_t sc_base = static_cast<int64_t>(b) * p.sc_ss + static_cast<int64_t>(g) * p.sc_sh;
    const char* kbase = static_cast<const char*>(p.k) + (kv_base + static_cast<int64_t>(lo) * p.kv_sc) * (B8 ? 1 : 2);
    const char* vbase = static_cast<const char*>(p.v) + (kv_base + static_cast<int64_t>(lo) * p.kv_sc) * (B8 ? 1 : 2);
    const int nrec = n_keys > 0 ? (n_keys - 1) * cb + ROWB : 0;
    const __amdgpu_buffer_rsrc_t krs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(kbase), static_cast<short>(0), nrec, 0x00020000);
    const __amdgpu_buffer_rsrc_t vrs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(vbase), static_cast<short>(0), nrec, 0x00020000);

    // slot i of thread tid holds task tid + i * NT: a K chunk in k[i], or four
    // 8-byte V pieces in v[i][0].xy, v[i][0].zw, v[i][1].xy, v[i][1].zw
    struct Regs {
        u32x4 k[NSLOT];
        u32x4 v[NSLOT][2];
        float ks, vs;
    };
    // (K and V slots are filled in separate passes, so no store is shared between
    // the two kinds and the slots stay in registers)
    auto load_tile = [&](Regs& rg, int t0) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < NSLOT; ++i) {
            const int e = tid + i * NT;
            if (e < K_TASKS) {
                const int voff = (e / GCH) * cb + (e % GCH) * 16;
                rg.k[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(krs, voff, t0 * cb, 0));
            }
        }
#pragma unroll
        for (int i = 0; i < NSLOT; ++i) {
            const int e = tid + i * NT;
            if (e >= K_TASKS && e < TASKS) {
                const int ev = e - K_TASKS;
                const int voff = 4 * (ev & 7) * cb + (ev >> 3) * 8;
                const u32x2 a0 = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(vrs, voff, t0 * cb, 0));
                const u32x2 a1 = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(vrs, voff, (t0 + 1) * cb, 0));
                const u32x2 a2 = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(vrs, voff, (t0 + 2) * cb, 0));
                const u32x2 a3 = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(vrs, voff, (t0 + 3) * cb, 0));
                rg.v[i][0] = u32x4{a0[0], a0[1], a1[0], a1[1]};
                rg.v[i][1] = u32x4{a2[0], a2[1], a3[0], a3[1]};
            }
        }
        if constexpr (B8) {
            if (tid < kTK) {
                const bool in = t0 + tid < n_keys;
                const int64_t si = sc_base + static_cast<int64_t>(lo + t0 + tid) * p.sc_sc;
                rg.ks = in ? p.ksc[si] : 0.f;
                rg.vs = in ? p.vsc[si] : 0.f;
            }
        }
    };
    // tile t0 is seen in full by every query vector of the work-group
    auto full_tile = [&](int t0) -> bool { return t0 + kTK <= n_full; };
    // mode 0: plain; 1: plain, and the V words are checked for Inf / NaN (a tile some
    // query vector sees in part); 2: V split into its finite part and indicator (the
    // second staging of a checked tile that held one)
    auto store_tile = [&](const Regs& rg, int mode) __attribute__((always_inline)) {
        uint32_t nfa = 0u;
#pragma unroll
        for (int i = 0; i < NSLOT; ++i) {
            const int e = tid + i * NT;
            if (e < K_TASKS) {
                const int key = e / GCH, ch = e % GCH;
                if constexpr (B8) {
                    const u32x4 rw = rg.k[i];
                    u32x4 w0, w1;
#pragma unroll
                    for (int j = 0; j < 2; ++j) {
                        w0[2 * j] = kpair_bf16<KT>(rw[j], 0);
                        w0[2 * j + 1] = kpair_bf16<KT>(rw[j], 1);
                        w1[2 * j] = kpair_bf16<KT>(rw[2 + j], 0);
                        w1[2 * j + 1] = kpair_bf16<KT>(rw[2 + j], 1);
                    }
                    *reinterpret_cast<u32x4*>(k_lds + k_off(key, 2 * ch, D)) = w0;
                    *reinterpret_cast<u32x4*>(k_lds + k_off(key, 2 * ch + 1, D)) = w1;
                } else {
                    *reinterpret_cast<u32x4*>(k_lds + k_off(key, ch, D)) = rg.k[i];
                }
            } else if (e < TASKS) {
                const int ev = e - K_TASKS;
                const int kg = ev & 7, hc = ev >> 3;        // keys 4 * kg + j, half chunk hc
                const int kb = kg >> 2, gq = kg & 3;        // keys kb * 16 + 4 * gq + j
                // the 8 bytes of key j: word pair (x[j >> 1] lanes 2 * (j & 1) + 0..1)
                uint32_t w[4][2];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    w[j][0] = rg.v[i][j >> 1][2 * (j & 1)];
                    w[j][1] = rg.v[i][j >> 1][2 * (j & 1) + 1];
                }
                if constexpr (B8) {
                    // dims hc * 8 + 4 * h + jj (byte jj of word h of each key).  Their
                    // V^T rows are hc * 8 + 4 * h + (jj ^ c), c = hc & 3, and the chunk
                    // swizzle depends on h only: the address is a per-half base with
                    // (jj ^ c) in bits 6..7, i.e. (base + (c << 6)) ^ (jj << 6).  Lanes
                    // with different c land in different bank quarters at each step.
                    const int c = hc & 3;
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        const int wbc = (hc * 8 + 4 * h + c) * 64 + ((gq ^ ((2 * hc + h) & 3)) << 4) + 8 * kb;
#pragma unroll
                        for (int jj = 0; jj < 4; jj += 2) {          // bytes jj, jj + 1 at once
                            uint32_t lo_e, lo_o, hi_e, hi_o;
                            vpairs_bf16<KT>(w[0][h], w[1][h], jj >> 1, lo_e, lo_o);
                            vpairs_bf16<KT>(w[2][h], w[3][h], jj >> 1, hi_e, hi_o);
                            if (CHK && mode != 0) {
                                nfa = store_v<F16>(vt_lds + (wbc ^ (jj << 6)), ind_off, lo_e, hi_e, mode == 2, nfa);
                                nfa = store_v<F16>(vt_lds + (wbc ^ ((jj + 1) << 6)), ind_off, lo_o, hi_o, mode == 2, nfa);
                            } else {
                                *reinterpret_cast<uint2*>(vt_lds + (wbc ^ (jj << 6))) = uint2{lo_e, hi_e};
                                *reinterpret_cast<uint2*>(vt_lds + (wbc ^ ((jj + 1) << 6))) = uint2{lo_o, hi_o};
                            }
                        }
                    }
                } else {
#pragma unroll
                for (int dd = 0; dd < EPH; ++dd) {
                    uint32_t lo2, hi2;
                    {
                        const int wi = dd >> 1;
                        if (dd & 1) {
                            lo2 = (w[0][wi] >> 16) | (w[1][wi] & 0xffff0000u);
                            hi2 = (w[2][wi] >> 16) | (w[3][wi] & 0xffff0000u);
                        } else {
                            lo2 = (w[0][wi] & 0xffffu) | (w[1][wi] << 16);
                            hi2 = (w[2][wi] & 0xffffu) | (w[3][wi] << 16);
                        }
                    }
                    if (CHK && mode != 0) nfa = store_v<F16>(vt_lds + vt_off(hc * EPH + dd, gq) + 8 * kb, ind_off, lo2, hi2, mode == 2, nfa);
                    else *reinterpret_cast<uint2*>(vt_lds + vt_off(hc * EPH + dd, gq) + 8 * kb) = uint2{lo2, hi2};
                }
                }
            }
        }
        if constexpr (B8) {
            if (tid < kTK) {
                ksc_lds[tid] = rg.ks;
                vsc_lds[tid] = rg.vs;
            }
        }
        if constexpr (CHK) {
            if (mode == 1) {                        // uniform
                const bool any = wave_any(nonfinite_found(nfa));
                if (lane == 0) wflag[wave] = any ? 1u : 0u;
            }
        }
    };
    // Stages tile t0 from rg; a tile some query vector sees in part is checked, and
    // staged again split if any wave found an Inf or NaN.  Returns that finding
    // (uniform).  Ends with a barrier: the tile is ready for every wave.
    auto stage = [&](const Regs& rg, int t0) __attribute__((always_inline)) -> bool {
        const bool chk = CHK && !full_tile(t0);
        store_tile(rg, chk ? 1 : 0);
        __syncthreads();
        if (!chk) return false;
        uint32_t f = 0u;
#pragma unroll
        for (int w = 0; w < W; ++w) f |= wflag[w];
        if (f == 0u) return false;
        store_tile(rg, 2);
        __syncthreads();
        return true;
    };


    // ---- running state ---------------------------------------------------------
    float m_use = kNegInf;     // exponent reference of o and l
    float m_true = kNegInf;    // largest visible non-NaN score seen
    float l_run = 0.f;
    bool nan_run = false;
    // visit counters of this lane's query vector (count, sum, sum of squares of
    // the cells it combines) live in LDS, so they hold no registers in the loop
    unsigned long long* my_dbg = dbg_lds + (wave * 16 + ln) * 3;
    if (p.dbg_visit && lg == 0) my_dbg[0] = my_dbg[1] = my_dbg[2] = 0ull;
    f32x4 o_acc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) o_acc[db] = f32x4{0.f, 0.f, 0.f, 0.f};

    // Operand read addresses written as base + immediate offset.  K (k_off): key
    // kb * 16 + ln, chunk kk * 4 + lg, XOR-ed with ln, which only touches the low two
    // bits of kk: four bases.  V^T (vt_off): dim db * 16 + ln, chunk lg; the row XOR
    // depends on db & 1 only and the chunk XOR not on db: two bases.
    int kread[4], vread[2];
#pragma unroll
    for (int q = 0; q < 4; ++q) kread[q] = ln * D * 2 + (((q * 4 + lg) ^ ln) << 4);
#pragma unroll
    for (int par = 0; par < 2; ++par) {
        const int x = (2 * par + (ln >> 3)) & 3;
        vread[par] = (ln ^ x) * 64 + ((lg ^ ((ln >> 2) & 3)) << 4);
    }

    // one tile of math on the staged K/V (the caller brackets it with barriers);
    // flagged: the tile's V held an Inf or NaN and was staged split
    auto tile_math = [&](int t0, bool flagged) __attribute__((always_inline)) {
        f32x4 s[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
            const u32x4 qk = *reinterpret_cast<const u32x4*>(qw_lds + kk * 1024);
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                const u32x4 a = *reinterpret_cast<const u32x4*>(k_lds + kread[kk & 3] + (kk >> 2) * 256 + kb * 16 * D * 2);
                s[kb] = mfma16x16x32<F16>(a, qk, s[kb]);
            }
        }
        // score e of this lane is key cell0 + off(e): off = (e >> 2) * 16 + (e & 3)
        const int cell0 = lo + t0 + 4 * lg;
        float sc[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) sc[e] = s[e >> 2][e & 3];
        if constexpr (B8) {
            const float4 k0 = *reinterpret_cast<const float4*>(ksc_lds + 4 * lg);
            const float4 k1 = *reinterpret_cast<const float4*>(ksc_lds + 16 + 4 * lg);
            sc[0] *= k0.x; sc[1] *= k0.y; sc[2] *= k0.z; sc[3] *= k0.w;
            sc[4] *= k1.x; sc[5] *= k1.y; sc[6] *= k1.z; sc[7] *= k1.w;
        }
        if (p.softcap > 0.f) {                      // uniform: softcap before ALiBi
#pragma unroll
            for (int e = 0; e < 8; ++e) sc[e] = p.softcap * tanhf(sc[e] / p.softcap);
        }
        if (p.alibi) {
#pragma unroll
            for (int e = 0; e < 8; ++e)
                sc[e] += slope * static_cast<float>(cell0 + (e >> 2) * 16 + (e & 3) - pos);
        }
        // Visibility: a tile whose keys every query vector of the work-group sees
        // (uniform test) skips the per-score masks.  A NaN score is left out of the
        // maximum (v_max_f32 returns the other operand) and shows up as a NaN weight,
        // hence a NaN running sum, which the epilogue turns into the NaN flag.
        const bool full = full_tile(t0);
        // partial tile: bit o of vword says whether key slot o (cell cell0 + o) is visible
        uint32_t vword;
        {
            const int vlim = lim - cell0;
            vword = vlim >= 32 ? 0xffffffffu : (vlim <= 0 ? 0u : (1u << vlim) - 1u);
            if (tree) {                             // uniform: window cells by path mask
                const unsigned long long path = *my_tpath;
                const int w0 = kvl - p.R - cell0;   // slot of the window's first node
                uint32_t keep;
                if (w0 >= 32) keep = 0xffffffffu;
                else if (w0 >= 0) keep = ((1u << w0) - 1u) | static_cast<uint32_t>(path << w0);
                else keep = w0 <= -64 ? 0u : static_cast<uint32_t>(path >> (-w0));
                vword &= keep;
            }
        }
        float tmax = kNegInf;
        if (full) {
#pragma unroll
            for (int e = 0; e < 8; ++e) tmax = fmaxf(tmax, sc[e]);
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) tmax = fmaxf(tmax, ((vword >> ((e >> 2) * 16 + (e & 3))) & 1u) ? sc[e] : kNegInf);
        }
        if (p.dbg_visit) {
            unsigned long long c = 0, sm = 0, sq = 0;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                if (full || ((vword >> ((e >> 2) * 16 + (e & 3))) & 1u)) {
                    const unsigned long long cell = cell0 + (e >> 2) * 16 + (e & 3);
                    c += 1;
                    sm += cell;
                    sq += cell * cell;
                }
            }
            atomicAdd(my_dbg + 0, c);
            atomicAdd(my_dbg + 1, sm);
            atomicAdd(my_dbg + 2, sq);
        }
        tmax = wave_max_x16(tmax);
        tmax = wave_max_x32(tmax);
        m_true = fmaxf(m_true, tmax);
        const bool need = (tmax > m_use + kLazy) || (m_use == kNegInf && tmax != kNegInf);
        if (wave_any(need)) {
            const float c = need ? rescale_factor(m_use, tmax) : 1.f;
            if (need) m_use = tmax;
            l_run *= c;
#pragma unroll
            for (int db = 0; db < NDB; ++db) o_acc[db] *= c;
        }
        // weights exp(s - m_use) (v_exp_f32; results below 2^-126 flush to zero)
        const float mls = m_use * kLog2e;
        float pv[8];
        if (full) {
#pragma unroll
            for (int e = 0; e < 8; ++e) pv[e] = __builtin_amdgcn_exp2f(fmaf(sc[e], kLog2e, -mls));
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e)
                pv[e] = ((vword >> ((e >> 2) * 16 + (e & 3))) & 1u) ? __builtin_amdgcn_exp2f(fmaf(sc[e], kLog2e, -mls)) : 0.f;
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) l_run += pv[e];
        if constexpr (B8) {
            const float4 v0 = *reinterpret_cast<const float4*>(vsc_lds + 4 * lg);
            const float4 v1 = *reinterpret_cast<const float4*>(vsc_lds + 16 + 4 * lg);
            const float vs[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
            // the row scale joins visible weights only: a NaN scale of a key this query
            // vector cannot see must not reach it
            if (full) {
#pragma unroll
                for (int e = 0; e < 8; ++e) pv[e] *= vs[e];
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) pv[e] = ((vword >> ((e >> 2) * 16 + (e & 3))) & 1u) ? pv[e] * vs[e] : 0.f;
            }
        }
        const u32x4 pop = u32x4{pack2<F16>(pv[0], pv[1]), pack2<F16>(pv[2], pv[3]),
                                pack2<F16>(pv[4], pv[5]), pack2<F16>(pv[6], pv[7])};
#pragma unroll
        // four V^T operand reads per group of four products (NDB is a multiple of
        // 4): each product waits on its own read, and with several in flight the
        // LDS latency is paid once per group rather than once per product
        for (int db = 0; db < NDB; db += 4) {
            const u32x4 a0 = *reinterpret_cast<const u32x4*>(vt_lds + vread[0] + db * 1024);
            const u32x4 a1 = *reinterpret_cast<const u32x4*>(vt_lds + vread[1] + (db + 1) * 1024);
            const u32x4 a2 = *reinterpret_cast<const u32x4*>(vt_lds + vread[0] + (db + 2) * 1024);
            const u32x4 a3 = *reinterpret_cast<const u32x4*>(vt_lds + vread[1] + (db + 3) * 1024);
            o_acc[db] = mfma16x16x32<F16>(a0, pop, o_acc[db]);
            o_acc[db + 1] = mfma16x16x32<F16>(a1, pop, o_acc[db + 1]);
            o_acc[db + 2] = mfma16x16x32<F16>(a2, pop, o_acc[db + 2]);
            o_acc[db + 3] = mfma16x16x32<F16>(a3, pop, o_acc[db + 3]);
        }
        // a tile seen in part whose staged V held a non-finite value (uniform): the
        // product above used its finite part; the visible non-finite values are
        // counted from the indicator tile and applied
        if constexpr (CHK) {
            if (flagged) {
                bool vis[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) vis[e] = (vword >> ((e >> 2) * 16 + (e & 3))) & 1u;
                const u32x4 pvis = u32x4{vis_pair<F16>(vis[0], vis[1]), vis_pair<F16>(vis[2], vis[3]),
                                         vis_pair<F16>(vis[4], vis[5]), vis_pair<F16>(vis[6], vis[7])};
#pragma unroll
                for (int db = 0; db < NDB; ++db) {
                    const u32x4 ai = *reinterpret_cast<const u32x4*>(vt_lds + ind_off + vread[db & 1] + db * 1024);
                    const f32x4 cnt = mfma16x16x32<F16>(ai, pvis, f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
                    for (int i = 0; i < 4; ++i) o_acc[db][i] = apply_nonfinite(o_acc[db][i], cnt[i]);
                    __builtin_amdgcn_sched_barrier(0);      // a rare path: one dim block at a time
                }
            }
        }
    };

    if constexpr (W < 12) {
        // two register sets: the loads of tile t + 2 are in flight during tiles t and t + 1
        Regs ra, rb;
        if (n_keys > 0) load_tile(ra, 0);
        if (n_keys > kTK) load_tile(rb, kTK);
        for (int t0 = 0; t0 < n_keys; t0 += 2 * kTK) {
            const bool fa = stage(ra, t0);
            if (t0 + 2 * kTK < n_keys) load_tile(ra, t0 + 2 * kTK);
            if (wave_live) tile_math(t0, fa);
            __syncthreads();
            if (t0 + kTK < n_keys) {
                const bool fb = stage(rb, t0 + kTK);
                if (t0 + 3 * kTK < n_keys) load_tile(rb, t0 + 3 * kTK);
                if (wave_live) tile_math(t0 + kTK, fb);
                __syncthreads();
            }
        }
    } else {
        // 12 waves share a SIMD three at a time (168 registers each): one set, the
        // loads of tile t + 1 are in flight during tile t
        Regs ra;
        if (n_keys > 0) load_tile(ra, 0);
        for (int t0 = 0; t0 < n_keys; t0 += kTK) {
            const bool fa = stage(ra, t0);
            if (t0 + kTK < n_keys) load_tile(ra, t0 + kTK);
            if (wave_live) tile_math(t0, fa);
            __syncthreads();
        }
    }

    // ---- epilogue: partials of this slice -------------------------------------
    if (!wave_live) return;
    float l = l_run;
    l = wave_sum_x16(l);
    l = wave_sum_x32(l);
    {
        // a NaN visible score made this lane's running sum NaN
        int tn = (l_run != l_run) ? 1 : 0;
        tn = wave_or_x16(tn);
        tn = wave_or_x32(tn);
        nan_run = tn != 0;
    }
    if (!ok) return;
    const bool bad = nan_run || m_true == kPosInf;
    const bool empty = !bad && m_true == kNegInf;
    float f = 1.f;
    if (!bad && !empty && m_use != m_true) f = exp2f((m_use - m_true) * kLog2e);
    l *= f;
    const int64_t pi = ((static_cast<int64_t>(b) * p.R + r) * p.Hq + h) * p.n_slices_max + t_split;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
        const int d0 = db * 16 + 4 * lg;
        float4 o;
        if (empty) o = float4{0.f, 0.f, 0.f, 0.f};
        else o = float4{o_acc[db][0] * f, o_acc[db][1] * f, o_acc[db][2] * f, o_acc[db][3] * f};
        *reinterpret_cast<float4*>(p.part_o + pi * D + d0) = o;
    }
    if (lg == 0) {
        p.part_ml[pi * 2 + 0] = nan_run ? __builtin_nanf("") : m_true;
        p.part_ml[pi * 2 + 1] = bad ? __builtin_nanf("") : (empty ? 0.f : l);
    }
    if (p.dbg_visit && lg == 0 && m % G == 0) {
        const int64_t di = ((static_cast<int64_t>(b) * p.R + r) * p.Hkv + g) * p.n_slices_max + t_split;
        p.dbg_visit[di * 3 + 0] = static_cast<int64_t>(my_dbg[0]);
        p.dbg_visit[di * 3 + 1] = static_cast<int64_t>(my_dbg[1]);
        p.dbg_visit[di * 3 + 2] = static_cast<int64_t>(my_dbg[2]);
    }
}

template <int KT, int D, int W>
__global__ __launch_bounds__(64 * W) void group_decode_kernel(MParams p) {
    extern __shared__ __align__(16) char smem[];
    for_each_decode_item(p, [&](int t, int gy, int bz) {
        group_unit<KT, D, W>(p, t, gy, bz, smem);
        __syncthreads();                                         // LDS is reused by the next item
    });
}

// ---------------------------------------------------------------------------
// launch
// ---------------------------------------------------------------------------
// Waves per work-group for nqb blocks of 16 query vectors (nqb >= 2): 4, 8 or 12,
// the fewest idle waves; more than 12 blocks are cut into query chunks.
inline int group_waves(int nqb) {
    if (nqb <= 4) return 4;
    if (nqb <= 8) return 8;
    if (nqb <= 12) return 12;
    const int c8 = (nqb + 7) / 8 * 8, c12 = (nqb + 11) / 12 * 12;
    return c12 <= c8 ? 12 : 8;
}

template <int KT, int D, int W>
hipError_t group_launch_one(const MParams& p, dim3 grid, hipStream_t st) {
    constexpr int smem = group_smem<D, W, KT>();
    // the LDS limit is raised (per device) before the occupancy query and any launch
    static DeviceCache cache;
    hipError_t attr = hipSuccess;
    const int resident = cache.get(0, [&attr]() {
        attr = hipFuncSetAttribute(reinterpret_cast<const void*>(&group_decode_kernel<KT, D, W>),
                                   hipFuncAttributeMaxDynamicSharedMemorySize, smem);
        if (attr != hipSuccess) return 0;
        int dev = 0, cus = 0, per_cu = 0;
        if (hipGetDevice(&dev) != hipSuccess) dev = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
            cus = 256;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, group_decode_kernel<KT, D, W>, 64 * W, smem) !=
                hipSuccess ||
            per_cu <= 0)
            per_cu = 1;
        return cus * per_cu;
    });
    if (attr != hipSuccess) return attr;
    const long long items = static_cast<long long>(grid.x) * grid.y * grid.z;
    hipLaunchKernelGGL((group_decode_kernel<KT, D, W>), dim3(decode_grid(items, resident)), dim3(64 * W), smem,
                       st, p);
    return hipGetLastError();
}

template <int KT, int D>
hipError_t group_launch_w(const MParams& p, dim3 grid, int w, hipStream_t st) {
    switch (w) {
    case 4: return group_launch_one<KT, D, 4>(p, grid, st);
    case 8: return group_launch_one<KT, D, 8>(p, grid, st);
    default: return group_launch_one<KT, D, 12>(p, grid, st);
    }
}

inline hipError_t group_launch(int dt, const MParams& p, dim3 grid, int w, hipStream_t st) {
    if (dt == SEL_ATTN_BF16)
        return p.D == 256 ? group_launch_w<SEL_ATTN_BF16, 256>(p, grid, w, st)
                          : group_launch_w<SEL_ATTN_BF16, 128>(p, grid, w, st);
    if (dt == SEL_ATTN_F16)
        return p.D == 256 ? group_launch_w<SEL_ATTN_F16, 256>(p, grid, w, st)
                          : group_launch_w<SEL_ATTN_F16, 128>(p, grid, w, st);
    if (dt == SEL_ATTN_I8)
        return p.D == 256 ? group_launch_w<SEL_ATTN_I8, 256>(p, grid, w, st)
                          : group_launch_w<SEL_ATTN_I8, 128>(p, grid, w, st);
    return p.D == 256 ? group_launch_w<SEL_ATTN_FP8, 256>(p, grid, w, st)
                      : group_launch_w<SEL_ATTN_FP8, 128>(p, grid, w, st);
}

}  // namespace mk
}  // namespace selattn
