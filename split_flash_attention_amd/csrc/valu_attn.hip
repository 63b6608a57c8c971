// Generic vector-ALU attention kernels: every storage type, decode and mask-mode
// prefill (selection mode runs on the matrix-core kernels only).
//
// One work-group owns up to 32 query vectors (a query vector is one (row,
// query head) pair of one kv head) and walks a key range in tiles of 32 keys
// with the online softmax of TensorFold PR #985 ("What this changes": a running
// max per fixed key tile, the correction exp(m_old - m_new), l and o rescaled,
// o / l at the end).  Tiles are fixed by key position, so results do not depend
// on how the range is split among work-groups beyond the slice boundaries.
//
// Also here: the log-sum-exp merge of split partials (TensorFold PR #2595
// attn_merge; strix-llama.cpp PR #115 split-K reduce) with NaN carried through
// (HartsyInference PR #910, review item 1 and its fix).
#include "common.h"
#include "device_cache.h"
#include "internal.h"

#include <algorithm>
#include <type_traits>

namespace selattn {
namespace {

constexpr int kTile = 32;       // keys per tile
constexpr int kQv = 32;         // query vectors per work-group
constexpr int kThreads = 256;
constexpr int kMaxD = 256;
constexpr int kCombineRound = 8;   // partial slices per lane in flight in the combine

enum Mode : int { kDecode = 0, kMask = 1 };

struct ValuParams {
    int mode;
    int Hq, Hkv, G, D;
    const float* q;
    const void* k;
    const void* v;
    int dt;
    int64_t kv_ss, kv_sc, kv_sh;
    const float* ksc;
    const float* vsc;
    int64_t sc_ss, sc_sc, sc_sh;
    float scale, softcap;
    const float* alibi;
    // decode
    int S, R, cap;
    const int32_t* kv_len;
    int causal;
    int slice_len, n_slices_max, n_qchunks;
    // prefill (mask mode)
    int n_kv;
    const int32_t* q_pos;
    const float* mask;
    int64_t m_sr, m_sh;
    int rows_per_wg, n_splits, split_step;
    // outputs
    float* out;
    float* part_o;
    float* part_ml;
    int64_t* dbg_visit;
    const int32_t* tree;       // decode: [S][R] parent tables of tree windows, or null
    const float* sinks;        // prefill without splits: [Hq] sink logits, or null
};

// LDS carve-up (bytes)
constexpr int kOffQ = 0;                                         // float [kQv][kMaxD]
// K rows are padded by 4 floats: 16-byte aligned for float4 reads, and the 16 rows one
// such read of a half-wave touches start on distinct bank groups
constexpr int kKs = kMaxD + 4;                                   // K row stride (floats)
constexpr int kOffK = kOffQ + kQv * kMaxD * 4;                   // float [kTile][kKs]
constexpr int kOffV = kOffK + kTile * kKs * 4;                   // float [kTile][kMaxD]
constexpr int kOffP = kOffV + kTile * kMaxD * 4;                 // float [kQv][kTile]
constexpr int kSmemBytes = kOffP + kQv * kTile * 4;

__global__ __launch_bounds__(kThreads) void valu_attn_kernel(ValuParams p) {
    extern __shared__ __align__(16) char smem[];
    float* qs = reinterpret_cast<float*>(smem + kOffQ);
    float* kt = reinterpret_cast<float*>(smem + kOffK);
    float* vt = reinterpret_cast<float*>(smem + kOffV);
    float* ps = reinterpret_cast<float*>(smem + kOffP);

    __shared__ int cell_t[kTile];
    __shared__ uint32_t vis[kQv];
    __shared__ float m_run[kQv], l_run[kQv], c_run[kQv];
    __shared__ int nan_run[kQv];
    __shared__ long long dbg[kQv][3];
    __shared__ unsigned long long tpath[kQv];     // tree windows: window nodes each query vector sees

    const int tid = threadIdx.x;
    const int D = p.D;
    const int G = p.G;
    const int t_split = blockIdx.x;
    const int g = blockIdx.y % p.Hkv;

    // ---- work unit ------------------------------------------------------
    int b = 0, m0 = 0, nq = 0, lo = 0, hi = 0, kvl = 0, row0 = 0;
    if (p.mode == kDecode) {
        b = blockIdx.z;
        const int qc = blockIdx.y / p.Hkv;
        kvl = min(max(p.kv_len[b], 0), p.cap);
        lo = t_split * p.slice_len;
        if (lo >= kvl) return;          // past this stream's slices: not written
        hi = min(lo + p.slice_len, kvl);
        m0 = qc * kQv;
        nq = min(kQv, p.R * G - m0);
        if (nq <= 0) return;
    } else {
        row0 = blockIdx.z * p.rows_per_wg;
        nq = min(p.rows_per_wg, p.R - row0) * G;
        lo = t_split * p.split_step;
        hi = min(lo + p.split_step, p.n_kv);
    }

    // query vector i -> (row, head)
    auto qrow = [&](int i) -> int {
        return p.mode == kDecode ? (m0 + i) / G : row0 + i / G;
    };
    auto qhead = [&](int i) -> int {
        return g * G + (p.mode == kDecode ? (m0 + i) % G : i % G);
    };
    auto qpos = [&](int i) -> int {
        return p.mode == kDecode ? kvl - p.R + qrow(i) : (p.q_pos ? p.q_pos[qrow(i)] : 0);
    };
    auto qvec_ptr = [&](int i) -> const float* {
        const int r = qrow(i), h = qhead(i);
        if (p.mode == kDecode) return p.q + ((static_cast<int64_t>(b) * p.R + r) * p.Hq + h) * D;
        return p.q + (static_cast<int64_t>(r) * p.Hq + h) * D;
    };

    // ---- load Q, init state ---------------------------------------------
    // (float4 pieces, every load of a thread issued before the stores: Q is 16-byte
    // aligned and D a multiple of 4)
    {
        constexpr int NQ4 = kQv * kMaxD / 4 / kThreads;
        float4 qr[NQ4];
#pragma unroll
        for (int u = 0; u < NQ4; ++u) {
            const int e = (tid + u * kThreads) * 4;
            if (e < nq * D) qr[u] = *reinterpret_cast<const float4*>(qvec_ptr(e / D) + e % D);
        }
#pragma unroll
        for (int u = 0; u < NQ4; ++u) {
            const int e = (tid + u * kThreads) * 4;
            if (e < nq * D) *reinterpret_cast<float4*>(qs + (e / D) * kMaxD + e % D) = qr[u];
        }
    }
    if (tid < kQv) {
        m_run[tid] = kNegInf;
        l_run[tid] = 0.f;
        c_run[tid] = 0.f;
        nan_run[tid] = 0;
        dbg[tid][0] = dbg[tid][1] = dbg[tid][2] = 0;
        // Tree windows (TensorFold PR #2595, kernel contract: heap-order parents):
        // the row's node and its ancestors; a parent entry outside [-1, a) ends the
        // walk, and the node index falls at every step, so it ends within R steps.
        unsigned long long path = 0;
        if (p.mode == kDecode && p.tree && tid < nq) {
            const int32_t* par = p.tree + static_cast<int64_t>(b) * p.R;
            int a = qrow(tid);
            while (a >= 0) {
                path |= 1ull << a;
                const int up = par[a];
                a = (up >= -1 && up < a) ? up : -1;
            }
        }
        tpath[tid] = path;
    }

    const int n_slots = hi - lo;
    __syncthreads();

    // cell of key slot k
    auto slot_cell = [&](int k) -> int { return lo + k; };
    // visibility of cell c for query vector i (c >= 0)
    auto visible = [&](int i, int c) -> bool {
        if (p.mode == kDecode) {
            if (p.tree) {
                const int t0 = kvl - p.R;
                return c < kvl && (c < t0 || ((tpath[i] >> (c - t0)) & 1ull));
            }
            const int lim = p.causal ? min(qpos(i) + 1, kvl) : kvl;
            return c < lim;
        }
        const float mv = p.mask[static_cast<int64_t>(qrow(i)) * p.m_sr +
                                static_cast<int64_t>(qhead(i)) * p.m_sh + c];
        if (mv == kNegInf) return false;
        return !(p.causal && c > qpos(i));
    };

    const int NI = kThreads / D;                 // query-vector groups in the P.V step
    const int d_own = tid % D;
    const int ig = tid / D;
    float acc[kQv];
#pragma unroll
    for (int u = 0; u < kQv; ++u) acc[u] = 0.f;

    for (int t0 = 0; t0 < n_slots; t0 += kTile) {
        if (tid < kTile) {
            const int k = t0 + tid;
            cell_t[tid] = k < n_slots ? slot_cell(k) : -1;
        }
        __syncthreads();
        // visibility bits (also decides which keys are loaded at all)
        if (tid < nq) {
            uint32_t bits = 0;
            for (int s = 0; s < kTile; ++s) {
                const int c = cell_t[s];
                if (c >= 0 && visible(tid, c)) bits |= 1u << s;
            }
            vis[tid] = bits;
        }
        __syncthreads();
        uint32_t any = 0;
        for (int i = 0; i < nq; ++i) any |= vis[i];
        if (any == 0) {            // nobody sees this tile: nothing is read
            __syncthreads();
            continue;
        }
        // stage K and V of the keys somebody sees: every 16-byte piece of the tile's
        // rows this thread takes is loaded at once (one round trip to memory per
        // tile), then widened to fp32 into LDS; storage type fixed per instantiation.
        // (The host checks that K, V and their strides are 16-byte aligned.)
        auto stage = [&](auto dt_tag) {
            constexpr int DT = decltype(dt_tag)::value;
            constexpr int ES = DT == SEL_ATTN_F32 ? 4 : ((DT == SEL_ATTN_F16 || DT == SEL_ATTN_BF16) ? 2 : 1);
            constexpr int EPC = 16 / ES;                          // elements per 16-byte piece
            constexpr int NPC = (kTile * kMaxD / EPC + kThreads - 1) / kThreads;   // pieces per thread
            const int cpr = D / EPC;                              // pieces per row
            const int n_pc = kTile * cpr;
            uint4 kr[NPC], vr[NPC];
            float ks[NPC], vs[NPC];
#pragma unroll
            for (int i = 0; i < NPC; ++i) {
                const int e = tid + i * kThreads;
                kr[i] = vr[i] = uint4{0u, 0u, 0u, 0u};
                ks[i] = vs[i] = 1.f;
                if (e < n_pc) {
                    const int s = e / cpr, ch = e % cpr;
                    const int c = cell_t[s];
                    if (c >= 0 && ((any >> s) & 1u)) {
                        const int64_t base = (p.mode == kDecode ? static_cast<int64_t>(b) * p.kv_ss : 0) +
                                             static_cast<int64_t>(c) * p.kv_sc +
                                             static_cast<int64_t>(g) * p.kv_sh + static_cast<int64_t>(ch) * EPC;
                        kr[i] = *reinterpret_cast<const uint4*>(static_cast<const char*>(p.k) + base * ES);
                        vr[i] = *reinterpret_cast<const uint4*>(static_cast<const char*>(p.v) + base * ES);
                        if constexpr (DT == SEL_ATTN_I8 || DT == SEL_ATTN_FP8) {
                            const int64_t sb = (p.mode == kDecode ? static_cast<int64_t>(b) * p.sc_ss : 0) +
                                               static_cast<int64_t>(c) * p.sc_sc +
                                               static_cast<int64_t>(g) * p.sc_sh;
                            ks[i] = p.ksc[sb];
                            vs[i] = p.vsc[sb];
                        }
                    }
                }
            }
            // element j of a 16-byte piece as a float (exact widening)
            auto elem = [](const uint4& w, int j) -> float {
                const uint32_t x = (j * ES / 4 == 0) ? w.x : (j * ES / 4 == 1) ? w.y : (j * ES / 4 == 2) ? w.z : w.w;
                if constexpr (DT == SEL_ATTN_F32) return __uint_as_float(x);
                else if constexpr (DT == SEL_ATTN_BF16) return bf16_to_f32(static_cast<uint16_t>(x >> (16 * (j & 1))));
                else if constexpr (DT == SEL_ATTN_F16) return f16_to_f32(static_cast<uint16_t>(x >> (16 * (j & 1))));
                else if constexpr (DT == SEL_ATTN_FP8) return e4m3_to_f32((x >> (8 * (j & 3))) & 0xffu);
                else return static_cast<float>(static_cast<int8_t>((x >> (8 * (j & 3))) & 0xffu));
            };
#pragma unroll
            for (int i = 0; i < NPC; ++i) {
                const int e = tid + i * kThreads;
                if (e < n_pc) {
                    const int s = e / cpr, d0 = (e % cpr) * EPC;
#pragma unroll
                    for (int j = 0; j < EPC; ++j) {
                        float kx = elem(kr[i], j), vx = elem(vr[i], j);
                        if constexpr (DT == SEL_ATTN_I8 || DT == SEL_ATTN_FP8) {
                            kx *= ks[i];
                            vx *= vs[i];
                        }
                        kt[s * kKs + d0 + j] = kx;
                        vt[s * kMaxD + d0 + j] = vx;
                    }
                }
            }
        };
        switch (p.dt) {
        case SEL_ATTN_F32: stage(std::integral_constant<int, SEL_ATTN_F32>{}); break;
        case SEL_ATTN_F16: stage(std::integral_constant<int, SEL_ATTN_F16>{}); break;
        case SEL_ATTN_BF16: stage(std::integral_constant<int, SEL_ATTN_BF16>{}); break;
        case SEL_ATTN_FP8: stage(std::integral_constant<int, SEL_ATTN_FP8>{}); break;
        default: stage(std::integral_constant<int, SEL_ATTN_I8>{}); break;
        }
        __syncthreads();
        // scores of visible pairs
        for (int e = tid; e < kQv * kTile; e += kThreads) {
            const int i = e / kTile, s = e % kTile;
            if (i >= nq || !((vis[i] >> s) & 1u)) continue;
            // four partial sums (D is a multiple of 4), so the multiply-adds overlap;
            // Q and K read four floats at a time
            float d0 = 0.f, d1 = 0.f, d2 = 0.f, d3 = 0.f;
            const float* qi = qs + i * kMaxD;
            const float* ks = kt + s * kKs;
#pragma unroll 4
            for (int d = 0; d < D; d += 4) {
                const float4 q4 = *reinterpret_cast<const float4*>(qi + d);
                const float4 k4 = *reinterpret_cast<const float4*>(ks + d);
                d0 = fmaf(q4.x, k4.x, d0);
                d1 = fmaf(q4.y, k4.y, d1);
                d2 = fmaf(q4.z, k4.z, d2);
                d3 = fmaf(q4.w, k4.w, d3);
            }
            const float dot = (d0 + d1) + (d2 + d3);
            const int c = cell_t[s];
            const float slope = p.alibi ? p.alibi[qhead(i)] : 0.f;
            const float mv = p.mode == kMask
                                 ? p.mask[static_cast<int64_t>(qrow(i)) * p.m_sr +
                                          static_cast<int64_t>(qhead(i)) * p.m_sh + c]
                                 : 0.f;
            ps[i * kTile + s] = score_pipeline(dot, p.scale, p.softcap, slope, c - qpos(i), mv);
        }
        __syncthreads();
        // online softmax update: a group of 32 threads per query vector, one thread
        // per key of the tile, the maximum, NaN flag and sum reduced by lane exchanges
        for (int i0 = 0; i0 < nq; i0 += kThreads / kTile) {
            const int i = i0 + tid / kTile;
            const int s = tid % kTile;
            const bool live = i < nq;
            const uint32_t bits = live ? vis[i] : 0u;
            const bool v = (bits >> s) & 1u;
            const float x = v ? ps[i * kTile + s] : kNegInf;
            int nanf = (v && x != x) ? 1 : 0;
            float mt = (v && x == x) ? x : kNegInf;
#pragma unroll
            for (int o = 1; o < kTile; o <<= 1) {
                mt = max_keep(mt, __shfl_xor(mt, o, kTile));
                nanf |= __shfl_xor(nanf, o, kTile);
            }
            const float m_old = live ? m_run[i] : kNegInf;
            const float m_new = max_keep(m_old, mt);
            const float c = rescale_factor(m_old, m_new);
            const float pe = v ? exp_diff(x, m_new) : 0.f;
            if (v) ps[i * kTile + s] = pe;
            float lsum = pe;
#pragma unroll
            for (int o = 1; o < kTile; o <<= 1) lsum += __shfl_xor(lsum, o, kTile);
            if (live && s == 0) {
                l_run[i] = l_run[i] * c + lsum;
                m_run[i] = m_new;
                c_run[i] = c;
                nan_run[i] = nan_run[i] | nanf;
                // visit counts of the row (its first query head), when asked for
                if (p.dbg_visit && ((p.mode == kDecode ? m0 + i : i) % G) == 0) {
                    long long n_vis = 0, sum_vis = 0, sq_vis = 0;
                    for (int t = 0; t < kTile; ++t) {
                        if (!((bits >> t) & 1u)) continue;
                        const long long cc = cell_t[t];
                        n_vis += 1;
                        sum_vis += cc;
                        sq_vis += cc * cc;
                    }
                    dbg[i][0] += n_vis;
                    dbg[i][1] += sum_vis;
                    dbg[i][2] += sq_vis;
                }
            }
        }
        __syncthreads();
        // o = o * c + sum_s p_s v_s over visible keys only
        if (ig < NI) {
            for (int u = 0; u < kQv; ++u) {
                const int i = ig + u * NI;
                if (i >= nq) break;
                const uint32_t bits = vis[i];
                // four partial sums over the tile's keys; a key the query vector does
                // not see is skipped (its V may hold anything)
                float a0 = acc[u] * c_run[i], a1 = 0.f, a2 = 0.f, a3 = 0.f;
#pragma unroll
                for (int s = 0; s < kTile; s += 4) {
                    const float4 p4 = *reinterpret_cast<const float4*>(ps + i * kTile + s);   // (one read, broadcast)
                    if ((bits >> s) & 1u) a0 = fmaf(p4.x, vt[s * kMaxD + d_own], a0);
                    if ((bits >> (s + 1)) & 1u) a1 = fmaf(p4.y, vt[(s + 1) * kMaxD + d_own], a1);
                    if ((bits >> (s + 2)) & 1u) a2 = fmaf(p4.z, vt[(s + 2) * kMaxD + d_own], a2);
                    if ((bits >> (s + 3)) & 1u) a3 = fmaf(p4.w, vt[(s + 3) * kMaxD + d_own], a3);
                }
                acc[u] = (a0 + a1) + (a2 + a3);
            }
        }
        __syncthreads();
    }

    // ---- epilogue -----------------------------------------------------------
    if (ig < NI) {
        for (int u = 0; u < kQv; ++u) {
            const int i = ig + u * NI;
            if (i >= nq) break;
            const int r = qrow(i), h = qhead(i);
            const float m = m_run[i], l = l_run[i];
            const bool split = p.mode == kDecode || p.n_splits > 1;
            const float z = (!split && p.sinks) ? p.sinks[h] : kNegInf;   // sink logit, unsplit only
            const bool bad = nan_run[i] || m == kPosInf || z != z || z == kPosInf;
            const bool empty = !bad && m == kNegInf;
            if (!split) {
                // with a sink (HartsyInference PR #910): M = max(m, z), and the
                // denominator gains exp(z - M)
                float f = 1.f / l;
                if (z != kNegInf && !bad && !empty) {
                    const float big = max_keep(m, z);
                    const float e = exp2f((m - big) * kLog2e);
                    f = e / fmaf(l, e, exp2f((z - big) * kLog2e));
                }
                float o = bad ? __builtin_nanf("") : (empty ? 0.f : acc[u] * f);
                p.out[(static_cast<int64_t>(r) * p.Hq + h) * D + d_own] = o;
            } else {
                int64_t pi;
                if (p.mode == kDecode)
                    pi = ((static_cast<int64_t>(b) * p.R + r) * p.Hq + h) * p.n_slices_max + t_split;
                else
                    pi = (static_cast<int64_t>(r) * p.Hq + h) * p.n_splits + t_split;
                p.part_o[pi * D + d_own] = empty ? 0.f : acc[u];
                if (d_own == 0) {
                    p.part_ml[pi * 2 + 0] = nan_run[i] ? __builtin_nanf("") : m;
                    p.part_ml[pi * 2 + 1] = bad ? __builtin_nanf("") : (empty ? 0.f : l);
                }
            }
        }
    }
    if (p.dbg_visit && tid < nq) {
        const int i = tid;
        const bool first_head = ((p.mode == kDecode ? m0 + i : i) % G) == 0;
        if (first_head) {
            const int r = qrow(i);
            int64_t di;
            if (p.mode == kDecode)
                di = ((static_cast<int64_t>(b) * p.R + r) * p.Hkv + g) * p.n_slices_max + t_split;
            else
                di = (static_cast<int64_t>(r) * p.Hkv + g) * p.n_splits + t_split;
            p.dbg_visit[di * 3 + 0] = dbg[i][0];
            p.dbg_visit[di * 3 + 1] = dbg[i][1];
            p.dbg_visit[di * 3 + 2] = dbg[i][2];
        }
    }
}

// ---------------------------------------------------------------------------
// split combine
// ---------------------------------------------------------------------------
// One wave per (stream, row, head), four per work-group.  Lane c of phase sp owns
// float4 column c of the output (L = D / 4 columns) and the slices sp, sp + nph,
// ... (nph = 64 / L phases), so all partial vectors of a row are read with
// independent loads at once; the phases are then summed by lane exchanges.
__global__ __launch_bounds__(256) void combine_kernel(sel_attn_combine_args a, int64_t units) {
    const int64_t unit = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);   // (b, r, h)
    if (unit >= units) return;                    // uniform over the wave
    const int D = a.head_dim;
    const int lane = threadIdx.x & 63;
    const int b = static_cast<int>(unit / (static_cast<int64_t>(a.n_row) * a.n_head_q));
    int ns = a.n_slices_max;
    if (a.kv_len) {
        const int n = min(max(a.kv_len[b], 0), a.cap);
        ns = min((n + a.slice_len - 1) / a.slice_len, a.n_slices_max);
    }
    const float* ml = a.part_ml + unit * a.n_slices_max * 2;
    const float* po = a.part_o + unit * a.n_slices_max * D;
    float* out = a.out + unit * D;

    // M = max over slices and the sink logit (NaN-aware).  The sink (HartsyInference
    // PR #910) is one more logit without a value: it enters M and the denominator.
    const int h = static_cast<int>(unit % a.n_head_q);
    const float z = a.sinks ? a.sinks[h] : kNegInf;
    bool nanf = z != z;
    float M = nanf ? kNegInf : z;
    for (int t = lane; t < ns; t += 64) {
        const float m = ml[2 * t];
        if (m != m) nanf = true;
        else M = max_keep(M, m);
    }
#pragma unroll
    for (int msk = 1; msk < 64; msk <<= 1) M = max_keep(M, __shfl_xor(M, msk, 64));
    nanf = __any(nanf);

    const int L = D / 4;                          // float4 columns of a partial
    const int nph = 64 / L;                       // slice phases
    const int sp = lane / L, c = lane - (lane / L) * L;
    if (nanf || M == kPosInf || M == kNegInf) {
        if (sp == 0) {
#ifdef SELATTN_PLANT_COMBINE_NAN_TO_ZERO
            // test-only planted mistake (never in a product build): NaN becomes 0
            const float x = (!nanf && M == kPosInf) ? __builtin_nanf("") : 0.f;
#else
            const float x = (nanf || M == kPosInf) ? __builtin_nanf("") : 0.f;
#endif
            reinterpret_cast<float4*>(out)[c] = float4{x, x, x, x};
        }
        return;
    }
    // kCombineRound slices per round: every load of the round is issued before any is used
    float4 num = {0.f, 0.f, 0.f, 0.f};
    float den = 0.f;
    for (int t0 = sp; t0 < ns; t0 += kCombineRound * nph) {
        float2 mlv[kCombineRound];
        float4 ov[kCombineRound];
#pragma unroll
        for (int j = 0; j < kCombineRound; ++j) {
            const int t = t0 + j * nph;
            if (t < ns) {
                mlv[j] = reinterpret_cast<const float2*>(ml)[t];
                ov[j] = reinterpret_cast<const float4*>(po + static_cast<int64_t>(t) * D)[c];
            } else {
                mlv[j] = float2{kNegInf, 0.f};
                ov[j] = float4{0.f, 0.f, 0.f, 0.f};
            }
        }
#pragma unroll
        for (int j = 0; j < kCombineRound; ++j) {
            if (mlv[j].x == kNegInf) continue;     // empty slice: contributes nothing
            const float w = exp2f((mlv[j].x - M) * kLog2e);
            den = fmaf(w, mlv[j].y, den);
            num.x = fmaf(w, ov[j].x, num.x);
            num.y = fmaf(w, ov[j].y, num.y);
            num.z = fmaf(w, ov[j].z, num.z);
            num.w = fmaf(w, ov[j].w, num.w);
        }
    }
    for (int msk = L; msk < 64; msk <<= 1) {
        num.x += __shfl_xor(num.x, msk, 64);
        num.y += __shfl_xor(num.y, msk, 64);
        num.z += __shfl_xor(num.z, msk, 64);
        num.w += __shfl_xor(num.w, msk, 64);
        den += __shfl_xor(den, msk, 64);
    }
    if (z != kNegInf) den += exp2f((z - M) * kLog2e);
    if (sp == 0) reinterpret_cast<float4*>(out)[c] = float4{num.x / den, num.y / den, num.z / den, num.w / den};
}

// Raises the kernel's LDS limit once per device (before its first launch there).
hipError_t prepare_kernel() {
    static DeviceCache cache;
    hipError_t err = hipSuccess;
    cache.get(0, [&err]() {
        err = hipFuncSetAttribute(reinterpret_cast<const void*>(&valu_attn_kernel),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, kSmemBytes);
        return err == hipSuccess ? 1 : 0;
    });
    return err;
}

}  // namespace

hipError_t launch_valu_decode(const sel_attn_decode_args& a, hipStream_t st) {
    hipError_t e = prepare_kernel();
    if (e != hipSuccess) return e;
    ValuParams p{};
    p.mode = kDecode;
    p.Hq = a.n_head_q; p.Hkv = a.n_head_kv; p.G = a.n_head_q / a.n_head_kv; p.D = a.head_dim;
    p.q = a.q; p.k = a.k; p.v = a.v; p.dt = a.kv_dtype;
    p.kv_ss = a.kv_stride_stream; p.kv_sc = a.kv_stride_cell; p.kv_sh = a.kv_stride_head;
    p.ksc = a.k_scale; p.vsc = a.v_scale;
    p.sc_ss = a.sc_stride_stream; p.sc_sc = a.sc_stride_cell; p.sc_sh = a.sc_stride_head;
    p.scale = a.scale; p.softcap = a.softcap; p.alibi = a.alibi_slopes;
    p.S = a.n_stream; p.R = a.n_row; p.cap = a.cap; p.kv_len = a.kv_len; p.causal = a.causal;
    p.slice_len = a.slice_len; p.n_slices_max = a.n_slices_max;
    p.n_qchunks = (a.n_row * p.G + kQv - 1) / kQv;
    p.part_o = a.part_o; p.part_ml = a.part_ml; p.dbg_visit = a.dbg_visit;
    p.tree = a.tree_parent;
    const int n_sl = std::min(a.n_slices_max, (a.cap + a.slice_len - 1) / a.slice_len);
    dim3 grid(n_sl, a.n_head_kv * p.n_qchunks, a.n_stream);
    hipLaunchKernelGGL(valu_attn_kernel, grid, dim3(kThreads), kSmemBytes, st, p);
    return hipGetLastError();
}

hipError_t launch_valu_prefill(const sel_attn_prefill_args& a, hipStream_t st) {
    hipError_t e = prepare_kernel();
    if (e != hipSuccess) return e;
    ValuParams p{};
    p.mode = kMask;
    p.Hq = a.n_head_q; p.Hkv = a.n_head_kv; p.G = a.n_head_q / a.n_head_kv; p.D = a.head_dim;
    p.q = a.q; p.k = a.k; p.v = a.v; p.dt = a.kv_dtype;
    p.kv_sc = a.kv_stride_cell; p.kv_sh = a.kv_stride_head;
    p.ksc = a.k_scale; p.vsc = a.v_scale;
    p.sc_sc = a.sc_stride_cell; p.sc_sh = a.sc_stride_head;
    p.scale = a.scale; p.softcap = a.softcap; p.alibi = a.alibi_slopes;
    p.R = a.n_row; p.n_kv = a.n_kv; p.q_pos = a.q_pos;
    p.mask = a.mask; p.m_sr = a.mask_stride_row; p.m_sh = a.mask_stride_head; p.causal = a.causal;
    p.n_splits = a.n_splits;
    p.split_step = (a.n_kv + a.n_splits - 1) / a.n_splits;
    p.rows_per_wg = std::max(1, kQv / p.G);
    p.out = a.out; p.part_o = a.part_o; p.part_ml = a.part_ml;
    p.dbg_visit = a.dbg_visit;
    p.sinks = a.sinks;
    const int n_rb = (a.n_row + p.rows_per_wg - 1) / p.rows_per_wg;
    dim3 grid(a.n_splits, a.n_head_kv, n_rb);
    hipLaunchKernelGGL(valu_attn_kernel, grid, dim3(kThreads), kSmemBytes, st, p);
    return hipGetLastError();
}

hipError_t launch_combine(const sel_attn_combine_args& a, hipStream_t st) {
    const int64_t units = static_cast<int64_t>(a.n_stream) * a.n_row * a.n_head_q;
    hipLaunchKernelGGL(combine_kernel, dim3(static_cast<unsigned>((units + 3) / 4)), dim3(256), 0, st, a, units);
    return hipGetLastError();
}

}  // namespace selattn
