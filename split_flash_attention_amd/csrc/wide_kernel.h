// Matrix-core split-K decode kernel for verify windows with int8 K/V: units of
// many query vectors (16 draft rows x 12 heads = 192 per (stream, slice, kv head)
// for the int8 verify workload), on v_mfma_f32_32x32x16_bf16 with one wave per
// SIMD (TensorFold PR #2595: one work-group per (stream, kv head, slice) of the
// attn_decode grid; partials merged by the log-sum-exp combine afterwards).
//
// A work-group takes a chunk of up to 192 query vectors in 32-column blocks:
// block j belongs to wave j & 3, so waves 0 and 1 own two blocks and waves 2 and
// 3 one.  Block 0 of a wave keeps its Q^T operands in registers, block 1 in this
// wave's part of LDS; the O^T accumulators (up to 256 values a lane) fill the
// AGPRs.  Per 32-key tile:
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
//
// Software pipeline: iteration t
//   * issues the loads of raw tile t + 2 (int8 K and V rows and their row scales),
//     HBM straight into LDS (buffer loads with the LDS destination, no registers);
//   * phase A: S^T of tile t.  Waves 0 and 1 run both their blocks (one K operand
//     read feeds both); waves 2 and 3 alternate their one block's steps between two
//     accumulators and, between the matrix instructions, widen raw tile t + 1 into
//     the bf16 K and V^T tiles;
//   * phase B: the softmax steps of tile t between the matrix instructions of
//     O^T += V^T . P^T of tile t - 1 (one V^T read feeds both blocks);
//   * waits for raw tile t + 2, then one work-group barrier.
// LDS: K tiles (bf16, two buffers: t is read while t + 1 is written), V^T tiles
// with their row scales (three buffers: t - 1 is read, t kept, t + 1 written), raw
// tiles (two buffers), block-1 Q^T of waves 0 and 1.  The barrier is a plain
// s_barrier after the wave's LDS operations, so loads in flight never hold it up.
//
// Register budget (one wave per SIMD: 256 VGPRs, 256 AGPRs): the score
// accumulators stay in VGPRs (inline asm) since the O^T accumulators take the
// AGPRs; the rare rescale of the accumulators goes through a short AGPR sequence.
// K rows in LDS are padded by 16 bytes so that one base register plus an immediate
// addresses every step and the 32 rows of an operand read fall on distinct bank
// groups.  A key no query vector of the chunk can see is never loaded; keys some
// query vectors see and others don't are excluded per score (int8 V is always
// finite and its row scale joins visible weights only).
#pragma once

#include <type_traits>

#include "mfma_kernel.h"

namespace selattn {
namespace mk {

constexpr int kWT = 32;          // keys per tile
constexpr int kWW = 4;           // waves per work-group
constexpr int kWQ = 192;         // query vectors per work-group: six 32-column blocks
constexpr int kW2 = 2;           // waves holding a second block

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

// Work-group barrier of the pipelined loop: the wave's LDS operations complete,
// then s_barrier.  Unlike __syncthreads it does not wait for the wave's buffer
// loads, so the raw tiles in flight to LDS keep streaming through it; a raw tile
// is waited for explicitly (wait_vm) before the barrier that publishes it.
// The memory clobber keeps the compiler from moving LDS accesses across it.
__device__ __forceinline__ void wide_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }
// LDS of the pipeline (bytes): K tile [32 keys][D] bf16 in rows padded by 16
// bytes; V^T tile [4 groups][D dims][8 keys] bf16 followed by the tile's K and V
// row scales [32] + [32]; raw tile: K [32][D] int8, V [32][D] int8, K scales [64],
// V scales [64] (slots of 64 keys, of which the loads fill the tile's 32).
template <int D>
constexpr int wide_krow() { return D * 2 + 16; }
template <int D>
constexpr int wide_kbuf() { return kWT * wide_krow<D>(); }
template <int D>
constexpr int wide_vbuf() { return D * kWT * 2 + 2 * kWT * 4; }
template <int D>
constexpr int wide_rbuf() { return 2 * kWT * D + 2 * 64 * 4; }
template <int D>
constexpr int wide_off_v() { return 2 * wide_kbuf<D>(); }
template <int D>
constexpr int wide_off_raw() { return wide_off_v<D>() + 3 * wide_vbuf<D>(); }
template <int D>
constexpr int wide_off_q1() { return wide_off_raw<D>() + 2 * wide_rbuf<D>(); }
template <int D>
constexpr int wide_off_tpath() { return wide_off_q1<D>() + kW2 * (D / 16) * 1024; }
template <int D>
constexpr int wide_smem() { return wide_off_tpath<D>() + kWQ * 8 + kWQ * 24 + kWQ * 4; }
static_assert(wide_smem<256>() <= 160 * 1024, "LDS of the D = 256 pipeline");

// Key of score i (0..15) of a lane in half h of the wave: 8 (i / 4) + 4 h + i % 4.
// Contraction chunk c of P.V takes the lane's scores 8c .. 8c + 7, i.e. the keys of
// V^T group 2c + h in this order.
__device__ __forceinline__ int wide_key(int i, int h) { return 8 * (i >> 2) + 4 * h + (i & 3); }

// byte offset of 16-byte chunk ch (dims 8 ch .. 8 ch + 7) of key row `key` in the K tile
template <int D>
__device__ __forceinline__ int wk_off(int key, int ch) { return key * wide_krow<D>() + (ch << 4); }
// byte offset of the 8 keys of group g at dim d in the V^T tile.  The 16-byte chunks
// of a group are stored in the order d ^ ((d >> 4) & 3): the widening writes dims
// 4 vq + dd of consecutive vq, 64 bytes apart, which would otherwise fall on 4 bank
// groups only; the operand reads (32 consecutive dims) only get permuted.
template <int D>
__device__ __forceinline__ int wv_off(int g, int d) { return (g * D + (d ^ ((d >> 4) & 3))) << 4; }

// o *= c for an accumulator held in an AGPR: read into a VGPR, multiply, write back
// (keeps the accumulators in the AGPRs through the rare rescale)
__device__ __forceinline__ void agpr_scale(float& o, float c) {
    float t;
    asm volatile("v_accvgpr_read_b32 %1, %0\n\tv_mul_f32 %1, %1, %2\n\tv_accvgpr_write_b32 %0, %1"
                 : "+a"(o), "=&v"(t)
                 : "v"(c));
}

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
    constexpr int K_TASKS = kWT * D / 16;        // widening: 16 int8 of one key row each
    constexpr int V_TASKS = 4 * D / 4;           // (group, 4 dims): 4 bytes of 8 rows each
    constexpr int NKL = (K_TASKS + NT - 1) / NT;
    constexpr int NDMA = kWT * D / 1024 / kWW;   // 1 KiB raw loads per wave, for K and for V
    constexpr int KBUF = wide_kbuf<D>();
    constexpr int VBUF = wide_vbuf<D>();
    constexpr int RBUF = wide_rbuf<D>();
    static_assert(V_TASKS <= NT && NKL <= 2 && NDMA >= 1, "task split");
    static_assert(2 * NDB == NS, "the O^T and S^T phases have the same step count");

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: scalar branches
    const int lane = tid & 63;
    const int l32 = lane & 31;
    const int h = lane >> 5;
    const int G = p.G;

    char* q1_lds = smem + wide_off_q1<D>() + wave * (NS * 1024) + lane * 16;   // waves 0, 1 only
    unsigned long long* tpath_lds = reinterpret_cast<unsigned long long*>(smem + wide_off_tpath<D>());   // [192]
    unsigned long long* dbg_lds = tpath_lds + kWQ;                                                   // [192][3]
    // ALiBi slope of each query vector: read from LDS in the loop, which then holds
    // no global load (a global load there would make the compiler wait for every
    // buffer load in flight, the raw tiles included, before reusing its register)
    float* slope_lds = reinterpret_cast<float*>(dbg_lds + 3 * kWQ);                                   // [192]

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

    // this wave's blocks: wave and wave + 4 of the chunk (the second for waves 0, 1)
    int blk[2];
    bool live[2];
    int qv_r[2], qv_h[2], qv_lim[2];
    bool qv_ok[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        blk[k] = wave + 4 * k;
        const int m0 = m_wg + 32 * blk[k];
        live[k] = (k == 0 || wave < kW2) && m0 < m_end;   // uniform over the wave
        const int m = m0 + l32;
        bool ok = live[k] && m < m_end;
        int r = m / G, hh = g * G + m % G;
        ok = ok && r < p.R;
        if (!ok) { r = 0; hh = g * G; }
        qv_ok[k] = ok;
        qv_r[k] = r;
        qv_h[k] = hh;
        const int pos = kvl - p.R + r;
        qv_lim[k] = ok ? min((p.causal && !tree) ? min(pos + 1, kvl) : kvl, hi) : -1;
        if (p.alibi && h == 0 && (k == 0 || wave < kW2)) slope_lds[32 * blk[k] + l32] = ok ? p.alibi[hh] : 0.f;
        if constexpr (TREE) {
            if (k == 0 || wave < kW2) {              // uniform: every lane takes part
                const unsigned long long path =
                    tree_path_mask_wave(p.tree + static_cast<int64_t>(b) * p.R, p.R, r);
                if (h == 0) tpath_lds[32 * blk[k] + l32] = path;
            }
        }
    }

    // Q^T operands, scale folded in: step st of lane l holds Q[qv l & 31][16 st + 8 h + j],
    // j = 0..7; block 0's in registers, block 1's in this wave's part of LDS
    u32x4 qop[NS];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        if (k == 1 && wave >= kW2) break;        // uniform
        const float* qp = p.q + ((static_cast<int64_t>(b) * p.R + qv_r[k]) * p.Hq + qv_h[k]) * D;
        const unsigned qmask = qv_ok[k] ? 0xffffffffu : 0u;
#pragma unroll
        for (int st = 0; st < NS; ++st) {
            // every lane loads (lanes without a query vector read a valid one, whose
            // bits are then masked off): no lane-divergent branch around the loads,
            // which would make the compiler wait for each load in turn (a select of a
            // loaded value is turned into such a branch, a mask is not)
            const float4 a = *reinterpret_cast<const float4*>(qp + 16 * st + 8 * h);
            const float4 c = *reinterpret_cast<const float4*>(qp + 16 * st + 8 * h + 4);
            const float x[8] = {a.x, a.y, a.z, a.w, c.x, c.y, c.z, c.w};
            u32x4 w;
#pragma unroll
            for (int j = 0; j < 4; ++j) w[j] = pack2<false>(x[2 * j] * p.scale, x[2 * j + 1] * p.scale) & qmask;
            if (k == 0) qop[st] = w;
            else *reinterpret_cast<u32x4*>(q1_lds + st * 1024) = w;
        }
    }

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

    // ---- raw tile loads, HBM -> LDS ----------------------------------------------
    // Buffer loads through descriptors that start at the unit's first key row and
    // end with its last needed row: rows past it read as zeros (the range check
    // covers the scalar offset, which carries the tile's row).  32-bit offsets:
    // cap * cell stride < 2^31 (and the same for the scales) is checked on the host.
    const int cb = static_cast<int>(p.kv_sc);
    const int64_t kv_base = static_cast<int64_t>(b) * p.kv_ss + static_cast<int64_t>(g) * p.kv_sh;
    const int64_t sc_base = static_cast<int64_t>(b) * p.sc_ss + static_cast<int64_t>(g) * p.sc_sh;
    const char* kbase = static_cast<const char*>(p.k) + kv_base + static_cast<int64_t>(lo) * p.kv_sc;
    const char* vbase = static_cast<const char*>(p.v) + kv_base + static_cast<int64_t>(lo) * p.kv_sc;
    const int nrec = n_keys > 0 ? (n_keys - 1) * cb + D : 0;
    const i32x4_t krs = raw_rsrc(kbase, nrec);
    const i32x4_t vrs = raw_rsrc(vbase, nrec);
    const int scb = static_cast<int>(p.sc_sc) * 4;
    const int nsc = n_keys > 0 ? (n_keys - 1) * scb + 4 : 0;
    const int64_t sc_first = sc_base + static_cast<int64_t>(lo) * p.sc_sc;
    const i32x4_t srs = raw_rsrc((wave == 0 ? p.ksc : p.vsc) + sc_first, nsc);
    // Wave w loads the 1 KiB pieces w NDMA .. w NDMA + NDMA - 1 of the raw K and V
    // rows (lane l: the 16 bytes at piece offset 16 l, i.e. row (1024 c + 16 l) / D),
    // wave 0 the K scales and wave 1 the V scales (lane l < 32: key l).  A wave thus has
    // 2 NDMA loads in flight per tile, 2 NDMA + 1 for waves 0 and 1.
    auto dma_tile = [&](int t) __attribute__((always_inline)) {
        char* raw = smem + wide_off_raw<D>() + (t & 1) * RBUF;
        const int soff = t * kWT * cb;
        // the per-lane offsets are recomputed here rather than kept across the loop
        int ln = lane;
        asm volatile("" : "+v"(ln));
#pragma unroll
        for (int i = 0; i < NDMA; ++i) {
            const int c = wave * NDMA + i;
            const int o = 1024 * c + 16 * ln;
            const int voff = (o / D) * cb + o % D;
            lds_dma<16>(krs, lds_addr(raw + 1024 * c), voff, soff);
            lds_dma<16>(vrs, lds_addr(raw + kWT * D + 1024 * c), voff, soff);
        }
        // (lanes of keys past the tile load nothing: the scales of the kv heads
        // interleave, so every extra key would fetch another sector)
        if (wave < 2 && ln < kWT) lds_dma<4>(srs, lds_addr(raw + 2 * kWT * D + wave * 256), ln * scb, t * kWT * scb);
    };
    // ---- widening raw tile -> K tile (bf16) and V^T tile (bf16) + row scales --------
    // Done by waves 2 and 3 alone (threads wt = tid - 128), which own one block and
    // would otherwise wait at the barriers for waves 0 and 1 and their two blocks.
    // Part p < NKW: K task wt + NW p (row e / (D / 16), 16 dims e % (D / 16)); then
    // 4 parts per V task wt + NW i (group vg, dims 4 vq .. 4 vq + 3), one dim each;
    // last part: the row scales (wt < 64).  All raw reads go out first (widen_read).
    constexpr int NW = 128;
    constexpr int NKW = K_TASKS / NW;            // K tasks per widening thread
    constexpr int NVW = V_TASKS / NW;            // V tasks per widening thread
    constexpr int NPARTS = NKW + 4 * NVW + 1;
    static_assert(K_TASKS % NW == 0 && V_TASKS % NW == 0 && NPARTS < NS, "widening split");
    u32x4 kraw[NKW];
    uint32_t vraw[NVW][8];
    float sraw;
    auto wt_now = [&]() __attribute__((always_inline)) {
        // recomputed where used rather than kept across the loop
        unsigned tq = static_cast<unsigned>(tid) - NW;
        asm volatile("" : "+v"(tq));
        return tq;
    };
    auto widen_read = [&](int t) __attribute__((always_inline)) {
        const unsigned wt = wt_now();
        const char* raw = smem + wide_off_raw<D>() + (t & 1) * RBUF;
#pragma unroll
        for (int i = 0; i < NKW; ++i) kraw[i] = *reinterpret_cast<const u32x4*>(raw + 16 * (wt + i * NW));
#pragma unroll
        for (int i = 0; i < NVW; ++i) {
            const unsigned v = wt + i * NW, vg = v / (D / 4), vq = v % (D / 4);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const unsigned key = 16 * (vg >> 1) + 8 * (j >> 2) + 4 * (vg & 1) + (j & 3);
                vraw[i][j] = *reinterpret_cast<const uint32_t*>(raw + kWT * D + key * D + 4 * vq);
            }
        }
        sraw = reinterpret_cast<const float*>(raw + 2 * kWT * D)[(wt / kWT % 2) * 64 + wt % kWT];
    };
    auto widen = [&](int t, auto partc) __attribute__((always_inline)) {
        constexpr int part = decltype(partc)::value;
        const unsigned wt = wt_now();
        char* kt = smem + (t & 1) * KBUF;
        char* vt = smem + wide_off_v<D>() + (t % 3) * VBUF;
        if constexpr (part < NKW) {
            const unsigned e = wt + part * NW;
            const int key = e / (D / 16), c16 = e % (D / 16);
            const u32x4 w = kraw[part];
            u32x4 w0, w1;
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                w0[2 * j] = kpair_bf16<KT>(w[j], 0);
                w0[2 * j + 1] = kpair_bf16<KT>(w[j], 1);
                w1[2 * j] = kpair_bf16<KT>(w[2 + j], 0);
                w1[2 * j + 1] = kpair_bf16<KT>(w[2 + j], 1);
            }
            *reinterpret_cast<u32x4*>(kt + wk_off<D>(key, 2 * c16)) = w0;
            *reinterpret_cast<u32x4*>(kt + wk_off<D>(key, 2 * c16 + 1)) = w1;
        } else if constexpr (part < NKW + 4 * NVW) {
            constexpr int i = (part - NKW) / 4, dd = (part - NKW) % 4;
            const unsigned v = wt + i * NW, vg = v / (D / 4), vq = v % (D / 4);
            u32x4 o;
#pragma unroll
            for (int j = 0; j < 4; ++j) o[j] = bpair_bf16<KT>(vraw[i][2 * j], dd, vraw[i][2 * j + 1], dd);
            *reinterpret_cast<u32x4*>(vt + wv_off<D>(vg, 4 * vq + dd)) = o;
        } else {
            if (wt < 2 * kWT) reinterpret_cast<float*>(vt + D * kWT * 2)[wt] = sraw;
        }
    };

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
            if (k == 1 && wave >= kW2) break;
            unsigned long long* d = dbg_lds + (32 * blk[k] + l32) * 3;
            d[0] = d[1] = d[2] = 0ull;
        }
    }
    // operand read bases: K (key l32, dims 8 h ..), V^T (group h, dim l32)
    const int kread = wk_off<D>(l32, h);
    // (dim 32 db + l32 sits at chunk 32 db + (l32 ^ ((l32 >> 4) ^ 2 (db & 1))))
    const int vread_even = wide_off_v<D>() + wv_off<D>(h, l32);
    const int vread_odd = wide_off_v<D>() + wv_off<D>(h, 32 + l32) - 32 * 16;

    // ---- online softmax of one block, in 16 stages --------------------------------
    // Stage q of block k works in place on the tile's scores s (lane: 16 scores of
    // its query vector, keys wide_key(i, h)); the stages are spread over the matrix
    // products of the next tile so that the vector ALU work runs while the matrix
    // core is busy.  ksr / vsr: the tile's K and V row scales of the lane's 16 keys.
    float4 ksr[4], vsr[4];
    struct Smx {
        uint32_t vword;     // visibility of the tile's key slots (partial tiles)
        bool full;          // every key of the tile is seen by every query vector
        bool resc;          // (uniform) the O^T accumulators take the factor c ...
        float c;            // ... once the previous tile's products are in
        float mls;
        u32x4 pop[2];       // P^T operands of the tile's two 16-key halves
    };
    auto read_ks = [&](int t) __attribute__((always_inline)) {
        const float* sc = reinterpret_cast<const float*>(smem + wide_off_v<D>() + (t % 3) * VBUF + D * kWT * 2);
#pragma unroll
        for (int a = 0; a < 4; ++a) ksr[a] = *reinterpret_cast<const float4*>(sc + 8 * a + 4 * h);
    };
    auto read_vs = [&](int t) __attribute__((always_inline)) {
        const float* sc = reinterpret_cast<const float*>(smem + wide_off_v<D>() + (t % 3) * VBUF + D * kWT * 2);
#pragma unroll
        for (int a = 0; a < 4; ++a) vsr[a] = *reinterpret_cast<const float4*>(sc + kWT + 8 * a + 4 * h);
    };
    auto smx = [&](int k, auto qc, f32x16& s, int t0, Smx& x) __attribute__((always_inline)) {
        constexpr int q = decltype(qc)::value;
        const int cell0 = lo + t0;                 // cell of key 0 of the tile
        if constexpr (q == 0) {
            // (the K row scales are in already)
            x.full = t0 + kWT <= n_full;
        } else if constexpr (q == 1) {
        } else if constexpr (q == 2) {
            if (p.softcap > 0.f) {                  // uniform: softcap before ALiBi
#pragma unroll
                for (int i = 0; i < 16; ++i) s[i] = p.softcap * tanhf(s[i] / p.softcap);
            }
            if (p.alibi) {
                const int pos = kvl - p.R + qv_r[k];
                const float slope = slope_lds[32 * blk[k] + l32];
#pragma unroll
                for (int i = 0; i < 16; ++i) s[i] += slope * static_cast<float>(cell0 + wide_key(i, h) - pos);
            }
            // bit j: key slot j of the tile is seen by this lane's query vector
            x.vword = 0xffffffffu;
            if (!x.full) {
                const int vlim = qv_lim[k] - cell0;
                x.vword = vlim >= 32 ? 0xffffffffu : (vlim <= 0 ? 0u : (1u << vlim) - 1u);
                if (tree) {
                    const unsigned long long path = tpath_lds[32 * blk[k] + l32];
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
                    if (!((x.vword >> wide_key(i, h)) & 1u)) s[i] = kNegInf;
            }
        } else if constexpr (q == 3) {
            // A NaN score is left out of the maximum (v_max_f32 returns the other
            // operand) and shows up as a NaN weight, hence a NaN running sum: the NaN flag.
            float tmax = kNegInf;
#pragma unroll
            for (int i = 0; i < 16; ++i) tmax = fmaxf(tmax, s[i]);
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
                unsigned long long* d = dbg_lds + (32 * blk[k] + l32) * 3;
                atomicAdd(d + 0, c);
                atomicAdd(d + 1, sm);
                atomicAdd(d + 2, sq);
            }
        } else if constexpr (q == 4) {
            float tmax = x.mls;
            tmax = wave_max_x32(tmax);
            m_true[k] = fmaxf(m_true[k], tmax);
            const bool need = (tmax > m_use[k] + kLazy) || (m_use[k] == kNegInf && tmax != kNegInf);
            // a lane whose reference was still -inf has o = 0 and l = 0: it takes the new
            // reference without any scaling of its accumulators
            const bool scale = need && m_use[k] != kNegInf;
            x.resc = wave_any(scale);
            x.c = scale ? rescale_factor(m_use[k], tmax) : 1.f;
            l_run[k] *= x.c;
            if (need) m_use[k] = tmax;
            // (no key seen yet: any finite reference keeps exp2 of an excluded key's -inf at 0)
            x.mls = m_use[k] == kNegInf ? 0.f : m_use[k] * kLog2e;
        } else if constexpr (q <= 12) {
            // weights exp(s - m_use) (v_exp_f32; below 2^-126 they flush to zero) for
            // two keys; the V row scale joins the seen weights only
            constexpr int i0 = 2 * (q - 5);
            const float w0 = __builtin_amdgcn_exp2f(fmaf(s[i0], kLog2e, -x.mls));
            const float w1 = __builtin_amdgcn_exp2f(fmaf(s[i0 + 1], kLog2e, -x.mls));
            l_run[k] += w0 + w1;
            s[i0] = w0 * vsr[i0 >> 2][i0 & 3];
            s[i0 + 1] = w1 * vsr[(i0 + 1) >> 2][(i0 + 1) & 3];
        } else if constexpr (q == 13) {
            if (!x.full) {
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    if (!((x.vword >> wide_key(i, h)) & 1u)) s[i] = 0.f;
            }
        } else if constexpr (q == 14) {
#pragma unroll
            for (int j = 0; j < 4; ++j) x.pop[0][j] = pack2<false>(s[2 * j], s[2 * j + 1]);
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) x.pop[1][j] = pack2<false>(s[8 + 2 * j], s[8 + 2 * j + 1]);
        }
    };

    // ---- the pipelined key loop ------------------------------------------------------
    // Iteration t: phase A computes the scores of tile t while tile t + 1 is widened;
    // phase B runs the softmax of tile t between the O^T products of tile t - 1 (the
    // last tile's products follow the loop).  A rescale the softmax of tile t asks
    // for is applied once the products of tile t - 1 are in.
    // prologue: raw tiles 0 and 1 loaded, tile 0 widened
    if (n_tiles > 0) dma_tile(0);
    if (n_tiles > 1) dma_tile(1);
    wait_vm<0>();
    wide_barrier();                               // raw tiles 0, 1 (and Q^T, paths) in LDS
    if (n_tiles > 0 && wave >= 2) {
        widen_read(0);
        static_for<0, NPARTS>([&](auto pc) { widen(0, pc); });
    }
    wide_barrier();                               // tile 0 widened; raw buffer 0 free

    auto key_loop = [&](auto two_c) __attribute__((always_inline)) {
        constexpr bool two = decltype(two_c)::value;
        // O^T of tile u for the wave's blocks (one V^T read feeds both), step i being
        // (key half i / NDB, dim block i % NDB); per_step(i) runs after step i
        auto products = [&](int u, const Smx& y0, const Smx& y1, auto&& after0, auto&& after1)
            __attribute__((always_inline)) {
            const char* vte = smem + vread_even + (u % 3) * VBUF;
            const char* vto = smem + vread_odd + (u % 3) * VBUF;
            auto vrd = [&](int i) -> u32x4 {
                const int db = i % NDB;
                return *reinterpret_cast<const u32x4*>((db & 1 ? vto : vte) + (i / NDB) * (2 * D * 16) + db * 512);
            };
            u32x4 va = vrd(0), vb = vrd(1);
            static_for<0, 2 * NDB>([&](auto ic) {
                constexpr int i = decltype(ic)::value;
                u32x4 vc = vb;
                if constexpr (i + 2 < 2 * NDB) vc = vrd(i + 2);
                // each matrix instruction is followed by vector work of its own, so the
                // next one does not hold the wave while the first still runs
                o_acc[0][i % NDB] = mfma32x32x16(va, y0.pop[i / NDB], o_acc[0][i % NDB]);
                after0(ic);
                __builtin_amdgcn_sched_barrier(0);
                if constexpr (two) o_acc[1][i % NDB] = mfma32x32x16(va, y1.pop[i / NDB], o_acc[1][i % NDB]);
                va = vb;
                vb = vc;
                after1(ic);
                __builtin_amdgcn_sched_barrier(0);
            });
        };
        auto rescale = [&](int k, const Smx& y) __attribute__((always_inline)) {
            if (y.resc) {                          // uniform
#pragma unroll
                for (int db = 0; db < NDB; ++db)
#pragma unroll
                    for (int e = 0; e < 16; ++e) {
                        float z = o_acc[k][db][e];
                        agpr_scale(z, y.c);
                        o_acc[k][db][e] = z;
                    }
            }
        };

        Smx xp0, xp1;                             // P^T of the previous tile (zero before tile 0)
#pragma unroll
        for (int c = 0; c < 2; ++c) xp0.pop[c] = xp1.pop[c] = u32x4{0u, 0u, 0u, 0u};
        for (int t = 0; t < n_tiles; ++t) {
            const int t0 = t * kWT;
            const bool next = t + 1 < n_tiles;
            // Nothing is in flight at the top of a tile (the previous one ended with a
            // full wait, or issued nothing).  Saying so here keeps the compiler, which
            // does not see the raw-tile loads, from placing the wait for a register it
            // reloads before the loop after the raw-tile loads, where they would hold it up.
            wait_vm<0>();
            if (t + 2 < n_tiles) dma_tile(t + 2);

            // ---- phase A: scores of tile t, widening of tile t + 1 ----
            f32x16 s0, s1;
            {
                // K and block-1 Q^T operands PF steps ahead (LDS latency under load)
                constexpr int PF = 4;
                const char* kt = smem + (t & 1) * KBUF;
                u32x4 kr[PF], qr[PF];
                static_for<0, PF>([&](auto jc) {
                    constexpr int j = decltype(jc)::value;
                    kr[j] = *reinterpret_cast<const u32x4*>(kt + kread + j * 32);
                    if constexpr (two) qr[j] = *reinterpret_cast<const u32x4*>(q1_lds + j * 1024);
                });
                static_for<0, NS>([&](auto stc) {
                    constexpr int st = decltype(stc)::value;
                    const u32x4 ka = kr[st % PF];
                    u32x4 qa{};
                    if constexpr (two) qa = qr[st % PF];
                    if constexpr (st + PF < NS) {
                        kr[st % PF] = *reinterpret_cast<const u32x4*>(kt + kread + (st + PF) * 32);
                        if constexpr (two) qr[st % PF] = *reinterpret_cast<const u32x4*>(q1_lds + (st + PF) * 1024);
                    }
                    // one block: its steps alternate between s0 and s1 (summed below).
                    // Waves 2, 3 (one block) widen tile t + 1: the raw reads at step 0,
                    // part p after the matrix instruction of step p + 1.
                    constexpr int part = st - 1;
                    const bool widener = !two && wave >= 2;   // uniform
                    if constexpr (st == 0) {
                        mfma_v_first(s0, ka, qop[st]);
                        if (widener && next) widen_read(t + 1);
                    } else if constexpr (!two && st == 1) {
                        mfma_v_first(s1, ka, qop[st]);
                    } else if constexpr (two || st % 2 == 0) {
                        mfma_v(s0, ka, qop[st]);
                    } else {
                        mfma_v(s1, ka, qop[st]);
                    }
                    if constexpr (!two && part >= 0 && part < NPARTS) {
                        if (widener && next) widen(t + 1, std::integral_constant<int, part>{});
                    }
                    __builtin_amdgcn_sched_barrier(0);
                    if constexpr (two) {
                        if constexpr (st == 0) mfma_v_first(s1, ka, qa);
                        else mfma_v(s1, ka, qa);
                    }
                    if constexpr (st == NS - 3) read_ks(t);
                    __builtin_amdgcn_sched_barrier(0);
                });
                wide_mfma_drain(s0);
                wide_mfma_drain(s1);
                if constexpr (!two) {
#pragma unroll
                    for (int e = 0; e < 16; ++e) s0[e] += s1[e];
                }
                // the K row scales join here (both blocks), so that they are not held
                // through phase B
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    s0[i] *= ksr[i >> 2][i & 3];
                    if constexpr (two) s1[i] *= ksr[i >> 2][i & 3];
                }
            }

            // ---- phase B: softmax of tile t, O^T products of tile t - 1 ----
            // block 0's stages take steps 0 .. NS/2 - 1, block 1's the rest
            Smx x0, x1;
            // (both blocks' stages in every step: two independent dependency chains)
            products(
                t == 0 ? 0 : t - 1, xp0, xp1,
                [&](auto ic) {
                    constexpr int st = decltype(ic)::value;
                    static_for<st * 16 / NS, (st + 1) * 16 / NS>([&](auto qc) { smx(0, qc, s0, t0, x0); });
                    if constexpr (st == 0) read_vs(t);
                },
                [&](auto ic) {
                    constexpr int st = decltype(ic)::value;
                    if constexpr (two)
                        static_for<st * 16 / NS, (st + 1) * 16 / NS>([&](auto qc) { smx(1, qc, s1, t0, x1); });
                });
            rescale(0, x0);
            if constexpr (two) rescale(1, x1);
            xp0 = x0;
            if constexpr (two) xp1 = x1;

            // raw tile t + 2 has landed for every wave before tile t + 1 widens it
            if (t + 2 < n_tiles) wait_vm<0>();
            wide_barrier();                       // tile t + 1 widened; raw buffer t & 1 free
        }
        // the O^T products of the last tile
        if (n_tiles > 0) products(n_tiles - 1, xp0, xp1, [&](auto) {}, [&](auto) {});
    };
    if (live[1]) key_loop(std::true_type{});
    else key_loop(std::false_type{});

    // ---- epilogue: partials of this slice -------------------------------------
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        if (!live[k]) continue;                    // uniform
        float l = wave_sum_x32(l_run[k]);
        int tn = (l_run[k] != l_run[k]) ? 1 : 0;   // a NaN visible score made a running sum NaN
        tn = wave_or_x32(tn);
        const bool nan_run = tn != 0;
        unsigned long long cnt = 0, sum = 0, sq = 0;
        if (p.dbg_visit) {
            const unsigned long long* d = dbg_lds + (32 * blk[k] + l32) * 3;
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
        if (p.dbg_visit && h == 0 && (m_wg + 32 * blk[k] + l32) % G == 0) {
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
