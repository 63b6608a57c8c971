// Matrix-core (MFMA) flash attention kernel template for gfx950: split-K decode
// and verify windows, prefill in selection or mask mode, bf16 / fp16 / int8 K/V.
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
// Tiles are loaded into registers one tile ahead (every 16-byte load of a tile
// is issued at once) and written to LDS at the top of the next iteration, so
// HBM latency overlaps the matrix-core work of the current tile.
//
// Key sources: a contiguous slice (decode, TensorFold PR #2595: one
// work-group per (stream, kv head, slice), partials merged afterwards), a
// contiguous range with an F32 mask (HartsyInference PR #910), or the sorted,
// de-duplicated selection list gathered in 32-cell tiles (strix-llama.cpp
// PR #115, Vulkan selected-key commit message: one work-group per query x kv
// head, list sorted in shared memory, invalid and repeated ids skipped).
// A key no query vector of the work-group can see is never loaded.
#pragma once

#include "arch.h"
#include "common.h"
#include "device_cache.h"
#include "internal.h"

#include <algorithm>

namespace selattn {
namespace mk {

constexpr int kTK = 32;          // keys per tile
constexpr float kLazy = 8.0f;    // slack of a lazily moved exponent reference, natural units
constexpr int kMaxSelM = 4096;   // longest selection list

enum Mode : int { kDecode = 0, kMask = 1, kSel = 2 };

struct MParams {
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
    // unit grid (x: slices / splits, y: kv heads x query chunks, z: streams / row blocks)
    int n_units_x, n_units_y, n_units_z;
    // outputs
    float* out;
    float* part_o;
    float* part_ml;
    int64_t* dbg_visit;
    int32_t* dbg_sel;
    const int32_t* tree;       // decode: [S][R] parent tables of tree windows, or null
    const float* sinks;        // prefill without splits: [Hq] sink logits, or null
};

// ---------------------------------------------------------------------------
// Tree-shaped verify windows (TensorFold PR #2595, kernel contract: tree widths
// with heap-order parents).  Node a of a window of R <= 64 nodes sees itself and
// its ancestors; parent[a] must lie in [-1, a), anything else makes a a root.
// Every lane of the wave calls this with uniform control flow.  Lane a < R builds
// node a's path mask by pointer jumping: after k rounds its mask holds the first
// 2^k nodes of the path and `up` the node 2^k steps above, so ceil(log2 R) rounds
// cover every path.  Returns the path mask of node r (0 <= r < R).
// ---------------------------------------------------------------------------
__device__ __forceinline__ unsigned long long tree_path_mask_wave(const int32_t* parent, int R, int r) {
    const int lane = threadIdx.x & 63;
    int up = -1;
    unsigned long long m = 0;
    if (lane < R) {
        const int x = parent[lane];
        up = (x >= -1 && x < lane) ? x : -1;
        m = 1ull << lane;
    }
    for (int span = 1; span < R; span <<= 1) {
        const int src = up < 0 ? 0 : up;
        const unsigned long long mu = wave_read64(m, src);
        const int uu = __shfl(up, src, 64);
        if (up >= 0) {
            m |= mu;
            up = uu;
        }
    }
    return wave_read64(m, r);
}

// Final normalisation with a sink logit z (HartsyInference PR #910: one more
// logit in the softmax, without a value).  The row's o is relative to reference
// `ref`, its sum l relative to its true maximum m (finite); z is finite or -inf
// (a NaN or +inf sink makes the row NaN before this is reached).  out = o * f.
__device__ __forceinline__ float sink_norm(float ref, float m, float l, float z) {
    const float big = z > m ? z : m;
    return exp2f((ref - big) * kLog2e) / fmaf(l, exp2f((m - big) * kLog2e), exp2f((z - big) * kLog2e));
}

// ---------------------------------------------------------------------------
// 16-bit conversions and LDS addressing
// ---------------------------------------------------------------------------
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

// two floats -> packed 16-bit pair, round to nearest even (one v_cvt_pk_* each)
template <bool F16>
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    if constexpr (F16) return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, f16x2_t));
    else return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}

// 1-byte K/V rows with one fp32 scale per row: int8 or e4m3
constexpr bool byte_kv(int kt) { return kt == SEL_ATTN_I8 || kt == SEL_ATTN_FP8; }

// byte `byte` of `word` as a float (exact): int8 by a sign-extending convert,
// e4m3 by the matrix-core unit's fp8 convert (v_cvt_f32_fp8, byte select)
template <int KT>
__device__ __forceinline__ float byte_float(uint32_t word, int byte) {
    if constexpr (KT == SEL_ATTN_FP8) {
        switch (byte) {
        case 0: return __builtin_amdgcn_cvt_f32_fp8(static_cast<int>(word), 0);
        case 1: return __builtin_amdgcn_cvt_f32_fp8(static_cast<int>(word), 1);
        case 2: return __builtin_amdgcn_cvt_f32_fp8(static_cast<int>(word), 2);
        default: return __builtin_amdgcn_cvt_f32_fp8(static_cast<int>(word), 3);
        }
    } else {
        return static_cast<float>(static_cast<int8_t>((word >> (8 * byte)) & 0xffu));
    }
}

// wait until at most N of the wave's buffer loads are outstanding
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 16, "vmcnt field");
    __builtin_amdgcn_s_waitcnt(N | (0x7 << 4) | (0xF << 8));
}

// Buffer load of 4 or 16 bytes a lane straight into LDS at lds + 4 or 16 lane (M0
// holds lds, one wait state after it is written; restored afterwards).  Written as
// asm so that the compiler, which cannot tell which LDS bytes such a load writes,
// does not put a wait for it in front of every later LDS read, nor count it among
// the loads it waits for; a loop waits for its raw tiles itself (wait_vm) before
// anything reads them.  No VGPR is written.
typedef int i32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ i32x4_t raw_rsrc(const void* base, int num_records) {
    const unsigned long long a = reinterpret_cast<unsigned long long>(base);
    i32x4_t r;
    r[0] = static_cast<int>(a & 0xffffffffull);
    r[1] = static_cast<int>((a >> 32) & 0xffffull);      // stride 0
    r[2] = num_records;
    r[3] = 0x00020000;
    return r;
}
template <int BYTES>
__device__ __forceinline__ void lds_dma(const i32x4_t& rs, unsigned lds, int voff, int soff) {
    static_assert(BYTES == 4 || BYTES == 16, "dword or dwordx4");
    int m0_saved;
    if constexpr (BYTES == 16)
        asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\tbuffer_load_dwordx4 %2, %3, %4 offen lds\n\t"
                     "s_mov_b32 m0, %0"
                     : "=&s"(m0_saved)
                     : "s"(lds), "v"(voff), "s"(rs), "s"(soff)
                     : "memory");
    else
        asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\tbuffer_load_dword %2, %3, %4 offen lds\n\t"
                     "s_mov_b32 m0, %0"
                     : "=&s"(m0_saved)
                     : "s"(lds), "v"(voff), "s"(rs), "s"(soff)
                     : "memory");
}
__device__ __forceinline__ unsigned lds_addr(const char* p) {
    return static_cast<unsigned>(reinterpret_cast<size_t>((const __attribute__((address_space(3))) char*)p));
}

// bf16 pair {bytes (wa, ba), (wb, bb)} of int8 or e4m3 data: both fit 8
// significant bits (e4m3: 4), so the high half of the float is the exact bf16;
// one v_perm_b32 takes both high halves
template <int KT>
__device__ __forceinline__ uint32_t bpair_bf16(uint32_t wa, int ba, uint32_t wb, int bb) {
    return __builtin_amdgcn_perm(__float_as_uint(byte_float<KT>(wb, bb)),
                                 __float_as_uint(byte_float<KT>(wa, ba)), 0x07060302u);
}

// e4m3: the two bytes of half `hi` of word w as a packed bf16 pair, exact (every e4m3
// value is a bf16 value): one v_cvt_scalef32_pk_bf16_fp8 with scale 1; the lower byte
// lands in the low half
__device__ __forceinline__ uint32_t fp8_pk_bf16(uint32_t w, bool hi) {
    if (hi) return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(static_cast<int>(w), 1.0f, true));
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(static_cast<int>(w), 1.0f, false));
}

// bf16 pair of bytes 2h and 2h + 1 of word w (one key, two adjacent dims)
template <int KT>
__device__ __forceinline__ uint32_t kpair_bf16(uint32_t w, int h) {
    if constexpr (KT == SEL_ATTN_FP8) return fp8_pk_bf16(w, h != 0);
    else return bpair_bf16<KT>(w, 2 * h, w, 2 * h + 1);
}

// bf16 pairs across keys a and b for the two dims of half h of their words:
// even = {a, b} at dim 2h, odd = {a, b} at dim 2h + 1
template <int KT>
__device__ __forceinline__ void vpairs_bf16(uint32_t wa, uint32_t wb, int h, uint32_t& even, uint32_t& odd) {
    if constexpr (KT == SEL_ATTN_FP8) {
        // bytes 2h, 2h + 1 of a and b interleaved as {a 2h, b 2h, a 2h+1, b 2h+1}, then one
        // pair convert per half: three instructions for the four values
        const uint32_t t = __builtin_amdgcn_perm(wb, wa, h != 0 ? 0x07030602u : 0x05010400u);
        even = fp8_pk_bf16(t, false);
        odd = fp8_pk_bf16(t, true);
    } else {
        even = bpair_bf16<KT>(wa, 2 * h, wb, 2 * h);
        odd = bpair_bf16<KT>(wa, 2 * h + 1, wb, 2 * h + 1);
    }
}

// byte offset of 16-byte chunk `ch` (8 dims) of key row `key` in the K tile; chunks
// are XOR-ed with (key & 15) so the 16 rows of one operand read hit distinct banks
__device__ __forceinline__ int k_off(int key, int ch, int D) {
    return key * D * 2 + ((ch ^ (key & 15)) << 4);
}
// byte offset of contraction chunk `cc` (8 keys) of dim row `d` in the V^T tile.
// Rows are 64 bytes, so four consecutive rows share the 64 LDS banks.  Row d is
// stored at pr = d ^ ((d >> 3) & 3) and its chunks are XOR-ed with (pr >> 2) & 3:
// the 16 rows one MFMA operand read touches then fall on distinct 16-byte bank
// slots, and so do the 32 lanes of a staging write (8 key groups x 4 dim chunks
// at the same offset within their 8 dims).
__device__ __forceinline__ int vt_off(int d, int cc) {
    const int pr = d ^ ((d >> 3) & 3);
    return pr * 64 + ((cc ^ ((pr >> 2) & 3)) << 4);
}

// ---------------------------------------------------------------------------
// Keys some query vectors of a tile see and others do not.  O^T += V^T . P^T gives
// such a key a zero weight for the query vectors that exclude it, and 0 * NaN or
// 0 * Inf is NaN: a non-finite V value would leak into outputs that must never
// read it (strix-llama.cpp PR #115, "Measurements": with poison=1 the masked cells
// are skipped, not weighted with zero).  Staging a tile whose visibility differs
// between the query vectors therefore also checks its V words for an all-ones
// exponent.  A tile that held an Inf or NaN is staged once more, before its
// registers are reused: V^T with every Inf / NaN half replaced by +0 (the product
// over it is the finite part, exact) and, beside it, an indicator tile of the same
// layout: 1 for NaN, 64 for +Inf, 4096 for -Inf.  The indicator tile times the
// visibility of each key (1 or 0) then counts, per output, the visible NaN, +Inf
// and -Inf values, and those counts turn the output into NaN or +-Inf as the sum
// over the visible keys would.  Tiles every query vector sees in full, and int8
// data (always finite), are staged as they are.
// ---------------------------------------------------------------------------

// Accumulates, for a word of two packed 16-bit values, a term whose bit 15 or 31
// ends up set iff that half has an all-ones exponent (Inf or NaN): the masked
// exponent plus its lowest bit carries into the sign position only then.
template <bool F16>
__device__ __forceinline__ uint32_t nonfinite_acc(uint32_t acc, uint32_t w) {
    constexpr uint32_t M = F16 ? 0x7C007C00u : 0x7F807F80u;
    constexpr uint32_t C = F16 ? 0x04000400u : 0x00800080u;
    return acc | ((w & M) + C);
}
__device__ __forceinline__ bool nonfinite_found(uint32_t acc) { return (acc & 0x80008000u) != 0u; }

// Splits a word of two packed 16-bit V values into its finite part (Inf and NaN
// halves replaced by +0) and the indicator of its non-finite halves (1 for NaN, 64
// for +Inf, 4096 for -Inf, as exact 16-bit floats; 0 for finite halves).  A product
// of indicators with 0/1 weights over at most 32 keys is an exact integer below
// 2^24 whose base-64 digits count the three kinds.
template <bool F16>
__device__ __forceinline__ void split_nonfinite(uint32_t w, uint32_t& fin, uint32_t& ind) {
    constexpr uint32_t EXP = F16 ? 0x7C00u : 0x7F80u;
    constexpr uint32_t MAN = F16 ? 0x03FFu : 0x007Fu;
    constexpr uint32_t ONE = F16 ? 0x3C00u : 0x3F80u;     // 1
    constexpr uint32_t C64 = F16 ? 0x5400u : 0x4280u;     // 64
    constexpr uint32_t C4K = F16 ? 0x6C00u : 0x4580u;     // 4096
    fin = 0u;
    ind = 0u;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const uint32_t x = (w >> (16 * h)) & 0xffffu;
        const bool nf = (x & EXP) == EXP;
        const uint32_t c = (x & MAN) ? ONE : ((x & 0x8000u) ? C4K : C64);
        fin |= (nf ? 0u : x) << (16 * h);
        ind |= (nf ? c : 0u) << (16 * h);
    }
}

// Packed 16-bit 1 / 0 pair: the visibility weights of the indicator product.
template <bool F16>
__device__ __forceinline__ uint32_t vis_pair(bool a, bool b) {
    constexpr uint32_t ONE = F16 ? 0x3C00u : 0x3F80u;
    return (a ? ONE : 0u) | ((b ? ONE : 0u) << 16);
}

// Output element o after a tile whose visible non-finite V values were counted as
// cnt (base-64 digits: NaN, +Inf, -Inf): adds NaN, +Inf and/or -Inf as the plain
// sum over the visible keys would (a +Inf and a -Inf together give NaN).
__device__ __forceinline__ float apply_nonfinite(float o, float cnt) {
    const int v = static_cast<int>(cnt);
    if (v == 0) return o;
    float add = 0.f;
    if (v & 63) add = __builtin_nanf("");
    else {
        if ((v >> 6) & 63) add += kPosInf;
        if (v >> 12) add += kNegInf;
    }
    return o + add;
}

// Stores one V^T word pair: plainly (split = false; the pair is checked into nfa),
// or split into its finite part at `at` and its indicator at `at + ind_off`.
template <bool F16>
__device__ __forceinline__ uint32_t store_v(char* at, int ind_off, uint32_t lo, uint32_t hi, bool split,
                                            uint32_t nfa) {
    if (!split) {
        *reinterpret_cast<uint2*>(at) = uint2{lo, hi};
        return nonfinite_acc<F16>(nonfinite_acc<F16>(nfa, lo), hi);
    }
    uint32_t flo, ilo, fhi, ihi;
    split_nonfinite<F16>(lo, flo, ilo);
    split_nonfinite<F16>(hi, fhi, ihi);
    *reinterpret_cast<uint2*>(at) = uint2{flo, fhi};
    *reinterpret_cast<uint2*>(at + ind_off) = uint2{ilo, ihi};
    return nfa;
}

// LDS: K tile, V^T tile, the tile's row scales, the waves' non-finite flags, then
// the selection list (selection mode) or the V^T indicator tile (CHK kernels).
template <int D, bool SEL, bool CHK>
constexpr int smem_bytes() {
    return kTK * D * 2 + D * 64 + 2 * kTK * 4 + 16 * 4 + (SEL ? kMaxSelM * 4 : 0) + (CHK ? D * 64 : 0);
}
template <int MODE, int KT>
constexpr bool check_v(int) { return MODE != kSel && KT != SEL_ATTN_I8; }

// ---------------------------------------------------------------------------
// the kernel
// ---------------------------------------------------------------------------
// One work unit: (slice, kv head x query chunk, stream) in decode mode,
// (split, kv head x query chunk, row block) in prefill modes.
template <int MODE, int KT, int D, int QB, int W>
__device__ __forceinline__ void attn_unit(const MParams& p, const int t_split, const int gy, const int bz,
                                          char* smem, int& s_nids) {
    constexpr bool F16 = (KT == SEL_ATTN_F16);
    constexpr bool B8 = byte_kv(KT);       // int8 or e4m3 rows with row scales
    constexpr int NKK = D / 32;                  // contraction steps for S^T
    constexpr int NDB = D / 16;                  // dim blocks of O^T
    constexpr int GCH = B8 ? D / 16 : D / 8;     // 16-byte chunks per K/V row in memory
    constexpr int NT = 64 * W;
    constexpr int K_TASKS = kTK * GCH;           // one 16-byte load each
    constexpr int V_TASKS = 8 * GCH;             // four 16-byte loads each: task e covers
                                                 // keys 4*(e & 7) + 0..3, chunk e >> 3
    constexpr int NKL = (K_TASKS + NT - 1) / NT;
    constexpr int NVL = (V_TASKS + NT - 1) / NT;
    constexpr int EPC = B8 ? 16 : 8;             // elements per 16-byte chunk
    // Visibility may differ between the query vectors of a tile in decode and mask
    // mode (causal or tree windows, per-row masks): their staged V is checked for
    // non-finite values (int8 data is always finite).  In selection mode every query
    // vector of a work-group belongs to one row and sees the same keys.
    constexpr bool CHK = check_v<MODE, KT>(0);

    char* k_lds = smem;                                            // kTK * D * 2
    char* vt_lds = smem + kTK * D * 2;                             // D * 64
    float* ksc_lds = reinterpret_cast<float*>(vt_lds + D * 64);    // kTK
    float* vsc_lds = ksc_lds + kTK;                                // kTK
    uint32_t* wflag = reinterpret_cast<uint32_t*>(vsc_lds + kTK);  // [16]: wave w staged a non-finite V value
    int* list = reinterpret_cast<int*>(wflag + 16);                // kMaxSelM (selection)
    constexpr int IND = kTK * D * 2 + D * 64 + 2 * kTK * 4 + 16 * 4 - kTK * D * 2;   // indicator tile - vt_lds

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int ln = lane & 15;        // query vector of a block / key row of a 16-key block
    const int lg = lane >> 4;        // lane group 0..3
    const int G = p.G;

    // ---- work unit ---------------------------------------------------------
    const int g = gy % p.Hkv;
    const int qchunk = gy / p.Hkv;
    int b = 0, kvl = 0, lo = 0, hi = 0, row0 = 0;
    if constexpr (MODE == kDecode) {
        b = bz;
        kvl = min(max(p.kv_len[b], 0), p.cap);
        lo = t_split * p.slice_len;
        if (lo >= kvl) return;            // past this stream's slices: nothing written
        hi = min(lo + p.slice_len, kvl);
    } else {
        row0 = bz * p.rows_per_wg;
        lo = t_split * p.split_step;
        hi = min(lo + p.split_step, p.n_kv);
    }
    const int m_wg = qchunk * p.qpw;               // first query vector of the work-group
    const int m_wave = m_wg + wave * QB * 16;       // first of this wave

    // query vector -> (row, head, position, causal limit); tree windows: cells from
    // tstart on are window nodes, visible by the query vector's path mask
    int qv_row[QB], qv_head[QB], qv_pos[QB], qv_lim[QB];
    unsigned long long qv_path[QB];
    bool qv_ok[QB];
    const bool tree = (MODE == kDecode) && p.tree != nullptr;
    const int tstart = tree ? kvl - p.R : 0x7fffffff;
#pragma unroll
    for (int k = 0; k < QB; ++k) {
        const int m = m_wave + 16 * k + ln;
        bool ok = m < p.M && m < m_wg + p.qpw;
        int r, h;
        if constexpr (MODE == kDecode) { r = m / G; h = g * G + m % G; ok = ok && r < p.R; }
        else if constexpr (MODE == kSel) { r = row0; h = g * G + m; }
        else { r = row0 + m / G; h = g * G + m % G; ok = ok && r < min(row0 + p.rows_per_wg, p.R); }
        if (!ok) {                        // padding: point at a real row, never used
            r = (MODE == kDecode) ? 0 : row0;
            h = g * G;
        }
        qv_ok[k] = ok;
        qv_row[k] = r;
        qv_head[k] = h;
        qv_path[k] = 0;
        if constexpr (MODE == kDecode) {
            qv_pos[k] = kvl - p.R + r;
            qv_lim[k] = (p.causal && !tree) ? min(qv_pos[k] + 1, kvl) : kvl;
            if (tree) qv_path[k] = tree_path_mask_wave(p.tree + static_cast<int64_t>(b) * p.R, p.R, r);
        } else {
            qv_pos[k] = p.q_pos ? p.q_pos[r] : 0;
            qv_lim[k] = (MODE == kMask && p.causal) ? qv_pos[k] + 1 : 0x7fffffff;
        }
        if (!ok) qv_lim[k] = -1;          // sees nothing
    }

    // ---- Q^T operands (scale folded in) ----------------------------------
    u32x4 qop[QB][NKK];
#pragma unroll
    for (int k = 0; k < QB; ++k) {
        const float* qp;
        if constexpr (MODE == kDecode)
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

    // ---- key slots to walk -------------------------------------------------
    int n_keys = 0;
    if constexpr (MODE == kSel) {
        // the row's list: invalid ids become +inf, bitonic sort, then drop repeats
        const int P = p.sel_pow2;
        const int32_t* srow = p.sel + static_cast<int64_t>(row0) * p.n_sel;
        for (int e = tid; e < P; e += NT) {
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
                for (int e = tid; e < P; e += NT) {
                    const int o = e ^ j;
                    if (o > e) {
                        const int x = list[e], y = list[o];
                        if ((x > y) == ((e & kq) == 0)) { list[e] = y; list[o] = x; }
                    }
                }
                __syncthreads();
            }
        }
        // stable in-place compaction by one lane: keeps the first of each run
        if (tid == 0) {
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
            if (tid == 0) dst[0] = n_ids;
            for (int e = tid; e < n_ids; e += NT) dst[1 + e] = list[e];
        }
        n_keys = n_ids * p.bs;
    } else {
        // no query vector of this work-group sees keys at or past the largest limit
        int lim_max = -1;
        const int m_end = min(p.M, m_wg + p.qpw);
        if (m_end > m_wg) {
            const int rbase = (MODE == kDecode) ? 0 : row0;
            const int r_first = rbase + m_wg / G;
            const int r_last = rbase + (m_end - 1) / G;
            for (int r = r_first; r <= r_last && r < p.R; ++r) {
                int l;
                if constexpr (MODE == kDecode) l = (p.causal && !tree) ? min(kvl - p.R + r + 1, kvl) : kvl;
                else l = p.causal ? (p.q_pos[r] + 1) : hi;
                lim_max = max(lim_max, l);
            }
        }
        n_keys = max(0, min(hi, lim_max) - lo);
    }

    // cell of key slot `kslot` (-1 for none)
    auto slot_cell = [&](int kslot) -> int {
        if (kslot >= n_keys) return -1;
        if constexpr (MODE == kSel) {
            const int c = list[kslot / p.bs] * p.bs + kslot % p.bs;
            return (c < p.n_kv && c >= lo && c < hi) ? c : -1;
        } else {
            return lo + kslot;
        }
    };

    const int64_t kv_base = (MODE == kDecode ? static_cast<int64_t>(b) * p.kv_ss : 0) +
                            static_cast<int64_t>(g) * p.kv_sh;
    const int64_t sc_base = (MODE == kDecode ? static_cast<int64_t>(b) * p.sc_ss : 0) +
                            static_cast<int64_t>(g) * p.sc_sh;
    const char* kbase = static_cast<const char*>(p.k) + kv_base * (B8 ? 1 : 2);
    const char* vbase = static_cast<const char*>(p.v) + kv_base * (B8 ? 1 : 2);
    const int64_t cell_bytes = p.kv_sc * (B8 ? 1 : 2);

    // ---- tile loads into registers -----------------------------------------
    u32x4 kreg[NKL];
    u32x4 vreg[NVL][4];
    float kscr = 0.f, vscr = 0.f;
    auto load_tile = [&](int t0) {
#pragma unroll
        for (int i = 0; i < NKL; ++i) {
            const int e = tid + i * NT;
            kreg[i] = u32x4{0u, 0u, 0u, 0u};
            if (e < K_TASKS) {
                const int cell = slot_cell(t0 + e / GCH);
                if (cell >= 0)
                    kreg[i] = *reinterpret_cast<const u32x4*>(kbase + cell * cell_bytes + (e % GCH) * 16);
            }
        }
#pragma unroll
        for (int i = 0; i < NVL; ++i) {
            const int e = tid + i * NT;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                vreg[i][j] = u32x4{0u, 0u, 0u, 0u};
                if (e < V_TASKS) {
                    const int cell = slot_cell(t0 + 4 * (e & 7) + j);
                    if (cell >= 0)
                        vreg[i][j] = *reinterpret_cast<const u32x4*>(vbase + cell * cell_bytes + (e >> 3) * 16);
                }
            }
        }
        if constexpr (B8) {
            if (tid < kTK) {
                const int cell = slot_cell(t0 + tid);
                kscr = cell >= 0 ? p.ksc[sc_base + cell * p.sc_sc] : 0.f;
                vscr = cell >= 0 ? p.vsc[sc_base + cell * p.sc_sc] : 0.f;
            }
        }
    };
    // registers -> LDS (K swizzled row-major, V transposed in contraction order);
    // with CHK, each wave records whether it staged a non-finite V value
    // split: the second staging of a tile that held an Inf or NaN (CHK only)
    auto store_tile = [&](bool split) {
        uint32_t nfa = 0u;
#pragma unroll
        for (int i = 0; i < NKL; ++i) {
            const int e = tid + i * NT;
            if (e < K_TASKS) {
                const int key = e / GCH, ch = e % GCH;
                if constexpr (B8) {
                    const u32x4 r = kreg[i];
                    u32x4 w0, w1;
#pragma unroll
                    for (int j = 0; j < 2; ++j) {
                        w0[2 * j] = kpair_bf16<KT>(r[j], 0);
                        w0[2 * j + 1] = kpair_bf16<KT>(r[j], 1);
                        w1[2 * j] = kpair_bf16<KT>(r[2 + j], 0);
                        w1[2 * j + 1] = kpair_bf16<KT>(r[2 + j], 1);
                    }
                    *reinterpret_cast<u32x4*>(k_lds + k_off(key, 2 * ch, D)) = w0;
                    *reinterpret_cast<u32x4*>(k_lds + k_off(key, 2 * ch + 1, D)) = w1;
                } else {
                    *reinterpret_cast<u32x4*>(k_lds + k_off(key, ch, D)) = kreg[i];
                }
            }
        }
#pragma unroll
        for (int i = 0; i < NVL; ++i) {
            const int e = tid + i * NT;
            if (e < V_TASKS) {
                const int kg = e & 7, ch = e >> 3;         // key group of 4, 16-byte chunk
                const int kb = kg >> 2, gq = kg & 3;       // keys kb*16 + 4*gq + j
#pragma unroll
                for (int dd = 0; dd < EPC; ++dd) {
                    uint32_t lo2, hi2;
                    if constexpr (B8) {
                        const int w = dd >> 2, by = dd & 3;
                        lo2 = bpair_bf16<KT>(vreg[i][0][w], by, vreg[i][1][w], by);
                        hi2 = bpair_bf16<KT>(vreg[i][2][w], by, vreg[i][3][w], by);
                    } else {
                        const int w = dd >> 1;
                        if (dd & 1) {
                            lo2 = (vreg[i][0][w] >> 16) | (vreg[i][1][w] & 0xffff0000u);
                            hi2 = (vreg[i][2][w] >> 16) | (vreg[i][3][w] & 0xffff0000u);
                        } else {
                            lo2 = (vreg[i][0][w] & 0xffffu) | (vreg[i][1][w] << 16);
                            hi2 = (vreg[i][2][w] & 0xffffu) | (vreg[i][3][w] << 16);
                        }
                    }
                    if constexpr (CHK) nfa = store_v<F16>(vt_lds + vt_off(ch * EPC + dd, gq) + 8 * kb, IND, lo2, hi2, split, nfa);
                    else *reinterpret_cast<uint2*>(vt_lds + vt_off(ch * EPC + dd, gq) + 8 * kb) = uint2{lo2, hi2};
                }
            }
        }
        if constexpr (B8) {
            if (tid < kTK) {
                ksc_lds[tid] = kscr;
                vsc_lds[tid] = vscr;
            }
        }
        if constexpr (CHK) {
            if (!split) {
                const bool any = wave_any(nonfinite_found(nfa));
                if (lane == 0) wflag[wave] = any ? 1u : 0u;
            }
        }
    };


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

    // Mask mode with one block of query vectors per wave: each lane's mask values of
    // a tile (for the cells it scores, where its query vector may see them) are
    // loaded a tile ahead, with the K/V rows.  With more blocks the registers are
    // short, and the values are read where they are used.
    constexpr bool MASK_AHEAD = MODE == kMask && QB == 1;
    float mcur[MASK_AHEAD ? QB : 1][8], mnext[MASK_AHEAD ? QB : 1][8];
    auto load_mask = [&](int t0, float (&mv)[MASK_AHEAD ? QB : 1][8]) {
        if constexpr (MASK_AHEAD) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int cell = slot_cell(t0 + (e >> 2) * 16 + 4 * lg + (e & 3));
#pragma unroll
                for (int k = 0; k < QB; ++k)
                    mv[k][e] = (cell >= 0 && cell < qv_lim[k])
                                   ? p.mask[static_cast<int64_t>(qv_row[k]) * p.m_sr +
                                            static_cast<int64_t>(qv_head[k]) * p.m_sh + cell]
                                   : 0.f;
            }
        }
    };

    if (n_keys > 0) {
        load_tile(0);
        load_mask(0, mcur);
    }
    for (int t0 = 0; t0 < n_keys; t0 += kTK) {
        store_tile(false);
        __syncthreads();
        // an Inf or NaN in this tile's V: staged again, split, before the registers
        // take the next tile (uniform)
        bool flagged = false;
        if constexpr (CHK) {
            uint32_t f = 0u;
#pragma unroll
            for (int w = 0; w < W; ++w) f |= wflag[w];
            flagged = f != 0u;
            if (flagged) {
                store_tile(true);
                __syncthreads();
            }
        }
        if (t0 + kTK < n_keys) {                          // in flight during this tile's math
            load_tile(t0 + kTK);
            load_mask(t0 + kTK, mnext);
        }

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
        for (int e = 0; e < 8; ++e) cell_of[e] = slot_cell(t0 + (e >> 2) * 16 + 4 * lg + (e & 3));

        u32x4 pop[QB];
        u32x4 pvis[QB];                 // flagged tiles: 0/1 visibility weights per block
#pragma unroll
        for (int k = 0; k < QB; ++k) {
            pvis[k] = u32x4{0u, 0u, 0u, 0u};
            float sc[8];
            bool vis[8];
            float tmax = kNegInf;
            bool tnan = false;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int kb = e >> 2, i = e & 3;
                const int cell = cell_of[e];
                bool v = cell >= 0 && cell < qv_lim[k] &&
                         (cell < tstart || ((qv_path[k] >> (cell - tstart)) & 1ull));
                float maskv = 0.f;
                if constexpr (MODE == kMask) {
                    if (v) {
                        if constexpr (MASK_AHEAD) maskv = mcur[k][e];
                        else maskv = p.mask[static_cast<int64_t>(qv_row[k]) * p.m_sr +
                                            static_cast<int64_t>(qv_head[k]) * p.m_sh + cell];
                        v = maskv != kNegInf;
                    }
                }
                float x = s[k][kb][i];
                if constexpr (B8) x *= ksc_lds[kb * 16 + 4 * lg + i];
#ifdef SELATTN_PLANT_ALIBI_BEFORE_SOFTCAP
                // test-only planted mistake (never in a product build): the bias first
                x += slope[k] * static_cast<float>(cell - qv_pos[k]);
                if (p.softcap > 0.f) x = p.softcap * tanhf(x / p.softcap);
#else
                if (p.softcap > 0.f) x = p.softcap * tanhf(x / p.softcap);
                x += slope[k] * static_cast<float>(cell - qv_pos[k]);
#endif
                x += maskv;
                vis[e] = v;
                sc[e] = x;
                if (v) {
                    if (x != x) tnan = true;
                    else tmax = max_keep(tmax, x);
                }
            }
            // combine over the four lane groups that hold this query vector
            tmax = max_keep(tmax, wave_partner_x16(tmax));
            tmax = max_keep(tmax, wave_partner_x32(tmax));
            int tn = tnan ? 1 : 0;
            tn = wave_or_x16(tn);
            tn = wave_or_x32(tn);
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
                // the row scale joins visible weights only (a NaN scale of a key this
                // query vector cannot see must not reach it)
                if constexpr (B8) w = vis[e] ? w * vsc_lds[(e >> 2) * 16 + 4 * lg + (e & 3)] : 0.f;
                pv[e] = w;
            }
            pop[k] = u32x4{pack2<F16>(pv[0], pv[1]), pack2<F16>(pv[2], pv[3]),
                           pack2<F16>(pv[4], pv[5]), pack2<F16>(pv[6], pv[7])};
            if constexpr (CHK) {
                if (flagged)
                    pvis[k] = u32x4{vis_pair<F16>(vis[0], vis[1]), vis_pair<F16>(vis[2], vis[3]),
                                    vis_pair<F16>(vis[4], vis[5]), vis_pair<F16>(vis[6], vis[7])};
            }
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
        // a non-finite V value in the tile: the visible ones counted and applied
        if constexpr (CHK) {
            if (flagged) {
#pragma unroll
                for (int db = 0; db < NDB; ++db) {
                    const u32x4 ai = *reinterpret_cast<const u32x4*>(vt_lds + IND + vt_off(db * 16 + ln, lg));
#pragma unroll
                    for (int k = 0; k < QB; ++k) {
                        const f32x4 cnt = mfma16x16x32<F16>(ai, pvis[k], f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
                        for (int i = 0; i < 4; ++i) o_acc[k][db][i] = apply_nonfinite(o_acc[k][db][i], cnt[i]);
                    }
                    __builtin_amdgcn_sched_barrier(0);      // a rare path: one dim block at a time
                }
            }
        }
        if constexpr (MASK_AHEAD) {
#pragma unroll
            for (int k = 0; k < QB; ++k)
#pragma unroll
                for (int e = 0; e < 8; ++e) mcur[k][e] = mnext[k][e];
        }
        __syncthreads();
    }

    // ---- epilogue ---------------------------------------------------------------
#pragma unroll
    for (int k = 0; k < QB; ++k) {
        float l = l_run[k];
        l = wave_sum_x16(l);
        l = wave_sum_x32(l);
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
                    acc += static_cast<long long>(
                        (static_cast<unsigned long long>(static_cast<unsigned>(ohi)) << 32) | olo);
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
        const bool split = (MODE == kDecode) || p.n_splits > 1;
        const float z = (!split && p.sinks) ? p.sinks[h] : kNegInf;    // sink logit, unsplit only
        const bool bad = nan_run[k] || m == kPosInf || z != z || z == kPosInf;
        const bool empty = !bad && m == kNegInf;
        int64_t pi;
        if constexpr (MODE == kDecode)
            pi = ((static_cast<int64_t>(b) * p.R + r) * p.Hq + h) * p.n_slices_max + t_split;
        else
            pi = (static_cast<int64_t>(r) * p.Hq + h) * p.n_splits + t_split;
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
            const int d0 = db * 16 + 4 * lg;
            float4 o;
            if (!split) {
                const float inv = (z != kNegInf && !bad && !empty) ? sink_norm(m, m, l, z) : 1.f / l;
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
            if (m_idx % G == 0) {           // the first query head of the row records its visits
                int64_t di;
                if constexpr (MODE == kDecode)
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

// ---------------------------------------------------------------------------
// Decode work list.  Only (stream, slice) pairs below a stream's depth hold
// work.  The (stream, slice, kv head) units are numbered densely, unit u goes to
// XCD u % 8, and the query chunks of a unit are taken by work-groups of that
// same XCD one after another (work-group w runs on XCD w % 8: dispatch is
// round-robin over the XCDs), so a unit's K/V slice is fetched into one L2 and
// shared by its chunks.  A persistent grid (a multiple of 8) walks the list, so
// the active units spread evenly over the chip whatever the mix of depths.
// Correctness does not depend on the placement, only locality does.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int decode_slices(const MParams& p, int b) {
    const int n = min(max(p.kv_len[b], 0), p.cap);
    return min((n + p.slice_len - 1) / p.slice_len, p.n_units_x);
}

// Calls fn(slice, kv head x chunk, stream) for every decode item of this work-group.
template <typename F>
__device__ __forceinline__ void for_each_decode_item(const MParams& p, F&& fn) {
    const int hkv = p.Hkv;
    const int nqc = p.n_units_y / hkv;
    int n_su = 0;
    for (int b = 0; b < p.n_units_z; ++b) n_su += decode_slices(p, b);
    const int n_u = n_su * hkv;
    const int xcd = blockIdx.x & 7;
    const int local = blockIdx.x >> 3;
    const int lstride = gridDim.x >> 3;
    const int n_ux = n_u > xcd ? (n_u - xcd + 7) / 8 : 0;
    const int items = n_ux * nqc;
    for (int li = local; li < items; li += lstride) {
        const int uu = li / nqc;
        const int qc = li - uu * nqc;
        const int u = uu * 8 + xcd;
        const int su = u / hkv;
        const int g = u - su * hkv;
        int base = 0, b = 0;
        for (; b < p.n_units_z - 1; ++b) {
            const int ns = decode_slices(p, b);
            if (su < base + ns) break;
            base += ns;
        }
        fn(su - base, qc * hkv + g, b);
    }
}

// Persistent decode grid: about one work-group per resident slot, a multiple of 8.
inline unsigned decode_grid(long long items, int resident) {
    long long n = std::min<long long>(items, resident);
    n = std::max<long long>(8, (n / 8) * 8);
    return static_cast<unsigned>(n);
}

// ---------------------------------------------------------------------------
// the kernel: prefill grids map one work-group to one unit; decode runs the
// persistent work list above.
// ---------------------------------------------------------------------------
template <int MODE, int KT, int D, int QB, int W>
__global__ __launch_bounds__(64 * W) void mfma_attn_kernel(MParams p) {
    extern __shared__ __align__(16) char smem[];
    __shared__ int s_nids;
    if constexpr (MODE == kDecode) {
        for_each_decode_item(p, [&](int t, int gy, int bz) {
            attn_unit<MODE, KT, D, QB, W>(p, t, gy, bz, smem, s_nids);
            __syncthreads();                                         // LDS is reused by the next item
        });
    } else {
        attn_unit<MODE, KT, D, QB, W>(p, blockIdx.x, blockIdx.y, blockIdx.z, smem, s_nids);
    }
}

// ---------------------------------------------------------------------------
// launch helpers
// ---------------------------------------------------------------------------
struct Shape {
    int qb;      // query blocks per wave: 1, 2 or 3
    int waves;   // waves per work-group: 1 or 4
};

inline Shape pick_shape(int M) {
    const int nqb = (M + 15) / 16;
    if (nqb <= 1) return {1, 1};
    if (nqb <= 4) return {1, 4};
    if (nqb <= 8) return {2, 4};
    return {3, 4};
}

// Work-groups of this kernel instance that fit on the device at once (cached per device).
template <int MODE, int KT, int D, int QB, int W>
int resident_groups() {
    static DeviceCache cache;
    return cache.get(0, []() {
        int dev = 0, cus = 0, per_cu = 0;
        if (hipGetDevice(&dev) != hipSuccess) dev = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
            cus = 256;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, mfma_attn_kernel<MODE, KT, D, QB, W>, 64 * W,
                                                         smem_bytes<D, MODE == kSel, check_v<MODE, KT>(0)>()) !=
                hipSuccess ||
            per_cu <= 0)
            per_cu = 1;
        return cus * per_cu;
    });
}

template <int MODE, int KT, int D, int QB, int W>
hipError_t launch_one(const MParams& p, dim3 grid, hipStream_t st) {
    constexpr int smem = smem_bytes<D, MODE == kSel, check_v<MODE, KT>(0)>();
    if constexpr (MODE == kDecode) {
        const long long items = static_cast<long long>(grid.x) * grid.y * grid.z;
        grid = dim3(decode_grid(items, resident_groups<MODE, KT, D, QB, W>()), 1, 1);
    }
    hipLaunchKernelGGL((mfma_attn_kernel<MODE, KT, D, QB, W>), grid, dim3(64 * W), smem, st, p);
    return hipGetLastError();
}

template <int MODE, int KT, int D>
hipError_t launch_shape(const MParams& p, dim3 grid, Shape sh, hipStream_t st) {
    if (sh.waves == 1) return launch_one<MODE, KT, D, 1, 1>(p, grid, st);
    switch (sh.qb) {
    case 1: return launch_one<MODE, KT, D, 1, 4>(p, grid, st);
    case 2: return launch_one<MODE, KT, D, 2, 4>(p, grid, st);
    default: return launch_one<MODE, KT, D, 3, 4>(p, grid, st);
    }
}

template <int MODE>
hipError_t launch_mode(int dt, const MParams& p, dim3 grid, Shape sh, hipStream_t st) {
    if (dt == SEL_ATTN_BF16)
        return p.D == 256 ? launch_shape<MODE, SEL_ATTN_BF16, 256>(p, grid, sh, st)
                          : launch_shape<MODE, SEL_ATTN_BF16, 128>(p, grid, sh, st);
    if (dt == SEL_ATTN_F16)
        return p.D == 256 ? launch_shape<MODE, SEL_ATTN_F16, 256>(p, grid, sh, st)
                          : launch_shape<MODE, SEL_ATTN_F16, 128>(p, grid, sh, st);
    if (dt == SEL_ATTN_I8)
        return p.D == 256 ? launch_shape<MODE, SEL_ATTN_I8, 256>(p, grid, sh, st)
                          : launch_shape<MODE, SEL_ATTN_I8, 128>(p, grid, sh, st);
    return p.D == 256 ? launch_shape<MODE, SEL_ATTN_FP8, 256>(p, grid, sh, st)
                      : launch_shape<MODE, SEL_ATTN_FP8, 128>(p, grid, sh, st);
}

}  // namespace mk
}  // namespace selattn
