// Single-wave matrix-core kernel for units of at most 16 query vectors: split-K
// decode with R * G <= 16 (the whole GQA group of one row) and selection-mode
// prefill with G <= 16.  Same arithmetic as mfma_kernel.h, shaped for HBM
// streaming at two waves per SIMD:
//   * 16-key tiles (K 16 x D and V^T D x 16 in LDS, 8 KiB each at D = 256), so the
//     next tile's loads fit in 64 registers per lane and a work-group needs 16 KiB
//     of LDS (plus the selection list);
//   * S^T = K . Q^T on v_mfma_f32_16x16x32 (one MFMA per 32 dims), each lane then
//     holds 4 scores of ONE query vector, which are exactly its P^T operand for
//     O^T += V^T . P^T on v_mfma_f32_16x16x16;
//   * lazy rescaling: the exponent reference m_use only moves when a score exceeds
//     it by more than 8 (weights stay below e^8), so o and l are rarely rescaled;
//     the true maximum is tracked alongside and applied once at the end, so the
//     result is the same softmax (TensorFold PR #985, "What this changes": the
//     correction exp(m_old - m_new) applied to l and o).
#pragma once

#include "mfma_kernel.h"

namespace selattn {
namespace mk {

constexpr int kLT = 16;          // keys per tile

// K tile: 16 rows of D 16-bit values; 16-byte chunks XOR-ed with (key & 15), so the
// 16 rows of one operand read land on 16 distinct chunks.
__device__ __forceinline__ int k16_off(int key, int ch, int D) {
    return key * D * 2 + ((ch ^ (key & 15)) << 4);
}
// V staging task e: keys 4 kg .. 4 kg + 3 of the tile, 16-byte chunk ch of their rows.
// Lanes 4q .. 4q + 3 take the same keys and consecutive chunks, so each lane quad of a
// load reads 64 contiguous bytes of one row (one cache tag lookup instead of four);
// each half-wave still covers four key groups of eight chunks, the set the V^T
// writes below are free of bank conflicts for.
template <int GCH>
__device__ __forceinline__ void v_task(int e, int& kg, int& ch) {
    constexpr int C = GCH < 8 ? GCH : 8;
    const int r = e % (4 * C);
    kg = r / C;
    ch = (e / (4 * C)) * C + r % C;
}

// V^T tile: row d holds 16 keys (32 bytes, four 8-byte slots of 4 keys).  Row d is
// stored at pr = d ^ ((d >> 3) & 7) and slot s at s ^ (2 * ((pr >> 3) & 1)): both the
// 16-row operand reads and the 32-lane staging writes then hit distinct banks.
__device__ __forceinline__ int vt16_off(int d, int slot) {
    const int pr = d ^ ((d >> 3) & 7);
    return pr * 32 + ((slot ^ (((pr >> 3) & 1) << 1)) << 3);
}

// LDS: K tile, V^T tile, the tile's int8 scales, the cells of the next two tiles
// (selection mode), the visit counters, the tree path masks, then the selection
// list (selection mode) or the V^T indicator tile (decode with mixed visibility).
template <int D>
constexpr int lean_base_smem() {
    return kLT * D * 2 + D * 32 + 2 * kLT * 4 + 2 * kLT * 4 + 16 * 3 * 8 + 16 * 8;
}
// Decode with int8 / e4m3 rows streams its raw tiles straight into LDS, two tiles
// ahead, through buffer loads that carry the LDS destination: a raw tile is K
// [kLT][D] bytes, V [kLT][D] bytes, then 64 K and 64 V row scales (loaded for 64
// keys, the first kLT used).  Two raw tiles take the place of the 16-bit K tile,
// which these rows do not use: their score products read K's raw bytes.
template <int D>
constexpr int lean_raw_tile() { return 2 * kLT * D + 2 * 64 * 4; }
template <int D>
constexpr int lean_raw_extra() { return 2 * lean_raw_tile<D>() - kLT * D * 2; }
template <int MODE, int KT>
constexpr bool lean_raw(int) { return MODE == kDecode && byte_kv(KT); }

// The tiles of a unit may be seen in part by some of its query vectors (decode with
// MIX), and their V may hold Inf or NaN (not int8).
template <int MODE, int KT, bool MIX>
constexpr bool lean_check(int) { return MODE == kDecode && MIX && KT != SEL_ATTN_I8; }

// CP: cache policy of the decode K/V stream loads (0 default, 2 non-temporal).
// MIX: decode rows of a unit may see different keys (several rows, causal or tree).
template <int MODE, int KT, int D, int CP, bool TREE, bool MIX>
__device__ __forceinline__ void lean_unit(const MParams& p, const int t_split, const int gy, const int bz,
                                          char* smem) {
    constexpr bool F16 = (KT == SEL_ATTN_F16);
    constexpr bool B8 = byte_kv(KT);       // int8 or e4m3 rows with row scales
    constexpr int NKK = D / 32;
    constexpr int NDB = D / 16;
    constexpr int GCH = B8 ? D / 16 : D / 8;        // 16-byte chunks per K/V row in memory
    constexpr int K_TASKS = kLT * GCH;              // one 16-byte load each
    constexpr int V_TASKS = 4 * GCH;                // task e: keys 4 kg + 0..3, chunk ch (v_task)
    constexpr int NKL = (K_TASKS + 63) / 64;
    constexpr int NVL = (V_TASKS + 63) / 64;
    constexpr int EPC = B8 ? 16 : 8;
    // MIX: the unit's rows see different keys (causal or tree windows of several
    // rows).  Its tiles that some query vectors see only in part have their staged V
    // staged with their non-finite V values split off into an indicator tile at
    // vt_lds + IND (int8 data is always finite); see split_nonfinite.  In selection
    // mode the query vectors of a wave are heads of one row.
    constexpr bool CHK = lean_check<MODE, KT, MIX>(0);
    constexpr int IND = lean_base_smem<D>() - kLT * D * 2;

    // RAW: raw tiles in LDS (decode with byte rows); otherwise register-staged tiles
    constexpr bool RAW = lean_raw<MODE, KT>(0);
    constexpr int RAWB = lean_raw_tile<D>();
    char* k_lds = smem;                          // 16-bit K tile, or (RAW) the two raw tiles
    char* vt_lds = smem + (RAW ? 2 * RAWB : kLT * D * 2);
    float* ksc_lds = reinterpret_cast<float*>(vt_lds + D * 32);
    float* vsc_lds = ksc_lds + kLT;
    int* tcell = reinterpret_cast<int*>(vsc_lds + kLT);                       // [2][kLT]
    unsigned long long* dbg_lds = reinterpret_cast<unsigned long long*>(tcell + 2 * kLT);   // [16][3]
    unsigned long long* tpath_lds = dbg_lds + 16 * 3;                                    // [16]
    int* list = reinterpret_cast<int*>(tpath_lds + 16);

    const int lane = threadIdx.x;
    const int ln = lane & 15;
    const int lg = lane >> 4;
    const int G = p.G;

    // ---- work unit ---------------------------------------------------------
    const int g = gy % p.Hkv;
    const int qchunk = gy / p.Hkv;
    int b = 0, kvl = 0, lo = 0, hi = 0, row0 = 0;
    if constexpr (MODE == kDecode) {
        b = bz;
        kvl = min(max(p.kv_len[b], 0), p.cap);
        lo = t_split * p.slice_len;
        if (lo >= kvl) return;
        hi = min(lo + p.slice_len, kvl);
    } else {
        row0 = bz;
        lo = t_split * p.split_step;
        hi = min(lo + p.split_step, p.n_kv);
    }
    const int m_wg = qchunk * 16;

    // this lane's query vector
    const int m = m_wg + ln;
    bool ok = m < p.M;
    int r, h;
    if constexpr (MODE == kDecode) { r = m / G; h = g * G + m % G; ok = ok && r < p.R; }
    else { r = row0; h = g * G + m; }
    if (!ok) { r = (MODE == kDecode) ? 0 : row0; h = g * G; }
    int pos, lim;
    constexpr bool tree = (MODE == kDecode) && TREE;     // tree windows (launched when p.tree is set)
    if constexpr (MODE == kDecode) {
        pos = kvl - p.R + r;
        lim = min((p.causal && !tree) ? min(pos + 1, kvl) : kvl, hi);
        // tree windows: the window nodes this query vector sees, kept in LDS for the
        // tiles that reach the window (read after the first tile's barrier)
        if constexpr (tree) {
            const unsigned long long path = tree_path_mask_wave(p.tree + static_cast<int64_t>(b) * p.R, p.R, r);
            if (lg == 0) tpath_lds[ln] = path;
        }
    } else {
        pos = p.q_pos ? p.q_pos[r] : 0;
        lim = 0x7fffffff;
    }
    if (!ok) lim = -1;

    // Q^T operands, scale folded in
    u32x4 qop[NKK];
    {
        const float* qp = (MODE == kDecode)
                              ? p.q + ((static_cast<int64_t>(b) * p.R + r) * p.Hq + h) * D
                              : p.q + (static_cast<int64_t>(r) * p.Hq + h) * D;
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
#pragma unroll
            for (int j = 0; j < 4; ++j) qop[kk][j] = pack2<F16>(x[2 * j] * p.scale, x[2 * j + 1] * p.scale);
        }
    }
    const float slope = (p.alibi && ok) ? p.alibi[h] : 0.f;

    // ---- key slots --------------------------------------------------------------
    int n_keys, n_full = 0;
    int id0 = 0;                               // selection: first list entry of this split
    if constexpr (MODE == kSel) {
        const int32_t* srow = p.sel + static_cast<int64_t>(row0) * p.n_sel;
        int n_ids = 0;
        // an id is valid iff 0 <= id < nblk
        const int nblk = static_cast<int>((static_cast<int64_t>(p.n_kv) + p.bs - 1) / p.bs);
#ifdef SELATTN_PLANT_KEEP_REPEATS
        // test-only planted mistake (never in a product build): the valid ids in list
        // order, repeats kept
        if (nblk <= kLT * D * 2 * 8) {
            for (int base = 0; base < p.n_sel; base += 64) {
                const int e = base + lane;
                const int x = e < p.n_sel ? srow[e] : -1;
                const bool keep = x >= 0 && x < nblk;
                const unsigned long long bal = __ballot(keep);
                const int rank = __popcll(bal & ((1ull << lane) - 1ull));
                if (keep) list[n_ids + rank] = x;
                n_ids += __popcll(bal);
            }
            __syncthreads();
        } else
#endif
        if (nblk <= kLT * D * 2 * 8) {
            // the row's valid ids as a bitmap over the blocks (in the K tile's LDS,
            // free until the first tile): set bits collapse repeats, and reading the
            // words in order gives the ids sorted; a prefix count over the lanes
            // places each word's ids
            uint32_t* bm = reinterpret_cast<uint32_t*>(k_lds);
            const int nw = (nblk + 31) >> 5;
            for (int w = lane; w < nw; w += 64) bm[w] = 0u;
            __syncthreads();
            for (int e = lane; e < p.n_sel; e += 64) {
                const int x = srow[e];
                if (x >= 0 && x < nblk) atomicOr(&bm[x >> 5], 1u << (x & 31));
            }
            __syncthreads();
            for (int base = 0; base < nw; base += 64) {
                const int w = base + lane;
                uint32_t bits = w < nw ? bm[w] : 0u;
                const int c = __popc(bits);
                int incl = c;                               // inclusive prefix count over the wave
#pragma unroll
                for (int d = 1; d < 64; d <<= 1) {
                    const int t = __shfl_up(incl, d, 64);
                    if (lane >= d) incl += t;
                }
                int pos = n_ids + incl - c;
                while (bits) {
                    list[pos++] = w * 32 + (__ffs(bits) - 1);
                    bits &= bits - 1u;
                }
                n_ids += __shfl(incl, 63, 64);
            }
            __syncthreads();
        } else {
            // the row's list: invalid ids become +inf, bitonic sort in LDS, then the
            // repeats are dropped by a wave-wide compaction (ballot + prefix count)
            const int P = p.sel_pow2;
            for (int e = lane; e < P; e += 64) {
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
                    for (int e = lane; e < P; e += 64) {
                        const int o = e ^ j;
                        if (o > e) {
                            const int x = list[e], y = list[o];
                            if ((x > y) == ((e & kq) == 0)) { list[e] = y; list[o] = x; }
                        }
                    }
                    __syncthreads();
                }
            }
            // keep element e if it is valid and differs from element e - 1; kept
            // elements move down to their rank (never above their own index, and each
            // block is read before it is written, so in place is safe)
            int prev = -1;
            for (int base = 0; base < P; base += 64) {
                const int e = base + lane;
                const int x = e < P ? list[e] : 0x7fffffff;
                const int up = __shfl_up(x, 1, 64);          // every lane takes part in the exchange
                const int before = lane > 0 ? up : prev;
                const bool keep = x != 0x7fffffff && x != before;
                const unsigned long long bal = __ballot(keep);
                const int rank = __popcll(bal & ((1ull << lane) - 1ull));
                prev = __shfl(x, 63, 64);
                __syncthreads();
                if (keep) list[n_ids + rank] = x;
                n_ids += __popcll(bal);
                __syncthreads();
            }
        }
        if (p.dbg_sel && t_split == 0 && qchunk == 0) {
            int32_t* dst = p.dbg_sel + (static_cast<int64_t>(row0) * p.Hkv + g) * (1 + p.n_sel);
            if (lane == 0) dst[0] = n_ids;
            for (int e = lane; e < n_ids; e += 64) dst[1 + e] = list[e];
        }
        // A split covers cells [lo, hi): its ids are the sorted run from the first
        // whose block ends after lo to the last whose block starts before hi.
        int first = 0, last = 0;
        for (int base = 0; base < n_ids; base += 64) {
            const int e = base + lane;
            const int64_t x = e < n_ids ? list[e] : 0x7fffffff;
            first += __popcll(__ballot(e < n_ids && (x + 1) * p.bs <= lo));
            last += __popcll(__ballot(e < n_ids && x * p.bs < hi));
        }
        id0 = first;
        n_keys = max(0, last - first) * p.bs;
    } else {
        int lim_max = -1, lim_min = 0x7fffffff;
        const int m_end = min(p.M, m_wg + 16);
        for (int rr = m_wg / G; rr <= (m_end - 1) / G && rr < p.R; ++rr) {
            const int l = (p.causal && !tree) ? min(kvl - p.R + rr + 1, kvl) : kvl;
            lim_max = max(lim_max, l);
            lim_min = min(lim_min, tree ? max(kvl - p.R, 0) : l);
        }
        n_keys = max(0, min(hi, lim_max) - lo);
        n_full = max(0, min(hi, lim_min) - lo);        // slots every query vector sees
    }

    // Selection mode: the cells of a tile's 16 slots are looked up once, by lanes
    // 0..15, into tcell[tile & 1] (-1 for none), a tile ahead of their use.
    auto fill_cells = [&](int t0) {
        if constexpr (MODE == kSel) {
            if (lane < kLT) {
                const int kslot = t0 + lane;
                int c = -1;
                if (kslot < n_keys) {
                    const int id = list[id0 + kslot / p.bs];
                    const int cc = id * p.bs + kslot % p.bs;
                    if (cc < p.n_kv && cc >= lo && cc < hi) c = cc;
                }
                tcell[((t0 / kLT) & 1) * kLT + lane] = c;
            }
        }
    };

    const int64_t kv_base = (MODE == kDecode ? static_cast<int64_t>(b) * p.kv_ss : 0) +
                            static_cast<int64_t>(g) * p.kv_sh;
    const int64_t sc_base = (MODE == kDecode ? static_cast<int64_t>(b) * p.sc_ss : 0) +
                            static_cast<int64_t>(g) * p.sc_sh;
    // K and V rows are read with buffer loads.  The descriptor of a decode unit
    // starts at its first key row and ends at the end of its last visible row, so
    // the rows past it (the tail of the last tile) read as zeros without a test;
    // in selection mode it covers the whole cache and an absent cell gets an offset
    // past the end.  Offsets are 32-bit (cell stride * cells < 2^31, checked on the host).
    constexpr int ROWB = D * (B8 ? 1 : 2);
    const int cb = static_cast<int>(p.kv_sc * (B8 ? 1 : 2));
    const char* kbase = static_cast<const char*>(p.k) + kv_base * (B8 ? 1 : 2);
    const char* vbase = static_cast<const char*>(p.v) + kv_base * (B8 ? 1 : 2);
    int nrec;
    if constexpr (MODE == kSel) {
        nrec = (p.n_kv - 1) * cb + ROWB;
    } else {
        kbase += static_cast<int64_t>(lo) * cb;
        vbase += static_cast<int64_t>(lo) * cb;
        nrec = n_keys > 0 ? (n_keys - 1) * cb + ROWB : 0;
    }
    const __amdgpu_buffer_rsrc_t krs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(kbase), static_cast<short>(0), nrec, 0x00020000);
    const __amdgpu_buffer_rsrc_t vrs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(vbase), static_cast<short>(0), nrec, 0x00020000);
    constexpr int kAbsent = 0x7ffffff0;        // an offset past any descriptor's end
    // Cache policy of the decode K/V stream: non-temporal when a unit is read by one
    // work-group only (the rows are used once and should not displace reusable
    // lines); the default when several query chunks share it through the L2.
    constexpr int kStream = CP;
    const int voff_k = (lane / GCH) * cb + (lane % GCH) * 16;            // decode: K task of lane
    int vkg0, vch0;                                                       // V task of lane (the
    v_task<GCH>(lane, vkg0, vch0);                                        // i-th load adds 16 i chunks)
    const int voff_v = 4 * vkg0 * cb + vch0 * 16;                         // decode: V task of lane

    // RAW: raw tile `buf` of the tile starting at key t0.  Load c of K (and of V)
    // fills its bytes 1024 c .. 1024 c + 1023, lane l the 16 at 1024 c + 16 l: key
    // (1024 c + 16 l) / D, slot s = ((1024 c + 16 l) mod D) / 16 of the row, which
    // holds 16-byte chunk s ^ ksw(key) of K (s ^ vsw(key) of V) so that the operand
    // and staging reads below meet no bank conflicts.  Lane l < kLT of the two scale
    // loads takes key l.  2 NRK + 2 loads a tile, all of the wave.
    constexpr int NRK = kLT * D / 1024;
    constexpr int NDT = 2 * NRK + 2;
    auto ksw = [](int key) { return key & (GCH - 1); };
    auto vsw = [](int key) { return GCH >= 16 ? 8 * ((key >> 2) & 1) : 0; };
    auto dma_tile = [&](int t0, int buf) __attribute__((always_inline)) {
        if constexpr (RAW) {
            const int scb = static_cast<int>(p.sc_sc) * 4;
            const int nsc = n_keys > 0 ? (n_keys - 1) * scb + 4 : 0;
            const int64_t sc_first = sc_base + static_cast<int64_t>(lo) * p.sc_sc;
            const i32x4_t krw = raw_rsrc(kbase, nrec), vrw = raw_rsrc(vbase, nrec);
            const i32x4_t ksr = raw_rsrc(p.ksc + sc_first, nsc), vsr = raw_rsrc(p.vsc + sc_first, nsc);
            char* raw = smem + buf * RAWB;
            int l = lane;
            asm volatile("" : "+v"(l));            // recomputed here, not held across the loop
            // the tile's previous contents have been read (the last K operand read
            // fed a matrix instruction already issued; staging ran earlier)
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
            for (int c = 0; c < NRK; ++c) {
                const int pos = 1024 * c + 16 * l;
                const int key = pos / D, slot = (pos % D) >> 4;
                lds_dma<16>(krw, lds_addr(raw + 1024 * c), key * cb + ((slot ^ ksw(key)) << 4), t0 * cb);
                lds_dma<16>(vrw, lds_addr(raw + kLT * D + 1024 * c), key * cb + ((slot ^ vsw(key)) << 4), t0 * cb);
            }
            if (l < kLT) {                         // the tile's keys only (interleaved heads)
                lds_dma<4>(ksr, lds_addr(raw + 2 * kLT * D), l * scb, t0 * scb);
                lds_dma<4>(vsr, lds_addr(raw + 2 * kLT * D + 256), l * scb, t0 * scb);
            }
        }
    };

    u32x4 kreg[NKL];
    u32x4 vreg[NVL][4];
    float kscr = 0.f, vscr = 0.f;
    auto load_tile = [&](int t0) {
        const int* tc = tcell + ((t0 / kLT) & 1) * kLT;
#pragma unroll
        for (int i = 0; i < NKL; ++i) {
            const int e = lane + 64 * i;
            if constexpr (MODE == kSel) {
                const int cell = e < K_TASKS ? tc[e / GCH] : -1;
                const int off = cell >= 0 ? cell * cb + (e % GCH) * 16 : kAbsent;
                kreg[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(krs, off, 0, 0));
            } else {
                const int off = e < K_TASKS ? voff_k : kAbsent;
                kreg[i] = __builtin_bit_cast(
                    u32x4, __builtin_amdgcn_raw_buffer_load_b128(krs, off, t0 * cb + i * (64 / GCH) * cb, kStream));
            }
        }
#pragma unroll
        for (int i = 0; i < NVL; ++i) {
            const int e = lane + 64 * i;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if constexpr (MODE == kSel) {
                    int kg, ch;
                    v_task<GCH>(e, kg, ch);
                    const int cell = e < V_TASKS ? tc[4 * kg + j] : -1;
                    const int off = cell >= 0 ? cell * cb + ch * 16 : kAbsent;
                    vreg[i][j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(vrs, off, 0, 0));
                } else {
                    const int off = e < V_TASKS ? voff_v : kAbsent;
                    vreg[i][j] = __builtin_bit_cast(
                        u32x4, __builtin_amdgcn_raw_buffer_load_b128(vrs, off, (t0 + j) * cb + 256 * i, kStream));
                }
            }
        }
        if constexpr (B8) {
            if (lane < kLT) {
                int cell;
                if constexpr (MODE == kSel) cell = tc[lane];
                else cell = t0 + lane < n_keys ? lo + t0 + lane : -1;
                kscr = cell >= 0 ? p.ksc[sc_base + cell * p.sc_sc] : 0.f;
                vscr = cell >= 0 ? p.vsc[sc_base + cell * p.sc_sc] : 0.f;
            }
        }
    };
    // mode 0: plain; 1: plain, and the V words are checked for Inf / NaN (a tile some
    // query vector sees in part); 2: V split into its finite part and indicator (the
    // second staging of a checked tile that held one).  Returns (wave-uniform) whether
    // a checked tile held one.
    // (RAW: from raw tile `buf` in LDS; K stays raw, its operands are widened as read)
    auto store_tile = [&](int mode, int buf) -> bool {
        uint32_t nfa = 0u;
        const char* raw = smem + buf * RAWB;
#pragma unroll
        for (int i = 0; i < NKL; ++i) {
            const int e = lane + 64 * i;
            if (!RAW && e < K_TASKS) {
                const int key = e / GCH, ch = e % GCH;
                if constexpr (B8) {
                    const u32x4 rw = kreg[i];
                    u32x4 w0, w1;
#pragma unroll
                    for (int j = 0; j < 2; ++j) {
                        w0[2 * j] = kpair_bf16<KT>(rw[j], 0);
                        w0[2 * j + 1] = kpair_bf16<KT>(rw[j], 1);
                        w1[2 * j] = kpair_bf16<KT>(rw[2 + j], 0);
                        w1[2 * j + 1] = kpair_bf16<KT>(rw[2 + j], 1);
                    }
                    *reinterpret_cast<u32x4*>(k_lds + k16_off(key, 2 * ch, D)) = w0;
                    *reinterpret_cast<u32x4*>(k_lds + k16_off(key, 2 * ch + 1, D)) = w1;
                } else {
                    *reinterpret_cast<u32x4*>(k_lds + k16_off(key, ch, D)) = kreg[i];
                }
            }
        }
#pragma unroll
        for (int i = 0; i < NVL; ++i) {
            const int e = lane + 64 * i;
            if (V_TASKS >= 64 * (i + 1) || e < V_TASKS) {   // (no branch when every lane has a task)
                int kg, ch;
                v_task<GCH>(e, kg, ch);
                if constexpr (B8) {
                    u32x4 vw[4];
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        if constexpr (RAW) {
                            const int key = 4 * kg + j;
                            vw[j] = *reinterpret_cast<const u32x4*>(raw + kLT * D + key * D + ((ch ^ vsw(key)) << 4));
                        } else {
                            vw[j] = vreg[i][j];
                        }
                    }
                    // dims dd, dd + 1 (bytes of half (dd >> 1) & 1 of word dd >> 2) at once
#pragma unroll
                    for (int dd = 0; dd < EPC; dd += 2) {
                        const int w = dd >> 2, h = (dd >> 1) & 1;
                        uint32_t lo_e, lo_o, hi_e, hi_o;
                        vpairs_bf16<KT>(vw[0][w], vw[1][w], h, lo_e, lo_o);
                        vpairs_bf16<KT>(vw[2][w], vw[3][w], h, hi_e, hi_o);
                        if (CHK && mode != 0) {
                            nfa = store_v<F16>(vt_lds + vt16_off(ch * EPC + dd, kg), IND, lo_e, hi_e, mode == 2, nfa);
                            nfa = store_v<F16>(vt_lds + vt16_off(ch * EPC + dd + 1, kg), IND, lo_o, hi_o, mode == 2, nfa);
                        } else {
                            *reinterpret_cast<uint2*>(vt_lds + vt16_off(ch * EPC + dd, kg)) = uint2{lo_e, hi_e};
                            *reinterpret_cast<uint2*>(vt_lds + vt16_off(ch * EPC + dd + 1, kg)) = uint2{lo_o, hi_o};
                        }
                    }
                } else {
#pragma unroll
                    for (int dd = 0; dd < EPC; ++dd) {
                        const int w = dd >> 1;
                        uint32_t lo2, hi2;
                        if (dd & 1) {
                            lo2 = (vreg[i][0][w] >> 16) | (vreg[i][1][w] & 0xffff0000u);
                            hi2 = (vreg[i][2][w] >> 16) | (vreg[i][3][w] & 0xffff0000u);
                        } else {
                            lo2 = (vreg[i][0][w] & 0xffffu) | (vreg[i][1][w] << 16);
                            hi2 = (vreg[i][2][w] & 0xffffu) | (vreg[i][3][w] << 16);
                        }
                        if (CHK && mode != 0) nfa = store_v<F16>(vt_lds + vt16_off(ch * EPC + dd, kg), IND, lo2, hi2, mode == 2, nfa);
                        else *reinterpret_cast<uint2*>(vt_lds + vt16_off(ch * EPC + dd, kg)) = uint2{lo2, hi2};
                    }
                }
            }
        }
        if constexpr (RAW) {
            // (every lane: lanes l, l + 16, l + 32, l + 48 copy the same value, and no
            // branch splits the scheduling region the staging shares with the products)
            const int k = lane & (kLT - 1);
            ksc_lds[k] = reinterpret_cast<const float*>(raw + 2 * kLT * D)[k];
            vsc_lds[k] = reinterpret_cast<const float*>(raw + 2 * kLT * D + 256)[k];
        } else if constexpr (B8) {
            if (lane < kLT) {
                ksc_lds[lane] = kscr;
                vsc_lds[lane] = vscr;
            }
        }
        if constexpr (CHK) return mode == 1 && wave_any(nonfinite_found(nfa));
        return false;
    };


    // ---- running state ---------------------------------------------------------
    float m_use = kNegInf;     // exponent reference of o and l
    float m_true = kNegInf;    // largest visible non-NaN score seen
    float l_run = 0.f;
    f32x4 o_acc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) o_acc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
    // visit counters of this lane's query vector in LDS (no registers in the loop)
    unsigned long long* my_dbg = dbg_lds + ln * 3;
    if (p.dbg_visit && lg == 0) my_dbg[0] = my_dbg[1] = my_dbg[2] = 0ull;

    // Operand read addresses as base + immediate offset.  K (k16_off): row ln, chunk
    // kk * 4 + lg XOR-ed with ln, which only touches the low two bits of kk: four
    // bases.  V^T (vt16_off): dim db * 16 + ln, whose row XOR (2 * db + (ln >> 3)) & 7
    // repeats with db & 3 and whose slot XOR does not depend on db: four bases.
    int kread[4], vread[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        kread[q] = ln * D * 2 + (((q * 4 + lg) ^ ln) << 4);
        vread[q] = (ln ^ ((2 * q + (ln >> 3)) & 7)) * 32 + ((lg ^ (((ln >> 3) & 1) << 1)) << 3);
    }
    // RAW: the 8 bytes of dims 8 (4 kk + lg) .. + 7 of key ln lie in chunk c = 2 kk +
    // (lg >> 1), half lg & 1, stored at slot c ^ ksw(ln): the byte offset is
    // kraw ^ (kk << 5) (the slot bits above bit 0 hold kk ^ (ln >> 1))
    const int kraw = ln * D + ((((lg >> 1) ^ (ln & 1)) << 4) | ((lg & 1) << 3)) +
                     ((((ln >> 1) & (GCH / 2 - 1))) << 5);

    if (n_keys > 0) {
        fill_cells(0);
        __syncthreads();                        // tcell written by lanes 0..15, read by all
        if constexpr (RAW) {
            dma_tile(0, 0);
            if (kLT < n_keys) dma_tile(kLT, 1);
        } else {
            load_tile(0);
        }
    }
    for (int t0 = 0; t0 < n_keys; t0 += kLT) {
        const int buf = (t0 / kLT) & 1;
        if constexpr (RAW) {
            // raw tile t0 has landed (the next one's loads may still be in flight)
            if (t0 + kLT < n_keys) wait_vm<NDT>();
            else wait_vm<0>();
        }
        // uniform: every query vector sees the whole tile
        const bool full = (MODE == kDecode) && t0 + kLT <= n_full;
        // Byte rows without the non-finite check, one V staging task per lane (RAW1):
        // the score products read raw K, not the staged V^T, so the tile's V staging
        // runs between them, one step after each product (the products form one
        // dependent chain, which would otherwise leave the vector ALU idle).
        constexpr bool RAW1 = RAW && !CHK && V_TASKS == 64;
        bool flagged = false;
        if constexpr (!RAW1) {
            flagged = store_tile(CHK && !full ? 1 : 0, buf);
            if (flagged) store_tile(2, buf);           // the registers (raw tile) still hold the tile
            if (t0 + kLT < n_keys) fill_cells(t0 + kLT);
            __syncthreads();
        }
        if constexpr (!RAW) {
            if (t0 + kLT < n_keys) load_tile(t0 + kLT);
        }

        f32x4 s = {0.f, 0.f, 0.f, 0.f};
        if constexpr (RAW) {
            const char* kr = smem + buf * RAWB;
            // every raw operand read is issued before the first product: left to
            // itself the scheduler waits for each read right before its product, which
            // puts one LDS round trip per 32 dims on the tile's critical path
            uint2 kw[NKK];
#pragma unroll
            for (int kk = 0; kk < NKK; ++kk) kw[kk] = *reinterpret_cast<const uint2*>(kr + (kraw ^ (kk << 5)));
            if constexpr (RAW1) {
                // the lane's V task (keys 4 kg .. 4 kg + 3, chunk ch) and the row scales
                int kg, ch;
                v_task<GCH>(lane, kg, ch);
                u32x4 vw[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int key = 4 * kg + j;
                    vw[j] = *reinterpret_cast<const u32x4*>(kr + kLT * D + key * D + ((ch ^ vsw(key)) << 4));
                }
                const int k = lane & (kLT - 1);         // (lanes l, l + 16, ... copy the same value)
                ksc_lds[k] = reinterpret_cast<const float*>(kr + 2 * kLT * D)[k];
                vsc_lds[k] = reinterpret_cast<const float*>(kr + 2 * kLT * D + 256)[k];
                __builtin_amdgcn_sched_barrier(0);
                // product kk, then staging steps (dims 2 j, 2 j + 1 of the task's chunk)
#pragma unroll
                for (int kk = 0; kk < NKK; ++kk) {
                    const uint2 w = kw[kk];
                    const u32x4 a = u32x4{kpair_bf16<KT>(w.x, 0), kpair_bf16<KT>(w.x, 1), kpair_bf16<KT>(w.y, 0),
                                          kpair_bf16<KT>(w.y, 1)};
                    s = mfma16x16x32<F16>(a, qop[kk], s);
#pragma unroll
                    for (int j = kk * (EPC / 2) / NKK; j < (kk + 1) * (EPC / 2) / NKK; ++j) {
                        const int dd = 2 * j, wi = dd >> 2, h = (dd >> 1) & 1;
                        uint32_t lo_e, lo_o, hi_e, hi_o;
                        vpairs_bf16<KT>(vw[0][wi], vw[1][wi], h, lo_e, lo_o);
                        vpairs_bf16<KT>(vw[2][wi], vw[3][wi], h, hi_e, hi_o);
                        *reinterpret_cast<uint2*>(vt_lds + vt16_off(ch * EPC + dd, kg)) = uint2{lo_e, hi_e};
                        *reinterpret_cast<uint2*>(vt_lds + vt16_off(ch * EPC + dd + 1, kg)) = uint2{lo_o, hi_o};
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
                __syncthreads();                       // V^T and row scales staged
            } else {
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int kk = 0; kk < NKK; ++kk) {
                    const uint2 w = kw[kk];
                    const u32x4 a = u32x4{kpair_bf16<KT>(w.x, 0), kpair_bf16<KT>(w.x, 1), kpair_bf16<KT>(w.y, 0),
                                          kpair_bf16<KT>(w.y, 1)};
                    s = mfma16x16x32<F16>(a, qop[kk], s);
                }
            }
            // the raw tile two ahead goes into this buffer, whose K, V and scales are read
            if (t0 + 2 * kLT < n_keys) dma_tile(t0 + 2 * kLT, buf);
        } else {
#pragma unroll
            for (int kk = 0; kk < NKK; ++kk) {
                const u32x4 a = *reinterpret_cast<const u32x4*>(k_lds + kread[kk & 3] + (kk >> 2) * 256);
                s = mfma16x16x32<F16>(a, qop[kk], s);
            }
        }

        // scores of keys 4 * lg + i of the tile: scale (int8 key scale), softcap,
        // ALiBi; visibility; tile maximum.  A NaN score is left out of the maximum
        // (v_max_f32 returns the other operand) and shows up as a NaN weight, hence
        // a NaN running sum, which the epilogue turns into the NaN flag.
        int cell[4];
        if constexpr (MODE == kSel) {
            const int4 c4 = *reinterpret_cast<const int4*>(tcell + ((t0 / kLT) & 1) * kLT + 4 * lg);
            cell[0] = c4.x; cell[1] = c4.y; cell[2] = c4.z; cell[3] = c4.w;
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) cell[i] = lo + t0 + 4 * lg + i;
        }
        bool vis[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) vis[i] = full || (cell[i] >= 0 && cell[i] < lim);
        if constexpr (tree) {
            if (!full) {                               // uniform: window cells by path mask
                const unsigned long long path = tpath_lds[ln];
                const int ts = kvl - p.R;
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    vis[i] = vis[i] && (cell[i] < ts || ((path >> ((cell[i] - ts) & 63)) & 1ull));
            }
        }
        float sc[4] = {s[0], s[1], s[2], s[3]};
        if constexpr (B8) {
            const float4 k4 = *reinterpret_cast<const float4*>(ksc_lds + 4 * lg);
            sc[0] *= k4.x; sc[1] *= k4.y; sc[2] *= k4.z; sc[3] *= k4.w;
        }
        if (p.softcap > 0.f) {
#pragma unroll
            for (int i = 0; i < 4; ++i) sc[i] = p.softcap * tanhf(sc[i] / p.softcap);
        }
        if (p.alibi) {
#pragma unroll
            for (int i = 0; i < 4; ++i) sc[i] += slope * static_cast<float>(cell[i] - pos);
        }
        float tmax = kNegInf;
#pragma unroll
        for (int i = 0; i < 4; ++i) tmax = fmaxf(tmax, vis[i] ? sc[i] : kNegInf);
        if (p.dbg_visit) {
            unsigned long long c = 0, sm = 0, sq = 0;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                if (vis[i]) {
                    const unsigned long long ce = static_cast<unsigned long long>(cell[i]);
                    c += 1;
                    sm += ce;
                    sq += ce * ce;
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
        float pe[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            pe[i] = vis[i] ? __builtin_amdgcn_exp2f(fmaf(sc[i], kLog2e, -mls)) : 0.f;
            l_run += pe[i];
        }
        if constexpr (B8) {
            // the row scale joins visible weights only: a NaN scale of a key this query
            // vector cannot see must not reach it
            const float4 v4 = *reinterpret_cast<const float4*>(vsc_lds + 4 * lg);
            const float vs[4] = {v4.x, v4.y, v4.z, v4.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) pe[i] = vis[i] ? pe[i] * vs[i] : 0.f;
        }
        const u32x2 pop = u32x2{pack2<F16>(pe[0], pe[1]), pack2<F16>(pe[2], pe[3])};
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
            const u32x2 a = *reinterpret_cast<const u32x2*>(vt_lds + vread[db & 3] + db * 512);
            o_acc[db] = mfma16x16x16<F16>(a, pop, o_acc[db]);
        }
        if constexpr (CHK) {
            // a tile seen in part whose staged V held a non-finite value: the product
            // above used its finite part; the visible non-finite values are counted
            // from the indicator tile and applied
            if (flagged) {
                const u32x2 pvis = u32x2{vis_pair<F16>(vis[0], vis[1]), vis_pair<F16>(vis[2], vis[3])};
#pragma unroll
                for (int db = 0; db < NDB; ++db) {
                    const u32x2 ai = *reinterpret_cast<const u32x2*>(vt_lds + IND + vread[db & 3] + db * 512);
                    const f32x4 cnt = mfma16x16x16<F16>(ai, pvis, f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
                    for (int i = 0; i < 4; ++i) o_acc[db][i] = apply_nonfinite(o_acc[db][i], cnt[i]);
                    __builtin_amdgcn_sched_barrier(0);      // a rare path: one dim block at a time
                }
            }
        }
        __syncthreads();
    }

    // ---- epilogue ---------------------------------------------------------------
    float l = l_run;
    l = wave_sum_x16(l);
    l = wave_sum_x32(l);
    int tn = (l_run != l_run) ? 1 : 0;           // a NaN visible score made a running sum NaN
    tn = wave_or_x16(tn);
    tn = wave_or_x32(tn);
    const bool nan_run = tn != 0;
    if (!ok) return;
    bool bad = nan_run || m_true == kPosInf;
    const bool split = (MODE == kDecode) || p.n_splits > 1;
    const float z = (!split && p.sinks) ? p.sinks[h] : kNegInf;    // sink logit, unsplit only
    if (z != z || z == kPosInf) bad = true;
    const bool empty = !bad && m_true == kNegInf;
    // move o and l from the lazy reference to the true maximum
    float f = 1.f;
    if (!bad && !empty && m_use != m_true) f = exp2f((m_use - m_true) * kLog2e);
    l *= f;
    float fin = f / l;                          // unsplit: out = o * fin
    if (!split && z != kNegInf && !bad && !empty) fin = sink_norm(m_use, m_true, l, z);
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
            const float inv = fin;
            if (bad) o = float4{__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""), __builtin_nanf("")};
            else if (empty) o = float4{0.f, 0.f, 0.f, 0.f};
            else o = float4{o_acc[db][0] * inv, o_acc[db][1] * inv, o_acc[db][2] * inv, o_acc[db][3] * inv};
            *reinterpret_cast<float4*>(p.out + (static_cast<int64_t>(r) * p.Hq + h) * D + d0) = o;
        } else {
            if (empty) o = float4{0.f, 0.f, 0.f, 0.f};
            else o = float4{o_acc[db][0] * f, o_acc[db][1] * f, o_acc[db][2] * f, o_acc[db][3] * f};
            *reinterpret_cast<float4*>(p.part_o + pi * D + d0) = o;
        }
    }
    if (split && lg == 0) {
        p.part_ml[pi * 2 + 0] = nan_run ? __builtin_nanf("") : m_true;
        p.part_ml[pi * 2 + 1] = bad ? __builtin_nanf("") : (empty ? 0.f : l);
    }
    if (p.dbg_visit && lg == 0 && m % G == 0) {
        int64_t di;
        if constexpr (MODE == kDecode)
            di = ((static_cast<int64_t>(b) * p.R + r) * p.Hkv + g) * p.n_slices_max + t_split;
        else
            di = (static_cast<int64_t>(r) * p.Hkv + g) * p.n_splits + t_split;
        p.dbg_visit[di * 3 + 0] = static_cast<int64_t>(my_dbg[0]);
        p.dbg_visit[di * 3 + 1] = static_cast<int64_t>(my_dbg[1]);
        p.dbg_visit[di * 3 + 2] = static_cast<int64_t>(my_dbg[2]);
    }
}

template <int MODE, int KT, int D, int CP, bool TREE, bool MIX>
__global__ __launch_bounds__(64, 2) void lean_attn_kernel(MParams p) {
    extern __shared__ __align__(16) char smem[];
    if constexpr (MODE == kDecode) {
        for_each_decode_item(p, [&](int t, int gy, int bz) {
            lean_unit<MODE, KT, D, CP, TREE, MIX>(p, t, gy, bz, smem);
            __syncthreads();
        });
    } else {
        lean_unit<MODE, KT, D, CP, TREE, MIX>(p, blockIdx.x, blockIdx.y, blockIdx.z, smem);
    }
}

template <int MODE, int KT, int D, int CP, bool TREE, bool MIX>
int lean_resident_groups(int smem) {
    static DeviceCache cache;
    return cache.get(smem, [smem]() {
        int dev = 0, cus = 0, per_cu = 0;
        if (hipGetDevice(&dev) != hipSuccess) dev = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
            cus = 256;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, lean_attn_kernel<MODE, KT, D, CP, TREE, MIX>, 64,
                                                         smem) != hipSuccess ||
            per_cu <= 0)
            per_cu = 1;
        return cus * per_cu;
    });
}

template <int MODE, int KT, int D, int CP, bool TREE, bool MIX>
hipError_t lean_launch_one(const MParams& p, dim3 grid, hipStream_t st) {
    const int smem = lean_base_smem<D>() + (MODE == kSel ? p.sel_pow2 * 4 : 0) +
                     (lean_check<MODE, KT, MIX>(0) ? D * 32 : 0) + (lean_raw<MODE, KT>(0) ? lean_raw_extra<D>() : 0);
    if constexpr (MODE == kDecode) {
        const long long items = static_cast<long long>(grid.x) * grid.y * grid.z;
        grid = dim3(decode_grid(items, lean_resident_groups<MODE, KT, D, CP, TREE, MIX>(smem)), 1, 1);
    }
    hipLaunchKernelGGL((lean_attn_kernel<MODE, KT, D, CP, TREE, MIX>), grid, dim3(64), smem, st, p);
    return hipGetLastError();
}

template <int MODE, int KT, int CP, bool TREE, bool MIX>
hipError_t lean_launch_dim(const MParams& p, dim3 grid, hipStream_t st) {
    return p.D == 256 ? lean_launch_one<MODE, KT, 256, CP, TREE, MIX>(p, grid, st)
                      : lean_launch_one<MODE, KT, 128, CP, TREE, MIX>(p, grid, st);
}

template <int MODE, int CP, bool TREE, bool MIX>
hipError_t lean_launch_dt(int dt, const MParams& p, dim3 grid, hipStream_t st) {
    if (dt == SEL_ATTN_BF16) return lean_launch_dim<MODE, SEL_ATTN_BF16, CP, TREE, MIX>(p, grid, st);
    if (dt == SEL_ATTN_F16) return lean_launch_dim<MODE, SEL_ATTN_F16, CP, TREE, MIX>(p, grid, st);
    if (dt == SEL_ATTN_I8) return lean_launch_dim<MODE, SEL_ATTN_I8, CP, TREE, MIX>(p, grid, st);
    return lean_launch_dim<MODE, SEL_ATTN_FP8, CP, TREE, MIX>(p, grid, st);
}

// A decode unit is read by its one work-group (the kernel is launched with one
// query chunk per kv head), so decode streams K/V with non-temporal loads;
// selection mode keeps the default policy.  Tree windows, and causal windows of
// several rows (whose rows see different keys), get their own variants so that
// the one-row decode loop carries neither path masks nor non-finite checks.
template <int MODE>
hipError_t lean_launch(int dt, const MParams& p, dim3 grid, hipStream_t st) {
    if constexpr (MODE == kDecode) {
        if (p.tree) return lean_launch_dt<MODE, 2, true, true>(dt, p, grid, st);
        if (p.R > 1 && p.causal) return lean_launch_dt<MODE, 2, false, true>(dt, p, grid, st);
        return lean_launch_dt<MODE, 2, false, false>(dt, p, grid, st);
    } else {
        return lean_launch_dt<MODE, 0, false, false>(dt, p, grid, st);
    }
}

}  // namespace mk
}  // namespace selattn
