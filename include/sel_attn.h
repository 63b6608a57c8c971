/*
 * sel_attn.h - selected-key and split-K flash attention on AMD MI355X (gfx950).
 *
 * A C ABI over hand-written HIP kernels.  Every pointer in an argument struct
 * is a DEVICE pointer unless stated otherwise; every call is asynchronous on
 * the HIP stream passed as `hip_stream` (a hipStream_t, NULL = the default
 * stream) and never synchronises the host.
 *
 * Ownership: the caller owns every buffer.  The library never allocates,
 * frees or keeps a pointer after a call returns.  Its only state is the
 * scratch array of sel_attn_decode_noalloc (one per device, held until the
 * process ends) and per-device launch settings it looks up once.
 *
 * Errors: every entry point validates its arguments on the host before any
 * HIP call and returns a negative status (nothing is launched) when they are
 * unusable.  Data-dependent conditions are NOT errors: invalid or duplicate
 * selection ids, NaN or infinite values in Q, K, V, scales or mask, kv_len
 * values outside [0, cap] (clamped), all have defined results below.  The
 * library never aborts the process.
 *
 * Numerics (the semantics each kernel implements; the FP64 oracle in the test
 * suite is the definition):
 *   s_j = scale * (q . k_j)                 k_j widened exactly (int8: q8 * k_scale)
 *   if softcap > 0:  s_j = softcap * tanh(s_j / softcap)      (softcap first ...)
 *   if alibi:        s_j += slope[h] * (j - pos)              (... then ALiBi ...)
 *   if mask:         s_j += mask[row][j]   (F32, never clamped; added last)
 *   out = sum_j exp(s_j - m) v_j / (sum_j exp(s_j - m) + exp(sink_h - m))
 *         over the visible keys, m = max(max_j s_j, sink_h); without sinks the
 *         sink term is absent (the same as sink_h = -inf).
 *   - a key outside the visible set is never read (NaN stored there has no
 *     effect); a -inf mask entry removes the key from the visible set;
 *   - an empty visible set, or one whose scores are all -inf, gives +0.0;
 *   - any NaN score in the visible set, or a +inf maximum, gives NaN in every
 *     output dim of that (row, head); NaN in v_j at dim d gives NaN at dim d;
 *   - the sink counts as one more score for these rules: a NaN or +inf sink
 *     gives NaN, a -inf sink changes nothing, and an empty row gives +0.0 with
 *     any other sink.
 *   Query head h reads kv head h / (n_head_q / n_head_kv).
 *   Accumulation is fp32; bf16/fp16/int8 paths round Q (and the softmax
 *   weights before the P.V product) to bf16 or fp16 for the matrix cores.
 *
 * Sources (page title; part of the page):
 *   online softmax and fixed key tiles ... TensorFold PR #985, "What this changes";
 *   split decode over slices + merge ..... TensorFold PR #2595, PR body and
 *                                          "Kernel contract";
 *   maskless selected-key attention ...... strix-llama.cpp PR #115, "Overview"
 *                                          and the Vulkan selected-key commit message;
 *   softcap/ALiBi order, F32 mask, zero rows, NaN through the combine,
 *   attention-sink logit ................. HartsyInference PR #910, PR body,
 *                                          review and the M03 follow-up comment;
 *   tree-shaped verify windows ........... TensorFold PR #2595, "Kernel contract"
 *                                          (tree widths with heap-order parents).
 */
#ifndef SEL_ATTN_H
#define SEL_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SEL_ATTN_ABI_VERSION 2

/* status codes */
#define SEL_ATTN_OK            0
#define SEL_ATTN_EINVAL       (-1) /* null pointer, bad size, inconsistent arguments */
#define SEL_ATTN_EUNSUPPORTED (-2) /* valid request this library does not implement */
#define SEL_ATTN_EWORKSPACE   (-3) /* partial buffer too small for the slices */
#define SEL_ATTN_EHIP         (-4) /* the HIP runtime reported an error at launch */

/* storage type of K and V (Q, mask, scales, partials and outputs are fp32) */
#define SEL_ATTN_F32  0
#define SEL_ATTN_F16  1
#define SEL_ATTN_BF16 2
#define SEL_ATTN_I8   3 /* int8 rows, one fp32 scale per (cell, kv head) row */
#define SEL_ATTN_FP8  4 /* e4m3 rows (maximum 448, no infinities, 0x7f/0xff NaN), one fp32
                           scale per (cell, kv head) row (TensorFold PR #911: scale amax / 448) */

/* op ids for sel_attn_supports */
#define SEL_ATTN_OP_DECODE  1
#define SEL_ATTN_OP_PREFILL 2
#define SEL_ATTN_OP_COMBINE 3

/*
 * Split-K decode over key slices (TensorFold PR #2595: the attn_decode grid of
 * rows, heads and slices; PR #911: verify windows of up to 16 streams x 16 rows).
 *
 * Stream b holds kv_len[b] cells (clamped to [0, cap]); its n_row query rows
 * are the newest rows of that cache: row r sits at position
 * pos = kv_len[b] - n_row + r and sees cells [0, pos] when `causal`, else
 * [0, kv_len[b]).  ALiBi uses (j - pos).
 *
 * Tree windows (tree_parent != NULL; TensorFold PR #2595: tree widths 1..16
 * with heap-order parents): the window cells kv_len[b] - n_row + a, a in
 * [0, n_row), are the nodes of a tree; tree_parent[b*n_row + a] is the parent
 * of node a, which must precede it (-1 or any entry outside [-1, a) makes a a
 * root).  Row r then sees every cell before the window plus the window cells
 * of r and its ancestors; `causal` is ignored and pos is as above.  n_row must
 * be at most 64 (else EUNSUPPORTED).  The table is read on the device.
 *
 * Slice t covers cells
 * [t*slice_len, (t+1)*slice_len); a stream has ceil(kv_len[b] / slice_len)
 * slices and the kernel writes, for every one of them and every (row, head),
 * an unnormalised partial:
 *   part_o [S][R][Hq][n_slices_max][D]  sum_j exp(s_j - m) v_j
 *   part_ml[S][R][Hq][n_slices_max][2]  { m, l }: m = max s_j (NaN if any score
 *                                       is NaN), l = sum_j exp(s_j - m);
 *   a slice the row cannot see gets m = -inf, l = 0, o = 0.
 * Slices at or past a stream's slice count are not written.
 *
 * Layouts: q fp32 [S][R][Hq][D] contiguous.  K and V element (b, cell, g, d)
 * at b*kv_stride_stream + cell*kv_stride_cell + g*kv_stride_head + d
 * (strides in elements; d contiguous).  Int8 scales (b, cell, g) at
 * b*sc_stride_stream + cell*sc_stride_cell + g*sc_stride_head.
 * K, V must be 16-byte aligned and every K/V stride a multiple of 16 bytes.
 *
 * Requirements (else EINVAL): non-null q, k, v, kv_len, part_o, part_ml;
 * positive sizes; n_head_q % n_head_kv == 0; slice_len > 0; cap > 0;
 * I8 and FP8 need k_scale and v_scale.  EUNSUPPORTED: head_dim not 64, 128 or 256;
 * unknown dtype; softcap < 0 or not finite; scale not finite; K/V, q or
 * part_o not 16-byte aligned.  EWORKSPACE: n_slices_max * slice_len < cap.
 */
typedef struct sel_attn_decode_args {
    int32_t n_stream, n_row, n_head_q, n_head_kv, head_dim;
    int32_t cap;                 /* cells allocated per stream */
    const float* q;
    const void* k;
    const void* v;
    int32_t kv_dtype;            /* SEL_ATTN_F32 / F16 / BF16 / I8 / FP8 */
    int64_t kv_stride_stream, kv_stride_cell, kv_stride_head;
    const float* k_scale;        /* I8 and FP8 only */
    const float* v_scale;        /* I8 and FP8 only */
    int64_t sc_stride_stream, sc_stride_cell, sc_stride_head;
    const int32_t* kv_len;       /* [S] device */
    int32_t causal;
    float scale;
    float softcap;               /* 0 = off */
    const float* alibi_slopes;   /* [Hq] or NULL */
    int32_t slice_len;
    int32_t n_slices_max;
    float* part_o;
    float* part_ml;
    int64_t* dbg_visit;          /* NULL, or [S][R][Hkv][n_slices_max][3]: for each
                                    slice the kernel ran, {count, sum cell, sum cell^2}
                                    of the cells it combined for that row */
    const int32_t* tree_parent;  /* NULL, or [S][R] device: tree windows (above) */
} sel_attn_decode_args;

/*
 * Log-sum-exp merge of split partials (TensorFold PR #2595 attn_merge;
 * strix-llama.cpp PR #115 split-K reduce; NaN kept per HartsyInference
 * PR #910 review item 1).  For each (b, r, h): M = max over the stream's slices
 * of m (NaN if any is NaN); M NaN or +inf -> NaN output; M = -inf -> +0.0;
 * else out = sum_t w_t o_t / sum_t w_t l_t with w_t = exp(m_t - M), slices
 * with m_t = -inf skipped.  With sinks (fp32 [Hq] device, one logit per query
 * head; HartsyInference PR #910) M also takes sinks[h] and the denominator
 * gains exp(sinks[h] - M); a NaN sink gives NaN.  The sink is applied here
 * only, once per (b, r, h): decode partials never hold it.
 * Slice count of stream b: ceil(min(max(kv_len[b], 0), cap) / slice_len) when
 * kv_len is given, else n_slices_max for every stream.
 * out fp32 [S][R][Hq][D] contiguous.  EINVAL: null part_o/part_ml/out,
 * non-positive sizes, kv_len given with slice_len <= 0 or cap <= 0.
 * EUNSUPPORTED: head_dim not 64/128/256; part_o or out not 16-byte aligned;
 * part_ml not 8-byte aligned.
 */
typedef struct sel_attn_combine_args {
    int32_t n_stream, n_row, n_head_q, head_dim;
    int32_t n_slices_max;
    const int32_t* kv_len;       /* [S] device, or NULL */
    int32_t slice_len;
    int32_t cap;
    const float* part_o;
    const float* part_ml;
    float* out;
    const float* sinks;          /* [Hq] device, or NULL */
} sel_attn_combine_args;

/*
 * Prefill attention in exactly one of two modes.
 *
 * Selection mode (sel != NULL, mask == NULL; strix-llama.cpp PR #115): row r's
 * visible cells are the union over its list sel[r][0..n_sel) of the cells
 * [id*block_size, (id+1)*block_size) ∩ [0, n_kv) of each VALID id
 * (0 <= id and id*block_size < n_kv).  Invalid and repeated ids are skipped;
 * no causal or other mask applies.  1 <= n_sel <= 4096, block_size >= 1.
 *
 * Mask mode (mask != NULL, sel == NULL; HartsyInference PR #910): key j < n_kv
 * is visible to row r unless mask[r*mask_stride_row + h*mask_stride_head + j]
 * is -inf, or causal and j > q_pos[r].  mask_stride_head 0 broadcasts one
 * [R][n_kv] mask over the heads.
 *
 * q fp32 [R][Hq][D]; K/V element (cell, g, d) at cell*kv_stride_cell +
 * g*kv_stride_head + d, int8 scales at cell*sc_stride_cell + g*sc_stride_head.
 * q_pos int32 [R] is required when causal or ALiBi is used.
 *
 * n_splits == 1: out fp32 [R][Hq][D], with the sink logits `sinks` (fp32 [Hq]
 * device, or NULL) in the softmax.  n_splits > 1: the key range [0, n_kv)
 * is cut into n_splits ranges of ceil(n_kv / n_splits) cells and partials in
 * the decode format are written to part_o [R][Hq][n_splits][D] and
 * part_ml [R][Hq][n_splits][2] (`sinks` is not read); sel_attn_split_combine
 * with n_stream = 1, n_slices_max = n_splits, kv_len = NULL and the sinks
 * merges them.
 *
 * Debug outputs (NULL to skip): dbg_visit int64 [R][Hkv][n_splits][3]
 * {count, sum cell, sum cell^2} of the cells combined; dbg_sel int32
 * [R][Hkv][1 + n_sel]: the number of unique valid ids, then those ids in the
 * ascending order the kernel visits them (written by split 0).
 *
 * EINVAL: null q/k/v, both or neither of sel/mask, out (or partials) null,
 * non-positive sizes, n_head_q % n_head_kv, q_pos missing, n_sel outside
 * [1, 4096], block_size < 1, n_splits < 1.  EUNSUPPORTED as for decode, and
 * also: more than 32 query heads per kv head in mask mode; selection mode with
 * fp32 K/V or head_dim 64.  q, out and part_o must be 16-byte aligned.
 */
typedef struct sel_attn_prefill_args {
    int32_t n_row, n_head_q, n_head_kv, head_dim;
    int32_t n_kv;
    const float* q;
    const void* k;
    const void* v;
    int32_t kv_dtype;
    int64_t kv_stride_cell, kv_stride_head;
    const float* k_scale;
    const float* v_scale;
    int64_t sc_stride_cell, sc_stride_head;
    const int32_t* q_pos;
    float scale;
    float softcap;
    const float* alibi_slopes;
    /* selection mode */
    const int32_t* sel;
    int32_t n_sel;
    int32_t block_size;
    /* mask mode */
    const float* mask;
    int64_t mask_stride_row, mask_stride_head;
    int32_t causal;
    /* outputs */
    int32_t n_splits;
    float* out;
    float* part_o;
    float* part_ml;
    int64_t* dbg_visit;
    int32_t* dbg_sel;
    const float* sinks;          /* [Hq] device, or NULL (n_splits == 1 only) */
} sel_attn_prefill_args;

/* Entry points.  Return SEL_ATTN_OK or a negative status; see above. */
int sel_attn_decode(const sel_attn_decode_args* a, void* hip_stream);
int sel_attn_split_combine(const sel_attn_combine_args* a, void* hip_stream);
int sel_attn_prefill(const sel_attn_prefill_args* a, void* hip_stream);

/*
 * Partial-buffer sizes a decode call needs (TensorFold PR #911: the partials
 * arena is sized after admission for the streams admitted).  Writes the bytes
 * of part_o and part_ml for n_slices_max = ceil(cap / slice_len); either
 * output pointer may be NULL.  Returns a status (host-only, no HIP call).
 */
int sel_attn_decode_workspace(const sel_attn_decode_args* a, size_t* part_o_bytes,
                              size_t* part_ml_bytes);

/*
 * Capability probe (strix-llama.cpp PR #115: supports_op takes the op exactly
 * when the kernel does).  op is SEL_ATTN_OP_*; args points to the matching
 * struct.  Returns 1 when the call with these arguments would be accepted,
 * 0 otherwise.  Host-only: validates, launches nothing.
 */
int sel_attn_supports(int op, const void* args);

/* Static text for a status code. */
const char* sel_attn_strerror(int status);

/* SEL_ATTN_ABI_VERSION of the built library. */
int sel_attn_abi_version(void);

/* sizeof of the argument struct of `op` (SEL_ATTN_OP_*), 0 if unknown: lets a
 * binding check its mirror of the structs against the built library. */
size_t sel_attn_args_size(int op);

/* Which kernel family a call with these arguments uses: 0 = generic vector
 * ALU kernel, 1 = matrix-core (MFMA) kernel; negative status if invalid. */
int sel_attn_decode_path(const sel_attn_decode_args* a);
int sel_attn_prefill_path(const sel_attn_prefill_args* a);

/*
 * Decode and combine without any allocation, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.  It computes exactly what sel_attn_decode followed by
 * sel_attn_split_combine computes (same kernels), and writes the combined
 * output out fp32 [S][R][Hq][D] (16-byte aligned), with the optional sink
 * logits `sinks` fp32 [Hq] (device, or NULL) as in the combine.
 *
 * The split partials live in a scratch array of SEL_ATTN_NOALLOC_SCRATCH_BYTES
 * that the library holds on each device it runs on until the process ends: a
 * call needs S * R * Hq * ceil(cap / slice_len) * (head_dim + 2) * 4 bytes of
 * it (the 16-stream split-K and the 16 x 16-row verify workloads fit).  The
 * call allocates and frees nothing, on the host or the device.
 *
 * Arguments: as sel_attn_decode, except that a->part_o and a->part_ml must be
 * NULL and a->n_slices_max is ignored (ceil(cap / slice_len) is used).
 * Status: EINVAL for a NULL a or out, or partial pointers given; EWORKSPACE
 * when the partials would exceed the scratch; otherwise the statuses of
 * sel_attn_decode and sel_attn_split_combine, checked before anything runs;
 * EHIP if the scratch cannot be looked up on the current device.
 * Every call on one device uses that device's one scratch array: calls that
 * overlap on one device (two streams, two host threads) race and must be
 * ordered by the caller.  Nothing in the scratch needs clearing between calls.
 */
#define SEL_ATTN_NOALLOC_SCRATCH_BYTES (64u * 1024u * 1024u)
int sel_attn_decode_noalloc(const sel_attn_decode_args* a, float* out, const float* sinks,
                            void* hip_stream);

#ifdef __cplusplus
}
#endif

#endif /* SEL_ATTN_H */
