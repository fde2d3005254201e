/*
 * psc.h — sample packing and document-causal ("varlen") attention on AMD
 * Instinct MI355X (gfx950).  C ABI of libpsc.so.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Pointers are DEVICE pointers unless the comment says (host).
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Every
 *    call that takes a stream only enqueues work on it and returns; outputs are
 *    ready when the stream reaches that point.
 *  - Return value: PSC_OK (0) or a negative psc_status.  Arguments are checked
 *    on the host before anything is enqueued; on any error nothing is launched
 *    and no output is touched.  A failed launch returns PSC_ERR_HIP.
 *  - The library allocates no device memory.  The caller owns every buffer,
 *    including the scratch `workspace`, whose size comes from the matching
 *    *_workspace / *_sizes call and whose address must be 16-byte aligned
 *    (PSC_ERR_WORKSPACE when it is null or short, PSC_ERR_INVALID when it is
 *    misaligned).  No pointer is kept after a call returns.
 *  - Calls are reentrant; two calls that share an output or a workspace buffer
 *    must not overlap in time.
 *  - No C++ exception crosses this interface.
 *
 * Source of the operations: the InternEvo documentation page
 * "数据加载与流程" (data flow) defines packing, labels, cu_seqlens and indexes
 * (sections "Dataloader加载数据", "获取Dataloader数据", "处理数据") and the
 * grouped query/key/value head layout (section "ISP并行模式下数据流程");
 * "Sample Packing：长序列 LLM 训练的 Attention 问题及优化" defines the
 * block-diagonal causal mask (section 三) and the per-document decomposition
 * used here (section 5.1).
 */
#ifndef PSC_H_
#define PSC_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum psc_status {
  PSC_OK = 0,
  PSC_ERR_INVALID = -1,     /* bad argument: null pointer, size, stride, alignment */
  PSC_ERR_UNSUPPORTED = -2, /* valid but not implemented (e.g. head_dim 96) */
  PSC_ERR_WORKSPACE = -3,   /* workspace null or smaller than required */
  PSC_ERR_CAPACITY = -4,    /* an output buffer capacity is too small */
  PSC_ERR_HIP = -5          /* the HIP runtime reported an error at launch */
} psc_status;

typedef enum psc_pack_mode {
  PSC_BUILD_PACK = 0,   /* carry-over packing (build_pack) */
  PSC_BUILD_UNPACK = 1  /* truncate to SEQ_LEN, at most micro_bsz docs a row, zero pad (build_unpack) */
} psc_pack_mode;

typedef enum psc_dtype {
  PSC_F32 = 0,
  PSC_BF16 = 1
} psc_dtype;

/* Human-readable text for a status code (static storage). */
const char* psc_strerror(int status);

/* Library version, major*10000 + minor*100 + patch. */
int psc_version(void);

/* ------------------------------------------------------------------------ */
/* Packing                                                                   */
/* ------------------------------------------------------------------------ */

/*
 * psc_pack_sizes — host-only sizing for psc_pack_build.
 *
 *   n_rows        (host out) rows to allocate: build_pack ceil(n_tokens / PL),
 *                 build_unpack ceil(n_docs / micro_bsz), PL = micro_bsz*seq_len.
 *   max_segments  (host out) capacity bound for cu_seqlens (which then needs
 *                 max_segments + 1 entries): build_pack n_docs + 2*n_rows,
 *                 build_unpack n_docs + n_rows.
 *   workspace_bytes (host out) scratch needed by psc_pack_build.
 * Errors: PSC_ERR_INVALID for an unknown mode, negative counts, micro_bsz or
 * seq_len < 1, a packed length above 2^30, or a null output pointer.
 */
int psc_pack_sizes(int mode, int64_t n_docs, int64_t n_tokens, int32_t micro_bsz,
                   int32_t seq_len, int64_t* n_rows, int64_t* max_segments,
                   size_t* workspace_bytes);

/*
 * psc_pack_build — pack documents into rows of PL = micro_bsz*seq_len tokens.
 *
 * InternEvo "数据加载与流程", section "Dataloader加载数据":
 *  - PSC_BUILD_PACK: documents are laid end to end and cut every PL tokens; a
 *    document crossing a cut continues at the start of the next row; only the
 *    last row is padded.
 *  - PSC_BUILD_UNPACK: each document is cut to its first seq_len tokens, rows
 *    take micro_bsz documents each in order, and are padded to PL.
 * Labels: the next token of the same document, -100 on a document's last token
 * and on padding (formed before a document is split across rows, after it is
 * truncated).  Padding ids are 0.  Documents with no tokens are skipped.
 * Segments (section "获取Dataloader数据"): each row is cut at its start, at
 * every document start inside it, and at the start of its padding tail; the
 * padding tail is a segment of its own.  indexes count from 0 in every segment.
 *
 * Inputs
 *   tokens       int32 [n_tokens]           token ids, documents back to back
 *   doc_offsets  int64 [n_docs + 1]         doc d = tokens[doc_offsets[d] .. doc_offsets[d+1]);
 *                                           precondition: doc_offsets[0] == 0, non-decreasing,
 *                                           doc_offsets[n_docs] == n_tokens.  Offsets outside
 *                                           [0, n_tokens] are clamped, never dereferenced.
 *   n_rows       must equal psc_pack_sizes' n_rows.
 * Outputs (all written in full)
 *   input_ids, labels, indexes  int32 [n_rows][PL]
 *   cu_seqlens   int32 [max_segments + 1]   all rows' boundaries, flattened: row r's
 *                                           boundary b is stored as r*PL + b, so the
 *                                           array runs from 0 to rows_filled*PL.
 *                                           Entries after index n_seg are not written.
 *   row_seg_ptr  int32 [n_rows + 1]         row r's boundaries are
 *                                           cu_seqlens[row_seg_ptr[r] .. row_seg_ptr[r+1]].
 *   row_valid_len int32 [n_rows] or NULL    tokens before the row's padding.
 *   stats        int32 [4]                  n_seg, max_seqlen (longest segment, padding
 *                                           included), rows_filled, and 1 if doc_offsets
 *                                           broke its precondition so badly that the
 *                                           segments overran max_segments (else 0).
 * Rows past rows_filled (only when build_unpack meets empty documents) hold
 * padding only and no segment.
 * Errors: PSC_ERR_INVALID (null pointer, sizes inconsistent with
 * psc_pack_sizes), PSC_ERR_CAPACITY (max_segments too small),
 * PSC_ERR_WORKSPACE, PSC_ERR_HIP.
 */
int psc_pack_build(int mode, const int32_t* tokens, const int64_t* doc_offsets,
                   int64_t n_docs, int64_t n_tokens, int32_t micro_bsz, int32_t seq_len,
                   int64_t n_rows, int32_t* input_ids, int32_t* labels, int32_t* indexes,
                   int32_t* cu_seqlens, int64_t max_segments, int32_t* row_seg_ptr,
                   int32_t* row_valid_len, int32_t* stats, void* workspace,
                   size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------ */
/* Data steps after the packer                                                */
/* ------------------------------------------------------------------------ */
/*
 * InternEvo "数据加载与流程", section "处理数据".  cu_seqlens, row_seg_ptr and
 * row_valid_len are psc_pack_build's outputs (flattened cu_seqlens: row r's
 * boundaries are cu_seqlens[row_seg_ptr[r] .. row_seg_ptr[r+1]], offset by
 * r*packed_len); n_cu = number of entries of the cu_seqlens buffer
 * (max_segments + 1).  Reads are clamped to each row, so inconsistent
 * boundaries cannot address outside the buffers.  Errors: PSC_ERR_INVALID
 * (null pointer with a nonzero size, negative or oversized sizes, tp or rank
 * out of range, length not a multiple of tp), PSC_ERR_HIP.
 */

/* psc_row_max_seqlen — packed_data_normalizer's max_seqlen: out[r] = the
 * longest segment of row r (padding tail included), int32 [n_rows]. */
int psc_row_max_seqlen(const int32_t* cu_seqlens, int64_t n_cu, const int32_t* row_seg_ptr, int64_t n_rows,
                       int32_t* out, void* stream);

/* psc_unpack_data — unpack_data: document i < micro_bsz of packed row r
 * (input_ids, labels [n_rows, packed_len]) goes to row r*micro_bsz + i of
 * out_ids, out_labels [n_rows*micro_bsz, seq_len], cut to seq_len, padded
 * with ids 0 and labels -100.  A segment starting at or past row_valid_len[r]
 * is the padding tail, not a document; a row's documents past micro_bsz are
 * dropped (only carry-over rows can have them). */
int psc_unpack_data(const int32_t* input_ids, const int32_t* labels, int64_t n_rows, int32_t packed_len,
                    const int32_t* cu_seqlens, int64_t n_cu, const int32_t* row_seg_ptr,
                    const int32_t* row_valid_len, int32_t micro_bsz, int32_t seq_len, int32_t* out_ids,
                    int32_t* out_labels, void* stream);

/* psc_split_sequence — split_data_sequence_parallel of one int32 array
 * [rows, length] (input_ids, labels or indexes; packed or unpacked): rank
 * `rank` of `tp` gets out [rows, length/tp] = in[:, rank*length/tp ...).
 * length must be a multiple of tp, 0 <= rank < tp. */
int psc_split_sequence(const int32_t* in, int64_t rows, int32_t length, int32_t tp, int32_t rank, int32_t* out,
                       void* stream);

/* ------------------------------------------------------------------------ */
/* Rotary position embedding from the packer's indexes                      */
/* ------------------------------------------------------------------------ */

/*
 * psc_rope — rotate q [T, hq, D] and k [T, hkv, D] in place by the position of
 * each token inside its document, positions[t] (int32 [T]; the packer's
 * `indexes`, which restart at 0 in every segment: InternEvo "数据加载与流程",
 * section "获取Dataloader数据").  Dims i and i + D/2 (i < D/2) of every head
 * turn by theta_i = positions[t] * base^(-2i/D):
 *   x_i' = x_i cos - x_{i+D/2} sin,   x_{i+D/2}' = x_{i+D/2} cos + x_i sin,
 * the rotate-half form of apply_rotary_pos_emb(q, k, cos, sin) (XTuner
 * sequence-parallel page, section "实现方案").  inverse != 0 turns by -theta
 * (the backward pass: it maps dq', dk' to the gradients of q, k).
 * The angle is reduced modulo 2*pi in fp64, products are fp32, results are
 * rounded to `dtype` once.  Addressing: base + t*tok_stride + h*D + d
 * (elements); base and tok_stride*sizeof(element) must be multiples of 16
 * bytes.  k may be NULL (then hkv is ignored).  head_dim: 32, 64, 128 for
 * both dtypes; base > 0 and finite.
 * Errors: PSC_ERR_INVALID (null q or positions, alignment, stride below
 * heads*D, bad base), PSC_ERR_UNSUPPORTED (head_dim), PSC_ERR_HIP.
 */
int psc_rope(int dtype, void* q, int64_t q_tok_stride, int32_t hq, void* k, int64_t k_tok_stride,
             int32_t hkv, int64_t total_tokens, int32_t head_dim, const int32_t* positions, float base,
             int inverse, void* stream);

/* ------------------------------------------------------------------------ */
/* Document-causal attention                                                 */
/* ------------------------------------------------------------------------ */

/*
 * Shapes shared by the attention calls.  T = total_tokens (all rows laid end to
 * end; a row end is always a segment end, so rows need no separate handling).
 *   q   [T, hq,  D] ; k, v [T, hkv, D] ; out, dout [T, hq, D]
 * Each is addressed as base + t*tok_stride + h*D + d (strides in elements), so
 * q, k, v may be views into one packed qkv buffer.  tok_stride >= heads*D;
 * for PSC_BF16, base and tok_stride*2 must be multiples of 16 bytes and
 * tok_stride at most 2^25 elements (a 64-row tile's byte offsets fit 32 bits);
 * otherwise PSC_ERR_INVALID.
 * cu_seqlens int32 [n_segments + 1]: 0 = c_0 < c_1 < ... < c_n = T (strictly
 * increasing).  This is a precondition: release builds do not check it (every
 * access is still clamped to [0, T), so a bad array gives wrong results, never
 * an access outside the tensors); builds with debug checks (psc_debug_checks()
 * returns 1) run psc_check_cu_seqlens first, wait for it, and return
 * PSC_ERR_INVALID before any launch when it fails.  max_seqlen >= the longest
 * segment (used for scratch sizing only; never for addressing).
 * Query head h reads key/value head h / (hq/hkv) (grouped-query attention:
 * InternEvo "数据加载与流程", section "ISP并行模式下数据流程", qkv split).
 * softmax_scale <= 0 selects 1/sqrt(D).
 * head_dim: 32, 64 or 128 for both dtypes (PSC_BF16 runs head_dim 32 in its
 * 64-column kernels with the extra columns zeroed; results are those of the
 * 32 columns).
 * Accuracy of PSC_BF16 (P and dS are rounded to bf16 before their products):
 * against fp64 attention of the same bf16 inputs of unit scale, O, lse, dQ,
 * dK and dV were measured within max-abs 2e-2 and rel-L2 5e-3 for
 * softmax_scale up to 1.5/sqrt(D) and up to 4 query heads per key/value head
 * at head_dim 64 and 128 (up to 2 at head_dim 32).  Beyond that the max-abs
 * error of the gradients grows while rel-L2 stays near 2e-3: softmax_scale
 * 1.75/sqrt(D) gave dK 3.1e-2 and 0.2 at D = 128 (2.26/sqrt(D)) dK 3.2e-2 and
 * dQ 2.8e-2; 8 query heads per key/value head at D = 128 gave dV 2.07e-2 and
 * 4 at head_dim 32 dK 2.01e-2 (dK and dV sum the rounding of every head of
 * the group).
 *
 * Every token i of segment [s, e) attends to keys j with s <= j <= i and to
 * nothing else (one causal triangle per document, "Sample Packing：长序列 LLM
 * 训练的 Attention 问题及优化", section 三); no mask is ever stored and no tile
 * outside the triangles is visited (section 5.1).
 */

/* psc_varlen_attn_workspace — scratch bytes for pass 0 (psc_varlen_attn_fwd),
 * 1 (psc_varlen_attn_bwd), 2 (psc_varlen_attn_fwd_rope) or 3
 * (psc_varlen_attn_bwd_rope). */
int psc_varlen_attn_workspace(int pass, int dtype, int64_t total_tokens, int32_t n_segments,
                              int32_t max_seqlen, int32_t hq, int32_t hkv, int32_t head_dim,
                              size_t* bytes /* host out */);

/*
 * psc_varlen_attn_fwd
 *   out  [T, hq, D] in `dtype`, row stride out_tok_stride.
 *   lse  float32 [hq, T]: natural-log log-sum-exp of the scaled scores of each
 *        (head, token) over its causal prefix inside its document.
 * Accumulation is fp32; PSC_BF16 multiplies in bf16 (Q K^T, and P V with P
 * rounded to bf16), PSC_F32 entirely in fp32.
 */
int psc_varlen_attn_fwd(int dtype, const void* q, const void* k, const void* v,
                        int64_t q_tok_stride, int64_t k_tok_stride, int64_t v_tok_stride,
                        const int32_t* cu_seqlens, int32_t n_segments, int32_t max_seqlen,
                        int64_t total_tokens, int32_t hq, int32_t hkv, int32_t head_dim,
                        float softmax_scale, void* out, int64_t out_tok_stride, float* lse,
                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * psc_varlen_attn_fwd_noalloc — psc_varlen_attn_fwd for callers that cannot
 * allocate device memory or pass a workspace: code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation.  Same arguments,
 * results (bit for bit) and errors as psc_varlen_attn_fwd, minus the
 * workspace: the tile schedule goes to a 4 MiB scratch array built into the
 * library, one per GPU, held from its first use until the process ends.  The
 * caller still owns out and lse.  No hipMalloc, hipFree or allocating call is
 * made.  The first call on a device looks the array's address up
 * (hipGetSymbolAddress); later calls only launch.  Calls that overlap in time
 * on one GPU share the array and race: serialise them (one stream, or events).
 * Returns PSC_ERR_WORKSPACE, before any HIP call, when the workspace that
 * psc_varlen_attn_workspace reports for these sizes exceeds 4 MiB (the tile
 * list takes 16 bytes per query tile of 32 to 128 rows and about 20 bytes per
 * segment: millions of tokens).
 */
int psc_varlen_attn_fwd_noalloc(int dtype, const void* q, const void* k, const void* v,
                                int64_t q_tok_stride, int64_t k_tok_stride, int64_t v_tok_stride,
                                const int32_t* cu_seqlens, int32_t n_segments, int32_t max_seqlen,
                                int64_t total_tokens, int32_t hq, int32_t hkv, int32_t head_dim,
                                float softmax_scale, void* out, int64_t out_tok_stride, float* lse,
                                void* stream);

/*
 * psc_varlen_attn_bwd — gradients of sum(dout * out) for the forward above.
 *   out, lse: the forward's outputs for the same inputs.
 *   The workspace also carries -D_i (D_i = <dout_i, out_i>) and -lse_i / scale
 *   between the two kernels of the pass (dQ first, then dK/dV).
 *   grad_dtype: PSC_F32 (dq, dk, dv float32) or, for PSC_BF16 inputs only,
 *   PSC_BF16 (each gradient accumulated in fp32 and rounded to bf16 once, to
 *   nearest even, when stored; a bf16 gradient therefore also carries that
 *   rounding, half a bf16 ulp of its value).  PSC_F32 inputs with PSC_BF16
 *   gradients: PSC_ERR_UNSUPPORTED; any other grad_dtype: PSC_ERR_INVALID.
 *   dq [T, hq, D], dk [T, hkv, D], dv [T, hkv, D] in grad_dtype, contiguous
 *   (token stride heads*D), 16-byte aligned.  dk and dv sum over the hq/hkv
 *   query heads of each key/value head.  All three are written in full.
 */
int psc_varlen_attn_bwd(int dtype, int grad_dtype, const void* q, const void* k, const void* v,
                        const void* out, const void* dout, const float* lse,
                        int64_t q_tok_stride, int64_t k_tok_stride, int64_t v_tok_stride,
                        int64_t out_tok_stride, int64_t dout_tok_stride,
                        const int32_t* cu_seqlens, int32_t n_segments, int32_t max_seqlen,
                        int64_t total_tokens, int32_t hq, int32_t hkv, int32_t head_dim,
                        float softmax_scale, void* dq, void* dk, void* dv,
                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * Rotary embedding fused with the attention (bf16, head_dim 64 or 128).
 *
 * The model rotates q and k by each token's position inside its segment before
 * attention (InternEvo "数据加载与流程", section "获取Dataloader数据": the
 * packer's indexes; XTuner sequence-parallel page, section "实现方案": the
 * rotation right before attention), and its backward turns dq and dk back.
 * The turn is the one psc_rope applies (rotate-half pairs i, i + D/2 by
 * positions[t] * base^(-2i/D); same angles and arithmetic, so the results are
 * those of psc_rope followed by the plain attention calls, bit for bit).
 * positions: int32 [T], 0 <= positions[t] < max_seqlen (true of the packer's
 * indexes; other values are clamped into that range, never out of bounds).
 *
 * psc_varlen_attn_fwd_rope — attention of the rotated q and k.  q and k are
 *   rotated IN PLACE (on return they hold the rotated q~, k~ that the backward
 *   takes): k by the rotation kernel, q inside the attention kernel as each
 *   row is loaded (then written back).  Other arguments as
 *   psc_varlen_attn_fwd; workspace from psc_varlen_attn_workspace(2, ...)
 *   (it also holds the step's cos/sin table).
 * psc_varlen_attn_bwd_rope — gradients with respect to the UNROTATED q, k
 *   (and v) from the rotated q~, k~ the forward left: the dQ and dK kernels
 *   turn their results back by -theta before storing them, so no separate
 *   rotation pass over the gradients is needed.  Other arguments as
 *   psc_varlen_attn_bwd; workspace from psc_varlen_attn_workspace(3, ...).
 * Errors: as the plain calls, plus PSC_ERR_UNSUPPORTED for fp32 inputs or a
 * head_dim other than 64 and 128, PSC_ERR_INVALID for a null positions or a
 * rope_base that is not positive and finite.
 */
int psc_varlen_attn_fwd_rope(int dtype, void* q, void* k, const void* v,
                             int64_t q_tok_stride, int64_t k_tok_stride, int64_t v_tok_stride,
                             const int32_t* cu_seqlens, int32_t n_segments, int32_t max_seqlen,
                             int64_t total_tokens, int32_t hq, int32_t hkv, int32_t head_dim,
                             const int32_t* positions, float rope_base, float softmax_scale,
                             void* out, int64_t out_tok_stride, float* lse,
                             void* workspace, size_t workspace_bytes, void* stream);

int psc_varlen_attn_bwd_rope(int dtype, int grad_dtype, const void* q_rot, const void* k_rot,
                             const void* v, const void* out, const void* dout, const float* lse,
                             int64_t q_tok_stride, int64_t k_tok_stride, int64_t v_tok_stride,
                             int64_t out_tok_stride, int64_t dout_tok_stride,
                             const int32_t* cu_seqlens, int32_t n_segments, int32_t max_seqlen,
                             int64_t total_tokens, int32_t hq, int32_t hkv, int32_t head_dim,
                             const int32_t* positions, float rope_base, float softmax_scale,
                             void* dq, void* dk, void* dv,
                             void* workspace, size_t workspace_bytes, void* stream);

/*
 * psc_check_cu_seqlens — device check of the cu_seqlens precondition
 * (InternEvo "数据加载与流程", section "获取Dataloader数据": boundaries of the
 * documents and padding of each row, from 0 to the packed length).  Enqueues
 * one kernel on `stream` that reads cu_seqlens[0 .. n_segments] and writes
 * flags[0] (int32, device) = 0 if 0 = c_0 < c_1 < ... < c_n = total_tokens,
 * else the OR of PSC_CU_BAD_START (c_0 != 0), PSC_CU_BAD_END
 * (c_n != total_tokens) and PSC_CU_NOT_INCREASING (some c_{i+1} <= c_i).
 * Errors: PSC_ERR_INVALID (null pointer, negative or oversized sizes),
 * PSC_ERR_HIP.
 */
enum { PSC_CU_BAD_START = 1, PSC_CU_BAD_END = 2, PSC_CU_NOT_INCREASING = 4 };
int psc_check_cu_seqlens(const int32_t* cu_seqlens, int32_t n_segments, int64_t total_tokens,
                         int32_t* flags, void* stream);

/* psc_cu_seqlens_status — host-only: PSC_OK for a flags word of 0 from
 * psc_check_cu_seqlens, PSC_ERR_INVALID for any other value. */
int psc_cu_seqlens_status(int32_t flags);

/* psc_debug_checks — 1 if this library was built with debug checks (the
 * attention calls then validate cu_seqlens before launching), else 0. */
int psc_debug_checks(void);

/* ------------------------------------------------------------------------ */
/* Instrumentation                                                           */
/* ------------------------------------------------------------------------ */

/*
 * Kernel timing with HIP events.  While enabled, every launch of the kernels
 * below is bracketed by two events recorded on the launch stream (the whole
 * packer sequence counts as one "pack" launch).  psc_timing_read waits for the
 * recorded events and returns the summed elapsed time and launch count since
 * the last reset.  Host-side bookkeeping is thread safe; disabled by default.
 * psc_timing_select limits the timed kernels to those whose bit (1 << k,
 * k a psc_kernel) is set in kernel_mask (all of them by default, 0xFFFFFFFF),
 * so a measurement can keep the events of one kernel alone in its timed
 * region; it never fails.
 */
typedef enum psc_kernel {
  PSC_K_PACK = 0,
  PSC_K_ATTN_SCHEDULE = 1,
  PSC_K_ATTN_FWD = 2,
  PSC_K_ATTN_BWD_PRE = 3, /* reserved: not launched any more (the dQ kernel computes D) */
  PSC_K_ATTN_BWD_DKDV = 4,
  PSC_K_ATTN_BWD_DQ = 5,
  PSC_K_ROPE = 6,
  PSC_K_DATA_STEPS = 7
} psc_kernel;

int psc_timing_enable(int enable);
int psc_timing_select(uint32_t kernel_mask);
int psc_timing_reset(void);
int psc_timing_read(int kernel, double* total_ms /* host out */, int64_t* launches /* host out */);
const char* psc_kernel_name(int kernel);

#ifdef __cplusplus
}
#endif
#endif /* PSC_H_ */
