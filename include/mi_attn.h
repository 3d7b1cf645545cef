/*
 * mi_attn.h: C ABI of the masked FlashAttention forward for AMD MI355X (gfx950).
 *
 * The operation is softmax attention with an additive mask, computed tile by tile
 * with an online (running max / running sum) softmax, as the ExecuTorch pull request
 * #10466 page describes in its "Summary" (query and key dimensions both split into
 * chunks, the softmax state rescaled as chunks arrive and finalised at the end), with
 * the guard that page asks for: a chunk whose logits are all -inf must not create NaN.
 *
 * Conventions shared by every entry point:
 *  - All tensor pointers are DEVICE pointers owned by the caller. The library keeps no
 *    pointer after a call returns.
 *  - Every call validates its arguments on the host first. On a non-zero return nothing
 *    has been enqueued and no output was touched; attn_last_error() gives a message.
 *  - Work is enqueued on `stream` (a hipStream_t; NULL means the default stream).
 *    Temporary device memory (split-KV partial results, top-k ranks, kept-key lists) is a
 *    block the library allocates once per GPU and reuses across calls, holding it until
 *    the process ends. A call on another stream than the block's previous user first
 *    makes its stream wait, on the device, for that user's work; host threads calling
 *    concurrently take turns while enqueueing. The library does not synchronise with the
 *    host, except when a call needs a larger block than it holds: it then waits for the
 *    earlier calls' use of the old block to end before freeing it.
 *  - Layouts are row-major and contiguous:
 *      q, out      [B, Hq,  Lq, d]   elements of `dtype`
 *      k, v        [B, Hkv, Lk, d]   elements of `dtype`
 *      lse         [B, Hq,  Lq]      fp32
 *      mask        [Lq, Lk]          fp32, the same for every batch and head
 *      zero_hold   [B, Hkv, Lk]      fp32, one value per key of each KV head
 *  - Query row i sits at absolute key position p_i = Lk - Lq + i (bottom-right
 *    alignment). This is how causal attention over past keys works without padding
 *    the queries (FastChat pull request #2315 page, "Enable use_cache support with
 *    Flash-Attention"). When Lq == Lk it is the ordinary top-left causal mask.
 *  - Query head h reads KV head h / (Hq / Hkv): MHA when Hq == Hkv, GQA/MQA when
 *    Hq % Hkv == 0, an error otherwise (InfiniTrain pull request #193 page,
 *    "Framework and autograd").
 */
#ifndef MI_ATTN_H
#define MI_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MI_ATTN_ABI_VERSION 9

/* element types of q, k, v, out */
#define MI_ATTN_F32 0
#define MI_ATTN_F16 1
#define MI_ATTN_BF16 2

/* mask kinds */
#define MI_ATTN_MASK_NONE 0   /* every key visible                                        */
#define MI_ATTN_MASK_CAUSAL 1 /* key j visible iff j <= p_i                                */
#define MI_ATTN_MASK_WINDOW 2 /* key j visible iff p_i - window_left <= j <= p_i           */
#define MI_ATTN_MASK_DENSE 3  /* logit += mask[i, j]; -inf hides the key                   */
#define MI_ATTN_MASK_TOPK 4   /* causal, and j in the row's dynamic top-k: logit += zh[j]  */

/* return codes */
#define MI_ATTN_OK 0
#define MI_ATTN_EINVAL (-1)       /* invalid argument                                  */
#define MI_ATTN_EUNSUPPORTED (-2) /* valid but not supported by this build (e.g. d)   */
#define MI_ATTN_EHIP (-3)         /* a HIP runtime call or a launch failed            */

/*
 * attn_fwd: out = softmax(scale * q k^T + M) v, and lse = log-sum-exp of that row (natural
 * log) over the same masked, biased, scaled logits.
 *
 *   M is chosen by mask_kind (see MI_ATTN_MASK_*). For the dense kind `mask` is added to
 *   the scaled logits before the softmax, as the ExecuTorch page ("Summary") and the
 *   flash-sparse-attention issue #11 page ("Next Steps", item 1) require; finite non-zero
 *   values are allowed and only -inf hides a key. For the top-k kind the mask is built
 *   from zero_hold as dynamic_mask_topk() defines it, with keep_k keys per row.
 *
 *   A row in which every key is hidden gets out = 0 and lse = -inf, never NaN.
 *
 *   q, k, v, out   device pointers, layouts above, element type `dtype`.
 *   lse            device pointer to fp32 [B,Hq,Lq], or NULL to skip writing it.
 *   scale          multiplies q k^T (typically 1/sqrt(d)); must be finite.
 *   window_left    used by MI_ATTN_MASK_WINDOW only; must be >= 0.
 *   mask           required (non-NULL) for MI_ATTN_MASK_DENSE, ignored otherwise.
 *   zero_hold      required for MI_ATTN_MASK_TOPK, ignored otherwise.
 *   keep_k         used by MI_ATTN_MASK_TOPK only; must be >= 1.
 *   dtype          MI_ATTN_F32, MI_ATTN_F16 or MI_ATTN_BF16. fp32 inputs are computed
 *                  in fp32 throughout; fp16/bf16 inputs use fp32 accumulation and the
 *                  output is rounded to nearest-even in the input type.
 *   stream         hipStream_t (as void*), NULL for the default stream.
 *
 *   Supported head dims: fp16/bf16: 64 and 128; fp32: any multiple of 4 up to 256.
 *   Returns MI_ATTN_OK, MI_ATTN_EINVAL (sizes <= 0, Hq % Hkv != 0, non-finite scale,
 *   unknown mask_kind or dtype, a required pointer NULL, keep_k < 1, window_left < 0),
 *   MI_ATTN_EUNSUPPORTED (head dim not in the list above) or MI_ATTN_EHIP.
 *   A mask argument is never silently ignored: the kinds that need one reject NULL.
 */
int attn_fwd(const void* q, const void* k, const void* v, void* out, float* lse,
             int B, int Hq, int Hkv, int Lq, int Lk, int d, float scale,
             int mask_kind, int window_left, const float* mask, const float* zero_hold,
             int keep_k, int dtype, void* stream);

/*
 * dynamic_mask_topk: the dynamic top-k mask on its own, as the flash-sparse-attention
 * issue #11 page ("Overview", "Current Status") separates it from the attention kernel:
 * zero_hold values computed ahead of time select, per query row, which keys stay visible.
 *
 *   Total order of the keys of one (b, h): zero_hold descending, ties to the lower key
 *   index, -0.0 equal to +0.0. rank[b,h,j] is key j's place in that order (0 = first).
 *   Row i allows keys j <= p_i when causal != 0, every key otherwise. If the row allows
 *   more than keep_k keys, tau[b,h,i] is the keep_k-th smallest rank among them (keys
 *   with rank <= tau are kept); otherwise it is INT32_MAX and every allowed key is kept.
 *
 *   zero_hold  device fp32 [B,H,Lk] (no NaN).
 *   rank       device int32 [B,H,Lk], written.
 *   tau        device int32 [B,H,Lq], written.
 *   keep_bits  device uint32 [B,H,Lq,ceil(Lk/32)] or NULL; when given, bit (j % 32) of
 *              word j / 32 is set iff row i keeps key j.
 *   Returns MI_ATTN_OK, MI_ATTN_EINVAL or MI_ATTN_EHIP.
 */
int dynamic_mask_topk(const float* zero_hold, int B, int H, int Lq, int Lk, int keep_k,
                      int causal, int32_t* rank, int32_t* tau, uint32_t* keep_bits,
                      void* stream);

/*
 * attn_fwd_varlen: the same forward for a batch of sequences of different lengths whose
 * keys and values sit in a paged cache or packed back to back. It is the varlen call the
 * vLLM pull request #11277 page asks to align with (queries packed with cu_seqlens_q, key
 * counts from cu_seqlens_k, max_seqlen_q/k, a block table, causal and window masks) and,
 * with k_new/v_new, the form the same page's reply describes for its own backend: the
 * cached keys and the new tokens' keys are passed separately, so the new ones need not
 * be written into the cache before attention reads them.
 *
 *   Sequence s has Lq_s = cu_seqlens_q[s+1] - cu_seqlens_q[s] queries and
 *   Lk_s = cu_seqlens_k[s+1] - cu_seqlens_k[s] keys; its query i sits at position
 *   Lk_s - Lq_s + i (bottom-right, as in attn_fwd), and GQA maps heads as in attn_fwd.
 *
 *   q, out        [total_q, Hq, d] token-major; sequence s owns rows cu_seqlens_q[s] ...
 *   lse           fp32 [total_q, Hq] (token-major), or NULL.
 *   k, v          block_table != NULL: paged cache [kv_rows, page_size, Hkv, d]; key j of
 *                 sequence s is slot j % page_size of page
 *                 block_table[s * max_pages + j / page_size].
 *                 block_table == NULL: packed [kv_rows, Hkv, d]; key j of sequence s is
 *                 row cu_seqlens_k[s] + j.
 *   k_new, v_new  both NULL (single source), or both [total_q, Hkv, d]: then the last Lq_s
 *                 keys of sequence s are its own rows of k_new/v_new (row
 *                 cu_seqlens_q[s] + i is key Lk_s - Lq_s + i) and k/v supply only the
 *                 first Lk_s - Lq_s keys. A sequence with Lk_s < Lq_s then has no valid
 *                 split; its rows come back fully masked (out 0, lse -inf).
 *   cu_seqlens_q, cu_seqlens_k  device int32 [num_seqs + 1], nondecreasing, cu_seqlens_q
 *                 from 0 to total_q.
 *   max_seqlen_q, max_seqlen_k  the largest Lq_s and Lk_s (host values, >= 0); they only
 *                 steer how the key range is split across workgroups.
 *   block_table   device int32 [num_seqs, max_pages], or NULL (packed form).
 *   max_pages     columns of block_table (>= 1 when it is given).
 *   page_size     keys per page, a power of two (paged form; ignored when packed).
 *   kv_rows       pages (paged) or rows (packed) held by k and v, >= 1.
 *   mask_kind     MI_ATTN_MASK_NONE, _CAUSAL or _WINDOW (window_left >= 0).
 *   alibi_slopes, softcap  the score modifiers the vLLM page lists in the varlen call it
 *                 quotes, as in attn_fwd_ex (device fp32 [Hq] or NULL; softcap finite,
 *                 >= 0, 0 = off), with each sequence's own positions: key j of sequence
 *                 s gets -slope_h * |Lk_s - Lq_s + i - j|.
 *   dtype         MI_ATTN_F16 or MI_ATTN_BF16, d 64 or 128; fp32 accumulation.
 *
 *   The int32 device arrays are not read on the host. If they break the rules above,
 *   the affected rows hold unspecified values, but every read stays inside the arrays
 *   described here (indices are clamped) and nothing is written outside out and lse.
 *   total_q == 0 enqueues nothing. Temporary device memory, taken and released on the
 *   stream like attn_fwd's: the work-unit schedule (8 bytes per (sequence, query block))
 *   and, when the key range is split, fp32 partials of splits * total_q * Hq * (d + 1)
 *   values.
 *   Returns MI_ATTN_OK, MI_ATTN_EINVAL (negative sizes, Hq % Hkv != 0, a required pointer
 *   NULL, exactly one of k_new/v_new given, page_size not a power of two, non-finite
 *   scale, window_left < 0, softcap negative or not finite, unknown dtype or mask_kind), MI_ATTN_EUNSUPPORTED (fp32, the
 *   dense or top-k mask, head dim other than 64/128) or MI_ATTN_EHIP.
 */
int attn_fwd_varlen(const void* q, const void* k, const void* v, void* out, float* lse,
                    const int32_t* cu_seqlens_q, int max_seqlen_q,
                    const int32_t* cu_seqlens_k, int max_seqlen_k,
                    int num_seqs, int total_q, int Hq, int Hkv, int d, float scale,
                    int mask_kind, int window_left,
                    const int32_t* block_table, int max_pages, int page_size, int kv_rows,
                    const void* k_new, const void* v_new, const float* alibi_slopes, float softcap,
                    int dtype, void* stream);

/*
 * attn_fwd_ex: attn_fwd with general layouts, per-head masks and score modifiers.
 *
 * The vLLM pull request #11277 page lists, in the varlen call its reviewers ask backends
 * to align with ("API alignment" request), two score modifiers beside the mask:
 * alibi_slopes and softcap; the InfiniTrain pull request #193 page names the same two
 * among its unsupported features ("TODO"), next to an external custom mask. Neither page
 * defines them; this library takes the convention of the varlen API the vLLM page
 * quotes, in this order:
 *   t     = scale * q.k                                   (the scaled score)
 *   t     = softcap * tanh(t / softcap)                  when softcap > 0
 *   t    -= alibi_slopes[h] * |p_i - j|                  when alibi_slopes != NULL
 *   logit = t + M[b, h, i, j]                            (the mask of mask_kind)
 * with p_i = Lk - Lq + i as in attn_fwd, then the guarded softmax of attn_fwd (out 0 and
 * lse -inf for a row with no visible key).
 *
 *   q, k, v, out      device pointers; element (b, h, row, c) of q sits at
 *                     q + b*q_stride[0] + h*q_stride[1] + row*q_stride[2] + c (elements,
 *                     the head dimension contiguous), likewise k/v (over KV heads) and
 *                     out. A transposed KV cache [B, Lk, Hkv, d] is k_stride =
 *                     {Lk*Hkv*d, d, Hkv*d}. Strides are >= 0; out must not overlap itself
 *                     or the inputs. For fp16/bf16 the pointers are 16-byte aligned and
 *                     every stride a multiple of 8 elements, and (Lk - 1) * k_stride[2] + d
 *                     (likewise for v) must stay below 2^30 elements.
 *   lse               fp32 [B, Hq, Lq] contiguous, or NULL.
 *   mask              fp32 device; element (b, h, i, j) at mask + b*mask_stride[0] +
 *                     h*mask_stride[1] + i*mask_stride[2] + j*mask_stride[3]; a zero stride
 *                     shares the mask over that dimension ({0, 0, Lk, 1} is the single
 *                     [Lq, Lk] mask of attn_fwd). Required by MI_ATTN_MASK_DENSE. With
 *                     MI_ATTN_MASK_TOPK it is optional and, when given, added to the kept
 *                     keys' logits together with their zero_hold values. Ignored otherwise.
 *   zero_hold, keep_k as in attn_fwd ([B, Hkv, Lk] contiguous).
 *   topk_causal       MI_ATTN_MASK_TOPK: 1 selects among the keys j <= p_i (attn_fwd's
 *                     rule), 0 among all keys (every row keeps the same keep_k keys), as
 *                     dynamic_mask_topk's causal argument.
 *   alibi_slopes      fp32 device [Hq] or NULL.
 *   softcap           >= 0 and finite; 0 turns it off.
 *   Returns attn_fwd's codes; MI_ATTN_EINVAL also for args == NULL, a negative stride,
 *   a zero out stride over a dimension longer than 1, a misaligned pointer or stride, a
 *   negative or non-finite softcap, or topk_causal other than 0/1; MI_ATTN_EUNSUPPORTED
 *   for K/V rows too far apart.
 */
typedef struct {
  const void* q;
  const void* k;
  const void* v;
  void* out;
  float* lse;
  int64_t q_stride[3];    /* batch, head, row (elements) */
  int64_t k_stride[3];
  int64_t v_stride[3];
  int64_t out_stride[3];
  int B, Hq, Hkv, Lq, Lk, d;
  float scale;
  int mask_kind;
  int window_left;
  const float* mask;
  int64_t mask_stride[4]; /* batch, head, query row, key (elements) */
  const float* zero_hold;
  int keep_k;
  int topk_causal;
  const float* alibi_slopes;
  float softcap;
  int dtype;
} attn_fwd_args_t;

int attn_fwd_ex(const attn_fwd_args_t* args, void* stream);

/*
 * attn_fwd_dump: attn_fwd_ex (same arguments and results) that also writes the
 * intermediates of ONE key tile of ONE workgroup of the MFMA prefill kernel, so that a
 * single block can be compared with a reference step by step, as the
 * flash-sparse-attention issue #11 page proposes for locating a wrong mask application
 * ("Next Steps": dump the intermediate logits, mask values and output of one block).
 * The workgroup is the one of batch b, KV head kv_head and query block query_block
 * (attn_fwd_plan's block_m rows: the query rows of the KV head's G query heads, row
 * r = (i - query_block * block_m / G) * G + (h - kv_head * G), query-major); tile is the
 * 64-key tile index (key range [64 tile, 64 tile + 64)), or the tile of the block's
 * kept-key list when topk_list_cap > 0. dump (device, fp32, MI_ATTN_DUMP_FLOATS) receives
 *   S[128][64]   scale * q k^T + mask of the tile, natural-log units (-inf where hidden)
 *   P[128][64]   exp(S - m), fp32 before rounding to the 16-bit type of the P V product
 *   m[128]       the reference maximum m of the running softmax after this tile (natural
 *                log units; it trails the true running maximum by at most 8 ln 2)
 *   l[128]       the running sum after this tile, so l exp(m) = sum of exp(S) over the
 *                keys visited so far
 * Rows past the block's rows and tiles the kernel skips (hidden entirely) are not written.
 * MI_ATTN_EUNSUPPORTED when the call does not take the MFMA prefill path with 64-key tiles
 * (see attn_fwd_plan: path 1 and block_n 64; d = 64 with the none / causal / window kinds
 * takes 128-key tiles) or carries a score modifier (ALiBi slopes, softcap > 0, or a dense
 * mask added to top-k), MI_ATTN_EINVAL for an index out of range or a NULL dump. The dump
 * runs its own kernel instances (one workgroup per query block); the results are those
 * of attn_fwd_ex.
 */
#define MI_ATTN_DUMP_FLOATS (2 * 128 * 64 + 2 * 128)
int attn_fwd_dump(const attn_fwd_args_t* args, int b, int kv_head, int query_block, int tile, float* dump,
                  void* stream);

/*
 * attn_bwd: gradients of attn_fwd, as the InfiniTrain pull request #193 page pairs the
 * FlashAttention forward with its backward ("main changes": forward and backward for
 * FP16/BF16 with head dims 64 and 128; the autograd function keeps what the backward
 * needs, "Framework and autograd"). With Z = scale * q k^T + M (M as in attn_fwd) and
 * P = softmax(Z) by rows, recomputed from the forward's lse:
 *     dv = P^T dout                      dP = dout v^T
 *     dZ = P * (dP - rowsum(dout * out)) (the softmax Jacobian)
 *     dq = scale * dZ k                  dk = scale * dZ^T q
 * With GQA a KV head's dk and dv are the sums over the Hq / Hkv query heads that read it.
 * No gradient flows into mask or zero_hold. A row whose keys are all hidden (lse = -inf)
 * contributes nothing and gets dq = 0.
 *
 *   q, k, v, out, lse   the forward's inputs and results (layouts of attn_fwd; lse must
 *                       be the one attn_fwd wrote for these inputs, not NULL).
 *   dout                device, [B, Hq, Lq, d] `dtype`: the gradient of out.
 *   dq, dk, dv          device, written (not accumulated), layouts of q, k and v. They
 *                       must not overlap the inputs. q, k, v, out, dout, dq, dk and dv
 *                       are 16-byte aligned, lse 4-byte aligned (else MI_ATTN_EINVAL).
 *   B .. keep_k, dtype  as in attn_fwd (the top-k kind selects causally, as attn_fwd).
 *   stream              as in attn_fwd. Temporary device memory: 12 bytes per query
 *                       row (its LSE, rowsum(dout * out) and a mask index), plus the
 *                       top-k ranks for that kind.
 *
 *   fp16/bf16 only (fp32 returns MI_ATTN_EUNSUPPORTED), head dims 64 and 128, at most
 *   128 query heads per KV head, Hq * Lq * d * 2 below 2^31 bytes, B * Hq * Lq * 12 below
 *   2^31. Products take fp16/bf16
 *   operands (P and dZ are rounded to the input type before the second products) with
 *   fp32 accumulation; dq, dk and dv are rounded to nearest-even in the input type.
 *   Returns attn_fwd's codes.
 */
int attn_bwd(const void* q, const void* k, const void* v, const void* out, const float* lse,
             const void* dout, void* dq, void* dk, void* dv,
             int B, int Hq, int Hkv, int Lq, int Lk, int d, float scale,
             int mask_kind, int window_left, const float* mask, const float* zero_hold,
             int keep_k, int dtype, void* stream);

/*
 * attn_fwd_noalloc: attn_fwd for callers that cannot allocate device memory during the
 * call (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc). Same arguments, same kernels and the same results as attn_fwd, but the
 * temporary memory (split-KV partials, top-k ranks, thresholds, sorted key chunks and
 * kept-key lists, dense-mask tile flags) comes from a fixed scratch array of
 * MI_ATTN_NOALLOC_MAX_WORKSPACE bytes that the library holds on each GPU it runs on until
 * the process ends; the call itself allocates and frees nothing.
 *  - A call whose plan needs more than MI_ATTN_NOALLOC_MAX_WORKSPACE bytes (see
 *    attn_plan_t.workspace_bytes) returns MI_ATTN_EUNSUPPORTED before enqueuing anything.
 *  - Every call on one GPU shares that GPU's array, which keeps the last call's contents
 *    (nothing in it needs to start at zero): calls that overlap on one GPU (different
 *    streams, or different host threads) race and must be serialised by the caller.
 *  - The first call on a device looks up the array's device address there (on the
 *    device `stream` belongs to); it fails with MI_ATTN_EHIP if that lookup fails.
 */
#define MI_ATTN_NOALLOC_MAX_WORKSPACE 33554432
int attn_fwd_noalloc(const void* q, const void* k, const void* v, void* out, float* lse,
                     int B, int Hq, int Hkv, int Lq, int Lk, int d, float scale,
                     int mask_kind, int window_left, const float* mask, const float* zero_hold,
                     int keep_k, int dtype, void* stream);

/* which kernels attn_fwd would run for a shape (host-only query, no GPU work) */
typedef struct {
  int path;          /* 0 fp32 row kernel; 1 MFMA prefill (split over keys, with an LSE merge,
                        when there are few workgroups); 2 split-KV decode + LSE merge        */
  int block_m;       /* query rows per workgroup (rows of all heads sharing a KV head)   */
  int block_n;       /* keys per KV tile (128 for d = 64 with the none / causal / window
                        kinds on path 1, else 64; 32 on path 2)                           */
  int splits;        /* key-range splits merged by log-sum-exp (paths 1, 2); 1 if unsplit */
  int grid;          /* query blocks of the main kernel, one workgroup each; on path 1 with
                        the none / causal / window kinds and one split, more blocks than the
                        GPU holds at once run on that many resident workgroups, each taking
                        several blocks                                                    */
  int mask_summary;  /* 1 when a per-tile dense-mask summary kernel runs first            */
  size_t workspace_bytes; /* temporary device memory the call takes                     */
  int topk_list_cap; /* top-k on path 1: keys per query block's kept-key list (the block's
                        tiles are runs of that list); 0 when every tile of the causal range
                        is visited and masked per element                                  */
} attn_plan_t;

/*
 * attn_fwd_plan: fill *plan for the arguments attn_fwd would get (pointers are not
 * needed). Validates exactly as attn_fwd does and returns the same error codes. Runs on
 * the host only; usable without a GPU.
 */
int attn_fwd_plan(int B, int Hq, int Hkv, int Lq, int Lk, int d, int mask_kind,
                  int window_left, int keep_k, int dtype, attn_plan_t* plan);

/*
 * attn_set_debug: process-wide debug switches (not thread-safe; for tests and tuning).
 *   no_skip      1: visit every KV tile, even ones the mask hides entirely.
 *   force_path   -1: automatic; 0/1/2 force the path numbers of attn_plan_t (a forced
 *                path that cannot run the arguments makes attn_fwd return
 *                MI_ATTN_EUNSUPPORTED; path 2 needs (Hq / Hkv) * Lq <= 32).
 *   force_splits 0: automatic; n > 0 asks for n key-range splits on paths 1 and 2 (fewer
 *                when the key range has fewer tiles).
 */
void attn_set_debug(int no_skip, int force_path, int force_splits);

/*
 * attn_read_stream: read `bytes` bytes at device pointer `src` once, as a plain stream of
 * 16-byte loads (with the non-temporal cache hint when `nontemporal` != 0, the hint the
 * split-KV decode kernel puts on its V loads), and write one XOR of the data per
 * MI_ATTN_READ_STREAM_CHUNK bytes to sink[0 .. ceil(bytes / MI_ATTN_READ_STREAM_CHUNK) - 1]
 * (device memory, caller-owned). No page defines this operation: it is a measurement aid,
 * the practical HBM read ceiling that the decode path's bandwidth is reported against.
 * `src` must be 16-byte aligned and `bytes` a positive multiple of 16, else MI_ATTN_EINVAL
 * (nothing enqueued). MI_ATTN_EHIP if the launch fails. Enqueued on `stream`, no sync.
 */
#define MI_ATTN_READ_STREAM_CHUNK 2097152
int attn_read_stream(const void* src, size_t bytes, int nontemporal, uint32_t* sink, void* stream);

/*
 * attn_last_error: message for the last non-zero return on the calling thread ("" if
 * none). Every rejected argument (a mask kind without its pointer, an unsupported head
 * dimension, Hq % Hkv != 0, ...) returns an error code with a message here instead of
 * being ignored or silently replaced: the InfiniTrain pull request #193 page ("TODO",
 * and the review comment under it) notes that its flash path ignored a parsed mask and
 * asks for an error or a fallback in that case.
 * Ownership: the string is owned by the library (thread-local storage) and stays valid
 * until the next call on the same thread. Never fails.
 */
const char* attn_last_error(void);

/*
 * attn_abi_version: MI_ATTN_ABI_VERSION of the loaded library. A caller compiled against
 * this header asserts that the loaded library has the same version before relying on
 * its semantics (argument lists, mask conventions such as the bottom-right alignment),
 * as the FastChat pull request #2315 page does with an assert on the flash-attn version
 * so that the corrected q_len != kv_len causal behaviour is guaranteed to be present.
 * Host-only; never fails.
 */
int attn_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* MI_ATTN_H */
