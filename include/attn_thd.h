/*
 * attn_thd.h -- C ABI of the MI355X (gfx950) THD varlen attention library.
 *
 * Fused scaled-dot-product attention, forward (O and the softmax statistic
 * LSE) and backward (dQ, dK, dV), over packed variable-length sequences in
 * THD layout, with grouped-query attention and the "padding" and
 * "padding_causal" masks (the causal triangle aligned top-left or
 * bottom-right).
 *
 * Operation (TransformerEngine issue 3333 "FusedAttention (cuDNN) THD
 * backward produces wrong gradients on sm_120", section "Reproduction": a
 * per-sequence SDPA; issue 3216 "flash-attn-4 4.0.0b11: ... wrong dQ/dK/dV
 * at head_dim=256", section "Reproduce": GQA by repeating KV heads, scale,
 * causal triangle).  For every sequence b and query head h, with
 * g = h / (hq / hkv):
 *     S   = scale * Q_bh K_bg^T             (Lq_b x Lk_b)
 *     P   = softmax over the allowed keys    (padding: all real keys;
 *                                             padding_causal: key j <= query i;
 *                                             bottom-right: j <= i + Lk_b - Lq_b)
 *     O   = P V_bg,     LSE_i = ln sum_{j allowed} exp(S_ij)
 *   backward, from dO:
 *     dP = dO V^T, Delta_i = sum_c dO_ic O_ic, dS = P o (dP - Delta)
 *     dQ = scale dS K,  dK_g = scale sum_{h in g} dS^T Q,  dV_g = sum_{h in g} P^T dO
 *
 * Boundaries (issue 2892 "SIGSEGV in fused_attn_fwd when cu_seqlens_q !=
 * cu_seqlens_q_padded ...", section "Expected Behavior"): cu_seqlens_* give
 * the REAL token counts and drive the mask; cu_seqlens_*_padded give the
 * MEMORY layout and drive indexing; outputs keep the padded layout.  The
 * real tokens of sequence b are rows [cu_padded[b], cu_padded[b] + L_b) of
 * its slot; the rest of the slot is padding.  Issue 2448 "Inconsistent
 * fused_attn_bwd results of dk, dv under THD layout + GQA on multiple
 * calls", section "Expected behavior": KV rows of a sequence without valid
 * queries get dK = dV = 0, and no result depends on earlier calls.
 *
 * Layouts (all row-major, contiguous, head_dim fastest):
 *   q, out, dout, dq : [total_q,  hq,  d]  dtype (bf16 or fp16)
 *   k, v, dk, dv     : [total_kv, hkv, d]  same dtype
 *   lse              : [total_q,  hq]      float32, natural log
 *   cu_seqlens_*     : int32 [batch + 1], device memory, non-decreasing
 * A NULL cu_seqlens_*_padded pointer means "same as the real array".
 *
 * Every row the method does not reach is written explicitly on every call:
 * out = dq = +0.0 and lse = -inf on query rows outside the real ranges (and
 * on real query rows of a sequence with no real key); dk = dv = +0.0 on KV
 * rows outside the real ranges and on every KV row of a sequence with no
 * real query.  Outputs may therefore be uninitialised on entry.
 *
 * Ownership: every pointer is caller-owned device memory.  The library
 * never allocates, frees or caches device memory and keeps no pointer after
 * a call returns.  The workspace is scratch whose contents are undefined on
 * entry (garbage or NaN is fine): each call initialises every byte it
 * reads.  Calls are asynchronous on `stream` (a hipStream_t; NULL = the
 * default stream); no host<->device copy and no synchronisation happen
 * inside.  Concurrent calls need distinct workspaces.
 *
 * Errors: host-checkable argument errors return a non-zero status before
 * anything is enqueued (no partial writes).  Bad DEVICE data in the
 * cu_seqlens arrays (decreasing entries, a real length above its padded
 * slot, a slot beyond total_*) cannot be seen from the host: the call then
 * treats every sequence as empty -- all outputs are written as for
 * uncovered rows -- and sets a status word in the workspace, readable with
 * attn_thd_read_device_status().  The library never reads or writes out of
 * bounds on such data.
 *
 * Results are deterministic: repeated calls with the same inputs give
 * bitwise identical outputs, whatever ran before (no atomics in any
 * floating-point reduction).
 */
#ifndef ATTN_THD_H
#define ATTN_THD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ATTN_THD_OK = 0,
  ATTN_THD_EINVAL = 1,        /* bad argument: null pointer, negative size, hq % hkv != 0, ... */
  ATTN_THD_EUNSUPPORTED = 2,  /* d not a multiple of 8 in [8, 256], or unknown dtype / mask */
  ATTN_THD_EWORKSPACE = 3,    /* workspace NULL, too small or not 256-byte aligned */
  ATTN_THD_ELAUNCH = 4,       /* the HIP runtime rejected a kernel launch */
  ATTN_THD_ESCRATCH = 5       /* attn_bwd_thd_noalloc: the problem needs more than its static scratch */
} attn_thd_status;

enum { ATTN_THD_BF16 = 0, ATTN_THD_FP16 = 1 };                        /* dtype     */
enum {                                                                /* mask_type */
  ATTN_THD_MASK_PADDING = 0,
  ATTN_THD_MASK_PADDING_CAUSAL = 1,               /* top-left:     key j <= query i           */
  ATTN_THD_MASK_PADDING_CAUSAL_BOTTOM_RIGHT = 2   /* bottom-right: key j <= query i + Lk - Lq */
};

/* Device status bits (attn_thd_read_device_status). */
enum {
  ATTN_THD_DEV_OK = 0,
  ATTN_THD_DEV_BAD_SEQLENS = 1  /* cu_seqlens data inconsistent; outputs written as all-uncovered */
};

/*
 * Bytes of workspace attn_fwd_thd / attn_bwd_thd need for these sizes
 * (the same figure serves both).  Returns 0 on invalid sizes.  It holds the
 * work lists, the per-sequence table and two fp32 [total_q, hq] vectors,
 * and, when the backward spreads a GQA group's query heads over several
 * dK/dV workgroups per key tile (groups of 8 or more query heads whose key
 * tiles alone give fewer than 4096 workgroups), fp32 partial dK / dV planes
 * of 2 x split x total_kv x hkv x d floats, split being a power of two that
 * divides the group and leaves every workgroup at least 2 of its heads.  Since fewer key tokens can mean more planes, the calls
 * also accept a smaller workspace as long as it holds the rest (one sized
 * for a problem with more key tokens does): the backward then halves split
 * until its planes fit, down to 1.  Results are deterministic for a given
 * workspace_bytes; two calls that differ only in it may round dK / dV
 * differently.
 */
size_t attn_thd_workspace_size(int32_t batch, int32_t total_q, int32_t total_kv,
                               int32_t hq, int32_t hkv, int32_t d);

/*
 * Forward.  Writes out [total_q, hq, d] and lse [total_q, hq] (float32).
 *   scale         softmax scale (no default at this level; 1/sqrt(d) is usual)
 *   max_seqlen_*  an upper-bound hint only; correctness never depends on it
 *   mask_type     ATTN_THD_MASK_PADDING, ATTN_THD_MASK_PADDING_CAUSAL (the
 *                 triangle aligned top-left: query i sees keys j <= i) or
 *                 ATTN_THD_MASK_PADDING_CAUSAL_BOTTOM_RIGHT (aligned at the
 *                 sequence ends: j <= i + Lk - Lq, so the last query sees
 *                 every key).  The pages use the causal mask only with
 *                 Lq == Lk, where both alignments agree; a query row that
 *                 sees no key (bottom-right with Lq > Lk) gets out = +0.0,
 *                 lse = -inf and dq = +0.0.
 *   dtype         ATTN_THD_BF16 or ATTN_THD_FP16 (q, k, v, out)
 */
attn_thd_status attn_fwd_thd(
    const void* q, const void* k, const void* v, void* out, float* lse,
    const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_kv,
    const int32_t* cu_seqlens_q_padded, const int32_t* cu_seqlens_kv_padded,
    int32_t batch, int32_t total_q, int32_t total_kv,
    int32_t max_seqlen_q, int32_t max_seqlen_kv,
    int32_t hq, int32_t hkv, int32_t d, float scale, int32_t mask_type, int32_t dtype,
    void* workspace, size_t workspace_bytes, void* stream);

/*
 * Backward.  Reads q, k, v, out, dout and lse (as written by attn_fwd_thd
 * for the same arguments) and writes dq [total_q, hq, d], dk and dv
 * [total_kv, hkv, d].  dK/dV of a KV head are summed over the hq/hkv query
 * heads of its group in a fixed order.  Other arguments as attn_fwd_thd.
 */
attn_thd_status attn_bwd_thd(
    const void* q, const void* k, const void* v, const void* out, const void* dout,
    const float* lse, void* dq, void* dk, void* dv,
    const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_kv,
    const int32_t* cu_seqlens_q_padded, const int32_t* cu_seqlens_kv_padded,
    int32_t batch, int32_t total_q, int32_t total_kv,
    int32_t max_seqlen_q, int32_t max_seqlen_kv,
    int32_t hq, int32_t hkv, int32_t d, float scale, int32_t mask_type, int32_t dtype,
    void* workspace, size_t workspace_bytes, void* stream);

/*
 * The backward without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc).  Same operation, arguments,
 * layouts, outputs and error codes as attn_bwd_thd, and the same kernels,
 * except that it never spreads a GQA group over several dK/dV workgroups
 * (where attn_bwd_thd does, see attn_thd_workspace_size, its dK and dV are
 * summed in another order and can differ from attn_bwd_thd's in the last
 * bits; both are deterministic).  The scratch the kernels need (the work
 * lists, the per-sequence table and the per-row Delta and LSE*log2(e)
 * vectors) lives in a file-scope device array of
 * ATTN_THD_NOALLOC_SCRATCH_BYTES that the library holds on each GPU it runs
 * on until the process ends.  The call allocates nothing (no hipMalloc, no
 * allocating library routine); it looks up that GPU's copy of the array once
 * per device, on its first call there.
 *   - Problems whose workspace without partial planes exceeds
 *     ATTN_THD_NOALLOC_SCRATCH_BYTES are rejected with ATTN_THD_ESCRATCH
 *     before anything is launched (the 65536-token, 64-head problem needs
 *     about 34 MB).
 *   - The stream must belong to the current device (else ATTN_THD_EINVAL).
 *   - Every call on a GPU shares that GPU's array, and the array keeps the
 *     last call's contents: calls that overlap on one GPU (two streams, two
 *     threads) race and must be serialised by the caller.  Nothing in the
 *     array needs to start at zero: every call writes what it reads first,
 *     as with a caller-owned workspace.
 *   - Bad device data zero-fill the outputs as in attn_bwd_thd; the status
 *     word stays inside the library (attn_thd_read_device_status cannot
 *     reach it).
 */
#define ATTN_THD_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

attn_thd_status attn_bwd_thd_noalloc(
    const void* q, const void* k, const void* v, const void* out, const void* dout,
    const float* lse, void* dq, void* dk, void* dv,
    const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_kv,
    const int32_t* cu_seqlens_q_padded, const int32_t* cu_seqlens_kv_padded,
    int32_t batch, int32_t total_q, int32_t total_kv,
    int32_t max_seqlen_q, int32_t max_seqlen_kv,
    int32_t hq, int32_t hkv, int32_t d, float scale, int32_t mask_type, int32_t dtype,
    void* stream);

/*
 * Batched layouts read in place, as THD views (TransformerEngine issue 3216,
 * section "Reproduce", runs its sbhd [seq, batch, heads, d] tensors through
 * DotProductAttention; bshd is the same with batch first).  Every sequence
 * has a slot of seqlen_q query tokens and seqlen_kv key tokens:
 *   BSHD  q, out, dout, dq : [batch, seqlen_q,  hq,  d]   (token i of b is row b*seqlen_q + i)
 *         k, v, dk, dv     : [batch, seqlen_kv, hkv, d]
 *   SBHD  q, out, dout, dq : [seqlen_q,  batch, hq,  d]   (token i of b is row i*batch + b)
 *         k, v, dk, dv     : [seqlen_kv, batch, hkv, d]
 *   lse                    : float32, one value per (row, query head), rows in
 *                            the same order as q: [batch, seqlen_q, hq] for
 *                            BSHD, [seqlen_q, batch, hq] for SBHD
 * cu_seqlens_q / cu_seqlens_kv (int32 [batch + 1], device) give the REAL
 * lengths as in THD, each at most its slot; the real tokens are the first of
 * the slot and the rest is padding (written as for THD).  NULL means every
 * sequence fills its slot.  The operation, masks, outputs written, workspace
 * (attn_thd_workspace_size(batch, batch*seqlen_q, batch*seqlen_kv, hq, hkv,
 * d)), errors and stream semantics are those of attn_fwd_thd / attn_bwd_thd.
 * Extra error: ATTN_THD_EINVAL when batch*seqlen exceeds INT32_MAX or a
 * 256-token strided tile spans more than 2 GiB; ATTN_THD_EUNSUPPORTED for an
 * unknown layout.
 */
enum { ATTN_THD_LAYOUT_BSHD = 1, ATTN_THD_LAYOUT_SBHD = 2 };   /* layout */

attn_thd_status attn_fwd_batched(
    const void* q, const void* k, const void* v, void* out, float* lse,
    const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_kv, int32_t layout,
    int32_t batch, int32_t seqlen_q, int32_t seqlen_kv,
    int32_t hq, int32_t hkv, int32_t d, float scale, int32_t mask_type, int32_t dtype,
    void* workspace, size_t workspace_bytes, void* stream);

attn_thd_status attn_bwd_batched(
    const void* q, const void* k, const void* v, const void* out, const void* dout,
    const float* lse, void* dq, void* dk, void* dv,
    const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_kv, int32_t layout,
    int32_t batch, int32_t seqlen_q, int32_t seqlen_kv,
    int32_t hq, int32_t hkv, int32_t d, float scale, int32_t mask_type, int32_t dtype,
    void* workspace, size_t workspace_bytes, void* stream);

/*
 * Chunked form (the building block of context parallelism, where each GPU
 * holds chunks of a long sequence; issue 3333, section "What we ruled out",
 * mentions it only in passing).  The slots of a THD call hold
 * chunks of longer sequences: q_pos0[b] / kv_pos0[b] (int32 [batch], device;
 * either may be NULL = all 0) are the positions in its whole sequence of the
 * first real query / key of chunk b.  With mask_type
 * ATTN_THD_MASK_PADDING_CAUSAL, key j is visible to query i iff
 * kv_pos0[b] + j <= q_pos0[b] + i: the causal rule of the whole sequence
 * restricted to the two chunks (positions with another mask: EINVAL).
 *
 * attn_fwd_thd_chunk writes the PARTIAL result of the chunk's keys: out and
 * lse as attn_fwd_thd over the visible keys of the chunk (a query that sees
 * none: out = +0.0, lse = -inf).  attn_merge_thd combines two partials of
 * the same queries over disjoint key sets, in place on (out, lse):
 *     LSE = ln(e^lse + e^lse_part),
 *     O   = e^(lse - LSE) out + e^(lse_part - LSE) out_part,
 * elementwise over [total_q, hq] rows (both -inf: out = +0.0, lse = -inf),
 * in fp32, rounded once to dtype.  Merging the partials of every key chunk
 * gives the attention over the whole keys.
 *
 * attn_bwd_thd_chunk is attn_bwd_thd for one (query chunk, key chunk) pair,
 * reading out and lse of the WHOLE attention (merged) for these queries, so
 * that P and Delta = rowsum(dO o O) are the whole sequence's: its dq is the
 * chunk pair's share of dQ, its dk / dv the pair's share of dK / dV.
 * accumulate is a bit mask: with ATTN_THD_ACC_DQ the call adds its share
 * into dq, with ATTN_THD_ACC_DKDV into dk and dv (fp32 sum, one rounding),
 * and an accumulated output keeps every row the call does not reach (no zero
 * fill); outputs without their bit are written as attn_bwd_thd writes them.
 * Summing over key chunks gives dQ, over query chunks dK and dV.
 *
 * Other arguments, layouts, workspace, errors and stream semantics as
 * attn_fwd_thd / attn_bwd_thd (max_seqlen hints are not taken).  events /
 * n_events: NULL / 0, or stage events as for the *_timed entry points.
 */
/*
 * Dropout on the attention probabilities (issue 2448, "Steps/Code to
 * reproduce bug", runs with dropout 0.0; the mask below is the library's own
 * specification).  attn_fwd_thd / attn_bwd_thd with dropout_p in
 * [0, 255.5/256), a 64-bit seed and a 32-bit call offset (advance it between
 * calls that need different masks; the forward and its backward take the
 * same values):
 *   O = (P o D) V,  D_ij = keep_ij * 256 / (256 - t),  t = round(256 p),
 * LSE that of the softmax itself; the backward is the exact gradient of
 * that O (dV = (P o D)^T dO, dS = P o (D o dO V^T - Delta)).  keep_ij for
 * sequence b (its index in the batch), query head h, query i and key j
 * (positions in the sequence): the Philox4x32-10 generator (Salmon et al.,
 * SC'11) with key (seed low word, seed high word) and counter
 * (j >> 2, i >> 2, b, offset * hq + h) gives four words x0..x3; keep iff
 * byte (j & 3) of x[i & 3] is >= t.  dropout_p = 0 is the plain call.
 * Extra error: EINVAL for dropout_p outside its range or NaN.  events /
 * n_events as for the *_timed entry points (NULL / 0: none).
 */
attn_thd_status attn_fwd_thd_dropout(
    const void* q, const void* k, const void* v, void* out, float* lse,
    const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_kv,
    const int32_t* cu_seqlens_q_padded, const int32_t* cu_seqlens_kv_padded,
    int32_t batch, int32_t total_q, int32_t total_kv,
    int32_t hq, int32_t hkv, int32_t d, float scale, int32_t mask_type,
    float dropout_p, uint64_t seed, uint32_t offset, int32_t dtype,
    void* workspace, size_t workspace_bytes, void* stream,
    void* const* events, int32_t n_events);

attn_thd_status attn_bwd_thd_dropout(
    const void* q, const void* k, const void* v, const void* out, const void* dout,
    const float* lse, void* dq, void* dk, void* dv,
    const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_kv,
    const int32_t* cu_seqlens_q_padded, const int32_t* cu_seqlens_kv_padded,
    int32_t batch, int32_t total_q, int32_t total_kv,
    int32_t hq, int32_t hkv, int32_t d, float scale, int32_t mask_type,
    float dropout_p, uint64_t seed, uint32_t offset, int32_t dtype,
    void* workspace, size_t workspace_bytes, void* stream,
    void* const* events, int32_t n_events);

/*
 * Forward from FP8 inputs (issue 2892, "SIGSEGV in fused_attn_fwd when
 * cu_seqlens_q != cu_seqlens_q_padded with FP8 blockwise", runs this forward
 * on THD inputs with real != padded boundaries; the arithmetic below is the
 * library's own specification of it):
 *   q8, k8, v8  E4M3 codes (OCP 8-bit floating point, torch.float8_e4m3fn),
 *               same shapes and layouts as q, k, v of attn_fwd_thd, 8-byte
 *               aligned; descale_* > 0 their per-tensor float factors:
 *   O   = softmax(scale * descale_q * descale_k * Q8 K8^T + mask) (descale_v * V8)
 *   LSE = natural log-sum-exp of those scaled scores (float32 [total_q, hq])
 * out is written in out_dtype (ATTN_THD_BF16 or ATTN_THD_FP16).  For head
 * dims 48..256 that are multiples of 16, with q8 and k8 16-byte aligned, the
 * scores are taken on the 8-bit products (gfx950 E4M3 MFMA) straight from the
 * codes; otherwise q and k are decoded too.  v is always decoded (exactly:
 * every E4M3 value is a bf16 and an fp16 value) into a 16-bit copy in the
 * workspace, whose size is attn_thd_fp8_workspace_size(...) (larger than
 * attn_thd_workspace_size).
 * Boundaries, masks, written rows, errors and stream semantics as
 * attn_fwd_thd; NaN codes propagate.  events / n_events: NULL / 0, or 5
 * events around the stages decode, scheduler, forward kernel, zero fill.
 */
size_t attn_thd_fp8_workspace_size(int32_t batch, int32_t total_q, int32_t total_kv,
                                   int32_t hq, int32_t hkv, int32_t d);

attn_thd_status attn_fwd_thd_fp8(
    const void* q8, const void* k8, const void* v8,
    float descale_q, float descale_k, float descale_v, void* out, float* lse,
    const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_kv,
    const int32_t* cu_seqlens_q_padded, const int32_t* cu_seqlens_kv_padded,
    int32_t batch, int32_t total_q, int32_t total_kv,
    int32_t hq, int32_t hkv, int32_t d, float scale, int32_t mask_type, int32_t out_dtype,
    void* workspace, size_t workspace_bytes, void* stream,
    void* const* events, int32_t n_events);

/*
 * Backward of attn_fwd_thd_fp8 (the same issue's inputs): the gradients with
 * respect to the real-valued inputs Q = descale_q Q8, K = descale_k K8,
 * V = descale_v V8 of the forward above, by the same softmax-gradient
 * identity as attn_bwd_thd:
 *   dV = P^T dO,  dS = P o (dO V^T - Delta),  Delta = rowsum(dO o O),
 *   dQ = scale dS K,  dK = scale dS^T Q.
 * q8, k8, v8 and the descales as given to the forward (8-byte aligned codes);
 * out and lse are the forward's results, dout the gradient of out; out, dout,
 * dq, dk and dv are in dtype (ATTN_THD_BF16 or ATTN_THD_FP16), with the
 * layouts of attn_bwd_thd.  The codes are decoded exactly into 16-bit copies
 * in the workspace (attn_thd_fp8_workspace_size(...) bytes) and the descales
 * are folded into three fp32 factors: the products run on the codes with
 * score scale scale*descale_q*descale_k, dS is carried as dS / descale_v,
 * and dQ, dK are multiplied out by scale*descale_k*descale_v and
 * scale*descale_q*descale_v.  With dtype fp16, dS / descale_v is rounded to
 * fp16 before its products, so it must stay below 65504 in magnitude.
 * Returns ATTN_THD_EINVAL for a descale that is not finite and > 0 or makes
 * one of the factors overflow; boundaries, masks, written rows, other errors
 * and stream semantics as attn_bwd_thd.  events / n_events: NULL / 0, or 7
 * events around the stages decode, scheduler, dQ (+ Delta), dK/dV, zero fill
 * (q rows), zero fill (kv rows).
 */
attn_thd_status attn_bwd_thd_fp8(
    const void* q8, const void* k8, const void* v8,
    float descale_q, float descale_k, float descale_v,
    const void* out, const void* dout, const float* lse, void* dq, void* dk, void* dv,
    const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_kv,
    const int32_t* cu_seqlens_q_padded, const int32_t* cu_seqlens_kv_padded,
    int32_t batch, int32_t total_q, int32_t total_kv,
    int32_t hq, int32_t hkv, int32_t d, float scale, int32_t mask_type, int32_t dtype,
    void* workspace, size_t workspace_bytes, void* stream,
    void* const* events, int32_t n_events);

enum { ATTN_THD_ACC_DQ = 1, ATTN_THD_ACC_DKDV = 2 };   /* accumulate bits */

attn_thd_status attn_fwd_thd_chunk(
    const void* q, const void* k, const void* v, void* out, float* lse,
    const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_kv,
    const int32_t* cu_seqlens_q_padded, const int32_t* cu_seqlens_kv_padded,
    const int32_t* q_pos0, const int32_t* kv_pos0,
    int32_t batch, int32_t total_q, int32_t total_kv,
    int32_t hq, int32_t hkv, int32_t d, float scale, int32_t mask_type, int32_t dtype,
    void* workspace, size_t workspace_bytes, void* stream,
    void* const* events, int32_t n_events);

attn_thd_status attn_bwd_thd_chunk(
    const void* q, const void* k, const void* v, const void* out, const void* dout,
    const float* lse, void* dq, void* dk, void* dv,
    const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_kv,
    const int32_t* cu_seqlens_q_padded, const int32_t* cu_seqlens_kv_padded,
    const int32_t* q_pos0, const int32_t* kv_pos0,
    int32_t batch, int32_t total_q, int32_t total_kv,
    int32_t hq, int32_t hkv, int32_t d, float scale, int32_t mask_type, int32_t accumulate,
    int32_t dtype, void* workspace, size_t workspace_bytes, void* stream,
    void* const* events, int32_t n_events);

/*
 * out [total_q, hq, d] (dtype), lse [total_q, hq] fp32: updated in place;
 * out_part, lse_part: the other partial, same shapes, read only.  No
 * workspace.  Errors: EINVAL (sizes, NULL or misaligned pointers),
 * EUNSUPPORTED (d or dtype).
 */
attn_thd_status attn_merge_thd(void* out, float* lse, const void* out_part, const float* lse_part,
                               int32_t total_q, int32_t hq, int32_t d, int32_t dtype,
                               void* stream);

/*
 * Instrumented variants for benchmarks.  Same arguments and behaviour as
 * attn_fwd_thd / attn_bwd_thd (attn_fwd_batched / attn_bwd_batched for the
 * *_batched_timed pair), plus an array of caller-created HIP events
 * (hipEvent_t, passed as void*) that the call records on `stream`:
 * events[i] just before stage i is launched and events[n_events-1] after the
 * last stage, so hipEventElapsedTime(events[i], events[i+1]) is stage i.
 *   forward  (n_events = 4): scheduler, forward kernel, zero fill
 *   backward (n_events = 6): scheduler, dQ kernel (which also forms
 *                            Delta = rowsum(dO o O)), dK/dV kernel (and the
 *                            sum of its partial planes for a spread GQA
 *                            group), zero fill (query rows), zero fill (key rows)
 * A NULL `events` or another n_events returns ATTN_THD_EINVAL.  An entry
 * of `events` may be NULL: that boundary is not recorded (a caller timing one
 * stage passes only the two events around it, and adds no other records to
 * the stream).
 */
attn_thd_status attn_fwd_thd_timed(
    const void* q, const void* k, const void* v, void* out, float* lse,
    const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_kv,
    const int32_t* cu_seqlens_q_padded, const int32_t* cu_seqlens_kv_padded,
    int32_t batch, int32_t total_q, int32_t total_kv,
    int32_t max_seqlen_q, int32_t max_seqlen_kv,
    int32_t hq, int32_t hkv, int32_t d, float scale, int32_t mask_type, int32_t dtype,
    void* workspace, size_t workspace_bytes, void* stream,
    void* const* events, int32_t n_events);

attn_thd_status attn_bwd_thd_timed(
    const void* q, const void* k, const void* v, const void* out, const void* dout,
    const float* lse, void* dq, void* dk, void* dv,
    const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_kv,
    const int32_t* cu_seqlens_q_padded, const int32_t* cu_seqlens_kv_padded,
    int32_t batch, int32_t total_q, int32_t total_kv,
    int32_t max_seqlen_q, int32_t max_seqlen_kv,
    int32_t hq, int32_t hkv, int32_t d, float scale, int32_t mask_type, int32_t dtype,
    void* workspace, size_t workspace_bytes, void* stream,
    void* const* events, int32_t n_events);

attn_thd_status attn_fwd_batched_timed(
    const void* q, const void* k, const void* v, void* out, float* lse,
    const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_kv, int32_t layout,
    int32_t batch, int32_t seqlen_q, int32_t seqlen_kv,
    int32_t hq, int32_t hkv, int32_t d, float scale, int32_t mask_type, int32_t dtype,
    void* workspace, size_t workspace_bytes, void* stream,
    void* const* events, int32_t n_events);

attn_thd_status attn_bwd_batched_timed(
    const void* q, const void* k, const void* v, const void* out, const void* dout,
    const float* lse, void* dq, void* dk, void* dv,
    const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_kv, int32_t layout,
    int32_t batch, int32_t seqlen_q, int32_t seqlen_kv,
    int32_t hq, int32_t hkv, int32_t d, float scale, int32_t mask_type, int32_t dtype,
    void* workspace, size_t workspace_bytes, void* stream,
    void* const* events, int32_t n_events);

/* Human-readable name of a status code (static string, never NULL). */
const char* attn_thd_status_string(int32_t status);

/*
 * Test helper: waits for `stream`, then copies the device status word of
 * the last call that used `workspace` into *status_out (ATTN_THD_DEV_* bits).
 * This one synchronises; the compute entry points never do.
 */
attn_thd_status attn_thd_read_device_status(const void* workspace, void* stream,
                                            int32_t* status_out);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_THD_H */
