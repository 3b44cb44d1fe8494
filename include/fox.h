/*
 * fox.h -- C ABI of libfox: causal Forgetting-Transformer (FoX) attention on MI355X (gfx950).
 *
 * What is computed.  With l_t = log f_t (the log forget gate of token t of one
 * (batch, head) sequence) and c_i = sum_{t<=i} l_t:
 *
 *     s_ij  = scale * q_i . k_j + (c_i - c_j)          for j <= i   (weight 0 for j > i)
 *     lse_i = ln sum_j exp(s_ij)                      O_i = sum_j exp(s_ij - lse_i) v_j
 *
 * Sources: "Forgetting Transformer (FoX) Attention" module page
 * (frankenstein-transformer docs), ForgettingAttention.forward -- cumulative
 * sum of log gates, bias cum[i] - cum[j] added after the scaled q k^T (the bias
 * is not scaled), decoder-mode mask of the strict upper triangle, softmax over
 * keys, times v; and the foxwindow README, opening paragraph -- the same score
 * written as q.k + sum over t = j+1..i of log g_t.  lse is not defined on the
 * pages; here it is the natural-log log-sum-exp of the full logit row.
 *
 * Conventions shared by every entry point:
 *  - All pointers are DEVICE pointers (hipMalloc'd or equivalent) owned by the
 *    caller.  The library never allocates, frees or synchronises.
 *  - Every call is asynchronous on `stream` (0 = the null stream), like a
 *    kernel launch; results are valid once the stream has been synchronised.
 *  - The library keeps no mutable global state: calls are reentrant and
 *    thread-safe.  Calls that write the same buffers race like any kernels.
 *  - Tensors are dense row-major with the shapes given; Q/K/V/O element type
 *    is `dtype` (fp32 or bf16), gates / prefix sums / lse are always fp32.
 *  - Q/K/V/O pointers must be 16-byte aligned; fp32 vectors 4-byte aligned.
 *  - Argument errors are detected on the host, before anything is launched,
 *    and returned as a status; no exception or abort crosses the ABI.
 *  - Preconditions NOT checked (they would need device reads): gate values are
 *    finite and <= 0 (gates in (0,1)); buffers have the stated sizes.
 */
#ifndef FOX_H_
#define FOX_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status, dtype and layout values travel as int32_t, not as enum types: a caller may pass
   any integer (an unknown dtype is rejected with FOX_ERR_UNSUPPORTED, an unknown status gets
   "unknown status"), and an out-of-range value of an enum type would be undefined in C++. */
typedef int32_t fox_status_t;
enum fox_status_code {
  FOX_OK = 0,
  FOX_ERR_INVALID_ARG = 1, /* null pointer, size <= 0 or too large, bad scale, misaligned pointer */
  FOX_ERR_UNSUPPORTED = 2, /* head dim not in {32, 64, 128}, unknown dtype */
  FOX_ERR_WORKSPACE = 3,   /* decode workspace missing or smaller than fox_attn_decode_workspace_bytes() */
  FOX_ERR_HIP = 4,         /* the HIP runtime reported an error at launch */
  FOX_ERR_SCRATCH = 5      /* fox_attn_decode_noalloc: the sizes need more than FOX_DECODE_SCRATCH_BYTES */
};

typedef int32_t fox_dtype_t;
enum fox_dtype_code {
  FOX_F32 = 0, /* IEEE binary32 */
  FOX_BF16 = 1 /* bfloat16; products accumulate in fp32, outputs rounded to nearest even */
};

typedef int32_t fox_layout_t;
enum fox_layout_code {
  FOX_HEAD_MAJOR = 0, /* q/k/v/o [b, h, n, d]; logf / lse / c [b, h, n] */
  FOX_TOKEN_MAJOR = 1 /* q/k/v/o [b, n, h, d]; logf / lse / c [b, n, h] */
};

/* Largest sequence length / cache length accepted (keeps all index arithmetic in range). */
#define FOX_MAX_SEQ (1 << 22)

/*
 * fox_logf_cumsum -- inclusive prefix sum of log forget gates along the sequence.
 *   FoX module page, ForgettingAttention.forward: cumulative sum of log f over
 *   the sequence axis, per (batch, head).
 *
 *   logf : [rows, n] fp32, input (rows = batch * heads).
 *   c    : [rows, n] fp32, output; c[r, i] = sum_{t<=i} logf[r, t], accumulated
 *          in fp64 and rounded once to fp32.  May not alias logf.
 *   rows, n : > 0, n <= FOX_MAX_SEQ.
 */
fox_status_t fox_logf_cumsum(const float* logf, float* c, int64_t rows, int64_t n, hipStream_t stream);

/*
 * fox_attn_fwd -- causal FoX attention forward (prefill) over whole sequences.
 *   FoX module page, ForgettingAttention.forward (decoder mode), from the
 *   projected, head-split q, k, v onwards (the output projection is not part
 *   of it).
 *
 *   q, k, v : [b, h, n, d] of `dtype`, inputs.
 *   logf    : [b, h, n] fp32, input log forget gates.
 *   o       : [b, h, n, d] of `dtype`, output (bf16: rounded to nearest even).
 *   lse     : [b, h, n] fp32, output log-sum-exp (natural log) of each logit row, or NULL.
 *   c       : [b, h, n] fp32, output prefix sums of logf (as fox_logf_cumsum), or NULL;
 *             these seed a decode cache.
 *   d       : head dim, one of 32, 64, 128.
 *   scale   : multiplier of q.k (finite, > 0); the module uses d ** -0.5.
 *   Outputs must not alias inputs.
 */
fox_status_t fox_attn_fwd(const void* q, const void* k, const void* v, const float* logf, void* o, float* lse,
                          float* c, int64_t b, int64_t h, int64_t n, int64_t d, float scale, fox_dtype_t dtype,
                          hipStream_t stream);

/*
 * fox_attn_fwd_noncausal -- FoX attention forward without the causal mask.
 *   FoX module page, ForgettingAttention.forward in its default (not decoder)
 *   mode: the same scaled q k^T plus bias cum[i] - cum[j], softmax over every
 *   key of the sequence.  For a key after the query (j > i) the bias is
 *   c_i - c_j = -(sum_{t=i+1..j} log f_t) >= 0, so later keys are weighted up.
 *
 *   Arguments, layouts, outputs and errors exactly as fox_attn_fwd; lse is the
 *   log-sum-exp over all n keys of each row.
 */
fox_status_t fox_attn_fwd_noncausal(const void* q, const void* k, const void* v, const float* logf, void* o,
                                    float* lse, float* c, int64_t b, int64_t h, int64_t n, int64_t d, float scale,
                                    fox_dtype_t dtype, hipStream_t stream);

/*
 * fox_attn_fwd_ex -- fox_attn_fwd / fox_attn_fwd_noncausal with the tensor layout chosen.
 *   FoX module page, ForgettingAttention.forward: the q, k, v projections are formed as
 *   [batch, seq, heads, head_dim] and permuted to [batch, heads, seq, head_dim] before the
 *   attention; FOX_TOKEN_MAJOR takes the tensors before that permute (no copy needed), the
 *   gates likewise as [batch, seq, heads], and writes o, lse and c in the same layout.
 *
 *   causal : nonzero for decoder mode (fox_attn_fwd), zero for the unmasked mode.
 *   layout : FOX_HEAD_MAJOR or FOX_TOKEN_MAJOR (else FOX_ERR_UNSUPPORTED); with
 *            FOX_TOKEN_MAJOR, (n + 64) * h * d * sizeof(element) must not exceed 2^31 - 1
 *            (else FOX_ERR_UNSUPPORTED).
 *   Every other argument, the results and the errors as fox_attn_fwd.
 */
fox_status_t fox_attn_fwd_ex(const void* q, const void* k, const void* v, const float* logf, void* o, float* lse,
                             float* c, int64_t b, int64_t h, int64_t n, int64_t d, float scale, fox_dtype_t dtype,
                             int causal, fox_layout_t layout, hipStream_t stream);

/*
 * fox_attn_fwd_pruned_workspace_bytes -- bytes of scratch fox_attn_fwd_pruned needs
 * (one float per (batch, head, 64-key tile)).  Returns 0 for invalid sizes.
 */
size_t fox_attn_fwd_pruned_workspace_bytes(int64_t b, int64_t h, int64_t n, int64_t d);

/*
 * fox_attn_fwd_pruned -- fox_attn_fwd with gate-aware tile skipping.
 *   foxwindow README, "The window is a first-passage time": the gate bias
 *   sum_{t=j+1..i} log f_t only falls as the key j moves away from the query i,
 *   so beyond some distance every key's weight is negligible.  Walking the key
 *   tiles down from the diagonal, a query block stops once, for each of its rows,
 *   the bound  scale * |q_i| * max_j |k_j| + (c_i - c_j1)  on every remaining score
 *   (Cauchy-Schwarz; j1 the highest remaining key) lies more than (25 + log2 n) * ln 2
 *   below the row's running max: the skipped keys then weigh less than 2^-24 of the
 *   row sum, so O and lse equal fox_attn_fwd's to fp32 rounding.  Gates near 1
 *   (long windows) skip little; fp32 inputs are not pruned (full computation).
 *
 *   Arguments as fox_attn_fwd, plus
 *   workspace, workspace_bytes : device scratch of at least
 *              fox_attn_fwd_pruned_workspace_bytes(b, h, n, d) bytes, 16-byte aligned,
 *              not overlapping any other argument; contents on entry are ignored.
 *   c is produced by the prefix-sum kernel (same values as fox_logf_cumsum).
 */
fox_status_t fox_attn_fwd_pruned(const void* q, const void* k, const void* v, const float* logf, void* o,
                                 float* lse, float* c, void* workspace, size_t workspace_bytes, int64_t b, int64_t h,
                                 int64_t n, int64_t d, float scale, fox_dtype_t dtype, hipStream_t stream);

/*
 * fox_attn_bwd_workspace_bytes -- bytes of scratch fox_attn_bwd needs:
 * b*h*(3*npad + 3*n) floats plus b*h*nblk doubles, npad = n rounded up to a multiple of 64,
 * nblk = n rounded up to a multiple of 128, divided by 32.  Returns 0 for invalid sizes.
 */
size_t fox_attn_bwd_workspace_bytes(int64_t b, int64_t h, int64_t n, int64_t d);

/*
 * fox_attn_bwd -- gradients of FoX attention (decoder or unmasked mode), head-major.
 *   The pages derive no backward pass.  This is the chain rule through fox_attn_fwd's
 *   definition (FoX module page, ForgettingAttention.forward), for a loss whose gradient
 *   with respect to O is dout:
 *     P = softmax(S), dv = P^T dout, dS = P * (dout v^T - rowsum(dout * O)),
 *     dq = scale dS k, dk = scale dS^T q, and for the gates, with c_i - c_j in every score,
 *     dlogf_t = sum over i >= t of (rowsum(dS)_i - colsum(dS)_i)
 *   (the row sums of dS vanish in exact arithmetic; the kernels keep them, with both sums
 *   taken over the same fp32 dS values, so that their rounding cancels in dlogf).  The gate
 *   prefix sums are rebuilt from logf in fp64 and split at 32-position blocks, so the bias of
 *   each score carries rounding of the size of the bias itself, however large |c| grows.  In the
 *   unmasked mode rowsum(dout * O) is replaced by its exact equal sum_j P_ij (dout v^T)_ij,
 *   computed in fp32 by an extra pass (the O given is rounded to `dtype`, and that rounding
 *   would not cancel in dlogf there).
 *
 *   q, k, v, o, dout : [b, h, n, d] of `dtype`, inputs; o and lse as fox_attn_fwd (same mode)
 *                      wrote them for these q, k, v, logf and scale.
 *   lse      : [b, h, n] fp32, input (fox_attn_fwd's output).
 *   logf     : [b, h, n] fp32, input: the log forget gates the forward was given.
 *   dq, dk, dv : [b, h, n, d] of `dtype`, outputs (bf16: rounded to nearest even).
 *   dtype    : FOX_BF16 (P and dS rounded to bf16 as MFMA operands, fp32 accumulation) or FOX_F32
 *              (fp32 throughout, on the vector ALU; n up to 65535 * 64).
 *   dlogf    : [b, h, n] fp32, output: the gradient with respect to logf.
 *   workspace, workspace_bytes : device scratch of at least fox_attn_bwd_workspace_bytes(b, h, n, d)
 *              bytes, 16-byte aligned; contents on entry are ignored.
 *   causal   : nonzero for decoder mode, zero for the unmasked mode.
 *   Errors as fox_attn_fwd; every output and the workspace must not overlap any other buffer
 *   (FOX_ERR_INVALID_ARG).
 *   Every output element has one writer (no atomics): repeated calls give identical results.
 */
fox_status_t fox_attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                          const float* lse, const float* logf, void* dq, void* dk, void* dv, float* dlogf,
                          void* workspace, size_t workspace_bytes, int64_t b, int64_t h, int64_t n, int64_t d,
                          float scale, fox_dtype_t dtype, int causal, hipStream_t stream);

/*
 * fox_attn_bwd_ex -- fox_attn_bwd with the tensor layout chosen.
 *   FoX module page, ForgettingAttention.forward: the projections are formed as
 *   [batch, seq, heads, head_dim] before the permute to head-major; FOX_TOKEN_MAJOR reads q, k,
 *   v, o, dout as [b, n, h, d] and lse, logf as [b, n, h], and writes dq, dk, dv as [b, n, h, d]
 *   and dlogf as [b, n, h], the layout fox_attn_fwd_ex(..., FOX_TOKEN_MAJOR) reads and writes.
 *
 *   layout : FOX_HEAD_MAJOR or FOX_TOKEN_MAJOR (else FOX_ERR_UNSUPPORTED); with
 *            FOX_TOKEN_MAJOR, (n + 256) * h * d * sizeof(element) must not exceed 2^31 - 1
 *            (else FOX_ERR_UNSUPPORTED).
 *   Every other argument, the workspace size, the results (bit for bit, element by element)
 *   and the errors as fox_attn_bwd.
 */
fox_status_t fox_attn_bwd_ex(const void* q, const void* k, const void* v, const void* o, const void* dout,
                             const float* lse, const float* logf, void* dq, void* dk, void* dv, float* dlogf,
                             void* workspace, size_t workspace_bytes, int64_t b, int64_t h, int64_t n, int64_t d,
                             float scale, fox_dtype_t dtype, int causal, fox_layout_t layout, hipStream_t stream);

/*
 * fox_attn_bwd_staged_workspace_bytes -- bytes of scratch fox_attn_bwd_staged needs:
 * fox_attn_bwd_workspace_bytes(b, h, n, d) rounded up to a multiple of 256, plus b*h*T*8192,
 * T = sum over kb < ceil(n/128) of (ceil(n/32) - 4*kb) (the dS tiles at or below the diagonal:
 * about n*n bytes per head, so 8.7 GB for b*h = 32 and n = 16384).  Returns 0 for invalid sizes,
 * d other than 128, or n whose T*8192 exceeds 2^31 - 1 (n above 46272).
 */
size_t fox_attn_bwd_staged_workspace_bytes(int64_t b, int64_t h, int64_t n, int64_t d);

/*
 * fox_attn_bwd_staged -- fox_attn_bwd_ex in decoder mode for bf16 tensors with d = 128,
 *   trading memory for time: the key-stationary kernel writes the bf16 dS it forms (the values its
 *   own dK and column sums use) to the workspace, and dQ = scale dS k and the row sums of dS are
 *   read from there by a contraction kernel, instead of a query-stationary kernel forming S and
 *   dP a second time.  Same chain rule and definition as fox_attn_bwd (FoX module page,
 *   ForgettingAttention.forward); results agree with fox_attn_bwd to bf16 rounding of dq (not bit
 *   for bit: the row sums of dS and dQ are taken from the key side's dS).
 *
 *   Arguments as fox_attn_bwd_ex (decoder mode; layout FOX_HEAD_MAJOR or FOX_TOKEN_MAJOR, the
 *   results of the two bit for bit the same), with
 *   workspace, workspace_bytes : device scratch of at least
 *              fox_attn_bwd_staged_workspace_bytes(b, h, n, d) bytes, 16-byte aligned, not
 *              overlapping any other argument; contents on entry are ignored.
 *   Errors as fox_attn_bwd_ex, and FOX_ERR_UNSUPPORTED for a dtype other than FOX_BF16, d other
 *   than 128, or n too large for the staged tiles (see the workspace query).
 */
fox_status_t fox_attn_bwd_staged(const void* q, const void* k, const void* v, const void* o, const void* dout,
                                 const float* lse, const float* logf, void* dq, void* dk, void* dv, float* dlogf,
                                 void* workspace, size_t workspace_bytes, int64_t b, int64_t h, int64_t n, int64_t d,
                                 float scale, fox_dtype_t dtype, fox_layout_t layout, hipStream_t stream);

/*
 * fox_attn_decode_workspace_bytes -- bytes of scratch fox_attn_decode needs for
 * these sizes (split-K partial results).  Returns 0 for invalid sizes.
 */
size_t fox_attn_decode_workspace_bytes(int64_t s, int64_t h, int64_t l, int64_t d);

/*
 * fox_attn_decode -- one causal FoX decode step per (sequence, head) against a KV cache.
 *   The last query row of fox_attn_fwd's definition.  The pages define no
 *   decode; the cache semantics are this library's: the caller has already
 *   written the new token's k and v at slot l-1, and slots 0..l-2 of c_cache
 *   hold the prefix sums c_0..c_{l-2} (e.g. from fox_attn_fwd's `c`).
 *
 *   q        : [s, h, d] of `dtype`, the new tokens' queries.
 *   k_cache  : [s, h, l, d] of `dtype`; v_cache likewise.
 *   c_cache  : [s, h, l] fp32; slots 0..l-2 read, slot l-1 WRITTEN with
 *              c_{l-1} = c_{l-2} + logf_new (logf_new when l == 1).
 *   logf_new : [s, h] fp32, the new tokens' log forget gates.
 *   o        : [s, h, d] of `dtype`, output.
 *   lse      : [s, h] fp32, output (natural log), or NULL.
 *   workspace, workspace_bytes : device scratch of at least
 *              fox_attn_decode_workspace_bytes(s, h, l, d) bytes, 16-byte aligned;
 *              contents on entry are ignored.
 *   scale    : multiplier of q.k (finite, > 0).
 */
fox_status_t fox_attn_decode(const void* q, const void* k_cache, const void* v_cache, float* c_cache,
                             const float* logf_new, void* o, float* lse, void* workspace, size_t workspace_bytes,
                             int64_t s, int64_t h, int64_t l, int64_t d, float scale, fox_dtype_t dtype,
                             hipStream_t stream);

/* Bytes of the fixed device scratch behind fox_attn_decode_noalloc (per device, held until the
 * process ends): fox_attn_decode_workspace_bytes(s, h, l, d) must not exceed it, which admits
 * up to about 32 000 (sequence, head) pairs at d = 128 (a record of d + 2 floats per pair and
 * split; at least 8192 records in all when the cache is long). */
#define FOX_DECODE_SCRATCH_BYTES (16u << 20)

/*
 * fox_attn_decode_noalloc -- fox_attn_decode without a workspace argument, for callers that
 *   cannot allocate device memory: code under HIP graph capture, tight serving loops, harnesses
 *   that forbid allocation.  The split records go to a fixed device array inside the library
 *   (FOX_DECODE_SCRATCH_BYTES per device, reserved when the library's code is loaded on the
 *   device); the call itself allocates, frees and clears nothing.  The kernels and the results
 *   are those of fox_attn_decode, bit for bit.
 *
 *   Arguments, layouts, outputs and errors as fox_attn_decode, without workspace and
 *   workspace_bytes, plus FOX_ERR_SCRATCH when fox_attn_decode_workspace_bytes(s, h, l, d)
 *   exceeds FOX_DECODE_SCRATCH_BYTES (nothing is launched).  `stream` must belong to the current
 *   device.  Every call on one device uses that device's one array: calls that may overlap on a
 *   device (other streams, other threads) race on it and must be serialised by the caller.
 */
fox_status_t fox_attn_decode_noalloc(const void* q, const void* k_cache, const void* v_cache, float* c_cache,
                                     const float* logf_new, void* o, float* lse, int64_t s, int64_t h, int64_t l,
                                     int64_t d, float scale, fox_dtype_t dtype, hipStream_t stream);

/*
 * fox_attn_decode_ragged -- fox_attn_decode for a batch of sequences of different lengths.
 *   Same step and cache convention per sequence, with sequence s using only the first
 *   cache_lens[s] slots of caches allocated for l slots: its new token's k, v sit at slot
 *   cache_lens[s]-1 and that slot of c_cache is written.  Slots past cache_lens[s] are
 *   neither read nor written.
 *
 *   cache_lens : [s] int32 DEVICE array, 4-byte aligned, values in [1, l] (read by the
 *                kernels; values outside are clamped to [1, l], never used to address
 *                memory outside the caches).
 *   l          : the caches' slot capacity (the third dimension of k_cache / v_cache / c_cache).
 *   Every other argument, the workspace size (fox_attn_decode_workspace_bytes(s, h, l, d))
 *   and the errors as fox_attn_decode.
 */
fox_status_t fox_attn_decode_ragged(const void* q, const void* k_cache, const void* v_cache, float* c_cache,
                                    const float* logf_new, const int32_t* cache_lens, void* o, float* lse,
                                    void* workspace, size_t workspace_bytes, int64_t s, int64_t h, int64_t l,
                                    int64_t d, float scale, fox_dtype_t dtype, hipStream_t stream);

/*
 * fox_attn_decode_paged -- fox_attn_decode_ragged with the caches held in fixed-size pages.
 *   The pages define no cache; this is the ragged step with each sequence's slots reached
 *   through a page table, the layout that lets serving engines grow caches without copying.
 *   Logical slot j of sequence s (j < cache_lens[s]) lives at row j % page_size of physical
 *   page block_table[s * max_pages + j / page_size]; the new token's k, v sit at slot
 *   cache_lens[s]-1 and that slot of c_pages is written.
 *
 *   q        : [s, h, d] of `dtype`, the new tokens' queries.
 *   k_pages, v_pages : [num_pages, h, page_size, d] of `dtype`: page p holds page_size
 *              consecutive slots of every head.
 *   c_pages  : [num_pages, h, page_size] fp32, the prefix sums at the same positions; slots
 *              0 .. cache_lens[s]-2 read, slot cache_lens[s]-1 WRITTEN (as fox_attn_decode).
 *   block_table : [s, max_pages] int32 DEVICE array; entries in [0, num_pages) (clamped on
 *              the device, so a bad entry never addresses memory outside the pools).
 *   cache_lens  : [s] int32 DEVICE array; values in [1, max_pages * page_size] (clamped).
 *   logf_new, o, lse, scale, dtype : as fox_attn_decode.
 *   page_size : a power of two in [16, 4096]; max_pages * page_size <= FOX_MAX_SEQ.
 *   workspace, workspace_bytes : at least
 *              fox_attn_decode_workspace_bytes(s, h, max_pages * page_size, d) bytes.
 *   Pages may be shared between sequences for reading; two sequences whose new tokens map to
 *   the same page slot race on its c write.  Errors as fox_attn_decode_ragged.
 */
fox_status_t fox_attn_decode_paged(const void* q, const void* k_pages, const void* v_pages, float* c_pages,
                                   const int32_t* block_table, const int32_t* cache_lens, const float* logf_new,
                                   void* o, float* lse, void* workspace, size_t workspace_bytes, int64_t s,
                                   int64_t h, int64_t num_pages, int64_t page_size, int64_t max_pages, int64_t d,
                                   float scale, fox_dtype_t dtype, hipStream_t stream);

/* Static English text for a status code (never NULL). */
const char* fox_status_string(fox_status_t status);

#ifdef __cplusplus
}
#endif

#endif /* FOX_H_ */
