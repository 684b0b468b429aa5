/*
 * gdla.h - C ABI of the MI355X (gfx950) GDLA forward-pass library, libgdla.so.
 *
 * GDLA (Grouped Differential Latent Attention) is the attention layer of
 * "Motif 3: Technical Report".  Per token x_t of one layer:
 *   - query: low-rank down-projection c_Q = x W_DQ^T, RMSNorm -> c_Qn, and
 *     up-projection q = c_Qn W_UQ^T into H = nS + nN heads of d_nope + d_rope
 *     dims (report, GDLA definition paragraph);
 *   - KV: one joint down-projection [c_KV | k_R] = x W_DKV^T giving the
 *     compressed latent and a decoupled rotary key; RMSNorm of the latent and
 *     a single up-projection [K^C | V] = c_KVn W_UKV^T into nN content-key and
 *     value heads shared by both query paths (report, GDLA summary and
 *     definition paragraphs);
 *   - RoPE on the rotary parts only (rotate-half form; "Open-Source Frontier
 *     Models: Architecture and Benchmarks of Rnj-1 and Motif-2", section 2
 *     and its implementation section);
 *   - causal or sliding-window softmax attention for nS = g * nN signal heads
 *     and nN noise heads (Rnj-1/Motif-2 page, section 1; report, definition
 *     paragraph);
 *   - D_t = H_S,t - lambda_t * Repeat_g(H_N,t), lambda_t = sigmoid(x_t W_l^T),
 *     then an element-wise sigmoid gate from c_Qn and the output projection
 *     y = (gate * D) W_O^T (report, definition paragraph).
 *
 * Conventions (readings where the report is silent):
 *   - every weight is [out, in] row-major (y = x W^T);
 *   - W_UQ rows: head h occupies rows h*(d_nope+d_rope) .. +d_nope+d_rope-1,
 *     content part first, rotary part last; heads 0..nS-1 are signal heads,
 *     nS..nS+nN-1 noise heads;
 *   - W_UKV rows: all nN content-key heads (nN*d_nope rows) then all nN value
 *     heads (nN*d_v rows);
 *   - W_DKV rows: the kv_rank latent rows, then the d_rope rotary-key rows;
 *   - signal head j and noise head j/g both attend with KV head j/g; signal
 *     head j subtracts noise head j/g;
 *   - RoPE angle for pair (i, i + d_rope/2) at position p is
 *     p * rope_base^(-2i/d_rope); positions are pos_offset + t, 0-based;
 *   - softmax scale 1/sqrt(d_nope + d_rope); window W > 0 lets position t
 *     attend keys s with t - W < s <= t; W <= 0 is full causal;
 *   - RMSNorm: c / sqrt(mean(c^2) + rms_eps) * gain.
 *
 * Ownership and threading: every buffer is device memory owned by the
 * caller.  The library allocates no device memory for data and never
 * synchronizes: all work is enqueued on `stream` (a hipStream_t; NULL = the
 * default stream) and inputs must stay valid until the stream reaches it.
 * Calls that share output or workspace buffers must be ordered on one stream.
 * Its state is a thread-local error string and, for the plain GEMMs it runs
 * on hipBLASLt (the bf16 prefill's output projection, residual as its C term,
 * and the backward's gradient GEMMs), a hipBLASLt handle per thread and device
 * and the algorithm chosen per shape, created on that thread's first such
 * call (which also loads hipBLASLt's kernels; make it outside any stream
 * capture) and kept until the process ends.  Decode does not use hipBLASLt.
 *
 * Environment (testing): GDLA_NO_HIPBLASLT=1 runs those GEMMs on the
 * library's own GEMM instead (also the fallback when hipBLASLt offers no
 * algorithm for a shape).  GDLA_ATTN_SUM_LIMIT sets the bound on a query's
 * running softmax row sum past which the bf16 prefill attention takes the
 * tile's max and rescales (default 2^32, clamped to [1, 2^32]; read at every
 * launch).  A small bound sends every key tile through the rescale path;
 * results agree to rounding for any value.
 *
 * Errors: every argument is checked on the host before anything is enqueued;
 * a call that returns non-OK has launched nothing.  GDLA_ERR_HIP means a
 * launch failed; gdla_last_error() has the detail.  Faults that happen
 * asynchronously in a kernel surface at the caller's next synchronization.
 */
#ifndef GDLA_H
#define GDLA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  GDLA_OK = 0,
  GDLA_ERR_INVALID_ARG = 1,   /* null required pointer, bad size, misaligned pointer */
  GDLA_ERR_UNSUPPORTED = 2,   /* shape / dtype combination no kernel covers */
  GDLA_ERR_WORKSPACE = 3,     /* workspace missing or smaller than *_workspace_size */
  GDLA_ERR_HIP = 4            /* a HIP launch or runtime call failed */
} gdla_status;

typedef enum {
  GDLA_BF16 = 0,   /* bf16 storage, fp32 accumulation (MFMA path) */
  GDLA_FP32 = 1    /* fp32 storage and arithmetic (vector-ALU path) */
} gdla_dtype;

/* Where YaRN's temperature m = 1 + 0.1 ln s is applied (see gdla_config). */
typedef enum {
  GDLA_YARN_TEMP_ROTARY = 0,   /* cos and sin times m: the rotary term of each logit scales by m^2 */
  GDLA_YARN_TEMP_LOGIT = 1     /* the whole logit times m^2; cos and sin unscaled */
} gdla_yarn_temperature;

typedef struct {
  int32_t d_model;   /* token width */
  int32_t q_rank;    /* query latent width */
  int32_t kv_rank;   /* KV latent width */
  int32_t n_noise;   /* nN: noise heads = expanded KV heads */
  int32_t group;     /* g: signal heads per noise head; nS = g * nN */
  int32_t d_nope;    /* content part of a query/key head */
  int32_t d_rope;    /* rotary part of a query/key head (even) */
  int32_t d_v;       /* value head width */
  int32_t window;    /* <= 0: full causal; else keys t-window < s <= t */
  float rope_base;   /* RoPE base, e.g. 10000 */
  float rms_eps;     /* RMSNorm epsilon, e.g. 1e-6 */
  gdla_dtype dtype;  /* one dtype for x, y, weights, gains and cache */
  /* YaRN extension of the rotary frequencies ("Open-Source Frontier Models:
   * Architecture and Benchmarks of Rnj-1 and Motif-2", YaRN section and its
   * listing; the Motif 3 report's long-context paragraph uses it, factor 64
   * over a native 4K, on its full-attention layers).  Applied when
   * yarn_factor > 1 and window <= 0 (full-causal layers only); zero-filled
   * fields mean plain RoPE.  Pair i of wavelength l_i = 2 pi / theta_i keeps
   * theta_i below yarn_orig_len / yarn_beta_fast, becomes theta_i / s above
   * yarn_orig_len / yarn_beta_slow and is interpolated linearly in l_i in
   * between.  The temperature m = 1 + 0.1 ln s goes where yarn_temperature
   * says: GDLA_YARN_TEMP_ROTARY (0, the listing) multiplies cos and sin by
   * m, so only the rotary part of every logit scales, by m^2 (the content
   * part of a GDLA head carries no rotation); GDLA_YARN_TEMP_LOGIT (1, the
   * page's prose, which puts the temperature on the softmax logits, and the
   * DeepSeek form of YaRN the report names) multiplies the whole logit by
   * m^2 and leaves cos and sin unscaled.  Invalid when yarn_factor > 1 unless
   * yarn_orig_len > 0 and yarn_beta_fast > yarn_beta_slow > 0, or when
   * yarn_temperature is neither value. */
  float yarn_factor;       /* s */
  int32_t yarn_orig_len;   /* native context length */
  float yarn_beta_fast;
  float yarn_beta_slow;
  int32_t yarn_temperature;   /* gdla_yarn_temperature */
} gdla_config;

typedef struct {          /* device pointers, all [out, in] row-major, dtype of the config */
  const void* w_dq;       /* [q_rank, d_model] */
  const void* g_q;        /* [q_rank]            RMSNorm gain of the query latent */
  const void* w_dkv;      /* [kv_rank + d_rope, d_model] */
  const void* g_kv;       /* [kv_rank]           RMSNorm gain of the KV latent */
  const void* w_lambda;   /* [nS, d_model] */
  const void* w_uq;       /* [(nS + nN) * (d_nope + d_rope), q_rank] */
  const void* w_ukv;      /* [nN * d_nope + nN * d_v, kv_rank] */
  const void* w_gate;     /* [nS * d_v, q_rank] */
  const void* w_o;        /* [d_model, nS * d_v] */
} gdla_weights;

/* Support limits of the bf16 path (the fp32 path takes any positive sizes with
 * d_rope even, d_nope + d_rope <= 256, d_v <= 256, and L <= 8192):
 *   d_nope = 128, d_rope = 64, d_v = 128, group + 1 <= 8,
 *   d_model, q_rank, kv_rank and nS * d_v multiples of 64.
 * Prefill (gdla_prefill, gdla_prefill_packed) stores the score operands --
 * queries, content keys, rotary keys -- as fp16: 11-bit significands cut
 * the score rounding error 8x against bf16, but every query and key element
 * must stay below 65504 in magnitude (beyond it the element becomes +-inf
 * and the output of that row NaN).  The cache rows, values and Z stay bf16;
 * decode and the training forward keep bf16 queries and keys.        */

/* Bytes of workspace gdla_prefill needs for B sequences of L tokens
 * (0 if the configuration is invalid). */
size_t gdla_prefill_workspace_size(const gdla_config* cfg, int32_t B, int32_t L);

/* One GDLA layer over B sequences of L tokens (report, GDLA definition
 * paragraph; hybrid schedules call it once per layer with that layer's window).
 *   x          [B, L, d_model]  input tokens
 *   y          [B, L, d_model]  output; y = residual + (gate * D) W_O^T when
 *                               residual != NULL, else (gate * D) W_O^T.
 *                               y may alias residual but not x otherwise.
 *   residual   nullable [B, L, d_model]
 *   pos_offset position of token 0 of every sequence (>= 0)
 *   cache      nullable [B, cache_capacity, kv_rank + d_rope]: rows
 *              pos_offset .. pos_offset + L - 1 of each sequence receive
 *              [c_KVn | RoPE(k_R)], the layout gdla_decode reads
 *   cache_capacity  rows per sequence in cache (>= pos_offset + L when cache
 *              is given)
 *   workspace  device buffer of at least gdla_prefill_workspace_size bytes,
 *              256-byte aligned; its contents on return are the
 *              intermediates listed by gdla_prefill_workspace_layout.
 * All pointers 16-byte aligned. */
gdla_status gdla_prefill(const gdla_config* cfg, const gdla_weights* w, int32_t B, int32_t L,
                         int64_t pos_offset, const void* x, void* y, const void* residual,
                         void* cache, int32_t cache_capacity, void* workspace,
                         size_t workspace_bytes, void* stream);

/* Stages of one prefill layer, in launch order.  gdla_prefill runs them all;
 * gdla_prefill_stages runs a subset on the same workspace (for per-stage
 * timing and profiling: later stages read what earlier calls left there). */
enum {
  GDLA_STAGE_DOWN = 1,     /* fused down-projection x -> [c_Q | c_KV | k_R | lambda logit] */
  GDLA_STAGE_PREP = 2,     /* RMSNorms, rotary key, lambda, RoPE table, cache rows */
  GDLA_STAGE_EXPAND = 4,   /* latent expansion into content keys and values */
  GDLA_STAGE_QG = 8,       /* query up-projection (RoPE) and sigmoid gate */
  GDLA_STAGE_ATTN = 16,    /* signal + noise attention, differential, gate -> Z */
  GDLA_STAGE_OUT = 32,     /* output projection (+ residual) -> y */
  GDLA_STAGE_ALL = 63
};

/* gdla_prefill restricted to the stages in the `stages` mask (same arguments,
 * same checks).  A stage reads the workspace contents earlier stages of a
 * call with the same cfg, B and L left there; running a stage whose inputs
 * were never produced computes on undefined data (but stays in bounds). */
gdla_status gdla_prefill_stages(const gdla_config* cfg, const gdla_weights* w, int32_t B, int32_t L,
                                int64_t pos_offset, const void* x, void* y, const void* residual,
                                void* cache, int32_t cache_capacity, void* workspace,
                                size_t workspace_bytes, void* stream, uint32_t stages);

/* Byte offsets of the intermediates inside the prefill workspace after a call
 * (for inspection and tests).  T = B*L tokens; elements are in the config
 * dtype unless marked fp32 -- except that in the bf16 configuration the
 * score operands q, kc and kr are fp16 (11-bit significands: the scores
 * carry an eighth of the bf16 rounding error; values must stay below 65504
 * in magnitude).
 *   down   [T, q_rank + kv_rank + d_rope + nS] fp32: c_Q | c_KV | k_R | lambda logit
 *   cqn    [T, q_rank]            normalized query latent
 *   ckvn   bf16: [T, 2*kv_rank]   normalized KV latent as hi | lo, where
 *                                 hi = bf16(c_KVn) and lo = bf16(c_KVn - hi);
 *          fp32: [T, kv_rank]
 *   kr     [T, d_rope]            RoPE'd rotary key (fp16 in the bf16 configuration)
 *   lam    [T, nS] fp32           lambda
 *   rope   [T, d_rope/2, 2] fp32  cos, sin of each position's RoPE angles
 *   q      [T, H*(d_nope+d_rope)] query heads, rotary parts RoPE'd (fp16 in the bf16 configuration)
 *   gate   [T, nS*d_v] fp32       sigmoid gate
 *   kc     [T, nN*d_nope]         content keys (fp16 in the bf16 configuration)
 *   vt     [nN*d_v, Tp]           values transposed: token t in column t;
 *                                 Tp = T rounded up to 64, columns T.. zero
 *   z      [T, nS*d_v]            gate * D                                     */
typedef struct {
  int64_t down, cqn, ckvn, kr, lam, rope, q, gate, kc, vt, z;
} gdla_prefill_layout;
gdla_status gdla_prefill_workspace_layout(const gdla_config* cfg, int32_t B, int32_t L,
                                          gdla_prefill_layout* out);

/* Bytes of workspace gdla_decode needs for B sequences (0 if invalid). */
size_t gdla_decode_workspace_size(const gdla_config* cfg, int32_t B);

/* One decode step: one new token per sequence attends its cached context
 * through the compressed latent (report, GDLA summary paragraph: only the
 * normalized latent and the rotary key are kept per position).
 *   x           [B, d_model]  the new tokens
 *   y           [B, d_model]  output (gate * D) W_O^T
 *   cache       [B, capacity, kv_rank + d_rope]; rows 0 .. cache_lens[b]-1 are
 *               read, row cache_lens[b] is written with the new token's
 *               [c_KVn | RoPE(k_R)] before it is attended
 *   cache_lens  device int32 [B]: tokens already cached per sequence; the new
 *               token's position.  Read on the device (never on the host); it
 *               must be in [0, capacity - 1].  The caller advances it.
 * bf16 only, kv_rank in {128, 256, 512}, at most 80 query heads
 * (n_noise * (group + 1)); otherwise GDLA_ERR_UNSUPPORTED.  All pointers
 * 16-byte aligned. */
gdla_status gdla_decode(const gdla_config* cfg, const gdla_weights* w, int32_t B,
                        const void* x, void* y, void* cache, const int32_t* cache_lens,
                        int32_t capacity, void* workspace, size_t workspace_bytes,
                        void* stream);

/* gdla_decode for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  The
 * same step with the same results as gdla_decode (same checks, limits and
 * kernels), but its workspace is a library-owned device array of
 * GDLA_DECODE_NOALLOC_SCRATCH_BYTES per GPU instead of a caller buffer; the
 * caller still passes x, y, the cache and cache_lens.  The array is set aside
 * by the loader the first time a process uses this entry point on a device
 * and held until the process ends.
 *   - GDLA_ERR_WORKSPACE (nothing launched) when gdla_decode_workspace_size
 *     of cfg and B exceeds the array: B <= 64 fits at 80 query heads and a
 *     512-wide latent, about B <= 100 at 64 heads.
 *   - stream must belong to the current device (GDLA_ERR_INVALID_ARG
 *     otherwise); NULL is the current device's default stream.
 *   - Every call on one GPU shares that GPU's array, and nothing in it
 *     survives between calls that the step needs: calls whose work overlaps
 *     in time on one GPU (different streams, or unordered host threads) race
 *     on it and give undefined results; order them on one stream.
 * The library allocates nothing on this path (no hipMalloc, hipFree or
 * allocating library call). */
#define GDLA_DECODE_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)
gdla_status gdla_decode_noalloc(const gdla_config* cfg, const gdla_weights* w, int32_t B,
                                const void* x, void* y, void* cache, const int32_t* cache_lens,
                                int32_t capacity, void* stream);

/* A paged latent cache ("Open-Source Frontier Models: Architecture and
 * Benchmarks of Rnj-1 and Motif-2", section 2, prefill sequence diagram: the
 * normalized KV rows are stored in the blocks of a PagedAttention cache).
 * The positions of sequence b are cut into blocks of page_rows; block j lives
 * in pool page block_table[b * max_pages + j], so position p is row
 * p % page_rows of page block_table[b * max_pages + p / page_rows].
 *   pages        device [num_pages, page_rows, kv_rank + d_rope], config
 *                dtype, 16-byte aligned; rows hold [c_KVn | RoPE(k_R)]
 *   block_table  device int32 [sequences, max_pages], 4-byte aligned; read
 *                on the device only
 *   page_rows    rows per page: a power of two, at least 32
 *   max_pages    block-table columns (> 0); positions run up to
 *                page_rows * max_pages - 1 (that product at most 2^30)
 *   num_pages    pages in the pool (> 0)
 * Table entries are not trusted: a position whose entry lies outside
 * [0, num_pages), or beyond the table, is neither written nor read (decode
 * leaves such rows out of the attention).  Pages may sit anywhere in the
 * pool and in any order; calls that write one row from two places race. */
typedef struct {
  void* pages;
  const int32_t* block_table;
  int32_t page_rows;
  int32_t max_pages;
  int32_t num_pages;
} gdla_paged_cache;

/* Bytes of workspace gdla_prefill_packed needs for n_seq sequences holding T
 * tokens in all (0 if the configuration or the sizes are not supported). */
size_t gdla_prefill_packed_workspace_size(const gdla_config* cfg, int32_t n_seq, int64_t T);

/* One GDLA layer over n_seq complete sequences packed end to end into one
 * stream of T tokens (report, long-context training paragraph: whole
 * sequences packed together).  Each sequence is the layer applied to it alone: its
 * tokens attend only to earlier tokens of the same sequence, at positions
 * that restart at pos_offsets[b].
 *   cu_seqlens   device int32 [n_seq + 1], read on the device only: sequence b
 *                holds stream rows cu_seqlens[b] .. cu_seqlens[b+1] - 1.  It
 *                must be nondecreasing from cu_seqlens[0] = 0 to
 *                cu_seqlens[n_seq] = T (empty sequences allowed).  Other
 *                values cause no access outside the buffers, but rows that
 *                no sequence holds get unspecified outputs.
 *   pos_offsets  nullable device int32 [n_seq]: position of each sequence's
 *                first token (>= 0; NULL means 0 for all)
 *   x, y, residual  [T, d_model], as in gdla_prefill
 *   cache        nullable: every token's row [c_KVn | RoPE(k_R)] goes to its
 *                position in the paged cache, sequence b through row b of
 *                the block table (the layout gdla_decode_paged reads)
 *   workspace    at least gdla_prefill_packed_workspace_size bytes, 256-byte
 *                aligned
 * The attention runs one work item per (sequence, query block), ordered by
 * cost, heaviest first (the report's longest-processing-time rule, applied to
 * the workgroups of one GPU).  Limits: n_seq >= 0, T >= 0 (T = 0 is a no-op),
 * T <= 2^20 and n_seq <= 2^20 (bf16), T <= 8192 (fp32).  All pointers 16-byte
 * aligned except cu_seqlens and pos_offsets (4-byte). */
gdla_status gdla_prefill_packed(const gdla_config* cfg, const gdla_weights* w, int32_t n_seq, int64_t T,
                                const int32_t* cu_seqlens, const int32_t* pos_offsets, const void* x,
                                void* y, const void* residual, const gdla_paged_cache* cache,
                                void* workspace, size_t workspace_bytes, void* stream);

/* gdla_decode against a paged cache (same workspace size and limits): the new
 * token of sequence b is written at position cache_lens[b] through row b of
 * the block table, then attends positions 0 .. cache_lens[b] (the window's
 * part of them) read through the same row.  cache_lens[b] must be below
 * page_rows * max_pages; a sequence outside that gets y = 0 and writes
 * nothing, as in gdla_decode.  B * max_pages at most 2^28
 * (GDLA_ERR_UNSUPPORTED beyond). */
gdla_status gdla_decode_paged(const gdla_config* cfg, const gdla_weights* w, int32_t B, const void* x,
                              void* y, const gdla_paged_cache* cache, const int32_t* cache_lens,
                              void* workspace, size_t workspace_bytes, void* stream);

/* Weight gradients of one layer: fp32 device buffers with the shapes of the
 * matching gdla_weights fields (gains [q_rank] and [kv_rank]), overwritten. */
typedef struct {
  float* w_dq; float* g_q; float* w_dkv; float* g_kv; float* w_lambda;
  float* w_uq; float* w_ukv; float* w_gate; float* w_o;
} gdla_grads;

/* Bytes of workspace gdla_backward needs for B sequences of L tokens (0 if
 * the configuration or sizes are not supported). */
size_t gdla_backward_workspace_size(const gdla_config* cfg, int32_t B, int32_t L);

/* Backward of one GDLA layer (gdla_prefill's layer, without residual): given
 * its input x and the gradient dy of its output, the gradient dx and every
 * weight gradient.  The forward's activations are recomputed from x inside
 * the call (report, training-infrastructure paragraph: activations are
 * recomputed for the backward pass), so the caller keeps only x.
 *   x, dy      [B, L, d_model], config dtype
 *   dx         [B, L, d_model] out, config dtype; must not alias x or dy
 *   grads      every pointer non-NULL, fp32, overwritten (not accumulated)
 *   workspace  at least gdla_backward_workspace_size bytes, 256-byte aligned
 * bf16 only (GDLA_ERR_UNSUPPORTED otherwise); the bf16 shape limits of
 * gdla_prefill, q_rank + kv_rank <= 2048, B*L <= 2^22 and positions below
 * 2^30.  All pointers 16-byte aligned. */
gdla_status gdla_backward(const gdla_config* cfg, const gdla_weights* w, int32_t B, int32_t L,
                          int64_t pos_offset, const void* x, const void* dy, void* dx,
                          const gdla_grads* grads, void* workspace, size_t workspace_bytes,
                          void* stream);

/* Bytes of workspace gdla_backward_packed needs for n_seq sequences holding
 * T tokens (0 if unsupported, or if n_seq = 0). */
size_t gdla_backward_packed_workspace_size(const gdla_config* cfg, int32_t n_seq, int64_t T);

/* gdla_backward over a packed stream: gdla_prefill_packed's layer (report,
 * long-context training paragraph: complete sequences packed together;
 * training-infrastructure paragraph: activations recomputed for the backward
 * pass).  Each sequence is differentiated as the layer applied to it alone:
 * its rows of dx are its own, and every weight gradient is the sum over the
 * sequences.
 *   cu_seqlens, pos_offsets  as in gdla_prefill_packed (device int32, read on
 *                the device only; other values cause no access outside the
 *                buffers, but rows no sequence holds get unspecified dx and
 *                the weight gradients then include their contributions)
 *   x, dy        [T, d_model], config dtype
 *   dx           [T, d_model] out; must not alias x or dy
 *   grads        as in gdla_backward (overwritten)
 *   workspace    at least gdla_backward_packed_workspace_size bytes, 256-byte
 *                aligned
 * The attention backward runs one work item per (sequence, block of 32
 * queries) for dQ and per (sequence, block of 128 keys) for dK and dV.
 * Limits: bf16 only, the shape limits of gdla_backward, T <= 2^22 (T = 0 is
 * a no-op), n_seq <= 2^20.  All pointers 16-byte aligned except cu_seqlens
 * and pos_offsets (4-byte). */
gdla_status gdla_backward_packed(const gdla_config* cfg, const gdla_weights* w, int32_t n_seq, int64_t T,
                                 const int32_t* cu_seqlens, const int32_t* pos_offsets, const void* x,
                                 const void* dy, void* dx, const gdla_grads* grads, void* workspace,
                                 size_t workspace_bytes, void* stream);

/* Latent expansion alone (report, GDLA summary and definition paragraphs):
 * c_KVn = RMSNorm(c_KV) * g_kv, [K^C | V] = c_KVn W_UKV^T.
 *   c_kv    [T, ld_c] raw latent (first kv_rank columns used), ld_c >= kv_rank
 *   g_kv    [kv_rank] gain;  w_ukv  [nN*d_nope + nN*d_v, kv_rank]
 *   k_nope  [T, nN, d_nope] out
 *   v       [T, nN, d_v]    out
 *   c_norm  [T, kv_rank]    out: c_KVn rounded to the dtype (the GEMM's input)
 * Row-major, dtype of the config, 16-byte aligned; T >= 0 (T = 0 is a no-op).
 * Unlike gdla_prefill (which feeds the expansion the latent split into bf16
 * hi and lo parts), this standalone call expands the rounded c_norm. */
gdla_status gdla_latent_expand(const gdla_config* cfg, int64_t T, const void* c_kv, int64_t ld_c,
                               const void* g_kv, const void* w_ukv, void* k_nope, void* v,
                               void* c_norm, void* stream);

const char* gdla_status_string(gdla_status s);

/* Detail of the last non-OK status returned on the calling thread ("" if none). */
const char* gdla_last_error(void);

/* Library version, major * 10000 + minor * 100 + patch. */
int32_t gdla_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GDLA_H */
