/*
 * ctxattn.h -- C ABI of the MI355X (gfx950) context-parallel attention core.
 *
 * One rank's share of context-parallel attention: a resident query shard attends
 * a sequence of K/V chunks as a ring delivers them, each step emitting a partial
 * output plus per-row log-sum-exp (LSE), and partials are combined by the
 * LSE-corrected merge. The same merge combines DCP decode shards.
 *
 * Sources (pages as published):
 *  - "Kernel reference: ring_attention_const_max_fwd const-max ring attention"
 *    (AWS Neuron docs): Overview (ring schedule), Design (bound, pure-addition
 *    fold), Implementation (norms, global key max, accumulate then normalise,
 *    1e-37 clamp), Interface (q/k/v token-major [b, seqlen, h, d], o [b, h, seqlen, d],
 *    softmax_scale default 1/sqrt(d), lse = c + log(sum_exp)).
 *  - "DCP (Decode Context Parallelism)" (AWS Neuron docs): DCP Decode compute
 *    pattern (local attention, partial LSE, weight = exp(local_lse - global_lse)),
 *    local_filled computation, slot mapping (position -> (pos // I) % W).
 *  - "Sharding the Input" (iop.systems): ring attention, striped attention.
 *
 * Conventions for every entry point:
 *  - All tensor arguments are DEVICE pointers owned by the caller; the library
 *    never allocates, frees or retains them, and keeps no state between calls.
 *  - Calls are asynchronous on `stream` (a hipStream_t; NULL = default stream).
 *    Only argument validation and the launch are synchronous; kernel faults
 *    surface at the caller's next synchronisation.
 *  - Return CA_OK or an error status. On error nothing is launched, and
 *    ca_last_error() returns a message for the calling thread.
 *  - Unsupported shapes or types return CA_ERR_UNSUPPORTED; there is no silent
 *    fallback to another path (the kernel reference page, Best practices: the
 *    only correct path gets no selector, violations fail loudly).
 *  - softmax_scale <= 0 selects 1/sqrt(D).
 *  - LSE values are natural logarithms; a row that sees no key has
 *    lse = -inf and output 0.
 *  - A [B, S, H, D] input is described by element strides (b, s, h); the D axis
 *    must be contiguous and every row 16-byte aligned.
 */
#ifndef CTXATTN_H
#define CTXATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  CA_OK = 0,
  CA_ERR_NULL = 1,         /* a required pointer is NULL */
  CA_ERR_SHAPE = 2,        /* sizes or strides are inconsistent */
  CA_ERR_DTYPE = 3,        /* unknown dtype code */
  CA_ERR_UNSUPPORTED = 4,  /* valid request this library does not implement */
  CA_ERR_WORKSPACE = 5,    /* workspace missing or too small */
  CA_ERR_HIP = 6           /* the HIP runtime reported an error */
} ca_status;

typedef enum { CA_BF16 = 0, CA_FP32 = 1 } ca_dtype;

/* Key visibility inside one step, on LOCAL indices i (query) and j (key). Under a
 * striped ring (token t on rank t mod cp, local index t div cp), global causality
 * reduces per step to INCL when the chunk's source rank <= the query rank, and to
 * STRICT otherwise. */
typedef enum {
  CA_MASK_NONE = 0,
  CA_MASK_CAUSAL_INCL = 1,   /* key j visible iff j <= i */
  CA_MASK_CAUSAL_STRICT = 2  /* key j visible iff j <  i */
} ca_mask;

/* Phase bits of the const-max step. */
enum { CA_PHASE_ACCUMULATE = 0, CA_PHASE_INIT = 1, CA_PHASE_FINAL = 2 };

/* Element strides of a [B, S, H, D] tensor (D stride is 1). */
typedef struct {
  int64_t b;
  int64_t s;
  int64_t h;
} ca_strides;

/*
 * ring_attn_step -- online-max (flash-style) attention of the resident query shard
 * against ONE K/V chunk, emitting the chunk's partial output and per-row LSE.
 * Source: kernel reference page, Design "Dropping the online max buys a better
 * layout" (the online-max path keeps a running row max, row sum and a rescaled
 * accumulator); "Sharding the Input", ring attention (blockwise attention per
 * K/V block).
 *
 *   q      [B, Sq, H, D] bf16 or fp32 (dtype), strides q_strides
 *   k, v   [B, Sk, H, D] same dtype, strides kv_strides (shared by k and v)
 *   mask   ca_mask on local indices
 *   o      OUT [B, H, Sq, D] fp32, contiguous: softmax(s) @ v over visible keys
 *   lse    OUT [B, H, Sq] fp32, contiguous: log sum_j exp(scale * q_i . k_j)
 *   workspace, workspace_bytes
 *          optional device scratch (see ring_attn_workspace_size). NULL: one workgroup
 *          per 256 query rows (bf16). Given, and the call is one that one workgroup per
 *          256 rows would leave the device's workgroup slots more than a tenth idle: the call's
 *          (query tile, key tile) iterations are cut into ranges of equal cost (each query
 *          tile's start counts as a few iterations), about one per workgroup the device
 *          holds at once, and query tiles split between ranges are combined in
 *          the library, in key order (results do not depend on timing). The workspace must
 *          be 256-byte aligned and all zero before its first use; every call leaves it
 *          ready for the next. Calls that may run at the same time need separate
 *          workspaces. Ignored by the vector kernel (below) and by calls that do not split.
 * Supported: D in {64, 128} for both dtypes; MHA (same H for q and kv). bf16 with D == 128
 * runs on the MFMA kernel (the head size the kernel reference page's Interface asserts);
 * fp32, and bf16 with D == 64, run on a vector kernel with fp32 arithmetic (bf16 elements
 * widened as loaded), which never splits and runs about 20x slower (a 40-head 9450 x 9450
 * step on MI355X: about 55 TFLOP/s for bf16 D == 64, 35 for fp32 D == 128, against about
 * 1150 for bf16 D == 128 on the MFMA kernel). Sk == 0 is allowed (all rows empty). Errors: CA_ERR_NULL, CA_ERR_SHAPE,
 * CA_ERR_DTYPE, CA_ERR_UNSUPPORTED, CA_ERR_WORKSPACE (too small), CA_ERR_HIP.
 */
ca_status ring_attn_step(const void* q, ca_strides q_strides,
                         const void* k, const void* v, ca_strides kv_strides,
                         int dtype, int B, int H, int Sq, int Sk, int D,
                         float softmax_scale, int mask,
                         float* o, float* lse,
                         void* workspace, size_t workspace_bytes, void* stream);

/*
 * ring_attn_step_fold -- ring_attn_step whose partial is merged in place into a prior
 * one: the incremental form of the LSE merge of per-chunk partials. The rows of o and
 * lse hold a partial (O_p, lse_p) of the same queries on entry (e.g. an earlier chunk's
 * ring_attn_step output); on return they hold its merge with this chunk's (O_t, lse_t):
 * M = max(lse_p, lse_t), L = M + log(e^(lse_p - M) + e^(lse_t - M)),
 * O = e^(lse_p - L) O_p + e^(lse_t - L) O_t, lse = L; a row empty on both sides stays
 * O = 0, lse = -inf. Folding the chunks of a ring one after another gives the n-way
 * lse_merge of their partials up to rounding.
 * Source: "Sharding the Input" (ring attention: each block's result rescaled by the
 * running log-sum-exp and combined), and the DCP page's merge of partial outputs by
 * their LSE.
 *
 * Arguments, layouts, support and errors: as ring_attn_step, with o and lse IN/OUT
 * (contiguous fp32; lse_p may be -inf). A call reads each row of o and lse once and
 * writes it once; calls into the same o / lse must not overlap in time.
 */
ca_status ring_attn_step_fold(const void* q, ca_strides q_strides,
                              const void* k, const void* v, ca_strides kv_strides,
                              int dtype, int B, int H, int Sq, int Sk, int D,
                              float softmax_scale, int mask,
                              float* o, float* lse,
                              void* workspace, size_t workspace_bytes, void* stream);

/*
 * ring_attn_step_hop -- ring_attn_step and, in the same call, the ring's next K/V hop
 * (what kv_chunk_copy does): hop_bytes bytes copied from hop_src_k to hop_dst_k and
 * from hop_src_v to hop_dst_v. Where the step's last round of workgroups leaves CUs
 * free (a key-split step cut into fewer ranges than the device holds; the last, partly
 * filled round of an unsplit one), the copy runs in the same launch on those CUs, so
 * the hop overlaps the step without a stream of its own; otherwise it is an ordinary
 * copy launched just ahead of the step on the same stream. Either way both are done
 * when work queued after the call on the stream starts.
 * Source: kernel reference page, Implementation, the ring loop (the next chunk moves
 * while the current one is computed); "Sharding the Input", ring attention.
 *
 * Arguments, layouts, support and errors: as ring_attn_step, plus
 *   hop_dst_k, hop_dst_v  OUT device buffers of hop_bytes each
 *   hop_src_k, hop_src_v  IN device buffers of hop_bytes each
 *   hop_bytes             0: no hop (the call is ring_attn_step); else a multiple of 16,
 *                         with all four pointers 16-byte aligned (CA_ERR_SHAPE), non-NULL
 *                         (CA_ERR_NULL)
 * The destinations must not overlap the sources or any input, output or workspace of
 * the step (they are written while the step runs). Bytes move unchanged (bit copy).
 */
ca_status ring_attn_step_hop(const void* q, ca_strides q_strides,
                             const void* k, const void* v, ca_strides kv_strides,
                             int dtype, int B, int H, int Sq, int Sk, int D,
                             float softmax_scale, int mask,
                             float* o, float* lse,
                             void* workspace, size_t workspace_bytes,
                             void* hop_dst_k, void* hop_dst_v,
                             const void* hop_src_k, const void* hop_src_v, size_t hop_bytes,
                             void* stream);

/*
 * ring_attn_step_fold_hop -- ring_attn_step_fold and, in the same call, the ring's next
 * K/V hop, exactly as ring_attn_step_hop adds one to ring_attn_step (in the step's launch
 * on the CUs its last round leaves free, else as a copy just ahead of it). A ring whose
 * steps fold into running partials can so carry its hops in the steps as well.
 * Source: kernel reference page, Implementation, the ring loop; "Sharding the Input",
 * ring attention (running log-sum-exp combination).
 *
 * Arguments, layouts, support and errors: as ring_attn_step_fold, plus the hop arguments
 * of ring_attn_step_hop with the same requirements.
 */
ca_status ring_attn_step_fold_hop(const void* q, ca_strides q_strides,
                                  const void* k, const void* v, ca_strides kv_strides,
                                  int dtype, int B, int H, int Sq, int Sk, int D,
                                  float softmax_scale, int mask,
                                  float* o, float* lse,
                                  void* workspace, size_t workspace_bytes,
                                  void* hop_dst_k, void* hop_dst_v,
                                  const void* hop_src_k, const void* hop_src_v, size_t hop_bytes,
                                  void* stream);

/*
 * ring_attn_step_pair -- two consecutive ring steps in one launch, once both chunks have
 * arrived: attention of the resident query shard against the keys of chunk 1 and then of
 * chunk 2, which by the LSE merge ("Kernel reference: ring_attention_const_max_fwd", the
 * ring loop; the context-parallelism page, merging partial attention by LSE) equals the two
 * steps' partials merged. It halves the per-launch work that does not scale with the keys
 * (each query tile's Q load, copy prologue, epilogue and fold) where steps are short.
 *   q               as ring_attn_step
 *   k1, v1          [B, Sk1, H, D] the first chunk; Sk1 a multiple of 32
 *   k2, v2          [B, Sk2, H, D] the second chunk, with the first chunk's strides kv_strides
 *   fold            0: o and lse receive the two chunks' partial (as ring_attn_step);
 *                   1: they hold a prior partial and receive its merge (as ring_attn_step_fold)
 *   workspace       as ring_attn_step, sized for Sk1 + Sk2 keys
 *   hop_*, hop2_*   up to two ring hops carried by the same launch, each as ring_attn_step_hop
 *                   (hop2_src_k == NULL: one hop; hop_bytes 0: none); both hop_bytes long
 * No mask (the steps it pairs are non-causal). Supported: bf16, D == 128 (the MFMA kernel),
 * MHA. Sk1 == 0 or Sk2 == 0 runs the other chunk as ring_attn_step. Errors as
 * ring_attn_step_hop, and CA_ERR_UNSUPPORTED when Sk1 is not a multiple of 32.
 */
ca_status ring_attn_step_pair(const void* q, ca_strides q_strides,
                              const void* k1, const void* v1, const void* k2, const void* v2,
                              ca_strides kv_strides, int dtype, int B, int H, int Sq, int Sk1, int Sk2,
                              int D, float softmax_scale, int fold, float* o, float* lse,
                              void* workspace, size_t workspace_bytes,
                              void* hop_dst_k, void* hop_dst_v, const void* hop_src_k,
                              const void* hop_src_v, void* hop2_dst_k, void* hop2_dst_v,
                              const void* hop2_src_k, const void* hop2_src_v, size_t hop_bytes,
                              void* stream);

/*
 * ring_attn_workspace_size -- bytes of step workspace that ring_attn_step and
 * ring_attn_const_max_step (mask CA_MASK_NONE) need for these sizes on the CURRENT
 * device (the split depends on its compute-unit count). 0: the call does not split
 * (fp32, no key tiles, or enough query tiles to fill the device). The bytes are per-call
 * scratch: split partials (2 * workgroups * 256 rows * (D + 2) fp32) and one counter per
 * (query tile, wave).
 */
ca_status ring_attn_workspace_size(int dtype, int B, int H, int Sq, int Sk, int D, int mask,
                                   size_t* bytes);

/*
 * key_sqnorm_max -- per (b, h) maximum over the chunk's keys of |k_j|^2.
 * Source: kernel reference page, Implementation "Transpose prologue with fused
 * norms" (K folds per-token |k|^2 into a running max, one value per head) and
 * "Global key max" (all_reduce(max) across the ring). On one device the
 * all-reduce is the max-fold over chunks: accumulate = 0 overwrites kmax_sq with
 * this chunk's maxima, accumulate = 1 folds them into kmax_sq by max.
 *   k        [B, S, H, D], strides ks; D a multiple of 8 in [8, 128]; H <= 4096
 *   kmax_sq  IN/OUT [B, H] fp32
 * Errors: CA_ERR_NULL, CA_ERR_SHAPE, CA_ERR_DTYPE, CA_ERR_UNSUPPORTED (D, H), CA_ERR_HIP.
 */
ca_status key_sqnorm_max(const void* k, ca_strides ks, int dtype, int B, int S, int H, int D,
                         float* kmax_sq, int accumulate, void* stream);

/*
 * const_max_bound -- per query row bound c_i = scale * |q_i| * sqrt(kmax_sq[b, h]).
 * Source: kernel reference page, Design "Picking a max that is safe without
 * measuring it" (Cauchy-Schwarz: c_i >= every score of row i) and Implementation
 * "Assembling the bound" (one square root of scale^2 * kmax_sq * |q_i|^2).
 *   q        [B, Sq, H, D], strides qs; D a multiple of 8 in [8, 128]; H <= 256
 *   kmax_sq  [B, H] fp32 (from key_sqnorm_max over every chunk of the ring)
 *   c        OUT [B, H, Sq] fp32
 * Errors: CA_ERR_NULL, CA_ERR_SHAPE, CA_ERR_DTYPE, CA_ERR_UNSUPPORTED (D, H), CA_ERR_HIP.
 */
ca_status const_max_bound(const void* q, ca_strides qs, int dtype, int B, int Sq, int H, int D,
                          float softmax_scale, const float* kmax_sq, float* c, void* stream);

/*
 * ring_attn_const_max_step -- one ring step of const-max attention: p = exp(s - c_i)
 * with the fixed per-row bound, folded into a running unnormalised accumulator by
 * pure addition; the FINAL step normalises once.
 * Source: kernel reference page, Design "A static bound makes the ring reduction
 * pure addition", Implementation "Accumulate, then normalize once" (fp32
 * accumulator, row sum clamped to 1e-37 before the single division), Interface
 * (lse = c + log(sum_exp); non-causal, MHA).
 *
 *   q, k, v   as ring_attn_step (no mask: the method is non-causal)
 *   c         [B, H, Sq] fp32 bound from const_max_bound (identical for every step)
 *   acc       IN/OUT fp32 accumulator: [B, H, Sq, D] unnormalised output followed
 *             by [B, H, Sq] row sums (B*H*Sq*(D+1) floats). May be NULL when
 *             phase == INIT|FINAL (a single chunk).
 *   phase     CA_PHASE_INIT: first chunk (acc is overwritten, not read);
 *             CA_PHASE_FINAL: last chunk (o and lse are written, acc is not);
 *             CA_PHASE_ACCUMULATE (0): any middle chunk.
 *   o         OUT (FINAL only) [B, H, Sq, D], o_dtype CA_FP32 or CA_BF16:
 *             acc_o / max(acc_sum, 1e-37)
 *   lse       OUT (FINAL only, nullable) [B, H, Sq] fp32: c + log(max(acc_sum, 1e-37))
 *   workspace, workspace_bytes   as ring_attn_step (size for mask CA_MASK_NONE); split
 *             query tiles add their segments' sums in key order
 * Supported: as ring_attn_step.
 */
ca_status ring_attn_const_max_step(const void* q, ca_strides q_strides,
                                   const void* k, const void* v, ca_strides kv_strides,
                                   int dtype, int B, int H, int Sq, int Sk, int D,
                                   float softmax_scale, const float* c, float* acc, int phase,
                                   void* o, int o_dtype, float* lse,
                                   void* workspace, size_t workspace_bytes, void* stream);

/*
 * ring_attn_const_max_step_hop -- ring_attn_const_max_step and, in the same call, the
 * ring's next K/V hop, exactly as ring_attn_step_hop adds one to ring_attn_step (in the
 * step's launch on the CUs its last round leaves free, else as a copy just ahead of it).
 * Source: kernel reference page, Implementation, the ring loop.
 * Arguments, layouts, support and errors: as ring_attn_const_max_step, plus the hop
 * arguments of ring_attn_step_hop with the same requirements.
 */
ca_status ring_attn_const_max_step_hop(const void* q, ca_strides q_strides,
                                       const void* k, const void* v, ca_strides kv_strides,
                                       int dtype, int B, int H, int Sq, int Sk, int D,
                                       float softmax_scale, const float* c, float* acc, int phase,
                                       void* o, int o_dtype, float* lse,
                                       void* workspace, size_t workspace_bytes,
                                       void* hop_dst_k, void* hop_dst_v,
                                       const void* hop_src_k, const void* hop_src_v, size_t hop_bytes,
                                       void* stream);

/*
 * const_max_sink_prologue -- the bound prologue with sink keys taken out of the max.
 * Source: kernel reference page, "Adapting this kernel" (attention sinks: a handful of
 * keys whose norms dwarf the rest inflate max_j |k_j| for every row; excluding those keys
 * from the max reduction recovers the bound) and the prologue passages cited at
 * key_sqnorm_max. A key is a sink when |k_j| > theta * (mean key norm of its (b, h) over
 * every chunk); its exact contribution comes from sink_attention_partial.
 *   k            chunk c, batch b, token t, head h at k + c*chunk_stride + b*ks.b + t*ks.s
 *                + h*ks.h (elements); cp chunks of S_local tokens (the ring's pool); D a
 *                multiple of 8 in [8, 128]; key index of (c, t) = c * S_local + t
 *   theta        threshold factor (<= 0: no sinks)
 *   sink_cap     1..64 sinks per (b, h); a head with more candidates keeps the plain max
 *                and an empty list
 *   kmax_sq      OUT [B, H] max |k|^2 over every key
 *   kmax_sq_robust OUT [B, H] max |k|^2 over the non-sink keys (feed it to const_max_bound)
 *   knorm_sum    OUT [B, H] sum of |k| (scratch of the threshold)
 *   sink_idx     OUT [B, H, sink_cap] int32 sink key indices, ascending; sink_cnt OUT [B, H]
 * The threshold's sum is accumulated with float atomics, so a key within rounding of the
 * threshold may land on either side between runs; both are exact (a sink is attended
 * exactly). Errors: CA_ERR_NULL, CA_ERR_SHAPE, CA_ERR_DTYPE, CA_ERR_UNSUPPORTED, CA_ERR_HIP.
 */
ca_status const_max_sink_prologue(const void* k, int64_t chunk_stride, ca_strides ks, int dtype, int cp,
                                  int B, int S_local, int H, int D, float theta, int sink_cap,
                                  float* kmax_sq, float* kmax_sq_robust, float* knorm_sum,
                                  int32_t* sink_idx, int32_t* sink_cnt, void* stream);

/*
 * ring_attn_const_max_step_sinks -- ring_attn_const_max_step with the listed sink keys
 * left out of the fold (their scores may exceed the robust bound). Same arguments, plus
 *   sink_idx, sink_cnt, sink_cap  the lists from const_max_sink_prologue
 *   key_offset   key index of this chunk's first key (source rank * S_local)
 * bf16 only. Errors as ring_attn_const_max_step.
 */
ca_status ring_attn_const_max_step_sinks(const void* q, ca_strides qs, const void* k, const void* v,
                                         ca_strides kvs, int dtype, int B, int H, int Sq, int Sk, int D,
                                         float softmax_scale, const float* c, float* acc, int phase,
                                         void* o, int o_dtype, float* lse, const int32_t* sink_idx,
                                         const int32_t* sink_cnt, int sink_cap, int64_t key_offset,
                                         void* workspace, size_t workspace_bytes, void* stream);

/*
 * sink_attention_partial -- exact (online-max) attention of every query row against the
 * sink keys alone, as a partial output and LSE to merge (lse_merge) with the sink-robust
 * const-max result. Gathers the listed K and V rows from the pool, then runs the bf16 step
 * kernel with a per-head key count.
 *   q            [B, Sq, H, D] bf16, strides qs
 *   k, v         the pool as in const_max_sink_prologue (bf16; shared strides)
 *   o            OUT [B, H, Sq, D] fp32; lse OUT [B, H, Sq] (-inf for a head with no sink)
 *   workspace    sink_attention_workspace_size() bytes
 * Supported: D == 128. Errors: CA_ERR_NULL, CA_ERR_SHAPE, CA_ERR_UNSUPPORTED,
 * CA_ERR_WORKSPACE, CA_ERR_HIP.
 */
ca_status sink_attention_partial(const void* q, ca_strides qs, const void* k, const void* v,
                                 int64_t chunk_stride, ca_strides kvs, int cp, int B, int H, int Sq,
                                 int S_local, int D, float softmax_scale, const int32_t* sink_idx,
                                 const int32_t* sink_cnt, int sink_cap, float* o, float* lse,
                                 void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of device workspace sink_attention_partial needs for these sizes. */
ca_status sink_attention_workspace_size(int B, int H, int D, int sink_cap, size_t* bytes);


/*
 * lse_merge -- LSE-corrected merge of n partial attention results.
 * Source: DCP page, DCP Decode compute pattern steps 4-7: gather the partial LSEs,
 * global_lse = log sum_s exp(lse_s), weight_s = exp(lse_s - global_lse), output =
 * sum_s weight_s * o_s. Also the fold of ring-step partials ("Sharding the Input",
 * ring attention; kernel reference page, Design: online-softmax ring bookkeeping).
 *
 *   o_parts    [n, rows, D] fp32, contiguous (partial s at o_parts + s*rows*D)
 *   lse_parts  [n, rows] fp32 (-inf marks an empty partial; it weighs 0)
 *   o_out      OUT [rows, D], o_dtype CA_FP32 or CA_BF16 (may not alias o_parts)
 *   lse_out    OUT [rows] fp32 global LSE, nullable
 * All partials -inf -> output 0 and lse -inf. Requires n >= 1, D % 4 == 0.
 */
ca_status lse_merge(int n, const float* o_parts, const float* lse_parts, int64_t rows, int D,
                    void* o_out, int o_dtype, float* lse_out, void* stream);

/*
 * dcp_decode_partial -- one DCP shard's decode attention: every query head of every
 * sequence attends the tokens resident in this shard's paged KV cache, giving the
 * shard's partial output and LSE (to be merged across shards with lse_merge).
 * Source: DCP page, DCP Decode compute pattern steps 3-4 (gathered Q against the
 * local KV shard, partial LSE), local_filled computation (tokens resident per
 * shard), slot mapping (blocks of interleave_size tokens dealt round-robin).
 *
 *   q            [B, Hq, D] bf16 contiguous (one decode token per sequence)
 *   k_pool       [num_blocks, Hkv, block_size, D] bf16: token-major blocks
 *   v_pool       [num_blocks, Hkv, D, block_size] bf16: d-major blocks (this
 *                library's V cache layout: each block's values stored transposed
 *                so that a block feeds the P.V matrix product without a shuffle).
 *                A cache kept token-major per block ([num_blocks, block_size, Hkv, D],
 *                as paged-attention servers commonly hold it) is not read directly:
 *                its writer stores each new token's K row at k_pool[blk, h, slot, :]
 *                and its V row at v_pool[blk, h, :, slot] (a D-element scatter with
 *                stride block_size), once per token at cache-write time; an existing
 *                token-major cache is converted once by that same permutation.
 *   block_table  [B, max_blocks] int32: physical block of the sequence's shard-local
 *                block j (shard-local token t is slot t % block_size of block
 *                t / block_size); entries past the sequence's blocks are ignored;
 *                an id outside [0, num_blocks) reads as an all-zero block
 *   num_blocks   blocks in k_pool and v_pool; at least 1 when max_blocks > 0
 *                (CA_ERR_SHAPE otherwise: an empty pool has no block to read, so a
 *                caller with nothing resident passes max_blocks = 0)
 *   local_lens   [B] int32: tokens of each sequence resident on this shard
 *                (local_filled); values are clamped to [0, max_blocks * block_size]
 *   o            OUT [B, Hq, D] fp32 partial output; lse OUT [B, Hq] fp32
 *   workspace    device scratch of at least dcp_decode_workspace_size() bytes
 * Query head h uses KV head h / (Hq / Hkv). Supported: D in {64, 128}, block_size == 16,
 * Hq % Hkv == 0, Hq / Hkv <= 16. A sequence with local_lens 0 yields o = 0, lse = -inf.
 */
ca_status dcp_decode_partial(const void* q, const void* k_pool, const void* v_pool,
                             const int32_t* block_table, const int32_t* local_lens,
                             int B, int Hq, int Hkv, int D, int block_size, int max_blocks,
                             int num_blocks, float softmax_scale, float* o, float* lse,
                             void* workspace, size_t workspace_bytes, void* stream);

/*
 * dcp_decode_partial_noalloc -- dcp_decode_partial for callers that cannot allocate device
 * memory or pass a workspace: code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation. Same arguments, results and kernels as dcp_decode_partial, minus
 * the workspace: the split partials go to a fixed scratch array of the library, 80 MiB on
 * each GPU it runs on, allocated when the library's device code is loaded and held until
 * the process ends. The call allocates nothing (no hipMalloc, no allocating library call).
 *   Limit: B * Hq * splits * (D + 1) * 4 bytes, splits = ceil(max_blocks * block_size /
 *   1536) made odd (what dcp_decode_workspace_size reports), must fit in
 *   80 MiB (e.g. B = 32, Hq = 64, D = 128 allows max_blocks up to 7584 blocks of 16), else
 *   CA_ERR_WORKSPACE with the sizes in the message.
 *   Every call on one GPU shares that GPU's scratch: calls that may overlap in time on one
 *   GPU (different streams, or other threads) race and must be serialised by the caller;
 *   calls in order on one stream are safe. Nothing in the scratch needs clearing between
 *   calls (every split partial that a call reads, the call writes first).
 * Errors: as dcp_decode_partial, with CA_ERR_WORKSPACE for sizes over the limit and
 * CA_ERR_HIP if the scratch's device address cannot be found.
 */
ca_status dcp_decode_partial_noalloc(const void* q, const void* k_pool, const void* v_pool,
                                     const int32_t* block_table, const int32_t* local_lens,
                                     int B, int Hq, int Hkv, int D, int block_size, int max_blocks,
                                     int num_blocks, float softmax_scale, float* o, float* lse,
                                     void* stream);

/*
 * dcp_decode_partial_active -- one DCP shard's decode step with the page's two-part
 * mask: the prior tokens this shard holds plus the current decode token, which only
 * the shard owning its position attends, so that the merged result counts it once.
 * Source: DCP page, "Active Token Handling and dcp_active_mask" (prior_mask over slots
 * [0, local_filled), the current token's slot gated by owner == dcp_rank, owner from
 * pos_in_vblock) and "local_filled Computation" (the resident count, computed here on
 * the device from each sequence's prior length N).
 *
 *   q, k_pool, v_pool, block_table, num_blocks, softmax_scale, o, lse, workspace:
 *                as dcp_decode_partial (the cache holds this shard's prior tokens)
 *   prior_lens   [B] int32: prior tokens N of each sequence, a global count; the
 *                current token sits at position N
 *   k_cur, v_cur [B, Hkv, D] bf16 contiguous: the current token's K and V (every shard
 *                of the group holds the same values)
 *   rank, world  this shard's DCP rank and the group size (0 <= rank < world)
 *   interleave   positions per interleave block; must divide block_size
 * The shard's resident count is local_filled(N, rank, block_size, interleave, world),
 * clamped to max_blocks * block_size. A shard with no resident token that does not own
 * position N yields o = 0, lse = -inf. Errors as dcp_decode_partial, and CA_ERR_SHAPE
 * for a rank outside the group.
 */
ca_status dcp_decode_partial_active(const void* q, const void* k_pool, const void* v_pool,
                                    const int32_t* block_table, const int32_t* prior_lens,
                                    const void* k_cur, const void* v_cur, int rank, int world,
                                    int interleave, int B, int Hq, int Hkv, int D, int block_size,
                                    int max_blocks, int num_blocks, float softmax_scale, float* o,
                                    float* lse, void* workspace, size_t workspace_bytes, void* stream);

/*
 * segmented_attention_partial -- one rank's DCP prefill attention for a chunk: every query
 * of the chunk against this rank's prior tokens (in the paged cache) and its slice of the
 * chunk, causal on global positions; the rank's partial output and LSE, to be merged
 * across the group with lse_merge (the page's LSE all-gather and reduce-scatter).
 * Source: DCP page, "Segmented Attention CP": Purpose, API and Algorithm steps 1-4
 * (prior read from the cache and masked by slot count, prior + current keys, causal mask
 * from global positions: prior slot s at (s / I)(W I) + R I + s % I, chunk token j at
 * prior_global + (j / I)(W I) + R I + j % I, query i at prior_global + i).
 *
 *   q             [1, S, Hq, D] bf16, strides qs: every query of the chunk, in global order
 *   k_cur, v_cur  [1, S_local, Hkv, D] bf16, strides kvs: this rank's slice of the chunk
 *                 (S_local = S / world; S a multiple of world * interleave)
 *   k_cache       [num_blocks, Hkv, 16, D] bf16 and v_cache [num_blocks, Hkv, D, 16] bf16:
 *                 the paged prior cache in dcp_decode_partial's layout
 *   block_table   [max_blocks] int32: physical block of prior slot s / 16; an id outside
 *                 [0, num_blocks) reads as an all-zero block
 *   prior_tokens  this rank's prior slots (local_filled of the global prior length; 0 on
 *                 the first chunk). Every prior position precedes every query of the
 *                 chunk, so the prior keys carry no mask.
 *   rank, world, interleave   the rank's place in the DCP group and the interleave size
 *   o             OUT [Hq, S, D] fp32; lse OUT [Hq, S] fp32 (natural log; -inf for a query
 *                 that sees no key of this rank)
 *   workspace     segmented_attention_workspace_size() bytes (0 when prior_tokens == 0)
 * Query head h reads K/V head h / (Hq / Hkv). Supported: D == 128, Hkv <= 16, one
 * sequence per call. Errors: CA_ERR_NULL, CA_ERR_SHAPE, CA_ERR_UNSUPPORTED,
 * CA_ERR_WORKSPACE, CA_ERR_HIP.
 */
ca_status segmented_attention_partial(const void* q, ca_strides qs, const void* k_cur, const void* v_cur,
                                      ca_strides kvs, const void* k_cache, const void* v_cache,
                                      const int32_t* block_table, int max_blocks, int num_blocks,
                                      int prior_tokens, int rank, int world, int interleave, int Hq,
                                      int Hkv, int S, int S_local, int D, float softmax_scale, float* o,
                                      float* lse, void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of device workspace segmented_attention_partial needs for these sizes. */
ca_status segmented_attention_workspace_size(int Hq, int Hkv, int S, int D, int prior_tokens,
                                             size_t* bytes);

/* Bytes of device workspace dcp_decode_partial needs for these sizes. */
ca_status dcp_decode_workspace_size(int B, int Hq, int D, int block_size, int max_blocks,
                                    size_t* bytes);

/*
 * kv_chunk_copy -- the ring's K/V hop on one device: one asynchronous copy kernel
 * on `stream` moves one K chunk (src_k -> dst_k) and one V chunk (src_v -> dst_v),
 * `bytes` each. All four pointers must be 16-byte aligned and bytes a multiple of
 * 16 (CA_ERR_SHAPE otherwise); bytes == 0 is a no-op. Source and destination must
 * not overlap.
 * Source: kernel reference page, Implementation "The ring loop" (rotating K/V
 * buffers, the next hop launched while the current step computes).
 */
ca_status kv_chunk_copy(void* dst_k, void* dst_v, const void* src_k, const void* src_v,
                        size_t bytes, void* stream);

/* Message describing the last non-OK status returned on this thread. */
const char* ca_last_error(void);

/* Library version, e.g. "0.1.0". */
const char* ca_version(void);

#ifdef __cplusplus
}
#endif

#endif /* CTXATTN_H */
