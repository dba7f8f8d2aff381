/*
 * libsqa: scaled-dot-product attention forward with decoupled query and
 * key/value head counts, for AMD Instinct MI355X (gfx950).
 *
 * One call, sqa_attn_fwd, computes for every batch b, query head h and
 * query position i
 *
 *     out[b,i,h,:] = sum_j softmax_j( scale * <q[b,i,h,:], k[b,j,g,:]> ) v[b,j,g,:]
 *
 * where g = floor(h / (H_q / H_kv)) is the key/value head that query head h
 * shares, and j runs over all S positions (causal = 0) or over j <= i
 * (causal = 1).
 *
 * Sources:
 *   - Sparse Query Attention ("Sparse Query Attention (SQA): A
 *     Computationally Efficient Attention Mechanism with Query Heads
 *     Reduction", abstract): SQA lowers the number of query heads H_q, not
 *     the number of key/value heads, and the score and P.V work falls in
 *     proportion to H_q.  The arithmetic per head is unchanged.
 *   - Grouped heads ("Paper explainer: GQA - Grouped-Query Attention",
 *     section on MHA/MQA/GQA with the GQA equations and the grouping
 *     figure): H_kv groups of H_q/H_kv consecutive query heads, each group
 *     reading one key/value head.  H_kv = H_q is MHA, H_kv = 1 is MQA.  The
 *     page's PyTorch module asserts that the head count is divisible by the
 *     group count.
 *   - The attention call itself (same page, PyTorch module): softmax of the
 *     scaled scores times V, with is_causal giving the lower-triangular mask.
 *
 * Layout.  All four tensors are dense and contiguous in BSHD order: element
 * (b, s, h, e) sits at ((b*S + s)*H + h)*d + e, with H = H_q for q and out
 * and H = H_kv for k and v.  This is the layout of the projections before the
 * page's transpose, so no transpose is needed on either side.
 *
 * Ownership.  The caller allocates and owns every buffer (device memory).
 * The attention entry points keep no state, allocate nothing, and only
 * enqueue kernels on `stream` (the null stream is allowed); the call returns
 * before the work is done, and it can be captured into a HIP graph.  The
 * layer entry point also keeps a GEMM library handle per device (see
 * sqa_layer_fwd), and sqa_attn_decode_noalloc uses a fixed scratch array
 * that the library holds on each GPU (see there).  All entry points are safe
 * to call from several host threads at once (sqa_attn_decode_noalloc only
 * when the calls' executions do not overlap on one GPU).
 */
#ifndef SQA_H
#define SQA_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Opaque HIP stream handle (same type as hipStream_t). */
typedef struct ihipStream_t* sqa_stream_t;

typedef enum {
  SQA_OK = 0,
  SQA_ERR_INVALID_ARGUMENT = 1, /* a documented precondition does not hold */
  SQA_ERR_UNSUPPORTED = 2,      /* valid arguments the library has no kernel for */
  SQA_ERR_HIP = 3               /* the HIP runtime refused the launch */
} sqa_status;

typedef enum {
  SQA_BF16 = 0, /* bf16 in and out, fp32 accumulation, bf16 MFMA */
  SQA_FP32 = 1  /* fp32 in and out, fp32 arithmetic */
} sqa_dtype;

/*
 * Attention forward.
 *
 *   q    [B, S, H_q,  d]   device pointer, dtype elements, 16-byte aligned
 *   k    [B, S, H_kv, d]   device pointer, dtype elements, 16-byte aligned
 *   v    [B, S, H_kv, d]   device pointer, dtype elements, 16-byte aligned
 *   out  [B, S, H_q,  d]   device pointer, written in full; must not
 *                          overlap q, k or v
 *   B, S       batch size and sequence length (queries and keys have the
 *              same length S); B*S == 0 is a successful no-op
 *   H_q, H_kv  query and key/value head counts: H_q >= H_kv >= 1 and
 *              H_q % H_kv == 0
 *   d          head dimension: 32, 64 or 128
 *              (H_q * d and H_kv * d at most 2^22: UNSUPPORTED beyond)
 *   scale      finite multiplier of the scores (1/sqrt(d) is usual)
 *   causal     0 = every query sees all S keys; 1 = query i sees keys j <= i
 *   stream     HIP stream to enqueue on (NULL = null stream)
 *
 * Returns SQA_OK after enqueueing.  SQA_ERR_INVALID_ARGUMENT and
 * SQA_ERR_UNSUPPORTED are decided from the arguments alone, before any HIP
 * call, and leave out untouched.  SQA_ERR_HIP reports a launch the runtime
 * refused.  Faults during execution surface at the caller's next
 * synchronisation on the stream.
 *
 * Speed: bf16 runs on bf16 MFMA kernels (the performance path).  The fp32
 * forward and backward (sqa_attn_bwd) run on the fp32 matrix cores
 * (v_mfma_f32_32x32x2_f32): the forward at 104-132 TFLOP/s measured at
 * S = 4096-32768, the backward at up to 91 TFLOP/s credited at 10*d flops
 * per pair (fp32 matrix peak 157.3); the fp32 decode (sqa_attn_decode) on
 * the same matrix cores with the bf16 decode's split plan.
 */
sqa_status sqa_attn_fwd(const void* q, const void* k, const void* v, void* out, int64_t B,
                        int64_t S, int32_t H_q, int32_t H_kv, int32_t d, sqa_dtype dtype,
                        float scale, int causal, sqa_stream_t stream);

/*
 * Attention forward that also returns the row log-normaliser
 *
 *   lse[b, i, h] = ln( sum_j exp(scale * <q[b,i,h,:], k[b,j,g,:]>) )
 *
 * over the same visible keys j: the logarithm of the row sum D_ii of
 * A = exp(scores) in the row-normalised form D(A)^-1 A V ("Beyond Classical
 * Attention: Quantum Attention" review, proposed-method section).  With it the
 * probabilities can be rebuilt as exp(score - lse) without a second pass over
 * the keys (what a backward pass needs).
 *
 *   lse  [B, S, H_q] fp32, device pointer, 4-byte aligned, must not overlap
 *        q, k, v or out; may be NULL (then this is sqa_attn_fwd).
 * All other arguments, the layout, ownership and error behaviour are those
 * of sqa_attn_fwd.  With lse given, the bf16 kernels keep a running row
 * maximum on every key tile, so that the probabilities that carry the row
 * sum stay close to 1 and the log-normaliser is accurate; sqa_attn_fwd (lse
 * NULL) fixes the softmax shift at the first tile's maximum at d = 64 and 128,
 * which is 3-4 % faster and gives the same output up to bf16 rounding.
 */
sqa_status sqa_attn_fwd_lse(const void* q, const void* k, const void* v, void* out, float* lse,
                            int64_t B, int64_t S, int32_t H_q, int32_t H_kv, int32_t d,
                            sqa_dtype dtype, float scale, int causal, sqa_stream_t stream);

/*
 * Attention backward: gradients of out with respect to q, k and v for the
 * upstream gradient dout = dL/dout.  The pages define only the forward
 * computation; this is its exact derivative (softmax Jacobian), with the
 * gradients of a shared K/V head summed over the H_q/H_kv query heads that
 * read it (GQA explainer: grouping figure, expand in the PyTorch module):
 *
 *   P = exp(scale*q.k - lse), dP = dout.v, D_i = <dout_i, out_i>,
 *   dS = P (dP - D), dq = scale dS k, dk = scale dS^T q, dv = P^T dout.
 *
 *   q, k, v, out, dout   the forward's inputs and output and the upstream
 *                        gradient (dout shaped like out), dtype elements,
 *                        16-byte aligned, BSHD as in sqa_attn_fwd
 *   lse                  [B, S, H_q] fp32 from sqa_attn_fwd_lse, 4-byte aligned
 *   dq                   [B, S, H_q, d] output, written in full
 *   dk, dv               [B, S, H_kv, d] outputs, written in full
 *   workspace            caller-owned scratch of at least
 *                        sqa_attn_bwd_workspace_size(B, S, H_q) bytes,
 *                        16-byte aligned; contents are overwritten
 *   workspace_bytes      its size
 *   B ... stream         as for sqa_attn_fwd (same scale and causal as the
 *                        forward that produced out and lse)
 *
 * Outputs and workspace must not overlap each other or any input.  Errors as
 * for sqa_attn_fwd, and SQA_ERR_UNSUPPORTED when the workspace size would not
 * fit int64.  bf16: MFMA kernels with fp32 accumulation, probabilities and dS
 * rounded to bf16 for the products; fp32: fp32 MFMA kernels with fp32
 * probabilities and dS.
 */
sqa_status sqa_attn_bwd(const void* q, const void* k, const void* v, const void* out, const void* dout,
                        const float* lse, void* dq, void* dk, void* dv, void* workspace,
                        int64_t workspace_bytes, int64_t B, int64_t S, int32_t H_q, int32_t H_kv,
                        int32_t d, sqa_dtype dtype, float scale, int causal, sqa_stream_t stream);

/* Workspace bytes sqa_attn_bwd needs (2 fp32 values per query row and head,
 * rows padded to a multiple of 64); -1 for invalid sizes or a size beyond
 * int64. */
int64_t sqa_attn_bwd_workspace_size(int64_t B, int64_t S, int32_t H_q);

/*
 * Decode attention: one new query token per sequence against that
 * sequence's key/value cache (the inference step whose cost the GQA
 * explainer's background section attributes to reading the cache, 2*H_kv*d
 * values per cached position; the SQA abstract names this bandwidth-bound
 * regime as the one GQA/MQA address).  Per sequence b and query head h:
 *
 *   out[b,h,:] = sum_{j < len_b} softmax_j(scale * <q[b,h,:], k[b,j,g,:]>) v[b,j,g,:]
 *   lse[b,h]   = log sum_{j < len_b} exp(scale * <q[b,h,:], k[b,j,g,:]>)
 *
 * with g = floor(h / (H_q/H_kv)) as in sqa_attn_fwd: the causal forward's
 * row len_b - 1, for a token whose own key/value is already in the cache.
 *
 *   q          [B, H_q, d] of `dtype`, device, 16-byte aligned
 *   k_cache    [B, S_max, H_kv, d] of `dtype` (BSHD), device, 16-byte aligned;
 *   v_cache    positions >= len_b are never read
 *   seqlens    [B] int32 device array of cache lengths, 4-byte aligned, or
 *              NULL for S_max everywhere.  A length above S_max counts as
 *              S_max; a length <= 0 gives out = 0 and lse = -inf.
 *   out        [B, H_q, d] output of `dtype`, 16-byte aligned
 *   lse        [B, H_q] fp32 output (natural log), 4-byte aligned, or NULL
 *   workspace  caller-owned device scratch of at least
 *              sqa_attn_decode_workspace_size(...) bytes, 16-byte aligned;
 *              holds per-split partial results, overwritten
 *   B, S_max, H_q, H_kv, d, scale, stream   as for sqa_attn_fwd
 *
 * Outputs and workspace must not overlap each other or any input.
 * SQA_ERR_INVALID_ARGUMENT as for sqa_attn_fwd (and for a short workspace);
 * SQA_ERR_UNSUPPORTED for d not in {32, 64, 128}, H_q * d or H_kv * d above
 * 2^22, S_max > 2^30, or B * S_max * H_q * (d + 2) * 4 beyond int64 (the
 * split plan's bound).  B == 0
 * is a successful no-op.  Asynchronous on `stream`.  A split kernel and a
 * combine kernel: bf16 MFMA with fp32 accumulation and probabilities rounded
 * to bf16 for the P.V product, or fp32 MFMA with fp32 probabilities.
 */
sqa_status sqa_attn_decode(const void* q, const void* k_cache, const void* v_cache, const int32_t* seqlens,
                           void* out, float* lse, void* workspace, int64_t workspace_bytes, int64_t B,
                           int64_t S_max, int32_t H_q, int32_t H_kv, int32_t d, sqa_dtype dtype, float scale,
                           sqa_stream_t stream);

/* Workspace bytes sqa_attn_decode needs; -1 for invalid sizes or a split
 * plan beyond int64 (B * max(S_max, 1) * H_q * (d + 2) * 4). */
int64_t sqa_attn_decode_workspace_size(int64_t B, int64_t S_max, int32_t H_q, int32_t H_kv, int32_t d);

/*
 * Decode without a workspace, for callers that cannot allocate device memory
 * (work captured into a HIP graph, tight serving loops, harnesses that forbid
 * allocation).  Same computation, arguments and layout as sqa_attn_decode,
 * minus the workspace: the split kernel's partial results go to a fixed
 * scratch array of SQA_DECODE_SCRATCH_BYTES that the library holds on each
 * GPU it runs on until the process ends.  This call allocates nothing.  Its
 * first call on a GPU looks up that GPU's copy of the array (a HIP symbol
 * lookup, no allocation).
 *
 * Splits are lengthened, if needed, so that the partial results fit:
 * B * H_q * n_splits * (d + 2) * 4 bytes <= SQA_DECODE_SCRATCH_BYTES.  The
 * result can then differ from sqa_attn_decode's in rounding only (a
 * different split of the same sum).  SQA_ERR_UNSUPPORTED when even one split
 * per head does not fit: B * H_q * (d + 2) * 4 > SQA_DECODE_SCRATCH_BYTES
 * (more than 32263 sequence-heads at d = 128).
 *
 * Every call on one GPU shares that GPU's array, and the array keeps the last
 * call's contents: two calls whose execution overlaps on the same GPU (on
 * different streams, or from different host threads without ordering) race
 * on it and give undefined results.  Calls ordered on one stream are safe.
 * Other errors as for sqa_attn_decode.
 */
#define SQA_DECODE_SCRATCH_BYTES ((int64_t)16 << 20)
sqa_status sqa_attn_decode_noalloc(const void* q, const void* k_cache, const void* v_cache, const int32_t* seqlens,
                                   void* out, float* lse, int64_t B, int64_t S_max, int32_t H_q, int32_t H_kv,
                                   int32_t d, sqa_dtype dtype, float scale, sqa_stream_t stream);

/*
 * Full attention layer forward with decoupled head counts: the GQA
 * explainer's PyTorch module (q/k/v projections, K/V heads shared by groups
 * of query heads, scaled dot-product attention, output projection; section on
 * the PyTorch implementation) with the query-head count free, as Sparse Query
 * Attention proposes (SQA abstract: fewer query heads, so fewer attention
 * FLOPs and narrower q and output projections):
 *
 *   [q | k | v] = x W_qkv^T,   attn = sqa_attn_fwd(q, k, v),   out = attn W_o^T
 *
 *   x          [B, S, d_model] bf16, device, 16-byte aligned
 *   w_qkv      [(H_q + 2 H_kv) d, d_model] bf16: the q, k and v projection
 *              weights (nn.Linear layout, out x in) stacked in that order;
 *              rows h d ... h d + d - 1 of each block belong to head h
 *   w_o        [d_model, H_q d] bf16 (nn.Linear layout)
 *   out        [B, S, d_model] bf16 output
 *   workspace  caller-owned device scratch of at least
 *              sqa_layer_workspace_size(B, S, H_q, H_kv, d) bytes, 16-byte
 *              aligned: the projection output, the attention output and the
 *              GEMM library's workspace; overwritten
 *   B, S, H_q, H_kv, d, scale, causal, stream   as for sqa_attn_fwd
 *
 * The projections run on hipBLASLt (bf16 inputs and outputs, fp32
 * accumulation); the library creates one hipBLASLt handle per device on
 * first use and keeps it, with the chosen GEMM algorithms, until the process
 * ends.  q, k and v are rounded to bf16 after the projection and the
 * attention output before the output projection.  out must not overlap any
 * input or the workspace; the workspace must not overlap any input.
 * SQA_ERR_INVALID_ARGUMENT as for sqa_attn_fwd (also d_model < 1 or a short
 * workspace); SQA_ERR_UNSUPPORTED for d not in {32, 64, 128},
 * (H_q + 2 H_kv) * d above 2^22, d_model not a multiple of 8 or S > 2^30; SQA_ERR_HIP for a HIP or hipBLASLt failure.
 */
sqa_status sqa_layer_fwd(const void* x, const void* w_qkv, const void* w_o, void* out, void* workspace,
                         int64_t workspace_bytes, int64_t B, int64_t S, int32_t d_model, int32_t H_q, int32_t H_kv,
                         int32_t d, float scale, int causal, sqa_stream_t stream);

/* Workspace bytes sqa_layer_fwd needs; -1 for invalid sizes. */
int64_t sqa_layer_workspace_size(int64_t B, int64_t S, int32_t H_q, int32_t H_kv, int32_t d);

/* Static, NUL-terminated description of a status code. */
const char* sqa_status_string(sqa_status status);

#ifdef __cplusplus
}
#endif

#endif /* SQA_H */
