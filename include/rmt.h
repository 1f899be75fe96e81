/*
 * rmt.h -- C ABI of the diagonal-batched recurrent-memory-transformer library
 * (librmt.so, built for AMD Instinct MI355X / gfx950).
 *
 * The method.  A recurrent memory transformer (RMT) reads one long sequence
 * as S segments of n tokens.  Layer l keeps m memory rows.  Cell (l, s)
 * consumes A = [M(l, s-1); X(l-1, s)] (m memory rows, then n segment rows)
 * and produces R = m + n rows Y; rows [0, n) become X(l, s), rows [n, R)
 * become M(l, s).  Cell (l, s) needs only (l-1, s) and (l, s-1), so all
 * cells on an anti-diagonal d = l + s are independent and run together, each
 * with its own layer's weights, as one grouped launch per stage
 * ("Diagonal Batching for Recurrent Memory Transformers", skill page:
 * Core Concept; Architecture Overview -- Diagonal Reorganization, Dependency
 * Preservation, GroupedGEMM Operations, GPU Kernel Optimization).  The
 * reordering is exact and needs no retraining ("Diagonal Batching Unlocks
 * Parallelism in Recurrent Memory Transformers for Long Contexts",
 * abstract).
 *
 * Conventions shared by every call:
 *   - Every call returns RMT_OK (0) or a negative error code; a thread-local
 *     message describing the last error is returned by rmt_last_error().
 *   - "device" pointers are HIP device allocations on the current device
 *     (for example torch tensors' data_ptr()); "host" pointers are CPU memory.
 *   - The library never takes ownership of caller memory and never allocates
 *     device memory: packed weights and the activation workspace live in
 *     buffers the caller allocates (for example torch tensors) and attaches
 *     with rmt_model_bind, sized by rmt_workspace_bytes.  Device work is
 *     queued on the caller's HIP stream and returns before it finishes;
 *     faults inside kernels surface at the caller's next synchronisation.
 *   - Matrices are row-major.  Mathematical weights are W[d_in][d_out], so a
 *     cell computes Y = A W.
 */
#ifndef RMT_H
#define RMT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Error codes. */
#define RMT_OK 0
#define RMT_EINVAL (-1)        /* bad argument: sizes, null pointers, ranges      */
#define RMT_EUNSUPPORTED (-2)  /* valid but not implemented (see each call)       */
#define RMT_EHIP (-3)          /* a HIP runtime call failed (message has details) */
#define RMT_ENOMEM (-4)        /* reserved (the library allocates no device memory) */
#define RMT_EWORKSPACE (-5)    /* a buffer the call needs is not bound, or too small */

/* Cell kinds: what one (layer, segment) cell computes on A [R x d].
 *   LINEAR_GELU  Y = GELU_erf(A W_l + b_l)                        (fp32 only)
 *   NORM_SWIGLU  Y = A + SwiGLU_l(RMSNorm_l(A))                    (bf16 only)
 *   LLAMA        H = A + Attn_l(RMSNorm1_l(A)) Wo_l;
 *                Y = H + SwiGLU_l(RMSNorm2_l(H))                   (bf16 only)
 *   ENCODER      H = A + MHA_l(LN1_l(A));
 *                Y = H + relu(LN2_l(H) W1_l + b1_l) W2_l + b2_l    (bf16 only)
 * with RMSNorm(x) = x * rsqrt(mean(x^2) + eps) * g,
 * SwiGLU(z) = (silu(z Wg) * (z Wu)) Wd, and Attn causal over the cell's R
 * rows with grouped-query heads (query head h reads KV head h / (Hq/Hkv)),
 * rotate-half RoPE at positions 0..R-1 within the cell, scale 1/sqrt(hd).
 * ENCODER is the layer the skill page's Implementation sketch stacks (torch
 * nn.TransformerEncoderLayer; its argument values are stripped from the
 * page, read here as pre-norm with a 4x ReLU feed-forward): LN(x) =
 * (x - mean) / sqrt(var + eps) * g + beta with the biased variance, and
 * MHA(z) = concat_h softmax(q_h k_h^T / sqrt(hd)) v_h Wo + bo over all R rows
 * (no mask, n_kv_heads == n_heads) with [q k v] = z Wqkv + bqkv. */
#define RMT_CELL_LINEAR_GELU 0
#define RMT_CELL_NORM_SWIGLU 1
#define RMT_CELL_LLAMA 2
#define RMT_CELL_ENCODER 3

/* Storage / arithmetic types.  A model's dtype is the type of its 16-bit
 * storage and MFMA operands (weights, normalised rows, Q/K/V, probabilities,
 * attention output, SwiGLU output); the residual stream, accumulation and
 * norm/softmax arithmetic are fp32 in every case.
 *   RMT_F32   LINEAR_GELU cells: everything fp32.
 *   RMT_BF16  bf16 operands (the other cells).
 *   RMT_F16   IEEE half operands, LLAMA cells only: the same MFMA rate and
 *             three more mantissa bits than bf16.  bf16 weights convert
 *             exactly unless their magnitude is below 2^-17 (rounded to
 *             fp16's 2^-24 grid) or above 65504 (rejected by no check:
 *             they become infinite). */
#define RMT_F32 0
#define RMT_BF16 1
#define RMT_F16 2

typedef struct rmt_config {
  int32_t cell;        /* RMT_CELL_*                                          */
  int32_t dtype;       /* RMT_F32 (LINEAR_GELU), RMT_BF16, or RMT_F16 (LLAMA) */
  int32_t L;           /* layers                                              */
  int32_t S;           /* segments per forward call                           */
  int32_t n;           /* segment tokens                                      */
  int32_t m;           /* memory rows per layer                               */
  int32_t d;           /* model width                                         */
  int32_t n_heads;     /* LLAMA, ENCODER: query heads Hq                      */
  int32_t n_kv_heads;  /* LLAMA: KV heads Hkv (Hq/Hkv 1, 2 or a multiple of 4);
                          ENCODER: equal to n_heads                           */
  int32_t head_dim;    /* LLAMA, ENCODER: hd, 64 or 128; Hq*hd == d           */
  int32_t ffn;         /* NORM_SWIGLU, LLAMA: SwiGLU width F; ENCODER: W1 width */
  int32_t vocab;       /* LLAMA: embedding rows V                             */
  float eps;           /* RMSNorm / LayerNorm epsilon                         */
  float rope_theta;    /* LLAMA: RoPE base                                    */
  int32_t post_norm;   /* ENCODER: 0 = pre-norm (the default reading), 1 =
                          post-norm (torch's norm_first=False): H = LN1(A +
                          MHA(A)), Y = LN2(H + FFN(H)); must be 0 otherwise   */
} rmt_config;

/* Mathematical-layout weights, stacked over layers (device pointers).
 * rmt_model_create records the pointers; rmt_model_bind(RMT_BUF_WEIGHTS)
 * packs them into the caller's weight buffer, after which the caller may free
 * them -- except `embed`, which every forward call reads and which must
 * outlive the model.  Element type of the
 * matrices: fp32 for RMT_F32 models; bf16 or fp32 for RMT_BF16 and RMT_F16
 * models, as given by `weight_dtype`, rounded to nearest even into the
 * model's 16-bit type while packing.  Gains,
 * shifts and biases (g1, g2, b, beta*, b*) are always fp32.  Unused fields
 * may be NULL.
 *   LINEAR_GELU: w [L][d][d], b [L][d]
 *   NORM_SWIGLU: g2 [L][d], wg [L][d][F], wu [L][d][F], wd [L][F][d]
 *   LLAMA:       g1 [L][d], wqkv [L][d][(Hq+2Hkv)*hd] (columns: Q heads,
 *                then K heads, then V heads, hd each), wo [L][Hq*hd][d],
 *                g2, wg, wu, wd as above, embed [V][d] (bf16).
 *   ENCODER:     g1, beta1 [L][d] (LN1), wqkv [L][d][3d] (Q, K, V heads as
 *                for LLAMA), bqkv [L][3d], wo [L][d][d], bo [L][d], g2, beta2
 *                [L][d] (LN2), w1 [L][d][F], b1 [L][F], w2 [L][F][d], b2 [L][d]. */
typedef struct rmt_weights {
  int32_t weight_dtype;  /* RMT_F32 or RMT_BF16: element type of w/wqkv/wo/wg/wu/wd */
  const void* w;
  const float* b;
  const float* g1;
  const void* wqkv;
  const void* wo;
  const float* g2;
  const void* wg;
  const void* wu;
  const void* wd;
  const void* embed;
  /* ENCODER */
  const float* beta1;
  const float* bqkv;
  const float* bo;
  const float* beta2;
  const void* w1;
  const float* b1;
  const void* w2;
  const float* b2;
} rmt_weights;

/* Outputs of a forward call (device pointers, caller-allocated), for each of
 * the B sequences (B = 1 unless set by rmt_model_set_batch):
 *   hidden [B][T][d] fp32: X(L-1, s) for every segment, in segment order.
 *   mem    [B][L][m][d] fp32: M(l, S-1), the memory after the last segment;
 *          it may alias the mem0 argument (in-place state update). */
typedef struct rmt_output {
  float* hidden;
  float* mem;
} rmt_output;

typedef struct rmt_model rmt_model;

/* Anti-diagonal schedule of the L x S (layer, segment) grid (host only,
 * thread-safe; skill page, Implementation: the scheduler's enumeration).
 * Diagonal k (k = 0 .. L+S-2) holds the cells (l, k-l) with 0 <= k-l < S,
 * layers ascending; diagonal k has min(k+1, L, S, L+S-1-k) cells.
 *   diag_ptr  host int32 [L+S]: diag_ptr[0] = 0, diag_ptr[k+1] - diag_ptr[k]
 *             cells in diagonal k, diag_ptr[L+S-1] = L*S.
 *   cells     host int32 [L*S][3]: (layer, segment, slot), slot = position
 *             of the cell within its diagonal.
 * Both pointers NULL: size query only.  Returns the number of diagonals
 * (L+S-1) on success, RMT_EINVAL if L < 1, S < 1, L*S overflows int32 or
 * exactly one pointer is NULL. */
int32_t rmt_diag_schedule(int32_t L, int32_t S, int32_t* diag_ptr, int32_t* cells);

/* Create a model handle: validates `cfg` and the presence of the weights the
 * cell needs, records the weight pointers (borrowed) and the stream later
 * device work is queued on (a hipStream_t; NULL = the default stream), and
 * sets *out.  Allocates only the host-side handle: no device memory and no
 * device work (both come with rmt_model_bind).
 * Errors: RMT_EINVAL (bad sizes or NULL weights the cell needs),
 * RMT_EUNSUPPORTED (Hq/Hkv not 1, 2 or a multiple of 4, an ENCODER with
 * n_kv_heads != n_heads, hd not 64/128, widths not multiples of 64, a LLAMA
 * cell whose m is not a multiple of 8 -- its QKV product reads the memory
 * rows and the segment rows from separate buffers in whole 8-row loads --,
 * ...). */
int32_t rmt_model_create(const rmt_config* cfg, const rmt_weights* w, void* stream,
                         rmt_model** out);

/* Caller-owned device buffers of a model.
 *   RMT_BUF_WEIGHTS    the packed weights ([L][N][K] bf16, K contiguous; for
 *                      128-wide heads the Q and K rows of each head are
 *                      grouped by RoPE rotation pair, which leaves the
 *                      attention unchanged),
 *                      gains, shifts and biases, the RoPE table and the
 *                      bad-token flag: fixed by the config, independent of S
 *                      and of the batch.
 *   RMT_BUF_WORKSPACE  the activations: per-launch buffers for up to
 *                      min(32, B L) cells (normalised rows, Q/K/V, attention
 *                      output, H, U), the X ping-pong pair of every sequence
 *                      and a second memory buffer [B][L][m][d]; for LLAMA
 *                      cells also the inputs of the RMSNorms that the rows'
 *                      producers prepare (16-bit copies y * gamma and sums of
 *                      y^2 over 64-column chunks, for every X slot, memory
 *                      row and H row) and the per-launch 1/rms rows.  Depends
 *                      on L, R, d, F and the batch B, not on S.
 * rmt_workspace_bytes writes the size in bytes that `kind` needs for the
 * model's current batch.  Errors: RMT_EINVAL. */
#define RMT_BUF_WEIGHTS 0
#define RMT_BUF_WORKSPACE 1
int32_t rmt_workspace_bytes(const rmt_model* model, int32_t kind, size_t* bytes);

/* Attach a caller-allocated device buffer (256-byte aligned, at least
 * rmt_workspace_bytes(kind) bytes) to the model; it is borrowed, must
 * outlive every call queued on it, and is never freed by the library.
 *   RMT_BUF_WEIGHTS: packs the weights recorded by rmt_model_create into the
 *     buffer on the model's stream and waits for the packing to finish (the
 *     mathematical-layout weights other than `embed` may be freed after
 *     this returns).  Bound once per model.
 *   RMT_BUF_WORKSPACE: the activation workspace; may be re-bound at any time
 *     (calls already queued keep using the previous buffer).  Its contents
 *     need no initialisation: every forward call writes each workspace byte
 *     it reads.
 * Errors: RMT_EINVAL (NULL model or buffer, misaligned buffer, bad kind,
 * weights bound twice), RMT_EWORKSPACE (buffer too small), RMT_EHIP. */
int32_t rmt_model_bind(rmt_model* model, int32_t kind, void* buffer, size_t bytes);

/* Re-target the model to S whole segments (T = S*n tokens) per forward call
 * (no allocation). */
int32_t rmt_model_set_segments(rmt_model* model, int32_t S);

/* Re-target the model to T >= 1 tokens per sequence and forward call (no
 * allocation): S = ceil(T / n) segments, the last of n' = T - (S-1) n rows
 * when T is not a multiple of n (the skill page's Implementation sketch
 * rounds the segment count up).  A short segment's cells have m + n' rows;
 * their first n' output rows become X(l, S-1) and the last m become
 * M(l, S-1), as for every other cell; they run in launches of their own.
 * The forward calls' token, input-row and hidden buffers then hold T rows per
 * sequence.  Errors: RMT_EINVAL (NULL model, T < 1, T too large). */
int32_t rmt_model_set_tokens(rmt_model* model, int64_t T);

/* Process B >= 1 independent sequences per forward call (default 1): the
 * batch dimension of the skill page's Implementation sketch.  Every diagonal
 * then covers the cells of all B sequences -- layer-major, sequence fastest,
 * in launches of at most 32 cells -- so B sequences fill the ramp diagonals
 * that one sequence leaves short of L cells.  The forward calls' buffers gain
 * a leading [B]: tokens [B][T] (or [B][T][d]), mem0 and out->mem
 * [B][L][m][d], out->hidden [B][T][d]; sequence b's results equal a B = 1
 * run on its inputs, bit for bit.  Allocates nothing: the workspace a batch
 * needs grows with B (rmt_workspace_bytes), and a bound workspace too small
 * for the new B must be replaced (rmt_model_bind) before the next forward
 * call, which otherwise returns RMT_EWORKSPACE.
 * Errors: RMT_EINVAL (NULL model, B < 1, sizes too large). */
int32_t rmt_model_set_batch(rmt_model* model, int32_t B);

/* Queue later forward calls on `stream` (a hipStream_t). */
int32_t rmt_model_set_stream(rmt_model* model, void* stream);

/* Bytes of the caller's device buffers bound to the model (weights +
 * workspace). */
int32_t rmt_model_device_bytes(const rmt_model* model, size_t* bytes);

/* Diagonal-batched forward pass over B sequences (rmt_model_set_batch;
 * B = 1 unless set) of T tokens each (T = S*n unless rmt_model_set_tokens
 * set another length).
 *   tokens  device: LLAMA -> int32 token ids [B][T] in [0, V) (ids outside
 *           that range read a zero embedding row and set the flag reported
 *           by rmt_model_check); other cells -> input rows X(-1, .)
 *           [B][T][d] (fp32 for RMT_F32 models, bf16 for RMT_BF16 models).
 *   mem0    device fp32 [B][L][m][d]: M(l, -1) of each sequence.
 *   out     see rmt_output (hidden [B][S*n][d], mem [B][L][m][d]).
 * For every diagonal k the library launches, on the model's stream, one
 * grouped kernel per stage covering all of the diagonal's cells (skill page,
 * Architecture Overview: GroupedGEMM Operations, GPU Kernel Optimization).
 * Asynchronous.  Errors: RMT_EINVAL (NULL pointers), RMT_EWORKSPACE (no
 * weight buffer bound, or no workspace large enough for the batch), RMT_EHIP. */
int32_t rmt_forward_diagonal(rmt_model* model, const void* tokens, const void* mem0,
                             rmt_output* out);

/* rmt_forward_diagonal for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same arguments, the same kernels and bitwise the same
 * results, but the activation workspace is the library's own static device
 * array of 64 MiB (per device, held until the process ends) instead of the
 * buffer bound with RMT_BUF_WORKSPACE, which this call neither needs nor
 * touches.  The weight buffer must be bound as for rmt_forward_diagonal.
 * The call allocates nothing and records no timing events.  Calls that
 * overlap on one device share that array and race: serialise them (for
 * example on one stream).  The array's contents carry over from call to
 * call; every call writes each workspace byte before reading it.
 * Errors: RMT_EINVAL (NULL pointers), RMT_EWORKSPACE (no weight buffer
 * bound, or rmt_workspace_bytes(RMT_BUF_WORKSPACE) above 64 MiB for the
 * current batch -- checked before any device call), RMT_EHIP. */
int32_t rmt_forward_diagonal_static(rmt_model* model, const void* tokens, const void* mem0,
                                    rmt_output* out);

/* The same computation cell by cell, segment-major (for b: for s: for l:),
 * one cell per launch: the sequential RMT schedule that the abstract of the
 * catalogue record compares diagonal batching against.  Same arguments and
 * results; bitwise equal to rmt_forward_diagonal. */
int32_t rmt_forward_sequential(rmt_model* model, const void* tokens, const void* mem0,
                               rmt_output* out);

/* Synchronise the model's stream and report whether any forward call since
 * the last check read a token id outside [0, V): *bad_tokens = 0 or 1. */
int32_t rmt_model_check(rmt_model* model, int32_t* bad_tokens);

/* Per-stage GPU timing.  When enabled, forward calls record a HIP event on
 * the model's stream after every launch (and one before the first), so the
 * time between consecutive events is one launch's duration on the stream.
 * rmt_model_stage_times synchronises the stream and returns, for each stage
 * (RMT_STAGE_*; for ENCODER cells NORM1/NORM2 are the LayerNorms -- with
 * post_norm, NORM1 is the bf16 copy of A and NORM2 both LayerNorms -- and
 * GATEUP/DOWN the feed-forward's W1 and W2 products), the summed milliseconds, the number of launches, and the
 * algorithmic flops and HBM bytes of those launches (compulsory operand and
 * result traffic, no re-reads), then clears the totals.  Host arrays of
 * RMT_NUM_STAGES entries; any of them may be NULL. */
#define RMT_STAGE_GATHER 0
#define RMT_STAGE_NORM1 1
#define RMT_STAGE_QKV 2
#define RMT_STAGE_ATTN 3
#define RMT_STAGE_OPROJ 4
#define RMT_STAGE_NORM2 5
#define RMT_STAGE_GATEUP 6
#define RMT_STAGE_DOWN 7
#define RMT_STAGE_LINEAR 8
#define RMT_NUM_STAGES 9
int32_t rmt_model_enable_timing(rmt_model* model, int32_t enable);
int32_t rmt_model_stage_times(rmt_model* model, double* ms, int64_t* launches, double* flops,
                              double* bytes);

/* The same per-stage totals restricted to the launches that covered between
 * g_lo and g_hi cells (inclusive) -- e.g. g_lo = g_hi = min(L, S) selects the
 * full diagonals, 1 .. min(L, S) - 1 the ramps of the "Diagonal
 * Reorganization" sweep in the Architecture Overview of the skill page.  The
 * one-off copy of mem0 counts as 0 cells.  Synchronises the stream; does not
 * clear the totals (call rmt_model_stage_times for that).  Errors: RMT_EINVAL
 * (NULL model, g_lo > g_hi), RMT_EHIP. */
int32_t rmt_model_stage_times_groups(rmt_model* model, int32_t g_lo, int32_t g_hi, double* ms,
                                     int64_t* launches, double* flops, double* bytes);

/* Release the handle (the model's stream is synchronised first).  The bound
 * buffers are the caller's and are left as they are.  NULL is accepted. */
int32_t rmt_model_destroy(rmt_model* model);

/* Pack mathematical-layout weights src [L][K][N] (fp32 or bf16 per
 * `src_dtype`, device) into the library's GEMM layout dst [L][N][K] bf16
 * (device, caller-allocated, L*N*K*2 bytes), on `stream`.  K and N must be
 * multiples of 8. */
int32_t rmt_pack_weight(int32_t L, int32_t K, int32_t N, const void* src, int32_t src_dtype,
                        void* dst, void* stream);

/* The grouped GEMM on its own (Architecture Overview: GroupedGEMM Operations):
 * C_g = A_g B_{layer[g]} for g < G, in one launch, MFMA with fp32
 * accumulation, result rounded to nearest even.
 *   A           device [G][M][K]
 *   B           device [Lw][N][K] as produced by rmt_pack_weight
 *   group_layer host int32 [G], each in [0, Lw)
 *   C           device [G][M][N]
 *   dtype       element type of A, B and C: RMT_BF16 or RMT_F16
 * 1 <= G <= 32 per call, K a multiple of 8, N a multiple of 64.
 * Errors: RMT_EINVAL (sizes, NULL pointers, a layer index outside [0, Lw)),
 * RMT_EUNSUPPORTED (dtype), RMT_EHIP. */
int32_t rmt_grouped_gemm(int32_t G, int32_t M, int32_t N, int32_t K, int32_t Lw, const void* A,
                         const void* B, const int32_t* group_layer, void* C, int32_t dtype,
                         void* stream);

/* Causal grouped-query attention on its own, over G cells of R rows each, in
 * one launch (the attention stage of the LLAMA cell; see the cell kinds
 * above): for query head h and row i of cell g,
 *   out[g][i][h*hd : (h+1)*hd] = sum_{j <= i} softmax_j(q_i . k_j / sqrt(hd)) v_j
 * with k, v from KV head h / (Hq/Hkv), softmax in fp32, bf16 output.
 *   qkv  device bf16 [G][R][(Hq+2Hkv)*hd]: per row the Q heads, then the K
 *        heads, then the V heads (RoPE, if any, already applied)
 *   out  device bf16 [G][R][Hq*hd]
 * 1 <= G <= 65535, R >= 1, hd in {64, 128}, Hq/Hkv 1, 2 or a positive
 * multiple of 4; one cell's qkv rows, R * (Hq+2Hkv) * hd * 2 bytes, below
 * 2 GiB (RMT_EINVAL otherwise).
 * Errors: RMT_EINVAL, RMT_EUNSUPPORTED (hd or head ratio), RMT_EHIP. */
int32_t rmt_causal_attention(int32_t G, int32_t R, int32_t n_heads, int32_t n_kv_heads,
                             int32_t head_dim, const void* qkv, void* out, void* stream);

/* Attention on its own, causal or not (causal != 0: the LLAMA cell's stage,
 * as rmt_causal_attention; causal == 0: the ENCODER cell's, every row
 * attending to all R rows of its cell), same layouts and types as
 * rmt_causal_attention.  Hq/Hkv must be 1, 2 or a positive multiple of 4.
 * Errors: RMT_EINVAL, RMT_EUNSUPPORTED (hd or head ratio), RMT_EHIP. */
int32_t rmt_attention(int32_t G, int32_t R, int32_t n_heads, int32_t n_kv_heads,
                      int32_t head_dim, int32_t causal, const void* qkv, void* out, void* stream);

/* Thread-local description of the last error (empty string if none). */
const char* rmt_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* RMT_H */
