/*
 * td.h -- C ABI of the block-diffusion denoise step for AMD MI355X (gfx950).
 *
 * One denoising step of the TwoTower diffusion denoiser, as described on the
 * news pages about NVIDIA's Nemotron-Labs-TwoTower:
 *   - news.chathome.org, "NVIDIA releases Nemotron-Labs-TwoTower: an
 *     open-weight diffusion language model built on a frozen autoregressive
 *     backbone": inference paragraph (the denoiser attends bidirectionally
 *     inside its block and, layer by layer, to the context tower's per-layer
 *     KV cache of the prompt and committed tokens); block-generation
 *     paragraph (a block of S [MASK] tokens is refined step by step and
 *     several tokens may commit per step); evaluation paragraph (confidence
 *     masking with threshold gamma = 0.8, block size S = 16).
 *   - aiboss88.com, "Nemotron-Labs-TwoTower", technical-principle section
 *     (bidirectional block attention plus cross-attention to the context
 *     tower).
 *
 * Conventions shared by every entry point
 *   Memory     Every data pointer is DEVICE memory owned by the caller.  The
 *              library never allocates, frees or keeps a pointer after a call
 *              returns; scratch space is the caller's workspace, sized by the
 *              *_workspace_bytes queries.  The library keeps no mutable
 *              global state, so calls on different streams may run at once
 *              as long as they use different workspaces.
 *   Streams    Work is enqueued in order on the caller's stream (a
 *              hipStream_t passed as td_stream_t; NULL = the null stream).
 *              The library never synchronises; outputs are valid once the
 *              stream has executed the work.
 *   Errors     All arguments are checked on the host before anything is
 *              enqueued: a non-zero return means nothing was enqueued and no
 *              output was written.  TD_ERR_HIP reports a launch failure seen
 *              right after enqueueing (outputs then undefined).  The device
 *              offsets array cannot be checked on the host; the kernels
 *              clamp every row index to [0, total_ctx), so inconsistent
 *              offsets give unspecified values but never an out-of-bounds
 *              access.
 *   Layouts    Row-major, innermost index last, no padding.
 *   Results    Deterministic: the same inputs give bitwise-identical outputs
 *              (no floating-point atomics; partials merged in a fixed order).
 *   Environment  Three variables override the launch plan, for testing the
 *              work split; results stay correct under any, only the speed
 *              changes:
 *                TD_ATTN_GRID=n     persistent attention workgroups (1..4096,
 *                                   default 256);
 *                TD_DECODE_GRID=n   workgroups of 4 waves of the decode-shaped
 *                                   attention (at most 16 query rows per KV
 *                                   head; 1..4096, default up to 256);
 *                TD_COMMIT_SPLIT=r  vocabulary slices per commit row.
 *              The two grids also set the attention workspace size, so set
 *              them before the workspace query.
 */
#ifndef TD_H
#define TD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TD_ABI_VERSION 2u

typedef enum {
  TD_OK = 0,
  TD_ERR_INVALID = -1,      /* a null pointer, a bad size or a bad value    */
  TD_ERR_UNSUPPORTED = -2,  /* valid but not implemented (e.g. D = 96)      */
  TD_ERR_WORKSPACE = -3,    /* ws too small or misaligned (256 B required)  */
  TD_ERR_HIP = -4           /* the HIP runtime reported a launch failure    */
} td_status;

typedef enum { TD_F32 = 0, TD_BF16 = 1 } td_dtype;

typedef void *td_stream_t;  /* a hipStream_t */

/*
 * Block attention of one denoiser attention layer (chathome, inference
 * paragraph; aiboss, technical principle).  For sequence b and query head h,
 * with KV head g = h / (Hq/Hkv):
 *   K = [k_ctx rows off[b] .. off[b+1]-1, head g ; k_blk[b, 0..S-1, g]]
 *   V = the same rows of v_ctx / v_blk
 *   out[b, :, h] = softmax(scale * q[b, :, h] K^T over all L_b + S keys) V
 * One softmax covers the cached context and the block: bidirectional inside
 * the block, every cached key visible, no mask.
 */
typedef struct {
  int32_t B;               /* sequences (blocks) in the batch, >= 1            */
  int32_t S;               /* block size, 1 .. 64                              */
  int32_t Hq, Hkv;         /* query / KV heads, Hq % Hkv == 0, Hq/Hkv <= 64    */
  int32_t D;               /* head dim.  bf16: 128 (the MFMA kernels).  fp32:
                              64 or 128, on a plain one-thread-per-query-row
                              kernel meant for small problems.  Any other
                              value: TD_ERR_UNSUPPORTED                      */
  td_dtype dtype;          /* dtype of q, k_*, v_*, out (one per call)         */
  float scale;             /* softmax scale; <= 0 selects 1/sqrt(D)            */
  const void *q;           /* [B, S, Hq, D]                                    */
  const void *k_blk;       /* [B, S, Hkv, D]  block keys                       */
  const void *v_blk;       /* [B, S, Hkv, D]  block values                     */
  const void *k_ctx;       /* [total_ctx, Hkv, D] context keys, packed per seq */
  const void *v_ctx;       /* [total_ctx, Hkv, D] context values               */
  const int64_t *ctx_offsets; /* DEVICE [B+1]: off[0] = 0, non-decreasing,
                                 off[B] = total_ctx; L_b = off[b+1]-off[b] >= 0 */
  int64_t total_ctx;       /* HOST copy of off[B]                              */
  int64_t max_ctx;         /* HOST copy of max_b L_b (sizes the launch grid)   */
  void *out;               /* [B, S, Hq, D], dtype as q; may not alias inputs  */
} td_attn_args;

/*
 * Confidence-masked commit of one block step (chathome, evaluation and
 * block-generation paragraphs).  For every position (b, i):
 *   token[b,i]   = lowest id j with logits[b,i,j] == max_j logits[b,i,j]
 *   maxprob[b,i] = 1 / sum_j exp(logits[b,i,j] - max)   (largest softmax prob.)
 * Per sequence b, with E = {i : masked_in[b,i] != 0}:
 *   C = {i in E : maxprob[b,i] >= gamma};  if C is empty and E is not,
 *   C = {the i in E with the largest maxprob, lowest i on ties}.
 *   commit[b,i] = (i in C); n_commit[b] = |C|
 *   masked_out[b,i] = masked_in[b,i] && !commit[b,i]
 *   tokens[b,i] = token[b,i] where commit[b,i], unchanged elsewhere
 *   *n_masked_left = number of nonzero masked_out over the whole batch
 * maxprob is computed in fp32 (relative error ~1e-6); gamma is compared as
 * the fp32 value given.
 */
typedef struct {
  int32_t B;               /* >= 1                                             */
  int32_t S;               /* 1 .. 64                                          */
  int32_t V;               /* vocabulary size, >= 1                            */
  td_dtype dtype;          /* dtype of logits                                  */
  float gamma;             /* confidence threshold, finite                     */
  const void *logits;      /* [B, S, V]                                        */
  const uint8_t *masked_in;/* [B, S] 1 = still [MASK] (eligible); NULL = all   */
  uint8_t *commit;         /* out [B, S]  1 = committed by this step           */
  int32_t *token;          /* out [B, S]  argmax id at EVERY position          */
  float *maxprob;          /* out [B, S] or NULL                               */
  int32_t *n_commit;       /* out [B] or NULL                                  */
  uint8_t *masked_out;     /* out [B, S] or NULL; may alias masked_in          */
  int32_t *tokens;         /* in/out [B, S] or NULL: ids written where committed */
  int32_t *n_masked_left;  /* out [1] or NULL                                  */
} td_commit_args;

/*
 * Context-cache append after a block has committed (chathome, block-generation
 * paragraph: once a block's positions have all committed, the context tower
 * takes in the committed tokens and its per-layer KV cache grows by them, so
 * the next block attends to them as context).  One attention layer's cache:
 * for every sequence b, with L_b = off[b+1] - off[b],
 *   off_out[b]         = off[b] + b*S                       (b = 0..B)
 *   k_out[off_out[b] + j] = k_ctx[off[b] + j]   for j < L_b   (old rows)
 *   k_out[off_out[b] + L_b + s] = k_new[b, s]   for s < S     (new rows)
 * and the same for v_out from v_ctx / v_new.  The cache is packed, so the
 * append is a copy into a second cache (callers alternate two buffers);
 * k_out and off_out are the next block's k_ctx and ctx_offsets, and the
 * next block's max_ctx is the old one plus S.
 */
typedef struct {
  int32_t B;               /* sequences, >= 1                                  */
  int32_t S;               /* rows appended per sequence, 0 .. 65536           */
  int32_t Hkv, D;          /* >= 1; a row, Hkv*D elements, must be a multiple of
                              16 bytes (TD_ERR_UNSUPPORTED otherwise)          */
  td_dtype dtype;          /* element type of every K/V array (copied bitwise) */
  const void *k_ctx;       /* [total_ctx, Hkv, D] cached keys, packed per seq  */
  const void *v_ctx;       /* [total_ctx, Hkv, D] cached values                */
  const int64_t *ctx_offsets; /* DEVICE [B+1]: as in td_attn_args            */
  int64_t total_ctx;       /* HOST copy of off[B]                              */
  const void *k_new;       /* [B, S, Hkv, D] the committed tokens' keys (from
                              the context tower); NULL allowed when S == 0     */
  const void *v_new;       /* [B, S, Hkv, D] their values                      */
  void *k_out;             /* out [total_ctx + B*S, Hkv, D]                    */
  void *v_out;             /* out [total_ctx + B*S, Hkv, D]                    */
  int64_t *offsets_out;    /* out DEVICE [B+1]                                 */
} td_append_args;

/*
 * LM head of the block positions fused with the commit (chathome,
 * block-generation and evaluation paragraphs: each denoising step scores the
 * vocabulary at every block position, then commits by confidence).  For
 * every position (b, i):
 *   logits[b,i,j] = sum_k hidden[b,i,k] * w_head[j,k]     (j = 0 .. V-1)
 * computed in fp32 from bf16 operands and never written to memory; then the
 * commit of td_commit_args over those logits (same outputs, same rules:
 * token = lowest argmax, maxprob = 1 / sum_j exp(logits - max), threshold
 * p >= gamma on the eligible positions, force-one).
 * Only eligible positions are scored: with masked_in given, the positions
 * whose masked_in is 0 (already committed) are left out of the product, and
 * their token is -1 and maxprob 0.  In a block's step loop the work so
 * shrinks with the number of positions still masked.
 */
typedef struct {
  int32_t B;               /* >= 1                                             */
  int32_t S;               /* 1 .. 64                                          */
  int32_t H;               /* hidden size: a multiple of 64, 64 .. 65536       */
  int32_t V;               /* vocabulary size, 1 .. 2^30                       */
  td_dtype dtype;          /* TD_BF16 (TD_ERR_UNSUPPORTED otherwise)           */
  float gamma;             /* confidence threshold, finite                     */
  const void *hidden;      /* [B, S, H] final hidden state of each position    */
  const void *w_head;      /* [V, H] LM-head weight, row j = token j, or its
                              packed copy (w_head_packed = 1)                  */
  const uint8_t *masked_in;/* [B, S] 1 = still [MASK] (eligible); NULL = all   */
  uint8_t *commit;         /* out [B, S]                                       */
  int32_t *token;          /* out [B, S]  argmax id at every eligible position,
                              -1 at the others                                 */
  float *maxprob;          /* out [B, S] or NULL (0 at ineligible positions)   */
  int32_t *n_commit;       /* out [B] or NULL                                  */
  uint8_t *masked_out;     /* out [B, S] or NULL; may alias masked_in          */
  int32_t *tokens;         /* in/out [B, S] or NULL: ids written where committed */
  int32_t *n_masked_left;  /* out [1] or NULL                                  */
  int32_t w_head_packed;   /* 0: w_head is [V, H] row-major; 1: w_head is the
                              packed copy td_lmhead_pack_head wrote            */
} td_lmhead_args;

/*
 * State-space core of one denoiser Mamba-2 layer over the block, its state
 * seeded from the context tower (chathome, inference paragraph: the
 * denoiser's Mamba-2 layers start from the context tower's state).  The
 * recurrence is Mamba-2's selective scan with one decay rate per head; for
 * sequence b, head h (group g = h / (H/G)) and tokens t = 0 .. S-1:
 *   st <- exp(dt[b,t,h] * A[h]) * st + dt[b,t,h] * x[b,t,h,:] (outer) Bm[b,t,g,:]
 *   y[b,t,h,:] = st . Cm[b,t,g,:] + D[h] * x[b,t,h,:]
 * with st = h0[b,h] before the first token.  Computed in fp32; y rounded to
 * bf16.  The state after the block is not returned (on the denoise path the
 * context tower recomputes it from the committed tokens).
 */
typedef struct {
  int32_t B;               /* sequences, >= 1                                  */
  int32_t S;               /* block tokens, 1 .. 16                            */
  int32_t H;               /* SSM heads, >= 1, a multiple of G                 */
  int32_t P;               /* head dim: 16, 32, 64 or 128                      */
  int32_t N;               /* state size: a multiple of 32, 32 .. 1024         */
  int32_t G;               /* groups of Bm / Cm, >= 1                          */
  const void *x;           /* [B, S, H, P] bf16                                */
  const float *dt;         /* [B, S, H] step sizes                             */
  const float *A;          /* [H] decay rates (negative)                       */
  const void *Bm;          /* [B, S, G, N] bf16 input projections              */
  const void *Cm;          /* [B, S, G, N] bf16 output projections             */
  const float *D;          /* [H] skip weights                                 */
  const float *h0;         /* [B, H, P, N] fp32 seed state                     */
  void *y;                 /* out [B, S, H, P] bf16                            */
} td_mamba_args;

/*
 * adaLN-single time conditioning between two denoiser layers (chathome,
 * inference paragraph: the diffusion timestep modulates every layer through
 * adaLN-single, about 1.5M parameters).  Read as PixArt-alpha's adaLN-single:
 * a projection of the timestep shared by all layers gives each sequence three
 * vectors (t_mod rows 0, 1, 2 = shift, scale, gate) and each layer adds its
 * own learned [3, H] table.  Layer l's output f joins the residual stream
 * through layer l's gate, and layer l+1 reads the RMS-normalised stream under
 * its own shift and scale; for sequence b and token s:
 *   r[b,s,:] = x[b,s,:] + (t_mod[b,2,:] + tab_gate) * f[b,s,:]   (x when f is NULL)
 *   h[b,s,:] = r[b,s,:] / sqrt(mean_j r[b,s,j]^2 + eps) * w_norm
 *                * (1 + t_mod[b,1,:] + tab_scale) + (t_mod[b,0,:] + tab_shift)
 * Computed in fp32.  r is rounded to bf16 and h is computed from the rounded
 * r (the stream is stored in bf16 between layers); h is rounded to bf16.
 */
typedef struct {
  int32_t B;               /* sequences, >= 0                                  */
  int32_t S;               /* tokens per sequence, >= 0                        */
  int32_t H;               /* hidden size, a multiple of 8, 8 .. 8192          */
  float eps;               /* RMSNorm epsilon, finite, >= 0                    */
  const void *x;           /* [B, S, H] bf16 residual stream                   */
  const void *f;           /* [B, S, H] bf16 output of layer l, or NULL        */
  const float *t_mod;      /* [B, 3, H] shared timestep vectors: shift, scale, gate */
  const float *tab_gate;   /* [H] layer l's gate row, or NULL (zeros)          */
  const float *tab_shift;  /* [H] layer l+1's shift row, or NULL (zeros)       */
  const float *tab_scale;  /* [H] layer l+1's scale row, or NULL (zeros)       */
  const float *w_norm;     /* [H] layer l+1's RMSNorm weight, or NULL (ones)   */
  void *r_out;             /* out [B, S, H] bf16 r; required when f is given,
                              unused otherwise; may be x itself               */
  void *h;                 /* out [B, S, H] bf16 input of layer l+1; may be x
                              or f itself                                      */
} td_adaln_args;

/* Library identity and struct sizes, for bindings to check their layout. */
uint32_t td_abi_version(void);
size_t td_sizeof_attn_args(void);
size_t td_sizeof_commit_args(void);
size_t td_sizeof_append_args(void);
size_t td_sizeof_lmhead_args(void);
size_t td_sizeof_mamba_args(void);
size_t td_sizeof_adaln_args(void);
const char *td_status_str(int status);

/* Workspace each call needs, in bytes (0 when none).  Pure host functions:
 * they validate the arguments' sizes (not pointers) and return 0 on invalid
 * sizes; pass a workspace of at least this many bytes, 256-byte aligned. */
size_t td_attn_workspace_bytes(const td_attn_args *a);
size_t td_commit_workspace_bytes(const td_commit_args *c);
size_t td_denoise_workspace_bytes(const td_attn_args *a, const td_commit_args *c);
size_t td_lmhead_commit_workspace_bytes(const td_lmhead_args *a);

/* Block attention (see td_attn_args).  Returns a td_status. */
int td_block_attn(const td_attn_args *a, void *ws, size_t ws_bytes, td_stream_t stream);

/* Confidence-masked commit (see td_commit_args).  Returns a td_status. */
int td_commit(const td_commit_args *c, void *ws, size_t ws_bytes, td_stream_t stream);

/* One denoise step: the block attention of one denoiser attention layer and
 * the commit of the block's logits, both enqueued on `stream`.  The logits
 * are an input: the layers between this attention and the LM head are not
 * part of this library.  a->B must equal c->B and a->S must equal c->S.
 * One workspace of td_denoise_workspace_bytes() serves both parts. */
int td_denoise_step(const td_attn_args *a, const td_commit_args *c, void *ws,
                    size_t ws_bytes, td_stream_t stream);

/* td_denoise_step gated by a device value, so that a block's whole step loop
 * (chathome, block-generation paragraph: a block is refined step by step
 * until every position has committed) can be enqueued with no host
 * synchronisation.  `gate` is a DEVICE int32 that every kernel of the step
 * reads first:
 *   *gate != 0  the step runs exactly as td_denoise_step;
 *   *gate == 0  the step does nothing, except that c->n_masked_left (if not
 *               NULL) is set to 0; no other output is written.
 * Passing the previous step's n_masked_left as the gate runs the steps while
 * positions remain masked and turns the rest into no-ops; since each step
 * commits at least one position per unfinished block, S such steps always
 * suffice.  The gate must not be this step's own c->n_masked_left (two
 * counters used alternately are the usual pattern).
 * Returns TD_ERR_INVALID for a NULL gate or one equal to c->n_masked_left;
 * otherwise as td_denoise_step. */
int td_denoise_step_if(const td_attn_args *a, const td_commit_args *c, const int32_t *gate,
                       void *ws, size_t ws_bytes, td_stream_t stream);

/* td_denoise_step with no workspace argument, for callers that cannot
 * allocate device memory while they run: code under stream capture, tight
 * serving loops, harnesses that forbid hipMalloc.  Its scratch is a
 * library-held device array of TD_NOALLOC_SCRATCH_BYTES bytes per GPU,
 * reserved when the library is loaded and held until the process ends; the
 * call itself allocates and frees nothing.  Results are those of
 * td_denoise_step with a workspace, bit for bit.
 * Limit: a call whose td_denoise_workspace_bytes() exceeds
 * TD_NOALLOC_SCRATCH_BYTES returns TD_ERR_WORKSPACE.  With the default
 * launch plan, blocks of more than 16 query rows per KV head need 33 to 50
 * MiB whatever the batch; decode-shaped blocks (at most 16 query rows per KV
 * head) need at most about 9 MiB plus 8 bytes per sequence, whatever the
 * context lengths.  A TD_ATTN_GRID or TD_DECODE_GRID override well above
 * the default is rejected.
 * Every call on one GPU shares that GPU's array: calls that may overlap on
 * one GPU (different streams, or different threads without ordering) race
 * on it and must not be made.  Nothing in the array needs clearing between
 * calls.  Otherwise as td_denoise_step: same validation and return codes;
 * TD_ERR_HIP also if the array's device address cannot be looked up. */
#define TD_NOALLOC_SCRATCH_BYTES (64u * 1024u * 1024u)
int td_denoise_step_noalloc(const td_attn_args *a, const td_commit_args *c, td_stream_t stream);

/* Fused LM head + commit (see td_lmhead_args).  hidden and w_head must be
 * 16-byte aligned, and B*S*H*2 below 2^32.  The workspace
 * (td_lmhead_commit_workspace_bytes) holds 16 bytes per (position, 256-token
 * slice of the vocabulary), 16 per position and the list of eligible
 * positions.  Returns a td_status. */
int td_lmhead_commit(const td_lmhead_args *a, void *ws, size_t ws_bytes, td_stream_t stream);

/* The LM-head weight rearranged once (at load time) for td_lmhead_commit:
 * [ceil(V/256)][H/64][256][64] bf16, i.e. for every 256-token slice of the
 * vocabulary and every 64-wide slice of the hidden size, the 256 x 64 block
 * td_lmhead_commit streams as one pipeline stage, stored contiguously (32 KiB);
 * rows past V are zero.  The result is the same bit for bit as with the
 * row-major weight, and each stage is read as one contiguous block.
 * td_lmhead_packed_bytes returns the packed size, ceil(V/256)*256*H*2 bytes
 * (0 for an invalid V or H).  td_lmhead_pack_head validates (H a multiple of
 * 64, 64 .. 65536; 1 <= V <= 2^30; both pointers 16-byte aligned and not
 * overlapping: TD_ERR_INVALID / TD_ERR_UNSUPPORTED) and enqueues the copy on
 * `stream`.  Returns a td_status. */
size_t td_lmhead_packed_bytes(int32_t V, int32_t H);
int td_lmhead_pack_head(const void *w_head, int32_t V, int32_t H, void *w_packed,
                        td_stream_t stream);

/* Mamba-2 block scan (see td_mamba_args).  Needs no workspace.  x, Bm, Cm
 * and h0 must be 16-byte aligned, y 8-byte aligned.  Returns a td_status. */
int td_mamba_block_scan(const td_mamba_args *a, td_stream_t stream);

/* adaLN-single modulation (see td_adaln_args).  Needs no workspace.  Every
 * pointer must be 16-byte aligned.  An output may be the same pointer as an
 * input, as stated above, but may not otherwise overlap an input, and r_out
 * and h may not overlap: checked on the host (TD_ERR_INVALID).  B*S = 0 is
 * valid and enqueues nothing.  Returns a td_status. */
int td_adaln_modulate(const td_adaln_args *a, td_stream_t stream);

/* Context-cache append (see td_append_args).  Needs no workspace.  Every
 * data pointer must be 16-byte aligned; no output may overlap an input or the
 * other output (k_out/v_out/offsets_out against k_ctx, v_ctx, k_new, v_new,
 * ctx_offsets): the ranges are checked on the host and TD_ERR_INVALID is
 * returned for an overlap, a misaligned or missing pointer or a bad size.
 * Each output row is written exactly once, so inconsistent device offsets give
 * unspecified values but never an access out of bounds.  Returns a
 * td_status. */
int td_cache_append(const td_append_args *p, td_stream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* TD_H */
