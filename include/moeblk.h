/*
 * moeblk.h -- C ABI of the local-expert MoE block for AMD MI355X (gfx950).
 *
 * One GPU's share of an expert-parallel MoE layer in a spec-verify decode step:
 * S token rows (1..128, all valid) are routed over E experts with sigmoid
 * top-k; the picks that land on this GPU's n_local experts run through MXFP4
 * gate_up -> SwiGLU -> MXFP4 down, each expert output is RMS-normalised, and
 * the routing-weighted sum is written as this GPU's fp32 partial.
 *
 * Sources (vLLM API pages):
 *   - Muse Spark K3 page (vllm.models.muse_spark.amd.mono.kernels.k3), module
 *     docstring, stages "A" (fp32 router logits), "route" (every token's top-8,
 *     the local experts' picks), "C, D" (MXFP4 gate_up / down decoded in
 *     registers, bf16 MFMA), "E" (per-pick post-expert norm and weighted sum
 *     into the expert-parallel partial); functions "mx_chunk", "fp4_mma",
 *     "dn_loads" (MXFP4 rows in 256-K chunks with e8m0 scales; the
 *     active-expert table).
 *   - Muse Spark K5 page (vllm.models.muse_spark.amd.mono.kernels.k5), module
 *     docstring: the HA routing tail hands top-k ids and weights to HM, the
 *     local-expert launch; every row tile is 16 tokens.
 *   - Kimi-K3 layer page (...specialized_decode.mono.layer), "k2_launch": router
 *     weight plus bias, MoE weights as separate value / scale tensors, shared
 *     expert gate_up / down weights, caller-provided scratch.
 *
 * Conventions (every entry point):
 *   - All pointers are device pointers unless stated otherwise, caller-owned,
 *     16-byte aligned, tensors contiguous row-major. The library never
 *     allocates or frees memory and never synchronises: work is enqueued on
 *     `stream` (NULL = the null stream) and the call returns.
 *   - bf16 tensors are passed as `const void*` (16-bit bf16 bit patterns).
 *   - Return value: MOE_OK, or a negative MOE_ERR_* code. Every argument check
 *     runs on the host before anything is enqueued, so a rejected call has no
 *     effect. MOE_ERR_HIP reports a failed launch (hipGetLastError).
 *   - Device data (ids, counts, ...) are trusted: they are not range-checked
 *     on the device beyond what each function states.
 *   - Calls on one stream run in order; the block is
 *       moe_route -> moe_bucket -> moe_expert_ffn -> moe_combine.
 */
#ifndef MOEBLK_H
#define MOEBLK_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOEBLK_ABI_VERSION 4 /* 2: moe_dims.bias_mode; 3: moe_route workspace;
                                4: moe_forward_static, moe_forward_one_launch */

/* status codes */
#define MOE_OK 0
#define MOE_ERR_NULL (-1)        /* a required pointer is NULL */
#define MOE_ERR_SHAPE (-2)       /* a size is out of range or inconsistent */
#define MOE_ERR_ALIGN (-3)       /* a pointer is not 16-byte aligned */
#define MOE_ERR_UNSUPPORTED (-4) /* a valid but unsupported parameter (which, renorm, ...) */
#define MOE_ERR_WORKSPACE (-5)   /* workspace smaller than moe_ffn_workspace_bytes() */
#define MOE_ERR_HIP (-6)         /* the HIP runtime reported an error */

/* weight selectors for the packing calls */
#define MOE_W13 0 /* gate_up: N = 2 I rows (rows [0, I) gate, [I, 2 I) up), K = d */
#define MOE_W2 1  /* down:    N = d rows, K = I */

/* Problem sizes, all in elements. Supported ranges:
 *   1 <= S <= 128; 128 <= d <= 16384, d % 128 == 0; 1 <= E <= 256;
 *   1 <= topk <= 8, topk <= E; 1 <= n_local <= 32;
 *   0 <= local_base, local_base + n_local <= E;
 *   128 <= I <= 8192, I % 128 == 0; renorm in {0, 1}; eps finite, >= 0;
 *   shared_I == 0 or (128 <= shared_I <= 8192, shared_I % 128 == 0);
 *   bias_mode in {0, 1}. */
typedef struct moe_dims {
  int32_t S;          /* token rows */
  int32_t d;          /* hidden size seen by the experts */
  int32_t E;          /* experts routed over (router rows) */
  int32_t topk;       /* picks per token */
  int32_t n_local;    /* experts held by this GPU */
  int32_t local_base; /* id of the first local expert; local ids are [local_base, local_base + n_local) */
  int32_t I;          /* expert intermediate size */
  int32_t renorm;     /* 1: w = sigmoid / sum of the token's topk sigmoids; 0: w = sigmoid */
  float eps;          /* post-expert RMSNorm epsilon */
  int32_t shared_I;   /* 0: no shared expert; else its intermediate size */
  int32_t bias_mode;  /* router bias: 0 part of the logit (ranking and sigmoid);
                         1 selection only (ranking key logit + bias, sigmoid of
                         the unbiased logit). The K3 page's "route_token"
                         summary breaks off after "sigmoid +", allowing both */
} moe_dims;

/* R_max = S * min(topk, n_local): the most local picks a call can have
 * (a token's picks are distinct experts). Bucket rows, h rows and routed y
 * rows are indexed 0 .. R_max - 1. */

int moe_abi_version(void);

/* A static English description of a status code. Never NULL. */
const char* moe_status_string(int status);

/* Host-only check of `dims` against the supported ranges: MOE_OK,
 * MOE_ERR_NULL, MOE_ERR_SHAPE or MOE_ERR_UNSUPPORTED. */
int moe_check_dims(const moe_dims* dims);

/* ------------------------------------------------------------------------ */
/* one-time weight packing (not part of the per-step path)                   */
/* ------------------------------------------------------------------------ */

/* Bytes of the packed MXFP4 weight `which` (MOE_W13 / MOE_W2) of all n_local
 * experts, or 0 if `dims` is invalid. Equals n_local * N * K * (1/2 + 1/32). */
size_t moe_packed_mxfp4_bytes(const moe_dims* dims, int which);

/* Repack canonical MXFP4 weights into the kernel's tile order (the role the
 * K3 page's "shuffled layouts" play: the same bytes, permuted so that each
 * wave load reads one contiguous 1 KiB).
 *   q      [n_local, N, K/2] uint8: two e2m1 codes a byte, element k of a row
 *          in byte k/2, the low nibble holding the even k;
 *   scales [n_local, N, K/32] uint8: e8m0 byte of elements 32 j .. 32 j + 31;
 *   packed [moe_packed_mxfp4_bytes(dims, which)] bytes, written.
 * The packed buffer is opaque: only moe_expert_ffn reads it. */
int moe_pack_mxfp4(const moe_dims* dims, int which, const void* q, const void* scales,
                   void* packed, hipStream_t stream);

/* The same for the shared expert's dense bf16 weights (needs shared_I > 0):
 * MOE_W13: ws13 [2 shared_I, d] (rows [0, shared_I) gate, then up);
 * MOE_W2:  ws2 [d, shared_I]. Packed size = N * K * 2 bytes. */
size_t moe_packed_bf16_bytes(const moe_dims* dims, int which);
int moe_pack_bf16(const moe_dims* dims, int which, const void* w, void* packed,
                  hipStream_t stream);

/* ------------------------------------------------------------------------ */
/* the block                                                                 */
/* ------------------------------------------------------------------------ */

/* Bytes of scratch moe_route needs: 0 for S <= 32; beyond, the router's
 * tiles split K into parts whose partial logits ([parts, S, E] fp32) the
 * top-k launch sums. 0 also if `dims` is invalid. */
size_t moe_route_workspace_bytes(const moe_dims* dims);

/* Router logits and top-k (K3 page stages "A" and "route"; K5 page, HA).
 *   x        [S, d] bf16 activations;
 *   w_router [E, d] fp32, finite (at S > 32 a non-finite weight makes its
 *            expert's logits NaN); bias [E] fp32 or NULL (bias_mode 0: added to the
 *            logit, before ranking and sigmoid; 1: added to the ranking key
 *            only);
 *   logits   [S, E] fp32, written: sum_j x[t][j] w_router[e][j], fp32
 *            accumulation, + bias[e] under bias_mode 0;
 *   topk_ids [S, topk] int32, written: the token's experts by descending key,
 *            equal keys to the lower id; the key is the logit, or under
 *            bias_mode 1 the fp32 sum logit + bias[e];
 *   topk_w   [S, topk] fp32, written: sigmoid(logit), divided by the sum over
 *            the token's topk picks when renorm = 1;
 *   workspace device scratch of at least moe_route_workspace_bytes (may be
 *            NULL when that is 0), caller-owned, no initial contents needed;
 *            calls sharing it must not overlap.
 * The fp32 sums run in a fixed order (deterministic): for S <= 32 each of
 * 1024 threads sums d / 1024 products and a fixed tree adds the threads'
 * sums; beyond, each weight is split exactly into three bf16 (whose products
 * with the bf16 x are exact in fp32) and 32-K blocks of bf16 MFMAs go
 * round-robin to 4 chains a K part, added pairwise, and the parts are added
 * in a fixed order. */
int moe_route(const moe_dims* dims, const void* x, const float* w_router, const float* bias,
              float* logits, int32_t* topk_ids, float* topk_w, void* workspace,
              size_t workspace_bytes, hipStream_t stream);

/* Bucketing of the local picks (K3 page stage "route"; "dn_loads": expert
 * table etab and count nv), deterministic, no atomics on the output.
 *   topk_ids [S, topk] int32: a token's ids must be distinct; ids outside
 *            [local_base, local_base + n_local) are not local;
 *   counts   [n_local] int32, written: picks of local expert el;
 *   offsets  [n_local + 1] int32, written: exclusive prefix sum of counts;
 *   rows     [R_max] int32, written: token of bucket row r (rows of expert
 *            el are offsets[el] .. offsets[el + 1] - 1, tokens ascending);
 *            -1 from offsets[n_local] on;
 *   pick_pos [S, topk] int32, written: bucket row of each pick, -1 if not local;
 *   active   [1 + n_local] int32, written: active[0] = number of local
 *            experts with a pick, then their local indices ascending, then -1. */
int moe_bucket(const moe_dims* dims, const int32_t* topk_ids, int32_t* counts, int32_t* offsets,
               int32_t* rows, int32_t* pick_pos, int32_t* active, hipStream_t stream);

/* Bytes of scratch moe_expert_ffn needs: the SwiGLU rows of every bucket row
 * (R_max x I bf16), with a shared expert those of every token (S x shared_I
 * bf16), then counters that order the down GEMMs after the gate_up GEMMs
 * inside one launch, and an error word. 0 if `dims` is invalid. */
size_t moe_ffn_workspace_bytes(const moe_dims* dims);

/* The expert FFNs (K3 page stages "C, D"): for every bucket row r of local
 * expert el (token t = rows[r]),
 *   gu = bf16( x[t] . W13[el]^T )                (MXFP4 decoded to bf16, fp32 accumulation)
 *   h  = bf16( silu(gu[0:I]) * gu[I:2I] )
 *   y[r] = bf16( h . W2[el]^T ),
 * and, if shared_I > 0, the same chain on every token t with the dense bf16
 * shared weights into y[R_max + t].
 *   x          [S, d] bf16;
 *   w13_packed, w2_packed: moe_pack_mxfp4 outputs;
 *   counts, offsets, rows, active: moe_bucket outputs (offsets and active are
 *              implied by counts and are not read by the current kernels);
 *   ws13_packed, ws2_packed: moe_pack_bf16 outputs, or NULL when shared_I == 0;
 *   y          [R_max + (shared_I ? S : 0), d] bf16, written for rows < offsets[n_local]
 *              and the shared rows; other rows are left as they were;
 *   workspace  device scratch of at least moe_ffn_workspace_bytes(dims). It must
 *              be zero-filled once before its first use; every call leaves its
 *              counters at zero again (the rest is undefined afterwards). The
 *              counters' place depends on the dims: a workspace used with
 *              other dims must be zero-filled again.
 *              Calls sharing a workspace must not overlap. The 32-bit word at
 *              byte offset moe_ffn_workspace_bytes(dims) - 256 is set nonzero by
 *              a call in which a wait hit its time bound (a correct run never
 *              does; that call's outputs are undefined and the workspace must
 *              be zero-filled again).
 * MXFP4 decode: element = e2m1 value x 2^(X - 127) for the block's e8m0 byte
 * X, as a bf16 operand; every byte is accepted: X = 0 scales by 2^-127 (bf16
 * subnormals are kept), X = 0xFF makes the block's 32 elements NaN (OCP MX
 * v1.0), and at X = 253 / 254 decoded magnitudes of 2^128 and more are +-inf.
 * NaNs and infinities then propagate by IEEE rules (a row's sum of squares
 * in moe_combine included).
 * The down GEMM of an expert needs all of its SwiGLU rows (K3 page, stages
 * "C, D"). Without a shared expert the FFNs are one launch: a down task
 * issues its first weight loads, then waits on a ready flag set once all of
 * its expert's gate_up tasks are done. With a shared expert they are two
 * launches, gate_up + SwiGLU then down. */
int moe_expert_ffn(const moe_dims* dims, const void* x, const void* w13_packed,
                   const void* w2_packed, const int32_t* counts, const int32_t* offsets,
                   const int32_t* rows, const int32_t* active, const void* ws13_packed,
                   const void* ws2_packed, void* y, void* workspace, size_t workspace_bytes,
                   hipStream_t stream);

/* Per-pick RMSNorm and the routing-weighted sum (K3 page stage "E"):
 *   out[t] = sum over t's slots s in order with pick_pos[t][s] >= 0 of
 *              topk_w[t][s] * y[p] / sqrt(mean(y[p]^2) + eps) * gamma
 *            (+ y[R_max + t] if shared_I > 0),  p = pick_pos[t][s];
 *   a token with no local pick (and no shared expert) gets zeros.
 *   y        moe_expert_ffn's output; topk_w, pick_pos as above;
 *   gamma    [d] bf16 norm weight, or NULL for ones;
 *   out      [S, d] fp32, overwritten (this GPU's partial). */
int moe_combine(const moe_dims* dims, const void* y, const float* topk_w, const int32_t* pick_pos,
                const void* gamma, float* out, hipStream_t stream);

/* ------------------------------------------------------------------------ */
/* the whole block in one call                                               */
/* ------------------------------------------------------------------------ */

/* Bytes of scratch moe_forward needs: moe_route's, then moe_expert_ffn's; 0
 * if `dims` is invalid. */
size_t moe_forward_workspace_bytes(const moe_dims* dims);

/* The whole block -- the work of moe_route, moe_bucket, moe_expert_ffn and
 * moe_combine -- on one stream (K3 page, stage "route": the routing is
 * computed inside the launch that consumes it): the router launch, then the
 * expert-FFN launch (two with a shared expert) whose first S + 1 workgroups
 * take the top-k and the bucketing while its expert tasks wait for the
 * routing, then the combine. Without a shared expert at S > 64 the top-k and
 * the bucketing are launches of their own, as in the four calls (measured
 * faster there). Arguments and outputs are those of the four
 * calls, with identical values (the same device code computes every value).
 * `workspace` follows the moe_expert_ffn rules (zero-filled once before first
 * use, error word at byte moe_forward_workspace_bytes - 256, calls sharing it
 * must not overlap): the expert-FFN launch's counters and flags return to
 * zero within it, and the combine launch clears the routing front's control
 * words for the next call (so moe_forward and moe_forward_one_launch may take
 * turns on one workspace); a workspace used with other dims must be
 * zero-filled again. */
int moe_forward(const moe_dims* dims, const void* x, const float* w_router, const float* bias,
                const void* w13_packed, const void* w2_packed, const void* ws13_packed,
                const void* ws2_packed, const void* gamma, float* logits, int32_t* topk_ids,
                float* topk_w, int32_t* counts, int32_t* offsets, int32_t* rows,
                int32_t* pick_pos, int32_t* active, void* y, float* out, void* workspace,
                size_t workspace_bytes, hipStream_t stream);

/* The whole block as ONE launch (Muse Spark K3 page, module docstring: the
 * layer as one persistent launch; stage "route": the routing computed inside
 * the launch that consumes it), for S <= 16, d <= 4096 and no shared expert.
 * The launch's first E workgroups compute one router row each (summed as the
 * router launch sums it), the next S + 1 take the top-k and the bucketing,
 * then the expert tasks (gate_up hands its SwiGLU rows to down on flags),
 * then one combine workgroup a token, which waits until its rows of y are
 * written; every hand-off is a device-scope counter or flag in the
 * workspace, and the last combine workgroup leaves them at zero for the next
 * call. Measured on MI355X it is not faster than moe_forward's three
 * launches (S = 8: about 2-3 us slower; S = 16: equal): each hand-off inside
 * the launch costs about what the launch boundary it replaces did.
 *   Arguments, outputs and workspace are moe_forward's (no shared expert:
 *   no ws13/ws2), with identical values; the workspace rules are the same
 *   (zero-filled once before first use; left ready for the next call with
 *   the same dims, through either entry point; calls sharing it must not
 *   overlap).
 * Returns MOE_ERR_UNSUPPORTED outside S <= 16, d <= 4096, shared_I == 0,
 * before anything is enqueued; otherwise moe_forward's codes. */
int moe_forward_one_launch(const moe_dims* dims, const void* x, const float* w_router,
                           const float* bias, const void* w13_packed, const void* w2_packed,
                           const void* gamma, float* logits, int32_t* topk_ids, float* topk_w,
                           int32_t* counts, int32_t* offsets, int32_t* rows, int32_t* pick_pos,
                           int32_t* active, void* y, float* out, void* workspace,
                           size_t workspace_bytes, hipStream_t stream);

/* For callers that cannot allocate (code under HIP graph capture, serving
 * loops, harnesses that forbid hipMalloc): moe_forward without a workspace
 * argument. Its scratch is a static device array of MOE_STATIC_SCRATCH_BYTES
 * in the library, one per GPU, held from the first call on that GPU until the
 * process ends. The call allocates nothing and calls no allocating routine.
 *   Arguments and outputs are moe_forward's, without workspace and
 *   workspace_bytes; the device is the current one (that of `stream`).
 *   wait_error: a device int32, or NULL: set to 0 at the start of the call
 *   and nonzero if a wait in the expert-FFN launch hit its time bound (a
 *   correct run never does; the outputs are then undefined).
 * Returns moe_forward's codes; MOE_ERR_WORKSPACE when moe_forward_workspace_
 * bytes(dims) exceeds MOE_STATIC_SCRATCH_BYTES (checked on the host before
 * anything is enqueued). Every call on a GPU shares that GPU's array and
 * clears its control words first: calls that overlap on one GPU (several
 * streams, several host threads) race and must not be made. Outputs are
 * bit-identical to moe_forward's for the same inputs. */
#define MOE_STATIC_SCRATCH_BYTES ((size_t)16 << 20)
int moe_forward_static(const moe_dims* dims, const void* x, const float* w_router,
                       const float* bias, const void* w13_packed, const void* w2_packed,
                       const void* ws13_packed, const void* ws2_packed, const void* gamma,
                       float* logits, int32_t* topk_ids, float* topk_w, int32_t* counts,
                       int32_t* offsets, int32_t* rows, int32_t* pick_pos, int32_t* active,
                       void* y, float* out, int32_t* wait_error, hipStream_t stream);

/* ------------------------------------------------------------------------ */
/* around the block: the latent projections                                  */
/* ------------------------------------------------------------------------ */

/* The steps next to the block (Muse Spark K5 page, HA routing tail and HB;
 * K3 page, stages "A" and "F"; the Kimi-K3 layer page's latent MoE in
 * "k2_launch": w_ld, ln_w, w_up):
 *   before: ffn_in [S, D] feeds the router and pre_expert_proj, a dense bf16
 *           projection to the latent width L the experts run on (a GPU holds
 *           a share of its rows); after the gather, pre_expert_norm gives the
 *           experts' input h [S, L];
 *   after:  post_expert_proj maps the summed expert partial [S, L] back to
 *           the model width (a share of its rows a GPU).
 * Sizes (elements). Supported ranges: 1 <= S <= 128; 128 <= K <= 16384,
 * K % 128 == 0; 64 <= N <= 16384, N % 64 == 0; 0 <= E <= 256; bias_mode in
 * {0, 1}; eps finite, >= 0. */
typedef struct moe_proj_dims {
  int32_t S;         /* token rows */
  int32_t K;         /* input width: D (moe_pre_expert) or L (moe_post_expert) */
  int32_t N;         /* weight rows held here = outputs a token (moe_latent_norm: L) */
  int32_t E;         /* moe_pre_expert: router rows held here, 0 = no router */
  int32_t bias_mode; /* moe_pre_expert: as moe_dims.bias_mode */
  float eps;         /* moe_latent_norm: RMSNorm epsilon */
} moe_proj_dims;

/* Host-only check of `dims`: MOE_OK, MOE_ERR_NULL, _SHAPE or _UNSUPPORTED. */
int moe_check_proj_dims(const moe_proj_dims* dims);

/* Packed size (N * K * 2 bytes, 0 if `dims` is invalid) and packing of a
 * dense bf16 weight w [N, K] (row n = output n) into the kernels' tile order.
 * The packed buffer is opaque: only moe_pre_expert / moe_post_expert read it. */
size_t moe_packed_dense_bytes(const moe_proj_dims* dims);
int moe_pack_dense(const moe_proj_dims* dims, const void* w, void* packed, hipStream_t stream);

/* Workspace bytes of moe_pre_expert / moe_post_expert (fp32 split-K
 * partials, counters, a bf16 copy of the post input); 0 if `dims` is
 * invalid. The workspace must be zero-filled once before its first use; every
 * call leaves its counters at zero again. Calls sharing one workspace must not
 * overlap. */
size_t moe_proj_workspace_bytes(const moe_proj_dims* dims);

/* Before the block (K5 page, HA: router and pre_expert_proj on ffn_in):
 *   ffn_in   [S, K] bf16;
 *   w_packed moe_pack_dense of w_pre [N, K] bf16;
 *   w_router [E, K] fp32, bias [E] fp32 or NULL, logits [S, E] fp32: as
 *            moe_route's logits (ignored when E == 0, may be NULL then);
 *   h_raw    [S, N] bf16, written: bf16(sum_k ffn_in[t][k] w_pre[n][k]),
 *            fp32 accumulation in K parts summed in part order, one rounding.
 * One launch: the router rows are workgroups of the projection's launch (for
 * K > 8192 the router has a launch of its own). */
int moe_pre_expert(const moe_proj_dims* dims, const void* ffn_in, const void* w_packed,
                   const float* w_router, const float* bias, float* logits, void* h_raw,
                   void* workspace, size_t workspace_bytes, hipStream_t stream);

/* pre_expert_norm (K5 page, HA: one token a CTA), on the whole latent. It
 * reads dims->S, dims->N (= L) and dims->eps; the other fields must still be
 * in range.
 *   h_raw [S, N] bf16 (N = L), gamma [N] bf16 or NULL (ones);
 *   h     [S, N] bf16, written: bf16(h_raw * r * gamma) with
 *         r = (sum_c h_raw[t][c]^2 / N + eps)^(-1/2), evaluated in fp64. */
int moe_latent_norm(const moe_proj_dims* dims, const void* h_raw, const void* gamma, void* h,
                    hipStream_t stream);

/* After the block (K3 page, stage "F"; K5 page, HB: post_expert_proj of the
 * summed expert partial):
 *   partial  [S, K] fp32 (the partials of all GPUs summed), rounded to bf16
 *            for the bf16 GEMM;
 *   w_packed moe_pack_dense of w_post [N, K] bf16;
 *   out      [S, N] bf16, written: bf16(sum_k bf16(partial[t][k]) w_post[n][k]),
 *            fp32 accumulation as in moe_pre_expert.
 * One launch at S <= 16 (its tasks round the partial as they read it); above,
 * two: the rounding of the partial, then the projection. */
int moe_post_expert(const moe_proj_dims* dims, const float* partial, const void* w_packed,
                    void* out, void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Top-k of given logits (the router part of moe_route alone), for logits
 * that moe_pre_expert computed: the arguments are moe_route's. With
 * bias_mode 0 the logits already hold the bias and `bias` is not read. */
int moe_topk(const moe_dims* dims, const float* logits, const float* bias, int32_t* topk_ids,
             float* topk_w, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MOEBLK_H */
