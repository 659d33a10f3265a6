/*
 * hla.h -- C ABI of the hybrid linear-softmax attention hot path (gfx950 / MI355X).
 *
 * The operators are the token mixers of SANA-Video 2.0's hybrid attention: gated
 * linear attention, which mixes tokens through a fixed-size per-head state in O(N),
 * and a gated softmax "anchor" that keeps exact, full-rank token interactions;
 * the two are interleaved 3:1 with a softmax anchor on every fourth layer
 * (SANA-Video 2.0 abstract, thelatestinai.com paper listing; ai-papers.net
 * summary, section on hybrid linear attention; lode.cx article, "How It Works").
 * The pages give no formulas. This library computes, per batch b and head h,
 * with rows of Q, K, V, G in R^{N x D} being tokens:
 *
 *   phi(x) = max(x, 0),  sigma(x) = 1 / (1 + exp(-x))
 *   linear : S = phi(K)^T V (D x D),  z = sum_n phi(K_n) (D)
 *            O_n = sigma(G_n) (.) (phi(Q_n) S) / (phi(Q_n) . z + eps)
 *   softmax: O = sigma(G) (.) softmax_rows(scale * Q K^T) V   (non-causal, no mask)
 *   stack  : x <- x + layer_l(Q_l, K_l, V_l, G_l) for l = 0 .. n_layers-1
 *
 * Memory layout of every tensor: [B, H, N, D], row-major and contiguous (D is the
 * fastest dimension). q, k, v and g share dtype dims->in_dtype; the output has
 * dims->out_dtype. All tensor and workspace pointers are DEVICE pointers owned by
 * the caller; the library allocates nothing and keeps no pointer after a call
 * returns. Pointer arrays and `kinds` of the stack call are HOST arrays.
 *
 * Supported combinations:
 *   in_dtype HLA_F32      -> out_dtype HLA_F32                 D in {32, 64, 128}
 *   in_dtype HLA_BF16     -> out_dtype HLA_BF16 or HLA_F32     D in {64, 128}
 *   in_dtype HLA_FP8_E4M3 -> out_dtype HLA_BF16 or HLA_F32     D in {64, 128}
 * bf16 paths multiply in bf16 on the matrix cores and accumulate in fp32; the fp32
 * paths compute in fp32 throughout. fp8 inputs (OCP e4m3: 1 sign, 4 exponent, 3
 * mantissa bits, bias 7, no infinities) take one byte per element. The softmax
 * anchor forms Q K^T from them on the fp8 matrix cores (exact products, fp32
 * sums), and so does the linear layer's state pass for phi(K)^T V (without a
 * write gate); everywhere else they are converted exactly to bf16 where the
 * kernels read them. Results are thus those of the bf16 path on the same values,
 * up to the fp32 summation order and the matrix instructions' internal
 * rounding of their sums (of Q K^T in the anchor, of phi(K)^T V and phi(Q) S in
 * the linear layer). hla_softmax_anchor_fp8p_fwd also rounds the probabilities
 * to e4m3.
 *
 * Errors: every argument is checked on the host before any HIP call. On error
 * nothing is enqueued and the output is untouched. On success the work is
 * enqueued on `stream` (a hipStream_t; NULL means the null stream) and the call
 * returns without synchronising; device faults surface at the caller's next sync.
 * Before launching, a call clears the calling thread's pending HIP error state
 * (hipGetLastError), so that HLA_ERR_HIP reports only errors of its own launches.
 * A tensor with B*H*N == 0 is empty: after the checks the call returns HLA_OK and
 * enqueues nothing (pointers may then be NULL). Calls are reentrant; calls that
 * share a workspace must be ordered on one stream. out/x must not overlap any
 * input or the workspace.
 */
#ifndef HLA_H
#define HLA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define HLA_ABI_VERSION 5

typedef enum { HLA_F32 = 0, HLA_BF16 = 1, HLA_FP8_E4M3 = 2 } hla_dtype;

typedef enum { HLA_LAYER_LINEAR = 0, HLA_LAYER_SOFTMAX = 1 } hla_layer_kind;

typedef enum {
  HLA_OK = 0,
  HLA_ERR_NULL_PTR = 1,    /* a required pointer is NULL */
  HLA_ERR_BAD_SHAPE = 2,   /* a dim < 0, D <= 0, or a byte size / index overflows */
  HLA_ERR_UNSUPPORTED = 3, /* D or dtype combination not built */
  HLA_ERR_BAD_ARG = 4,     /* eps, scale, accumulate, n_layers or a kind out of range */
  HLA_ERR_ALIGN = 5,       /* a tensor or workspace pointer is not 16-byte aligned */
  HLA_ERR_WORKSPACE = 6,   /* workspace_bytes smaller than required */
  HLA_ERR_HIP = 7          /* the HIP runtime reported an error at launch */
} hla_status;

typedef struct {
  int64_t B, H, N, D;  /* batch, heads, tokens, head dim */
  int32_t in_dtype;    /* hla_dtype of q, k, v, g */
  int32_t out_dtype;   /* hla_dtype of out / x */
} hla_dims;

/* ABI version of the loaded library (HLA_ABI_VERSION it was built with). */
int hla_abi_version(void);

/* Static, NUL-terminated name of a status code ("HLA_OK", ...); "HLA_UNKNOWN"
 * for a value outside the enum. */
const char* hla_status_str(int status);

/* Bytes of device workspace hla_linear_fwd (and the stack call) needs for `d`:
 * per-chunk partial states, B*H*C of them (D*D + D fp32 on the fp32 path; D*D
 * bf16 + D fp32 on the bf16 and fp8 paths), plus the reduced state in the form
 * the output pass reads. Host-only and pure: equal dims give equal sizes.
 * Returns 0 for invalid or unsupported dims, and for empty tensors. */
size_t hla_linear_workspace_bytes(const hla_dims* d);

/* Gated linear attention (non-causal) -- the O(N) fixed-size-state mixer of the
 * ai-papers.net summary, section on hybrid linear attention, and of the
 * SANA-Video 2.0 abstract. Computes O as defined above; accumulate = 0 stores
 * out = O, accumulate = 1 updates out += O in place. eps must be finite and
 * >= 0 (with eps = 0 a token with phi(Q_n) . z == 0 yields NaN; with eps > 0
 * such a token yields exactly 0). `workspace` is a device buffer of at least
 * hla_linear_workspace_bytes(d) bytes; its contents on entry do not matter. */
hla_status hla_linear_fwd(const hla_dims* d, const void* q, const void* k, const void* v,
                          const void* g, void* out, int accumulate, float eps, void* workspace,
                          size_t workspace_bytes, void* stream);

/* Allocation-free variant of hla_linear_fwd, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid it): same operator, arguments and results as hla_linear_fwd, but the
 * partial states and reduced state live in a scratch array of
 * HLA_NOALLOC_SCRATCH_BYTES that the library holds on each GPU it runs on (from
 * the module load until the process ends); no workspace argument, and the call
 * allocates nothing. Returns HLA_ERR_WORKSPACE, enqueuing nothing, when the call
 * would need more than that (hla_linear_workspace_bytes(d) above the limit), and
 * HLA_ERR_HIP if the scratch array's address cannot be found on the current
 * device (looked up once per device, on the first call there). The array's
 * contents on entry do not matter. Calls on one GPU share that GPU's array:
 * calls that overlap in time on one GPU (concurrent streams, or threads) race
 * and give undefined results; order them on one stream. */
#define HLA_NOALLOC_SCRATCH_BYTES (64u << 20)
hla_status hla_linear_fwd_noalloc(const hla_dims* d, const void* q, const void* k, const void* v,
                                  const void* g, void* out, int accumulate, float eps,
                                  void* stream);

/* Write-gated linear attention: as hla_linear_fwd, but each token writes into the
 * state with strength beta_n = sigma(W_n), one logit per token and head:
 *   S = sum_n beta_n phi(K_n)^T V_n,  z = sum_n beta_n phi(K_n)
 *   O_n = sigma(G_n) (.) (phi(Q_n) S) / (phi(Q_n) . z + eps)
 * (the gate that regulates what is written into the fixed-size state, ai-papers.net
 * summary, section on hybrid linear attention; the pages give no formula, this is
 * one reading of it). `w` is a device tensor [B, H, N], contiguous, dtype
 * d->in_dtype, 16-byte aligned; W = +inf reproduces hla_linear_fwd exactly, W = -inf
 * removes the token. Workspace, accumulate, eps and errors as in hla_linear_fwd
 * (HLA_ERR_NULL_PTR / HLA_ERR_ALIGN also for `w`). */
hla_status hla_linear_write_gated_fwd(const hla_dims* d, const void* q, const void* k,
                                      const void* v, const void* g, const void* w, void* out,
                                      int accumulate, float eps, void* workspace,
                                      size_t workspace_bytes, void* stream);

/* Bytes of device workspace hla_softmax_anchor_fwd needs for `d`: on the bf16
 * and fp8 paths a repacked copy of V (B*H*D*ceil(N/64)*64 bf16, V transposed with zero
 * keys past N) followed by room for the partial results of up to
 * P = min(1024, ceil(N/256) * B*H * ceil(N/64)) key-range pieces (P*256*(D+2)
 * fp32), used when the query blocks of an incomplete last batch of workgroups
 * are split along the keys; 0 on the fp32 path. Host-only and pure; 0 for
 * invalid or unsupported dims and for empty tensors. */
size_t hla_softmax_anchor_workspace_bytes(const hla_dims* d);

/* Gated softmax anchor (non-causal, no mask, no positional term) -- the periodic
 * gated-softmax layer that restores exact token interactions (SANA-Video 2.0
 * abstract; lode.cx article, "The Core Innovation"). scale must be finite and
 * > 0 (1/sqrt(D) is the usual choice). accumulate as in hla_linear_fwd.
 * `workspace` is a device buffer of at least hla_softmax_anchor_workspace_bytes(d)
 * bytes (may be NULL when that is 0); its contents on entry do not matter. */
hla_status hla_softmax_anchor_fwd(const hla_dims* d, const void* q, const void* k, const void* v,
                                  const void* g, void* out, int accumulate, float scale,
                                  void* workspace, size_t workspace_bytes, void* stream);

/* Gated softmax anchor with 8-bit probabilities, for fp8 (e4m3) inputs only --
 * one reading of the quantized inference the pages report (ai-papers.net
 * summary: quantization-aware training, 5.8 % lower latency, no number format
 * given). As hla_softmax_anchor_fwd, except that the softmax probabilities,
 * taken relative to a running row maximum and at most 2^8, are rounded to OCP
 * e4m3 (round to nearest even, subnormals kept) and P V runs on the fp8 matrix
 * cores with V in e4m3; the row sum adds the same rounded probabilities. With a
 * 3-bit fraction this rounding moves each probability by up to 2^-4 of itself
 * (2^-10 absolutely below 2^-6 of the row maximum), so outputs carry an error
 * of their own -- at the 480p and 720p shapes about 2.5e-2 of the largest
 * output, against about 2e-3 with bf16 probabilities. d->in_dtype must be
 * HLA_FP8_E4M3 (else HLA_ERR_UNSUPPORTED). hla_softmax_anchor_workspace_bytes(d)
 * bytes of workspace suffice (this call uses less: its copy of V is e4m3).
 * Arguments, accumulate and the other errors as in hla_softmax_anchor_fwd. */
hla_status hla_softmax_anchor_fp8p_fwd(const hla_dims* d, const void* q, const void* k,
                                       const void* v, const void* g, void* out, int accumulate,
                                       float scale, void* workspace, size_t workspace_bytes,
                                       void* stream);

/* Hybrid stack: for l = 0 .. n_layers-1 in order, x += layer_l(q[l], k[l], v[l], g[l])
 * where kinds[l] is HLA_LAYER_LINEAR or HLA_LAYER_SOFTMAX; SANA-Video 2.0 places a
 * softmax anchor on every fourth layer (lode.cx article, "How It Works";
 * ai-papers.net summary, section on hybrid linear attention). x has dtype
 * d->out_dtype and is updated in place (an fp32 x keeps the residual stream
 * exact to fp32 rounding). kinds, q, k, v, g are host arrays of n_layers
 * entries; each q[l] ... g[l] is a device tensor like those of hla_linear_fwd.
 * workspace must hold max(hla_linear_workspace_bytes(d) if some kind is linear,
 * hla_softmax_anchor_workspace_bytes(d) if some kind is softmax) bytes; layers
 * reuse it one after another. All layers are enqueued on `stream` in order. */
hla_status hla_hybrid_stack_fwd(const hla_dims* d, int n_layers, const int32_t* kinds,
                                const void* const* q, const void* const* k,
                                const void* const* v, const void* const* g, void* x, float eps,
                                float scale, void* workspace, size_t workspace_bytes,
                                void* stream);

/* Block attention residuals (AttnRes) routing -- SANA-Video 2.0 groups layers into
 * blocks of 8 and routes a summary of every completed block directly into later
 * linear layers through a query router shared across depth (ai-papers.net summary,
 * section on attention residuals; lode.cx article, "The Core Innovation"; SANA-Video
 * 2.0 abstract). The pages give no formula; this is one reading of it. Per token n
 * of each (b, h):
 *   q_n = x_n W,  a_i = q_n . s_i,n / sqrt(D),  out_n = x_n + sum_i softmax_i(a)_i s_i,n
 * where s_0 .. s_{n_blocks-1} are the summaries of the completed blocks (a block's
 * summary is its total update of the residual stream, x at its end minus x at its
 * start) and W is the router projection shared by every layer. out is the stream a
 * later linear layer's projections read.
 * dims: in_dtype = out_dtype = HLA_F32 (x, every summary and out: fp32
 * [B, H, N, D]), D in {64, 128}; otherwise HLA_ERR_UNSUPPORTED. `summaries` is a
 * HOST array of n_blocks DEVICE pointers, 0 <= n_blocks <= 16 (else HLA_ERR_BAD_ARG);
 * w_router is a DEVICE bf16 [D, D] row-major matrix (q_j = sum_k x_k W[k][j]).
 * q is formed on the matrix cores from x split into a bf16 hi + lo pair (about 16
 * significant bits; fp32 sums); scores, softmax and the mix are fp32. With
 * n_blocks = 0 out = x (a copy, or nothing when out == x). out may be x itself
 * (in place); it must not overlap a summary or W. All device pointers 16-byte
 * aligned. No workspace. */
hla_status hla_attnres_route_fwd(const hla_dims* d, int n_blocks, const void* const* summaries,
                                 const void* x, const void* w_router, void* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* HLA_H */
