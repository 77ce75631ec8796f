/*
 * sparse_ffn.h -- C ABI of the contextually sparse gated-FFN decode step on AMD Instinct
 * MI355X (gfx950).
 *
 * The method. A gated FFN computes, for a token x in R^d,
 *     g = Wg x (+ b),  u = Wu x,  a = act(g),  y = sum_i m_i a_i u_i Dt[i,:]
 * where m is a 0/1 mask over the f neurons and act is SiLU (SwiGLU) or ReLU (ReGLU).
 * Contextual sparsity picks m per token so that only the rows of Wu and Dt with m_i = 1
 * are read:
 *   - CATS ("CATS: Contextually-Aware Thresholding for Sparsity in Large Language
 *     Models", abstract): m_i = [|SiLU(g_i)| > t] with one calibrated threshold t per
 *     layer, so the dense gate itself is the score;
 *   - SVD predictor ("SVD Contextual Sparsity Predictors for Fast LLM Inference",
 *     abstract, Figures 1 and 3): a rank-r predictor p = L (Q x) + b with per-neuron
 *     thresholds tau picks candidate rows; the gate is evaluated on the candidates only
 *     and up/down only where ReLU(gate) > 0 (the sequential pipeline), or the gate, up
 *     and down rows of every candidate are read in one pass (the parallel pipeline,
 *     Table 2);
 *   - Sirius ("SIRIUS: Contexual Sparisty with Correction for Efficient LLMs",
 *     Approach): the full model re-runs a chunk of up to 16 tokens densely with the same
 *     weights to verify them.
 *
 * Layout. Every weight matrix is row-major [f, d], one row per neuron: w_gate and w_up
 * as in nn.Linear, and w_down_t = W_down transposed, so that the output weights of
 * neuron i are the contiguous row i. One copy of the weights serves the sparse, dense
 * and verification paths. Rows must be 16-byte aligned: d % 8 == 0 for bf16 and
 * d % 4 == 0 for fp32, and every pointer 16-byte aligned.
 *
 * Conventions for every compute call.
 *   - Pointers are DEVICE pointers unless marked (host). The caller owns every buffer;
 *     the library allocates nothing and keeps no pointer after the call returns.
 *   - The call validates its arguments on the host, enqueues its kernels on `stream`
 *     (a hipStream_t passed as void*, NULL = the null stream) and returns without
 *     synchronising. A negative status means nothing was enqueued, except SFN_EHIP,
 *     which reports a launch error from the HIP runtime. Device-side faults surface at
 *     the caller's next synchronisation. No C++ exception crosses the ABI.
 *   - Workspace: `ws` of `ws_bytes` bytes (256-byte aligned), sized by the
 *     *_workspace_size queries. Its first SFN_WORKSPACE_HEADER_BYTES (2 KiB) are
 *     reserved and must be zero-filled once when the workspace is allocated (e.g.
 *     torch.zeros). A call may use them between its own kernels (the one-token decode
 *     publishes per-tile counts there) but its last kernel zeroes them again, so they are
 *     zero whenever no call is in flight. Everything after them is scratch each call
 *     rewrites before reading, so any sequence of calls on one stream may share one
 *     workspace (sized for the largest of them). Calls that may run concurrently
 *     (different streams) need distinct workspaces.
 *   - Status word: the uint32 at byte SFN_WORKSPACE_STATUS_OFFSET of the workspace stays
 *     0 through every call that completes normally. The library's few device-side waits
 *     (workgroups of one launch waiting for each other's results, which only a device
 *     that never schedules some of them can stall) are bounded; one that gives up writes
 *     its SFN_STATUS_* code there and that call's outputs are invalid (y is NaN, or
 *     *n_cand is -1). The word stays set for the caller to read after a
 *     synchronisation; zero the whole header again before the workspace is reused.
 *   - Outputs are deterministic: identical inputs give bitwise identical y, index
 *     lists and thresholds (fixed reduction orders, no floating-point atomics). One
 *     exception, for calls that overlap on the device: see sparse_ffn_decode (one token,
 *     rows wider than 8 KB).
 *   - Arithmetic: products and sums in fp32 (bf16 inputs are widened exactly).
 */
#ifndef SPARSE_FFN_H
#define SPARSE_FFN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes (int). */
#define SFN_OK 0
#define SFN_EINVAL (-1)       /* null pointer where one is required, bad enum, k or s out of range */
#define SFN_ESHAPE (-2)       /* d, f, r, B or n outside the supported range */
#define SFN_EDTYPE (-3)       /* dtype not supported by this call */
#define SFN_EWORKSPACE (-4)   /* ws NULL or ws_bytes smaller than the query returns */
#define SFN_EALIGN (-5)       /* a pointer or a row not 16-byte aligned */
#define SFN_EUNSUPPORTED (-6) /* valid request this library does not implement */
#define SFN_EHIP (-7)         /* the HIP runtime reported an error on launch */
#define SFN_ETOOLARGE (-8)    /* sparse_ffn_decode_noalloc: more scratch than its fixed array */

/* Workspace header (see the conventions above). */
#define SFN_WORKSPACE_HEADER_BYTES 2048
#define SFN_WORKSPACE_STATUS_OFFSET 1024
#define SFN_STATUS_BALANCER_TIMEOUT 1u  /* sparse_ffn_decode / _svd: the one-token tile balancer */
#define SFN_STATUS_PREDICTOR_TIMEOUT 2u /* svd_predict: the scan over the tiles' counts */
#define SFN_NOALLOC_SCRATCH_BYTES 33554432 /* fixed scratch of sparse_ffn_decode_noalloc */

/* Weight (and token) dtypes. */
#define SFN_F32 0
#define SFN_BF16 1

/* Gate activations. */
#define SFN_ACT_SILU 0 /* SwiGLU: a = g * sigmoid(g); CATS scores |a| */
#define SFN_ACT_RELU 1 /* ReGLU:  a = max(g, 0) */

/* SVD pipelines ("SVD Contextual Sparsity Predictors for Fast LLM Inference", Table 2). */
#define SFN_PIPE_SEQUENTIAL 0 /* gate on the candidates, then up and down where act(gate) != 0 */
#define SFN_PIPE_PARALLEL 1   /* gate, up and down rows of every candidate in one pass */

/* Limits of this library. */
#define SFN_MAX_BATCH 4   /* tokens per sparse_ffn_decode call */
#define SFN_MAX_CHUNK 16  /* tokens per ffn_dense_chunk call (the Sirius chunk) */
#define SFN_MAX_D 16384
#define SFN_MAX_F 262144
#define SFN_MAX_RANK 1024 /* SVD predictor rank */

/* One FFN layer. All pointers device, each matrix [f, d] row-major in `wdtype`. */
typedef struct sfn_ffn {
  int32_t d;            /* hidden size */
  int32_t f;            /* intermediate size (neurons) */
  int32_t wdtype;       /* SFN_F32 or SFN_BF16: dtype of the three matrices and of x */
  int32_t act;          /* SFN_ACT_SILU or SFN_ACT_RELU */
  const void* w_gate;   /* [f, d] */
  const void* w_up;     /* [f, d] */
  const void* w_down_t; /* [f, d]: row i = neuron i's d output weights */
  const float* b_gate;  /* [f] gate bias, or NULL for none */
} sfn_ffn;

/* Rank-r SVD predictor of one layer's gate (bf16 factors). All pointers device. */
typedef struct sfn_svd {
  int32_t d, f, r;   /* hidden size, neurons, rank (8 <= r <= 1024, r % 8 == 0) */
  int32_t reserved;  /* must be 0 */
  const void* q;     /* [r, d] bf16: V_r^T, the top-r right singular vectors as rows */
  const void* l;     /* [f, r] bf16: U_r diag(sigma_r) */
  const float* b;    /* [f] gate bias added to the prediction, or NULL */
  const float* tau;  /* [f] per-neuron thresholds: candidate iff p_i > tau_i */
} sfn_svd;

/* Host. Bytes of workspace any call on `ffn` with up to `max_tokens` tokens needs
 * (decode: B <= 4; dense chunk: n <= 16; calibration: n tokens). 0 on invalid input.
 * Touches no HIP state. */
size_t sparse_ffn_workspace_size(const sfn_ffn* ffn, int32_t max_tokens);

/* Host. Bytes of workspace svd_predict on `svd` needs. 0 on invalid input. */
size_t svd_predict_workspace_size(const sfn_svd* svd);

/* Host. Static, NUL-terminated description of a status code. */
const char* sparse_ffn_strerror(int status);

/*
 * CATS threshold calibration ("CATS: Contextually-Aware Thresholding for Sparsity in
 * Large Language Models", abstract: one threshold per layer sets the activation
 * sparsity). Scores S = |act(x_cal Wg^T + b)| of n calibration tokens ([n, f], fp32),
 * N = n f, K = floor(k N + 1/2); *t_out = the K-th smallest score (1-based), exact
 * selection over the fp32 scores (radix select on their bit patterns), so that exactly
 * K scores satisfy S <= t when they are distinct. K = 0 gives -1 (every neuron active),
 * K = N gives +inf (none).
 *   x_cal      [n, d] in ffn->wdtype, 1 <= n <= 65536
 *   k          target sparsity in [0, 1]
 *   t_out      1 float (device), written
 *   scores_out [n, f] fp32 (device) or NULL: the scores the threshold was taken from
 */
int sparse_ffn_calibrate(const sfn_ffn* ffn, const void* x_cal, int32_t n, float k, float* t_out,
                         float* scores_out, void* ws, size_t ws_bytes, void* stream);

/*
 * One sparse decode step for B tokens (1 <= B <= 4) through one FFN layer.
 * Scores: g = Wg x + b, a = act(g); token b's neuron i is active iff
 *   mask_in != NULL:  mask_in[b, i] != 0                      (mask override)
 *   otherwise:        |a_i| > *t  and (cand == NULL or i in cand)
 * with t a device fp32 scalar (NULL means 0). Each token keeps its own mask; the rows
 * read from Wu and Dt are the union over the batch, each read once.
 *   y = sum_i m_bi a_bi u_bi Dt[i, :]  accumulated in fp32, [B, d] (device) or NULL to
 *       compute the masks only (mask-only mode reads Wg alone).
 * cand/n_cand: an ascending candidate list (from svd_predict) and its device count;
 *   the gate is evaluated on those rows only ("SVD Contextual Sparsity Predictors for
 *   Fast LLM Inference", Figure 3). Requires B == 1 and mask_in == NULL.
 * active_idx [B, f] int32 / n_active [B] int32 (device) or NULL: token b's active
 *   neurons in ascending order and their count.
 * One token with rows wider than 8 KB (d > 4096 in bf16): the workgroups of the call
 *   share out their up/down rows, each waiting until all of them have run their gate
 *   part, but only when all of them are resident at once, which the call finds out for
 *   itself. When they are not (another such call in flight on another stream, or other
 *   work holding compute units), each workgroup keeps its own rows and waits for nothing.
 *   The two ways add the rows in different orders: y is bitwise repeatable for calls that
 *   do not overlap, and otherwise equal to fp32 rounding. Should a wait still exceed about
 *   a second, y comes out NaN rather than wrong and the workspace status word reads
 *   SFN_STATUS_BALANCER_TIMEOUT.
 */
int sparse_ffn_decode(const sfn_ffn* ffn, const void* x, int32_t B, const float* t,
                      const int32_t* cand, const int32_t* n_cand, const uint8_t* mask_in,
                      float* y, int32_t* active_idx, int32_t* n_active, void* ws,
                      size_t ws_bytes, void* stream);

/*
 * sparse_ffn_decode without a workspace, for callers that cannot allocate or hand over
 * device memory: code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc. The same arguments (minus ws and ws_bytes), checks and results as
 * sparse_ffn_decode. The step's scratch is a fixed device array of
 * SFN_NOALLOC_SCRATCH_BYTES (32 MiB) inside the library, one on each GPU it runs on, held
 * until the process ends; the call allocates nothing. It holds the scratch of one-token
 * calls up to f = 65536 at any d (e.g. d 8192, f 28672: 9 MiB) and of batches of up to
 * four tokens at d <= 4096, f <= 65536; a call that needs more returns SFN_ETOOLARGE
 * before anything is enqueued.
 * The array is shared by every call on one GPU and keeps the last call's contents: each
 * call leaves its reserved first SFN_WORKSPACE_HEADER_BYTES zero again, as
 * sparse_ffn_decode leaves a workspace, so calls in order on one stream (or with a
 * synchronisation between them) are safe. Calls that can overlap on one GPU (different
 * streams, or several host threads) race on the array and give wrong results. A bounded
 * wait that gives up shows as NaN in y. The array's status word is not exposed; a give-up
 * leaves it set, and no later call reads it.
 */
int sparse_ffn_decode_noalloc(const sfn_ffn* ffn, const void* x, int32_t B, const float* t,
                              const int32_t* cand, const int32_t* n_cand, const uint8_t* mask_in,
                              float* y, int32_t* active_idx, int32_t* n_active, void* stream);

/*
 * Candidate rows in one pass for one token: the SVD predictor's parallel pipeline ("SVD
 * Contextual Sparsity Predictors for Fast LLM Inference", Table 2: parallel pipeline,
 * against the sequential one of sparse_ffn_decode's candidate mode). For the rows in the
 * candidate list the gate, up and down rows are read together:
 *   y = sum over i in cand of act(g_i) u_i Dt[i, :],   g = Wg x + b,  u = Wu x
 * accumulated in fp32. With ReLU this is the candidate mode's result (the gate zeroes
 * the rest), reading all three rows of every candidate but with no separate gate pass.
 *   x      [d] in ffn->wdtype
 *   cand   candidate rows (device int32; entries are clamped into [0, f)), n_cand its
 *          device count (clamped into [0, f]); any order, each row at most once
 *   y      [d] fp32 (device), written
 * Workspace: as sparse_ffn_decode for one token.
 */
int sparse_ffn_decode_parallel(const sfn_ffn* ffn, const void* x, const int32_t* cand,
                               const int32_t* n_cand, float* y, void* ws, size_t ws_bytes,
                               void* stream);

/*
 * SVD predictor for one token ("SVD Contextual Sparsity Predictors for Fast LLM
 * Inference", abstract and Figures 1-3): z = Q x (fp32), p = L z + b, candidates
 * {i : p_i > tau_i} written in ascending order.
 *   x        [d] bf16
 *   cand_idx [f] int32 (device), the first *n_cand entries written
 *   n_cand   1 int32 (device); -1 if the tiles' count exchange timed out (then the
 *            workspace status word reads SFN_STATUS_PREDICTOR_TIMEOUT; see the conventions)
 *   p_out    [f] fp32 (device) or NULL: the predictions
 */
int svd_predict(const sfn_svd* svd, const void* x, int32_t* cand_idx, int32_t* n_cand,
                float* p_out, void* ws, size_t ws_bytes, void* stream);

/*
 * Predictor and FFN in one call for one token, with no candidate list in between ("SVD
 * Contextual Sparsity Predictors for Fast LLM Inference", Figures 1 and 3, Table 2):
 * z = Q x, then each tile of rows computes p_i = L_i z + b_i for its own rows and
 * processes its candidates {i : p_i > tau_i} directly:
 *   SFN_PIPE_SEQUENTIAL: g_i = Wg_i x + b_gate_i on the candidates, active where
 *     |act(g_i)| > 0 (ReLU: g_i > 0), then y = sum over active i of act(g_i) u_i Dt[i, :];
 *     idx / n_idx: the active rows, ascending.
 *   SFN_PIPE_PARALLEL: y = sum over candidates i of act(g_i) u_i Dt[i, :], the gate, up
 *     and down rows read together; idx / n_idx: the candidate rows, ascending.
 * The same result as svd_predict followed by sparse_ffn_decode (candidate mode) or
 * sparse_ffn_decode_parallel, up to predictions that fall within rounding of tau.
 *   ffn, svd  one layer and its predictor: bf16 weights, svd->d == ffn->d, svd->f == ffn->f
 *   x         [d] bf16 (device)
 *   y         [d] fp32 (device), or NULL (sequential only) for the active rows alone
 *   idx       [f] int32 (device) or NULL, the first *n_idx entries written
 *   n_idx     1 int32 (device) or NULL
 * Workspace: at least sparse_ffn_svd_workspace_size(ffn, svd) bytes, 256-byte aligned,
 * shared with the other calls like theirs. Errors: SFN_EDTYPE for fp32 weights,
 * SFN_ESHAPE for mismatched shapes, SFN_EINVAL for a bad pipeline or nothing requested.
 */
size_t sparse_ffn_svd_workspace_size(const sfn_ffn* ffn, const sfn_svd* svd);
int sparse_ffn_decode_svd(const sfn_ffn* ffn, const sfn_svd* svd, const void* x,
                          int32_t pipeline, float* y, int32_t* idx, int32_t* n_idx,
                          void* ws, size_t ws_bytes, void* stream);

/*
 * Dense FFN over a chunk of n tokens (1 <= n <= 16), the Sirius verification pass
 * ("SIRIUS: Contexual Sparisty with Correction for Efficient LLMs", Approach: the full
 * model checks a chunk of sparse-generated tokens in parallel with the shared weights):
 *   Y[j, :] = sum_i act(g_ji) u_ji Dt[i, :]   for every neuron, fp32 [n, d].
 * bf16 weights with n >= 2 run on matrix cores (bf16 products, fp32 accumulation; the
 * intermediate h = act(g) u is rounded to bf16 for the second product). One token, and
 * fp32 weights, run through the decode kernels with threshold 0 (every neuron with
 * act(g) != 0, i.e. every one that contributes), with h in fp32.
 *   x  [n, d] in ffn->wdtype;  y [n, d] fp32
 */
int ffn_dense_chunk(const sfn_ffn* ffn, const void* x, int32_t n, float* y, void* ws,
                    size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SPARSE_FFN_H */
