/*
 * libmuon — one Muon optimizer step for a list of 2-D weight matrices on an
 * AMD Instinct MI355X (gfx950).  C ABI: plain pointers and sizes only.
 *
 * What a step computes, per matrix, follows "Muon: An optimizer for hidden
 * layers in neural networks" (synthesis note on papers.chlience.com),
 * section 4, the algorithm definition:
 *
 *   B  <- mu * B + G                        momentum accumulation
 *   M  =  B            (nesterov == 0)      input of the orthogonalisation
 *   M  =  G + mu * B   (nesterov != 0)      Nesterov-style reading
 *   X  =  M / (||M||_F + eps)               Frobenius normalisation
 *   X  =  X^T when rows > cols              smaller Gram matrix
 *   repeat ns_steps times (default 5):
 *       A = X X^T;  P = b A + c A A;  X = a X + P X
 *       (a, b, c) = (3.4445, -4.7750, 2.0315)
 *   O  =  X, transposed back when rows > cols
 *   W  <- W - lr * scale * O                parameter update
 *   W  <- W - lr * (lambda * W + scale * O)  with decoupled weight decay
 *                                            lambda (hp->weight_decay)
 *
 * Precision: G is float32 or bfloat16; W and B are float32 and updated in
 * place in float32.  For a Gram side m > 64 every matrix product of the
 * iteration runs on bf16 matrix cores with float32 accumulation; A and P are
 * stored as bf16; the iterate X is carried as a pair of bf16 values (high
 * part and rounding residual) so that the linear term a*X keeps ~16
 * significant bits.  The pair first holds M itself and the first
 * iteration applies 1 / (||M||_F + eps) in its float32 epilogues (the Gram
 * product scaled by its square), unless ||M||_F lies outside [2^-50, 2^50],
 * where the pair holds the normalised M instead.  For m <= 64 (few singular
 * values, where bf16 operand rounding does not average out and the work is
 * small) the iteration runs in float32 throughout.
 *
 * Memory: every pointer passed to the step calls is a DEVICE pointer on the
 * current HIP device, except the descriptor arrays themselves (mats, hp and
 * the pointer/size arrays of muon_orthogonalize), which are HOST memory read
 * only during the call.  All device memory is owned by the caller; the
 * library allocates no device memory and keeps no pointer after a call
 * returns (it keeps a small pinned host staging area for the descriptor
 * table it uploads into the workspace).
 *
 * Ordering: work is enqueued on `stream` (a hipStream_t; NULL = the default
 * stream) and the call returns without waiting.  Results are visible after
 * the caller synchronises the stream.  The caller keeps every buffer alive
 * until then.  Two calls that share a workspace must be ordered on one
 * stream (or synchronised) — the workspace holds the call's descriptor table
 * and intermediates.
 *
 * Errors: all arguments are validated on the host before anything is
 * enqueued, so an error return has no side effects.  A failing HIP launch
 * returns MUON_ERR_HIP; muon_last_error() then holds the HIP message.
 * Faults inside kernels surface at the caller's next synchronisation.
 * NaN or Inf in G propagates into B, W; it is not masked.
 */
#ifndef MUON_H_
#define MUON_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MUON_ABI_VERSION 7

typedef enum muon_status {
  MUON_OK = 0,
  MUON_ERR_INVALID_ARG = -1, /* null pointer, size < 1, bad hyper-parameter   */
  MUON_ERR_UNSUPPORTED = -2, /* shape beyond the supported maximum            */
  MUON_ERR_WORKSPACE = -3,   /* workspace missing, too small or misaligned    */
  MUON_ERR_ALIAS = -4,       /* W/G/B/workspace ranges overlap                */
  MUON_ERR_ALIGN = -5,       /* a matrix base pointer is not 16-byte aligned  */
  MUON_ERR_HIP = -6          /* a HIP runtime call or launch failed           */
} muon_status_t;

typedef enum muon_dtype { MUON_F32 = 0, MUON_BF16 = 1 } muon_dtype_t;

/* One weight matrix.  W, G, B are dense row-major rows x cols arrays
 * (leading dimension = cols), each 16-byte aligned, pairwise disjoint and
 * disjoint from every other matrix's arrays and from the workspace.
 * G has the dtype given by muon_hparams_t.g_dtype; W and B are float32.
 * `scale` multiplies the learning rate for this matrix (the per-parameter
 * update scale of the synthesis note's Moonlight results section; the
 * pages give no formula, so the caller supplies it; 1.0 = plain Muon). */
typedef struct muon_matrix {
  float* W;
  const void* G;
  float* B;
  int64_t rows;
  int64_t cols;
  float scale;
} muon_matrix_t;

/* Hyper-parameters shared by every matrix of a call.
 * mu: momentum (finite); lr: learning rate (finite);
 * eps: added to the Frobenius norm (finite, >= 0; 1e-7 is customary);
 * ns_steps: Newton-Schulz iterations, 0..MUON_MAX_NS_STEPS (5 is the usual);
 * nesterov: 0 = orthogonalise the momentum buffer, 1 = G + mu * B;
 * g_dtype: MUON_F32 or MUON_BF16;
 * weight_decay: decoupled ("AdamW-style") weight decay lambda of the
 *   Moonlight results section of the synthesis note (finite; 0 = none):
 *   W <- W - lr * (lambda * W + scale * O), formed as
 *   fma(-lr*scale, O, fma(-lr*lambda, W, W)) with lr*scale and lr*lambda
 *   rounded to float32 on the host. */
typedef struct muon_hparams {
  float mu;
  float lr;
  float eps;
  int32_t ns_steps;
  int32_t nesterov;
  int32_t g_dtype;
  float weight_decay;
} muon_hparams_t;

#define MUON_MAX_NS_STEPS 64
/* Largest supported dimension of a matrix (rows and cols each). */
#define MUON_MAX_DIM 65536
/* Largest supported short side (the Gram dimension min(rows, cols)). */
#define MUON_MAX_GRAM 16384

/* Bytes of device workspace muon_step needs for this list (0 if n == 0).
 * Returns 0 and sets muon_last_error() when the arguments are invalid.
 * The workspace must be 256-byte aligned. */
size_t muon_workspace_bytes(const muon_matrix_t* mats, int64_t n, const muon_hparams_t* hp);

/* One Muon step on `n` matrices (section 4 of the synthesis note, as above).
 * Updates W and B in place; G is read only.  All matrices are processed by
 * the same sequence of grouped launches (one launch per stage for the whole
 * list), so same-shape matrices such as separate Q, K and V share each
 * dispatch.  n == 0 is a no-op returning MUON_OK. */
muon_status_t muon_step(const muon_matrix_t* mats, int64_t n, const muon_hparams_t* hp,
                        void* workspace, size_t workspace_bytes, void* stream);

/* muon_step for callers that cannot allocate device memory (serving loops
 * and harnesses that forbid hipMalloc): the same kernels and the same bits
 * as muon_step, with the workspace in a static device array of the library
 * instead of a caller's buffer.  The array holds MUON_STATIC_WORKSPACE_BYTES
 * (64 MiB) on every GPU the library runs on, from the first use on that GPU
 * until the process ends; a call whose workspace (muon_workspace_bytes)
 * exceeds it returns MUON_ERR_WORKSPACE before anything is enqueued.  The
 * call allocates nothing: no device memory and no pinned host memory (its
 * descriptor table is copied from the call's own host memory, which the
 * copy has consumed when the call returns; so this entry point is not for
 * stream capture).  Every call on one GPU shares that GPU's array, which
 * keeps the last call's contents (every byte a call reads it writes first):
 * calls that overlap on one GPU (other threads, other streams) race and
 * must be ordered by the caller.  The address of the array is looked up once
 * per device, with that device current. */
#define MUON_STATIC_WORKSPACE_BYTES (64u * 1024u * 1024u)
muon_status_t muon_step_static(const muon_matrix_t* mats, int64_t n, const muon_hparams_t* hp, void* stream);

/* A recorded step, for training loops that run the same step many times on
 * the same buffers (the case where launching ~20 kernels per step from the
 * host costs more than the kernels themselves, e.g. a single 256 x 256
 * matrix).  muon_plan_create validates the call exactly as muon_step does,
 * binds its device buffers, uploads the descriptor table into the workspace
 * (synchronously, on `stream`) and records the step's launch sequence into
 * a HIP graph; each muon_plan_step replays it on `stream` as one graph
 * launch.  A replay is one Muon step on the bound buffers: it reads G's
 * current contents (the caller writes each step's gradient into the bound
 * G buffers) and updates W and B in place, with the hyper-parameters given
 * at creation (create a new plan to change mu, lr, eps, ns_steps, nesterov,
 * weight decay or any scale).  Results are bit-identical to muon_step on
 * the same inputs.  The caller keeps every bound buffer, the workspace
 * included, alive and otherwise untouched until muon_plan_destroy has
 * returned (it waits for the last replay); replays of one plan are ordered
 * one after another by the library, and other work on the bound buffers
 * must be ordered against them by the caller.  A plan belongs
 * to the device current at creation; muon_plan_step on another device is
 * MUON_ERR_INVALID_ARG.  n must be >= 1.  The graph holds no memset node
 * (the per-step counter is zeroed by a kernel). */
typedef struct muon_plan_s* muon_plan_t;
muon_status_t muon_plan_create(const muon_matrix_t* mats, int64_t n, const muon_hparams_t* hp, void* workspace,
                               size_t workspace_bytes, void* stream, muon_plan_t* out);
/* A replay on `stream` is ordered after the plan's previous replay,
 * whichever stream that ran on. */
muon_status_t muon_plan_step(muon_plan_t plan, void* stream);
/* Waits for the plan's last replay to end, then frees its graph (NULL is a
 * no-op); afterwards the caller may release the bound buffers. */
muon_status_t muon_plan_destroy(muon_plan_t plan);

/* Per-matrix diagnostics of one step: the layer-wise quantities that the
 * practice checklist of the synthesis note asks a Muon run to record
 * (item 4 of its local-discussion part: update RMS per matrix shape,
 * weight RMS, norm dynamics), plus a
 * non-finite flag.  With N = rows * cols:
 *   momentum_norm  ||M||_F, M the Newton-Schulz input (section 4), from the
 *                  same float32 block sums as the normalisation
 *   direction_rms  ||O||_F / sqrt(N), O the orthogonalised direction as the
 *                  update applies it, before lr and scale
 *   update_rms     ||W_new - W_old||_F / sqrt(N), the step actually applied
 *                  (decay included), each difference formed in float32
 *   weight_rms     ||W_new||_F / sqrt(N)
 *   nonfinite      bit 0: M holds a NaN or an infinity; bit 1: W_new does
 * The sums of squares are accumulated in float32 per lane and in float64
 * across lanes and work-groups, in a fixed order (repeatable bit for bit).
 * 32 bytes per entry; reserved words are written as 0. */
typedef struct muon_diag {
  float momentum_norm;
  float direction_rms;
  float update_rms;
  float weight_rms;
  int32_t nonfinite;
  int32_t reserved[3];
} muon_diag_t;

/* muon_step plus diagnostics: identical W and B results, and diag[i]
 * (DEVICE memory, n entries, 4-byte aligned, caller-owned, disjoint from
 * every other buffer of the call) describes matrix i once the stream
 * reaches the end of the call.  Needs the same workspace as muon_step; one
 * extra launch (stage MUON_STAGE_DIAG).  diag == NULL is MUON_ERR_INVALID_ARG. */
muon_status_t muon_step_diag(const muon_matrix_t* mats, int64_t n, const muon_hparams_t* hp,
                             muon_diag_t* diag, void* workspace, size_t workspace_bytes,
                             void* stream);

/* Orthogonalisation alone: O[i] = NS(M[i]) for float32 row-major inputs
 * M[i] (rows[i] x cols[i]) into float32 outputs O[i] of the same shape,
 * with the same normalisation, transpose rule and iteration as muon_step.
 * For tests and measurement of the Newton-Schulz stage.  M and O are arrays
 * of n device pointers held in host memory. */
size_t muon_orthogonalize_workspace_bytes(const int64_t* rows, const int64_t* cols, int64_t n,
                                          int32_t ns_steps);
muon_status_t muon_orthogonalize(const float* const* M, float* const* O, const int64_t* rows,
                                 const int64_t* cols, int64_t n, int32_t ns_steps, float eps,
                                 void* workspace, size_t workspace_bytes, void* stream);

/* Host-only description of how a call would be executed (no GPU needed).
 * Fills `info`; if `per_matrix` is non-NULL it must hold n entries. */
typedef struct muon_plan_info {
  int64_t workspace_bytes;
  int64_t launches;          /* kernel launches per call                    */
  int64_t gram_tiles;        /* work-groups of one Gram launch              */
  int64_t poly_tiles;        /* work-groups of one polynomial launch        */
  int64_t bx_tiles;          /* work-groups of one BX + aX launch           */
  int64_t ew_blocks;         /* work-groups of the momentum/norm launch     */
  int32_t tile;              /* symmetric tile edge of the first group      */
  int32_t reserved;
} muon_plan_info_t;

typedef struct muon_matrix_plan {
  int32_t transposed;   /* 1 when rows > cols: the iteration runs on M^T          */
  int32_t m;            /* Gram side min(rows, cols)                              */
  int32_t n;            /* long side max(rows, cols)                              */
  int32_t m_pad;        /* padded Gram side of the iterate buffers (zeros)        */
  int32_t n_pad;        /* padded long side of the iterate buffers (zeros)        */
  int32_t tile;         /* tile edge of the symmetric products; 0 = float32 path  */
  int32_t bx_tile_rows; /* Gram-side tile height of the BX product (0 on float32) */
  int32_t bx_tile_cols; /* long-side tile width of the BX product (0 on float32)  */
  int32_t fused_update; /* 1: the last BX launch writes W (or O) itself, from the  */
                        /* float32 accumulator; 0: a separate update pass reads   */
                        /* the final iterate pair (hi + lo)                       */
  int32_t xcd_edges;    /* bit s (s = 0 Gram, 1 polynomial, 2 BX) set when one of */
                        /* the 8 XCDs starts its share of that grouped launch     */
                        /* inside (or at the first tile of) this matrix's tiles   */
  int64_t x_offset;     /* byte offset of the iterate buffers in the workspace    */
} muon_matrix_plan_t;

muon_status_t muon_plan_query(const muon_matrix_t* mats, int64_t n, const muon_hparams_t* hp,
                              muon_plan_info_t* info, muon_matrix_plan_t* per_matrix);

/* Stage timing.  When enabled (per process), every launch the library makes
 * is bracketed by HIP events on the stream it is launched on;
 * muon_profile_read waits for the recorded events, adds their elapsed times
 * per stage to `ms` and the launch counts to `launches` (arrays of
 * MUON_STAGE_COUNT entries, caller-owned host memory), and clears them. */
typedef enum muon_stage {
  MUON_STAGE_MOMENTUM = 0, /* momentum, Frobenius partial sums and the */
                           /* unnormalised bf16 pair (first iteration  */
                           /* applies the normalisation)               */
  MUON_STAGE_NORM = 1,     /* per-matrix norm reduction                */
  MUON_STAGE_PREP = 2,     /* normalised iterate, only for matrices    */
                           /* that cannot fold it (m <= 64, ns_steps 0,*/
                           /* ||M||_F outside [2^-50, 2^50])           */
  MUON_STAGE_GRAM = 3,     /* A = X X^T (upper tiles + mirror)         */
  MUON_STAGE_POLY = 4,     /* P = b A + c A A (upper tiles + mirror)   */
  MUON_STAGE_BX = 5,       /* X = a X + P X                            */
  MUON_STAGE_UPDATE = 6,   /* W -= lr * scale * O (or O store)         */
  MUON_STAGE_UPLOAD = 7,   /* descriptor table copy                    */
  MUON_STAGE_BX_UPDATE = 8, /* last X = a X + P X with W -= lr*scale*O  */
                            /* applied in the same launch (wide tiles)  */
  MUON_STAGE_DIAG = 9,      /* per-matrix diagnostics (muon_step_diag)  */
  MUON_STAGE_COUNT = 10
} muon_stage_t;

muon_status_t muon_profile_enable(int32_t on);
muon_status_t muon_profile_read(double* ms, int64_t* launches);

/* QK-Clip: after a step, rescale attention query and key projections head by
 * head from each head's max logit, to keep attention logits from growing
 * without bound.  The synthesis note's results section (result 3, Kimi K2's
 * MuonClip) describes this rescale after the Muon step without a formula or
 * threshold; the reading implemented: rows h*head_dim .. (h+1)*head_dim-1
 * of W belong to head h (the (out, in) layout of a projection), and when
 * max_logit[h] > tau they are multiplied by sqrt(tau / max_logit[h])
 * (float32 division and square root, correctly rounded; one rounding per
 * element).  Clipping the query and the key projection of one attention
 * layer with the same max_logit array scales every logit of a clipped head
 * by tau / max_logit[h], so its max logit becomes tau; heads at or below
 * tau (or with a NaN max logit) are not touched.  An infinite max logit
 * zeroes the head's rows.
 *   W          DEVICE, rows x cols float32 row-major, 16-byte aligned,
 *              updated in place; disjoint from every other W of the call
 *   rows, cols >= 1, <= MUON_MAX_DIM; rows a multiple of head_dim
 *   head_dim   >= 1
 *   max_logit  DEVICE, rows / head_dim float32 entries, 4-byte aligned,
 *              read only (Q and K of one layer may share it)
 * tau: finite, > 0.  mats is HOST memory read during the call.  One launch
 * per 48 matrices (the descriptors travel as kernel arguments; no
 * workspace); a head whose factor is 1 costs one read.  Stream-ordered:
 * call it after muon_step on the same stream. */
typedef struct muon_qk_clip_matrix {
  float* W;
  int64_t rows;
  int64_t cols;
  int32_t head_dim;
  int32_t reserved;
  const float* max_logit;
} muon_qk_clip_matrix_t;
muon_status_t muon_qk_clip(const muon_qk_clip_matrix_t* mats, int64_t n, float tau, void* stream);

/* Bandwidth yardstick for the HBM-bound stages (the measurement side of the
 * boundary, not part of a step): copies `bytes` from src to dst (DEVICE
 * memory, 16-byte aligned, bytes a multiple of 16, disjoint) with a plain
 * streaming kernel that reads and writes every byte once, on `stream`.
 * variant 0..MUON_COPY_PROBE_VARIANTS-1: bit 0 selects nontemporal loads and
 * stores, bits 1-2 the grid (1024, 4096 or 16384 work-groups of 256 lanes,
 * each lane with four 16-byte loads in flight).  A benchmark times the
 * variants and takes the fastest as the measured copy ceiling. */
#define MUON_COPY_PROBE_VARIANTS 6
muon_status_t muon_copy_probe(const void* src, void* dst, size_t bytes, int32_t variant, void* stream);

const char* muon_status_string(muon_status_t status);
/* Message of the last error on the calling thread ("" if none). */
const char* muon_last_error(void);
int32_t muon_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MUON_H_ */
