/*
 * engram.h - C ABI of the Engram conditional-memory forward pass on MI355X (gfx950).
 *
 * The Engram module (architecture walk-through at yaoyuxiang.cn/news/830577,
 * sections 2.2 and 4.2-4.3; formula sheet at kwkr.cn/news/37585, sections 1-5)
 * looks up hashed n-grams of compressed token ids in multi-head embedding
 * tables, gates the retrieved memory against the hidden state of each branch,
 * and smooths it with a short causal depthwise conv plus a residual:
 *
 *   x        = remap[ids]                                    (compressed ids)
 *   s_k[t]   = x[t-k], or pad_id before the sequence start    (time shift)
 *   mix_n[t] = xor_{k<n} s_k[t] * m_k   (wrapping int64)
 *   idx      = mix_n mod p_{n,j}        (floored, in [0, p))  per order n, head j
 *   e[t]     = concat_{n,j} table_{n,j}[idx]                  (E = H * head_dim)
 *   K_h      = W_k,h e,  V = W_v e                            (no bias)
 *   s_h      = <RMSNorm(K_h) * gk_h, RMSNorm(Q_h) * gq_h> / sqrt(d), Q_h = hidden[t][h]
 *   g_h      = sigmoid(sign(s_h) * sqrt(max(|s_h|, gate_clamp)))
 *   Vg_h[t]  = g_h[t] * V[t]
 *   out_h[t] = Vg_h[t] + sum_j w_h[j] * Vg_h[t - (conv_kernel-1-j) * dilation]
 *
 * Conventions for every call:
 *  - Array arguments are DEVICE pointers, allocated and owned by the caller.
 *    tables, w_kv, gamma_k, gamma_q, conv_w, hidden, out, e and the value
 *    ring are 16-byte aligned (ENGRAM_EINVAL otherwise); ids, remap, gates and
 *    float32 gradient arrays need 4 bytes.
 *    The library allocates no memory; calls on different streams with
 *    disjoint outputs may run concurrently.  Its only global state is the
 *    per-GPU device array of engram_forward_noalloc (and that array's address
 *    on each GPU).
 *  - Calls validate their arguments on the host, enqueue kernels on `stream`
 *    (NULL = the null stream) and return without waiting.  A status other than
 *    ENGRAM_OK means nothing was enqueued.  Faults inside kernels surface as HIP
 *    errors at the caller's next synchronisation.
 *  - Layouts are dense row-major with the last index fastest.  N = batch*seqlen.
 *  - dtype selects the storage of tables, weights, gammas, conv taps, hidden,
 *    out and the value history: float32, or bfloat16 with float32 accumulation.
 *  - Token ids outside [0, vocab) are read as pad_id.  The debug build of the
 *    library (compiled with ENGRAM_DEBUG) checks the ids of every call that
 *    reads them on the host first and returns ENGRAM_EINVAL for one outside
 *    that range (the call then waits for the stream's earlier work).
 *  - No C++ exception crosses this interface.
 */
#ifndef ENGRAM_H
#define ENGRAM_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ENGRAM_MAX_ORDERS 8
#define ENGRAM_MAX_HEADS 64
#define ENGRAM_MAX_BRANCHES 16
#define ENGRAM_MAX_CONV_KERNEL 8
#define ENGRAM_MAX_LAYERS 16

typedef enum {
  ENGRAM_OK = 0,
  ENGRAM_EINVAL = -1,       /* invalid configuration or argument */
  ENGRAM_ENOMEM = -2,       /* workspace smaller than engram_workspace_size() */
  ENGRAM_EHIP = -3,         /* a HIP launch or API call failed */
  ENGRAM_EUNSUPPORTED = -4  /* valid configuration outside what the kernels handle */
} engram_status;

typedef enum { ENGRAM_F32 = 0, ENGRAM_BF16 = 1 } engram_dtype;

/* Hyper-parameters of one Engram layer and the shape of one call.
 * Host memory, read during the call only. */
typedef struct engram_config {
  int32_t batch;            /* B sequences */
  int32_t seqlen;           /* T new tokens per sequence (T = 1 for a decode step) */
  int32_t vocab;            /* raw vocabulary size V; remap has V entries */
  int32_t n_orders;         /* number of n-gram orders, 1..ENGRAM_MAX_ORDERS */
  int32_t orders[ENGRAM_MAX_ORDERS];   /* ascending n-gram orders, each in 1..ENGRAM_MAX_ORDERS */
  int32_t heads_per_order;  /* hash heads per order; H = n_orders * heads_per_order <= ENGRAM_MAX_HEADS */
  int32_t head_dim;         /* embedding width of one head; E = H * head_dim, E % 8 == 0 */
  int32_t hidden;           /* d, hidden size of one branch; d % 8 == 0 */
  int32_t hc_mult;          /* branches (hyper-connection channels), 1..ENGRAM_MAX_BRANCHES */
  int32_t conv_kernel;      /* short-conv taps, 1..ENGRAM_MAX_CONV_KERNEL (4 on the pages) */
  int32_t conv_dilation;    /* >= 1 (the largest order on the pages) */
  int32_t pad_id;           /* compressed id hashed for positions before the sequence start */
  int32_t dtype;            /* engram_dtype */
  float norm_eps;           /* RMSNorm epsilon, >= 0 */
  float gate_clamp;         /* lower clamp of |s| before the square root (1e-6 on the pages), >= 0 */
  int64_t multipliers[ENGRAM_MAX_ORDERS]; /* m_k for k < largest order: m_k multiplies the token k back */
  int64_t primes[ENGRAM_MAX_HEADS];       /* modulus (table rows) of each head, order-major, 1..2^31-1 */
} engram_config;

/* Layer parameters (device pointers, read only). Head h's table occupies rows
 * [sum_{h'<h} primes[h'], + primes[h]) of one stacked table. */
typedef struct engram_params {
  const int32_t *remap;     /* [vocab] raw -> compressed id; NULL: ids are already compressed */
  const void *tables;       /* [sum primes][head_dim] dtype; device memory, or pinned host memory
                               mapped into the device (hipHostMalloc, address from
                               hipHostGetDevicePointer): rows are then read over the host link
                               by a gather limited to 32 workgroups, so that work on other
                               streams keeps the rest of the GPU */
  const void *w_kv;         /* [(hc_mult+1)*hidden][E] dtype: key rows of branch 0..hc-1, then value rows */
  const void *gamma_k;      /* [hc_mult][hidden] dtype, RMSNorm scale of the keys */
  const void *gamma_q;      /* [hc_mult][hidden] dtype, RMSNorm scale of the queries (hidden states) */
  const void *conv_w;       /* [hc_mult][hidden][conv_kernel] dtype; tap conv_kernel-1 is the current position */
} engram_params;

/* Per-sequence decode state (device arrays owned by the caller). Rings hold the
 * most recent positions: absolute position p lives in slot p % ring length.
 * n_past[b] counts the tokens sequence b has consumed; 0 means a fresh
 * sequence, whose rings need no initialisation. */
typedef struct engram_state {
  int32_t *tok_ring;        /* [B][max_order-1] compressed ids (unused when max_order == 1) */
  void *v_ring;             /* [B][R][hidden] dtype, value projections; R = (conv_kernel-1)*conv_dilation + 1 */
  float *g_ring;            /* [B][R][hc_mult] gates */
  int64_t *n_past;          /* [B] */
} engram_state;

/* Bytes of workspace engram_forward needs for this configuration (0 when
 * the configuration is invalid). */
size_t engram_workspace_size(const engram_config *cfg);

/* Bytes of decode state per sequence, summed over the three rings (0 when invalid). */
size_t engram_state_bytes_per_sequence(const engram_config *cfg);

/* N-gram hash indices (formula sheet 1.2-1.3, time shift 4.2; walk-through 4.2).
 * ids: [B][T] raw token ids.  st: NULL for fresh sequences (pad history), or a
 * state whose token ring and n_past supply the tokens before position 0; it is
 * read, not advanced.  idx_out: [B][T][H] int32, the row within head h's table. */
engram_status engram_hash(const engram_config *cfg, const engram_params *prm, const int32_t *ids,
                          const engram_state *st, int32_t *idx_out, hipStream_t stream);

/* Hash indices of several Engram layers in one pass (formula sheet 1.4: each
 * layer hashes with its own multipliers, seeded per layer; walk-through 4.3:
 * one hash call gives every layer's indices, each layer takes its own).  The
 * layers share cfg's orders, heads and primes; multipliers: HOST array
 * [n_layers][ENGRAM_MAX_ORDERS] int64, layer l's m_k at [l][k] (cfg->multipliers
 * is not used).  n_layers: 1..ENGRAM_MAX_LAYERS.  idx_out: [n_layers][B][T][H]
 * int32, layer l's block equal to engram_hash with that layer's multipliers.
 * ids and st as in engram_hash. */
engram_status engram_hash_layers(const engram_config *cfg, const engram_params *prm, const int32_t *ids,
                                 const engram_state *st, const int64_t *multipliers, int32_t n_layers,
                                 int32_t *idx_out, hipStream_t stream);

/* Multi-head embedding lookup and concatenation into e_t (walk-through 2.2-1
 * and 4.3).  idx: [B][T][H] as written by engram_hash; entries outside
 * [0, primes[h]) are clamped into range.  e_out: [B][T][E] dtype, exact copies
 * of the table rows. */
engram_status engram_gather(const engram_config *cfg, const engram_params *prm, const int32_t *idx,
                            void *e_out, hipStream_t stream);

/* The same lookup on the host, for tables kept in host memory (walk-through
 * 4.4, inference offload): e_out[n][h] = row idx[n][h] of head h's table, exact
 * copies, idx clamped like engram_gather.  tables, idx and e_out are HOST
 * pointers (e.g. pinned memory, idx copied back from engram_hash's output, e_out
 * then copied to the device by the DMA engines, so the lookup takes no compute
 * units from the GPU).  Runs on up to n_threads host threads (<= 0: the host's
 * cores, at most 16) and returns when the rows are copied; makes no HIP call. */
engram_status engram_gather_host(const engram_config *cfg, const void *tables, const int32_t *idx, void *e_out,
                                 int32_t n_threads);

/* Key and value projections (formula sheet 2.2 steps 1 and 3): kv_out[n] =
 * w_kv . e[n], i.e. [B][T][hc_mult+1][hidden] dtype with the keys of each
 * branch first and the shared value last.  bf16 uses MFMA with float32
 * accumulation and one rounding at the store. */
engram_status engram_project(const engram_config *cfg, const engram_params *prm, const void *e,
                             void *kv_out, hipStream_t stream);

/* Gate, value fusion, short conv and residual (formula sheet 2.2-2.3 and 3.2;
 * walk-through 2.2-3).  kv: [B][T][hc_mult+1][hidden] dtype from
 * engram_project; hidden: [B][T][hc_mult][hidden] dtype; st: NULL (zero
 * history) or a state whose rings supply V and g before position 0, read and
 * not advanced.  g_out: [B][T][hc_mult] float32, receives the gates (required:
 * the conv reads them back); out: [B][T][hc_mult][hidden] dtype. */
engram_status engram_gate_conv(const engram_config *cfg, const engram_params *prm, const void *kv,
                               const void *hidden, const engram_state *st, float *g_out, void *out,
                               hipStream_t stream);

/* The whole module (walk-through 4.3, Engram.forward): ids [B][T] raw ids,
 * hidden [B][T][hc_mult][hidden] -> out [B][T][hc_mult][hidden].  workspace:
 * device memory of at least engram_workspace_size(cfg) bytes (ENGRAM_ENOMEM if
 * shorter).  st: NULL, or a state that the call continues and then advances
 * (rings updated, n_past += T), so a prefill followed by decode steps gives the
 * outputs of one prefill over the whole sequence. */
engram_status engram_forward(const engram_config *cfg, const engram_params *prm, const int32_t *ids,
                             const void *hidden, engram_state *st, void *out, void *workspace,
                             size_t workspace_bytes, hipStream_t stream);

/* Largest workspace (engram_workspace_size) engram_forward_noalloc serves. */
#define ENGRAM_NOALLOC_MAX_BYTES ((size_t)64 << 20)

/* engram_forward without a workspace argument, for callers that cannot
 * allocate (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the workspace is a device array inside the library, one
 * copy of ENGRAM_NOALLOC_MAX_BYTES per GPU it runs on, held until the process
 * ends.  It serves the GPU current on the calling thread (the stream's device).
 * Configurations whose engram_workspace_size exceeds ENGRAM_NOALLOC_MAX_BYTES
 * (e.g. 4096 tokens at hidden 1024 fit, 32768 tokens at hidden 2560 do not)
 * return ENGRAM_ENOMEM before anything is enqueued.  The call allocates
 * nothing (no hipMalloc, hipFree or allocating library routine).  Every call
 * on one GPU shares that array: calls that may overlap on one GPU (other
 * streams, other threads) race, so the caller serialises them.  Otherwise as
 * engram_forward, with the same results bit for bit. */
engram_status engram_forward_noalloc(const engram_config *cfg, const engram_params *prm, const int32_t *ids,
                                     const void *hidden, engram_state *st, void *out, hipStream_t stream);

/* The module on rows gathered beforehand (walk-through 4.4, inference with the
 * tables in host memory: the hash depends only on the token ids, so the rows a
 * layer needs can be looked up and brought to the device while the layers
 * before it run; e.g. engram_hash + engram_gather from host-resident tables on
 * a side stream).  e: [B][T][E] dtype, as written by engram_gather, 16-byte
 * aligned; the tables are not read (prm->tables may be NULL).  ids: needed only
 * when st is not NULL (the state's token ring is advanced from them).  Otherwise
 * as engram_forward, with the same workspace size; the caller orders the
 * gather before this call (same stream, or an event). */
engram_status engram_forward_gathered(const engram_config *cfg, const engram_params *prm, const int32_t *ids,
                                      const void *e, const void *hidden, engram_state *st, void *out,
                                      void *workspace, size_t workspace_bytes, hipStream_t stream);

/* Bytes of workspace engram_backward needs (0 when the configuration is invalid). */
size_t engram_backward_workspace_size(const engram_config *cfg);

/* Gradients of the module (the backward pass of a training step; the
 * walk-through, 4.4, trains it): the exact derivatives of engram_forward
 * without a state, for an upstream gradient dy = dL/dout.  The forward
 * quantities are recomputed from the inputs (same arguments as
 * engram_forward); nothing from a previous forward call is needed.
 *   dy, d_hidden: [B][T][hc_mult][hidden] dtype; d_hidden is written.
 *   d_tables [sum primes][head_dim], d_w_kv [(hc_mult+1)*hidden][E],
 *   d_gamma_k, d_gamma_q [hc_mult][hidden], d_conv_w [hc_mult][hidden][conv_kernel]:
 *   float32, ADDED to (zero them for plain gradients; only the table rows the
 *   hashes select change).
 * The table rows' sums over tokens use float32 atomics, so their last bits may
 * differ between runs (the gammas' and taps' sums are taken in a fixed order);
 * the gradients must be device memory.
 * workspace: device memory of at least engram_backward_workspace_size(cfg)
 * bytes, 256-byte aligned.  ENGRAM_EINVAL for a NULL or misaligned pointer
 * (hidden, dy, d_hidden 16-byte aligned), ENGRAM_ENOMEM for a short workspace,
 * both before anything is launched.  The gate's slope 1/(2 sqrt|s|) makes the
 * gradients through it as sensitive to rounding as the score s is close to 0. */
engram_status engram_backward(const engram_config *cfg, const engram_params *prm, const int32_t *ids,
                              const void *hidden, const void *dy, void *d_hidden, float *d_tables, float *d_w_kv,
                              float *d_gamma_k, float *d_gamma_q, float *d_conv_w, void *workspace,
                              size_t workspace_bytes, hipStream_t stream);

/* The forward of a training step (no state): the same output as
 * engram_forward, within rounding (the gate's sums are taken by a separate
 * kernel rather than in the projection's epilogue), that also keeps in
 * `workspace` the forward quantities the gradients need: the gathered rows,
 * their indices, K/V and the gate statistics.  workspace: device memory of at
 * least engram_backward_workspace_size(cfg) bytes, 256-byte aligned, owned by
 * the caller and left untouched until the matching engram_backward_saved.
 * ENGRAM_EINVAL / ENGRAM_ENOMEM as engram_forward, before anything is launched. */
engram_status engram_forward_train(const engram_config *cfg, const engram_params *prm, const int32_t *ids,
                                   const void *hidden, void *out, void *workspace, size_t workspace_bytes,
                                   hipStream_t stream);

/* engram_backward on the forward quantities that engram_forward_train left in
 * `workspace` (same cfg, parameters and hidden; issued after it on the same
 * stream or ordered by an event): the recomputation is skipped, so neither the
 * ids nor the tables are read (prm->tables may be NULL).  Gradients, their
 * accumulation and the errors as engram_backward. */
engram_status engram_backward_saved(const engram_config *cfg, const engram_params *prm, const void *hidden,
                                    const void *dy, void *d_hidden, float *d_tables, float *d_w_kv,
                                    float *d_gamma_k, float *d_gamma_q, float *d_conv_w, void *workspace,
                                    size_t workspace_bytes, hipStream_t stream);

/* engram_backward with the table gradient in row-sparse form, for tables too
 * large for a dense float32 gradient (the walk-through, 4.4, trains tables of
 * up to 100B parameters; a step reads at most N * H of their rows): the rows
 * the step's hashes select, each once, ascending, with the sum of the
 * gradient over the (token, head) pairs that selected them.
 *   row_index [N*H] int64, 8-byte aligned: row_index[0 .. *n_rows) are the
 *     stacked-table rows (written);
 *   d_rows [N*H][head_dim] float32: d_rows[i] is row_index[i]'s gradient
 *     (written, not added to: the rows differ from step to step);
 *   n_rows [1] int64 (device memory, written; read it after the stream's work).
 * The other gradients as engram_backward (added to, or written for d_hidden);
 * the row sums use float32 atomics, so their last bits may differ between
 * runs.  ENGRAM_EUNSUPPORTED when N*H >= 2^31.  Workspace: the same
 * engram_backward_workspace_size.  Errors as engram_backward. */
engram_status engram_backward_sparse(const engram_config *cfg, const engram_params *prm, const int32_t *ids,
                                     const void *hidden, const void *dy, void *d_hidden, int64_t *row_index,
                                     float *d_rows, int64_t *n_rows, float *d_w_kv, float *d_gamma_k,
                                     float *d_gamma_q, float *d_conv_w, void *workspace, size_t workspace_bytes,
                                     hipStream_t stream);

/* engram_backward_saved with the table gradient in row-sparse form (as
 * engram_backward_sparse), on the forward quantities engram_forward_train
 * left in `workspace`. */
engram_status engram_backward_saved_sparse(const engram_config *cfg, const engram_params *prm, const void *hidden,
                                           const void *dy, void *d_hidden, int64_t *row_index, float *d_rows,
                                           int64_t *n_rows, float *d_w_kv, float *d_gamma_k, float *d_gamma_q,
                                           float *d_conv_w, void *workspace, size_t workspace_bytes,
                                           hipStream_t stream);

/* Same as engram_forward, additionally recording events[2i] / events[2i+1]
 * (caller-created hipEvent_t) on `stream` around the i-th kernel it launches,
 * for i < n_events/2.  Returns the number of kernels in *n_kernels (nullable).
 * Names of those kernels: engram_forward_kernel_name(cfg, st != NULL, i). */
engram_status engram_forward_timed(const engram_config *cfg, const engram_params *prm, const int32_t *ids,
                                   const void *hidden, engram_state *st, void *out, void *workspace,
                                   size_t workspace_bytes, hipStream_t stream, hipEvent_t *events,
                                   int32_t n_events, int32_t *n_kernels);

/* Static name of the i-th kernel engram_forward launches for cfg, with or
 * without a state (NULL past the end). */
const char *engram_forward_kernel_name(const engram_config *cfg, int32_t with_state, int32_t i);

/* Static description of a status code. */
const char *engram_status_string(engram_status status);

#ifdef __cplusplus
}
#endif

#endif /* ENGRAM_H */
