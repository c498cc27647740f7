// Host side of the Engram C ABI (include/engram.h): argument validation, the
// per-call hash constants, the workspace layout of engram_forward and the
// order of kernel launches; and the host-memory gather for tables kept in
// host memory.  Allocates nothing; its only mutable state is the per-device
// address of engram_forward_noalloc's device array.
#include <math.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <thread>
#include <vector>

#include "engram_internal.h"

using namespace engram;

// Device memory of engram_forward_noalloc, for callers that cannot allocate:
// one copy per GPU the library runs on, held until the process ends.  Host
// code never uses this name as an address: each device's copy is looked up
// once with hipGetSymbolAddress and that address is what the kernels get.
constexpr size_t kScratchBytes = ENGRAM_NOALLOC_MAX_BYTES;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {

int max_order(const engram_config* c) { return c->orders[c->n_orders - 1]; }
int n_heads(const engram_config* c) { return c->n_orders * c->heads_per_order; }
int64_t emb_dim(const engram_config* c) { return (int64_t)n_heads(c) * c->head_dim; }
int64_t esize(const engram_config* c) { return c->dtype == ENGRAM_BF16 ? 2 : 4; }
// Positions the value and gate rings keep: the conv's history (K-1) D plus
// one, so that a decode step's new position never takes a slot the history
// reads (the decode tail writes the ring while other workgroups read it).
int ring_len(const engram_config* c) { return (c->conv_kernel - 1) * c->conv_dilation + 1; }

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

engram_status validate(const engram_config* c) {
  if (c == nullptr) return ENGRAM_EINVAL;
  if (c->batch < 0 || c->seqlen < 0 || c->vocab < 1) return ENGRAM_EINVAL;
  if ((int64_t)c->batch * c->seqlen > INT32_MAX / 2) return ENGRAM_EUNSUPPORTED;
  if (c->n_orders < 1 || c->n_orders > ENGRAM_MAX_ORDERS) return ENGRAM_EINVAL;
  for (int i = 0; i < c->n_orders; i++) {
    if (c->orders[i] < 1 || c->orders[i] > ENGRAM_MAX_ORDERS) return ENGRAM_EINVAL;
    if (i > 0 && c->orders[i] <= c->orders[i - 1]) return ENGRAM_EINVAL;
  }
  if (c->heads_per_order < 1 || n_heads(c) > ENGRAM_MAX_HEADS) return ENGRAM_EINVAL;
  for (int h = 0; h < n_heads(c); h++)
    if (c->primes[h] < 1 || c->primes[h] > INT32_MAX) return ENGRAM_EINVAL;
  if (c->dtype != ENGRAM_F32 && c->dtype != ENGRAM_BF16) return ENGRAM_EINVAL;
  if (c->head_dim < 1 || c->hidden < 1 || c->hc_mult < 1 || c->hc_mult > ENGRAM_MAX_BRANCHES) return ENGRAM_EINVAL;
  if (c->conv_kernel < 1 || c->conv_kernel > ENGRAM_MAX_CONV_KERNEL || c->conv_dilation < 1) return ENGRAM_EINVAL;
  if (!(c->norm_eps >= 0.f) || !(c->gate_clamp >= 0.f)) return ENGRAM_EINVAL;
  // 16-byte vectors along the hidden and embedding axes
  if (c->hidden % 8 != 0 || emb_dim(c) % 8 != 0) return ENGRAM_EUNSUPPORTED;
  if ((int64_t)(c->hc_mult + 1) * c->hidden > INT32_MAX / 4 || emb_dim(c) > INT32_MAX / 4) return ENGRAM_EUNSUPPORTED;
  if ((int64_t)c->conv_kernel * c->conv_dilation > INT32_MAX / 4) return ENGRAM_EUNSUPPORTED;
  return ENGRAM_OK;
}

engram_status check_params(const engram_config* c, const engram_params* p) {
  (void)c;
  if (p == nullptr || p->tables == nullptr || p->w_kv == nullptr || p->gamma_k == nullptr ||
      p->gamma_q == nullptr || p->conv_w == nullptr)
    return ENGRAM_EINVAL;
  if (!aligned(p->tables, 16) || !aligned(p->w_kv, 16) || !aligned(p->gamma_k, 16) || !aligned(p->gamma_q, 16) ||
      !aligned(p->conv_w, 16))
    return ENGRAM_EINVAL;
  return ENGRAM_OK;
}

// Grid cap of the gather when the tables are pinned host memory mapped into
// the device: 32 workgroups keep ~1 MB of row loads in flight, enough for the
// host link, and leave the other CUs to the work the prefetch overlaps.
constexpr int kHostGatherBlocks = 32;

int gather_grid_cap(const void* tables) {
  hipPointerAttribute_t at;
  const hipError_t pending = hipPeekAtLastError();
  if (hipPointerGetAttributes(&at, tables) != hipSuccess) {
    // not known to the runtime: treat as device memory; clear the query's own
    // error, but never one the caller had pending
    if (pending == hipSuccess) (void)hipGetLastError();
    return 0;
  }
  return at.type == hipMemoryTypeHost ? kHostGatherBlocks : 0;
}

#ifdef ENGRAM_DEBUG
// Debug builds only: the raw ids of a call must lie in [0, vocab) (release
// builds hash an id outside that range as pad_id).  The ids are copied to the
// host after the stream's earlier work, so the call waits.
engram_status check_ids(const engram_config* c, const int32_t* ids, hipStream_t s) {
  const int64_t n = (int64_t)c->batch * c->seqlen;
  if (n == 0 || ids == nullptr) return ENGRAM_OK;
  int32_t* h = (int32_t*)malloc((size_t)n * sizeof(int32_t));
  if (h == nullptr) return ENGRAM_EUNSUPPORTED;
  engram_status rc = ENGRAM_OK;
  if (hipStreamSynchronize(s) != hipSuccess || hipMemcpy(h, ids, (size_t)n * sizeof(int32_t), hipMemcpyDefault))
    rc = ENGRAM_EHIP;
  for (int64_t i = 0; rc == ENGRAM_OK && i < n; i++)
    if (h[i] < 0 || h[i] >= c->vocab) rc = ENGRAM_EINVAL;
  free(h);
  return rc;
}
#else
engram_status check_ids(const engram_config*, const int32_t*, hipStream_t) { return ENGRAM_OK; }
#endif

// the same, for calls that do not read the tables
engram_status check_params_no_tables(const engram_config* c, const engram_params* p) {
  (void)c;
  if (p == nullptr || p->w_kv == nullptr || p->gamma_k == nullptr || p->gamma_q == nullptr || p->conv_w == nullptr)
    return ENGRAM_EINVAL;
  if (!aligned(p->w_kv, 16) || !aligned(p->gamma_k, 16) || !aligned(p->gamma_q, 16) || !aligned(p->conv_w, 16))
    return ENGRAM_EINVAL;
  return ENGRAM_OK;
}

engram_status check_state(const engram_config* c, const engram_state* st) {
  if (st == nullptr) return ENGRAM_OK;
  if (st->n_past == nullptr) return ENGRAM_EINVAL;
  if (max_order(c) > 1 && st->tok_ring == nullptr) return ENGRAM_EINVAL;
  if (ring_len(c) > 0 && (st->v_ring == nullptr || st->g_ring == nullptr || !aligned(st->v_ring, 16)))
    return ENGRAM_EINVAL;
  return ENGRAM_OK;
}

void make_hash_consts(const engram_config* c, HashConsts* hc) {
  memset(hc, 0, sizeof(*hc));
  hc->n_orders = c->n_orders;
  hc->heads_per_order = c->heads_per_order;
  hc->n_heads = n_heads(c);
  hc->max_order = max_order(c);
  hc->pad_id = c->pad_id;
  hc->vocab = c->vocab;
  for (int i = 0; i < c->n_orders; i++) hc->orders[i] = c->orders[i];
  for (int k = 0; k < ENGRAM_MAX_ORDERS; k++) hc->mult[k] = (uint64_t)c->multipliers[k];
  int64_t off = 0;
  for (int h = 0; h < n_heads(c); h++) {
    const uint64_t p = (uint64_t)c->primes[h];
    hc->prime[h] = (uint32_t)p;
    hc->magic[h] = UINT64_MAX / p;
    hc->wrap[h] = (uint32_t)((UINT64_MAX % p + 1) % p);
    hc->row_off[h] = off;
    off += (int64_t)p;
  }
}

engram_status hip_status(hipError_t e) { return e == hipSuccess ? ENGRAM_OK : ENGRAM_EHIP; }

// Address of the current device's copy of `scratch`, looked up on the first
// call on that device (with that device current) and kept.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

engram_status device_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return ENGRAM_EHIP;
  if (dev < 0 || dev >= kMaxDevices) return ENGRAM_EUNSUPPORTED;
  try {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
      void* p = nullptr;
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return ENGRAM_EHIP;
      g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
  } catch (...) {
    return ENGRAM_EHIP;
  }
  return ENGRAM_OK;
}

size_t align_up(size_t x) { return (x + 255) & ~(size_t)255; }

// engram_forward runs the fused path (projection GEMM with the gate sums in
// its epilogue, then a small finalize kernel) when the weights are bf16 and the
// GEMM's channel tile divides the hidden size -- for some shapes with the value
// channels as a plain GEMM after the key channels (gemm_gate_plan); otherwise
// the projections are stored and a separate gate kernel reads them back.
GatePlan gate_plan(const engram_config* c) {
  if (c->dtype != ENGRAM_BF16) return GatePlan{0, false};
  return gemm_gate_plan((int64_t)c->batch * c->seqlen, c->hc_mult, c->hidden);
}

int fused_tile(const engram_config* c) { return gate_plan(c).tile; }

struct Workspace {
  void* e;         // [N][E]
  void* kv;        // unfused: [N][hc+1][d]
  void* v;         // fused: [N][d]
  float4* part;    // fused: [N][hc][d / 128]
  float* g;        // [N][hc]
  int64_t* past;   // [B]: n_past before the call (decode steps with a state)
  size_t bytes;
};

Workspace carve(const engram_config* c, void* base) {
  const int64_t N = (int64_t)c->batch * c->seqlen;
  const int tile = fused_tile(c);
  Workspace w = {};
  size_t off = 0;
  auto take = [&](size_t n) {
    void* p = (uint8_t*)base + off;
    off += align_up(n);
    return p;
  };
  w.e = take((size_t)N * emb_dim(c) * esize(c));
  if (tile) {
    w.v = take((size_t)N * c->hidden * esize(c));
    w.part = (float4*)take((size_t)N * c->hc_mult * (c->hidden / 128) * sizeof(float4));
  } else {
    w.kv = take((size_t)N * (c->hc_mult + 1) * c->hidden * esize(c));
  }
  w.g = (float*)take((size_t)N * c->hc_mult * sizeof(float));
  w.past = (int64_t*)take((size_t)c->batch * sizeof(int64_t));
  w.bytes = off;
  return w;
}

// Workspace of engram_backward: the forward quantities it recomputes, the
// gradients between steps and, where dW cannot read dkv and e as stored
// (float32, or chunks past 32-bit buffer offsets), their transposed copies
// (token axis padded to a multiple of 64 with zeros).
struct BwdWorkspace {
  void* e;          // [N][E]
  int32_t* idx;     // [N][H]
  void* kv;         // [N][hc+1][d]
  float4* stats;    // [N][hc] (g, s, rk, rq)
  float4* part;     // [N][hc][d/128]: the fused projection's gate sums (when the fused plan applies)
  float* g;         // [N][hc] gates (the conv of engram_forward_train reads them)
  void* dvg;        // [N][hc][d] dtype: gradient of the gated values (hc not a power of two)
  float* dgp;       // [N][n_dgp][hc]: dg partials of the fused conv kernel (hc a power of two)
  void* dkv;        // [N][hc+1][d]
  float* de;        // [N][E]
  void* wT;         // [E][(hc+1)d]
  void* dkvT;       // [S][(hc+1)d][Np/S]: token axis in S split-K chunks (null when dW reads dkv and e as stored)
  void* eT;         // [S][E][Np/S] (null alike)
  float* wpart;     // [S][(hc+1)d][E] when S > 1: the splits' products
  float* gpart;     // [gate_bwd_rows(N)][hc][d]: per-block sums for the gammas' gradients
  float* cpart;     // [conv_bwd_rows][hc][d][K]: per-block sums for the taps' gradients
  uint32_t* bits;   // row-sparse table gradient: [sparse_bitmap_words] bitmap of the rows used
  uint32_t* count;  // [sparse_groups] set bits per group of the bitmap
  uint32_t* first;  // [sparse_groups] first rank of each group
  uint32_t* bsum;   // [sparse_scan_blocks] block offsets of the group ranks
  uint32_t* wrank;  // [sparse_bitmap_words] first rank of each bitmap word
  uint32_t* rank;   // [N][H] rank of each pair's row
  int64_t Np;       // S chunks of Ks tokens (multiples of 64), zero past N
  int64_t Ks;
  int S;
  size_t bytes;
};

// dW = dKV^T e over the token axis, in `splits` chunks of Ks tokens, read from
// dkv [N][(hc+1)d] and e [N][E] as stored (bf16 path)
GemmTnArgs dw_args(const engram_config* c, const void* dkv, const void* e, float* out, int splits, int64_t Ks) {
  GemmTnArgs g;
  g.A = dkv;
  g.B = e;
  g.C = out;
  g.M = (int32_t)((int64_t)(c->hc_mult + 1) * c->hidden);
  g.N = (int32_t)emb_dim(c);
  g.K = (int64_t)c->batch * c->seqlen;
  g.Ks = Ks;
  g.lda = g.M;
  g.ldb = g.N;
  g.splits = splits;
  g.split_c = (int64_t)g.M * g.N;
  g.accumulate = splits > 1 ? 0 : 1;
  return g;
}

BwdWorkspace carve_bwd(const engram_config* c, void* base) {
  const int64_t N = (int64_t)c->batch * c->seqlen, E = emb_dim(c), O = (int64_t)(c->hc_mult + 1) * c->hidden;
  const int64_t es = esize(c);
  BwdWorkspace w = {};
  w.S = c->dtype == ENGRAM_BF16 ? gemm_k_splits(O, E, N) : 1;
  w.Ks = (N + (int64_t)w.S * 64 - 1) / ((int64_t)w.S * 64) * 64;
  w.Np = w.S * w.Ks;
  size_t off = 0;
  auto take = [&](size_t n) {
    void* p = (uint8_t*)base + off;
    off += align_up(n);
    return p;
  };
  w.e = take((size_t)(N * E * es));
  w.idx = (int32_t*)take((size_t)N * n_heads(c) * sizeof(int32_t));
  w.kv = take((size_t)(N * O * es));
  w.stats = (float4*)take((size_t)N * c->hc_mult * sizeof(float4));
  if (fused_tile(c)) w.part = (float4*)take((size_t)N * c->hc_mult * (c->hidden / 128) * sizeof(float4));
  w.g = (float*)take((size_t)N * c->hc_mult * sizeof(float));
  if (conv_bwd_fused(c->hc_mult))
    w.dgp = (float*)take((size_t)N * c->hc_mult * conv_bwd_dg_parts(c->hc_mult, c->hidden) * sizeof(float));
  else
    w.dvg = take((size_t)(N * c->hc_mult * c->hidden * es));
  w.dkv = take((size_t)(N * O * es));
  w.de = (float*)take((size_t)(N * E) * sizeof(float));
  w.wT = take((size_t)(E * O * es));
  if (c->dtype != ENGRAM_BF16 || !gemm_tn_fits(dw_args(c, nullptr, nullptr, nullptr, w.S, w.Ks))) {
    w.dkvT = take((size_t)(O * w.Np * es));
    w.eT = take((size_t)(E * w.Np * es));
  }
  w.wpart = w.S > 1 ? (float*)take((size_t)w.S * O * E * sizeof(float)) : nullptr;
  w.gpart = (float*)take((size_t)gate_bwd_rows(N) * c->hc_mult * c->hidden * sizeof(float));
  w.cpart = (float*)take((size_t)conv_bwd_rows(c->batch, c->seqlen) * c->hc_mult * c->hidden * c->conv_kernel *
                         sizeof(float));
  int64_t rows = 0;
  for (int h = 0; h < n_heads(c); h++) rows += c->primes[h];
  w.bits = (uint32_t*)take((size_t)sparse_bitmap_words(rows) * sizeof(uint32_t));
  w.count = (uint32_t*)take((size_t)sparse_groups(rows) * sizeof(uint32_t));
  w.first = (uint32_t*)take((size_t)sparse_groups(rows) * sizeof(uint32_t));
  w.bsum = (uint32_t*)take((size_t)sparse_scan_blocks(rows) * sizeof(uint32_t));
  w.wrank = (uint32_t*)take((size_t)sparse_bitmap_words(rows) * sizeof(uint32_t));
  w.rank = (uint32_t*)take((size_t)N * n_heads(c) * sizeof(uint32_t));
  w.bytes = off;
  return w;
}

const char* const kForwardKernels[] = {"hash_gather", "project_gemm", "gate", "short_conv", "advance_state"};
const char* const kFusedKernels[] = {"hash_gather", "project_gate_gemm", "gate_finalize", "short_conv",
                                     "advance_state"};
const char* const kSplitKernels[] = {"hash_gather", "project_gate_gemm", "project_value_gemm", "short_conv",
                                     "advance_state"};
const char* const kDecodeKernels[] = {"hash_gather", "project_gate_gemm", "decode_tail"};

// A decode step (T = 1) with a state on the fused, unsplit projection ends in
// one kernel (k_decode_tail) instead of gate_finalize, short_conv and
// advance_state.
bool decode_tail_path(const engram_config* c, bool with_state, bool gathered) {
  const GatePlan p = gate_plan(c);
  return with_state && !gathered && c->seqlen == 1 && p.tile && !p.split;
}

// The kernels a forward call launches, in order: *n of them from names[0]
// (gathered: without the hash and gather).
const char* const* forward_kernels(const engram_config* c, bool with_state, bool gathered, int* n) {
  if (decode_tail_path(c, with_state, gathered)) {
    *n = 3;
    return kDecodeKernels;
  }
  const GatePlan plan = gate_plan(c);
  const char* const* names = plan.split ? kSplitKernels : plan.tile ? kFusedKernels : kForwardKernels;
  *n = with_state ? 5 : 4;   // advance_state is last
  if (gathered) {
    *n -= 1;
    return names + 1;
  }
  return names;
}

GatherArgs gather_args(const engram_config* c, const engram_params* p, const int32_t* ids, const engram_state* st) {
  GatherArgs a;
  memset(&a, 0, sizeof a);
  a.ids = ids;
  a.remap = p->remap;
  a.tables = (const uint8_t*)p->tables;
  a.tok_ring = st ? st->tok_ring : nullptr;
  a.n_past = st ? st->n_past : nullptr;
  a.batch = c->batch;
  a.seqlen = c->seqlen;
  a.row_bytes = (int32_t)(c->head_dim * esize(c));
  return a;
}

GemmArgs gemm_args(const engram_config* c, const engram_params* p, const void* e, void* kv) {
  GemmArgs g;
  g.A = e;
  g.B = p->w_kv;
  g.C = kv;
  g.M = c->batch * c->seqlen;
  g.N = (c->hc_mult + 1) * c->hidden;
  g.K = (int32_t)emb_dim(c);
  return g;
}

GateArgs gate_args(const engram_config* c, const engram_params* p, const void* kv, const void* hidden, float* g) {
  GateArgs a;
  a.kv = kv;
  a.hidden = hidden;
  a.gamma_k = p->gamma_k;
  a.gamma_q = p->gamma_q;
  a.g_out = g;
  a.n_tok = c->batch * c->seqlen;
  a.hc = c->hc_mult;
  a.d = c->hidden;
  a.eps = c->norm_eps;
  a.clamp = c->gate_clamp;
  a.inv_sqrt_d = (float)(1.0 / sqrt((double)c->hidden));
  a.bf16 = c->dtype == ENGRAM_BF16;
  return a;
}

// value rows: the last block of kv rows (stride (hc+1)*d), or a [N][d] array
ConvArgs conv_args(const engram_config* c, const engram_params* p, const void* v, int64_t v_stride, const float* g,
                   void* out, const engram_state* st) {
  ConvArgs a;
  a.v = v;
  a.v_stride = v_stride;
  a.g = g;
  a.conv_w = p->conv_w;
  a.out = out;
  a.v_ring = st ? st->v_ring : nullptr;
  a.g_ring = st ? st->g_ring : nullptr;
  a.n_past = st ? st->n_past : nullptr;
  a.batch = c->batch;
  a.seqlen = c->seqlen;
  a.hc = c->hc_mult;
  a.d = c->hidden;
  a.ksize = c->conv_kernel;
  a.dil = c->conv_dilation;
  a.bf16 = c->dtype == ENGRAM_BF16;
  return a;
}

// Records events[2i] before and events[2i+1] after launch i when asked to.
struct Timer {
  hipEvent_t* ev;
  int n_ev;
  int i = 0;
  hipStream_t s;
  hipError_t before() { return (ev && 2 * i + 1 < n_ev) ? hipEventRecord(ev[2 * i], s) : hipSuccess; }
  hipError_t after() {
    hipError_t e = (ev && 2 * i + 1 < n_ev) ? hipEventRecord(ev[2 * i + 1], s) : hipSuccess;
    i++;
    return e;
  }
};

// The forward pass.  gathered == false: the hash and gather run first (K1)
// into the workspace.  gathered == true: e_in holds the rows already gathered
// (the caller's prefetch) and K1 is skipped; the tables are not read, and ids
// are needed only to advance a state.
engram_status forward_impl(const engram_config* c, const engram_params* p, const int32_t* ids, bool gathered,
                           const void* e_in, const void* hidden, engram_state* st, void* out, void* ws,
                           size_t ws_bytes, hipStream_t s, hipEvent_t* ev, int32_t n_ev, int32_t* n_kernels) {
  engram_status rc = validate(c);
  if (rc) return rc;
  if ((rc = gathered ? check_params_no_tables(c, p) : check_params(c, p))) return rc;
  if ((rc = check_state(c, st))) return rc;
  const int64_t N = (int64_t)c->batch * c->seqlen;
  const GatePlan plan = gate_plan(c);
  const bool tail = decode_tail_path(c, st != nullptr, gathered);
  int nk = 0;
  (void)forward_kernels(c, st != nullptr, gathered, &nk);
  if (n_kernels) *n_kernels = N == 0 ? 0 : nk;
  if (N == 0) return ENGRAM_OK;
  if ((!gathered || st != nullptr) && ids == nullptr) return ENGRAM_EINVAL;
  if (gathered && (e_in == nullptr || !aligned(e_in, 16))) return ENGRAM_EINVAL;
  if (hidden == nullptr || out == nullptr || ws == nullptr) return ENGRAM_EINVAL;
  if (!aligned(hidden, 16) || !aligned(out, 16) || !aligned(ws, 256)) return ENGRAM_EINVAL;
  const Workspace w = carve(c, ws);
  if (ws_bytes < w.bytes) return ENGRAM_ENOMEM;
  const bool bf16 = c->dtype == ENGRAM_BF16;
  if ((!gathered || st != nullptr) && (rc = check_ids(c, ids, s))) return rc;

  HashConsts hc;
  make_hash_consts(c, &hc);
  Timer tm{ev, n_ev, 0, s};
  hipError_t e;

  const void* e_rows = e_in;
  if (!gathered) {
    GatherArgs ga = gather_args(c, p, ids, st);
    ga.e_out = (uint8_t*)w.e;
    if (tail) ga.past_out = w.past;
    const int cap = gather_grid_cap(p->tables);
    if ((e = tm.before()) || (e = launch_hash_gather(hc, ga, true, s, cap)) || (e = tm.after()))
      return hip_status(e);
    e_rows = w.e;
  }

  const void* v;
  int64_t v_stride;
  if (w.kv == nullptr) {  // fused: projections with the gate sums, then g
    GemmGateArgs gg;
    gg.g = gemm_args(c, p, e_rows, nullptr);
    gg.hidden = hidden;
    gg.gamma_k = p->gamma_k;
    gg.gamma_q = p->gamma_q;
    gg.v_out = w.v;
    gg.partials = w.part;
    gg.hc = c->hc_mult;
    gg.d = c->hidden;
    gg.tile_n = plan.tile;
    if (plan.split) gg.g.N = c->hc_mult * c->hidden;   // key channels only
    if ((e = tm.before()) || (e = launch_gemm_gate_bf16(gg, s)) || (e = tm.after())) return hip_status(e);
    if (tail) {
      DecodeTailArgs dt;
      dt.partials = w.part;
      dt.v = w.v;
      dt.conv_w = p->conv_w;
      dt.out = out;
      dt.past = w.past;
      dt.ids = ids;
      dt.remap = p->remap;
      dt.vocab = c->vocab;
      dt.pad_id = c->pad_id;
      dt.tok_ring = st->tok_ring;
      dt.v_ring = st->v_ring;
      dt.g_ring = st->g_ring;
      dt.n_past = st->n_past;
      dt.batch = c->batch;
      dt.hc = c->hc_mult;
      dt.d = c->hidden;
      dt.ksize = c->conv_kernel;
      dt.dil = c->conv_dilation;
      dt.n_part = c->hidden / 128;
      dt.ring_len = ring_len(c);
      dt.tok_ring_len = max_order(c) - 1;
      dt.eps = c->norm_eps;
      dt.clamp = c->gate_clamp;
      dt.inv_sqrt_d = (float)(1.0 / sqrt((double)c->hidden));
      dt.bf16 = bf16;
      if ((e = tm.before()) || (e = launch_decode_tail(dt, s)) || (e = tm.after())) return hip_status(e);
      return ENGRAM_OK;
    }
    GateFinalizeArgs gf;
    gf.partials = w.part;
    gf.g_out = w.g;
    gf.n_tok = (int32_t)N;
    gf.hc = c->hc_mult;
    gf.d = c->hidden;
    gf.n_part = c->hidden / 128;   // one partial per 128 channels, whatever the tile
    gf.eps = c->norm_eps;
    gf.clamp = c->gate_clamp;
    gf.inv_sqrt_d = (float)(1.0 / sqrt((double)c->hidden));
    if (plan.split) {   // value channels: V = W_v e into the workspace, and the gates on the way
      GemmArgs gv = gemm_args(c, p, e_rows, w.v);
      gv.B = (const uint8_t*)p->w_kv + (int64_t)c->hc_mult * c->hidden * emb_dim(c) * esize(c);
      gv.N = c->hidden;
      if ((e = tm.before()) || (e = launch_gemm_bf16(gv, s, &gf)) || (e = tm.after())) return hip_status(e);
    } else if ((e = tm.before()) || (e = launch_gate_finalize(gf, s)) || (e = tm.after())) {
      return hip_status(e);
    }
    v = w.v;
    v_stride = c->hidden;
  } else {
    const GemmArgs gm = gemm_args(c, p, e_rows, w.kv);
    if ((e = tm.before()) || (e = bf16 ? launch_gemm_bf16(gm, s) : launch_gemm_f32(gm, s)) || (e = tm.after()))
      return hip_status(e);
    const GateArgs gt = gate_args(c, p, w.kv, hidden, w.g);
    if ((e = tm.before()) || (e = launch_gate(gt, s)) || (e = tm.after())) return hip_status(e);
    v = (const uint8_t*)w.kv + (int64_t)c->hc_mult * c->hidden * esize(c);
    v_stride = (int64_t)(c->hc_mult + 1) * c->hidden;
  }

  const ConvArgs cv = conv_args(c, p, v, v_stride, w.g, out, st);
  if ((e = tm.before()) || (e = launch_conv(cv, s)) || (e = tm.after())) return hip_status(e);

  if (st) {
    AdvanceArgs ad;
    ad.ids = ids;
    ad.remap = p->remap;
    ad.vocab = c->vocab;
    ad.pad_id = c->pad_id;
    ad.v = cv.v;
    ad.v_stride = cv.v_stride;
    ad.g = w.g;
    ad.tok_ring = st->tok_ring;
    ad.v_ring = st->v_ring;
    ad.g_ring = st->g_ring;
    ad.n_past = st->n_past;
    ad.batch = c->batch;
    ad.seqlen = c->seqlen;
    ad.hc = c->hc_mult;
    ad.d = c->hidden;
    ad.tok_ring_len = max_order(c) - 1;
    ad.ring_len = ring_len(c);
    ad.bf16 = bf16;
    if ((e = tm.before()) || (e = launch_advance(ad, s)) || (e = tm.after())) return hip_status(e);
  }
  return ENGRAM_OK;
}

// The table gradient in row-sparse form: the rows used, ascending, their
// gradients and their count (all device memory, written).
struct SparseOut {
  int64_t* row_index;
  float* d_rows;
  int64_t* n_rows;
};

// Checks shared by the backward entry points (ids only when the forward
// quantities are recomputed).
engram_status check_backward(const engram_config* cfg, const engram_params* prm, bool need_ids, const int32_t* ids,
                             const void* hidden, const void* dy, void* d_hidden, float* d_tables, float* d_w_kv,
                             float* d_gamma_k, float* d_gamma_q, float* d_conv_w, void* workspace,
                             size_t workspace_bytes, const SparseOut* sp = nullptr) {
  engram_status rc = validate(cfg);
  if (rc) return rc;
  if ((rc = need_ids ? check_params(cfg, prm) : check_params_no_tables(cfg, prm))) return rc;
  if ((int64_t)cfg->batch * cfg->seqlen == 0) return ENGRAM_OK;
  if (sp) {   // ranks are 32-bit
    if ((int64_t)cfg->batch * cfg->seqlen * n_heads(cfg) >= INT32_MAX) return ENGRAM_EUNSUPPORTED;
    if (sp->row_index == nullptr || sp->d_rows == nullptr || sp->n_rows == nullptr || !aligned(sp->row_index, 8) ||
        !aligned(sp->d_rows, 4) || !aligned(sp->n_rows, 8))
      return ENGRAM_EINVAL;
  } else if (d_tables == nullptr || !aligned(d_tables, 4)) {
    return ENGRAM_EINVAL;
  }
  if ((need_ids && ids == nullptr) || hidden == nullptr || dy == nullptr || d_hidden == nullptr ||
      d_w_kv == nullptr || d_gamma_k == nullptr || d_gamma_q == nullptr || d_conv_w == nullptr ||
      workspace == nullptr)
    return ENGRAM_EINVAL;
  if (!aligned(hidden, 16) || !aligned(dy, 16) || !aligned(d_hidden, 16) || !aligned(workspace, 256) ||
      !aligned(d_w_kv, 4) || !aligned(d_gamma_k, 4) || !aligned(d_gamma_q, 4) || !aligned(d_conv_w, 4))
    return ENGRAM_EINVAL;
  if (workspace_bytes < carve_bwd(cfg, nullptr).bytes) return ENGRAM_ENOMEM;
  return ENGRAM_OK;
}

// The forward quantities the gradients need, into the workspace: rows and
// indices, K/V, the gate statistics (and the gates alone, for a conv).
hipError_t forward_quantities(const engram_config* cfg, const engram_params* prm, const int32_t* ids,
                              const void* hidden, const BwdWorkspace& w, hipStream_t stream) {
  const bool bf16 = cfg->dtype == ENGRAM_BF16;
  HashConsts hc;
  make_hash_consts(cfg, &hc);
  hipError_t e;
  GatherArgs ga = gather_args(cfg, prm, ids, nullptr);
  ga.idx_out = w.idx;
  ga.e_out = (uint8_t*)w.e;
  if ((e = launch_hash_gather(hc, ga, true, stream, gather_grid_cap(prm->tables)))) return e;
  const GatePlan plan = gate_plan(cfg);
  if (w.part == nullptr) {   // K/V stored, then the gate statistics from them
    const GemmArgs gm = gemm_args(cfg, prm, w.e, w.kv);
    if ((e = bf16 ? launch_gemm_bf16(gm, stream) : launch_gemm_f32(gm, stream))) return e;
    GateArgs gt = gate_args(cfg, prm, w.kv, hidden, w.g);
    gt.stats = w.stats;
    return launch_gate(gt, stream);
  }
  // the fused projection as in engram_forward, with the keys stored as well,
  // and the statistics formed from its sums
  const int64_t hcd = (int64_t)cfg->hc_mult * cfg->hidden, O = hcd + cfg->hidden;
  GemmGateArgs gg;
  gg.g = gemm_args(cfg, prm, w.e, nullptr);
  gg.hidden = hidden;
  gg.gamma_k = prm->gamma_k;
  gg.gamma_q = prm->gamma_q;
  gg.v_out = (uint8_t*)w.kv + hcd * esize(cfg);
  gg.v_ld = O;
  gg.k_out = w.kv;
  gg.k_ld = O;
  gg.partials = w.part;
  gg.hc = cfg->hc_mult;
  gg.d = cfg->hidden;
  gg.tile_n = plan.tile;
  if (plan.split) gg.g.N = (int32_t)hcd;
  if ((e = launch_gemm_gate_bf16(gg, stream))) return e;
  GateFinalizeArgs gf;
  gf.partials = w.part;
  gf.g_out = w.g;
  gf.stats = w.stats;
  gf.n_tok = (int32_t)((int64_t)cfg->batch * cfg->seqlen);
  gf.hc = cfg->hc_mult;
  gf.d = cfg->hidden;
  gf.n_part = cfg->hidden / 128;
  gf.eps = cfg->norm_eps;
  gf.clamp = cfg->gate_clamp;
  gf.inv_sqrt_d = (float)(1.0 / sqrt((double)cfg->hidden));
  if (!plan.split) return launch_gate_finalize(gf, stream);
  GemmArgs gv = gemm_args(cfg, prm, w.e, (uint8_t*)w.kv + hcd * esize(cfg));
  gv.B = (const uint8_t*)prm->w_kv + hcd * emb_dim(cfg) * esize(cfg);
  gv.N = cfg->hidden;
  gv.ldc = O;
  return launch_gemm_bf16(gv, stream, &gf);
}

// Gradients from the forward quantities in the workspace.
engram_status gradients(const engram_config* cfg, const engram_params* prm, const void* hidden, const void* dy,
                        void* d_hidden, float* d_tables, float* d_w_kv, float* d_gamma_k, float* d_gamma_q,
                        float* d_conv_w, const BwdWorkspace& w, hipStream_t stream, const SparseOut* sp = nullptr) {
  const int64_t N = (int64_t)cfg->batch * cfg->seqlen;
  const bool bf16 = cfg->dtype == ENGRAM_BF16;
  const int64_t E = emb_dim(cfg), O = (int64_t)(cfg->hc_mult + 1) * cfg->hidden;
  const int es = (int)esize(cfg);
  HashConsts hc;
  make_hash_consts(cfg, &hc);
  hipError_t e;
  // conv, gate, value fusion
  ConvBwdArgs cb;
  cb.dy = dy;
  cb.kv = w.kv;
  cb.stats = w.stats;
  cb.conv_w = prm->conv_w;
  cb.dvg = w.dvg;
  cb.part = w.cpart;
  cb.span = conv_bwd_span(N);
  if (w.dgp) {
    cb.dkv = w.dkv;
    cb.dgp = w.dgp;
    cb.n_dgp = conv_bwd_dg_parts(cfg->hc_mult, cfg->hidden);
  }
  cb.batch = cfg->batch;
  cb.seqlen = cfg->seqlen;
  cb.hc = cfg->hc_mult;
  cb.d = cfg->hidden;
  cb.ksize = cfg->conv_kernel;
  cb.dil = cfg->conv_dilation;
  cb.bf16 = bf16;
  if ((e = launch_conv_bwd(cb, stream))) return hip_status(e);
  GateBwdArgs gb;
  gb.dvg = w.dvg;
  gb.dgp = w.dgp;
  gb.n_dgp = cb.n_dgp;
  gb.kv = w.kv;
  gb.hidden = hidden;
  gb.gamma_k = prm->gamma_k;
  gb.gamma_q = prm->gamma_q;
  gb.stats = w.stats;
  gb.dkv = w.dkv;
  gb.d_hidden = d_hidden;
  gb.part = w.gpart;
  gb.n_tok = (int32_t)N;
  gb.tpb = gate_bwd_tpb(N);
  gb.hc = cfg->hc_mult;
  gb.d = cfg->hidden;
  gb.clamp = cfg->gate_clamp;
  gb.inv_sqrt_d = (float)(1.0 / sqrt((double)cfg->hidden));
  gb.bf16 = bf16;
  if ((e = launch_gate_bwd(gb, stream))) return hip_status(e);
  // sums over tokens: d gamma_k = gamma_q S, d gamma_q = gamma_k S; the taps
  if ((e = launch_colsum(w.gpart, gate_bwd_rows(N), (int64_t)cfg->hc_mult * cfg->hidden, d_gamma_k, prm->gamma_q,
                         d_gamma_q, prm->gamma_k, bf16, stream)))
    return hip_status(e);
  if ((e = launch_colsum(w.cpart, conv_bwd_rows(cfg->batch, cfg->seqlen),
                         (int64_t)cfg->hc_mult * cfg->hidden * cfg->conv_kernel, d_conv_w, nullptr, nullptr, nullptr,
                         bf16, stream)))
    return hip_status(e);
  // de = dKV W (into float32), then the rows' gradients
  if ((e = launch_transpose(prm->w_kv, w.wT, O, E, O, es, stream))) return hip_status(e);
  GemmArgs g1;
  g1.A = w.dkv;
  g1.B = w.wT;
  g1.C = w.de;
  g1.M = (int32_t)N;
  g1.N = (int32_t)E;
  g1.K = (int32_t)O;
  g1.accumulate = 0;
  if ((e = bf16 ? launch_gemm_bf16_f32out(g1, stream) : launch_gemm_f32(g1, stream))) return hip_status(e);
  if (sp) {
    SparseRowsArgs sa;
    sa.hc = hc;
    sa.idx = w.idx;
    sa.de = w.de;
    sa.n_tok = N;
    sa.head_dim = cfg->head_dim;
    sa.table_rows = 0;
    for (int h = 0; h < hc.n_heads; h++) sa.table_rows += cfg->primes[h];
    sa.bits = w.bits;
    sa.count = w.count;
    sa.first = w.first;
    sa.bsum = w.bsum;
    sa.wrank = w.wrank;
    sa.pair_rank = w.rank;
    sa.row_index = sp->row_index;
    sa.d_rows = sp->d_rows;
    sa.n_rows = sp->n_rows;
    if ((e = launch_sparse_rows(sa, stream))) return hip_status(e);
  } else if ((e = launch_scatter_add(hc, w.idx, w.de, d_tables, N, cfg->head_dim, stream))) {
    return hip_status(e);
  }
  // dW += dKV^T e
  // (in S split-K chunks of the token axis when the output has too few tiles
  // to fill the chip; the chunks' products are then added in chunk order)
  if (w.dkvT == nullptr) {   // bf16: the operands as stored, through transposing LDS reads
    const GemmTnArgs g2 = dw_args(cfg, w.dkv, w.e, w.S > 1 ? w.wpart : d_w_kv, w.S, w.Ks);
    if ((e = launch_gemm_tn_bf16_f32out(g2, stream))) return hip_status(e);
    if (w.S > 1 && (e = launch_colsum(w.wpart, w.S, O * E, d_w_kv, nullptr, nullptr, nullptr, bf16, stream)))
      return hip_status(e);
    return ENGRAM_OK;
  }
  const int64_t chunk = w.S > 1 ? w.Ks : 0;
  if ((e = launch_transpose(w.dkv, w.dkvT, N, O, w.Np, es, stream, chunk))) return hip_status(e);
  if ((e = launch_transpose(w.e, w.eT, N, E, w.Np, es, stream, chunk))) return hip_status(e);
  GemmArgs g2;
  g2.A = w.dkvT;
  g2.B = w.eT;
  g2.C = w.S > 1 ? (void*)w.wpart : (void*)d_w_kv;
  g2.M = (int32_t)O;
  g2.N = (int32_t)E;
  g2.K = (int32_t)w.Ks;
  g2.accumulate = w.S > 1 ? 0 : 1;
  g2.splits = w.S;
  g2.split_a = O * w.Ks;
  g2.split_b = E * w.Ks;
  g2.split_c = O * E;
  if ((e = bf16 ? launch_gemm_bf16_f32out(g2, stream) : launch_gemm_f32(g2, stream))) return hip_status(e);
  if (w.S > 1 &&
      (e = launch_colsum(w.wpart, w.S, O * E, d_w_kv, nullptr, nullptr, nullptr, bf16, stream)))
    return hip_status(e);
  return ENGRAM_OK;
}


}  // namespace

extern "C" {

size_t engram_workspace_size(const engram_config* cfg) {
  if (validate(cfg)) return 0;
  return carve(cfg, nullptr).bytes;
}

size_t engram_state_bytes_per_sequence(const engram_config* cfg) {
  if (validate(cfg)) return 0;
  const size_t R = (size_t)ring_len(cfg);
  return (size_t)(max_order(cfg) - 1) * sizeof(int32_t) + R * cfg->hidden * esize(cfg) +
         R * cfg->hc_mult * sizeof(float) + sizeof(int64_t);
}

engram_status engram_hash(const engram_config* cfg, const engram_params* prm, const int32_t* ids,
                          const engram_state* st, int32_t* idx_out, hipStream_t stream) {
  engram_status rc = validate(cfg);
  if (rc) return rc;
  if (prm == nullptr) return ENGRAM_EINVAL;
  if ((rc = check_state(cfg, st))) return rc;
  if ((int64_t)cfg->batch * cfg->seqlen == 0) return ENGRAM_OK;
  if (ids == nullptr || idx_out == nullptr) return ENGRAM_EINVAL;
  if ((rc = check_ids(cfg, ids, stream))) return rc;
  HashConsts hc;
  make_hash_consts(cfg, &hc);
  GatherArgs a;
  memset(&a, 0, sizeof a);
  a.ids = ids;
  a.remap = prm->remap;
  a.idx_out = idx_out;
  a.tok_ring = st ? st->tok_ring : nullptr;
  a.n_past = st ? st->n_past : nullptr;
  a.batch = cfg->batch;
  a.seqlen = cfg->seqlen;
  a.row_bytes = (int32_t)(cfg->head_dim * esize(cfg));
  return hip_status(launch_hash_gather(hc, a, true, stream));
}

engram_status engram_hash_layers(const engram_config* cfg, const engram_params* prm, const int32_t* ids,
                                 const engram_state* st, const int64_t* multipliers, int32_t n_layers,
                                 int32_t* idx_out, hipStream_t stream) {
  engram_status rc = validate(cfg);
  if (rc) return rc;
  if (prm == nullptr || multipliers == nullptr || n_layers < 1 || n_layers > ENGRAM_MAX_LAYERS) return ENGRAM_EINVAL;
  if ((rc = check_state(cfg, st))) return rc;
  if ((int64_t)cfg->batch * cfg->seqlen == 0) return ENGRAM_OK;
  if (ids == nullptr || idx_out == nullptr) return ENGRAM_EINVAL;
  if ((rc = check_ids(cfg, ids, stream))) return rc;
  HashConsts hc;
  make_hash_consts(cfg, &hc);
  LayerMults lm;
  memset(&lm, 0, sizeof lm);
  lm.n_layers = n_layers;
  for (int l = 0; l < n_layers; l++)
    for (int k = 0; k < ENGRAM_MAX_ORDERS; k++) lm.mult[l][k] = (uint64_t)multipliers[l * ENGRAM_MAX_ORDERS + k];
  GatherArgs a;
  memset(&a, 0, sizeof a);
  a.ids = ids;
  a.remap = prm->remap;
  a.idx_out = idx_out;
  a.tok_ring = st ? st->tok_ring : nullptr;
  a.n_past = st ? st->n_past : nullptr;
  a.batch = cfg->batch;
  a.seqlen = cfg->seqlen;
  return hip_status(launch_hash_layers(hc, lm, a, stream));
}

engram_status engram_gather(const engram_config* cfg, const engram_params* prm, const int32_t* idx, void* e_out,
                            hipStream_t stream) {
  engram_status rc = validate(cfg);
  if (rc) return rc;
  if (prm == nullptr || prm->tables == nullptr || !aligned(prm->tables, 16)) return ENGRAM_EINVAL;
  if ((int64_t)cfg->batch * cfg->seqlen == 0) return ENGRAM_OK;
  if (idx == nullptr || e_out == nullptr || !aligned(e_out, 16)) return ENGRAM_EINVAL;
  HashConsts hc;
  make_hash_consts(cfg, &hc);
  GatherArgs a = gather_args(cfg, prm, nullptr, nullptr);
  a.idx_in = idx;
  a.e_out = (uint8_t*)e_out;
  return hip_status(launch_hash_gather(hc, a, false, stream, gather_grid_cap(prm->tables)));
}

engram_status engram_project(const engram_config* cfg, const engram_params* prm, const void* e, void* kv_out,
                             hipStream_t stream) {
  engram_status rc = validate(cfg);
  if (rc) return rc;
  if (prm == nullptr || prm->w_kv == nullptr || !aligned(prm->w_kv, 16)) return ENGRAM_EINVAL;
  if ((int64_t)cfg->batch * cfg->seqlen == 0) return ENGRAM_OK;
  if (e == nullptr || kv_out == nullptr || !aligned(e, 16) || !aligned(kv_out, 16)) return ENGRAM_EINVAL;
  const GemmArgs g = gemm_args(cfg, prm, e, kv_out);
  return hip_status(cfg->dtype == ENGRAM_BF16 ? launch_gemm_bf16(g, stream) : launch_gemm_f32(g, stream));
}

engram_status engram_gate_conv(const engram_config* cfg, const engram_params* prm, const void* kv, const void* hidden,
                               const engram_state* st, float* g_out, void* out, hipStream_t stream) {
  engram_status rc = validate(cfg);
  if (rc) return rc;
  if ((rc = check_params(cfg, prm)) || (rc = check_state(cfg, st))) return rc;
  if ((int64_t)cfg->batch * cfg->seqlen == 0) return ENGRAM_OK;
  if (kv == nullptr || hidden == nullptr || out == nullptr || g_out == nullptr) return ENGRAM_EINVAL;
  if (!aligned(kv, 16) || !aligned(hidden, 16) || !aligned(out, 16) || !aligned(g_out, 4)) return ENGRAM_EINVAL;
  hipError_t e = launch_gate(gate_args(cfg, prm, kv, hidden, g_out), stream);
  if (e) return hip_status(e);
  const void* v = (const uint8_t*)kv + (int64_t)cfg->hc_mult * cfg->hidden * esize(cfg);
  return hip_status(launch_conv(conv_args(cfg, prm, v, (int64_t)(cfg->hc_mult + 1) * cfg->hidden, g_out, out, st),
                                stream));
}

engram_status engram_forward(const engram_config* cfg, const engram_params* prm, const int32_t* ids,
                             const void* hidden, engram_state* st, void* out, void* workspace,
                             size_t workspace_bytes, hipStream_t stream) {
  return forward_impl(cfg, prm, ids, false, nullptr, hidden, st, out, workspace, workspace_bytes, stream, nullptr, 0,
                      nullptr);
}

engram_status engram_forward_noalloc(const engram_config* cfg, const engram_params* prm, const int32_t* ids,
                                     const void* hidden, engram_state* st, void* out, hipStream_t stream) {
  engram_status rc = validate(cfg);
  if (rc) return rc;
  if (carve(cfg, nullptr).bytes > kScratchBytes) return ENGRAM_ENOMEM;
  void* ws = nullptr;
  if ((rc = device_scratch(&ws))) return rc;
  return forward_impl(cfg, prm, ids, false, nullptr, hidden, st, out, ws, kScratchBytes, stream, nullptr, 0, nullptr);
}

engram_status engram_forward_gathered(const engram_config* cfg, const engram_params* prm, const int32_t* ids,
                                      const void* e, const void* hidden, engram_state* st, void* out, void* workspace,
                                      size_t workspace_bytes, hipStream_t stream) {
  return forward_impl(cfg, prm, ids, true, e, hidden, st, out, workspace, workspace_bytes, stream, nullptr, 0,
                      nullptr);
}

engram_status engram_forward_timed(const engram_config* cfg, const engram_params* prm, const int32_t* ids,
                                   const void* hidden, engram_state* st, void* out, void* workspace,
                                   size_t workspace_bytes, hipStream_t stream, hipEvent_t* events, int32_t n_events,
                                   int32_t* n_kernels) {
  if (events == nullptr && n_events != 0) return ENGRAM_EINVAL;
  return forward_impl(cfg, prm, ids, false, nullptr, hidden, st, out, workspace, workspace_bytes, stream, events,
                      n_events, n_kernels);
}

size_t engram_backward_workspace_size(const engram_config* cfg) {
  if (validate(cfg)) return 0;
  return carve_bwd(cfg, nullptr).bytes;
}

engram_status engram_backward(const engram_config* cfg, const engram_params* prm, const int32_t* ids,
                              const void* hidden, const void* dy, void* d_hidden, float* d_tables, float* d_w_kv,
                              float* d_gamma_k, float* d_gamma_q, float* d_conv_w, void* workspace,
                              size_t workspace_bytes, hipStream_t stream) {
  engram_status rc = check_backward(cfg, prm, true, ids, hidden, dy, d_hidden, d_tables, d_w_kv, d_gamma_k,
                                    d_gamma_q, d_conv_w, workspace, workspace_bytes);
  if (rc || (int64_t)cfg->batch * cfg->seqlen == 0) return rc;
  if ((rc = check_ids(cfg, ids, stream))) return rc;
  const BwdWorkspace w = carve_bwd(cfg, workspace);
  hipError_t e;
  if ((e = forward_quantities(cfg, prm, ids, hidden, w, stream))) return hip_status(e);
  return gradients(cfg, prm, hidden, dy, d_hidden, d_tables, d_w_kv, d_gamma_k, d_gamma_q, d_conv_w, w, stream);
}

engram_status engram_forward_train(const engram_config* cfg, const engram_params* prm, const int32_t* ids,
                                   const void* hidden, void* out, void* workspace, size_t workspace_bytes,
                                   hipStream_t stream) {
  engram_status rc = validate(cfg);
  if (rc) return rc;
  if ((rc = check_params(cfg, prm))) return rc;
  if ((int64_t)cfg->batch * cfg->seqlen == 0) return ENGRAM_OK;
  if (ids == nullptr || hidden == nullptr || out == nullptr || workspace == nullptr) return ENGRAM_EINVAL;
  if (!aligned(hidden, 16) || !aligned(out, 16) || !aligned(workspace, 256)) return ENGRAM_EINVAL;
  const BwdWorkspace w = carve_bwd(cfg, workspace);
  if (workspace_bytes < w.bytes) return ENGRAM_ENOMEM;
  if ((rc = check_ids(cfg, ids, stream))) return rc;
  hipError_t e;
  if ((e = forward_quantities(cfg, prm, ids, hidden, w, stream))) return hip_status(e);
  const void* v = (const uint8_t*)w.kv + (int64_t)cfg->hc_mult * cfg->hidden * esize(cfg);
  const ConvArgs cv = conv_args(cfg, prm, v, (int64_t)(cfg->hc_mult + 1) * cfg->hidden, w.g, out, nullptr);
  if ((e = launch_conv(cv, stream))) return hip_status(e);
  return ENGRAM_OK;
}

engram_status engram_backward_saved(const engram_config* cfg, const engram_params* prm, const void* hidden,
                                    const void* dy, void* d_hidden, float* d_tables, float* d_w_kv,
                                    float* d_gamma_k, float* d_gamma_q, float* d_conv_w, void* workspace,
                                    size_t workspace_bytes, hipStream_t stream) {
  engram_status rc = check_backward(cfg, prm, false, nullptr, hidden, dy, d_hidden, d_tables, d_w_kv, d_gamma_k,
                                    d_gamma_q, d_conv_w, workspace, workspace_bytes);
  if (rc || (int64_t)cfg->batch * cfg->seqlen == 0) return rc;
  return gradients(cfg, prm, hidden, dy, d_hidden, d_tables, d_w_kv, d_gamma_k, d_gamma_q, d_conv_w,
                   carve_bwd(cfg, workspace), stream);
}

engram_status engram_backward_sparse(const engram_config* cfg, const engram_params* prm, const int32_t* ids,
                                     const void* hidden, const void* dy, void* d_hidden, int64_t* row_index,
                                     float* d_rows, int64_t* n_rows, float* d_w_kv, float* d_gamma_k, float* d_gamma_q,
                                     float* d_conv_w, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  const SparseOut sp{row_index, d_rows, n_rows};
  engram_status rc = check_backward(cfg, prm, true, ids, hidden, dy, d_hidden, nullptr, d_w_kv, d_gamma_k,
                                    d_gamma_q, d_conv_w, workspace, workspace_bytes, &sp);
  if (rc || (int64_t)cfg->batch * cfg->seqlen == 0) return rc;
  if ((rc = check_ids(cfg, ids, stream))) return rc;
  const BwdWorkspace w = carve_bwd(cfg, workspace);
  hipError_t e;
  if ((e = forward_quantities(cfg, prm, ids, hidden, w, stream))) return hip_status(e);
  return gradients(cfg, prm, hidden, dy, d_hidden, nullptr, d_w_kv, d_gamma_k, d_gamma_q, d_conv_w, w, stream, &sp);
}

engram_status engram_backward_saved_sparse(const engram_config* cfg, const engram_params* prm, const void* hidden,
                                           const void* dy, void* d_hidden, int64_t* row_index, float* d_rows,
                                           int64_t* n_rows, float* d_w_kv, float* d_gamma_k, float* d_gamma_q,
                                           float* d_conv_w, void* workspace, size_t workspace_bytes,
                                           hipStream_t stream) {
  const SparseOut sp{row_index, d_rows, n_rows};
  engram_status rc = check_backward(cfg, prm, false, nullptr, hidden, dy, d_hidden, nullptr, d_w_kv, d_gamma_k,
                                    d_gamma_q, d_conv_w, workspace, workspace_bytes, &sp);
  if (rc || (int64_t)cfg->batch * cfg->seqlen == 0) return rc;
  return gradients(cfg, prm, hidden, dy, d_hidden, nullptr, d_w_kv, d_gamma_k, d_gamma_q, d_conv_w,
                   carve_bwd(cfg, workspace), stream, &sp);
}

engram_status engram_gather_host(const engram_config* cfg, const void* tables, const int32_t* idx, void* e_out,
                                 int32_t n_threads) {
  engram_status rc = validate(cfg);
  if (rc) return rc;
  const int64_t N = (int64_t)cfg->batch * cfg->seqlen;
  if (N == 0) return ENGRAM_OK;
  if (tables == nullptr || idx == nullptr || e_out == nullptr) return ENGRAM_EINVAL;
  const int H = n_heads(cfg);
  const size_t row = (size_t)cfg->head_dim * esize(cfg);
  int64_t off[ENGRAM_MAX_HEADS];
  int64_t acc = 0;
  for (int h = 0; h < H; h++) {
    off[h] = acc;
    acc += cfg->primes[h];
  }
  // row i = n*H + h of e_out is table row off[h] + idx[i] (clamped into [0, p_h) like engram_gather).
  // The rows are scattered over the table, so each thread asks for the cache
  // lines of the row kAhead places ahead before it copies the current one.
  const uint8_t* t = (const uint8_t*)tables;
  auto src = [&](int64_t i) {
    const int h = (int)(i % H);
    const int64_t r = std::min<int64_t>(std::max<int64_t>(idx[i], 0), (int64_t)cfg->primes[h] - 1);
    return t + (off[h] + r) * (int64_t)row;
  };
  auto copy = [&](int64_t lo, int64_t hi) {
    constexpr int kAhead = 16;
    uint8_t* e = (uint8_t*)e_out;
    auto prefetch = [&](int64_t i) {
      const uint8_t* p = src(i);
      for (size_t b = 0; b < row; b += 64) __builtin_prefetch(p + b, 0, 0);
      __builtin_prefetch(p + row - 1, 0, 0);
    };
    for (int64_t i = lo; i < std::min(hi, lo + kAhead); i++) prefetch(i);
    for (int64_t i = lo; i < hi; i++) {
      if (i + kAhead < hi) prefetch(i + kAhead);
      memcpy(e + i * row, src(i), row);
    }
  };
  const int64_t rows = N * H;
  int nt = n_threads > 0 ? n_threads : (int)std::thread::hardware_concurrency();
  // at least 8192 rows per thread: starting a thread costs about as much as copying that many
  nt = (int)std::max<int64_t>(1, std::min<int64_t>({(int64_t)nt, 16, rows / 8192 + 1}));
  if (nt == 1) {
    copy(0, rows);
    return ENGRAM_OK;
  }
  // Threads that cannot be started leave their share to this one; nothing
  // thrown crosses the C interface.
  std::vector<std::thread> pool;
  int started = 0;
  try {
    pool.reserve(nt);
    for (int k = 1; k < nt; k++) {
      pool.emplace_back(copy, rows * k / nt, rows * (k + 1) / nt);
      started = k;
    }
  } catch (...) {
  }
  copy(0, rows * 1 / nt);
  if (started + 1 < nt) copy(rows * (started + 1) / nt, rows);
  for (auto& th : pool) th.join();
  return ENGRAM_OK;
}

const char* engram_forward_kernel_name(const engram_config* cfg, int32_t with_state, int32_t i) {
  if (validate(cfg) || i < 0) return nullptr;
  int n = 0;
  const char* const* names = forward_kernels(cfg, with_state != 0, false, &n);
  return i < n ? names[i] : nullptr;
}

const char* engram_status_string(engram_status s) {
  switch (s) {
    case ENGRAM_OK: return "ok";
    case ENGRAM_EINVAL: return "invalid configuration or argument";
    case ENGRAM_ENOMEM: return "workspace too small";
    case ENGRAM_EHIP: return "HIP launch or API call failed";
    case ENGRAM_EUNSUPPORTED: return "configuration not supported by the kernels";
  }
  return "unknown status";
}

}  // extern "C"
