// C ABI of libsa: host-side validation, workspace carve-out and kernel launches.
// Every check runs before the first launch; on error nothing is launched.
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <atomic>
#include <mutex>

#include "sa_internal.h"

// Scratch of sa_sparse_decode_noalloc: one array per GPU (each device holds its own copy of
// the code object's data), held until the process ends.  Host code never uses the name of the
// array as an address: it looks up each device's address once (hipGetSymbolAddress, with the
// device current) and passes that pointer to the kernels.
static __device__ __align__(256) unsigned char scratch[SA_NOALLOC_SCRATCH_BYTES];

namespace {

// Debug builds: one check word per device (SA_DBG_* bits set by the kernels' checks),
// allocated and cleared on the first checked call with that device.  A checked entry point
// waits for its stream, reads the word and clears it; the bits of the last failing call stay
// readable through sa_debug_flags().  Release builds pass no word and never synchronise.
std::atomic<unsigned int> g_dbg_last{0};

// SA_LOG set (and not "0") in the environment: every launching entry point prints one line to
// stderr, after its checks and before its launches, with the configuration it launches for.
bool log_on() {
  const char* e = getenv("SA_LOG");
  return e && e[0] && !(e[0] == '0' && e[1] == 0);
}

void log_prefill(const char* name, const sa_shape* s, const sa_sparse_params* p, int tpb,
                 const void* stream) {
  if (!log_on()) return;
  static const char* const est[] = {"pooled", "relative", "relative_mxfp4"};
  const int e = p->estimator >= 0 && p->estimator <= 2 ? p->estimator : 0;
  fprintf(stderr,
          "[sa] %s: B=%d Hq=%d Hkv=%d d=%d N=%d head_map=%s block_q=%d block_k=%d sink=%d "
          "local=%d granularity=%s estimator=%s step=%d row_tiles_per_block=%d stream=%p\n",
          name, s->batch, s->n_q_heads, s->n_kv_heads, s->head_dim, s->seq_q,
          s->kv_head_of_q ? "given" : "h/G", p->block_q, p->block_k, p->sink_tokens,
          p->local_tokens, p->granularity == SA_STRIPE ? "stripe" : "block", est[e], p->step, tpb,
          stream);
}

void log_decode(const char* name, const sa_shape* s, int block_k, const sa_decode_params* p,
                int n_splits, const char* summary, const void* stream) {
  if (!log_on()) return;
  fprintf(stderr,
          "[sa] %s: B=%d Hq=%d Hkv=%d d=%d L=%d block_k=%d top_k=%d top_p=%g sink=%d local=%d "
          "splits=%d summary=%s stream=%p\n",
          name, s->batch, s->n_q_heads, s->n_kv_heads, s->head_dim, s->seq_k,
          block_k, p ? p->top_k_blocks : 0, p ? (double)p->top_p : 0.0,
          p ? p->sink_tokens : 0, p ? p->local_tokens : 0, n_splits, summary, stream);
}
#ifdef SA_DEBUG
constexpr int kMaxDbgDevices = 64;
std::mutex g_dbg_mutex;
unsigned int* g_dbg_word[kMaxDbgDevices] = {};
#endif

unsigned int* debug_word() {
#ifdef SA_DEBUG
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDbgDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_dbg_mutex);
  if (!g_dbg_word[dev]) {
    void* p = nullptr;
    if (hipMalloc(&p, sizeof(unsigned int)) != hipSuccess) return nullptr;
    if (hipMemset(p, 0, sizeof(unsigned int)) != hipSuccess) return nullptr;
    g_dbg_word[dev] = (unsigned int*)p;
  }
  return g_dbg_word[dev];
#else
  return nullptr;
#endif
}

// The status of a checked call: st itself unless this is a debug build whose kernels set a
// check bit (then SA_ERR_CHECK, the bits kept for sa_debug_flags()).
sa_status debug_finish(sa_status st, unsigned int* word, hipStream_t stream) {
#ifdef SA_DEBUG
  if (st != SA_OK) return st;
  if (!word) return SA_ERR_DEVICE;
  unsigned int bits = 0;
  if (hipStreamSynchronize(stream) != hipSuccess) return SA_ERR_DEVICE;
  if (hipMemcpy(&bits, word, sizeof(bits), hipMemcpyDeviceToHost) != hipSuccess) return SA_ERR_DEVICE;
  if (bits == 0) return SA_OK;
  if (hipMemset(word, 0, sizeof(unsigned int)) != hipSuccess) return SA_ERR_DEVICE;
  g_dbg_last.store(bits);
  return SA_ERR_CHECK;
#else
  (void)word;
  (void)stream;
  return st;
#endif
}

constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

int ceil_div(int64_t a, int64_t b) { return (int)((a + b - 1) / b); }

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

float resolve_scale(float s, int d) {
  if (s > 0.f) return s;
  return (float)(1.0 / sqrt((double)d));
}

// The packing order of the query heads: qh[g * G + j] = the j-th query head (ascending) whose
// KV head is g.  Without a map, query head h uses KV head h / G, so qh is the identity.
sa_status make_head_map(const sa_shape* s, uint8_t* qh) {
  const int Hq = s->n_q_heads, Hkv = s->n_kv_heads, G = Hq / Hkv;
  if (!s->kv_head_of_q) {
    for (int h = 0; h < Hq; ++h) qh[h] = (uint8_t)h;
    return SA_OK;
  }
  for (int h = 0; h < Hq; ++h)
    if (s->kv_head_of_q[h] < 0 || s->kv_head_of_q[h] >= Hkv) return SA_ERR_PARAM;
  int fill[SA_MAX_Q_HEADS] = {0};
  for (int h = 0; h < Hq; ++h) {
    const int g = s->kv_head_of_q[h];
    if (fill[g] >= G) return SA_ERR_UNSUPPORTED;   // unequal group sizes cannot be packed
    qh[g * G + fill[g]++] = (uint8_t)h;
  }
  return SA_OK;
}

sa_status check_shape_common(const sa_shape* s) {
  if (!s) return SA_ERR_NULL;
  if (s->batch < 1 || s->n_q_heads < 1 || s->n_kv_heads < 1 || s->seq_q < 1 || s->seq_k < 1)
    return SA_ERR_SHAPE;
  if (s->n_q_heads % s->n_kv_heads != 0) return SA_ERR_SHAPE;
  const int G = s->n_q_heads / s->n_kv_heads;
  if (s->head_dim != 64 && s->head_dim != 128) return SA_ERR_UNSUPPORTED;
  if (s->n_q_heads > SA_MAX_Q_HEADS) return SA_ERR_UNSUPPORTED;
  if (G != 1 && G != 2 && G != 4 && G != 8) return SA_ERR_UNSUPPORTED;
  uint8_t qh[SA_MAX_Q_HEADS];
  return make_head_map(s, qh);
}

bool strides_ok(const int64_t st[3]) {
  for (int i = 0; i < 3; ++i)
    if (st[i] < 0 || (st[i] % 8) != 0) return false;
  return true;
}

sa_status check_prefill_shape(const sa_shape* s) {
  sa_status st = check_shape_common(s);
  if (st != SA_OK) return st;
  if (s->seq_q != s->seq_k) return SA_ERR_SHAPE;
  if (s->seq_q >= (1 << 30)) return SA_ERR_UNSUPPORTED;
  if (!strides_ok(s->q_stride) || !strides_ok(s->k_stride) || !strides_ok(s->v_stride) ||
      !strides_ok(s->o_stride))
    return SA_ERR_SHAPE;
  // head and token strides must at least cover one row of head_dim elements
  if (s->q_stride[2] < s->head_dim || s->k_stride[2] < s->head_dim ||
      s->v_stride[2] < s->head_dim || s->o_stride[2] < s->head_dim)
    return SA_ERR_SHAPE;
  // the attention addresses a K/V tile's rows with 32-bit byte offsets from the tile's start
  if (s->k_stride[1] >= (1 << 24) || s->v_stride[1] >= (1 << 24)) return SA_ERR_UNSUPPORTED;
  return SA_OK;
}

sa_status check_sparse_params(const sa_shape* s, const sa_sparse_params* p, bool need_theta) {
  if (!p) return SA_ERR_NULL;
  if (need_theta && !p->theta) return SA_ERR_NULL;
  if (p->granularity != SA_BLOCK && p->granularity != SA_STRIPE) return SA_ERR_PARAM;
  if (p->estimator != SA_EST_POOLED && p->estimator != SA_EST_RELATIVE &&
      p->estimator != SA_EST_RELATIVE_MXFP4)
    return SA_ERR_PARAM;
  if (p->estimator != SA_EST_POOLED && p->granularity != SA_BLOCK) return SA_ERR_UNSUPPORTED;
  if (p->step < 0) return SA_ERR_PARAM;
  if (p->sink_tokens < 0 || p->local_tokens < 1) return SA_ERR_PARAM;
  if (p->block_q != 64 && p->block_q != 128) return SA_ERR_UNSUPPORTED;
  // key blocks of 64, or of 32 (two per 64-key tile) for block lists
  if (p->block_k != 64 && !(p->block_k == 32 && p->granularity == SA_BLOCK)) return SA_ERR_UNSUPPORTED;
  if (isnan(p->softmax_scale) || isinf(p->softmax_scale)) return SA_ERR_PARAM;
  if (need_theta)
    for (int h = 0; h < s->n_q_heads; ++h)
      if (isnan(p->theta[h])) return SA_ERR_PARAM;
  return SA_OK;
}

struct EstLayout {
  size_t kq, sk, qq, sq, abar, bits, qr, sr, k4, k4s, xa, total;
  int W;
};

// with_state: room for the per-row anchors the anchor-state pass hands to the estimate
EstLayout est_layout(const sa_shape* s, const sa_sparse_params* p, bool with_state = false) {
  EstLayout L{};
  const int N = s->seq_q, D = s->head_dim, B = s->batch, Hkv = s->n_kv_heads, Hq = s->n_q_heads;
  const int nQB = ceil_div(N, p->block_q), nKB = ceil_div(N, p->block_k);
  const int nKT = ceil_div(N, 64);             // 64-key tiles (the unit keys are staged in)
  // stripe bit rows cover the padded key range (whole 64-key tiles)
  const int ncand = p->granularity == SA_STRIPE ? nKT * 64 : nKB;
  L.W = ceil_div(ncand, 32);
  size_t off = 0;
  L.kq = off;   off = align_up(off + (size_t)B * Hkv * nKT * 64 * D);
  L.sk = off;   off = align_up(off + (size_t)B * Hkv * nKB * sizeof(float));
  L.qq = off;   off = align_up(off + (size_t)B * Hq * nQB * D);
  L.sq = off;   off = align_up(off + (size_t)B * Hq * nQB * sizeof(float));
  L.abar = off; off = align_up(off + (size_t)B * Hq * nQB * sizeof(float));
  L.bits = off; off = align_up(off + (size_t)B * Hkv * nQB * L.W * sizeof(uint32_t));
  // relative estimators: int8 query rows + fp32 scales, or MXFP4 query rows (D/2 code bytes
  // and D/32 scale bytes per row, in the same regions) and MXFP4 key rows
  const size_t rows = p->estimator != SA_EST_POOLED ? (size_t)B * Hq * N : 0;
  const bool fp4 = p->estimator == SA_EST_RELATIVE_MXFP4;
  L.qr = off;   off = align_up(off + rows * (fp4 ? D / 2 : D));
  L.sr = off;   off = align_up(off + rows * (fp4 ? D / 32 : sizeof(float)));
  const size_t krows = fp4 ? (size_t)B * Hkv * nKT * 64 : 0;
  L.k4 = off;   off = align_up(off + krows * D / 2);
  L.k4s = off;  off = align_up(off + krows * D / 32);
  L.xa = off;   off = align_up(off + (with_state ? (size_t)B * Hq * N * sizeof(float) : 0));
  L.total = off;
  return L;
}

// calibration workspace: the estimate's scratch, one block list, both outputs, the errors
struct CalLayout {
  size_t est, counts, idx, o_ref, o_sp, err, total;
};

CalLayout cal_layout(const sa_shape* s, const sa_sparse_params* p) {
  CalLayout L{};
  const int N = s->seq_q;
  const int nQB = ceil_div(N, p->block_q), nKB = ceil_div(N, p->block_k);
  const size_t rows = (size_t)s->batch * s->n_kv_heads * nQB;
  const size_t oel = (size_t)s->batch * N * s->n_q_heads * s->head_dim;
  size_t off = 0;
  L.est = off;    off = align_up(off + est_layout(s, p).total);
  L.counts = off; off = align_up(off + rows * sizeof(int32_t));
  L.idx = off;    off = align_up(off + rows * nKB * sizeof(int32_t));
  L.o_ref = off;  off = align_up(off + oel * 2);
  L.o_sp = off;   off = align_up(off + oel * 2);
  L.err = off;    off = align_up(off + (size_t)s->n_q_heads * sizeof(double));
  L.total = off;
  return L;
}

struct DecLayout {
  size_t scores, selected, counts, partial, total;
};

int decode_splits(const sa_shape* s, const sa_decode_params* p) {
  if (p->n_splits > 0) return p->n_splits;
  // 64-key blocks (MFMA kernel, each workgroup streams its blocks): about one workgroup per
  // CU; other block sizes: enough workgroups to cover the chip several times over
  const int64_t target = p->block_k == 64 ? 256 : 2048;
  int n = 1;
  while ((int64_t)s->batch * s->n_kv_heads * n < target && n < 64) n <<= 1;
  return n;
}

DecLayout dec_layout(const sa_shape* s, const sa_decode_params* p) {
  DecLayout L{};
  const int nKB = ceil_div(s->seq_k, p->block_k);
  const int ns = decode_splits(s, p);
  size_t off = 0;
  L.scores = off;   off = align_up(off + (size_t)s->batch * s->n_kv_heads * nKB * sizeof(float));
  L.selected = off; off = align_up(off + (size_t)s->batch * s->n_kv_heads * p->top_k_blocks * sizeof(int32_t));
  L.counts = off;   off = align_up(off + (size_t)s->batch * s->n_kv_heads * sizeof(int32_t));
  L.partial = off;  off = align_up(off + (size_t)s->batch * s->n_q_heads * ns * (s->head_dim + 2) * sizeof(float));
  L.total = off;
  return L;
}

sa_status check_decode(const sa_shape* s, const sa_decode_params* p) {
  sa_status st = check_shape_common(s);
  if (st != SA_OK) return st;
  if (!p) return SA_ERR_NULL;
  if (s->seq_q != 1) return SA_ERR_SHAPE;
  if (p->block_k < 1 || p->top_k_blocks < 1 || p->sink_tokens < 0 || p->local_tokens < 1 ||
      p->n_splits < 0)
    return SA_ERR_PARAM;
  if (isnan(p->softmax_scale) || isinf(p->softmax_scale)) return SA_ERR_PARAM;
  if (!(p->top_p >= 0.f && p->top_p <= 1.f)) return SA_ERR_PARAM;
  if (ceil_div(s->seq_k, p->block_k) > 8192) return SA_ERR_UNSUPPORTED;
  // K must hold the whole forced set at every cache length: the blocks the sink tokens
  // overlap plus the most blocks a window of `local` tokens can overlap (unless K covers
  // every block of the cache, when everything is selected anyway)
  const int64_t f_max = ((int64_t)p->sink_tokens + p->block_k - 1) / p->block_k +
                        ((int64_t)p->local_tokens - 1) / p->block_k + 2;
  if (p->top_k_blocks < f_max && p->top_k_blocks < ceil_div(s->seq_k, p->block_k))
    return SA_ERR_PARAM;
  if (!strides_ok(s->q_stride) || !strides_ok(s->k_stride) || !strides_ok(s->v_stride) ||
      !strides_ok(s->o_stride))
    return SA_ERR_SHAPE;
  return SA_OK;
}

}  // namespace

extern "C" {

uint32_t sa_debug_flags(void) { return g_dbg_last.load(); }

const char* sa_status_string(sa_status st) {
  switch (st) {
    case SA_OK: return "ok";
    case SA_ERR_NULL: return "null pointer";
    case SA_ERR_SHAPE: return "invalid shape, stride or alignment";
    case SA_ERR_PARAM: return "invalid parameter";
    case SA_ERR_UNSUPPORTED: return "unsupported configuration";
    case SA_ERR_CAPACITY: return "list capacity too small";
    case SA_ERR_WORKSPACE: return "workspace missing or too small";
    case SA_ERR_DEVICE: return "device error";
    case SA_ERR_CHECK: return "invalid caller data found by a debug-build kernel check";
  }
  return "unknown status";
}

size_t sa_workspace_size(int op, const sa_shape* shape, const void* params) {
  if (!shape || !params) return 0;
  if (op == SA_OP_ESTIMATE || op == SA_OP_ESTIMATE_STATE) {
    const sa_sparse_params* p = (const sa_sparse_params*)params;
    if (check_prefill_shape(shape) != SA_OK || check_sparse_params(shape, p, true) != SA_OK) return 0;
    if (op == SA_OP_ESTIMATE_STATE && (p->estimator != SA_EST_POOLED || p->block_k != 64))
      return 0;
    return est_layout(shape, p, op == SA_OP_ESTIMATE_STATE).total;
  }
  if (op == SA_OP_CALIBRATE) {
    const sa_sparse_params* p = (const sa_sparse_params*)params;
    if (check_prefill_shape(shape) != SA_OK || check_sparse_params(shape, p, false) != SA_OK ||
        p->granularity != SA_BLOCK)
      return 0;
    return cal_layout(shape, p).total;
  }
  if (op == SA_OP_DECODE) {
    const sa_decode_params* p = (const sa_decode_params*)params;
    if (check_decode(shape, p) != SA_OK) return 0;
    return dec_layout(shape, p).total;
  }
  return 0;
}

}  // extern "C"

// The estimate, optionally preceded by the anchor-state pass (v and state non-null).
static sa_status estimate_impl(const sa_shape* shape, const sa_sparse_params* params, const void* q,
                               const void* k, const void* v, const sa_lists* out,
                               const sa_anchor_state* state, void* ws, size_t ws_bytes,
                               hipStream_t stream) {
  sa_status st = check_prefill_shape(shape);
  if (st != SA_OK) return st;
  st = check_sparse_params(shape, params, true);
  if (st != SA_OK) return st;
  if (!q || !k || !out || !out->counts || !out->idx) return SA_ERR_NULL;
  if (!aligned16(q) || !aligned16(k)) return SA_ERR_SHAPE;
  const bool with_state = state != nullptr;
  if (with_state) {
    if (params->estimator != SA_EST_POOLED || params->block_k != 64) return SA_ERR_UNSUPPORTED;
    if (!v || !state->o || !state->lse) return SA_ERR_NULL;
    if (!aligned16(v) || !aligned16(state->o) || ((uintptr_t)state->lse & 3u) != 0) return SA_ERR_SHAPE;
  }
  const int N = shape->seq_q;
  const int nKB = ceil_div(N, params->block_k), nQB = ceil_div(N, params->block_q);
  if (out->stride < 1) return SA_ERR_CAPACITY;
  if (params->granularity == SA_BLOCK && out->stride < nKB) return SA_ERR_CAPACITY;
  const EstLayout L = est_layout(shape, params, with_state);
  if (!ws) return SA_ERR_WORKSPACE;
  if (ws_bytes < L.total || ((uintptr_t)ws % kAlign) != 0) return SA_ERR_WORKSPACE;

  EstArgs a;
  memset(&a, 0, sizeof(a));
  a.q = (const uint16_t*)q;
  a.k = (const uint16_t*)k;
  a.qs0 = shape->q_stride[0]; a.qs1 = shape->q_stride[1]; a.qs2 = shape->q_stride[2];
  a.ks0 = shape->k_stride[0]; a.ks1 = shape->k_stride[1]; a.ks2 = shape->k_stride[2];
  a.B = shape->batch; a.Hq = shape->n_q_heads; a.Hkv = shape->n_kv_heads;
  a.G = a.Hq / a.Hkv; a.D = shape->head_dim; a.N = N;
  a.bq = params->block_q; a.bk = params->block_k;
  a.sink = params->sink_tokens; a.local = params->local_tokens;
  a.nQB = nQB; a.nKB = nKB; a.nKT = ceil_div(N, 64);
  a.c = resolve_scale(params->softmax_scale, a.D);
  char* base = (char*)ws;
  a.kq = (int8_t*)(base + L.kq);
  a.sk = (float*)(base + L.sk);
  a.qq = (int8_t*)(base + L.qq);
  a.sq = (float*)(base + L.sq);
  a.abar = (float*)(base + L.abar);
  a.bits = (uint32_t*)(base + L.bits);
  a.qr = (int8_t*)(base + L.qr);
  a.sr = (float*)(base + L.sr);
  a.k4 = (uint8_t*)(base + L.k4);
  a.k4s = (uint8_t*)(base + L.k4s);
  a.estimator = params->estimator;
  a.step = params->step;
  a.W = L.W;
  a.counts = out->counts;
  a.idx = out->idx;
  a.stride = out->stride;
  a.margins = out->margins;
  make_head_map(shape, a.qh);
  for (int j = 0; j < a.Hq; ++j) a.theta[j] = params->theta[a.qh[j]];
  if (with_state) {
    a.v = (const uint16_t*)v;
    a.vs0 = shape->v_stride[0]; a.vs1 = shape->v_stride[1]; a.vs2 = shape->v_stride[2];
    a.st_o = (uint16_t*)state->o;
    a.st_lse = state->lse;
    a.xa = (float*)(base + L.xa);
    a.xa_ready = 1;
    log_prefill("sa_estimate_mask_anchor_state", shape, params, params->block_q / 64, stream);
    if (launch_anchor_state(a, stream) != hipSuccess) return SA_ERR_DEVICE;
  } else {
    log_prefill("sa_estimate_mask", shape, params, params->block_q / 64, stream);
  }
  if (launch_estimate(a, params->granularity, stream) != hipSuccess) return SA_ERR_DEVICE;
  return SA_OK;
}

// The computation pass, optionally resuming from an anchor state.
static sa_status prefill_impl(const sa_shape* shape, const sa_sparse_params* params, const void* q,
                              const void* k, const void* v, const sa_lists* lists,
                              const sa_anchor_state* state, void* o, float* lse, hipStream_t stream) {
  sa_status st = check_prefill_shape(shape);
  if (st != SA_OK) return st;
  st = check_sparse_params(shape, params, false);
  if (st != SA_OK) return st;
  if (!q || !k || !v || !o || !lists || !lists->counts || !lists->idx) return SA_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return SA_ERR_SHAPE;
  if (state) {
    if (params->block_k != 64) return SA_ERR_UNSUPPORTED;
    if (!state->o || !state->lse) return SA_ERR_NULL;
    if (!aligned16(state->o) || ((uintptr_t)state->lse & 3u) != 0) return SA_ERR_SHAPE;
  }
  const int N = shape->seq_q;
  const int nKB = ceil_div(N, params->block_k), nQB = ceil_div(N, params->block_q);
  if (lists->stride < 1) return SA_ERR_CAPACITY;
  if (params->granularity == SA_BLOCK && lists->stride < nKB) return SA_ERR_CAPACITY;

  AttnArgs a;
  memset(&a, 0, sizeof(a));
  a.q = (const uint16_t*)q; a.k = (const uint16_t*)k; a.v = (const uint16_t*)v;
  a.o = (uint16_t*)o; a.lse = lse;
  a.qs0 = shape->q_stride[0]; a.qs1 = shape->q_stride[1]; a.qs2 = shape->q_stride[2];
  a.ks0 = shape->k_stride[0]; a.ks1 = shape->k_stride[1]; a.ks2 = shape->k_stride[2];
  a.vs0 = shape->v_stride[0]; a.vs1 = shape->v_stride[1]; a.vs2 = shape->v_stride[2];
  a.os0 = shape->o_stride[0]; a.os1 = shape->o_stride[1]; a.os2 = shape->o_stride[2];
  a.counts = lists->counts; a.idx = lists->idx; a.stride = lists->stride;
  a.B = shape->batch; a.Hq = shape->n_q_heads; a.Hkv = shape->n_kv_heads;
  a.G = a.Hq / a.Hkv; a.N = N; a.bq = params->block_q; a.nQB = nQB;
  a.tpb = params->block_q / 64;
  a.scale_log2 = resolve_scale(params->softmax_scale, shape->head_dim) * 1.4426950408889634f;
  a.stripe = params->granularity == SA_STRIPE;
  a.bk32 = params->block_k == 32;
  make_head_map(shape, a.qh);
  if (state) {
    a.st_o = (const uint16_t*)state->o;
    a.st_lse = state->lse;
    a.sink = params->sink_tokens;
    a.local = params->local_tokens;
  }
  a.dbg = debug_word();
  log_prefill(state ? "sa_sparse_prefill_resume" : "sa_sparse_prefill", shape, params, a.tpb, stream);
  if (launch_prefill(a, shape->head_dim, params->granularity, stream) != hipSuccess)
    return SA_ERR_DEVICE;
  return debug_finish(SA_OK, a.dbg, stream);
}

extern "C" {

sa_status sa_estimate_mask(const sa_shape* shape, const sa_sparse_params* params, const void* q,
                           const void* k, const sa_lists* out, void* ws, size_t ws_bytes,
                           hipStream_t stream) {
  return estimate_impl(shape, params, q, k, nullptr, out, nullptr, ws, ws_bytes, stream);
}

sa_status sa_estimate_mask_anchor_state(const sa_shape* shape, const sa_sparse_params* params,
                                        const void* q, const void* k, const void* v,
                                        const sa_lists* out, const sa_anchor_state* state, void* ws,
                                        size_t ws_bytes, hipStream_t stream) {
  if (!state) return SA_ERR_NULL;
  return estimate_impl(shape, params, q, k, v, out, state, ws, ws_bytes, stream);
}

sa_status sa_sparse_prefill(const sa_shape* shape, const sa_sparse_params* params, const void* q,
                            const void* k, const void* v, const sa_lists* lists, void* o,
                            float* lse, hipStream_t stream) {
  return prefill_impl(shape, params, q, k, v, lists, nullptr, o, lse, stream);
}

sa_status sa_sparse_prefill_resume(const sa_shape* shape, const sa_sparse_params* params,
                                   const void* q, const void* k, const void* v,
                                   const sa_lists* lists, const sa_anchor_state* state, void* o,
                                   float* lse, hipStream_t stream) {
  if (!state) return SA_ERR_NULL;
  return prefill_impl(shape, params, q, k, v, lists, state, o, lse, stream);
}

static void fill_dec_args(DecArgs& a, const sa_shape* s, int block_k) {
  memset(&a, 0, sizeof(a));
  a.qs0 = s->q_stride[0]; a.qs2 = s->q_stride[2];
  a.ks0 = s->k_stride[0]; a.ks1 = s->k_stride[1]; a.ks2 = s->k_stride[2];
  a.vs0 = s->v_stride[0]; a.vs1 = s->v_stride[1]; a.vs2 = s->v_stride[2];
  a.os0 = s->o_stride[0]; a.os2 = s->o_stride[2];
  a.B = s->batch; a.Hq = s->n_q_heads; a.Hkv = s->n_kv_heads; a.G = a.Hq / a.Hkv;
  a.D = s->head_dim; a.L = s->seq_k; a.bk = block_k;
  a.nKB = ceil_div(s->seq_k, block_k);
  make_head_map(s, a.qh);
}

sa_status sa_build_block_summary(const sa_shape* shape, int32_t block_k, const void* k_cache,
                                 const int32_t* cache_len, void* k_summary, hipStream_t stream) {
  sa_status st = check_shape_common(shape);
  if (st != SA_OK) return st;
  if (!k_cache || !cache_len || !k_summary) return SA_ERR_NULL;
  if (block_k < 1) return SA_ERR_PARAM;
  if (!strides_ok(shape->k_stride)) return SA_ERR_SHAPE;
  if (!aligned16(k_cache) || !aligned16(k_summary)) return SA_ERR_SHAPE;
  DecArgs a;
  fill_dec_args(a, shape, block_k);
  a.kc = (const uint16_t*)k_cache;
  a.cache_len = cache_len;
  a.ksum = (const uint16_t*)k_summary;
  a.dbg = debug_word();
  log_decode("sa_build_block_summary", shape, block_k, nullptr, 0, "bf16", stream);
  if (launch_block_summary(a, stream) != hipSuccess) return SA_ERR_DEVICE;
  return debug_finish(SA_OK, a.dbg, stream);
}

// shared by the bf16-, 4-bit- and FP4-summary decode entries (exactly one summary form given:
// k_summary, or codes with scales, or codes with exps)
static sa_status decode_impl(const sa_shape* shape, const sa_decode_params* params, const void* q,
                             const void* k_cache, const void* v_cache, const void* k_summary,
                             const void* codes, const void* scales, const void* exps,
                             const int32_t* cache_len,
                             void* o, float* lse, int32_t* selected, void* ws, size_t ws_bytes,
                             hipStream_t stream) {
  sa_status st = check_decode(shape, params);
  if (st != SA_OK) return st;
  if (!q || !k_cache || !v_cache || !cache_len || !o) return SA_ERR_NULL;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(o))
    return SA_ERR_SHAPE;
  if (k_summary ? !aligned16(k_summary)
                : (!aligned16(codes) || !aligned16(exps ? exps : scales)))
    return SA_ERR_SHAPE;
  const DecLayout L = dec_layout(shape, params);
  if (!ws) return SA_ERR_WORKSPACE;
  if (ws_bytes < L.total || ((uintptr_t)ws % kAlign) != 0) return SA_ERR_WORKSPACE;
  DecArgs a;
  fill_dec_args(a, shape, params->block_k);
  char* base = (char*)ws;
  a.q = (const uint16_t*)q;
  a.kc = (const uint16_t*)k_cache;
  a.vc = (const uint16_t*)v_cache;
  a.ksum = (const uint16_t*)k_summary;
  a.ksum_q4 = (const uint8_t*)codes;
  a.ksum_scale = (const uint16_t*)scales;
  a.ksum_exp = (const uint8_t*)exps;
  a.cache_len = cache_len;
  a.o = (uint16_t*)o;
  a.lse = lse;
  a.scores = (float*)(base + L.scores);
  a.selected = selected ? selected : (int32_t*)(base + L.selected);
  a.partial = (float*)(base + L.partial);
  a.sel_count = (int32_t*)(base + L.counts);
  a.top_p = params->top_p;
  a.top_k = params->top_k_blocks;
  a.sink = params->sink_tokens;
  a.local = params->local_tokens;
  a.n_splits = decode_splits(shape, params);
  a.c = resolve_scale(params->softmax_scale, shape->head_dim);
  a.dbg = debug_word();
  log_decode("sa_sparse_decode", shape, params->block_k, params, a.n_splits,
             k_summary ? "bf16" : exps ? "fp4" : "q4", stream);
  if (launch_decode(a, stream) != hipSuccess) return SA_ERR_DEVICE;
  return debug_finish(SA_OK, a.dbg, stream);
}

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// the current device's address of `scratch`, looked up on the first call with that device
sa_status scratch_of_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return SA_ERR_DEVICE;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
      return SA_ERR_DEVICE;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return SA_OK;
}
}  // namespace

sa_status sa_sparse_decode_noalloc(const sa_shape* shape, const sa_decode_params* params,
                                   const void* q, const void* k_cache, const void* v_cache,
                                   const void* k_summary, const int32_t* cache_len, void* o,
                                   float* lse, int32_t* selected, hipStream_t stream) {
  sa_status st = check_decode(shape, params);
  if (st != SA_OK) return st;
  if (!k_summary) return SA_ERR_NULL;
  if (dec_layout(shape, params).total > SA_NOALLOC_SCRATCH_BYTES) return SA_ERR_WORKSPACE;
  void* ws = nullptr;
  if ((st = scratch_of_current_device(&ws)) != SA_OK) return st;
  return decode_impl(shape, params, q, k_cache, v_cache, k_summary, nullptr, nullptr, nullptr,
                     cache_len, o, lse, selected, ws, SA_NOALLOC_SCRATCH_BYTES, stream);
}

sa_status sa_sparse_decode(const sa_shape* shape, const sa_decode_params* params, const void* q,
                           const void* k_cache, const void* v_cache, const void* k_summary,
                           const int32_t* cache_len, void* o, float* lse, int32_t* selected,
                           void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!k_summary) return SA_ERR_NULL;
  return decode_impl(shape, params, q, k_cache, v_cache, k_summary, nullptr, nullptr, nullptr,
                     cache_len, o, lse, selected, ws, ws_bytes, stream);
}

sa_status sa_quantize_block_summary(const sa_shape* shape, int32_t block_k, const void* k_summary,
                                    void* codes, void* scales, hipStream_t stream) {
  sa_status st = check_shape_common(shape);
  if (st != SA_OK) return st;
  if (!k_summary || !codes || !scales) return SA_ERR_NULL;
  if (block_k < 1) return SA_ERR_PARAM;
  if (!aligned16(k_summary) || !aligned16(codes) || !aligned16(scales)) return SA_ERR_SHAPE;
  const int64_t n_groups = (int64_t)shape->batch * ceil_div(shape->seq_k, block_k) *
                           shape->n_kv_heads * (shape->head_dim / 32);
  if (launch_summary_q4((const uint16_t*)k_summary, (uint8_t*)codes, (uint16_t*)scales, n_groups,
                        stream) != hipSuccess)
    return SA_ERR_DEVICE;
  return SA_OK;
}

sa_status sa_sparse_decode_q4(const sa_shape* shape, const sa_decode_params* params, const void* q,
                              const void* k_cache, const void* v_cache, const void* summary_codes,
                              const void* summary_scales, const int32_t* cache_len, void* o,
                              float* lse, int32_t* selected, void* ws, size_t ws_bytes,
                              hipStream_t stream) {
  if (!summary_codes || !summary_scales) return SA_ERR_NULL;
  return decode_impl(shape, params, q, k_cache, v_cache, nullptr, summary_codes, summary_scales,
                     nullptr, cache_len, o, lse, selected, ws, ws_bytes, stream);
}

sa_status sa_quantize_block_summary_fp4(const sa_shape* shape, int32_t block_k,
                                        const void* k_summary, void* codes, void* exps,
                                        hipStream_t stream) {
  sa_status st = check_shape_common(shape);
  if (st != SA_OK) return st;
  if (!k_summary || !codes || !exps) return SA_ERR_NULL;
  if (block_k < 1) return SA_ERR_PARAM;
  if (!aligned16(k_summary) || !aligned16(codes) || !aligned16(exps)) return SA_ERR_SHAPE;
  const int64_t n_groups = (int64_t)shape->batch * ceil_div(shape->seq_k, block_k) *
                           shape->n_kv_heads * (shape->head_dim / 32);
  if (launch_summary_fp4((const uint16_t*)k_summary, (uint8_t*)codes, (uint8_t*)exps, n_groups,
                         stream) != hipSuccess)
    return SA_ERR_DEVICE;
  return SA_OK;
}

sa_status sa_sparse_decode_fp4(const sa_shape* shape, const sa_decode_params* params, const void* q,
                               const void* k_cache, const void* v_cache, const void* summary_codes,
                               const void* summary_exps, const int32_t* cache_len, void* o,
                               float* lse, int32_t* selected, void* ws, size_t ws_bytes,
                               hipStream_t stream) {
  if (!summary_codes || !summary_exps) return SA_ERR_NULL;
  return decode_impl(shape, params, q, k_cache, v_cache, nullptr, summary_codes, nullptr,
                     summary_exps, cache_len, o, lse, selected, ws, ws_bytes, stream);
}

sa_status sa_calibrate_theta(const sa_shape* shape, const sa_sparse_params* params,
                             const void* q, const void* k, const void* v,
                             float tau0, float err_bound, int32_t max_halvings,
                             float* theta_out, float* err_out, int32_t* halvings_out,
                             void* ws, size_t ws_bytes, hipStream_t stream) {
  sa_status st = check_prefill_shape(shape);
  if (st != SA_OK) return st;
  st = check_sparse_params(shape, params, false);
  if (st != SA_OK) return st;
  if (params->granularity != SA_BLOCK) return SA_ERR_UNSUPPORTED;
  if (!q || !k || !v || !theta_out) return SA_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v)) return SA_ERR_SHAPE;
  if (!(tau0 > 0.f && tau0 <= 1.f) || !(err_bound > 0.f) || isinf(err_bound) ||
      max_halvings < 0 || max_halvings > 64)
    return SA_ERR_PARAM;
  const CalLayout L = cal_layout(shape, params);
  if (!ws) return SA_ERR_WORKSPACE;
  if (ws_bytes < L.total || ((uintptr_t)ws % kAlign) != 0) return SA_ERR_WORKSPACE;

  const int B = shape->batch, N = shape->seq_q, Hq = shape->n_q_heads, D = shape->head_dim;
  const int nKB = ceil_div(N, params->block_k);
  char* base = (char*)ws;
  sa_lists lists;
  lists.counts = (int32_t*)(base + L.counts);
  lists.idx = (int32_t*)(base + L.idx);
  lists.stride = nKB;
  lists.margins = nullptr;
  // both outputs contiguous [B, N, Hq, D]
  sa_shape so = *shape;
  so.o_stride[0] = (int64_t)N * Hq * D;
  so.o_stride[1] = (int64_t)Hq * D;
  so.o_stride[2] = D;
  void* o_ref = base + L.o_ref;
  void* o_sp = base + L.o_sp;
  double* err_d = (double*)(base + L.err);
  const size_t est_bytes = L.counts - L.est;

  float theta[SA_MAX_Q_HEADS];
  int kh[SA_MAX_Q_HEADS];
  sa_sparse_params p = *params;
  p.theta = theta;
  // full attention: every causal block kept
  for (int h = 0; h < Hq; ++h) theta[h] = INFINITY;
  if ((st = sa_estimate_mask(&so, &p, q, k, &lists, base + L.est, est_bytes, stream)) != SA_OK) return st;
  if ((st = sa_sparse_prefill(&so, &p, q, k, v, &lists, o_ref, nullptr, stream)) != SA_OK) return st;

  const double theta0 = -log((double)tau0), ln2 = log(2.0);
  for (int h = 0; h < Hq; ++h) {
    kh[h] = 0;
    theta[h] = (float)theta0;
  }
  double err_h[SA_MAX_Q_HEADS];
  for (int round = 0;; ++round) {
    if ((st = sa_estimate_mask(&so, &p, q, k, &lists, base + L.est, est_bytes, stream)) != SA_OK) return st;
    if ((st = sa_sparse_prefill(&so, &p, q, k, v, &lists, o_sp, nullptr, stream)) != SA_OK) return st;
    if (launch_head_l1((const uint16_t*)o_ref, (const uint16_t*)o_sp, B, N, Hq, D, err_d, stream) !=
        hipSuccess)
      return SA_ERR_DEVICE;
    if (hipMemcpyAsync(err_h, err_d, Hq * sizeof(double), hipMemcpyDeviceToHost, stream) != hipSuccess ||
        hipStreamSynchronize(stream) != hipSuccess)
      return SA_ERR_DEVICE;
    bool done = true;
    for (int h = 0; h < Hq; ++h) {
      err_h[h] /= (double)B * N;
      if (!(err_h[h] < err_bound) && kh[h] < max_halvings) done = false;
    }
    if (done) break;
    for (int h = 0; h < Hq; ++h)
      if (!(err_h[h] < err_bound) && kh[h] < max_halvings) {
        ++kh[h];
        theta[h] = (float)(theta0 + kh[h] * ln2);
      }
  }
  for (int h = 0; h < Hq; ++h) {
    theta_out[h] = theta[h];
    if (err_out) err_out[h] = (float)err_h[h];
    if (halvings_out) halvings_out[h] = kh[h];
  }
  return SA_OK;
}

}  // extern "C"
