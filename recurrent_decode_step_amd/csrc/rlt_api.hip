// Host side of librlt.so: argument validation, buffer layouts, and the launch
// sequence of one decoder step.  All validation runs before any device work.
#include "rlt_internal.h"

#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <climits>
#include <mutex>
#include <string>
#include <vector>

namespace rlt {
thread_local PendingEvents g_pending_events;
}

using namespace rlt;

namespace {

thread_local std::string g_err;

rlt_status fail(rlt_status s, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return s;
}

rlt_status ok() {
  g_err.clear();
  return RLT_OK;
}

rlt_status hip_fail(hipError_t e, const char *what) {
  return fail(RLT_ERR_DEVICE, "%s: %s", what, hipGetErrorString(e));
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
int cdiv(int a, int b) { return (a + b - 1) / b; }

// Bump allocator over a caller buffer; with base == nullptr it only measures.
struct Arena {
  char *base;
  size_t off = 0;
  explicit Arena(void *b) : base(static_cast<char *>(b)) {}
  template <typename P> P *take(size_t bytes) {
    off = align256(off);
    P *p = base ? reinterpret_cast<P *>(base + off) : nullptr;
    off += bytes;
    return p;
  }
};

int esize_of(int dtype) { return dtype == RLT_DTYPE_BF16 ? 2 : 4; }
int kstep_of(int dtype) { return dtype == RLT_DTYPE_BF16 ? 32 : 16; }

// ---- GEMM plan.  K is cut into `parts` consecutive parts (one wavefront
// each, at most 16 k-steps per batch of loads); the cut depends on K only, so a
// row's result never depends on how many rows share the launch.
struct GemmPlan {
  int N, K, Np, KT, tiles, parts, tpw;
};

GemmPlan gemm_plan(int N, int K, int dtype) {
  GemmPlan p;
  p.N = N;
  p.K = K;
  p.Np = cdiv(N, 32) * 32;                     // whole pairs of 16-row tiles
  p.tiles = p.Np / 16;
  p.KT = cdiv(K, kstep_of(dtype));
  // K parts of 8+ k-steps (one wavefront each), at most 8; the cut depends on K only
  p.parts = std::max(1, std::min(kMaxParts, p.KT / 8));
  // two tiles per wavefront halve the activation reads; keep >= 128 workgroups
  p.tpw = (p.tiles >= 256 && dtype == RLT_DTYPE_BF16) ? 2 : 1;
  return p;
}

// batch-column blocking of a launch over n rows: 16, 32 or 64 rows per group
constexpr int kFillWorkgroups = 256;   // compute units of the part

struct ColPlan {
  int ncb, groups;
};
ColPlan col_plan(int n) {
  ColPlan c;
  const int blocks16 = cdiv(n, 16);
  c.ncb = blocks16 <= 1 ? 1 : (blocks16 <= 2 ? 2 : 4);
  c.groups = cdiv(n, c.ncb * 16);
  return c;
}

bool valid_dh(int dh) { return dh == 16 || dh == 32 || dh == 64 || dh == 128 || dh == 256; }

rlt_status check_config(const rlt_config *c) {
  if (!c) return fail(RLT_ERR_INVALID_ARG, "config is NULL");
  if (c->vocab < 1 || c->d_model < 1 || c->n_heads < 1 || c->n_layers < 1 || c->d_ffn < 1 ||
      c->window < 1)
    return fail(RLT_ERR_INVALID_ARG, "config dimensions must be positive");
  if (c->dtype != RLT_DTYPE_F32 && c->dtype != RLT_DTYPE_BF16)
    return fail(RLT_ERR_INVALID_ARG, "dtype must be RLT_DTYPE_F32 or RLT_DTYPE_BF16");
  if (c->head_dim * c->n_heads != c->d_model)
    return fail(RLT_ERR_SHAPE, "head_dim * n_heads (%d * %d) != d_model (%d)", c->head_dim,
                c->n_heads, c->d_model);
  if (!valid_dh(c->head_dim))
    return fail(RLT_ERR_UNSUPPORTED, "head_dim %d not in {16,32,64,128,256}", c->head_dim);
  if (c->d_model % 32 || c->d_ffn % 32)
    return fail(RLT_ERR_UNSUPPORTED, "d_model and d_ffn must be multiples of 32");
  if (c->mem_groups != 1 && c->mem_groups != c->n_layers)
    return fail(RLT_ERR_UNSUPPORTED, "mem_groups must be 1 or n_layers (got %d)", c->mem_groups);
  if (!(c->rms_eps >= 0.f) || !isfinite(c->rms_eps))
    return fail(RLT_ERR_INVALID_ARG, "rms_eps must be finite and >= 0");
  if (c->attn_chunk < 0) return fail(RLT_ERR_INVALID_ARG, "attn_chunk must be >= 0");
  return RLT_OK;
}

int chunk_of(const rlt_config *c) {
  const int cap = attn_chunk_max(c->dtype, c->head_dim);
  return c->attn_chunk > 0 ? std::min(c->attn_chunk, cap) : cap;
}

// ---------------------------------------------------------- static scratch
// Working memory of rlt_decoder_step_noalloc, for callers that cannot
// allocate: one array per device, held until the process ends.  Host code
// never names the array itself (its host-side symbol is no device address):
// the device address is looked up once per device with hipGetSymbolAddress,
// with that device current, and only that address is handed to kernels.
constexpr size_t kStaticScratchBytes = (size_t)16 << 20;
constexpr int kMaxDevices = 64;

}  // namespace

static __device__ __align__(256) char scratch[kStaticScratchBytes];

namespace {

std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

rlt_status static_scratch(int device, void **out) {
  *out = nullptr;
  if (device < 0 || device >= kMaxDevices)
    return fail(RLT_ERR_UNSUPPORTED, "device %d outside the static scratch table", device);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[device]) {
    int cur = -1;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (cur != device)
      return fail(RLT_ERR_INVALID_ARG, "the model's device %d must be current (device %d is)",
                  device, cur);
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "static scratch address");
    if (!p) return fail(RLT_ERR_DEVICE, "static scratch address is NULL");
    g_scratch_ptr[device] = p;
  }
  *out = g_scratch_ptr[device];
  return RLT_OK;
}

}  // namespace

// ------------------------------------------------------------------ handles
struct rlt_model {
  rlt_config cfg;
  uint64_t version;
  int device;
  int esize, chunk;
  GemmPlan p_merge, p_qkv, p_o, p_ffn1, p_ffn2, p_head;
  PackedMat wg, wout;
  std::vector<PackedMat> wqkv, wo, wqc, woc, w1, w2;
  float *s_star, *bg, *go, *g1, *g2, *g3;
};

struct ProfRec {
  hipEvent_t a, b;
  double bytes, flops;
  int cls;
};

// HIP event pairs recorded around the launches of selected kernel classes.
struct ProfLog {
  int mask = 0;
  int max = 0;
  int stride = 1;
  long long step_counter = 0;
  std::vector<ProfRec> recs;
  std::vector<hipEvent_t> pool;
};

struct rlt_state {
  rlt_config cfg;
  uint64_t version;
  int device;
  int B, max_tokens;
  size_t bytes;
  float *s;
  int *pos;
  char *ring_k, *ring_v;
  int *slots_dev;
  int *order_dev;            // [B] attention launch order of a ragged step (longest first)
  float *x, *sumsq;
  char *xg, *qbuf, *obuf, *hbuf;
  float *lscratch;           // [B][V] fp32 logits of a scored or generated step
  char *escratch;            // [B][d] e rows of generated tokens
  int *tok_dev;              // [B] the tokens of a generated step, contiguous
  std::vector<int> host_pos;
  std::vector<int> staged;   // slot list currently in slots_dev (empty: none)
  std::vector<int> staged_order;   // row order currently in order_dev
  std::vector<int> static_slots, static_order;   // host copies staged into the static scratch
  std::vector<StepPhase> step_tab[2];  // persistent step: phase tables (no head, head) being uploaded
  ProfLog plog;
};

namespace {

void model_plans(rlt_model *m) {
  const rlt_config &c = m->cfg;
  const int d = c.d_model, F = c.d_ffn;
  m->p_merge = gemm_plan(d, 2 * d, c.dtype);
  m->p_qkv = gemm_plan(3 * d, d, c.dtype);
  m->p_o = gemm_plan(d, d, c.dtype);
  m->p_ffn1 = gemm_plan(F, d, c.dtype);
  m->p_ffn2 = gemm_plan(d, F, c.dtype);
  m->p_head = gemm_plan(c.vocab, d, c.dtype);
}

size_t packed_bytes(const GemmPlan &g, int esize, int dtype) {
  return (size_t)g.Np * g.KT * kstep_of(dtype) * esize;
}

// model buffer layout (same walk for sizing and for carving)
size_t model_layout(rlt_model *m, void *base) {
  const rlt_config &c = m->cfg;
  const int L = c.n_layers, d = c.d_model;
  const int es = esize_of(c.dtype);
  Arena ar(base);
  auto mat = [&](const GemmPlan &g) {
    PackedMat pm;
    pm.N = g.N;
    pm.K = g.K;
    pm.Np = g.Np;
    pm.KT = g.KT;
    pm.p = ar.take<char>(packed_bytes(g, es, c.dtype));
    return pm;
  };
  m->wg = mat(m->p_merge);
  m->wqkv.resize(L);
  m->wo.resize(L);
  m->wqc.resize(L);
  m->woc.resize(L);
  m->w1.resize(L);
  m->w2.resize(L);
  for (int l = 0; l < L; ++l) {
    m->wqkv[l] = mat(m->p_qkv);
    m->wo[l] = mat(m->p_o);
    m->wqc[l] = mat(m->p_o);
    m->woc[l] = mat(m->p_o);
    m->w1[l] = mat(m->p_ffn1);
    m->w2[l] = mat(m->p_ffn2);
  }
  m->wout = mat(m->p_head);
  m->s_star = ar.take<float>((size_t)d * 4);
  m->bg = ar.take<float>((size_t)d * 4);
  m->go = ar.take<float>((size_t)d * 4);
  m->g1 = ar.take<float>((size_t)L * d * 4);
  m->g2 = ar.take<float>((size_t)L * d * 4);
  m->g3 = ar.take<float>((size_t)L * d * 4);
  return align256(ar.off);
}

size_t state_layout(const rlt_config &c, rlt_state *st, void *base, int B) {
  const int L = c.n_layers, d = c.d_model, H = c.n_heads, dh = c.head_dim, W = c.window;
  const int es = esize_of(c.dtype);
  Arena ar(base);
  st->s = ar.take<float>((size_t)B * d * 4);
  st->pos = ar.take<int>((size_t)B * 4);
  st->ring_k = ar.take<char>((size_t)L * B * H * W * dh * es);
  st->ring_v = ar.take<char>((size_t)L * B * H * W * dh * es);
  st->slots_dev = ar.take<int>((size_t)B * 4);
  st->order_dev = ar.take<int>((size_t)B * 4);
  st->x = ar.take<float>((size_t)B * d * 4);
  st->sumsq = ar.take<float>((size_t)cdiv(d, 16) * B * 4);
  const size_t rows16 = (size_t)cdiv(B, 16) * 16;   // packed activations: whole 16-row blocks
  st->xg = ar.take<char>(rows16 * d * es);
  st->qbuf = ar.take<char>((size_t)B * d * es);
  st->obuf = ar.take<char>(rows16 * d * es);
  st->hbuf = ar.take<char>(rows16 * c.d_ffn * es);
  st->lscratch = ar.take<float>((size_t)B * c.vocab * 4);
  st->escratch = ar.take<char>((size_t)B * d * es);
  st->tok_dev = ar.take<int>((size_t)B * 4);
  return align256(ar.off);
}

// Per-step working memory of the decoder step: the residual stream, the
// sum-of-squares partials, the packed normed GEMM inputs, q, the attention
// output, the FFN hidden layer and the staged slot list / row order.  It
// lives in the state (rlt_decoder_step) or in the library's static per-device
// array (rlt_decoder_step_noalloc).
struct StepScratch {
  float *x, *sumsq;
  char *xg, *qbuf, *obuf, *hbuf;
  int *slots_dev, *order_dev;
  int part_ld;               // leading dimension of the sum-of-squares partials
  bool shared;               // static array: shared by every call, nothing cached
  ProfLog *plog;             // null: no profiling
};

StepScratch state_scratch(rlt_state *st) {
  return StepScratch{st->x, st->sumsq, st->xg, st->qbuf, st->obuf, st->hbuf, st->slots_dev,
                     st->order_dev, st->B, false, &st->plog};
}

// The same buffers for n rows carved from `base` (nullptr: only measure).
size_t step_scratch_layout(const rlt_config &c, int n, void *base, StepScratch *w) {
  const int d = c.d_model;
  const int es = esize_of(c.dtype);
  const size_t rows16 = (size_t)cdiv(n, 16) * 16;
  Arena ar(base);
  w->slots_dev = ar.take<int>((size_t)n * 4);
  w->order_dev = ar.take<int>((size_t)n * 4);
  w->x = ar.take<float>((size_t)n * d * 4);
  w->sumsq = ar.take<float>((size_t)cdiv(d, 16) * n * 4);
  w->xg = ar.take<char>(rows16 * d * es);
  w->qbuf = ar.take<char>((size_t)n * d * es);
  w->obuf = ar.take<char>(rows16 * d * es);
  w->hbuf = ar.take<char>(rows16 * c.d_ffn * es);
  w->part_ld = n;
  w->shared = true;
  w->plog = nullptr;
  return align256(ar.off);
}

rlt_status check_state(const rlt_model *m, const rlt_state *st) {
  if (!m) return fail(RLT_ERR_INVALID_ARG, "model is NULL");
  if (!st) return fail(RLT_ERR_INVALID_ARG, "state is NULL");
  if (st->version != m->version)
    return fail(RLT_ERR_STALE, "state built for model version %llu, model is version %llu",
                (unsigned long long)st->version, (unsigned long long)m->version);
  const rlt_config &a = st->cfg, &b = m->cfg;
  if (a.d_model != b.d_model || a.n_layers != b.n_layers || a.n_heads != b.n_heads ||
      a.window != b.window || a.dtype != b.dtype || a.d_ffn != b.d_ffn || a.vocab != b.vocab ||
      a.mem_groups != b.mem_groups || a.attn_chunk != b.attn_chunk)
    return fail(RLT_ERR_CONVENTION, "state and model configurations differ");
  return RLT_OK;
}

rlt_status check_slots(const rlt_state *st, int n, const int32_t *slots) {
  if (n < 1 || n > st->B) return fail(RLT_ERR_INVALID_ARG, "n = %d outside [1, %d]", n, st->B);
  if (!slots) return RLT_OK;
  std::vector<char> seen(st->B, 0);
  for (int i = 0; i < n; ++i) {
    const int s = slots[i];
    if (s < 0 || s >= st->B) return fail(RLT_ERR_INVALID_ARG, "slot %d out of range", s);
    if (seen[s]) return fail(RLT_ERR_INVALID_ARG, "slot %d listed twice", s);
    seen[s] = 1;
  }
  return RLT_OK;
}

rlt_status check_memory_cfg(const rlt_config &c, const rlt_memory *mem, int max_slot) {
  if (!mem || !mem->k || !mem->v) return fail(RLT_ERR_INVALID_ARG, "memory K/V pointer is NULL");
  if (mem->capacity < 1) return fail(RLT_ERR_INVALID_ARG, "memory capacity < 1");
  if (mem->n_groups < c.mem_groups)
    return fail(RLT_ERR_INVALID_ARG, "memory holds %d groups, model reads %d", mem->n_groups,
                c.mem_groups);
  if (mem->n_seq <= max_slot)
    return fail(RLT_ERR_INVALID_ARG, "memory holds %d sequences, slot %d used", mem->n_seq, max_slot);
  if (mem->stride_pos < c.head_dim || mem->stride_head < 0 || mem->stride_seq < 0 ||
      mem->stride_group < 0)
    return fail(RLT_ERR_INVALID_ARG, "bad memory strides");
  const int es = esize_of(c.dtype);
  const int64_t strides[4] = {mem->stride_group, mem->stride_seq, mem->stride_head, mem->stride_pos};
  for (int64_t s : strides)
    if ((s * es) % 16) return fail(RLT_ERR_SHAPE, "memory strides must be multiples of 16 bytes");
  if (((uintptr_t)mem->k | (uintptr_t)mem->v) % 16)
    return fail(RLT_ERR_SHAPE, "memory pointers must be 16-byte aligned");
  return RLT_OK;
}

rlt_status check_memory(const rlt_model *m, const rlt_memory *mem, int max_slot) {
  return check_memory_cfg(m->cfg, mem, max_slot);
}

// Stage a slot list in device memory (only when it differs from the staged one).
rlt_status stage_slots(rlt_state *st, int n, const int32_t *slots, hipStream_t s) {
  if (st->staged.size() == (size_t)n && std::equal(slots, slots + n, st->staged.begin()))
    return RLT_OK;
  hipError_t e = hipMemcpyAsync(st->slots_dev, slots, (size_t)n * 4, hipMemcpyHostToDevice, s);
  if (e != hipSuccess) return hip_fail(e, "staging slot list");
  st->staged.assign(slots, slots + n);
  return RLT_OK;
}

hipEvent_t pooled_event(ProfLog &pl) {
  hipEvent_t e = nullptr;
  if (!pl.pool.empty()) {
    e = pl.pool.back();
    pl.pool.pop_back();
  } else if (hipEventCreate(&e) != hipSuccess) {
    e = nullptr;
  }
  return e;
}

void prof_release(ProfLog &pl) {
  for (ProfRec &r : pl.recs) {
    (void)hipEventDestroy(r.a);
    (void)hipEventDestroy(r.b);
  }
  for (hipEvent_t e : pl.pool) (void)hipEventDestroy(e);
  pl.recs.clear();
  pl.pool.clear();
}

rlt_status prof_begin(ProfLog &pl, int class_mask, int nclasses, int max_launches, int step_stride) {
  if (class_mask < 0 || class_mask >= (1 << nclasses))
    return fail(RLT_ERR_INVALID_ARG, "bad kernel class mask");
  if (max_launches < 0) return fail(RLT_ERR_INVALID_ARG, "max_launches < 0");
  if (step_stride < 1) return fail(RLT_ERR_INVALID_ARG, "step_stride < 1");
  pl.mask = class_mask;
  pl.max = max_launches;
  pl.stride = step_stride;
  pl.step_counter = 0;
  return ok();
}

rlt_status prof_collect(ProfLog &pl, int kclass, double *total_ms, int32_t *launches,
                        double *bytes_moved, double *flops) {
  double tot = 0, bytes = 0, fl = 0;
  int cnt = 0;
  std::vector<ProfRec> keep;
  for (ProfRec &r : pl.recs) {
    if (r.cls != kclass) {
      keep.push_back(r);
      continue;
    }
    float ms = 0.f;
    hipError_t e = hipEventSynchronize(r.b);
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, r.a, r.b);
    if (e != hipSuccess) return hip_fail(e, "profile events");
    tot += ms;
    bytes += r.bytes;
    fl += r.flops;
    ++cnt;
    pl.pool.push_back(r.a);
    pl.pool.push_back(r.b);
  }
  pl.recs.swap(keep);
  if (total_ms) *total_ms = tot;
  if (launches) *launches = cnt;
  if (bytes_moved) *bytes_moved = bytes;
  if (flops) *flops = fl;
  return ok();
}

// Times one launch of a selected class: the event pair is handed to the
// launch (rlt::launch binds it to the kernel's own dispatch), so the timing
// adds no packet to the stream and measures the kernel alone.
struct Prof {
  ProfLog &pl;
  int cls;
  bool on;
  hipEvent_t a = nullptr, b = nullptr;
  Prof(ProfLog &pl_, int cls_, hipStream_t)
      : pl(pl_), cls(cls_),
        on(((pl_.mask >> cls_) & 1) && (int)pl_.recs.size() < pl_.max &&
           pl_.step_counter % pl_.stride == 0) {
    if (on) {
      a = pooled_event(pl);
      b = pooled_event(pl);
      on = a && b;
    }
    if (on) g_pending_events = PendingEvents{a, b, false};
  }
  void done(double bytes, double flops = 0.0) {
    if (!on) return;
    on = false;
    const bool used = g_pending_events.used;
    g_pending_events = PendingEvents{};
    if (used) {
      pl.recs.push_back({a, b, bytes, flops, cls});
    } else {                    // nothing was launched: give the pair back
      pl.pool.push_back(a);
      pl.pool.push_back(b);
    }
  }
  ~Prof() {
    if (on) {                   // an error path left before done()
      g_pending_events = PendingEvents{};
      pl.pool.push_back(a);
      pl.pool.push_back(b);
    }
  }
};

// Enqueue one decoder step for n rows.  e rows: e_base + i*ld_e (elements);
// logits rows: logits + i*ld_logits (NULL: no head).  The slot list is already
// staged (identity == true: rows are slots 0..n-1).
rlt_status enqueue_step(const rlt_model *m, rlt_state *st, const StepScratch &w, int n,
                        bool identity, const int32_t *host_slots, const void *e, int64_t ld_e,
                        const rlt_memory *mem, float *logits, int64_t ld_logits, hipStream_t s) {
  const rlt_config &c = m->cfg;
  const int d = c.d_model, H = c.n_heads, dh = c.head_dim, W = c.window, L = c.n_layers;
  const int F = c.d_ffn, B = st->B, es = m->esize;
  hipError_t err;
  ProfLog no_prof;                                  // profiling off: mask 0
  ProfLog *plog = w.plog ? w.plog : &no_prof;

  // host mirror: algorithmic bytes of the two attentions (for profiling)
  double swa_len = 0, mem_len = 0;
  int tmin = INT_MAX, tmax = 0;
  for (int i = 0; i < n; ++i) {
    const int t = st->host_pos[identity ? i : host_slots[i]] + 1;
    swa_len += std::min(t, W);
    mem_len += t;
    tmin = std::min(tmin, t);
    tmax = std::max(tmax, t);
  }
  // Rows of different lengths (a ragged batch): the attention launches take
  // the rows longest first, so that the long rows do not form the tail of the
  // launch.  A row's result does not depend on the order.
  const int *order_dev = nullptr;
  if (tmax > tmin) {
    std::vector<int> ord(n);
    for (int i = 0; i < n; ++i) ord[i] = i;
    auto t_of = [&](int i) { return st->host_pos[identity ? i : host_slots[i]]; };
    std::stable_sort(ord.begin(), ord.end(), [&](int x, int y) { return t_of(x) > t_of(y); });
    if (w.shared) {
      // the static array is shared by every call: stage the order every time
      st->static_order = ord;
      err = hipMemcpyAsync(w.order_dev, st->static_order.data(), (size_t)n * 4,
                           hipMemcpyHostToDevice, s);
      if (err != hipSuccess) return hip_fail(err, "staging the attention row order");
    } else if (ord != st->staged_order) {
      st->staged_order = ord;
      err = hipMemcpyAsync(w.order_dev, st->staged_order.data(), (size_t)n * 4,
                           hipMemcpyHostToDevice, s);
      if (err != hipSuccess) {
        st->staged_order.clear();
        return hip_fail(err, "staging the attention row order");
      }
    }
    order_dev = w.order_dev;
  }

  const ColPlan cp = col_plan(n);
  GemmArgs base;
  memset(&base, 0, sizeof base);
  base.n_rows = n;
  base.slots = identity ? nullptr : w.slots_dev;
  base.pos = st->pos;
  base.s_state = st->s;
  base.d = d;
  base.sumsq = w.sumsq;
  base.n_parts = cdiv(d, 16);
  base.part_ld = w.part_ld;
  base.eps = c.rms_eps;
  base.x = w.x;
  base.x_in = w.x;
  base.xg = w.xg;
  base.sumsq_out = w.sumsq;
  base.H = H;
  base.dh = dh;
  base.W = W;
  base.kt_out = d / kstep_of(c.dtype);

  auto gemm = [&](const GemmPlan &g, const PackedMat &w, int act, int epi, GemmArgs a,
                  const char *what, double act_bytes, double out_bytes) -> rlt_status {
    a.wp = w.p;
    a.N = g.N;
    a.K = g.K;
    a.KT = g.KT;
    Prof p(*plog, RLT_K_GEMM, s);
    // narrower column groups until the launch has a workgroup per CU (results
    // per row do not depend on the grouping)
    ColPlan gc = cp;
    int tpw = gc.ncb <= 2 ? g.tpw : 1;           // registers: two tiles only up to 32 rows
    while (g.tpw == 1 && gc.ncb > 1 && (g.tiles / tpw) * gc.groups < kFillWorkgroups) {
      gc.ncb /= 2;
      gc.groups = cdiv(n, gc.ncb * 16);
      tpw = gc.ncb <= 2 ? g.tpw : 1;
    }
    // one 16-row column group whose tile pairs leave CUs without a workgroup
    // (N = 4096 at 16 rows or fewer): one tile per wavefront
    if (gc.ncb == 1 && tpw > 1 && (g.tiles / tpw) * gc.groups < kFillWorkgroups) tpw = 1;
    // ... and tile pairs whose last round of workgroups would leave CUs idle
    // where single tiles fill whole rounds (N = 12288 at 16 rows or fewer:
    // 384 workgroups against 768)
    if (gc.ncb == 1 && tpw > 1 && ((g.tiles / tpw) * gc.groups) % kFillWorkgroups != 0 &&
        (g.tiles * gc.groups) % kFillWorkgroups == 0)
      tpw = 1;
    // large batches: the persistent kernel (same arithmetic, activations in
    // registers, many tiles per workgroup)
    const hipError_t e2 =
        gemm_persistent_applies(c.dtype, act, epi, n, g.KT, g.parts)
            ? launch_gemm_persistent(c.dtype, epi, a, g.tiles, n, g.parts, s)
            : launch_gemm(c.dtype, gc.ncb, tpw, act, epi, a, g.tiles, gc.groups, g.parts, s);
    if (e2 != hipSuccess) return hip_fail(e2, what);
    p.done((double)g.N * g.K * es + act_bytes + out_bytes);
    return RLT_OK;
  };
  rlt_status rs;
  const double row_in = (double)n * d * es;         // a normed / plain [n][d] activation
  const double resid_out = (double)n * d * (8 + es); // x read + write, x*gamma out

  // gated merge: x = g*e + (1-g)*s, g = sigmoid(W_g [e ; s] + b_g)
  {
    GemmArgs a = base;
    a.act = e;
    a.ld_act = ld_e;
    a.bias = m->bg;
    a.gamma_next = m->g1;
    if ((rs = gemm(m->p_merge, m->wg, ACT_MERGE, EPI_MERGE, a, "merge gemm",
                   (double)n * d * (es + 4), (double)n * d * (4 + es))) != RLT_OK)
      return rs;
  }

  const size_t ring_layer = (size_t)B * H * W * dh * es;
  AttnArgs at;
  memset(&at, 0, sizeof at);
  at.slots = base.slots;
  at.order = order_dev;
  at.pos = st->pos;
  at.H = H;
  at.d = d;
  at.ch = m->chunk;
  at.kt_out = d / kstep_of(c.dtype);
  at.scale_log2 = (float)(1.4426950408889634 / sqrt((double)dh));

  for (int l = 0; l < L; ++l) {
    const bool last = l == L - 1;
    // (1) Q,K,V of RMSNorm(x; g1); k,v go to window entry (t-1) mod W
    {
      GemmArgs a = base;
      a.act = w.xg;
      a.ld_act = d;
      a.out = w.qbuf;
      a.ld_out = d;
      a.ring_k = st->ring_k + l * ring_layer;
      a.ring_v = st->ring_v + l * ring_layer;
      if ((rs = gemm(m->p_qkv, m->wqkv[l], ACT_PLAIN, EPI_QKV, a, "qkv gemm", row_in,
                     (double)n * 3 * d * es)) != RLT_OK)
        return rs;
    }
    // (2) sliding-window self-attention over window entries 0..min(t,W)-1
    {
      AttnArgs a = at;
      a.q = w.qbuf;
      a.out = w.obuf;
      a.kb = st->ring_k + l * ring_layer;
      a.vb = st->ring_v + l * ring_layer;
      a.s_seq = (int64_t)H * W * dh;
      a.s_head = (int64_t)W * dh;
      a.s_pos = dh;
      a.len_cap = W;
      Prof p(*plog, RLT_K_SWA, s);
      if ((err = launch_attn(c.dtype, dh, a, n, s)) != hipSuccess)
        return hip_fail(err, "window attention launch");
      p.done(swa_len * 2.0 * d * es + 2.0 * n * d * es);
    }
    // (3) x += W_O o
    {
      GemmArgs a = base;
      a.act = w.obuf;
      a.ld_act = d;
      a.gamma_next = m->g2 + (size_t)l * d;
      if ((rs = gemm(m->p_o, m->wo[l], ACT_PLAIN, EPI_RESID, a, "o gemm", row_in, resid_out)) !=
          RLT_OK)
        return rs;
    }
    // (4) cross-attention query of RMSNorm(x; g2)
    {
      GemmArgs a = base;
      a.act = w.xg;
      a.ld_act = d;
      a.out = w.qbuf;
      a.ld_out = d;
      if ((rs = gemm(m->p_o, m->wqc[l], ACT_PLAIN, EPI_STORE, a, "qc gemm", row_in,
                     (double)n * d * es)) != RLT_OK)
        return rs;
    }
    // (5) cross-attention to memory positions 1..t of group g(l)
    {
      const int grp = c.mem_groups == 1 ? 0 : l;
      AttnArgs a = at;
      a.q = w.qbuf;
      a.out = w.obuf;
      a.kb = static_cast<const char *>(mem->k) + (size_t)grp * mem->stride_group * es;
      a.vb = static_cast<const char *>(mem->v) + (size_t)grp * mem->stride_group * es;
      a.s_seq = mem->stride_seq;
      a.s_head = mem->stride_head;
      a.s_pos = mem->stride_pos;
      a.len_cap = 0x7fffffff;
      Prof p(*plog, RLT_K_CROSS, s);
      if ((err = launch_attn(c.dtype, dh, a, n, s)) != hipSuccess)
        return hip_fail(err, "cross attention launch");
      p.done(mem_len * 2.0 * d * es + 2.0 * n * d * es);
    }
    // (6) x += W_Oc o_c
    {
      GemmArgs a = base;
      a.act = w.obuf;
      a.ld_act = d;
      a.gamma_next = m->g3 + (size_t)l * d;
      if ((rs = gemm(m->p_o, m->woc[l], ACT_PLAIN, EPI_RESID, a, "oc gemm", row_in, resid_out)) !=
          RLT_OK)
        return rs;
    }
    // (7) GELU(W_1 RMSNorm(x; g3))
    {
      GemmArgs a = base;
      a.act = w.xg;
      a.ld_act = d;
      a.out = w.hbuf;
      a.ld_out = F;
      a.kt_out = F / kstep_of(c.dtype);
      if ((rs = gemm(m->p_ffn1, m->w1[l], ACT_PLAIN, EPI_GELU, a, "ffn1 gemm", row_in,
                     (double)n * F * es)) != RLT_OK)
        return rs;
    }
    // (8) x += W_2 h; the last layer also writes s_t
    {
      GemmArgs a = base;
      a.act = w.hbuf;
      a.ld_act = F;
      a.gamma_next = last ? m->go : m->g1 + (size_t)(l + 1) * d;
      if (last) {
        a.s_out = st->s;
        a.advance_pos = logits ? 0 : 1;
      }
      if ((rs = gemm(m->p_ffn2, m->w2[l], ACT_PLAIN, EPI_RESID, a, "ffn2 gemm",
                     (double)n * F * es, resid_out)) != RLT_OK)
        return rs;
    }
  }

  // head: logits = W_o RMSNorm(s_t; g_o)
  if (logits) {
    GemmArgs a = base;
    a.act = w.xg;
    a.ld_act = d;
    a.out = logits;
    a.ld_out = ld_logits;
    a.advance_pos = 1;
    if ((rs = gemm(m->p_head, m->wout, ACT_PLAIN, EPI_LOGITS, a, "head gemm", row_in,
                   (double)n * c.vocab * 4)) != RLT_OK)
      return rs;
  }

  for (int i = 0; i < n; ++i) st->host_pos[identity ? i : host_slots[i]] += 1;
  st->plog.step_counter += 1;
  return RLT_OK;
}

// ------------------------------------------------------- persistent step
// Workspace of rlt_run_sequence_persistent for n rows: the error word, one
// flag per item of a step (with the head), the two phase tables (a step
// without and with the head), and one output buffer per producing phase, so
// no address is written twice within one launch.  Producer k of the residual
// stream is the merge (k = 0) and, in layer l, the O, Oc and FFN-down
// products (k = 3l+1, 3l+2, 3l+3).
constexpr int kStepMaxGrid = 1024;

struct StepBufs {
  unsigned *err, *items;
  size_t n_items;
  StepPhase *tab[2];
  std::vector<float *> x, sumsq;     // [3L+1]
  std::vector<char *> xg;            // [3L+1]
  std::vector<char *> q, o;          // [2L]: (q, q_c), (window, cross) attention outputs
  std::vector<char *> h;             // [L]
};

int step_phases_max(const rlt_config &c) { return 2 + 8 * c.n_layers; }

// items of a step with the head: GEMM phases tiles x 16-row column groups,
// attention phases rows x heads
size_t step_items(const rlt_config &c, int n) {
  const int d = c.d_model, L = c.n_layers;
  const size_t cg = (size_t)cdiv(n, 16), nh = (size_t)n * c.n_heads;
  auto tiles = [](int N) { return (size_t)cdiv(N, 32) * 2; };
  return tiles(d) * cg +
         (size_t)L * ((tiles(3 * d) + 4 * tiles(d) + tiles(c.d_ffn)) * cg + 2 * nh) +
         tiles(c.vocab) * cg;
}

size_t step_layout(const rlt_config &c, int n, void *base, StepBufs *b) {
  const int L = c.n_layers, d = c.d_model, F = c.d_ffn;
  const int es = esize_of(c.dtype);
  const size_t rows16 = (size_t)cdiv(n, 16) * 16;
  Arena ar(base);
  b->err = ar.take<unsigned>(256);
  b->n_items = step_items(c, n);
  b->items = ar.take<unsigned>(b->n_items * 4);
  for (int t = 0; t < 2; ++t) b->tab[t] = ar.take<StepPhase>((size_t)step_phases_max(c) * sizeof(StepPhase));
  b->x.resize(3 * L + 1);
  b->sumsq.resize(3 * L + 1);
  b->xg.resize(3 * L + 1);
  for (int k = 0; k <= 3 * L; ++k) {
    b->x[k] = ar.take<float>((size_t)n * d * 4);
    b->sumsq[k] = ar.take<float>((size_t)cdiv(d, 16) * n * 4);
    b->xg[k] = ar.take<char>(rows16 * d * es);
  }
  b->q.resize(2 * L);
  b->o.resize(2 * L);
  for (int k = 0; k < 2 * L; ++k) {
    b->q[k] = ar.take<char>((size_t)n * d * es);
    b->o[k] = ar.take<char>(rows16 * d * es);
  }
  b->h.resize(L);
  for (int l = 0; l < L; ++l) b->h[l] = ar.take<char>(rows16 * F * es);
  return align256(ar.off);
}

// The phases of one step over all n = B slots of the state (identity slot
// list), in the launch chain's order and with its K parts; every GEMM phase
// uses 16-row tiles and 16-row column groups (a placement choice, invisible
// in the results).  with_head: the head phase is the last and advances the
// positions, otherwise the last FFN-down does.
// rlt_persistent_test_stall: waits look for an epoch no item stores
std::atomic<int> g_test_stall{0};

int fl_count_check(const std::vector<StepPhase> &tab) {
  return tab.empty() ? 0 : tab.back().fl + tab.back().nv;
}

void build_step_phases(const rlt_model *m, rlt_state *st, const rlt_memory *mem,
                       const StepBufs &b, bool with_head, std::vector<StepPhase> &out) {
  const rlt_config &c = m->cfg;
  const int d = c.d_model, H = c.n_heads, dh = c.head_dim, W = c.window, L = c.n_layers;
  const int F = c.d_ffn, n = st->B, es = m->esize;
  const int col_groups = cdiv(n, 16);
  out.clear();

  GemmArgs base;
  memset(&base, 0, sizeof base);
  base.n_rows = n;
  base.slots = nullptr;
  base.pos = st->pos;
  base.s_state = st->s;
  base.d = d;
  base.n_parts = cdiv(d, 16);
  base.part_ld = n;
  base.eps = c.rms_eps;
  base.H = H;
  base.dh = dh;
  base.W = W;
  base.kt_out = d / kstep_of(c.dtype);

  auto gemm = [&](const GemmPlan &g, const PackedMat &w, int act, int epi, GemmArgs a) {
    a.wp = w.p;
    a.N = g.N;
    a.K = g.K;
    a.KT = g.KT;
    gemm_grid(c.dtype, 1, 1, g.tiles, col_groups, &a);
    StepPhase ph;
    memset(&ph, 0, sizeof ph);
    ph.kind = STEP_GEMM;
    ph.act = act;
    ph.epi = epi;
    ph.nv = a.tile_groups * a.col_groups;
    ph.parts = g.parts;
    ph.g = a;
    out.push_back(ph);
  };
  AttnArgs at;
  memset(&at, 0, sizeof at);
  at.slots = nullptr;
  at.order = nullptr;
  at.pos = st->pos;
  at.H = H;
  at.d = d;
  at.ch = m->chunk;
  at.kt_out = d / kstep_of(c.dtype);
  at.scale_log2 = (float)(1.4426950408889634 / sqrt((double)dh));
  auto attn = [&](const AttnArgs &a) {
    StepPhase ph;
    memset(&ph, 0, sizeof ph);
    ph.kind = STEP_ATTN;
    ph.nv = n * H;
    ph.n_rows = n;
    ph.at = a;
    out.push_back(ph);
  };

  // gated merge (its e rows come with each launch)
  {
    GemmArgs a = base;
    a.bias = m->bg;
    a.gamma_next = m->g1;
    a.x = b.x[0];
    a.x_in = b.x[0];
    a.xg = b.xg[0];
    a.sumsq_out = b.sumsq[0];
    gemm(m->p_merge, m->wg, ACT_MERGE, EPI_MERGE, a);
  }
  const size_t ring_layer = (size_t)st->B * H * W * dh * es;
  for (int l = 0; l < L; ++l) {
    const bool last = l == L - 1;
    const int k0 = 3 * l;
    {  // Q, K, V of RMSNorm(x; g1); k, v to window entry (t-1) mod W
      GemmArgs a = base;
      a.act = b.xg[k0];
      a.ld_act = d;
      a.sumsq = b.sumsq[k0];
      a.out = b.q[2 * l];
      a.ld_out = d;
      a.ring_k = st->ring_k + l * ring_layer;
      a.ring_v = st->ring_v + l * ring_layer;
      gemm(m->p_qkv, m->wqkv[l], ACT_PLAIN, EPI_QKV, a);
    }
    {  // window attention
      AttnArgs a = at;
      a.q = b.q[2 * l];
      a.out = b.o[2 * l];
      a.kb = st->ring_k + l * ring_layer;
      a.vb = st->ring_v + l * ring_layer;
      a.s_seq = (int64_t)H * W * dh;
      a.s_head = (int64_t)W * dh;
      a.s_pos = dh;
      a.len_cap = W;
      attn(a);
    }
    {  // x += W_O o
      GemmArgs a = base;
      a.act = b.o[2 * l];
      a.ld_act = d;
      a.x_in = b.x[k0];
      a.x = b.x[k0 + 1];
      a.xg = b.xg[k0 + 1];
      a.sumsq_out = b.sumsq[k0 + 1];
      a.gamma_next = m->g2 + (size_t)l * d;
      gemm(m->p_o, m->wo[l], ACT_PLAIN, EPI_RESID, a);
    }
    {  // cross-attention query of RMSNorm(x; g2)
      GemmArgs a = base;
      a.act = b.xg[k0 + 1];
      a.ld_act = d;
      a.sumsq = b.sumsq[k0 + 1];
      a.out = b.q[2 * l + 1];
      a.ld_out = d;
      gemm(m->p_o, m->wqc[l], ACT_PLAIN, EPI_STORE, a);
    }
    {  // cross-attention to memory positions 1..t of group g(l)
      const int grp = c.mem_groups == 1 ? 0 : l;
      AttnArgs a = at;
      a.q = b.q[2 * l + 1];
      a.out = b.o[2 * l + 1];
      a.kb = static_cast<const char *>(mem->k) + (size_t)grp * mem->stride_group * es;
      a.vb = static_cast<const char *>(mem->v) + (size_t)grp * mem->stride_group * es;
      a.s_seq = mem->stride_seq;
      a.s_head = mem->stride_head;
      a.s_pos = mem->stride_pos;
      a.len_cap = 0x7fffffff;
      attn(a);
    }
    {  // x += W_Oc o_c
      GemmArgs a = base;
      a.act = b.o[2 * l + 1];
      a.ld_act = d;
      a.x_in = b.x[k0 + 1];
      a.x = b.x[k0 + 2];
      a.xg = b.xg[k0 + 2];
      a.sumsq_out = b.sumsq[k0 + 2];
      a.gamma_next = m->g3 + (size_t)l * d;
      gemm(m->p_o, m->woc[l], ACT_PLAIN, EPI_RESID, a);
    }
    {  // GELU(W_1 RMSNorm(x; g3))
      GemmArgs a = base;
      a.act = b.xg[k0 + 2];
      a.ld_act = d;
      a.sumsq = b.sumsq[k0 + 2];
      a.out = b.h[l];
      a.ld_out = F;
      a.kt_out = F / kstep_of(c.dtype);
      gemm(m->p_ffn1, m->w1[l], ACT_PLAIN, EPI_GELU, a);
    }
    {  // x += W_2 h; the last layer also writes s_t
      GemmArgs a = base;
      a.act = b.h[l];
      a.ld_act = F;
      a.x_in = b.x[k0 + 2];
      a.x = b.x[k0 + 3];
      a.xg = b.xg[k0 + 3];
      a.sumsq_out = b.sumsq[k0 + 3];
      a.gamma_next = last ? m->go : m->g1 + (size_t)(l + 1) * d;
      if (last) {
        a.s_out = st->s;
        a.advance_pos = with_head ? 0 : 1;
      }
      gemm(m->p_ffn2, m->w2[l], ACT_PLAIN, EPI_RESID, a);
    }
  }
  if (with_head) {  // logits = W_o RMSNorm(s_t; g_o) (the output comes with each launch)
    GemmArgs a = base;
    a.act = b.xg[3 * L];
    a.ld_act = d;
    a.sumsq = b.sumsq[3 * L];
    a.advance_pos = 1;
    gemm(m->p_head, m->wout, ACT_PLAIN, EPI_LOGITS, a);
  }

  // item flags and what each phase waits for: every phase reads the phase
  // before it.  GEMM after GEMM: every tile of the column group (the
  // normalised input needs the whole row); GEMM after attention: every head
  // of the column group's rows; attention after QKV or Qc: the tiles of its
  // head (q, k, v or q_c) of its row's column group.
  int fl = 0;
  for (size_t p = 0; p < out.size(); ++p) {
    StepPhase &ph = out[p];
    ph.n_rows = n;
    ph.fl = fl;
    fl += ph.nv;
    if (p == 0) {
      ph.dep_kind = DEP_NONE;
      continue;
    }
    const StepPhase &pr = out[p - 1];
    ph.dep = pr.fl;
    if (ph.kind == STEP_GEMM && pr.kind == STEP_GEMM) {
      ph.dep_kind = DEP_GEMM_CG;
      ph.dep_n = pr.g.tile_groups;
    } else if (ph.kind == STEP_GEMM) {
      ph.dep_kind = DEP_ATTN_ROWS;
      ph.dep_H = H;
    } else {
      ph.dep_kind = DEP_HEAD_TILES;
      ph.dep_n = pr.g.tile_groups;
      ph.dep_r = pr.epi == EPI_QKV ? 3 : 1;
      ph.dep_rs = d / 16;
      ph.dep_ht = dh / 16;
    }
  }
}

rlt_status check_positions(const rlt_state *st, const rlt_memory *mem, int n,
                           const int32_t *slots, int steps) {
  for (int i = 0; i < n; ++i) {
    const int slot = slots ? slots[i] : i;
    const long long last = (long long)st->host_pos[slot] + steps;
    if (last > mem->capacity)
      return fail(RLT_ERR_RANGE, "slot %d would reach position %lld > memory capacity %d", slot,
                  last, mem->capacity);
    if (last > st->max_tokens)
      return fail(RLT_ERR_RANGE, "slot %d would reach position %lld > max_tokens %d", slot, last,
                  st->max_tokens);
  }
  return RLT_OK;
}

// Zero device memory for calls that take no stream: the memset goes to the
// null stream and is waited for, so work later enqueued on any stream
// (blocking or not) finds the memory cleared.
hipError_t clear_now(void *p, size_t bytes) {
  hipError_t e = hipMemset(p, 0, bytes);
  if (e == hipSuccess) e = hipStreamSynchronize(nullptr);
  return e;
}

rlt_status device_health() {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "earlier device error");
  return RLT_OK;
}

void snapshot_offsets(const rlt_config *c, size_t *off_s, size_t *off_k, size_t *off_v,
                      size_t *rec) {
  const int es = esize_of(c->dtype);
  const size_t hist = (size_t)c->n_layers * c->n_heads * (c->window - 1) * c->head_dim * es;
  *off_s = 256;
  *off_k = *off_s + align256((size_t)c->d_model * 4);
  *off_v = *off_k + align256(hist);
  *rec = *off_v + align256(hist);
}

}  // namespace

// =================================================================== C ABI
extern "C" {

int32_t rlt_abi_version(void) { return RLT_ABI_VERSION; }

const char *rlt_status_str(rlt_status s) {
  switch (s) {
    case RLT_OK: return "RLT_OK";
    case RLT_ERR_INVALID_ARG: return "RLT_ERR_INVALID_ARG";
    case RLT_ERR_SHAPE: return "RLT_ERR_SHAPE";
    case RLT_ERR_RANGE: return "RLT_ERR_RANGE";
    case RLT_ERR_STALE: return "RLT_ERR_STALE";
    case RLT_ERR_CONVENTION: return "RLT_ERR_CONVENTION";
    case RLT_ERR_UNSUPPORTED: return "RLT_ERR_UNSUPPORTED";
    case RLT_ERR_DEVICE: return "RLT_ERR_DEVICE";
  }
  return "RLT_ERR_UNKNOWN";
}

const char *rlt_last_error(void) { return g_err.c_str(); }

size_t rlt_model_bytes(const rlt_config *cfg) {
  if (check_config(cfg) != RLT_OK) return 0;
  rlt_model m;
  m.cfg = *cfg;
  model_plans(&m);
  return model_layout(&m, nullptr);
}

rlt_status rlt_model_create(const rlt_config *cfg, const rlt_params *src, uint64_t model_version,
                            void *dev_buf, size_t bytes, void *stream, rlt_model **out) {
  rlt_status rs;
  if (!out) return fail(RLT_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  if ((rs = check_config(cfg)) != RLT_OK) return rs;
  if (!src) return fail(RLT_ERR_INVALID_ARG, "params is NULL");
  const void *need[] = {src->s_star, src->wg, src->bg, src->g1, src->g2, src->g3, src->wq,
                        src->wk,     src->wv, src->wo, src->wqc, src->woc, src->w1, src->w2,
                        src->go,     src->wout};
  for (const void *p : need)
    if (!p) return fail(RLT_ERR_INVALID_ARG, "a parameter pointer is NULL");
  if (!dev_buf) return fail(RLT_ERR_INVALID_ARG, "dev_buf is NULL");
  if ((uintptr_t)dev_buf % 256) return fail(RLT_ERR_SHAPE, "dev_buf must be 256-byte aligned");
  const size_t need_bytes = rlt_model_bytes(cfg);
  if (bytes < need_bytes)
    return fail(RLT_ERR_SHAPE, "model buffer %zu bytes < %zu required", bytes, need_bytes);
  if ((rs = device_health()) != RLT_OK) return rs;

  rlt_model *m = new rlt_model();
  m->cfg = *cfg;
  m->version = model_version;
  (void)hipGetDevice(&m->device);
  m->esize = esize_of(cfg->dtype);
  m->chunk = chunk_of(cfg);
  model_plans(m);
  model_layout(m, dev_buf);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int L = cfg->n_layers, d = cfg->d_model, F = cfg->d_ffn, es = m->esize;
  const size_t dd = (size_t)d * d * es;
  hipError_t e = hipSuccess;
  auto pack = [&](const void *p, int rows, int K, int tile_begin, int tile_end,
                  const PackedMat &dst) {
    if (e == hipSuccess) e = launch_pack_tiles(p, rows, K, K, tile_begin, tile_end, dst, cfg->dtype, s);
  };
  auto tiles = [](const PackedMat &pm) { return pm.Np / 16; };
  pack(src->wg, d, 2 * d, 0, tiles(m->wg), m->wg);
  for (int l = 0; l < L; ++l) {
    const char *wq = static_cast<const char *>(src->wq) + l * dd;
    const char *wk = static_cast<const char *>(src->wk) + l * dd;
    const char *wv = static_cast<const char *>(src->wv) + l * dd;
    pack(wq, d, d, 0, d / 16, m->wqkv[l]);
    pack(wk, d, d, d / 16, 2 * d / 16, m->wqkv[l]);
    pack(wv, d, d, 2 * d / 16, tiles(m->wqkv[l]), m->wqkv[l]);
    pack(static_cast<const char *>(src->wo) + l * dd, d, d, 0, tiles(m->wo[l]), m->wo[l]);
    pack(static_cast<const char *>(src->wqc) + l * dd, d, d, 0, tiles(m->wqc[l]), m->wqc[l]);
    pack(static_cast<const char *>(src->woc) + l * dd, d, d, 0, tiles(m->woc[l]), m->woc[l]);
    pack(static_cast<const char *>(src->w1) + (size_t)l * F * d * es, F, d, 0, tiles(m->w1[l]),
         m->w1[l]);
    pack(static_cast<const char *>(src->w2) + (size_t)l * d * F * es, d, F, 0, tiles(m->w2[l]),
         m->w2[l]);
  }
  pack(src->wout, cfg->vocab, d, 0, tiles(m->wout), m->wout);
  if (e == hipSuccess) e = launch_copy(m->s_star, src->s_star, (size_t)d * 4, s);
  if (e == hipSuccess) e = launch_copy(m->bg, src->bg, (size_t)d * 4, s);
  if (e == hipSuccess) e = launch_copy(m->go, src->go, (size_t)d * 4, s);
  if (e == hipSuccess) e = launch_copy(m->g1, src->g1, (size_t)L * d * 4, s);
  if (e == hipSuccess) e = launch_copy(m->g2, src->g2, (size_t)L * d * 4, s);
  if (e == hipSuccess) e = launch_copy(m->g3, src->g3, (size_t)L * d * 4, s);
  if (e != hipSuccess) {
    delete m;
    return hip_fail(e, "packing weights");
  }
  *out = m;
  return ok();
}

void rlt_model_destroy(rlt_model *m) { delete m; }

size_t rlt_state_bytes(const rlt_config *cfg, int32_t batch, int32_t max_tokens) {
  if (check_config(cfg) != RLT_OK || batch < 1 || max_tokens < 1) return 0;
  rlt_state st;
  st.cfg = *cfg;
  return state_layout(*cfg, &st, nullptr, batch);
}

rlt_status rlt_state_init(const rlt_model *m, int32_t batch, int32_t max_tokens, void *dev_buf,
                          size_t bytes, void *stream, rlt_state **out) {
  if (!out) return fail(RLT_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  if (!m) return fail(RLT_ERR_INVALID_ARG, "model is NULL");
  if (batch < 1) return fail(RLT_ERR_INVALID_ARG, "batch must be >= 1");
  if (max_tokens < 1) return fail(RLT_ERR_INVALID_ARG, "max_tokens must be >= 1");
  if (!dev_buf) return fail(RLT_ERR_INVALID_ARG, "dev_buf is NULL");
  if ((uintptr_t)dev_buf % 256) return fail(RLT_ERR_SHAPE, "dev_buf must be 256-byte aligned");
  const size_t need = rlt_state_bytes(&m->cfg, batch, max_tokens);
  if (bytes < need) return fail(RLT_ERR_SHAPE, "state buffer %zu bytes < %zu required", bytes, need);
  rlt_status rs;
  if ((rs = device_health()) != RLT_OK) return rs;
  rlt_state *st = new rlt_state();
  st->cfg = m->cfg;
  st->version = m->version;
  st->device = m->device;
  st->B = batch;
  st->max_tokens = max_tokens;
  st->bytes = bytes;
  state_layout(m->cfg, st, dev_buf, batch);
  st->host_pos.assign(batch, 0);
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = launch_state_init(st->s, st->pos, m->s_star, batch, m->cfg.d_model, nullptr,
                                   batch, s);
  if (e != hipSuccess) {
    delete st;
    return hip_fail(e, "state init");
  }
  *out = st;
  return ok();
}

void rlt_state_destroy(rlt_state *st) {
  if (!st) return;
  prof_release(st->plog);
  delete st;
}

rlt_status rlt_state_reset(const rlt_model *m, rlt_state *st, int32_t n, const int32_t *host_slots,
                           void *stream) {
  rlt_status rs;
  if ((rs = check_state(m, st)) != RLT_OK) return rs;
  if (!host_slots) return fail(RLT_ERR_INVALID_ARG, "host_slots is NULL");
  if ((rs = check_slots(st, n, host_slots)) != RLT_OK) return rs;
  if ((rs = device_health()) != RLT_OK) return rs;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if ((rs = stage_slots(st, n, host_slots, s)) != RLT_OK) return rs;
  hipError_t e = launch_state_init(st->s, st->pos, m->s_star, st->B, m->cfg.d_model, st->slots_dev,
                                   n, s);
  if (e != hipSuccess) return hip_fail(e, "reset");
  for (int i = 0; i < n; ++i) st->host_pos[host_slots[i]] = 0;
  return ok();
}

rlt_status rlt_decoder_step(const rlt_model *m, rlt_state *st, int32_t n, const int32_t *host_slots,
                            const void *dev_e, const rlt_memory *mem, float *dev_logits,
                            void *stream) {
  rlt_status rs;
  if ((rs = check_state(m, st)) != RLT_OK) return rs;
  if ((rs = check_slots(st, n, host_slots)) != RLT_OK) return rs;
  if (!dev_e) return fail(RLT_ERR_INVALID_ARG, "dev_e is NULL");
  int max_slot = n - 1;
  if (host_slots) max_slot = *std::max_element(host_slots, host_slots + n);
  if ((rs = check_memory(m, mem, max_slot)) != RLT_OK) return rs;
  if ((rs = check_positions(st, mem, n, host_slots, 1)) != RLT_OK) return rs;
  if ((rs = device_health()) != RLT_OK) return rs;
  hipStream_t s = static_cast<hipStream_t>(stream);
  bool identity = true;
  if (host_slots)
    for (int i = 0; i < n; ++i) identity = identity && host_slots[i] == i;
  if (!identity && (rs = stage_slots(st, n, host_slots, s)) != RLT_OK) return rs;
  if ((rs = enqueue_step(m, st, state_scratch(st), n, identity, host_slots, dev_e,
                         m->cfg.d_model, mem, dev_logits, m->cfg.vocab, s)) != RLT_OK)
    return rs;
  return ok();
}

rlt_status rlt_decoder_step_noalloc(const rlt_model *m, rlt_state *st, int32_t n,
                                    const int32_t *host_slots, const void *dev_e,
                                    const rlt_memory *mem, float *dev_logits, void *stream) {
  rlt_status rs;
  if ((rs = check_state(m, st)) != RLT_OK) return rs;
  if ((rs = check_slots(st, n, host_slots)) != RLT_OK) return rs;
  if (!dev_e) return fail(RLT_ERR_INVALID_ARG, "dev_e is NULL");
  StepScratch w;
  const size_t need = step_scratch_layout(m->cfg, n, nullptr, &w);
  if (need > kStaticScratchBytes)
    return fail(RLT_ERR_RANGE,
                "a step of %d rows needs %zu bytes of working memory, more than the %zu bytes "
                "of the static scratch; split the call or use rlt_decoder_step",
                n, need, kStaticScratchBytes);
  int max_slot = n - 1;
  if (host_slots) max_slot = *std::max_element(host_slots, host_slots + n);
  if ((rs = check_memory(m, mem, max_slot)) != RLT_OK) return rs;
  if ((rs = check_positions(st, mem, n, host_slots, 1)) != RLT_OK) return rs;
  if ((rs = device_health()) != RLT_OK) return rs;
  void *base = nullptr;
  if ((rs = static_scratch(m->device, &base)) != RLT_OK) return rs;
  step_scratch_layout(m->cfg, n, base, &w);
  hipStream_t s = static_cast<hipStream_t>(stream);
  bool identity = true;
  if (host_slots)
    for (int i = 0; i < n; ++i) identity = identity && host_slots[i] == i;
  if (!identity) {
    // staged into the shared array on every call
    st->static_slots.assign(host_slots, host_slots + n);
    const hipError_t e = hipMemcpyAsync(w.slots_dev, st->static_slots.data(), (size_t)n * 4,
                                        hipMemcpyHostToDevice, s);
    if (e != hipSuccess) return hip_fail(e, "staging slot list");
  }
  if ((rs = enqueue_step(m, st, w, n, identity, host_slots, dev_e, m->cfg.d_model, mem,
                         dev_logits, m->cfg.vocab, s)) != RLT_OK)
    return rs;
  return ok();
}

rlt_status rlt_run_sequence(const rlt_model *m, rlt_state *st, int32_t T, const void *dev_e,
                            const rlt_memory *mem, float *dev_logits, int32_t logits_mode,
                            void *stream) {
  rlt_status rs;
  if ((rs = check_state(m, st)) != RLT_OK) return rs;
  if (T < 1) return fail(RLT_ERR_INVALID_ARG, "T must be >= 1");
  if (!dev_e) return fail(RLT_ERR_INVALID_ARG, "dev_e is NULL");
  if (logits_mode != RLT_LOGITS_ALL && logits_mode != RLT_LOGITS_LAST &&
      logits_mode != RLT_LOGITS_NONE)
    return fail(RLT_ERR_INVALID_ARG, "bad logits_mode");
  if (logits_mode != RLT_LOGITS_NONE && !dev_logits)
    return fail(RLT_ERR_INVALID_ARG, "dev_logits is NULL");
  if ((rs = check_memory(m, mem, st->B - 1)) != RLT_OK) return rs;
  if ((rs = check_positions(st, mem, st->B, nullptr, T)) != RLT_OK) return rs;
  if ((rs = device_health()) != RLT_OK) return rs;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int d = m->cfg.d_model, V = m->cfg.vocab, es = m->esize;
  for (int k = 0; k < T; ++k) {
    const void *ek = static_cast<const char *>(dev_e) + (size_t)k * d * es;
    float *lk = nullptr;
    int64_t ld = V;
    if (logits_mode == RLT_LOGITS_ALL) {
      lk = dev_logits + (size_t)k * V;
      ld = (int64_t)T * V;
    } else if (logits_mode == RLT_LOGITS_LAST && k == T - 1) {
      lk = dev_logits;
    }
    if ((rs = enqueue_step(m, st, state_scratch(st), st->B, true, nullptr, ek, (int64_t)T * d,
                           mem, lk, ld, s)) !=
        RLT_OK)
      return rs;
  }
  return ok();
}

int32_t rlt_fused_supported(const rlt_config *cfg) {
  if (!cfg || check_config(cfg) != RLT_OK || cfg->dtype != RLT_DTYPE_F32) return 0;
  if (cfg->n_layers > kFusedMaxLayers || cfg->n_heads * cfg->window > 256) return 0;
  return fused_lds_bytes(cfg->d_model, cfg->n_heads, cfg->head_dim, cfg->n_layers, cfg->d_ffn,
                         cfg->vocab, cfg->window, 0) <= kFusedMaxLds;
}

rlt_status rlt_run_sequence_fused(const rlt_model *m, rlt_state *st, int32_t T, const void *dev_e,
                                  const rlt_memory *mem, float *dev_logits, int32_t logits_mode,
                                  void *stream) {
  rlt_status rs;
  if ((rs = check_state(m, st)) != RLT_OK) return rs;
  if (!rlt_fused_supported(&m->cfg))
    return fail(RLT_ERR_UNSUPPORTED,
                "the fused run takes fp32 models of at most %d layers with heads x window <= 256 "
                "whose weights fit in %zu bytes of LDS", kFusedMaxLayers, kFusedMaxLds);
  if (T < 1) return fail(RLT_ERR_INVALID_ARG, "T must be >= 1");
  if (!dev_e) return fail(RLT_ERR_INVALID_ARG, "dev_e is NULL");
  if (logits_mode != RLT_LOGITS_ALL && logits_mode != RLT_LOGITS_LAST &&
      logits_mode != RLT_LOGITS_NONE)
    return fail(RLT_ERR_INVALID_ARG, "bad logits_mode");
  if (logits_mode != RLT_LOGITS_NONE && !dev_logits)
    return fail(RLT_ERR_INVALID_ARG, "dev_logits is NULL");
  if ((rs = check_memory(m, mem, st->B - 1)) != RLT_OK) return rs;
  if ((rs = check_positions(st, mem, st->B, nullptr, T)) != RLT_OK) return rs;
  if ((rs = device_health()) != RLT_OK) return rs;
  const rlt_config &c = m->cfg;
  FusedArgs a;
  memset(&a, 0, sizeof a);
  a.d = c.d_model;
  a.H = c.n_heads;
  a.dh = c.head_dim;
  a.L = c.n_layers;
  a.F = c.d_ffn;
  a.V = c.vocab;
  a.W = c.window;
  a.G = c.mem_groups;
  a.T = T;
  a.B = st->B;
  a.eps = c.rms_eps;
  a.scale = (float)(1.0 / sqrt((double)c.head_dim));
  a.wg = static_cast<const float *>(m->wg.p);
  a.bg = m->bg;
  a.wout = static_cast<const float *>(m->wout.p);
  a.go = m->go;
  for (int l = 0; l < c.n_layers; ++l) {
    a.wqkv[l] = static_cast<const float *>(m->wqkv[l].p);
    a.wo[l] = static_cast<const float *>(m->wo[l].p);
    a.wqc[l] = static_cast<const float *>(m->wqc[l].p);
    a.woc[l] = static_cast<const float *>(m->woc[l].p);
    a.w1[l] = static_cast<const float *>(m->w1[l].p);
    a.w2[l] = static_cast<const float *>(m->w2[l].p);
  }
  a.g1 = m->g1;
  a.g2 = m->g2;
  a.g3 = m->g3;
  a.s = st->s;
  a.pos = st->pos;
  a.ring_k = reinterpret_cast<float *>(st->ring_k);
  a.ring_v = reinterpret_cast<float *>(st->ring_v);
  a.e = static_cast<const float *>(dev_e);
  a.mk = static_cast<const float *>(mem->k);
  a.mv = static_cast<const float *>(mem->v);
  a.sg = mem->stride_group;
  a.ss = mem->stride_seq;
  a.sh = mem->stride_head;
  a.sp = mem->stride_pos;
  a.logits = dev_logits;
  a.logits_mode = logits_mode;
  // one shared memory group: the positions the call reads (through the
  // furthest slot's last one) stay in LDS for the whole call when they fit
  if (c.mem_groups == 1) {
    int last = 0;
    for (int i = 0; i < st->B; ++i) last = std::max(last, st->host_pos[i] + T);
    if (fused_lds_bytes(c.d_model, c.n_heads, c.head_dim, c.n_layers, c.d_ffn, c.vocab, c.window,
                        last) <= kFusedMaxLds)
      a.mres = last;
  }
  const hipError_t e = launch_fused_run(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "fused run launch");
  for (int i = 0; i < st->B; ++i) st->host_pos[i] += T;
  return ok();
}

size_t rlt_persistent_workspace_bytes(const rlt_config *cfg, int32_t n) {
  if (check_config(cfg) != RLT_OK || n < 1) return 0;
  StepBufs b;
  return step_layout(*cfg, n, nullptr, &b);
}

rlt_status rlt_run_sequence_persistent(const rlt_model *m, rlt_state *st, int32_t T,
                                       const void *dev_e, const rlt_memory *mem,
                                       float *dev_logits, int32_t logits_mode,
                                       void *dev_workspace, size_t workspace_bytes,
                                       void *stream) {
  rlt_status rs;
  if ((rs = check_state(m, st)) != RLT_OK) return rs;
  if (T < 1) return fail(RLT_ERR_INVALID_ARG, "T must be >= 1");
  if (!dev_e) return fail(RLT_ERR_INVALID_ARG, "dev_e is NULL");
  if (logits_mode != RLT_LOGITS_ALL && logits_mode != RLT_LOGITS_LAST &&
      logits_mode != RLT_LOGITS_NONE)
    return fail(RLT_ERR_INVALID_ARG, "bad logits_mode");
  if (logits_mode != RLT_LOGITS_NONE && !dev_logits)
    return fail(RLT_ERR_INVALID_ARG, "dev_logits is NULL");
  if (!dev_workspace) return fail(RLT_ERR_INVALID_ARG, "workspace is NULL");
  if ((uintptr_t)dev_workspace % 256) return fail(RLT_ERR_SHAPE, "workspace must be 256-byte aligned");
  const rlt_config &c = m->cfg;
  StepBufs b;
  const size_t need = step_layout(c, st->B, nullptr, &b);
  if (workspace_bytes < need)
    return fail(RLT_ERR_SHAPE, "workspace %zu bytes < %zu required", workspace_bytes, need);
  const int grid = step_grid(c.dtype, c.head_dim);
  if (grid < 8 || grid > kStepMaxGrid)
    return fail(RLT_ERR_UNSUPPORTED, "no persistent step for this dtype and head_dim %d",
                c.head_dim);
  if ((rs = check_memory(m, mem, st->B - 1)) != RLT_OK) return rs;
  if ((rs = check_positions(st, mem, st->B, nullptr, T)) != RLT_OK) return rs;
  if ((rs = device_health()) != RLT_OK) return rs;
  hipStream_t s = static_cast<hipStream_t>(stream);
  step_layout(c, st->B, dev_workspace, &b);
  // phase tables for steps without and with the head
  for (int t = 0; t < 2; ++t) {
    build_step_phases(m, st, mem, b, t == 1, st->step_tab[t]);
    hipError_t e = hipMemcpyAsync(b.tab[t], st->step_tab[t].data(),
                                  st->step_tab[t].size() * sizeof(StepPhase),
                                  hipMemcpyHostToDevice, s);
    if (e != hipSuccess) return hip_fail(e, "phase table upload");
  }
  // the error word and the item flags start at zero in every call; step k
  // of the call stores epoch k + 1
  if ((size_t)fl_count_check(st->step_tab[1]) != b.n_items)
    return fail(RLT_ERR_DEVICE, "item count mismatch in the persistent step tables");
  hipError_t e = launch_zero(b.err, (size_t)((char *)b.tab[0] - (char *)b.err), s);
  if (e != hipSuccess) return hip_fail(e, "item flag reset");
  const int d = c.d_model, V = c.vocab, es = m->esize;
  for (int k = 0; k < T; ++k) {
    StepRun r;
    r.e = static_cast<const char *>(dev_e) + (size_t)k * d * es;
    r.ld_e = (int64_t)T * d;
    r.logits = nullptr;
    r.ld_logits = V;
    if (logits_mode == RLT_LOGITS_ALL) {
      r.logits = dev_logits + (size_t)k * V;
      r.ld_logits = (int64_t)T * V;
    } else if (logits_mode == RLT_LOGITS_LAST && k == T - 1) {
      r.logits = dev_logits;
    }
    const int t = r.logits ? 1 : 0;
    r.ph = b.tab[t];
    r.n_phases = (int)st->step_tab[t].size();
    r.items = b.items;
    r.err = b.err;
    r.epoch = (unsigned)k + 1u;
    r.wait_epoch = r.epoch + (g_test_stall.load() ? 1u : 0u);
    e = launch_step(c.dtype, c.head_dim, r, grid, s);
    if (e != hipSuccess) return hip_fail(e, "persistent step launch");
  }
  for (int i = 0; i < st->B; ++i) st->host_pos[i] += T;
  return ok();
}

void rlt_persistent_test_stall(int32_t on) { g_test_stall.store(on ? 1 : 0); }

rlt_status rlt_persistent_check(void *dev_workspace, void *stream) {
  if (!dev_workspace) return fail(RLT_ERR_INVALID_ARG, "workspace is NULL");
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(e, "stream synchronize");
  // the error word opens the workspace
  const char *p = static_cast<const char *>(dev_workspace);
  unsigned err = 0;
  e = hipMemcpy(&err, p, 4, hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_fail(e, "reading the error word");
  if (err) return fail(RLT_ERR_DEVICE, "a wait of the persistent step timed out");
  return ok();
}

rlt_status rlt_score_sequence(const rlt_model *m, rlt_state *st, int32_t T, const void *dev_e,
                              const rlt_memory *mem, const int32_t *dev_tokens, float *dev_logprob,
                              void *stream) {
  rlt_status rs;
  if ((rs = check_state(m, st)) != RLT_OK) return rs;
  if (T < 1) return fail(RLT_ERR_INVALID_ARG, "T must be >= 1");
  if (!dev_e) return fail(RLT_ERR_INVALID_ARG, "dev_e is NULL");
  if (!dev_tokens) return fail(RLT_ERR_INVALID_ARG, "dev_tokens is NULL");
  if (!dev_logprob) return fail(RLT_ERR_INVALID_ARG, "dev_logprob is NULL");
  if ((rs = check_memory(m, mem, st->B - 1)) != RLT_OK) return rs;
  if ((rs = check_positions(st, mem, st->B, nullptr, T)) != RLT_OK) return rs;
  if ((rs = device_health()) != RLT_OK) return rs;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int d = m->cfg.d_model, V = m->cfg.vocab, es = m->esize;
  for (int k = 0; k < T; ++k) {
    // the step's logits go to the state's scratch; the score of the token
    // that step k+1 will consume is read from them before it is consumed
    const void *ek = static_cast<const char *>(dev_e) + (size_t)k * d * es;
    if ((rs = enqueue_step(m, st, state_scratch(st), st->B, true, nullptr, ek, (int64_t)T * d,
                           mem, st->lscratch, V,
                           s)) != RLT_OK)
      return rs;
    ScoreArgs sa;
    sa.logits = st->lscratch;
    sa.ld = V;
    sa.tokens = dev_tokens + k;
    sa.ld_tok = T;
    sa.out = dev_logprob + k;
    sa.ld_out = T;
    sa.V = V;
    Prof p(st->plog, RLT_K_EXTRA, s);
    const hipError_t e = launch_score(sa, st->B, s);
    if (e != hipSuccess) return hip_fail(e, "score launch");
    p.done((double)st->B * V * 4 * 2);
  }
  return ok();
}

rlt_status rlt_generate(const rlt_model *m, rlt_state *st, int32_t n_steps,
                        const float *dev_logits0, const rlt_encoder_table *enc,
                        const rlt_memory *mem, const rlt_sampling *smp, const float *dev_u,
                        int32_t *dev_tokens, float *dev_logprob, float *dev_logits_last,
                        void *stream) {
  rlt_status rs;
  if ((rs = check_state(m, st)) != RLT_OK) return rs;
  if (n_steps < 1) return fail(RLT_ERR_INVALID_ARG, "n_steps must be >= 1");
  if (!dev_logits0 || !enc || !enc->e || !enc->k || !enc->v || !smp || !dev_u || !dev_tokens ||
      !dev_logprob)
    return fail(RLT_ERR_INVALID_ARG, "a required pointer is NULL");
  if (!(smp->temperature > 0.f) || smp->top_k < 1)
    return fail(RLT_ERR_INVALID_ARG, "temperature must be > 0 and top_k >= 1");
  if ((rs = check_memory(m, mem, st->B - 1)) != RLT_OK) return rs;
  if ((rs = check_positions(st, mem, st->B, nullptr, n_steps)) != RLT_OK) return rs;
  if ((rs = device_health()) != RLT_OK) return rs;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const rlt_config &c = m->cfg;
  const int B = st->B, V = c.vocab, d = c.d_model;
  for (int j = 0; j < n_steps; ++j) {
    // 1-2: sample from the preceding state's logits, record token and log-prob
    SampleArgs sa;
    sa.logits = j == 0 ? dev_logits0 : st->lscratch;
    sa.ld = V;
    sa.u = dev_u + j;
    sa.ld_u = n_steps;
    sa.tokens = dev_tokens + j;
    sa.ld_tok = n_steps;
    sa.tokens2 = nullptr;
    sa.logprob = dev_logprob + j;
    sa.ld_lp = n_steps;
    sa.V = V;
    sa.top_k = std::min(smp->top_k, V);
    sa.inv_temp = 1.0f / smp->temperature;
    Prof ps(st->plog, RLT_K_EXTRA, s);
    hipError_t e = launch_sample(sa, B, s);
    if (e != hipSuccess) return hip_fail(e, "sample launch");
    ps.done((double)B * V * 4 * 2);
    // 3: stand-in encoder: e row and memory entry pos of every group
    EncodeArgs ea;
    ea.tokens = dev_tokens + j;
    ea.ld_tok = n_steps;
    ea.tab_e = enc->e;
    ea.tab_k = enc->k;
    ea.tab_v = enc->v;
    ea.e_out = st->escratch;
    ea.mem_k = const_cast<void *>(mem->k);
    ea.mem_v = const_cast<void *>(mem->v);
    ea.s_group = mem->stride_group;
    ea.s_seq = mem->stride_seq;
    ea.s_head = mem->stride_head;
    ea.s_pos = mem->stride_pos;
    ea.slots = nullptr;
    ea.pos = st->pos;
    ea.d = d;
    ea.H = c.n_heads;
    ea.dh = c.head_dim;
    ea.V = V;
    ea.G = c.mem_groups;
    Prof pe(st->plog, RLT_K_EXTRA, s);
    e = launch_encode(c.dtype, ea, B, s);
    if (e != hipSuccess) return hip_fail(e, "encode launch");
    pe.done((double)B * (d + 2.0 * c.mem_groups * d) * m->esize * 2);
    // 4: consume it once; the logits of the new state go to the scratch (and
    // to dev_logits_last on the last step)
    float *lg = (j == n_steps - 1 && dev_logits_last) ? dev_logits_last : st->lscratch;
    if ((rs = enqueue_step(m, st, state_scratch(st), B, true, nullptr, st->escratch, d, mem, lg,
                           V, s)) != RLT_OK)
      return rs;
  }
  return ok();
}

int32_t rlt_state_position(const rlt_state *st, int32_t slot) {
  if (!st || slot < 0 || slot >= st->B) return -1;
  return st->host_pos[slot];
}

size_t rlt_snapshot_bytes(const rlt_config *cfg, int32_t n) {
  if (check_config(cfg) != RLT_OK || n < 1) return 0;
  size_t a, b, c, rec;
  snapshot_offsets(cfg, &a, &b, &c, &rec);
  return rec * (size_t)n;
}

rlt_status rlt_state_export(const rlt_model *m, const rlt_state *st, int32_t n,
                            const int32_t *host_slots, void *dev_snap, void *stream) {
  rlt_status rs;
  if ((rs = check_state(m, st)) != RLT_OK) return rs;
  if (!host_slots) return fail(RLT_ERR_INVALID_ARG, "host_slots is NULL");
  if ((rs = check_slots(st, n, host_slots)) != RLT_OK) return rs;
  if (!dev_snap) return fail(RLT_ERR_INVALID_ARG, "dev_snap is NULL");
  if ((uintptr_t)dev_snap % 256) return fail(RLT_ERR_SHAPE, "dev_snap must be 256-byte aligned");
  if ((rs = device_health()) != RLT_OK) return rs;
  hipStream_t s = static_cast<hipStream_t>(stream);
  rlt_state *mst = const_cast<rlt_state *>(st);
  if ((rs = stage_slots(mst, n, host_slots, s)) != RLT_OK) return rs;
  SnapArgs a;
  memset(&a, 0, sizeof a);
  snapshot_offsets(&m->cfg, &a.off_s, &a.off_k, &a.off_v, &a.rec_bytes);
  a.snap = dev_snap;
  a.s = st->s;
  a.pos = st->pos;
  a.ring_k = st->ring_k;
  a.ring_v = st->ring_v;
  a.slots = st->slots_dev;
  a.n = n;
  a.B = st->B;
  a.L = m->cfg.n_layers;
  a.H = m->cfg.n_heads;
  a.W = m->cfg.window;
  a.dh = m->cfg.head_dim;
  a.d = m->cfg.d_model;
  a.dtype = m->cfg.dtype;
  a.version = m->version;
  hipError_t e = launch_export(a, s);
  if (e != hipSuccess) return hip_fail(e, "export");
  return ok();
}

rlt_status rlt_state_import(const rlt_model *m, rlt_state *st, int32_t n, const int32_t *host_slots,
                            const void *dev_snap, void *stream) {
  rlt_status rs;
  if ((rs = check_state(m, st)) != RLT_OK) return rs;
  if (!host_slots) return fail(RLT_ERR_INVALID_ARG, "host_slots is NULL");
  if ((rs = check_slots(st, n, host_slots)) != RLT_OK) return rs;
  if (!dev_snap) return fail(RLT_ERR_INVALID_ARG, "dev_snap is NULL");
  if ((uintptr_t)dev_snap % 256) return fail(RLT_ERR_SHAPE, "dev_snap must be 256-byte aligned");
  if ((rs = device_health()) != RLT_OK) return rs;
  hipStream_t s = static_cast<hipStream_t>(stream);
  SnapArgs a;
  memset(&a, 0, sizeof a);
  snapshot_offsets(&m->cfg, &a.off_s, &a.off_k, &a.off_v, &a.rec_bytes);
  // read the headers back and check them before touching the state
  std::vector<int> pos(n);
  for (int i = 0; i < n; ++i) {
    unsigned char hd[48];
    hipError_t e = hipMemcpyAsync(hd, static_cast<const char *>(dev_snap) + (size_t)i * a.rec_bytes,
                                  48, hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return hip_fail(e, "reading snapshot header");
    uint32_t magic, fmt;
    int32_t f[8];
    uint64_t ver;
    memcpy(&magic, hd, 4);
    memcpy(&fmt, hd + 4, 4);
    memcpy(f, hd + 8, 32);
    memcpy(&ver, hd + 40, 8);
    const rlt_config &c = m->cfg;
    if (magic != 0x534C5452u || fmt != 1u)
      return fail(RLT_ERR_CONVENTION, "record %d: not a snapshot record", i);
    if (f[0] != c.d_model || f[1] != c.n_heads || f[2] != c.head_dim || f[3] != c.n_layers)
      return fail(RLT_ERR_CONVENTION, "record %d: shape differs from the model", i);
    if (f[4] != c.window) return fail(RLT_ERR_CONVENTION, "record %d: window %d != %d", i, f[4], c.window);
    if (f[5] != c.dtype) return fail(RLT_ERR_CONVENTION, "record %d: dtype differs", i);
    if (ver != m->version)
      return fail(RLT_ERR_CONVENTION, "record %d: model version %llu != %llu", i,
                  (unsigned long long)ver, (unsigned long long)m->version);
    if (f[6] < 0 || f[6] > st->max_tokens)
      return fail(RLT_ERR_CONVENTION, "record %d: position %d outside [0, max_tokens]", i, f[6]);
    pos[i] = f[6];
  }
  if ((rs = stage_slots(st, n, host_slots, s)) != RLT_OK) return rs;
  a.csnap = dev_snap;
  a.s = st->s;
  a.pos = st->pos;
  a.ring_k = st->ring_k;
  a.ring_v = st->ring_v;
  a.slots = st->slots_dev;
  a.n = n;
  a.B = st->B;
  a.L = m->cfg.n_layers;
  a.H = m->cfg.n_heads;
  a.W = m->cfg.window;
  a.dh = m->cfg.head_dim;
  a.d = m->cfg.d_model;
  a.dtype = m->cfg.dtype;
  a.version = m->version;
  hipError_t e = launch_import(a, s);
  if (e != hipSuccess) return hip_fail(e, "import");
  for (int i = 0; i < n; ++i) st->host_pos[host_slots[i]] = pos[i];
  return ok();
}

rlt_status rlt_profile_begin(rlt_state *st, int32_t class_mask, int32_t max_launches,
                             int32_t step_stride) {
  if (!st) return fail(RLT_ERR_INVALID_ARG, "state is NULL");
  return prof_begin(st->plog, class_mask, RLT_K_NCLASSES, max_launches, step_stride);
}

rlt_status rlt_profile_collect(rlt_state *st, int32_t kclass, double *total_ms, int32_t *launches,
                               double *bytes_moved) {
  if (!st) return fail(RLT_ERR_INVALID_ARG, "state is NULL");
  if (kclass < 0 || kclass >= RLT_K_NCLASSES) return fail(RLT_ERR_INVALID_ARG, "bad kernel class");
  return prof_collect(st->plog, kclass, total_ms, launches, bytes_moved, nullptr);
}

}  // extern "C"

// ================================================================== encoder
// Host side of the token-parallel causal encoder: its own weights (embedding,
// final gain, memory projections), references to the decoder's tied layer
// weights, the encoder cache, and the launch sequence of one rlt_encode call.

struct rlt_encoder {
  const rlt_model *m;
  int device;
  char *emb;                       // [V][d] model dtype
  float *ge;                       // [d]
  std::vector<PackedMat> wkvm;     // per group: N = 2d (K rows, then V rows), K = d
};

struct rlt_encoder_state {
  rlt_config cfg;
  uint64_t version;
  int device;
  int B, max_tokens, max_rows;
  char *cache_k, *cache_v;         // [L][B][H][max_tokens][dh] model dtype
  int *slots_dev, *p0_dev;         // [B] slot and first position of each listed sequence
  int *pos_dev;                    // [B] position of every slot (fast one-token calls)
  float *x;                        // [R][d] residual stream
  char *abuf, *qbuf, *obuf, *hbuf, *ebuf;   // [R][d] / [R][F] model dtype
  float *split;                    // K-split partial tiles of the fast short-call GEMMs
  unsigned *split_cnt;             // parts finished per output tile (0 between launches)
  std::vector<int> host_pos;
  std::vector<int> tbl;            // host copy of the staged slot / position table
  std::vector<int> pos_tbl;        // host copy of the staged positions (fast calls)
  bool fast = false;               // RLT_ENC_FAST: short calls on the decoder's kernel forms
  ProfLog plog;
};

namespace {

bool encoder_supported(const rlt_config &c) {
  return !(c.dtype == RLT_DTYPE_BF16 && c.head_dim < 32);
}

size_t encoder_layout(const rlt_config &c, rlt_encoder *enc, void *base) {
  const int d = c.d_model, es = esize_of(c.dtype);
  Arena ar(base);
  enc->emb = ar.take<char>((size_t)c.vocab * d * es);
  enc->ge = ar.take<float>((size_t)d * 4);
  const GemmPlan g = gemm_plan(2 * d, d, c.dtype);
  enc->wkvm.resize(c.mem_groups);
  for (PackedMat &pm : enc->wkvm) {
    pm.N = g.N;
    pm.K = g.K;
    pm.Np = g.Np;
    pm.KT = g.KT;
    pm.p = ar.take<char>(packed_bytes(g, es, c.dtype));
  }
  return align256(ar.off);
}

size_t encoder_state_layout(const rlt_config &c, rlt_encoder_state *es, void *base, int B, int cap,
                            int R) {
  const int L = c.n_layers, d = c.d_model, H = c.n_heads, dh = c.head_dim;
  const int e = esize_of(c.dtype);
  Arena ar(base);
  es->cache_k = ar.take<char>((size_t)L * B * H * cap * dh * e);
  es->cache_v = ar.take<char>((size_t)L * B * H * cap * dh * e);
  es->slots_dev = ar.take<int>((size_t)B * 4);
  es->p0_dev = ar.take<int>((size_t)B * 4);
  es->pos_dev = ar.take<int>((size_t)B * 4);
  es->x = ar.take<float>((size_t)R * d * 4);
  es->abuf = ar.take<char>((size_t)R * d * e);
  es->qbuf = ar.take<char>((size_t)R * d * e);
  es->obuf = ar.take<char>((size_t)R * d * e);
  es->hbuf = ar.take<char>((size_t)R * c.d_ffn * e);
  es->ebuf = ar.take<char>((size_t)R * d * e);
  es->split = ar.take<float>(pgemm_split_bytes(std::max(3 * d, c.d_ffn)));
  es->split_cnt = ar.take<unsigned>(pgemm_split_counters(std::max(3 * d, c.d_ffn)) * 4);
  return align256(ar.off);
}

PGemmArgs pgemm_args(const PackedMat &w, const void *act, int64_t lda, const EncRows &rows) {
  PGemmArgs a{};
  a.a = act;
  a.lda = lda;
  a.wp = w.p;
  a.N = w.N;
  a.Np = w.Np;
  a.K = w.K;
  a.KT = w.KT;
  a.rows = rows;
  return a;
}

rlt_status enqueue_encode(const rlt_encoder *enc, rlt_encoder_state *es, const std::vector<int> &slots,
                          int T, const int32_t *dev_tokens, void *dev_e, const rlt_memory *mem,
                          hipStream_t s);

}  // namespace

extern "C" {

size_t rlt_encoder_bytes(const rlt_model *m) {
  if (!m || !encoder_supported(m->cfg)) return 0;
  rlt_encoder enc;
  return encoder_layout(m->cfg, &enc, nullptr);
}

rlt_status rlt_encoder_create(const rlt_model *m, const rlt_encoder_params *src, void *dev_buf,
                              size_t bytes, void *stream, rlt_encoder **out) {
  if (!out) return fail(RLT_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  if (!m) return fail(RLT_ERR_INVALID_ARG, "model is NULL");
  if (!src || !src->emb || !src->ge || !src->wkm || !src->wvm)
    return fail(RLT_ERR_INVALID_ARG, "an encoder parameter pointer is NULL");
  const rlt_config &c = m->cfg;
  if (!encoder_supported(c))
    return fail(RLT_ERR_UNSUPPORTED, "the bf16 encoder kernels need head_dim >= 32 (got %d)",
                c.head_dim);
  if (!dev_buf) return fail(RLT_ERR_INVALID_ARG, "dev_buf is NULL");
  if ((uintptr_t)dev_buf % 256) return fail(RLT_ERR_SHAPE, "dev_buf must be 256-byte aligned");
  const size_t need = rlt_encoder_bytes(m);
  if (bytes < need) return fail(RLT_ERR_SHAPE, "encoder buffer %zu bytes < %zu required", bytes, need);
  rlt_status rs;
  if ((rs = device_health()) != RLT_OK) return rs;
  rlt_encoder *enc = new rlt_encoder();
  enc->m = m;
  enc->device = m->device;
  encoder_layout(c, enc, dev_buf);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int d = c.d_model, es = esize_of(c.dtype);
  const size_t dd = (size_t)d * d * es;
  hipError_t e = launch_copy(enc->emb, src->emb, (size_t)c.vocab * d * es, s);
  if (e == hipSuccess) e = launch_copy(enc->ge, src->ge, (size_t)d * 4, s);
  for (int g = 0; g < c.mem_groups && e == hipSuccess; ++g) {
    const PackedMat &pm = enc->wkvm[g];
    e = launch_pack_tiles(static_cast<const char *>(src->wkm) + g * dd, d, d, d, 0, d / 16, pm,
                          c.dtype, s);
    if (e == hipSuccess)
      e = launch_pack_tiles(static_cast<const char *>(src->wvm) + g * dd, d, d, d, d / 16,
                            pm.Np / 16, pm, c.dtype, s);
  }
  if (e != hipSuccess) {
    delete enc;
    return hip_fail(e, "packing encoder weights");
  }
  *out = enc;
  return ok();
}

void rlt_encoder_destroy(rlt_encoder *enc) { delete enc; }

size_t rlt_encoder_state_bytes(const rlt_config *cfg, int32_t batch, int32_t max_tokens,
                               int32_t max_rows) {
  if (check_config(cfg) != RLT_OK || !encoder_supported(*cfg) || batch < 1 || max_tokens < 1 ||
      max_rows < 1)
    return 0;
  rlt_encoder_state es;
  return encoder_state_layout(*cfg, &es, nullptr, batch, max_tokens, max_rows);
}

rlt_status rlt_encoder_state_init(const rlt_encoder *enc, int32_t batch, int32_t max_tokens,
                                  int32_t max_rows, void *dev_buf, size_t bytes,
                                  rlt_encoder_state **out) {
  if (!out) return fail(RLT_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  if (!enc) return fail(RLT_ERR_INVALID_ARG, "encoder is NULL");
  if (batch < 1 || max_tokens < 1 || max_rows < 1)
    return fail(RLT_ERR_INVALID_ARG, "batch, max_tokens and max_rows must be >= 1");
  if (!dev_buf) return fail(RLT_ERR_INVALID_ARG, "dev_buf is NULL");
  if ((uintptr_t)dev_buf % 256) return fail(RLT_ERR_SHAPE, "dev_buf must be 256-byte aligned");
  const rlt_config &c = enc->m->cfg;
  const size_t need = rlt_encoder_state_bytes(&c, batch, max_tokens, max_rows);
  if (bytes < need)
    return fail(RLT_ERR_SHAPE, "encoder state buffer %zu bytes < %zu required", bytes, need);
  rlt_encoder_state *es = new rlt_encoder_state();
  es->cfg = c;
  es->version = enc->m->version;
  es->device = enc->device;
  es->B = batch;
  es->max_tokens = max_tokens;
  es->max_rows = max_rows;
  encoder_state_layout(c, es, dev_buf, batch, max_tokens, max_rows);
  es->host_pos.assign(batch, 0);
  // the fast short-call GEMMs' tile counters start at zero (and every launch
  // leaves them at zero)
  const hipError_t e = clear_now(es->split_cnt,
                                 pgemm_split_counters(std::max(3 * c.d_model, c.d_ffn)) * 4);
  if (e != hipSuccess) {
    delete es;
    return hip_fail(e, "clearing the encoder state's tile counters");
  }
  *out = es;
  return ok();
}

void rlt_encoder_state_destroy(rlt_encoder_state *es) {
  if (!es) return;
  prof_release(es->plog);
  delete es;
}

rlt_status rlt_encoder_state_reset(rlt_encoder_state *es, int32_t n, const int32_t *host_slots) {
  if (!es) return fail(RLT_ERR_INVALID_ARG, "encoder state is NULL");
  if (!host_slots) return fail(RLT_ERR_INVALID_ARG, "host_slots is NULL");
  if (n < 1 || n > es->B) return fail(RLT_ERR_INVALID_ARG, "n = %d outside [1, %d]", n, es->B);
  for (int i = 0; i < n; ++i)
    if (host_slots[i] < 0 || host_slots[i] >= es->B)
      return fail(RLT_ERR_INVALID_ARG, "slot %d out of range", host_slots[i]);
  for (int i = 0; i < n; ++i) es->host_pos[host_slots[i]] = 0;
  return ok();
}

rlt_status rlt_encoder_state_set_mode(rlt_encoder_state *es, int32_t mode) {
  if (!es) return fail(RLT_ERR_INVALID_ARG, "encoder state is NULL");
  if (mode != RLT_ENC_EXACT && mode != RLT_ENC_FAST)
    return fail(RLT_ERR_INVALID_ARG, "mode must be RLT_ENC_EXACT or RLT_ENC_FAST (got %d)", mode);
  if (mode == RLT_ENC_FAST) {
    // tile counters at zero (they are after every complete launch; this
    // re-arms them after a launch that did not complete)
    const hipError_t e = clear_now(es->split_cnt,
                                   pgemm_split_counters(std::max(3 * es->cfg.d_model, es->cfg.d_ffn)) * 4);
    if (e != hipSuccess) return hip_fail(e, "clearing the encoder state's tile counters");
  }
  es->fast = mode == RLT_ENC_FAST;
  return ok();
}

int32_t rlt_encoder_position(const rlt_encoder_state *es, int32_t slot) {
  if (!es || slot < 0 || slot >= es->B) return -1;
  return es->host_pos[slot];
}

rlt_status rlt_encode(const rlt_encoder *enc, rlt_encoder_state *es, int32_t n,
                      const int32_t *host_slots, int32_t T, const int32_t *dev_tokens, void *dev_e,
                      const rlt_memory *mem, void *stream) {
  if (!enc) return fail(RLT_ERR_INVALID_ARG, "encoder is NULL");
  if (!es) return fail(RLT_ERR_INVALID_ARG, "encoder state is NULL");
  const rlt_model *m = enc->m;
  const rlt_config &c = m->cfg;
  if (es->version != m->version)
    return fail(RLT_ERR_STALE, "encoder state built for model version %llu, model is version %llu",
                (unsigned long long)es->version, (unsigned long long)m->version);
  if (n < 1 || n > es->B) return fail(RLT_ERR_INVALID_ARG, "n = %d outside [1, %d]", n, es->B);
  if (T < 1) return fail(RLT_ERR_INVALID_ARG, "T must be >= 1");
  if ((long long)n * T > es->max_rows)
    return fail(RLT_ERR_SHAPE, "n * T = %lld rows > max_rows %d", (long long)n * T, es->max_rows);
  if (!dev_tokens) return fail(RLT_ERR_INVALID_ARG, "dev_tokens is NULL");
  std::vector<int> slots(n);
  std::vector<char> seen(es->B, 0);
  int max_slot = 0;
  for (int i = 0; i < n; ++i) {
    const int sl = host_slots ? host_slots[i] : i;
    if (sl < 0 || sl >= es->B) return fail(RLT_ERR_INVALID_ARG, "slot %d out of range", sl);
    if (seen[sl]) return fail(RLT_ERR_INVALID_ARG, "slot %d listed twice", sl);
    seen[sl] = 1;
    slots[i] = sl;
    max_slot = std::max(max_slot, sl);
  }
  rlt_status rs;
  if ((rs = check_memory(m, mem, max_slot)) != RLT_OK) return rs;
  for (int i = 0; i < n; ++i) {
    const long long last = (long long)es->host_pos[slots[i]] + T;
    if (last > mem->capacity)
      return fail(RLT_ERR_RANGE, "slot %d would reach position %lld > memory capacity %d",
                  slots[i], last, mem->capacity);
    if (last > es->max_tokens)
      return fail(RLT_ERR_RANGE, "slot %d would reach position %lld > max_tokens %d", slots[i],
                  last, es->max_tokens);
  }
  if ((uintptr_t)dev_e % 16) return fail(RLT_ERR_SHAPE, "dev_e must be 16-byte aligned");
  if ((rs = device_health()) != RLT_OK) return rs;
  return enqueue_encode(enc, es, slots, T, dev_tokens, dev_e, mem, static_cast<hipStream_t>(stream));
}

}  // extern "C"

namespace {
// The device work of rlt_encode for validated arguments: the listed slots'
// next T tokens (dev_tokens [n][T]), e rows to dev_e (null: the state's
// scratch), memory entries written, positions advanced.
rlt_status enqueue_encode(const rlt_encoder *enc, rlt_encoder_state *es, const std::vector<int> &slots,
                          int T, const int32_t *dev_tokens, void *dev_e, const rlt_memory *mem,
                          hipStream_t s) {
  rlt_status rs;
  const rlt_model *m = enc->m;
  const rlt_config &c = m->cfg;
  const int n = (int)slots.size();
  const int L = c.n_layers, d = c.d_model, F = c.d_ffn, H = c.n_heads, dh = c.head_dim;
  const int esz = esize_of(c.dtype);
  const int R = n * T;
  // slot / first-position table of this call (host copy kept until the next call)
  es->tbl.resize(2 * (size_t)n);
  double attn_pairs = 0.0;     // sum over rows of the attended positions
  double kv_positions = 0.0;   // cache positions each sequence's attention reads
  for (int i = 0; i < n; ++i) {
    es->tbl[i] = slots[i];
    es->tbl[n + i] = es->host_pos[slots[i]];
    attn_pairs += (double)T * es->tbl[n + i] + 0.5 * (double)T * (T + 1);
    kv_positions += (double)es->tbl[n + i] + T;
  }
  hipError_t e = hipMemcpyAsync(es->slots_dev, es->tbl.data(), (size_t)n * 4, hipMemcpyHostToDevice, s);
  if (e == hipSuccess)
    e = hipMemcpyAsync(es->p0_dev, es->tbl.data() + n, (size_t)n * 4, hipMemcpyHostToDevice, s);
  // fast one-token calls: the positions of all slots, indexed by slot
  const bool fast_attn = es->fast && T == 1;
  if (e == hipSuccess && fast_attn) {
    es->pos_tbl = es->host_pos;
    e = hipMemcpyAsync(es->pos_dev, es->pos_tbl.data(), (size_t)es->B * 4, hipMemcpyHostToDevice, s);
  }
  if (e != hipSuccess) return hip_fail(e, "staging the slot table");
  const EncRows rows{es->slots_dev, es->p0_dev, T, R};

  auto gemm = [&](const PGemmArgs &a, int epi, const char *what) -> rlt_status {
    Prof p(es->plog, RLT_E_GEMM, s);
    PGemmArgs b = a;
    b.split = es->split;
    b.split_cnt = es->split_cnt;
    const hipError_t err = es->fast ? launch_pgemm_fast(c.dtype, epi, b, s) : launch_pgemm(c.dtype, epi, a, s);
    const double flops = 2.0 * R * a.N * a.K;
    const double out_bytes = epi == PEPI_RESID ? (double)R * a.N * 8 : (double)R * a.N * esz;
    p.done((double)a.N * a.K * esz + (double)R * a.K * esz + out_bytes, flops);
    return err == hipSuccess ? RLT_OK : hip_fail(err, what);
  };
  auto other = [&](hipError_t err, const char *what) -> rlt_status {
    return err == hipSuccess ? RLT_OK : hip_fail(err, what);
  };
  const size_t layer_cache = (size_t)es->B * H * es->max_tokens * dh * esz;
  const int64_t s_seq = (int64_t)H * es->max_tokens * dh, s_head = (int64_t)es->max_tokens * dh;

  {
    Prof p(es->plog, RLT_E_OTHER, s);
    e = launch_enc_embed(c.dtype, dev_tokens, R, enc->emb, c.vocab, d, es->x, s);
    p.done((double)R * 4 + (double)R * d * (esz + 4));
    if ((rs = other(e, "embedding")) != RLT_OK) return rs;
  }
  auto norm = [&](const float *gamma, void *out) -> rlt_status {
    Prof p(es->plog, RLT_E_OTHER, s);
    const hipError_t err = launch_enc_norm(c.dtype, es->x, d, gamma, c.rms_eps, out, d, R, d, s);
    p.done((double)R * d * (4 + esz) + (double)d * 4);
    return other(err, "rmsnorm");
  };
  for (int l = 0; l < L; ++l) {
    char *ck = es->cache_k + l * layer_cache, *cv = es->cache_v + l * layer_cache;
    if ((rs = norm(m->g1 + (size_t)l * d, es->abuf)) != RLT_OK) return rs;
    PGemmArgs a = pgemm_args(m->wqkv[l], es->abuf, d, rows);
    a.out = es->qbuf;
    a.ld_out = d;
    a.kb = ck;
    a.vb = cv;
    a.s_seq = s_seq;
    a.s_head = s_head;
    a.s_pos = dh;
    a.d = d;
    a.H = H;
    a.dh = dh;
    if ((rs = gemm(a, PEPI_QKV, "qkv gemm")) != RLT_OK) return rs;
    if (fast_attn) {
      // the decoder's attention over the encoder cache as memory: position
      // p of a slot attends to cache positions 0..p (entry p written above)
      AttnArgs at{};
      at.q = es->qbuf;
      at.out = es->obuf;
      at.kb = ck;
      at.vb = cv;
      at.s_seq = s_seq;
      at.s_head = s_head;
      at.s_pos = dh;
      at.len_cap = 0x7fffffff;
      at.ch = m->chunk;
      at.slots = es->slots_dev;
      at.pos = es->pos_dev;
      at.H = H;
      at.d = d;
      at.scale_log2 = (float)(1.4426950408889634 / sqrt((double)dh));
      Prof p(es->plog, RLT_E_ATTN, s);
      e = launch_attn_rows(c.dtype, dh, at, n, s);
      p.done(2.0 * R * d * esz + 2.0 * kv_positions * d * esz, 4.0 * attn_pairs * d);
      if ((rs = other(e, "attention (fast one-token form)")) != RLT_OK) return rs;
    } else {
      FAttnArgs fa{};
      fa.q = es->qbuf;
      fa.ldq = d;
      fa.out = es->obuf;
      fa.ldo = d;
      fa.kb = ck;
      fa.vb = cv;
      fa.s_seq = s_seq;
      fa.s_head = s_head;
      fa.s_pos = dh;
      fa.rows = rows;
      fa.H = H;
      fa.scale_log2 = (float)(1.4426950408889634 / sqrt((double)dh));
      Prof p(es->plog, RLT_E_ATTN, s);
      e = launch_fattn(c.dtype, dh, fa, s);
      p.done(2.0 * R * d * esz + 2.0 * kv_positions * d * esz, 4.0 * attn_pairs * d);
      if ((rs = other(e, "causal attention")) != RLT_OK) return rs;
    }
    a = pgemm_args(m->wo[l], es->obuf, d, rows);
    a.x = es->x;
    a.ld_x = d;
    if ((rs = gemm(a, PEPI_RESID, "o gemm")) != RLT_OK) return rs;
    if ((rs = norm(m->g3 + (size_t)l * d, es->abuf)) != RLT_OK) return rs;
    a = pgemm_args(m->w1[l], es->abuf, d, rows);
    a.out = es->hbuf;
    a.ld_out = F;
    if ((rs = gemm(a, PEPI_GELU, "ffn-up gemm")) != RLT_OK) return rs;
    a = pgemm_args(m->w2[l], es->hbuf, F, rows);
    a.x = es->x;
    a.ld_x = d;
    if ((rs = gemm(a, PEPI_RESID, "ffn-down gemm")) != RLT_OK) return rs;
  }
  void *e_out = dev_e ? dev_e : es->ebuf;
  if ((rs = norm(enc->ge, e_out)) != RLT_OK) return rs;
  for (int g = 0; g < c.mem_groups; ++g) {
    PGemmArgs a = pgemm_args(enc->wkvm[g], e_out, d, rows);
    a.kb = static_cast<char *>(const_cast<void *>(mem->k)) + (size_t)g * mem->stride_group * esz;
    a.vb = static_cast<char *>(const_cast<void *>(mem->v)) + (size_t)g * mem->stride_group * esz;
    a.s_seq = mem->stride_seq;
    a.s_head = mem->stride_head;
    a.s_pos = mem->stride_pos;
    a.d = d;
    a.H = H;
    a.dh = dh;
    if ((rs = gemm(a, PEPI_MEM, "memory projection gemm")) != RLT_OK) return rs;
  }
  for (int i = 0; i < n; ++i) es->host_pos[slots[i]] += T;
  es->plog.step_counter += 1;
  return ok();
}

}  // namespace

extern "C" {

rlt_status rlt_encoder_profile_begin(rlt_encoder_state *es, int32_t class_mask,
                                     int32_t max_launches) {
  if (!es) return fail(RLT_ERR_INVALID_ARG, "encoder state is NULL");
  return prof_begin(es->plog, class_mask, RLT_E_NCLASSES, max_launches, 1);
}

rlt_status rlt_encoder_profile_collect(rlt_encoder_state *es, int32_t kclass, double *total_ms,
                                       int32_t *launches, double *flops, double *bytes_moved) {
  if (!es) return fail(RLT_ERR_INVALID_ARG, "encoder state is NULL");
  if (kclass < 0 || kclass >= RLT_E_NCLASSES) return fail(RLT_ERR_INVALID_ARG, "bad kernel class");
  return prof_collect(es->plog, kclass, total_ms, launches, bytes_moved, flops);
}

size_t rlt_encoder_snapshot_bytes(const rlt_config *cfg, int32_t capacity, int32_t n) {
  if (check_config(cfg) != RLT_OK || capacity < 0 || n < 1) return 0;
  const size_t sec = align256((size_t)cfg->n_layers * cfg->n_heads * capacity * cfg->head_dim *
                              esize_of(cfg->dtype));
  return (256 + 2 * sec) * (size_t)n;
}

}  // extern "C"

namespace {
constexpr uint32_t kEncSnapMagic = 0x454C5452u;   // encoder-cache record

// slot list checks shared by the encoder snapshot calls; the slots and the
// given positions are staged in es's table
rlt_status enc_snap_stage(rlt_encoder_state *es, int n, const int32_t *host_slots,
                          const std::vector<int> &pos, hipStream_t s) {
  if (n < 1 || n > es->B) return fail(RLT_ERR_INVALID_ARG, "n = %d outside [1, %d]", n, es->B);
  std::vector<char> seen(es->B, 0);
  es->tbl.resize(2 * (size_t)n);
  for (int i = 0; i < n; ++i) {
    const int sl = host_slots[i];
    if (sl < 0 || sl >= es->B) return fail(RLT_ERR_INVALID_ARG, "slot %d out of range", sl);
    if (seen[sl]) return fail(RLT_ERR_INVALID_ARG, "slot %d listed twice", sl);
    seen[sl] = 1;
    es->tbl[i] = sl;
    es->tbl[n + i] = pos[i];
  }
  hipError_t e = hipMemcpyAsync(es->slots_dev, es->tbl.data(), (size_t)n * 4, hipMemcpyHostToDevice, s);
  if (e == hipSuccess)
    e = hipMemcpyAsync(es->p0_dev, es->tbl.data() + n, (size_t)n * 4, hipMemcpyHostToDevice, s);
  return e == hipSuccess ? RLT_OK : hip_fail(e, "staging the snapshot table");
}

EncSnapArgs enc_snap_args(const rlt_encoder *enc, const rlt_encoder_state *es, int n, int cap) {
  const rlt_config &c = enc->m->cfg;
  EncSnapArgs a;
  memset(&a, 0, sizeof a);
  a.rec_bytes = rlt_encoder_snapshot_bytes(&c, cap, 1);
  a.off_k = 256;
  a.off_v = 256 + (a.rec_bytes - 256) / 2;
  a.cache_k = es->cache_k;
  a.cache_v = es->cache_v;
  a.slots = es->slots_dev;
  a.pos = es->p0_dev;
  a.n = n;
  a.B = es->B;
  a.L = c.n_layers;
  a.H = c.n_heads;
  a.dh = c.head_dim;
  a.max_tokens = es->max_tokens;
  a.cap = cap;
  a.esize = esize_of(c.dtype);
  return a;
}
}  // namespace

extern "C" {

rlt_status rlt_encoder_state_export(const rlt_encoder *enc, rlt_encoder_state *es, int32_t n,
                                    const int32_t *host_slots, int32_t capacity, void *dev_snap,
                                    void *stream) {
  if (!enc || !es) return fail(RLT_ERR_INVALID_ARG, "encoder or encoder state is NULL");
  if (!host_slots || !dev_snap) return fail(RLT_ERR_INVALID_ARG, "host_slots or dev_snap is NULL");
  if ((uintptr_t)dev_snap % 256) return fail(RLT_ERR_SHAPE, "dev_snap must be 256-byte aligned");
  if (es->version != enc->m->version)
    return fail(RLT_ERR_STALE, "encoder state built for model version %llu, model is version %llu",
                (unsigned long long)es->version, (unsigned long long)enc->m->version);
  if (capacity < 0) return fail(RLT_ERR_INVALID_ARG, "capacity must be >= 0");
  if (n < 1 || n > es->B) return fail(RLT_ERR_INVALID_ARG, "n = %d outside [1, %d]", n, es->B);
  std::vector<int> pos(n);
  for (int i = 0; i < n; ++i) {
    if (host_slots[i] < 0 || host_slots[i] >= es->B)
      return fail(RLT_ERR_INVALID_ARG, "slot %d out of range", host_slots[i]);
    pos[i] = es->host_pos[host_slots[i]];
    if (pos[i] > capacity)
      return fail(RLT_ERR_RANGE, "slot %d holds %d positions > capacity %d", host_slots[i], pos[i],
                  capacity);
  }
  rlt_status rs;
  if ((rs = device_health()) != RLT_OK) return rs;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if ((rs = enc_snap_stage(es, n, host_slots, pos, s)) != RLT_OK) return rs;
  EncSnapArgs a = enc_snap_args(enc, es, n, capacity);
  const rlt_config &c = enc->m->cfg;
  a.snap = dev_snap;
  const uint32_t hdr[12] = {kEncSnapMagic, 1u, (uint32_t)c.d_model, (uint32_t)c.n_heads,
                            (uint32_t)c.head_dim, (uint32_t)c.n_layers, (uint32_t)c.dtype, 0u,
                            (uint32_t)capacity, 0u, (uint32_t)(enc->m->version & 0xffffffffu),
                            (uint32_t)(enc->m->version >> 32)};
  memcpy(a.hdr, hdr, sizeof hdr);
  const hipError_t e = launch_enc_snap(a, true, s);
  if (e != hipSuccess) return hip_fail(e, "encoder snapshot export");
  return ok();
}

rlt_status rlt_encoder_state_import(const rlt_encoder *enc, rlt_encoder_state *es, int32_t n,
                                    const int32_t *host_slots, int32_t capacity,
                                    const void *dev_snap, void *stream) {
  if (!enc || !es) return fail(RLT_ERR_INVALID_ARG, "encoder or encoder state is NULL");
  if (!host_slots || !dev_snap) return fail(RLT_ERR_INVALID_ARG, "host_slots or dev_snap is NULL");
  if ((uintptr_t)dev_snap % 256) return fail(RLT_ERR_SHAPE, "dev_snap must be 256-byte aligned");
  if (es->version != enc->m->version)
    return fail(RLT_ERR_STALE, "encoder state built for model version %llu, model is version %llu",
                (unsigned long long)es->version, (unsigned long long)enc->m->version);
  if (capacity < 0) return fail(RLT_ERR_INVALID_ARG, "capacity must be >= 0");
  if (n < 1 || n > es->B) return fail(RLT_ERR_INVALID_ARG, "n = %d outside [1, %d]", n, es->B);
  rlt_status rs;
  if ((rs = device_health()) != RLT_OK) return rs;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const rlt_config &c = enc->m->cfg;
  const size_t rec = rlt_encoder_snapshot_bytes(&c, capacity, 1);
  // read the headers back and check them before touching the state
  std::vector<uint32_t> hd((size_t)n * 12);
  for (int i = 0; i < n; ++i) {
    hipError_t e = hipMemcpyAsync(hd.data() + (size_t)i * 12,
                                  static_cast<const char *>(dev_snap) + (size_t)i * rec, 48,
                                  hipMemcpyDeviceToHost, s);
    if (e != hipSuccess) return hip_fail(e, "reading encoder snapshot headers");
  }
  hipError_t e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(e, "reading encoder snapshot headers");
  std::vector<int> pos(n);
  for (int i = 0; i < n; ++i) {
    const uint32_t *f = hd.data() + (size_t)i * 12;
    const uint64_t ver = (uint64_t)f[10] | ((uint64_t)f[11] << 32);
    if (f[0] != kEncSnapMagic || f[1] != 1u)
      return fail(RLT_ERR_CONVENTION, "record %d: not an encoder snapshot record", i);
    if ((int)f[2] != c.d_model || (int)f[3] != c.n_heads || (int)f[4] != c.head_dim ||
        (int)f[5] != c.n_layers || (int)f[6] != c.dtype)
      return fail(RLT_ERR_CONVENTION, "record %d: shape or dtype differs from the model", i);
    if ((int)f[8] != capacity)
      return fail(RLT_ERR_CONVENTION, "record %d: capacity %u != %d", i, f[8], capacity);
    if (ver != enc->m->version)
      return fail(RLT_ERR_CONVENTION, "record %d: model version %llu != %llu", i,
                  (unsigned long long)ver, (unsigned long long)enc->m->version);
    pos[i] = (int)f[7];
    if (pos[i] < 0 || pos[i] > capacity || pos[i] > es->max_tokens)
      return fail(RLT_ERR_CONVENTION, "record %d: position %d outside [0, min(capacity, max_tokens)]",
                  i, pos[i]);
  }
  if ((rs = enc_snap_stage(es, n, host_slots, pos, s)) != RLT_OK) return rs;
  EncSnapArgs a = enc_snap_args(enc, es, n, capacity);
  a.csnap = dev_snap;
  e = launch_enc_snap(a, false, s);
  if (e != hipSuccess) return hip_fail(e, "encoder snapshot import");
  for (int i = 0; i < n; ++i) es->host_pos[host_slots[i]] = pos[i];
  return ok();
}

rlt_status rlt_generate_encoded(const rlt_model *m, rlt_state *st, int32_t n_steps,
                                const float *dev_logits0, const rlt_encoder *enc,
                                rlt_encoder_state *es, const rlt_memory *mem,
                                const rlt_sampling *smp, const float *dev_u, int32_t *dev_tokens,
                                float *dev_logprob, float *dev_logits_last, void *stream) {
  rlt_status rs;
  if ((rs = check_state(m, st)) != RLT_OK) return rs;
  if (n_steps < 1) return fail(RLT_ERR_INVALID_ARG, "n_steps must be >= 1");
  if (!dev_logits0 || !enc || !es || !smp || !dev_u || !dev_tokens || !dev_logprob)
    return fail(RLT_ERR_INVALID_ARG, "a required pointer is NULL");
  if (enc->m != m) return fail(RLT_ERR_INVALID_ARG, "the encoder belongs to another model");
  if (es->version != m->version)
    return fail(RLT_ERR_STALE, "encoder state built for model version %llu, model is version %llu",
                (unsigned long long)es->version, (unsigned long long)m->version);
  if (!(smp->temperature > 0.f) || smp->top_k < 1)
    return fail(RLT_ERR_INVALID_ARG, "temperature must be > 0 and top_k >= 1");
  const int B = st->B;
  if (es->B < B) return fail(RLT_ERR_SHAPE, "encoder state has %d slots < %d", es->B, B);
  if (es->max_rows < B)
    return fail(RLT_ERR_SHAPE, "encoder state max_rows %d < %d slots", es->max_rows, B);
  for (int b = 0; b < B; ++b) {
    // the token sampled after position p is encoded at encoder position p
    if (es->host_pos[b] != st->host_pos[b])
      return fail(RLT_ERR_RANGE, "slot %d: %d tokens encoded but %d consumed", b, es->host_pos[b],
                  st->host_pos[b]);
    if ((long long)es->host_pos[b] + n_steps > es->max_tokens)
      return fail(RLT_ERR_RANGE, "slot %d would pass the encoder's max_tokens %d", b, es->max_tokens);
  }
  if ((rs = check_memory(m, mem, B - 1)) != RLT_OK) return rs;
  if ((rs = check_positions(st, mem, B, nullptr, n_steps)) != RLT_OK) return rs;
  if ((rs = device_health()) != RLT_OK) return rs;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const rlt_config &c = m->cfg;
  const int V = c.vocab, d = c.d_model;
  std::vector<int> slots(B);
  for (int b = 0; b < B; ++b) slots[b] = b;
  for (int j = 0; j < n_steps; ++j) {
    // 1-2: sample from the preceding state's logits, record token and log-prob
    SampleArgs sa;
    sa.logits = j == 0 ? dev_logits0 : st->lscratch;
    sa.ld = V;
    sa.u = dev_u + j;
    sa.ld_u = n_steps;
    sa.tokens = dev_tokens + j;
    sa.ld_tok = n_steps;
    sa.tokens2 = st->tok_dev;
    sa.logprob = dev_logprob + j;
    sa.ld_lp = n_steps;
    sa.V = V;
    sa.top_k = std::min(smp->top_k, V);
    sa.inv_temp = 1.0f / smp->temperature;
    Prof ps(st->plog, RLT_K_EXTRA, s);
    hipError_t e = launch_sample(sa, B, s);
    if (e != hipSuccess) return hip_fail(e, "sample launch");
    ps.done((double)B * V * 4 * 2);
    // 3: the causal encoder over the new token of every slot (its cache holds
    // the earlier ones): e row to the state's scratch, memory entries written
    if ((rs = enqueue_encode(enc, es, slots, 1, st->tok_dev, st->escratch, mem, s)) != RLT_OK)
      return rs;
    // 4: consume it once
    float *lg = (j == n_steps - 1 && dev_logits_last) ? dev_logits_last : st->lscratch;
    if ((rs = enqueue_step(m, st, state_scratch(st), B, true, nullptr, st->escratch, d, mem, lg,
                           V, s)) != RLT_OK)
      return rs;
  }
  return ok();
}

}  // extern "C"

// ================================================================== training
extern "C" {

size_t rlt_bptt_workspace_bytes_segmented(const rlt_config *cfg, int32_t batch, int32_t T,
                                          int32_t segment) {
  if (check_config(cfg) != RLT_OK || cfg->dtype != RLT_DTYPE_F32 || batch < 1 || T < 1 ||
      T > kTrainMaxPos || segment < 0)
    return 0;
  return train_workspace_bytes(*cfg, batch, T, segment);
}

size_t rlt_bptt_workspace_bytes(const rlt_config *cfg, int32_t batch, int32_t T) {
  return rlt_bptt_workspace_bytes_segmented(cfg, batch, T, 0);
}

rlt_status rlt_bptt(const rlt_config *cfg, const rlt_params *params, int32_t batch, int32_t T,
                    const float *dev_e, const rlt_memory *mem, const int32_t *dev_targets,
                    const rlt_bptt_opts *opts, const rlt_params *grads, float *dev_de,
                    const rlt_memory *dmem, float *dev_loss, void *dev_workspace,
                    size_t workspace_bytes, void *stream) {
  rlt_status rs;
  if ((rs = check_config(cfg)) != RLT_OK) return rs;
  if (cfg->dtype != RLT_DTYPE_F32)
    return fail(RLT_ERR_UNSUPPORTED, "backpropagation through time is implemented for fp32 models");
  if (!params || !grads) return fail(RLT_ERR_INVALID_ARG, "params or grads is NULL");
  const void *need[] = {params->s_star, params->wg, params->bg, params->g1, params->g2, params->g3,
                        params->wq, params->wk, params->wv, params->wo, params->wqc, params->woc,
                        params->w1, params->w2, params->go, params->wout,
                        grads->s_star, grads->wg, grads->bg, grads->g1, grads->g2, grads->g3,
                        grads->wq, grads->wk, grads->wv, grads->wo, grads->wqc, grads->woc,
                        grads->w1, grads->w2, grads->go, grads->wout};
  for (const void *p : need)
    if (!p) return fail(RLT_ERR_INVALID_ARG, "a parameter or gradient pointer is NULL");
  if (batch < 1 || T < 1) return fail(RLT_ERR_INVALID_ARG, "batch and T must be >= 1");
  if (T > kTrainMaxPos)
    return fail(RLT_ERR_UNSUPPORTED, "T = %d > %d positions per attention row", T, kTrainMaxPos);
  if (!dev_e || !dev_targets || !dev_loss) return fail(RLT_ERR_INVALID_ARG, "e, targets or loss is NULL");
  if ((rs = check_memory_cfg(*cfg, mem, batch - 1)) != RLT_OK) return rs;
  if (mem->capacity < T)
    return fail(RLT_ERR_RANGE, "memory capacity %d < T = %d", mem->capacity, T);
  if (dmem) {
    if (!dmem->k || !dmem->v) return fail(RLT_ERR_INVALID_ARG, "memory gradient pointer is NULL");
    if (dmem->stride_group != mem->stride_group || dmem->stride_seq != mem->stride_seq ||
        dmem->stride_head != mem->stride_head || dmem->stride_pos != mem->stride_pos)
      return fail(RLT_ERR_SHAPE, "memory gradients must have the memory's strides");
    if (((uintptr_t)dmem->k | (uintptr_t)dmem->v) % 16)
      return fail(RLT_ERR_SHAPE, "memory gradient pointers must be 16-byte aligned");
  }
  int chunk = 0, detach = 0, segment = 0;
  if (opts) {
    chunk = opts->chunk;
    detach = opts->detach;
    segment = opts->segment;
  }
  if (chunk < 0) return fail(RLT_ERR_INVALID_ARG, "chunk must be >= 0");
  if (segment < 0) return fail(RLT_ERR_INVALID_ARG, "segment must be >= 0");
  if (detach & ~(RLT_DETACH_S | RLT_DETACH_KV)) return fail(RLT_ERR_INVALID_ARG, "unknown detach bits");
  const size_t need_ws = rlt_bptt_workspace_bytes_segmented(cfg, batch, T, segment);
  if (!dev_workspace) return fail(RLT_ERR_INVALID_ARG, "workspace is NULL");
  if ((uintptr_t)dev_workspace % 256) return fail(RLT_ERR_SHAPE, "workspace must be 256-byte aligned");
  if (workspace_bytes < need_ws)
    return fail(RLT_ERR_SHAPE, "workspace %zu bytes < %zu required", workspace_bytes, need_ws);
  if ((rs = device_health()) != RLT_OK) return rs;
  TrainArgs a{};
  a.c = *cfg;
  a.p = params;
  a.gr = grads;
  a.B = batch;
  a.T = T;
  a.e = dev_e;
  a.mk = static_cast<const float *>(mem->k);
  a.mv = static_cast<const float *>(mem->v);
  a.m_group = mem->stride_group;
  a.m_seq = mem->stride_seq;
  a.m_head = mem->stride_head;
  a.m_pos = mem->stride_pos;
  a.dmk = dmem ? static_cast<float *>(const_cast<void *>(dmem->k)) : nullptr;
  a.dmv = dmem ? static_cast<float *>(const_cast<void *>(dmem->v)) : nullptr;
  a.tg = dev_targets;
  a.chunk = chunk;
  a.detach = detach;
  a.segment = segment;
  a.de = dev_de;
  a.loss = dev_loss;
  const hipError_t e = launch_bptt(a, dev_workspace, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "bptt");
  return ok();
}

}  // extern "C"
