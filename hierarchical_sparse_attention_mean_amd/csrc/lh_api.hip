// C ABI of liblighthouse.so: argument validation, buffer layouts and the launch
// sequence of the Lighthouse layer ("Long Context Pre-Training with Lighthouse
// Attention", Sec. 3.2-3.6).  Nothing here allocates, frees or synchronises;
// every call only enqueues kernels on the caller's stream -- except while the
// calling thread has stage timing switched on (lh_timing_begin / lh_timing_end),
// when each stage's launches are bracketed by a pair of HIP events.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <string>
#include <vector>

#include "lh_internal.h"

namespace lh {
thread_local LaunchTiming *t_launch_timing = nullptr;

hipError_t launch_attn_fwd_valu(int io, int d, int BH, int S, int Sq, const void *qt, const void *kt, const void *vt,
                                float *ot, float *lse, hipStream_t st);
hipError_t launch_attn_fwd_mfma(int d, int BH, int S, int Sq, const void *qt, const void *kt, const void *vt,
                                float *ot, float *lse, hipStream_t st);
hipError_t launch_attn_bwd_valu(int io, int d, int BH, int S, int Sq, const void *qt, const void *kt, const void *vt,
                                const float *ot, const float *lse, const float *dot, float *delta, float *dqt,
                                float *dkt, float *dvt, int part, hipStream_t st);
hipError_t launch_attn_bwd_mfma(int d, int BH, int S, int Sv, const void *qt, const void *kt, const void *vt,
                                const void *dotb, const float *rows, float *dqt, float *dkt, float *dvt, int part,
                                hipStream_t st);
hipError_t launch_attn_rowstats(int d, int BH, int S, const void *dout, int dout_bf16, const float *o,
                                const float *lse, float *pairs, float *delta, hipStream_t st);
}  // namespace lh

namespace {

thread_local std::string g_err;

// Stage timing (per host thread, off unless lh_timing_begin was called).
struct TimedSpan {
  int stage;
  hipEvent_t start, stop;
};
thread_local bool t_timing = false;
thread_local std::vector<TimedSpan> t_spans;

void timing_clear() {
  for (const TimedSpan &sp : t_spans) {
    (void)hipEventDestroy(sp.start);
    (void)hipEventDestroy(sp.stop);
  }
  t_spans.clear();
}

// Times the launches of one stage while timing is on; does nothing otherwise,
// or for a negative stage (a call that creates nothing).  The launches inside
// the span carry its events (lh::launch): the start event on the first kernel,
// the stop event on every kernel, the last one's standing.  A span with no
// launch, or whose events cannot be created, is dropped from the timing (the
// launches are unaffected).
class Span {
 public:
  Span(int stage, hipStream_t s) : stage_(stage) {
    (void)s;
    if (!t_timing || stage < 0) return;
    if (hipEventCreate(&lt_.start) != hipSuccess) return;
    if (hipEventCreate(&lt_.stop) != hipSuccess) {
      (void)hipEventDestroy(lt_.start);
      return;
    }
    lt_.started = false;
    prev_ = lh::t_launch_timing;
    lh::t_launch_timing = &lt_;
    open_ = true;
  }
  ~Span() {
    if (!open_) return;
    lh::t_launch_timing = prev_;
    if (lt_.started) {
      t_spans.push_back({stage_, lt_.start, lt_.stop});
    } else {
      (void)hipEventDestroy(lt_.start);
      (void)hipEventDestroy(lt_.stop);
    }
  }
  Span(const Span &) = delete;
  Span &operator=(const Span &) = delete;

 private:
  int stage_;
  bool open_ = false;
  lh::LaunchTiming lt_{};
  lh::LaunchTiming *prev_ = nullptr;
};

lh_status fail(lh_status st, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
lh_status fail(lh_status st, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

size_t align_up(size_t x) { return (x + 255) & ~(size_t)255; }

bool aligned16(const void *p) { return p && ((uintptr_t)p & 15u) == 0; }

size_t elem_size(int dt) { return dt == LH_BF16 ? 2 : 4; }

// Validates the shape and fills `s`.  Host-only.
lh_status make_shape(int B, int H, int64_t N, int d, int L, int p, int64_t topk, lh_dtype io, lh::Shape *s) {
  memset(s, 0, sizeof *s);
  if (B < 1 || H < 1) return fail(LH_EINVAL, "B and H must be >= 1 (got B=%d H=%d)", B, H);
  if ((int64_t)B * H > (1 << 20)) return fail(LH_EUNSUPPORTED, "B*H too large");
  if (N < 1) return fail(LH_EINVAL, "N must be >= 1 (got %lld)", (long long)N);
  if (d != 64 && d != 128) return fail(LH_EUNSUPPORTED, "head dimension d must be 64 or 128 (got %d)", d);
  if (io != LH_F32 && io != LH_BF16) return fail(LH_EINVAL, "io dtype must be LH_F32 or LH_BF16");
  if (L < 1) return fail(LH_EINVAL, "L must be >= 1 (got %d)", L);
  if (L > 8) return fail(LH_EUNSUPPORTED, "L must be <= 8 (got %d)", L);
  if (p < 2) return fail(LH_EINVAL, "p must be >= 2 (got %d)", p);
  if (topk < 0) return fail(LH_EINVAL, "topk must be >= 0 (got %lld)", (long long)topk);
  if (N * (int64_t)d >= ((int64_t)1 << 31)) return fail(LH_EUNSUPPORTED, "N*d must be < 2^31");
  int64_t pw = 1;
  for (int l = 0; l < L; ++l) {
    if (l > 0) pw *= p;
    if (pw > N) return fail(LH_EDIVIS, "p^(L-1) = %d^%d exceeds N = %lld", p, L - 1, (long long)N);
  }
  if (N % pw != 0)
    return fail(LH_EDIVIS, "p^(L-1) = %lld must divide N = %lld", (long long)pw, (long long)N);
  s->BH = B * H;
  s->N = (int)N;
  s->d = d;
  s->L = L;
  s->p = p;
  s->io = io;
  s->topk = topk;
  int64_t acc = 0, w = 1;
  for (int l = 0; l < L; ++l) {
    s->pw[l] = (int)w;
    s->n[l] = (int)(N / w);
    s->off[l] = (int)acc;
    acc += N / w;
    w *= p;
  }
  s->P = (int)acc;
  s->E = (int)(acc - s->n[L - 1]);
  // budget (L-1) p k capped by the candidates, decided without forming the
  // product when it would exceed them (so it cannot overflow): per <= 7 (2^31 - 1),
  // and below the cap per * topk < E + per
  int64_t budget = 0;
  if (L > 1) {
    const int64_t per = (int64_t)(L - 1) * p;
    budget = (topk >= (s->E + per - 1) / per) ? s->E : per * topk;
  }
  s->Bsel = (int)budget;
  s->S = s->n[L - 1] + s->Bsel;
  s->Sv = (s->S + 63) & ~63;
  if ((int64_t)s->S * d >= ((int64_t)1 << 31)) return fail(LH_EUNSUPPORTED, "S*d must be < 2^31");
  s->ntile = (s->N + lh::kCompactTile - 1) / lh::kCompactTile;
  const int wpg = lh::pool_score_windows(d, L, p);
  s->npool = (s->n[L - 1] + wpg - 1) / wpg;
  return LH_OK;
}

void saved_layout(const lh::Shape &s, lh_saved_layout_t *o) {
  const size_t BH = (size_t)s.BH, P = (size_t)s.P, S = (size_t)s.S, d = (size_t)s.d;
  const size_t es = elem_size(s.io);
  size_t cur = 0;
  auto take = [&](size_t bytes) {
    const size_t at = cur;
    cur = align_up(cur + bytes);
    return at;
  };
  o->scores = take(4 * BH * 2 * P);
  o->flags = take(BH * P);
  o->slot = take(4 * BH * P);
  o->coords = take(4 * BH * S);
  const size_t Sv = (size_t)s.Sv;
  o->qt = take(es * BH * Sv * d);
  o->kt = take(es * BH * Sv * d);
  o->vt = take(es * BH * Sv * d);
  o->ot = take(4 * BH * S * d);
  o->lse = take(4 * BH * S);
  o->total = cur;
  o->P = s.P;
  o->E = s.E;
  o->Bsel = s.Bsel;
  o->S = s.S;
  o->Sv = s.Sv;
}

void fwd_ws_layout(const lh::Shape &s, lh::FwdWs *w) {
  const size_t BH = (size_t)s.BH, d = (size_t)s.d, es = elem_size(s.io);
  size_t cur = 0;
  auto take = [&](size_t bytes) {
    const size_t at = cur;
    cur = align_up(cur + bytes);
    return at;
  };
  memset(w, 0, sizeof *w);
  for (int l = 1; l < s.L; ++l)
    for (int t = 0; t < 3; ++t) w->lev[l][t] = take(es * BH * (size_t)s.n[l] * d);
  w->brange = take(8 * BH * 2 * (size_t)s.npool);
  w->state = take(sizeof(lh::TopkState) * BH);
  w->hist = take(4 * BH * lh::kHistBins);
  const int nbf = lh::topk_blocks(s.P, lh::kFilterBlocks);
  w->cstride = (long long)nbf * lh::topk_chunk(s.P, nbf);
  w->cand = take(8 * BH * (size_t)w->cstride);
  w->ccount = take(4 * BH * (size_t)lh::kFilterBlocks);
  w->tilecount = take(4 * BH * (size_t)s.ntile);
  w->total = cur;
}

void bwd_ws_layout(const lh::Shape &s, lh::BwdWs *w) {
  const size_t BH = (size_t)s.BH, S = (size_t)s.S, d = (size_t)s.d;
  size_t cur = 0;
  auto take = [&](size_t bytes) {
    const size_t at = cur;
    cur = align_up(cur + bytes);
    return at;
  };
  const bool bf = s.io == LH_BF16;
  w->dot = take(bf ? 0 : 4 * BH * S * d);
  w->dotb = take(bf ? 2 * BH * (size_t)s.Sv * d : 0);
  w->delta = take(bf ? 0 : 4 * BH * S);
  w->rows = take(bf ? 8 * BH * (size_t)s.Sv : 0);
  w->dqt = take(4 * BH * S * d);
  w->dkt = take(4 * BH * S * d);
  w->dvt = take(4 * BH * S * d);
  w->total = cur;
}

// ---- projection-inclusive layer ----

lh_status make_layer(int B, int H, int64_t N, int d_model, int d, int L, int p, int64_t topk, lh_dtype io,
                     lh::Shape *s) {
  lh_status st = make_shape(B, H, N, d, L, p, topk, io, s);
  if (st != LH_OK) return st;
  if (d_model < 64 || d_model % 64 != 0 || d_model > (1 << 16))
    return fail(LH_EUNSUPPORTED, "d_model must be a positive multiple of 64, at most 65536 (got %d)", d_model);
  if ((int64_t)H * d > (1 << 16)) return fail(LH_EUNSUPPORTED, "H*d must be at most 65536");
  return LH_OK;
}

void layer_layout(const lh::Shape &s, int d_model, lh_layer_layout_t *o) {
  (void)d_model;
  const size_t head = elem_size(s.io) * (size_t)s.BH * (size_t)s.N * (size_t)s.d;
  size_t cur = 0;
  auto take = [&](size_t bytes) {
    const size_t at = cur;
    cur = align_up(cur + bytes);
    return at;
  };
  o->q = take(head);
  o->k = take(head);
  o->v = take(head);
  o->o = take(head);
  lh_saved_layout_t inner;
  saved_layout(s, &inner);
  o->inner = take(inner.total);
  o->inner_bytes = inner.total;
  o->total = cur;
}

// Weight gradients contract over the N tokens of each batch element, so the
// product is split along the tokens; partials are [B][splits][M][N] fp32.
// bf16: splits = 8 n (each XCD runs n of them) into equal chunks of whole
// 32-token stages, with the work-groups of an XCD (n x tiles x B) a multiple of
// its 32 compute units and at least two per unit, so that every compute unit
// gets the same work; failing that, about 1024 work-groups.
void wgrad_split(int M, int Nc, int64_t N, int B, int io, int *splits, int *kchunk) {
  const int tm = io == LH_BF16 ? 256 : 64;
  const int64_t tiles = ((M + tm - 1) / tm) * (int64_t)((Nc + tm - 1) / tm);
  if (io == LH_BF16) {
    for (int n = 1; n <= 64; ++n) {
      const int64_t sp = 8 * n, items = n * tiles * B;
      if (N % sp == 0 && (N / sp) % 32 == 0 && items % 32 == 0 && items >= 64) {
        *splits = (int)sp;
        *kchunk = (int)(N / sp);
        return;
      }
    }
  }
  const int64_t target = tiles >= 1024 ? 1 : 1024 / tiles;
  int64_t kc = (N + target - 1) / target;
  kc = (kc + 31) / 32 * 32;
  if (kc < 256) kc = 256;
  *kchunk = (int)kc;
  *splits = (int)((N + kc - 1) / kc);
}

// Backward workspace of the layer: dO, dQ, dK, dV in the head layout (io dtype),
// the inner backward workspace, and the fp32 split-K partials of the weight
// gradients (sized for the larger of X^T [dQ dK dV] and O^T dY).
struct LayerBwdWs {
  size_t dout, dq, dk, dv, inner, inner_bytes, part, total;
  int split_qkv, kchunk_qkv, split_o, kchunk_o;
};

void layer_bwd_layout(const lh::Shape &s, int B, int H, int d_model, LayerBwdWs *w) {
  const size_t head = elem_size(s.io) * (size_t)s.BH * (size_t)s.N * (size_t)s.d;
  size_t cur = 0;
  auto take = [&](size_t bytes) {
    const size_t at = cur;
    cur = align_up(cur + bytes);
    return at;
  };
  w->dout = take(head);
  w->dq = take(head);
  w->dk = take(head);
  w->dv = take(head);
  lh::BwdWs bw;
  bwd_ws_layout(s, &bw);
  w->inner = take(bw.total);
  w->inner_bytes = bw.total;
  const int Hd = H * s.d;
  wgrad_split(d_model, 3 * Hd, s.N, B, s.io, &w->split_qkv, &w->kchunk_qkv);
  wgrad_split(Hd, d_model, s.N, B, s.io, &w->split_o, &w->kchunk_o);
  const size_t pq = (size_t)B * w->split_qkv * (size_t)d_model * 3 * Hd;
  const size_t po = (size_t)B * w->split_o * (size_t)Hd * d_model;
  w->part = take(4 * (pq > po ? pq : po));
  w->total = cur;
}

// Row-major [R][C] per batch element (bstride elements apart).
lh::MatView view_plain(const void *p, long long C, long long bstride) {
  lh::MatView v{};
  v.p[0] = v.p[1] = v.p[2] = p;
  v.seg = v.hd = C;
  v.ld = C;
  v.bstride = bstride;
  return v;
}
// Head layout [B][H][N][d] of up to three tensors, as the [N][n H d] matrix of
// the layer (n = number of tensors: columns [i H d, (i+1) H d) are tensor i).
lh::MatView view_heads(const void *p0, const void *p1, const void *p2, int H, int64_t N, int d) {
  lh::MatView v{};
  v.p[0] = p0;
  v.p[1] = p1;
  v.p[2] = p2;
  v.seg = (long long)H * d;
  v.hd = d;
  v.hstride = N * d;
  v.ld = d;
  v.bstride = (long long)H * N * d;
  return v;
}
// Up to three [R][C] matrices side by side as one [R][n C] matrix.
lh::MatView view_side(const void *p0, const void *p1, const void *p2, long long C) {
  lh::MatView v = view_plain(p0, C, 0);
  v.p[1] = p1;
  v.p[2] = p2;
  return v;
}

lh::GemmArgs gemm(int M, int N, int K, const lh::MatView &a, const lh::MatView &b, const lh::MatView &c) {
  lh::GemmArgs g{};
  g.M = M;
  g.N = N;
  g.K = K;
  g.a = a;
  g.b = b;
  g.c = c;
  g.kchunk = K;
  g.splits = 1;
  return g;
}

lh_status hip_check(hipError_t e, const char *what) {
  if (e != hipSuccess) return fail(LH_EHIP, "%s: %s", what, hipGetErrorString(e));
  return LH_OK;
}

// Shared checks of the dense attention backward's operands (everything but
// its workspace).
lh_status check_attention_backward(const void *q, const void *k, const void *v, const float *o, const float *lse,
                                   const void *dout, float *dq, float *dk, float *dv, int BH, int64_t S, int d,
                                   lh_dtype io) {
  if (BH < 1 || S < 1) return fail(LH_EINVAL, "BH and S must be >= 1");
  if (d != 64 && d != 128) return fail(LH_EUNSUPPORTED, "head dimension d must be 64 or 128 (got %d)", d);
  if (io != LH_F32 && io != LH_BF16) return fail(LH_EINVAL, "io dtype must be LH_F32 or LH_BF16");
  if (S * (int64_t)d >= ((int64_t)1 << 31)) return fail(LH_EUNSUPPORTED, "S*d must be < 2^31");
  if (io == LH_BF16 && S % 64 != 0)
    return fail(LH_EUNSUPPORTED, "LH_BF16 needs S to be a multiple of 64 (got %lld)", (long long)S);
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(dout))
    return fail(LH_EINVAL, "q, k, v, o, dout must be non-NULL and 16-byte aligned");
  if (!aligned16(dq) || !aligned16(dk) || !aligned16(dv))
    return fail(LH_EINVAL, "dq, dk, dv must be non-NULL and 16-byte aligned");
  if (!lse || ((uintptr_t)lse & 3u)) return fail(LH_EINVAL, "lse must be non-NULL and 4-byte aligned");
  return LH_OK;
}

// Workspace bytes of the dense attention backward: the (LSE log2 e, delta)
// pair of every row (LH_BF16) or delta alone (LH_F32).
size_t attention_backward_ws(int BH, int64_t S, lh_dtype io) {
  return (io == LH_BF16 ? 8 : 4) * (size_t)BH * (size_t)S;
}

// The dense attention backward's launches, on validated operands, with its
// workspace at wsf; `timed`: bracket the stages for stage timing.
lh_status run_attention_backward(const void *q, const void *k, const void *v, const float *o, const float *lse,
                                 const void *dout, float *dq, float *dk, float *dv, int BH, int64_t S, int d,
                                 lh_dtype io, float *wsf, bool timed, hipStream_t hs) {
  lh_status st;
  {
    Span sp(timed ? LH_STAGE_SCATTER_BWD : -1, timed ? hs : nullptr);   // the row terms take the scatter adjoint's place
    if ((st = hip_check(lh::launch_attn_rowstats(d, BH, (int)S, dout, io == LH_BF16, o, lse,
                                                 io == LH_BF16 ? wsf : nullptr, io == LH_BF16 ? nullptr : wsf, hs),
                        "attention row terms")) != LH_OK)
      return st;
  }
  for (int part = 0; part < 2; ++part) {
    Span sp(timed ? (part == 0 ? LH_STAGE_ATTN_BWD_DQ : LH_STAGE_ATTN_BWD_DKDV) : -1, timed ? hs : nullptr);
    hipError_t e;
    if (io == LH_BF16)
      e = lh::launch_attn_bwd_mfma(d, BH, (int)S, (int)S, q, k, v, dout, wsf, dq, dk, dv, part, hs);
    else
      e = lh::launch_attn_bwd_valu(io, d, BH, (int)S, (int)S, q, k, v, o, lse, reinterpret_cast<const float *>(dout),
                                   wsf, dq, dk, dv, part, hs);
    if ((st = hip_check(e, "attention backward")) != LH_OK) return st;
  }
  return LH_OK;
}

}  // namespace

// ---- library-owned scratch of lh_attention_backward_noalloc ----
// One fixed array per GPU, in the library's code object: the dense attention
// backward's per-row workspace for callers that cannot allocate.  Host code
// never uses the name `scratch` as an address (on the host it is only a
// stand-in for the symbol): the device address of each GPU's copy comes from
// hipGetSymbolAddress, looked up once per device with that device current.
static constexpr size_t kScratchBytes = (size_t)32 << 20;   // 32 MiB
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_dev[kMaxScratchDevices];   // device address of `scratch` per device (null until looked up)

// Device address of `scratch` on the device that runs `hs`.
lh_status scratch_on(hipStream_t hs, void **out) {
  int dev = 0, cur = 0;
  lh_status st;
  if ((st = hip_check(hipStreamGetDevice(hs, &dev), "hipStreamGetDevice")) != LH_OK) return st;
  if (dev < 0 || dev >= kMaxScratchDevices) return fail(LH_EUNSUPPORTED, "device %d beyond the scratch table", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    if ((st = hip_check(hipGetDevice(&cur), "hipGetDevice")) != LH_OK) return st;
    if (cur != dev && (st = hip_check(hipSetDevice(dev), "hipSetDevice")) != LH_OK) return st;
    void *p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) (void)hipSetDevice(cur);
    if ((st = hip_check(e, "hipGetSymbolAddress(scratch)")) != LH_OK) return st;
    if (!p) return fail(LH_EHIP, "hipGetSymbolAddress(scratch) returned a null address");
    g_scratch_dev[dev] = p;
  }
  *out = g_scratch_dev[dev];
  return LH_OK;
}

}  // namespace

extern "C" {

const char *lh_status_string(lh_status s) {
  switch (s) {
    case LH_OK: return "ok";
    case LH_EINVAL: return "invalid argument";
    case LH_EDIVIS: return "p^(L-1) does not divide N";
    case LH_EUNSUPPORTED: return "unsupported shape or dtype";
    case LH_EWORKSPACE: return "buffer too small";
    case LH_EHIP: return "HIP error";
  }
  return "unknown status";
}

const char *lh_last_error(void) { return g_err.c_str(); }

lh_status lh_query(int B, int H, int64_t N, int d, int L, int p, int64_t topk, lh_dtype io, int64_t *S,
                   size_t *saved_bytes, size_t *fwd_ws_bytes, size_t *bwd_ws_bytes) {
  lh::Shape s;
  lh_status st = make_shape(B, H, N, d, L, p, topk, io, &s);
  if (st != LH_OK) return st;
  lh_saved_layout_t sl;
  saved_layout(s, &sl);
  lh::FwdWs fw;
  fwd_ws_layout(s, &fw);
  lh::BwdWs bw;
  bwd_ws_layout(s, &bw);
  if (S) *S = s.S;
  if (saved_bytes) *saved_bytes = sl.total;
  if (fwd_ws_bytes) *fwd_ws_bytes = fw.total;
  if (bwd_ws_bytes) *bwd_ws_bytes = bw.total;
  return LH_OK;
}

lh_status lh_saved_layout(int B, int H, int64_t N, int d, int L, int p, int64_t topk, lh_dtype io,
                          lh_saved_layout_t *out) {
  if (!out) return fail(LH_EINVAL, "out is NULL");
  lh::Shape s;
  lh_status st = make_shape(B, H, N, d, L, p, topk, io, &s);
  if (st != LH_OK) return st;
  saved_layout(s, out);
  return LH_OK;
}

lh_status lh_forward(const void *q, const void *k, const void *v, void *o, lh_dtype o_dtype, int B, int H, int64_t N,
                     int d, int L, int p, int64_t topk, lh_dtype io, void *saved, size_t saved_bytes, void *ws,
                     size_t ws_bytes, void *stream) {
  lh::Shape s;
  lh_status st = make_shape(B, H, N, d, L, p, topk, io, &s);
  if (st != LH_OK) return st;
  if (o_dtype != LH_F32 && o_dtype != LH_BF16) return fail(LH_EINVAL, "o_dtype must be LH_F32 or LH_BF16");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
    return fail(LH_EINVAL, "q, k, v, o must be non-NULL and 16-byte aligned");
  if (!aligned16(saved) || !aligned16(ws)) return fail(LH_EINVAL, "saved and ws must be non-NULL and 16-byte aligned");
  lh_saved_layout_t sl;
  saved_layout(s, &sl);
  lh::FwdWs fw;
  fwd_ws_layout(s, &fw);
  if (saved_bytes < sl.total)
    return fail(LH_EWORKSPACE, "saved buffer too small: %zu < %zu bytes", saved_bytes, sl.total);
  if (ws_bytes < fw.total) return fail(LH_EWORKSPACE, "forward workspace too small: %zu < %zu bytes", ws_bytes, fw.total);

  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  char *sv = reinterpret_cast<char *>(saved);
  float *scores = reinterpret_cast<float *>(sv + sl.scores);
  uint8_t *flags = reinterpret_cast<uint8_t *>(sv + sl.flags);
  int *slot = reinterpret_cast<int *>(sv + sl.slot);
  int *coords = reinterpret_cast<int *>(sv + sl.coords);
  float *ot = reinterpret_cast<float *>(sv + sl.ot);
  float *lse = reinterpret_cast<float *>(sv + sl.lse);

  // (i)+(ii) pyramid and scores in one pass over Q, K, V (which also clears the
  // top-k state and histogram and records each work-group's score range)
  {
    Span sp(LH_STAGE_POOL_SCORE, hs);
    if ((st = hip_check(lh::launch_pool_score(s, q, k, v, ws, fw, scores, hs), "pool_score")) != LH_OK) return st;
  }
  // (ii) selection
  {
    Span sp(LH_STAGE_TOPK, hs);
    if ((st = hip_check(lh::launch_topk(s, ws, fw, scores, flags, hs), "topk")) != LH_OK) return st;
  }
  // (iii) topological compaction + gather
  {
    Span sp(LH_STAGE_GATHER, hs);
    if ((st = hip_check(lh::launch_compact_gather(s, q, k, v, ws, fw, flags, slot, coords, sv + sl.qt, sv + sl.kt,
                                                  sv + sl.vt, hs),
                        "compact_gather")) != LH_OK)
      return st;
  }
  // (iii) causal attention over the sub-sequence
  {
    Span sp(LH_STAGE_ATTN_FWD, hs);
    hipError_t e;
    if (s.io == LH_BF16)
      e = lh::launch_attn_fwd_mfma(s.d, s.BH, s.S, s.Sv, sv + sl.qt, sv + sl.kt, sv + sl.vt, ot, lse, hs);
    else
      e = lh::launch_attn_fwd_valu(s.io, s.d, s.BH, s.S, s.Sv, sv + sl.qt, sv + sl.kt, sv + sl.vt, ot, lse, hs);
    if ((st = hip_check(e, "attention")) != LH_OK) return st;
  }
  // (iv) scatter-back
  {
    Span sp(LH_STAGE_SCATTER, hs);
    if ((st = hip_check(lh::launch_scatter(s, slot, coords, ot, o, o_dtype, hs), "scatter")) != LH_OK) return st;
  }
  return LH_OK;
}

lh_status lh_backward(const void *q, const void *k, const void *v, const void *dout, lh_dtype dout_dtype,
                      const void *saved, size_t saved_bytes, void *dq, void *dk, void *dv, lh_dtype grad_dtype, int B,
                      int H, int64_t N, int d, int L, int p, int64_t topk, lh_dtype io, void *ws, size_t ws_bytes,
                      void *stream) {
  lh::Shape s;
  lh_status st = make_shape(B, H, N, d, L, p, topk, io, &s);
  if (st != LH_OK) return st;
  if (dout_dtype != LH_F32 && dout_dtype != LH_BF16) return fail(LH_EINVAL, "dout_dtype must be LH_F32 or LH_BF16");
  if (grad_dtype != LH_F32 && grad_dtype != LH_BF16) return fail(LH_EINVAL, "grad_dtype must be LH_F32 or LH_BF16");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(dout))
    return fail(LH_EINVAL, "q, k, v, dout must be non-NULL and 16-byte aligned");
  if (!aligned16(dq) || !aligned16(dk) || !aligned16(dv))
    return fail(LH_EINVAL, "dq, dk, dv must be non-NULL and 16-byte aligned");
  if (!aligned16(saved) || !aligned16(ws)) return fail(LH_EINVAL, "saved and ws must be non-NULL and 16-byte aligned");
  lh_saved_layout_t sl;
  saved_layout(s, &sl);
  lh::BwdWs bw;
  bwd_ws_layout(s, &bw);
  if (saved_bytes < sl.total)
    return fail(LH_EWORKSPACE, "saved buffer too small: %zu < %zu bytes", saved_bytes, sl.total);
  if (ws_bytes < bw.total) return fail(LH_EWORKSPACE, "backward workspace too small: %zu < %zu bytes", ws_bytes, bw.total);
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  const char *sv = reinterpret_cast<const char *>(saved);
  char *wb = reinterpret_cast<char *>(ws);
  const int *slot = reinterpret_cast<const int *>(sv + sl.slot);
  const int *coords = reinterpret_cast<const int *>(sv + sl.coords);
  const float *ot = reinterpret_cast<const float *>(sv + sl.ot);
  const float *lse = reinterpret_cast<const float *>(sv + sl.lse);
  float *dot = reinterpret_cast<float *>(wb + bw.dot);
  uint16_t *dotb = reinterpret_cast<uint16_t *>(wb + bw.dotb);
  float *delta = reinterpret_cast<float *>(wb + bw.delta);
  float *rows = reinterpret_cast<float *>(wb + bw.rows);
  float *dqt = reinterpret_cast<float *>(wb + bw.dqt);
  float *dkt = reinterpret_cast<float *>(wb + bw.dkt);
  float *dvt = reinterpret_cast<float *>(wb + bw.dvt);
  (void)q;
  (void)k;
  (void)v;
  // adjoint of the scatter: dO~ (and delta = rowsum(dO~ * O~))
  {
    Span sp(LH_STAGE_SCATTER_BWD, hs);
    if ((st = hip_check(lh::launch_scatter_bwd(s, dout, dout_dtype, slot, coords, ot, lse, dot, dotb, delta, rows, hs),
                        "scatter_bwd")) != LH_OK)
      return st;
  }
  // adjoint of the sub-sequence attention: dQ~, then dK~ and dV~
  for (int part = 0; part < 2; ++part) {
    Span sp(part == 0 ? LH_STAGE_ATTN_BWD_DQ : LH_STAGE_ATTN_BWD_DKDV, hs);
    hipError_t e;
    if (s.io == LH_BF16)
      e = lh::launch_attn_bwd_mfma(s.d, s.BH, s.S, s.Sv, sv + sl.qt, sv + sl.kt, sv + sl.vt, dotb, rows, dqt, dkt,
                                   dvt, part, hs);
    else
      e = lh::launch_attn_bwd_valu(s.io, s.d, s.BH, s.S, s.Sv, sv + sl.qt, sv + sl.kt, sv + sl.vt, ot, lse, dot, delta,
                                   dqt, dkt, dvt, part, hs);
    if ((st = hip_check(e, "attention backward")) != LH_OK) return st;
  }
  // adjoint of the gather and of the pooling
  {
    Span sp(LH_STAGE_POOL_BWD, hs);
    if ((st = hip_check(lh::launch_pool_bwd(s, slot, dqt, dkt, dvt, dq, dk, dv, grad_dtype, hs), "pool_bwd")) !=
        LH_OK)
      return st;
  }
  return LH_OK;
}

lh_status lh_attention_forward(const void *q, const void *k, const void *v, float *o, float *lse, int BH, int64_t S,
                               int d, lh_dtype io, void *stream) {
  if (BH < 1 || S < 1) return fail(LH_EINVAL, "BH and S must be >= 1");
  if (d != 64 && d != 128) return fail(LH_EUNSUPPORTED, "head dimension d must be 64 or 128 (got %d)", d);
  if (io != LH_F32 && io != LH_BF16) return fail(LH_EINVAL, "io dtype must be LH_F32 or LH_BF16");
  if (S * (int64_t)d >= ((int64_t)1 << 31)) return fail(LH_EUNSUPPORTED, "S*d must be < 2^31");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
    return fail(LH_EINVAL, "q, k, v, o must be non-NULL and 16-byte aligned");
  if (lse && ((uintptr_t)lse & 3u)) return fail(LH_EINVAL, "lse must be 4-byte aligned");
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  hipError_t e;
  if (io == LH_BF16) e = lh::launch_attn_fwd_mfma(d, BH, (int)S, (int)S, q, k, v, o, lse, hs);
  else e = lh::launch_attn_fwd_valu(io, d, BH, (int)S, (int)S, q, k, v, o, lse, hs);
  return hip_check(e, "attention");
}

lh_status lh_attention_backward(const void *q, const void *k, const void *v, const float *o, const float *lse,
                                const void *dout, float *dq, float *dk, float *dv, int BH, int64_t S, int d,
                                lh_dtype io, void *ws, size_t ws_bytes, void *stream) {
  lh_status st = check_attention_backward(q, k, v, o, lse, dout, dq, dk, dv, BH, S, d, io);
  if (st != LH_OK) return st;
  if (!aligned16(ws)) return fail(LH_EINVAL, "ws must be non-NULL and 16-byte aligned");
  const size_t need = attention_backward_ws(BH, S, io);
  if (ws_bytes < need) return fail(LH_EWORKSPACE, "workspace too small: %zu < %zu bytes", ws_bytes, need);
  return run_attention_backward(q, k, v, o, lse, dout, dq, dk, dv, BH, S, d, io, reinterpret_cast<float *>(ws), true,
                                reinterpret_cast<hipStream_t>(stream));
}

lh_status lh_attention_backward_noalloc(const void *q, const void *k, const void *v, const float *o,
                                        const float *lse, const void *dout, float *dq, float *dk, float *dv, int BH,
                                        int64_t S, int d, lh_dtype io, void *stream) {
  lh_status st = check_attention_backward(q, k, v, o, lse, dout, dq, dk, dv, BH, S, d, io);
  if (st != LH_OK) return st;
  const size_t need = attention_backward_ws(BH, S, io);
  if (need > kScratchBytes)
    return fail(LH_EWORKSPACE,
                "BH*S = %lld rows need %zu bytes of scratch, beyond the library's fixed %zu bytes "
                "(at most %zu rows in this dtype); use lh_attention_backward with a workspace",
                (long long)BH * (long long)S, need, kScratchBytes, kScratchBytes / (io == LH_BF16 ? 8 : 4));
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  void *sp = nullptr;
  if ((st = scratch_on(hs, &sp)) != LH_OK) return st;
  // every row of the scratch that the backward reads is written by its first
  // kernel in the same call, so nothing needs clearing
  return run_attention_backward(q, k, v, o, lse, dout, dq, dk, dv, BH, S, d, io, reinterpret_cast<float *>(sp), false,
                                hs);
}

lh_status lh_layer_query(int B, int H, int64_t N, int d_model, int d, int L, int p, int64_t topk, lh_dtype io,
                         int64_t *S, size_t *saved_bytes, size_t *fwd_ws_bytes, size_t *bwd_ws_bytes) {
  lh::Shape s;
  lh_status st = make_layer(B, H, N, d_model, d, L, p, topk, io, &s);
  if (st != LH_OK) return st;
  lh_layer_layout_t ll;
  layer_layout(s, d_model, &ll);
  lh::FwdWs fw;
  fwd_ws_layout(s, &fw);
  LayerBwdWs bw;
  layer_bwd_layout(s, B, H, d_model, &bw);
  if (S) *S = s.S;
  if (saved_bytes) *saved_bytes = ll.total;
  if (fwd_ws_bytes) *fwd_ws_bytes = fw.total;
  if (bwd_ws_bytes) *bwd_ws_bytes = bw.total;
  return LH_OK;
}

lh_status lh_layer_saved_layout(int B, int H, int64_t N, int d_model, int d, int L, int p, int64_t topk, lh_dtype io,
                                lh_layer_layout_t *out) {
  if (!out) return fail(LH_EINVAL, "out is NULL");
  lh::Shape s;
  lh_status st = make_layer(B, H, N, d_model, d, L, p, topk, io, &s);
  if (st != LH_OK) return st;
  layer_layout(s, d_model, out);
  return LH_OK;
}

lh_status lh_layer_forward(const void *x, const void *wq, const void *wk, const void *wv, const void *wo, void *y,
                           lh_dtype y_dtype, int B, int H, int64_t N, int d_model, int d, int L, int p, int64_t topk,
                           lh_dtype io, void *saved, size_t saved_bytes, void *ws, size_t ws_bytes, void *stream) {
  lh::Shape s;
  lh_status st = make_layer(B, H, N, d_model, d, L, p, topk, io, &s);
  if (st != LH_OK) return st;
  if (y_dtype != LH_F32 && y_dtype != LH_BF16) return fail(LH_EINVAL, "y_dtype must be LH_F32 or LH_BF16");
  if (!aligned16(x) || !aligned16(wq) || !aligned16(wk) || !aligned16(wv) || !aligned16(wo) || !aligned16(y))
    return fail(LH_EINVAL, "x, wq, wk, wv, wo, y must be non-NULL and 16-byte aligned");
  if (!aligned16(saved) || !aligned16(ws)) return fail(LH_EINVAL, "saved and ws must be non-NULL and 16-byte aligned");
  lh_layer_layout_t ll;
  layer_layout(s, d_model, &ll);
  lh::FwdWs fw;
  fwd_ws_layout(s, &fw);
  if (saved_bytes < ll.total)
    return fail(LH_EWORKSPACE, "saved buffer too small: %zu < %zu bytes", saved_bytes, ll.total);
  if (ws_bytes < fw.total) return fail(LH_EWORKSPACE, "forward workspace too small: %zu < %zu bytes", ws_bytes, fw.total);
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  char *sv = reinterpret_cast<char *>(saved);
  const int Hd = H * d;
  // Q, K, V = X W_Q, X W_K, X W_V, written in the head layout
  {
    Span sp(LH_STAGE_PROJ, hs);
    const lh::GemmArgs g = gemm((int)N, 3 * Hd, d_model, view_plain(x, d_model, N * d_model),
                                view_side(wq, wk, wv, Hd), view_heads(sv + ll.q, sv + ll.k, sv + ll.v, H, N, d));
    if ((st = hip_check(lh::launch_gemm(g, true, false, io, io, B, hs), "projection")) != LH_OK) return st;
  }
  // the Lighthouse attention of every head
  if ((st = lh_forward(sv + ll.q, sv + ll.k, sv + ll.v, sv + ll.o, io, B, H, N, d, L, p, topk, io, sv + ll.inner,
                       ll.inner_bytes, ws, ws_bytes, stream)) != LH_OK)
    return st;
  // Y = [O_0 .. O_{H-1}] W_O
  {
    Span sp(LH_STAGE_OUT_PROJ, hs);
    const lh::GemmArgs g = gemm((int)N, d_model, Hd, view_heads(sv + ll.o, nullptr, nullptr, H, N, d),
                                view_plain(wo, d_model, 0), view_plain(y, d_model, N * d_model));
    if ((st = hip_check(lh::launch_gemm(g, true, false, io, y_dtype, B, hs), "output projection")) != LH_OK)
      return st;
  }
  return LH_OK;
}

lh_status lh_layer_backward(const void *x, const void *wq, const void *wk, const void *wv, const void *wo,
                            const void *dy, const void *saved, size_t saved_bytes, void *dx, lh_dtype dx_dtype,
                            float *dwq, float *dwk, float *dwv, float *dwo, int B, int H, int64_t N, int d_model,
                            int d, int L, int p, int64_t topk, lh_dtype io, void *ws, size_t ws_bytes, void *stream) {
  lh::Shape s;
  lh_status st = make_layer(B, H, N, d_model, d, L, p, topk, io, &s);
  if (st != LH_OK) return st;
  if (dx_dtype != LH_F32 && dx_dtype != LH_BF16) return fail(LH_EINVAL, "dx_dtype must be LH_F32 or LH_BF16");
  if (!aligned16(x) || !aligned16(wq) || !aligned16(wk) || !aligned16(wv) || !aligned16(wo) || !aligned16(dy))
    return fail(LH_EINVAL, "x, wq, wk, wv, wo, dy must be non-NULL and 16-byte aligned");
  if (!aligned16(dx) || !aligned16(dwq) || !aligned16(dwk) || !aligned16(dwv) || !aligned16(dwo))
    return fail(LH_EINVAL, "dx, dwq, dwk, dwv, dwo must be non-NULL and 16-byte aligned");
  if (!aligned16(saved) || !aligned16(ws)) return fail(LH_EINVAL, "saved and ws must be non-NULL and 16-byte aligned");
  lh_layer_layout_t ll;
  layer_layout(s, d_model, &ll);
  LayerBwdWs bw;
  layer_bwd_layout(s, B, H, d_model, &bw);
  if (saved_bytes < ll.total)
    return fail(LH_EWORKSPACE, "saved buffer too small: %zu < %zu bytes", saved_bytes, ll.total);
  if (ws_bytes < bw.total) return fail(LH_EWORKSPACE, "backward workspace too small: %zu < %zu bytes", ws_bytes, bw.total);
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  const char *sv = reinterpret_cast<const char *>(saved);
  char *wb = reinterpret_cast<char *>(ws);
  float *part = reinterpret_cast<float *>(wb + bw.part);
  const int Hd = H * d;
  const lh::MatView vdy = view_plain(dy, d_model, N * d_model);
  // dO = dY W_O^T (head layout) and dW_O = O^T dY
  {
    Span sp(LH_STAGE_OUT_PROJ_BWD, hs);
    const lh::GemmArgs g = gemm((int)N, Hd, d_model, vdy, view_plain(wo, d_model, 0),
                                view_heads(wb + bw.dout, nullptr, nullptr, H, N, d));
    if ((st = hip_check(lh::launch_gemm(g, true, true, io, io, B, hs), "dO")) != LH_OK) return st;
    lh::GemmArgs gw = gemm(Hd, d_model, (int)N, view_heads(sv + ll.o, nullptr, nullptr, H, N, d), vdy,
                           view_plain(part, d_model, (long long)bw.split_o * Hd * d_model));
    gw.kchunk = bw.kchunk_o;
    gw.splits = bw.split_o;
    gw.zstride = (long long)Hd * d_model;
    if ((st = hip_check(lh::launch_gemm(gw, false, false, io, LH_F32, B, hs), "dW_O")) != LH_OK) return st;
    if ((st = hip_check(lh::launch_split_reduce(part, B * bw.split_o, Hd, d_model, view_plain(dwo, d_model, 0), hs),
                        "dW_O reduce")) != LH_OK)
      return st;
  }
  // dQ, dK, dV through the Lighthouse attention (selection frozen)
  if ((st = lh_backward(sv + ll.q, sv + ll.k, sv + ll.v, wb + bw.dout, io, sv + ll.inner, ll.inner_bytes, wb + bw.dq,
                        wb + bw.dk, wb + bw.dv, io, B, H, N, d, L, p, topk, io, wb + bw.inner, bw.inner_bytes,
                        stream)) != LH_OK)
    return st;
  // dX = dQ W_Q^T + dK W_K^T + dV W_V^T and dW_{Q,K,V} = X^T d{Q,K,V}
  {
    Span sp(LH_STAGE_PROJ_BWD, hs);
    const lh::MatView vg = view_heads(wb + bw.dq, wb + bw.dk, wb + bw.dv, H, N, d);
    const lh::GemmArgs g = gemm((int)N, d_model, 3 * Hd, vg, view_side(wq, wk, wv, Hd),
                                view_plain(dx, d_model, N * d_model));
    if ((st = hip_check(lh::launch_gemm(g, true, true, io, dx_dtype, B, hs), "dX")) != LH_OK) return st;
    lh::GemmArgs gw = gemm(d_model, 3 * Hd, (int)N, view_plain(x, d_model, N * d_model), vg,
                           view_plain(part, 3 * Hd, (long long)bw.split_qkv * d_model * 3 * Hd));
    gw.kchunk = bw.kchunk_qkv;
    gw.splits = bw.split_qkv;
    gw.zstride = (long long)d_model * 3 * Hd;
    if ((st = hip_check(lh::launch_gemm(gw, false, false, io, LH_F32, B, hs), "dW_QKV")) != LH_OK) return st;
    if ((st = hip_check(lh::launch_split_reduce(part, B * bw.split_qkv, d_model, 3 * Hd, view_side(dwq, dwk, dwv, Hd),
                                                hs),
                        "dW_QKV reduce")) != LH_OK)
      return st;
  }
  return LH_OK;
}

const char *lh_stage_name(int stage) {
  switch (stage) {
    case LH_STAGE_POOL_SCORE: return "pool_score";
    case LH_STAGE_TOPK: return "topk";
    case LH_STAGE_GATHER: return "gather";
    case LH_STAGE_ATTN_FWD: return "attn_fwd";
    case LH_STAGE_SCATTER: return "scatter";
    case LH_STAGE_SCATTER_BWD: return "scatter_bwd";
    case LH_STAGE_ATTN_BWD_DQ: return "attn_bwd_dq";
    case LH_STAGE_ATTN_BWD_DKDV: return "attn_bwd_dkdv";
    case LH_STAGE_POOL_BWD: return "pool_bwd";
    case LH_STAGE_PROJ: return "proj";
    case LH_STAGE_OUT_PROJ: return "out_proj";
    case LH_STAGE_OUT_PROJ_BWD: return "out_proj_bwd";
    case LH_STAGE_PROJ_BWD: return "proj_bwd";
    default: return "unknown";
  }
}

lh_status lh_timing_begin(void) {
  timing_clear();
  t_timing = true;
  return LH_OK;
}

lh_status lh_timing_end(double *ms, int *spans, int n) {
  if (n < 0 || (n > 0 && (!ms || !spans))) return fail(LH_EINVAL, "ms and spans must hold n >= 0 entries");
  t_timing = false;
  for (int i = 0; i < n; ++i) {
    ms[i] = 0.0;
    spans[i] = 0;
  }
  lh_status st = LH_OK;
  for (const TimedSpan &sp : t_spans) {
    float t = 0.f;
    hipError_t e = hipEventSynchronize(sp.stop);
    if (e == hipSuccess) e = hipEventElapsedTime(&t, sp.start, sp.stop);
    if (e != hipSuccess) {
      if (st == LH_OK) st = fail(LH_EHIP, "stage timing: %s", hipGetErrorString(e));
      continue;
    }
    if (sp.stage < n) {
      ms[sp.stage] += t;
      spans[sp.stage] += 1;
    }
  }
  timing_clear();
  return st;
}

}  // extern "C"
