// Fused pyramid pooling + scoring: one pass over Q, K and V.
//
// "Long Context Pre-Training with Lighthouse Attention":
//   Sec. 3.3  level l entry i is the mean of Q (and K, V alike) over the base
//             window [i p^l, (i+1) p^l - 1];
//   Sec. 3.4  level-0 scores are the per-head l2 norms ||Q_t|| (query score QK)
//             and ||K_t|| (key score KQ); coarser levels take the max of the
//             level-0 scores over their window.
// For the top-k that follows it also records, per work-group, the range of the
// candidates' score bits it produced (levels 0..L-2), and its V plane clears the
// top-k's per-head state and histogram (nothing else touches them before the
// top-k's first pass, which starts after this kernel has finished).
//
// Work mapping: grid plane z = 0, 1, 2 pools Q, K, V respectively; the Q and K
// planes also compute the query and key scores.  A work-group of 256 threads
// covers RG row-groups x CH column chunks of EL elements (EL = 8 up to five
// levels, 4 beyond, which halves the per-level accumulators so that more
// wavefronts fit).  Row-group rg owns one coarsest window of G = p^(L-1)
// consecutive rows and walks it top to bottom, reading its rows in batches
// (2 rows up to three levels, 4 at five, 8 otherwise) one batch ahead of their
// use, so every pooled window and every max-pool lives in one thread's
// registers; only the norm of a row needs a reduction, across the CH lanes that
// hold it (adjacent lanes of one wavefront, reduced with xor shuffles).  At
// five levels (when p divides RG) the p sub-windows of a coarsest window are
// walked by p row-groups of one work-group and the coarsest level is summed
// from theirs through LDS, in sub-window order: a window of p^4 rows walked by
// one row-group would leave too few threads for the memory system.
#include "lh_internal.h"

namespace lh {

namespace {

constexpr int kMaxL = 8;   // most levels handled by the register-resident accumulators

template <typename T> struct Vec4;
template <> struct Vec4<float> {
  static __device__ __forceinline__ void load(const float *p, float (&x)[4]) {
    const float4 a = *reinterpret_cast<const float4 *>(p);
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
  }
  static __device__ __forceinline__ void store(float *p, const float (&x)[4]) {
    *reinterpret_cast<float4 *>(p) = make_float4(x[0], x[1], x[2], x[3]);
  }
};
template <> struct Vec4<uint16_t> {
  static __device__ __forceinline__ void store(uint16_t *p, const float (&x)[4]) {
    *reinterpret_cast<uint2 *>(p) = make_uint2((unsigned)f32_to_bf16_rne(x[0]) | ((unsigned)f32_to_bf16_rne(x[1]) << 16),
                                               (unsigned)f32_to_bf16_rne(x[2]) | ((unsigned)f32_to_bf16_rne(x[3]) << 16));
  }
};

template <typename T> struct Vec8;
template <> struct Vec8<float> {
  static __device__ __forceinline__ void load(const float *p, float (&x)[8]) {
    const float4 a = reinterpret_cast<const float4 *>(p)[0];
    const float4 b = reinterpret_cast<const float4 *>(p)[1];
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w; x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
  }
  static __device__ __forceinline__ void store(float *p, const float (&x)[8]) {
    reinterpret_cast<float4 *>(p)[0] = make_float4(x[0], x[1], x[2], x[3]);
    reinterpret_cast<float4 *>(p)[1] = make_float4(x[4], x[5], x[6], x[7]);
  }
};
template <> struct Vec8<uint16_t> {
  static __device__ __forceinline__ void store(uint16_t *p, const float (&x)[8]) {
    unsigned int w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w[i] = (unsigned int)f32_to_bf16_rne(x[2 * i]) | ((unsigned int)f32_to_bf16_rne(x[2 * i + 1]) << 16);
    reinterpret_cast<uint4 *>(p)[0] = make_uint4(w[0], w[1], w[2], w[3]);
  }
};

template <typename T, int N> struct VecN;
template <typename T> struct VecN<T, 4> : Vec4<T> {};
template <typename T> struct VecN<T, 8> : Vec8<T> {};


// One lane's EL elements of a row as loaded (unconverted), so that a batch of
// rows in flight costs EL * sizeof(T) bytes of registers per row.
template <typename T, int EL> struct Raw;
template <> struct Raw<uint16_t, 8> {
  uint4 a;
  __device__ __forceinline__ void load(const uint16_t *p) { a = *reinterpret_cast<const uint4 *>(p); }
  __device__ __forceinline__ void unpack(float (&x)[8]) const {
    const unsigned int w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = __uint_as_float(w[i] << 16);
      x[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  }
};
template <> struct Raw<uint16_t, 4> {
  uint2 a;
  __device__ __forceinline__ void load(const uint16_t *p) { a = *reinterpret_cast<const uint2 *>(p); }
  __device__ __forceinline__ void unpack(float (&x)[4]) const {
    x[0] = __uint_as_float(a.x << 16); x[1] = __uint_as_float(a.x & 0xFFFF0000u);
    x[2] = __uint_as_float(a.y << 16); x[3] = __uint_as_float(a.y & 0xFFFF0000u);
  }
};
template <int EL> struct Raw<float, EL> {
  float v[EL];
  __device__ __forceinline__ void load(const float *p) { VecN<float, EL>::load(p, v); }
  __device__ __forceinline__ void unpack(float (&x)[EL]) const {
#pragma unroll
    for (int e = 0; e < EL; ++e) x[e] = v[e];
  }
};

template <typename T, int D, int ML, bool SPLIT>
__global__ __launch_bounds__(256) void k_pool_score(Shape s, const T *__restrict__ q, const T *__restrict__ k,
                                                    const T *__restrict__ v, char *__restrict__ ws, FwdWs w,
                                                    float *__restrict__ scores) {
  constexpr int EL = ML <= 5 ? 8 : 4;   // elements per lane
  constexpr int CH = D / EL;            // threads per row
  constexpr int RG = 256 / CH;          // row-groups per work-group
  // rows of a window read per batch, two batches in flight (measured: short
  // windows favour occupancy, long ones more bytes in flight)
  constexpr int NB = ML <= 3 ? 2 : (ML == 5 ? 4 : 8);
  const int h = blockIdx.y;
  const int z = blockIdx.z;             // 0: Q and its scores, 1: K and its scores, 2: V
  const bool scored = z < 2;
  const int j = threadIdx.x % CH;
  const int rg = threadIdx.x / CH;
  const int L = s.L;
  const int G = s.pw[L - 1];
  // SPLIT: the p row-groups rg = p c .. p c + p - 1 of the work-group walk the
  // p sub-windows of its coarsest window c, GW = G / p rows each
  const int nsub = SPLIT ? s.p : 1;
  const int sub = rg % nsub;
  const int GW = G / nsub;
  const long long win = (long long)blockIdx.x * (RG / nsub) + rg / nsub;   // coarsest window index
  const bool active = win < s.n[L - 1];
  const T *x = z == 0 ? q : (z == 1 ? k : v);
  const long long hoff = (long long)h * s.N * D;
  float *sc = scores + (long long)h * 2 * s.P + (z == 1 ? s.P : 0);   // QK or KQ stream
  if (z == 2) {   // clear head h's top-k state and histogram, spread over the plane's work-groups
    unsigned int *hh = reinterpret_cast<unsigned int *>(ws + w.hist) + (long long)h * kHistBins;
    for (int i = blockIdx.x * 256 + threadIdx.x; i < kHistBins; i += gridDim.x * 256) hh[i] = 0u;
    if (blockIdx.x == 0 && threadIdx.x < (int)(sizeof(TopkState) / 4))
      reinterpret_cast<unsigned int *>(reinterpret_cast<TopkState *>(ws + w.state) + h)[threadIdx.x] = 0u;
  }

  // running window sums and max-pooled scores per level l >= 1 (ML >= L levels)
  float acc[ML][EL], mx[ML];
#pragma unroll
  for (int l = 0; l < ML; ++l) {
    mx[l] = 0.f;
#pragma unroll
    for (int e = 0; e < EL; ++e) acc[l][e] = 0.f;
  }
  unsigned int umin = 0xFFFFFFFFu, umax = 0u;

  const long long t0 = win * G + (long long)sub * GW;
  // the rows of the (sub-)window are read in batches of NB, one batch ahead of
  // their use (rows past the window clamp to its last row, unused)
  const long long last = active ? t0 + GW - 1 : 0;
  const T *xh = x + hoff + j * EL;
  Raw<T, EL> cur[NB], nxt[NB];
  auto load_batch = [&](Raw<T, EL>(&b)[NB], int r0) {
#pragma unroll
    for (int u = 0; u < NB; ++u) b[u].load(xh + (active ? min(t0 + r0 + u, last) : 0) * D);
  };
  load_batch(cur, 0);
  for (int r0 = 0; r0 < GW; r0 += NB) {
    if (r0 + NB < GW) load_batch(nxt, r0 + NB);
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      const int r = r0 + u;   // GW is a multiple of p^l for every level l completed here
      if (r >= GW) break;
      const long long t = t0 + r;
      float xr[EL];
      cur[u].unpack(xr);
#pragma unroll
      for (int e = 0; e < EL; ++e) xr[e] = active ? xr[e] : 0.f;
      float a = 0.f;
      if (scored) {
        float sq = 0.f;
#pragma unroll
        for (int e = 0; e < EL; ++e) sq = fmaf(xr[e], xr[e], sq);
#pragma unroll
        for (int m = 1; m < CH; m <<= 1) sq += __shfl_xor(sq, m, CH);
        a = sqrtf(sq);
        if (active && j == 0) {
          sc[t] = a;
          if (L > 1) {
            umin = min(umin, __float_as_uint(a));
            umax = max(umax, __float_as_uint(a));
          }
        }
      }
      if (L == 1) continue;
      // level 1 accumulates rows; level l+1 accumulates completed level-l windows
#pragma unroll
      for (int e = 0; e < EL; ++e) acc[1][e] += xr[e];
      mx[1] = fmaxf(mx[1], a);
#pragma unroll
      for (int l = 1; l < ML; ++l) {
        if (l >= L) break;
        if (((r + 1) % s.pw[l]) != 0) break;   // window of level l not complete yet
        const long long i = (t + 1) / s.pw[l] - 1;
        const float inv = 1.0f / (float)s.pw[l];
        if (active) {
          float mean[EL];
#pragma unroll
          for (int e = 0; e < EL; ++e) mean[e] = acc[l][e] * inv;
          VecN<T, EL>::store(reinterpret_cast<T *>(ws + w.lev[l][z]) + ((long long)h * s.n[l] + i) * D + j * EL, mean);
          if (scored && j == 0) {
            sc[s.off[l] + (int)i] = mx[l];
            if (l <= L - 2) {
              umin = min(umin, __float_as_uint(mx[l]));
              umax = max(umax, __float_as_uint(mx[l]));
            }
          }
        }
        if (l + 1 < ML && l + 1 < L) {
#pragma unroll
          for (int e = 0; e < EL; ++e) acc[l + 1][e] += acc[l][e];
          mx[l + 1] = fmaxf(mx[l + 1], mx[l]);
        }
#pragma unroll
        for (int e = 0; e < EL; ++e) acc[l][e] = 0.f;
        mx[l] = 0.f;
      }
    }
#pragma unroll
    for (int u = 0; u < NB; ++u) cur[u] = nxt[u];
  }
  if constexpr (SPLIT) {
    // acc[L-1], mx[L-1] hold this sub-window's level-(L-2) sum and max (L == ML); the
    // first row-group of the window adds the p of them in sub-window order,
    // as one walk over the whole window would
    __shared__ float part[256][EL];
    __shared__ float pmx[RG];
    static_assert(!SPLIT || ML == 5, "split walks serve five levels (L == ML)");
#pragma unroll
    for (int e = 0; e < EL; ++e) part[threadIdx.x][e] = acc[ML - 1][e];
    if (j == 0) pmx[rg] = mx[ML - 1];
    __syncthreads();
    if (sub == 0 && active) {
      float tot[EL], m = 0.f;
#pragma unroll
      for (int e = 0; e < EL; ++e) tot[e] = 0.f;
      for (int q = 0; q < nsub; ++q) {
#pragma unroll
        for (int e = 0; e < EL; ++e) tot[e] += part[threadIdx.x + q * CH][e];
        m = fmaxf(m, pmx[rg + q]);
      }
      const float inv = 1.0f / (float)G;
#pragma unroll
      for (int e = 0; e < EL; ++e) tot[e] *= inv;
      VecN<T, EL>::store(reinterpret_cast<T *>(ws + w.lev[L - 1][z]) + ((long long)h * s.n[L - 1] + win) * D + j * EL,
                         tot);
      if (scored && j == 0) sc[s.off[L - 1] + (int)win] = m;
    }
  }
  if (L == 1 || !scored) return;
  // range of this work-group's candidate score bits (min > max if it has none);
  // the union over both streams' work-groups contains every key's upper half,
  // the larger of its two scores
#pragma unroll
  for (int m = 32; m > 0; m >>= 1) {
    umin = min(umin, (unsigned int)__shfl_xor((int)umin, m));
    umax = max(umax, (unsigned int)__shfl_xor((int)umax, m));
  }
  __shared__ unsigned int red_min[4], red_max[4];
  const int wv = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    red_min[wv] = umin;
    red_max[wv] = umax;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned int mn = min(min(red_min[0], red_min[1]), min(red_min[2], red_min[3]));
    const unsigned int mxv = max(max(red_max[0], red_max[1]), max(red_max[2], red_max[3]));
    reinterpret_cast<uint2 *>(ws + w.brange)[((long long)h * 2 + z) * s.npool + blockIdx.x] = make_uint2(mn, mxv);
  }
}

}  // namespace

template <typename T, int D>
static void pool_score_ml(const Shape &s, dim3 grid, const void *q, const void *k, const void *v, char *ws,
                          const FwdWs &w, float *scores, hipStream_t st) {
  const T *qq = (const T *)q, *kk = (const T *)k, *vv = (const T *)v;
  if (s.L <= 2)
    lh::launch(k_pool_score<T, D, 2, false>, grid, 256, 0, st, s, qq, kk, vv, ws, w, scores);
  else if (s.L == 3)
    lh::launch(k_pool_score<T, D, 3, false>, grid, 256, 0, st, s, qq, kk, vv, ws, w, scores);
  else if (s.L == 4)
    lh::launch(k_pool_score<T, D, 4, false>, grid, 256, 0, st, s, qq, kk, vv, ws, w, scores);
  else if (s.L == 5 && pool_score_split(D, 5, s.p))
    lh::launch(k_pool_score<T, D, 5, true>, grid, 256, 0, st, s, qq, kk, vv, ws, w, scores);
  else if (s.L == 5)
    lh::launch(k_pool_score<T, D, 5, false>, grid, 256, 0, st, s, qq, kk, vv, ws, w, scores);
  else
    lh::launch(k_pool_score<T, D, kMaxL, false>, grid, 256, 0, st, s, qq, kk, vv, ws, w, scores);
}

hipError_t launch_pool_score(const Shape &s, const void *q, const void *k, const void *v, void *ws,
                             const FwdWs &w, float *scores, hipStream_t st) {
  if (s.L > kMaxL) return hipErrorInvalidValue;
  dim3 grid(s.npool, s.BH, 3);   // one plane per tensor: Q, K, V; s.npool = coarsest windows / row-groups
  char *wsb = reinterpret_cast<char *>(ws);
  if (s.io == LH_BF16) {
    if (s.d == 128) pool_score_ml<uint16_t, 128>(s, grid, q, k, v, wsb, w, scores, st);
    else pool_score_ml<uint16_t, 64>(s, grid, q, k, v, wsb, w, scores, st);
  } else {
    if (s.d == 128) pool_score_ml<float, 128>(s, grid, q, k, v, wsb, w, scores, st);
    else pool_score_ml<float, 64>(s, grid, q, k, v, wsb, w, scores, st);
  }
  return hipGetLastError();
}

}  // namespace lh
