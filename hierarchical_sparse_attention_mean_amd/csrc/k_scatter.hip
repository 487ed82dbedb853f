// Scatter-back (forward) and the two adjoint passes that read the slot map.
//
// "Long Context Pre-Training with Lighthouse Attention", Sec. 3.6: the output
// of a selected entry (l, i) is written to the base positions of its window
// shifted by p^l - 1, i.e. [(i+1) p^l - 1, (i+2) p^l - 2] (clipped at N - 1);
// within a level these ranges are disjoint and adjacent, across levels the
// contributions are summed, so each position receives at most L of them.  The
// paper uses a deterministic integer-atomic scatter.  Here the integer
// arithmetic is kept -- every contribution is quantised to int64 fixed point
// with 32 fractional bits (round half to even) and the integers are summed, so
// the result does not depend on summation order -- but the atomics are not
// needed: the one entry of level l covering position t is
// i = floor((t+1) / p^l) - 1, so each output element pulls its <= L
// contributions and owns its accumulator.
//
// When p is a power of two the scatter groups positions that share their
// coarser entries: in one pass (k_scatter_one) where level-0 entries are dense,
// otherwise in two (coarser levels for every position, then the few positions
// with a selected level-0 entry; k_scatter_hi / k_scatter_lo).
//
// Adjoints (Sec. 3.2: gradients flow through scatter, attention, gather and
// pool; the selection is frozen):
//   k_scatter_bwd  dO~_m = sum of dO_t over the scatter range of entry m
//                  (k_scatter_bwd_walk + k_scatter_delta at four levels or more);
//   k_pool_bwd     dX_t = sum_l [entry (l, floor(t/p^l)) selected] dX~_slot / p^l
//                  for X in {Q, K, V} (gather adjoint fused with pool adjoint).
#include <type_traits>

#include "lh_internal.h"

namespace lh {

namespace {

__device__ __forceinline__ long long to_fixed(float x) {
  // x * 2^32 is exact in fp32; round half to even, then the integer value is exact in int64
  return (long long)rintf(x * 4294967296.0f);
}

__device__ __forceinline__ float from_fixed(long long a) {
  return (float)((double)a * 2.3283064365386963e-10);   // * 2^-32, then fp32 round-to-nearest-even
}

constexpr int kMaxL = 8;   // levels supported (validated on the host)

__device__ __forceinline__ void store_row8(void *o, int o_dtype, long long off, const float (&q)[8]) {
  if (o_dtype == LH_BF16) {
    uint4 w;
    w.x = (unsigned)f32_to_bf16_rne(q[0]) | ((unsigned)f32_to_bf16_rne(q[1]) << 16);
    w.y = (unsigned)f32_to_bf16_rne(q[2]) | ((unsigned)f32_to_bf16_rne(q[3]) << 16);
    w.z = (unsigned)f32_to_bf16_rne(q[4]) | ((unsigned)f32_to_bf16_rne(q[5]) << 16);
    w.w = (unsigned)f32_to_bf16_rne(q[6]) | ((unsigned)f32_to_bf16_rne(q[7]) << 16);
    *reinterpret_cast<uint4 *>(reinterpret_cast<uint16_t *>(o) + off) = w;
  } else {
    float *of = reinterpret_cast<float *>(o) + off;
    *reinterpret_cast<float4 *>(of) = make_float4(q[0], q[1], q[2], q[3]);
    *reinterpret_cast<float4 *>(of + 4) = make_float4(q[4], q[5], q[6], q[7]);
  }
}

__device__ __forceinline__ void load_row8(const float *p, float (&x)[8]) {
  const float4 x0 = *reinterpret_cast<const float4 *>(p);
  const float4 x1 = *reinterpret_cast<const float4 *>(p + 4);
  x[0] = x0.x; x[1] = x0.y; x[2] = x0.z; x[3] = x0.w; x[4] = x1.x; x[5] = x1.y; x[6] = x1.z; x[7] = x1.w;
}

// Any p.  One thread per (position, 8-element chunk).  Positions are numbered
// u = t + 1 and a work-group covers u in [b TP, (b + 1) TP), TP = 256 / (D / 8):
// for every level whose p^l divides TP, the entries it reads (i = u / p^l - 1)
// are read by this work-group only.  Slot lookups are issued before the rows.
template <int D>
__global__ __launch_bounds__(256) void k_scatter(Shape s, const int *__restrict__ slot, const float *__restrict__ ot,
                                                 void *__restrict__ o, int o_dtype) {
  constexpr int C8 = D / 8;
  const int h = blockIdx.y;
  const int c = threadIdx.x % C8;
  const int u = blockIdx.x * (256 / C8) + threadIdx.x / C8;
  if (u < 1 || u > s.N) return;
  const int *sl = slot + (long long)h * s.P;
  const float *ob = ot + (long long)h * s.S * D + c * 8;
  int m[kMaxL];
#pragma unroll
  for (int l = 0; l < kMaxL; ++l) {
    m[l] = -1;
    if (l < s.L) {
      const int i = u / s.pw[l] - 1;
      if (i >= 0) m[l] = sl[s.off[l] + i];
    }
  }
  double a[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) a[e] = 0.0;
  bool big = false;
#pragma unroll
  for (int l = 0; l < kMaxL; ++l) {
    if (m[l] < 0) continue;
    float x[8];
    load_row8(ob + (long long)m[l] * D, x);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      big |= !(fabsf(x[e]) < 262144.f);
      a[e] += (double)rintf(x[e] * 4294967296.0f);
    }
  }
  float q[8];
  if (!big) {
#pragma unroll
    for (int e = 0; e < 8; ++e) q[e] = (float)(a[e] * 2.3283064365386963e-10);
  } else {
    long long b[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int l = 0; l < kMaxL; ++l) {
      if (m[l] < 0) continue;
      for (int e = 0; e < 8; ++e) b[e] += to_fixed(ob[(long long)m[l] * D + e]);
    }
    for (int e = 0; e < 8; ++e) q[e] = from_fixed(b[e]);
  }
  store_row8(o, o_dtype, ((long long)h * s.N + (u - 1)) * D + c * 8, q);
}

constexpr int kScatterOneGroups = 1;   // groups of 4 positions per thread in k_scatter_one

// p a power of two >= 4, in two passes (where few positions have a selected
// level-0 entry; k_scatter_one below otherwise).
//   k_scatter_hi   one thread per (8 positions u = u0 .. u0 + 7, u = t + 1, u0
//                  a multiple of 8; 8-element chunk).  Every level with
//                  p^l >= 8 has one entry for all eight (i = (u0 >> l log2 p)
//                  - 1), looked up and read once; at p = 4 level 1 has one per
//                  group of four.  All lookups are issued first, then all rows;
//                  each position's sum is fixed_out's, formed with the shared
//                  levels' terms first (every partial sum is an exact integer
//                  in fp64, so the value is the same), on the same large-value
//                  condition.  Writes every position's sum over its coarser
//                  levels.
//   k_scatter_lo   one thread per (gathered row, 8-element chunk); rows of
//                  level 0 (a few percent of them) rewrite their position's
//                  output with the full sum, their own row included.
// Both form the same fixed-point sum, so the result does not depend on which
// pass wrote a position last.
//
// fixed_out: the fixed-point sum of a position's contributions (k_scatter forms
// the same sum inline), i.e. the sum over its selected entries of RNE(x 2^32)
// as an integer, converted back with one rounding (* 2^-32 -> fp32 RNE, then
// bf16 RNE if the output is bf16).  RNE(x 2^32) is
// an integer that fp32 rintf gives exactly; while every |x| < 2^18 each term is
// below 2^50 in magnitude and the sum of at most kMaxL of them is exact in
// fp64, which is then the same integer as the int64 sum (and (double)int64
// gives the same value): that path is taken unless some |x| >= 2^18, where the
// int64 sum is formed instead.
template <int LM>
__device__ __forceinline__ void fixed_out(const float (&xs)[LM][8], const bool (&has)[LM], float (&q)[8]) {
  bool big = false;
  double a[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) a[e] = 0.0;
#pragma unroll
  for (int l = 0; l < LM; ++l) {
    if (!has[l]) continue;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      big |= !(fabsf(xs[l][e]) < 262144.f);
      a[e] += (double)rintf(xs[l][e] * 4294967296.0f);
    }
  }
  if (!big) {
#pragma unroll
    for (int e = 0; e < 8; ++e) q[e] = (float)(a[e] * 2.3283064365386963e-10);
  } else {
    for (int e = 0; e < 8; ++e) {
      long long b = 0;
      for (int l = 0; l < LM; ++l)
        if (has[l]) b += to_fixed(xs[l][e]);
      q[e] = from_fixed(b);
    }
  }
}

// p a power of two, in one pass: one thread per (group of 4 positions u =
// u0 .. u0 + 3, u0 a multiple of 4; 8-element chunk).  The group shares its
// entry of every level with p^l >= 4 (one per pair at level 1 at P2); those
// slots are looked up together with the slots of the group's four level-0
// entries, and the coarser rows and the selected level-0 rows are then loaded
// together.  The coarser levels are summed once per group (per pair at P2) in
// exact fixed point, each position adds its level-0 term, and every position is
// written once with its full sum.  On the large-value path (some |x| >= 2^18)
// the coarser rows are read again and the int64 sum formed, as fixed_out does.
template <int D, int LM, bool P2>
__global__ __launch_bounds__(256) void k_scatter_one(Shape s, const int *__restrict__ slot,
                                                     const float *__restrict__ ot, void *__restrict__ o, int o_dtype) {
  constexpr int C8 = D / 8;
  constexpr int NG = kScatterOneGroups;
  constexpr int GPP = 256 / C8;    // groups per pass of the work-group
  constexpr int NPR = P2 ? 2 : 1;  // coarse sums per group
  const int h = blockIdx.y;
  const int c = threadIdx.x % C8;
  const int lg = __builtin_ctz(s.p);
  const int *sl = slot + (long long)h * s.P;
  const float *ob = ot + (long long)h * s.S * D + c * 8;
  int u0[NG], mh[NG][LM], m1[NG], m0[NG][4];
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    u0[g] = 4 * (blockIdx.x * (GPP * NG) + g * GPP + threadIdx.x / C8);
#pragma unroll
    for (int l = 0; l < LM; ++l) {
      mh[g][l] = -1;
      if (l >= 1 && l < s.L && u0[g] <= s.N) {
        const int i = (u0[g] >> (l * lg)) - 1;
        if (i >= 0) mh[g][l] = sl[s.off[l] + i];
      }
    }
    m1[g] = -1;
    if (P2 && s.L > 1 && u0[g] + 2 <= s.N) m1[g] = sl[s.off[1] + (u0[g] >> 1)];   // i = (u0 + 2) / 2 - 1
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = u0[g] + r - 1;
      m0[g][r] = (t >= 0 && t < s.N) ? sl[t] : -1;
    }
  }
  float x0[NG][4][8];
#pragma unroll
  for (int g = 0; g < NG; ++g)
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (m0[g][r] >= 0) load_row8(ob + (long long)m0[g][r] * D, x0[g][r]);
  // coarse sums: A[g][pr] = sum of RNE(x 2^32) over the coarser levels of the
  // group (pair pr at P2), exact in fp64 unless big[g]
  double A[NG][NPR][8];
  bool big[NG];
  {
    float xs[NG][LM][8], x1[P2 ? NG : 1][8];
#pragma unroll
    for (int g = 0; g < NG; ++g) {
#pragma unroll
      for (int l = 1; l < LM; ++l)
        if (mh[g][l] >= 0) load_row8(ob + (long long)mh[g][l] * D, xs[g][l]);
      if constexpr (P2)
        if (m1[g] >= 0) load_row8(ob + (long long)m1[g] * D, x1[g]);
    }
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      big[g] = false;
      double sh[8];   // levels 2 .. (shared by both pairs at P2), then level 1
#pragma unroll
      for (int e = 0; e < 8; ++e) sh[e] = 0.0;
#pragma unroll
      for (int l = 2; l < LM; ++l) {
        if (mh[g][l] < 0) continue;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          big[g] |= !(fabsf(xs[g][l][e]) < 262144.f);
          sh[e] += (double)rintf(xs[g][l][e] * 4294967296.0f);
        }
      }
#pragma unroll
      for (int pr = 0; pr < NPR; ++pr) {
        const bool has1 = pr == 0 ? mh[g][1] >= 0 : m1[g] >= 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          A[g][pr][e] = sh[e];
          if (has1) {
            const float x = pr == 0 ? xs[g][1][e] : x1[P2 ? g : 0][e];
            big[g] |= !(fabsf(x) < 262144.f);
            A[g][pr][e] += (double)rintf(x * 4294967296.0f);
          }
        }
      }
    }
  }
#pragma unroll
  for (int g = 0; g < NG; ++g) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = u0[g] + r - 1;
      if (t < 0 || t >= s.N) continue;
      const int pr = P2 ? (r >> 1) : 0;
      bool bg = big[g];
      double a[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        a[e] = A[g][pr][e];
        if (m0[g][r] >= 0) {
          bg |= !(fabsf(x0[g][r][e]) < 262144.f);
          a[e] += (double)rintf(x0[g][r][e] * 4294967296.0f);
        }
      }
      float q[8];
      if (!bg) {
#pragma unroll
        for (int e = 0; e < 8; ++e) q[e] = (float)(a[e] * 2.3283064365386963e-10);
      } else {
        // int64 path: the position's terms again, from memory
        long long b[8];
        for (int e = 0; e < 8; ++e) b[e] = m0[g][r] >= 0 ? to_fixed(x0[g][r][e]) : 0;
        for (int l = 1; l < LM; ++l) {
          const int m = (P2 && l == 1 && pr == 1) ? m1[g] : mh[g][l];
          if (m < 0) continue;
          float x[8];
          load_row8(ob + (long long)m * D, x);
          for (int e = 0; e < 8; ++e) b[e] += to_fixed(x[e]);
        }
        for (int e = 0; e < 8; ++e) q[e] = from_fixed(b[e]);
      }
      store_row8(o, o_dtype, ((long long)h * s.N + t) * D + c * 8, q);
    }
  }
}

template <int D, int LM>
__global__ __launch_bounds__(256) void k_scatter_hi(Shape s, const int *__restrict__ slot,
                                                    const float *__restrict__ ot, void *__restrict__ o, int o_dtype) {
  constexpr int C8 = D / 8;
  constexpr int UPP = 256 / C8;   // 8-position units per work-group
  const int h = blockIdx.y;
  const int c = threadIdx.x % C8;
  const int lg = __builtin_ctz(s.p);
  const int *sl = slot + (long long)h * s.P;
  const float *ob = ot + (long long)h * s.S * D + c * 8;
  const int u0 = 8 * (blockIdx.x * UPP + threadIdx.x / C8);
  if (u0 > s.N) return;
  // level 1 at p = 4 has one entry per group of four; the levels l >= ls one
  // for all eight positions
  const int l4 = s.p == 4 ? 1 : 0;
  const int ls = l4 + 1;
  auto look = [&](int l, int u) {
    if (l < 1 || l >= s.L || u > s.N) return -1;
    const int i = (u >> (l * lg)) - 1;
    return i >= 0 ? sl[s.off[l] + i] : -1;
  };
  int mg[2], mc[LM];
#pragma unroll
  for (int g = 0; g < 2; ++g) mg[g] = l4 > 0 ? look(l4, u0 + 4 * g) : -1;
#pragma unroll
  for (int l = 0; l < LM; ++l) mc[l] = l >= ls ? look(l, u0) : -1;
  float xg[2][8], xc[LM][8];
#pragma unroll
  for (int g = 0; g < 2; ++g)
    if (mg[g] >= 0) load_row8(ob + (long long)mg[g] * D, xg[g]);
#pragma unroll
  for (int l = 1; l < LM; ++l)
    if (mc[l] >= 0) load_row8(ob + (long long)mc[l] * D, xc[l]);
  auto add = [&](const float (&x)[8], double (&a)[8], bool &bg) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      bg |= !(fabsf(x[e]) < 262144.f);
      a[e] += (double)rintf(x[e] * 4294967296.0f);
    }
  };
  bool big = false;
  double A[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) A[e] = 0.0;
#pragma unroll
  for (int l = 1; l < LM; ++l)
    if (mc[l] >= 0) add(xc[l], A, big);
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    const int ug = u0 + 4 * g;
    if (ug > s.N) break;
    bool bg = big;
    double a[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) a[e] = A[e];
    if (mg[g] >= 0) add(xg[g], a, bg);
    float qv[8];
    if (!bg) {
#pragma unroll
      for (int e = 0; e < 8; ++e) qv[e] = (float)(a[e] * 2.3283064365386963e-10);
    } else {
      for (int e = 0; e < 8; ++e) {
        long long b = mg[g] >= 0 ? to_fixed(xg[g][e]) : 0;
        for (int l = 1; l < LM; ++l)
          if (mc[l] >= 0) b += to_fixed(xc[l][e]);
        qv[e] = from_fixed(b);
      }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = ug + r - 1;
      if (t >= 0 && t < s.N) store_row8(o, o_dtype, ((long long)h * s.N + t) * D + c * 8, qv);
    }
  }
}

template <int D, int LM>
__global__ __launch_bounds__(256) void k_scatter_lo(Shape s, const int *__restrict__ slot,
                                                    const int *__restrict__ coords, const float *__restrict__ ot,
                                                    void *__restrict__ o, int o_dtype) {
  constexpr int C8 = D / 8;
  const int h = blockIdx.y;
  const int c = threadIdx.x % C8;
  const int m = blockIdx.x * (256 / C8) + threadIdx.x / C8;
  if (m >= s.S) return;
  const int t = coords[(long long)h * s.S + m];
  if (t >= s.N) return;   // not a level-0 entry (flat indices of level 0 are 0 .. N-1)
  const int lg = __builtin_ctz(s.p);
  const int u = t + 1;
  const int *sl = slot + (long long)h * s.P;
  const float *ob = ot + (long long)h * s.S * D + c * 8;
  int mh[LM];
  mh[0] = m;
#pragma unroll
  for (int l = 1; l < LM; ++l) {
    mh[l] = -1;
    if (l < s.L) {
      const int i = (u >> (l * lg)) - 1;
      if (i >= 0) mh[l] = sl[s.off[l] + i];
    }
  }
  float xs[LM][8];
  bool has[LM];
#pragma unroll
  for (int l = 0; l < LM; ++l) {
    has[l] = mh[l] >= 0;
    if (has[l]) load_row8(ob + (long long)mh[l] * D, xs[l]);
  }
  float q[8];
  fixed_out<LM>(xs, has, q);
  store_row8(o, o_dtype, ((long long)h * s.N + t) * D + c * 8, q);
}

// One thread per (slot m, 8-column chunk): 256 / (D / 8) slots per work-group.
// dO~_m = sum of dO over the entry's scatter range (t ascending), then
//   delta_m = sum_d dO~[m][d] * O~[m][d]
// with dO~ as the attention backward will read it (bf16-rounded in bf16 mode).
// fp32 mode writes dO~ in fp32 and delta; bf16 mode writes dO~ in bf16
// (row-major, head stride Sv, zero rows S..Sv-1) and the per-row pair
// (LSE log2(e), delta) (zeros on the padding rows).
template <int D, bool BF16>
__global__ __launch_bounds__(256) void k_scatter_bwd(Shape s, const void *__restrict__ dout, int dout_dtype,
                                                     const int *__restrict__ coords, const float *__restrict__ ot,
                                                     float *__restrict__ dot32, uint16_t *__restrict__ dotb,
                                                     float *__restrict__ delta, const float *__restrict__ lse,
                                                     float *__restrict__ rows) {
  constexpr int C8 = D / 8;
  constexpr int SPB = 256 / C8;
  const int h = blockIdx.y;
  const int c = threadIdx.x % C8;
  const int m = blockIdx.x * SPB + threadIdx.x / C8;
  const bool active = m < s.S;
  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
  float o8[8];
  if (active) {
    const int f = coords[(long long)h * s.S + m];
    int l = 0;
    while (l + 1 < s.L && f >= s.off[l + 1]) ++l;
    const int i = f - s.off[l];
    const int lo = (i + 1) * s.pw[l] - 1;
    const int hi = min(s.N - 1, lo + s.pw[l] - 1);
    const float4 a0 = *reinterpret_cast<const float4 *>(ot + ((long long)h * s.S + m) * D + c * 8);
    const float4 a1 = *reinterpret_cast<const float4 *>(ot + ((long long)h * s.S + m) * D + c * 8 + 4);
    o8[0] = a0.x; o8[1] = a0.y; o8[2] = a0.z; o8[3] = a0.w; o8[4] = a1.x; o8[5] = a1.y; o8[6] = a1.z; o8[7] = a1.w;
    const long long base = ((long long)h * s.N) * D + c * 8;
    if (dout_dtype == LH_BF16) {
      const uint16_t *src = reinterpret_cast<const uint16_t *>(dout) + base;
      // rows t ascending, 16 rows in flight while at least 16 remain, then 4,
      // then 1 (ranges of 16 rows and more are the coarser levels'): the
      // additions are the same, in the same order
      auto rows_bf16 = [&](int t0, auto n) {
        constexpr int R = decltype(n)::value;
        uint4 w[R];
#pragma unroll
        for (int u = 0; u < R; ++u) w[u] = *reinterpret_cast<const uint4 *>(src + (long long)(t0 + u) * D);
#pragma unroll
        for (int u = 0; u < R; ++u) {
          const unsigned v[4] = {w[u].x, w[u].y, w[u].z, w[u].w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            acc[2 * e] += __uint_as_float(v[e] << 16);
            acc[2 * e + 1] += __uint_as_float(v[e] & 0xFFFF0000u);
          }
        }
      };
      int t = lo;
      for (; t + 15 <= hi; t += 16) rows_bf16(t, std::integral_constant<int, 16>{});
      for (; t + 3 <= hi; t += 4) rows_bf16(t, std::integral_constant<int, 4>{});
      for (; t <= hi; ++t) {
        const uint4 w = *reinterpret_cast<const uint4 *>(src + (long long)t * D);
        const unsigned v[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc[2 * e] += __uint_as_float(v[e] << 16);
          acc[2 * e + 1] += __uint_as_float(v[e] & 0xFFFF0000u);
        }
      }
    } else {
      const float *src = reinterpret_cast<const float *>(dout) + base;
      for (int t = lo; t <= hi; ++t) {
        const float4 x0 = *reinterpret_cast<const float4 *>(src + (long long)t * D);
        const float4 x1 = *reinterpret_cast<const float4 *>(src + (long long)t * D + 4);
        acc[0] += x0.x; acc[1] += x0.y; acc[2] += x0.z; acc[3] += x0.w;
        acc[4] += x1.x; acc[5] += x1.y; acc[6] += x1.z; acc[7] += x1.w;
      }
    }
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) o8[e] = 0.f;
  }
  uint16_t hb[8];
  if constexpr (BF16) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      hb[e] = f32_to_bf16_rne(acc[e]);
      acc[e] = bf16_to_f32(hb[e]);
    }
  }
  float dl = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) dl = fmaf(acc[e], o8[e], dl);
#pragma unroll
  for (int x = 1; x < C8; x <<= 1) dl += __shfl_xor(dl, x);
  if constexpr (BF16) {
    if (m < s.Sv) {
      uint4 w;
      w.x = (unsigned)hb[0] | ((unsigned)hb[1] << 16);
      w.y = (unsigned)hb[2] | ((unsigned)hb[3] << 16);
      w.z = (unsigned)hb[4] | ((unsigned)hb[5] << 16);
      w.w = (unsigned)hb[6] | ((unsigned)hb[7] << 16);
      *reinterpret_cast<uint4 *>(dotb + ((long long)h * s.Sv + m) * D + c * 8) = w;
      if (c == 0)
        *reinterpret_cast<float2 *>(rows + 2 * ((long long)h * s.Sv + m)) =
            active ? make_float2(lse[(long long)h * s.S + m] * 1.4426950408889634f, dl) : make_float2(0.f, 0.f);
    }
  } else {
    if (active) {
      if (c == 0) delta[(long long)h * s.S + m] = dl;
      float *dst = dot32 + ((long long)h * s.S + m) * D + c * 8;
      *reinterpret_cast<float4 *>(dst) = make_float4(acc[0], acc[1], acc[2], acc[3]);
      *reinterpret_cast<float4 *>(dst + 4) = make_float4(acc[4], acc[5], acc[6], acc[7]);
    }
  }
}

constexpr int kWalkCoarse = 2;   // most levels k_scatter_bwd_walk combines through LDS

// Position-major scatter adjoint, when p = 2^LG is 2 or 4 and the coarsest
// range p^(L-1) fits a work-group's span W = RG GW.  In u = t + 1 the range of
// entry (l, i) is the aligned block [(i+1) p^l, (i+2) p^l), so a walk over u
// in aligned blocks meets every entry's range exactly once, like the pooling
// walk of the forward: row group g of the work-group (C8 lanes, 8 columns
// each) reads the dO rows of its GW = p^A consecutive positions once (all
// loads issued together), sums the ranges of levels 0 .. A in registers (level l's sum
// is the sum of its p children's, levels ascending), and on completing the
// range of a selected entry writes its dO~ row; the work-group then forms the
// ranges of levels A+1 .. L-1 from its row groups' block sums through LDS, in
// row-group order.  dO is read once (k_scatter_bwd reads a row once per
// selected entry covering it, up to L times).  The walk reads no O~: delta and
// the row pairs come from k_scatter_delta afterwards, so no step of the walk
// waits on a load that depends on a slot.
template <int D, bool BF16, int GW, int LG>
__global__ __launch_bounds__(256) void k_scatter_bwd_walk(Shape s, const void *__restrict__ dout, int dout_dtype,
                                                          const int *__restrict__ slot, float *__restrict__ dot32,
                                                          uint16_t *__restrict__ dotb) {
  constexpr int C8 = D / 8;
  constexpr int RG = 256 / C8;
  constexpr int W = RG * GW;           // u positions per work-group
  constexpr int NB = GW;               // rows per batch: all of the row group's rows in flight at once
  constexpr int A = __builtin_ctz(GW) / LG;   // levels 1 .. A summed in registers (p^A = GW)
  static_assert((1 << (A * LG)) == GW, "GW is a power of p");
  // slots of the block's entries of levels 1 .. A: level l has GW >> (l LG) of them, at sbase(l)
  constexpr auto sbase = [](int l) {
    int o = 0;
    for (int k = 1; k < l; ++k) o += GW >> (k * LG);
    return o;
  };
  constexpr int NSL = sbase(A + 1) > 0 ? sbase(A + 1) : 1;
  __shared__ __attribute__((aligned(16))) float part[RG][D + 4];   // rows of (D + 4) floats: 16-byte aligned
  const int h = blockIdx.y;
  const int c = threadIdx.x % C8, g = threadIdx.x / C8;
  const int *sl = slot + (long long)h * s.P;
  const int ub = blockIdx.x * W + g * GW;   // first u of this row group's block
  const long long dbase = ((long long)h * s.N) * D + c * 8;

  // dO~ row of entry slot m with range sum x (rounded to bf16 in bf16 mode)
  auto emit = [&](int m, const float (&x)[8]) {
    if constexpr (BF16) {
      uint4 w;
      w.x = (unsigned)f32_to_bf16_rne(x[0]) | ((unsigned)f32_to_bf16_rne(x[1]) << 16);
      w.y = (unsigned)f32_to_bf16_rne(x[2]) | ((unsigned)f32_to_bf16_rne(x[3]) << 16);
      w.z = (unsigned)f32_to_bf16_rne(x[4]) | ((unsigned)f32_to_bf16_rne(x[5]) << 16);
      w.w = (unsigned)f32_to_bf16_rne(x[6]) | ((unsigned)f32_to_bf16_rne(x[7]) << 16);
      *reinterpret_cast<uint4 *>(dotb + ((long long)h * s.Sv + m) * D + c * 8) = w;
    } else {
      float *dst = dot32 + ((long long)h * s.S + m) * D + c * 8;
      *reinterpret_cast<float4 *>(dst) = make_float4(x[0], x[1], x[2], x[3]);
      *reinterpret_cast<float4 *>(dst + 4) = make_float4(x[4], x[5], x[6], x[7]);
    }
  };
  // slot of the entry of level l whose range ends at u, or -1
  auto slot_at = [&](int l, int u) {
    const int i = (u >> (l * LG)) - 1;
    return (i >= 0 && i < s.n[l]) ? sl[s.off[l] + i] : -1;
  };

  int msl[NSL];
#pragma unroll
  for (int l = 1; l <= A; ++l)
#pragma unroll
    for (int k = 0; k < (GW >> (l * LG)); ++k) msl[sbase(l) + k] = slot_at(l, ub + ((k + 1) << (l * LG)) - 1);
  // the entries of levels A+1 .. L-1 whose range this row group combines (see
  // below), looked up ahead of the walk
  constexpr int NCO = kWalkCoarse;   // levels above A (the launcher dispatches L - 1 - A <= kWalkCoarse)
  int mco[NCO];
#pragma unroll
  for (int j = 0; j < NCO; ++j) {
    const int l = A + 1 + j;
    mco[j] = -1;
    if (l < s.L && g < W / s.pw[l]) mco[j] = slot_at(l, blockIdx.x * W + (g + 1) * s.pw[l] - 1);
  }
  float acc[A + 1][8];   // acc[l]: running range sum of level l >= 1; acc[0]: the block sum
#pragma unroll
  for (int l = 0; l <= A; ++l)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[l][e] = 0.f;
#pragma unroll
  for (int r0 = 0; r0 < GW; r0 += NB) {
    // a batch of NB rows (zeros outside 0 <= t < N) and their level-0 slots
    uint4 raw[NB];
    float xf[BF16 ? 1 : NB][8];
    int m0[NB];
#pragma unroll
    for (int r = 0; r < NB; ++r) {
      const int t = ub + r0 + r - 1;
      const bool ok = t >= 0 && t < s.N;
      m0[r] = ok ? sl[t] : -1;
      if constexpr (BF16) {
        raw[r] = ok ? *reinterpret_cast<const uint4 *>(reinterpret_cast<const uint16_t *>(dout) + dbase +
                                                       (long long)t * D)
                    : make_uint4(0u, 0u, 0u, 0u);
      } else {
        if (ok) load_row8(reinterpret_cast<const float *>(dout) + dbase + (long long)t * D, xf[r]);
        else
#pragma unroll
          for (int e = 0; e < 8; ++e) xf[r][e] = 0.f;
      }
    }
#pragma unroll
    for (int r = 0; r < NB; ++r) {
      const int rr = r0 + r;
      float x[8];
      if constexpr (BF16) {
        const unsigned v[4] = {raw[r].x, raw[r].y, raw[r].z, raw[r].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          x[2 * e] = __uint_as_float(v[e] << 16);
          x[2 * e + 1] = __uint_as_float(v[e] & 0xFFFF0000u);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = xf[r][e];
      }
      if (m0[r] >= 0) emit(m0[r], x);   // level 0: the row itself
      if constexpr (A == 0) {
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[0][e] = x[e];   // the block sum (GW = 1)
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[1][e] += x[e];
#pragma unroll
        for (int l = 1; l <= A; ++l) {
          if (((rr + 1) & ((1 << (l * LG)) - 1)) != 0) break;   // range of level l not complete
          const int m = msl[sbase(l) + (rr >> (l * LG))];
          if (m >= 0) emit(m, acc[l]);
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            if (l < A) acc[l + 1][e] += acc[l][e];
            else acc[0][e] = acc[l][e];   // the block sum (level A)
            acc[l][e] = 0.f;
          }
        }
      }
    }
  }
  if (A + 1 >= s.L) return;   // every level handled in registers
  // levels A+1 .. L-1: sums of consecutive row groups' block sums, in order
#pragma unroll
  for (int e = 0; e < 8; ++e) part[g][c * 8 + e] = acc[0][e];
  __syncthreads();
#pragma unroll
  for (int j = 0; j < NCO; ++j) {
    if (mco[j] < 0) continue;   // no such level, range or selection
    const int per = s.pw[A + 1 + j] / GW;   // row groups per range of the level
    // x = part[g per] + part[g per + 1] + ... element by element, in order;
    // each partial row read as two 16-byte vectors, the loads independent
    float x[8];
    auto get = [&](int r, float (&y)[8]) {
      const float4 u = *reinterpret_cast<const float4 *>(&part[g * per + r][c * 8]);
      const float4 v = *reinterpret_cast<const float4 *>(&part[g * per + r][c * 8 + 4]);
      y[0] = u.x; y[1] = u.y; y[2] = u.z; y[3] = u.w; y[4] = v.x; y[5] = v.y; y[6] = v.z; y[7] = v.w;
    };
    get(0, x);
#pragma unroll 4
    for (int r = 1; r < per; ++r) {
      float y[8];
      get(r, y);
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] += y[e];
    }
    emit(mco[j], x);
  }
}

// delta_m = rowsum(dO~_m o O~_m) with dO~ as the walk stored it (bf16 in bf16
// mode), in the arithmetic k_scatter_bwd uses (an fma chain over a lane's 8
// elements, then a xor-shuffle tree over the row's C8 lanes), so the two give
// the same bits.  bf16 mode writes the row pair (LSE log2(e), delta) and zeros
// on the padding rows S .. Sv-1 (dO~ and pair); fp32 mode writes delta.  One
// thread per (row, 8 columns).
template <int D, bool BF16>
__global__ __launch_bounds__(256) void k_scatter_delta(Shape s, const float *__restrict__ ot,
                                                       const float *__restrict__ dot32, uint16_t *__restrict__ dotb,
                                                       float *__restrict__ delta, const float *__restrict__ lse,
                                                       float *__restrict__ rows) {
  constexpr int C8 = D / 8;
  const int h = blockIdx.y;
  const int c = threadIdx.x % C8;
  const int m = blockIdx.x * (256 / C8) + threadIdx.x / C8;   // the C8 lanes of a row exit together
  if (m >= (BF16 ? s.Sv : s.S)) return;
  if (BF16 && m >= s.S) {
    *reinterpret_cast<uint4 *>(dotb + ((long long)h * s.Sv + m) * D + c * 8) = make_uint4(0u, 0u, 0u, 0u);
    if (c == 0) *reinterpret_cast<float2 *>(rows + 2 * ((long long)h * s.Sv + m)) = make_float2(0.f, 0.f);
    return;
  }
  float y[8], o8[8];
  if constexpr (BF16) {
    const uint4 w = *reinterpret_cast<const uint4 *>(dotb + ((long long)h * s.Sv + m) * D + c * 8);
    const unsigned v[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      y[2 * e] = __uint_as_float(v[e] << 16);
      y[2 * e + 1] = __uint_as_float(v[e] & 0xFFFF0000u);
    }
  } else {
    load_row8(dot32 + ((long long)h * s.S + m) * D + c * 8, y);
  }
  load_row8(ot + ((long long)h * s.S + m) * D + c * 8, o8);
  float dl = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) dl = fmaf(y[e], o8[e], dl);
#pragma unroll
  for (int xo = 1; xo < C8; xo <<= 1) dl += __shfl_xor(dl, xo);
  if (c == 0) {
    if constexpr (BF16)
      *reinterpret_cast<float2 *>(rows + 2 * ((long long)h * s.Sv + m)) =
          make_float2(lse[(long long)h * s.S + m] * 1.4426950408889634f, dl);
    else
      delta[(long long)h * s.S + m] = dl;
  }
}

// One thread per 8 consecutive elements of a position's row of dQ, dK, dV
// (16-byte stores); slots of the position's entries looked up first.
// Arithmetic: per level in ascending order, acc = fma(dX~, 1/p^l, acc).
template <int D>
__global__ __launch_bounds__(256) void k_pool_bwd(Shape s, const int *__restrict__ slot, const float *__restrict__ dqt,
                                                  const float *__restrict__ dkt, const float *__restrict__ dvt,
                                                  void *__restrict__ dq, void *__restrict__ dk, void *__restrict__ dv,
                                                  int grad_dtype) {
  constexpr int C8 = D / 8;
  const int h = blockIdx.y;
  const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (long long)s.N * C8) return;
  const int t = (int)(idx / C8);
  const int c = (int)(idx % C8);
  const int *sl = slot + (long long)h * s.P;
  const long long hs = (long long)h * s.S;
  int m[kMaxL];
#pragma unroll
  for (int l = 0; l < kMaxL; ++l) m[l] = (l < s.L) ? sl[s.off[l] + t / s.pw[l]] : -1;
  float acc[3][8];
#pragma unroll
  for (int u = 0; u < 3; ++u)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[u][e] = 0.f;
  const float *src[3] = {dqt, dkt, dvt};
#pragma unroll
  for (int l = 0; l < kMaxL; ++l) {
    if (m[l] < 0) continue;
    const float inv = 1.f / (float)s.pw[l];
    const long long ro = (hs + m[l]) * D + c * 8;
#pragma unroll
    for (int u = 0; u < 3; ++u) {
      float x[8];
      load_row8(src[u] + ro, x);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[u][e] = fmaf(x[e], inv, acc[u][e]);
    }
  }
  const long long off = ((long long)h * s.N + t) * D + c * 8;
  void *dst[3] = {dq, dk, dv};
#pragma unroll
  for (int u = 0; u < 3; ++u) store_row8(dst[u], grad_dtype, off, acc[u]);
}

// p a power of two, p >= 4.  One thread per (gradient u = blockIdx.z of dQ, dK,
// dV; group of 4 positions t0 .. t0 + 3, t0 a multiple of 4; 8-element chunk):
// the group shares its entry (l, t0 >> l log2 p) of every level l >= 1 and has
// one level-0 entry per position.  All slots first, then all rows; the same
// per-position arithmetic as k_pool_bwd (levels ascending,
// acc = fma(dX~, 1/p^l, acc)).
template <int D, int LM>
__global__ __launch_bounds__(256) void k_pool_bwd_g4(Shape s, const int *__restrict__ slot,
                                                     const float *__restrict__ dqt, const float *__restrict__ dkt,
                                                     const float *__restrict__ dvt, void *__restrict__ dq,
                                                     void *__restrict__ dk, void *__restrict__ dv, int grad_dtype) {
  constexpr int C8 = D / 8;
  const int h = blockIdx.y;
  const int u = blockIdx.z;
  const int c = threadIdx.x % C8;
  const int t0 = 4 * (blockIdx.x * (256 / C8) + threadIdx.x / C8);
  if (t0 >= s.N) return;
  const int lg = __builtin_ctz(s.p);
  const int *sl = slot + (long long)h * s.P;
  const float *src = (u == 0 ? dqt : u == 1 ? dkt : dvt) + (long long)h * s.S * D + c * 8;
  int m0[4], mh[LM];
#pragma unroll
  for (int r = 0; r < 4; ++r) m0[r] = (t0 + r < s.N) ? sl[t0 + r] : -1;
#pragma unroll
  for (int l = 1; l < LM; ++l) mh[l] = (l < s.L) ? sl[s.off[l] + (t0 >> (l * lg))] : -1;
  float xh[LM][8], x0[4][8];
#pragma unroll
  for (int l = 1; l < LM; ++l)
    if (mh[l] >= 0) load_row8(src + (long long)mh[l] * D, xh[l]);
#pragma unroll
  for (int r = 0; r < 4; ++r)
    if (m0[r] >= 0) load_row8(src + (long long)m0[r] * D, x0[r]);
  void *dst = u == 0 ? dq : u == 1 ? dk : dv;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    if (t0 + r >= s.N) continue;
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.f;
    if (m0[r] >= 0)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = fmaf(x0[r][e], 1.f, acc[e]);
#pragma unroll
    for (int l = 1; l < LM; ++l) {
      if (mh[l] < 0) continue;
      const float inv = 1.f / (float)s.pw[l];
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = fmaf(xh[l][e], inv, acc[e]);
    }
    store_row8(dst, grad_dtype, ((long long)h * s.N + t0 + r) * D + c * 8, acc);
  }
}

}  // namespace

hipError_t launch_scatter(const Shape &s, const int *slot, const int *coords, const float *ot, void *o,
                          int o_dtype, hipStream_t st) {
  const int per = 256 / (s.d / 8);   // positions (or groups of 4 positions) per pass of a work-group
  if (s.p >= 2 && (s.p & (s.p - 1)) == 0 && (s.p >= 4 || (s.N & 1) == 0)) {
    // One pass where level-0 entries are dense, two passes elsewhere.  Their
    // density follows the budget.  Measured at N = 98,304: at p >= 4 the one
    // pass is faster from Bsel = N / 4 on (L = 3, k = 3,072 / 6,144: 56% / 69%
    // of the HBM peak vs 53% / 48%), slower below (k = 1,536: 49% vs 57%; 512K,
    // where 3% of the positions have a level-0 entry: 0.39 vs 0.28 ms); at
    // p = 2 at every budget measured (k = 1,536 / 4,096: 64% / 69% vs 59% /
    // 54%), so p = 2 always takes it.
    const bool one = s.p == 2 || 4LL * s.Bsel >= s.N;
    const int gpb = per * kScatterOneGroups;
    dim3 grid((unsigned)((s.N / 4 + 1 + gpb - 1) / gpb), s.BH);   // k_scatter_one: groups u0 = 0, 4, ..., <= N
    dim3 g8((unsigned)((s.N / 8 + 1 + per - 1) / per), s.BH);     // k_scatter_hi: units u0 = 0, 8, ..., <= N
    dim3 glo((unsigned)((s.S + per - 1) / per), s.BH);            // k_scatter_lo: gathered rows
#define LH_SC(D, LM, P2)                                                                             \
  do {                                                                                               \
    if (one) {                                                                                       \
      lh::launch(k_scatter_one<D, LM, P2>, grid, 256, 0, st, s, slot, ot, o, o_dtype);               \
    } else {                                                                                         \
      lh::launch(k_scatter_hi<D, LM>, g8, 256, 0, st, s, slot, ot, o, o_dtype);                     \
      lh::launch(k_scatter_lo<D, LM>, glo, 256, 0, st, s, slot, coords, ot, o, o_dtype);             \
    }                                                                                                \
  } while (0)
#define LH_SCL(D, P2)                   \
  do {                                  \
    if (s.L <= 3) LH_SC(D, 3, P2);      \
    else if (s.L == 4) LH_SC(D, 4, P2); \
    else if (s.L == 5) LH_SC(D, 5, P2); \
    else LH_SC(D, kMaxL, P2);           \
  } while (0)
    if (s.d == 128) {
      if (s.p == 2) LH_SCL(128, true);
      else LH_SCL(128, false);
    } else {
      if (s.p == 2) LH_SCL(64, true);
      else LH_SCL(64, false);
    }
#undef LH_SCL
#undef LH_SC
  } else {
    dim3 grid((unsigned)((s.N + 1 + per - 1) / per), s.BH);       // u = 0 .. N
    if (s.d == 128) lh::launch(k_scatter<128>, grid, 256, 0, st, s, slot, ot, o, o_dtype);
    else lh::launch(k_scatter<64>, grid, 256, 0, st, s, slot, ot, o, o_dtype);
  }
  return hipGetLastError();
}

hipError_t launch_scatter_bwd(const Shape &s, const void *dout, int dout_dtype, const int *slot, const int *coords,
                              const float *ot, const float *lse, float *dot32, uint16_t *dotb, float *delta,
                              float *rows, hipStream_t st) {
  const bool bf = s.io == LH_BF16;
  // position-major walk: four or more levels (where k_scatter_bwd's re-reads of
  // dO dominate), p = 2 or 4, and the coarsest range fits a work-group's span
  if ((s.p == 2 || s.p == 4) && s.L >= 4) {
    // rows per row group: the largest p^a <= 16 (4 at four levels, measured
    // faster: more, shorter row groups) with a <= L - 1
    int gw = 1, a = 0;
    while (a + 1 < s.L && gw * s.p <= (s.L == 4 ? 4 : 16)) {
      gw *= s.p;
      ++a;
    }
    const int rg = 256 / (s.d / 8);
    const long long span = (long long)rg * gw;
    if (gw > 1 && s.pw[s.L - 1] <= span && s.L - 1 - a <= kWalkCoarse) {
      const int nwg = (int)((s.N + 1 + span - 1) / span);
      dim3 grid((unsigned)nwg, s.BH);
      dim3 gd((unsigned)(((bf ? s.Sv : s.S) + rg - 1) / rg), s.BH);
#define LH_SW(D, B, G, LG)                                                                                     \
  do {                                                                                                          \
    lh::launch(k_scatter_bwd_walk<D, B, G, LG>, grid, 256, 0, st, s, dout, dout_dtype, slot, dot32, dotb);     \
    lh::launch(k_scatter_delta<D, B>, gd, 256, 0, st, s, ot, (const float *)dot32, dotb, delta, lse, rows);   \
  } while (0)
#define LH_SWG(D, B)                          \
  do {                                        \
    if (s.p == 4) {                           \
      if (gw == 16) LH_SW(D, B, 16, 2);       \
      else LH_SW(D, B, 4, 2);                 \
    } else {                                  \
      if (gw == 16) LH_SW(D, B, 16, 1);       \
      else if (gw == 8) LH_SW(D, B, 8, 1);    \
      else if (gw == 4) LH_SW(D, B, 4, 1);    \
      else LH_SW(D, B, 2, 1);                 \
    }                                         \
  } while (0)
      if (s.d == 128) {
        if (bf) LH_SWG(128, true);
        else LH_SWG(128, false);
      } else {
        if (bf) LH_SWG(64, true);
        else LH_SWG(64, false);
      }
#undef LH_SWG
#undef LH_SW
      return hipGetLastError();
    }
  }
  // bf16 mode also writes the zero padding rows / columns up to Sv (a multiple of 64)
  const int spb = 256 / (s.d / 8);
  dim3 grid((unsigned)(((s.io == LH_BF16 ? s.Sv : s.S) + spb - 1) / spb), s.BH);
#define LH_SB(D, B) lh::launch(k_scatter_bwd<D, B>, grid, 256, 0, st, s, dout, dout_dtype, coords, ot, dot32, dotb, delta, lse, rows)
  if (s.d == 128) {
    if (bf) LH_SB(128, true);
    else LH_SB(128, false);
  } else {
    if (bf) LH_SB(64, true);
    else LH_SB(64, false);
  }
#undef LH_SB
  return hipGetLastError();
}

hipError_t launch_pool_bwd(const Shape &s, const int *slot, const float *dqt, const float *dkt, const float *dvt,
                           void *dq, void *dk, void *dv, int grad_dtype, hipStream_t st) {
  const int per = 256 / (s.d / 8);
  if (s.p >= 4 && (s.p & (s.p - 1)) == 0) {
    dim3 grid((unsigned)(((s.N + 3) / 4 + per - 1) / per), s.BH, 3);
#define LH_PB(D, LM) lh::launch(k_pool_bwd_g4<D, LM>, grid, 256, 0, st, s, slot, dqt, dkt, dvt, dq, dk, dv, grad_dtype)
    if (s.d == 128) {
      if (s.L <= 3) LH_PB(128, 3);
      else if (s.L == 4) LH_PB(128, 4);
      else if (s.L == 5) LH_PB(128, 5);
      else LH_PB(128, kMaxL);
    } else {
      if (s.L <= 3) LH_PB(64, 3);
      else if (s.L == 4) LH_PB(64, 4);
      else if (s.L == 5) LH_PB(64, 5);
      else LH_PB(64, kMaxL);
    }
#undef LH_PB
  } else {
    const long long n = (long long)s.N * (s.d / 8);
    dim3 grid((unsigned)((n + 255) / 256), s.BH);
    if (s.d == 128) lh::launch(k_pool_bwd<128>, grid, 256, 0, st, s, slot, dqt, dkt, dvt, dq, dk, dv, grad_dtype);
    else lh::launch(k_pool_bwd<64>, grid, 256, 0, st, s, slot, dqt, dkt, dvt, dq, dk, dv, grad_dtype);
  }
  return hipGetLastError();
}

}  // namespace lh
