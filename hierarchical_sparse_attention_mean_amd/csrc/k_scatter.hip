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
// Adjoints (Sec. 3.2: gradients flow through scatter, attention, gather and
// pool; the selection is frozen):
//   k_scatter_bwd  dO~_m = sum of dO_t over the scatter range of entry m;
//   k_pool_bwd     dX_t = sum_l [entry (l, floor(t/p^l)) selected] dX~_slot / p^l
//                  for X in {Q, K, V} (gather adjoint fused with pool adjoint).
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

// One thread per 8 consecutive elements of an output row (16-byte stores).  The
// slots of the entries that reach position t at each level are looked up
// first, then their rows are read.  Fixed-point sum: sum over the levels of
// RNE(x 2^32) as an integer, converted back with one rounding.  RNE(x 2^32) is
// an integer that fp32 rintf gives exactly; while every |x| < 2^18 each term is
// below 2^50 in magnitude and the sum of at most kMaxL of them is exact in
// fp64, which is then the same integer as the int64 sum (and (double)int64
// gives the same value): that path is taken unless some |x| >= 2^18, where the
// int64 sum is formed instead.
template <int D>
__global__ __launch_bounds__(256) void k_scatter(Shape s, const int *__restrict__ slot, const float *__restrict__ ot,
                                                 void *__restrict__ o, int o_dtype) {
  constexpr int C8 = D / 8;   // 8-element chunks per row
  const int h = blockIdx.y;
  const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (long long)s.N * C8) return;
  const int t = (int)(idx / C8);
  const int c = (int)(idx % C8);
  const int *sl = slot + (long long)h * s.P;
  const float *ob = ot + (long long)h * s.S * D + c * 8;
  int m[kMaxL];
#pragma unroll
  for (int l = 0; l < kMaxL; ++l) {
    m[l] = -1;
    if (l < s.L) {
      const int i = (t + 1) / s.pw[l] - 1;
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
    const float4 x0 = *reinterpret_cast<const float4 *>(ob + (long long)m[l] * D);
    const float4 x1 = *reinterpret_cast<const float4 *>(ob + (long long)m[l] * D + 4);
    const float x[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      big |= !(fabsf(x[e]) < 262144.f);
      a[e] += (double)rintf(x[e] * 4294967296.0f);
    }
  }
  float r[8];
  if (!big) {
#pragma unroll
    for (int e = 0; e < 8; ++e) r[e] = (float)(a[e] * 2.3283064365386963e-10);
  } else {
    long long b[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int l = 0; l < kMaxL; ++l) {
      if (m[l] < 0) continue;
      for (int e = 0; e < 8; ++e) b[e] += to_fixed(ob[(long long)m[l] * D + e]);
    }
    for (int e = 0; e < 8; ++e) r[e] = from_fixed(b[e]);
  }
  const long long off = ((long long)h * s.N + t) * D + c * 8;
  if (o_dtype == LH_BF16) {
    uint4 w;
    w.x = (unsigned)f32_to_bf16_rne(r[0]) | ((unsigned)f32_to_bf16_rne(r[1]) << 16);
    w.y = (unsigned)f32_to_bf16_rne(r[2]) | ((unsigned)f32_to_bf16_rne(r[3]) << 16);
    w.z = (unsigned)f32_to_bf16_rne(r[4]) | ((unsigned)f32_to_bf16_rne(r[5]) << 16);
    w.w = (unsigned)f32_to_bf16_rne(r[6]) | ((unsigned)f32_to_bf16_rne(r[7]) << 16);
    *reinterpret_cast<uint4 *>(reinterpret_cast<uint16_t *>(o) + off) = w;
  } else {
    float *of = reinterpret_cast<float *>(o) + off;
    *reinterpret_cast<float4 *>(of) = make_float4(r[0], r[1], r[2], r[3]);
    *reinterpret_cast<float4 *>(of + 4) = make_float4(r[4], r[5], r[6], r[7]);
  }
}

__device__ __forceinline__ float4 ld4(const void *p, long long off, int dtype) {
  if (dtype == LH_BF16) {
    const uint2 w = *reinterpret_cast<const uint2 *>(reinterpret_cast<const uint16_t *>(p) + off);
    return make_float4(__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xFFFF0000u), __uint_as_float(w.y << 16),
                       __uint_as_float(w.y & 0xFFFF0000u));
  }
  return *reinterpret_cast<const float4 *>(reinterpret_cast<const float *>(p) + off);
}

// One work-group per 64 consecutive slots; 4 lanes per slot, each summing D/4
// columns of dO over the entry's scatter range (t ascending), then
//   delta_m = sum_d dO~[m][d] * O~[m][d]   (the softmax-backward row term)
// with dO~ as the attention backward will read it (bf16-rounded in bf16 mode).
// fp32 mode writes dO~ in fp32 and delta; bf16 mode writes dO~ in bf16
// (row-major, head stride Sv, zero rows S..Sv-1) and the per-row pair
// (LSE log2(e), delta) that the MFMA backward loads with each query tile
// (zeros on the padding rows).
template <int D, bool BF16>
__global__ __launch_bounds__(256) void k_scatter_bwd(Shape s, const void *__restrict__ dout, int dout_dtype,
                                                     const int *__restrict__ coords, const float *__restrict__ ot,
                                                     float *__restrict__ dot32, uint16_t *__restrict__ dotb,
                                                     float *__restrict__ delta, const float *__restrict__ lse,
                                                     float *__restrict__ rows) {
  constexpr int DP = D / 4;
  const int h = blockIdx.y;
  const int m0 = blockIdx.x * 64;
  const int r = threadIdx.x >> 2;
  const int part = threadIdx.x & 3;
  const int m = m0 + r;
  const bool active = m < s.S;   // rows S..Sv-1 are written as zeros (bf16 mode)
  float acc[DP];
#pragma unroll
  for (int e = 0; e < DP; ++e) acc[e] = 0.f;
  if (active) {
    const int f = coords[(long long)h * s.S + m];
    int l = 0;
    while (l + 1 < s.L && f >= s.off[l + 1]) ++l;
    const int i = f - s.off[l];
    const int lo = (i + 1) * s.pw[l] - 1;
    const int hi = min(s.N - 1, lo + s.pw[l] - 1);
    for (int t = lo; t <= hi; ++t) {
      const long long base = ((long long)h * s.N + t) * D + part * DP;
#pragma unroll
      for (int e = 0; e < DP; e += 4) {
        const float4 x = ld4(dout, base + e, dout_dtype);
        acc[e] += x.x;
        acc[e + 1] += x.y;
        acc[e + 2] += x.z;
        acc[e + 3] += x.w;
      }
    }
  }
  const long long row = ((long long)h * s.S + m) * D + part * DP;
  const long long rowv = ((long long)h * s.Sv + m) * D + part * DP;   // bf16 dO~: head stride Sv
  float dl = 0.f;
  uint16_t hb[BF16 ? DP : 1];   // dO~ as the attention backward reads it (bf16 mode)
  if constexpr (BF16) {
#pragma unroll
    for (int e = 0; e < DP; ++e) {
      hb[e] = f32_to_bf16_rne(acc[e]);
      acc[e] = bf16_to_f32(hb[e]);
    }
  }
  if (active) {
#pragma unroll
    for (int e = 0; e < DP; e += 4) {
      const float4 o4 = *reinterpret_cast<const float4 *>(ot + row + e);
      dl = fmaf(acc[e], o4.x, dl);
      dl = fmaf(acc[e + 1], o4.y, dl);
      dl = fmaf(acc[e + 2], o4.z, dl);
      dl = fmaf(acc[e + 3], o4.w, dl);
    }
  }
  dl += __shfl_xor(dl, 1);
  dl += __shfl_xor(dl, 2);
  if constexpr (BF16) {
    if (m < s.Sv) {
#pragma unroll
      for (int e = 0; e < DP; e += 8) {
        uint4 w;
        w.x = (unsigned)hb[e] | ((unsigned)hb[e + 1] << 16);
        w.y = (unsigned)hb[e + 2] | ((unsigned)hb[e + 3] << 16);
        w.z = (unsigned)hb[e + 4] | ((unsigned)hb[e + 5] << 16);
        w.w = (unsigned)hb[e + 6] | ((unsigned)hb[e + 7] << 16);
        *reinterpret_cast<uint4 *>(dotb + rowv + e) = w;
      }
    }
  }
  if constexpr (BF16) {
    if (part == 0 && m < s.Sv)
      *reinterpret_cast<float2 *>(rows + 2 * ((long long)h * s.Sv + m)) =
          active ? make_float2(lse[(long long)h * s.S + m] * 1.4426950408889634f, dl) : make_float2(0.f, 0.f);
  }
  if (active) {
    if constexpr (!BF16) {
      if (part == 0) delta[(long long)h * s.S + m] = dl;
#pragma unroll
      for (int e = 0; e < DP; e += 4)
        *reinterpret_cast<float4 *>(dot32 + row + e) = make_float4(acc[e], acc[e + 1], acc[e + 2], acc[e + 3]);
    }
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
      const float4 x0 = *reinterpret_cast<const float4 *>(src[u] + ro);
      const float4 x1 = *reinterpret_cast<const float4 *>(src[u] + ro + 4);
      const float x[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[u][e] = fmaf(x[e], inv, acc[u][e]);
    }
  }
  const long long off = ((long long)h * s.N + t) * D + c * 8;
  void *dst[3] = {dq, dk, dv};
#pragma unroll
  for (int u = 0; u < 3; ++u) {
    if (grad_dtype == LH_BF16) {
      uint4 w;
      w.x = (unsigned)f32_to_bf16_rne(acc[u][0]) | ((unsigned)f32_to_bf16_rne(acc[u][1]) << 16);
      w.y = (unsigned)f32_to_bf16_rne(acc[u][2]) | ((unsigned)f32_to_bf16_rne(acc[u][3]) << 16);
      w.z = (unsigned)f32_to_bf16_rne(acc[u][4]) | ((unsigned)f32_to_bf16_rne(acc[u][5]) << 16);
      w.w = (unsigned)f32_to_bf16_rne(acc[u][6]) | ((unsigned)f32_to_bf16_rne(acc[u][7]) << 16);
      *reinterpret_cast<uint4 *>(reinterpret_cast<uint16_t *>(dst[u]) + off) = w;
    } else {
      float *of = reinterpret_cast<float *>(dst[u]) + off;
      *reinterpret_cast<float4 *>(of) = make_float4(acc[u][0], acc[u][1], acc[u][2], acc[u][3]);
      *reinterpret_cast<float4 *>(of + 4) = make_float4(acc[u][4], acc[u][5], acc[u][6], acc[u][7]);
    }
  }
}

}  // namespace

hipError_t launch_scatter(const Shape &s, const int *slot, const float *ot, void *o, int o_dtype, hipStream_t st) {
  const long long n = (long long)s.N * (s.d / 8);
  dim3 grid((unsigned)((n + 255) / 256), s.BH);
  if (s.d == 128) k_scatter<128><<<grid, 256, 0, st>>>(s, slot, ot, o, o_dtype);
  else k_scatter<64><<<grid, 256, 0, st>>>(s, slot, ot, o, o_dtype);
  return hipGetLastError();
}

hipError_t launch_scatter_bwd(const Shape &s, const void *dout, int dout_dtype, const int *coords, const float *ot,
                              const float *lse, float *dot32, uint16_t *dotb, float *delta, float *rows,
                              hipStream_t st) {
  // bf16 mode also writes the zero padding rows / columns up to Sv (a multiple of 64)
  dim3 grid((unsigned)(((s.io == LH_BF16 ? s.Sv : s.S) + 63) / 64), s.BH);
  const bool bf = s.io == LH_BF16;
#define LH_SB(D, B) k_scatter_bwd<D, B><<<grid, 256, 0, st>>>(s, dout, dout_dtype, coords, ot, dot32, dotb, delta, lse, rows)
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
  const long long n = (long long)s.N * (s.d / 8);
  dim3 grid((unsigned)((n + 255) / 256), s.BH);
  if (s.d == 128) k_pool_bwd<128><<<grid, 256, 0, st>>>(s, slot, dqt, dkt, dvt, dq, dk, dv, grad_dtype);
  else k_pool_bwd<64><<<grid, 256, 0, st>>>(s, slot, dqt, dkt, dvt, dq, dk, dv, grad_dtype);
  return hipGetLastError();
}

}  // namespace lh
