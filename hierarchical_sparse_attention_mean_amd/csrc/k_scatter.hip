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

template <int D>
__global__ __launch_bounds__(256) void k_scatter(Shape s, const int *__restrict__ slot, const float *__restrict__ ot,
                                                 void *__restrict__ o, int o_dtype) {
  constexpr int C4 = D / 4;   // float4 chunks per row
  const int h = blockIdx.y;
  const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (long long)s.N * C4) return;
  const int t = (int)(idx / C4);
  const int c = (int)(idx % C4);
  const int *sl = slot + (long long)h * s.P;
  const float4 *ob = reinterpret_cast<const float4 *>(ot + (long long)h * s.S * D);
  long long a0 = 0, a1 = 0, a2 = 0, a3 = 0;
  for (int l = 0; l < s.L; ++l) {
    const int i = (t + 1) / s.pw[l] - 1;
    if (i < 0) break;   // coarser levels start even later
    const int m = sl[s.off[l] + i];
    if (m < 0) continue;
    const float4 x = ob[(long long)m * C4 + c];
    a0 += to_fixed(x.x);
    a1 += to_fixed(x.y);
    a2 += to_fixed(x.z);
    a3 += to_fixed(x.w);
  }
  const float r0 = from_fixed(a0), r1 = from_fixed(a1), r2 = from_fixed(a2), r3 = from_fixed(a3);
  const long long off = ((long long)h * s.N + t) * D + c * 4;
  if (o_dtype == LH_BF16) {
    uint2 w;
    w.x = (unsigned)f32_to_bf16_rne(r0) | ((unsigned)f32_to_bf16_rne(r1) << 16);
    w.y = (unsigned)f32_to_bf16_rne(r2) | ((unsigned)f32_to_bf16_rne(r3) << 16);
    *reinterpret_cast<uint2 *>(reinterpret_cast<uint16_t *>(o) + off) = w;
  } else {
    *reinterpret_cast<float4 *>(reinterpret_cast<float *>(o) + off) = make_float4(r0, r1, r2, r3);
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

template <int D>
__global__ __launch_bounds__(256) void k_pool_bwd(Shape s, const int *__restrict__ slot, const float *__restrict__ dqt,
                                                  const float *__restrict__ dkt, const float *__restrict__ dvt,
                                                  void *__restrict__ dq, void *__restrict__ dk, void *__restrict__ dv,
                                                  int grad_dtype) {
  constexpr int C4 = D / 4;
  const int h = blockIdx.y;
  const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (long long)s.N * C4) return;
  const int t = (int)(idx / C4);
  const int c = (int)(idx % C4);
  const int *sl = slot + (long long)h * s.P;
  const long long hs = (long long)h * s.S;
  float4 aq = make_float4(0.f, 0.f, 0.f, 0.f), ak = aq, av = aq;
  for (int l = 0; l < s.L; ++l) {
    const int m = sl[s.off[l] + t / s.pw[l]];
    if (m < 0) continue;
    const float inv = 1.f / (float)s.pw[l];
    const long long ro = (hs + m) * D + c * 4;
    const float4 x = *reinterpret_cast<const float4 *>(dqt + ro);
    const float4 y = *reinterpret_cast<const float4 *>(dkt + ro);
    const float4 z = *reinterpret_cast<const float4 *>(dvt + ro);
    aq.x = fmaf(x.x, inv, aq.x); aq.y = fmaf(x.y, inv, aq.y); aq.z = fmaf(x.z, inv, aq.z); aq.w = fmaf(x.w, inv, aq.w);
    ak.x = fmaf(y.x, inv, ak.x); ak.y = fmaf(y.y, inv, ak.y); ak.z = fmaf(y.z, inv, ak.z); ak.w = fmaf(y.w, inv, ak.w);
    av.x = fmaf(z.x, inv, av.x); av.y = fmaf(z.y, inv, av.y); av.z = fmaf(z.z, inv, av.z); av.w = fmaf(z.w, inv, av.w);
  }
  const long long off = ((long long)h * s.N + t) * D + c * 4;
  if (grad_dtype == LH_BF16) {
    const float4 *src[3] = {&aq, &ak, &av};
    void *dst[3] = {dq, dk, dv};
    for (int u = 0; u < 3; ++u) {
      uint2 w;
      w.x = (unsigned)f32_to_bf16_rne(src[u]->x) | ((unsigned)f32_to_bf16_rne(src[u]->y) << 16);
      w.y = (unsigned)f32_to_bf16_rne(src[u]->z) | ((unsigned)f32_to_bf16_rne(src[u]->w) << 16);
      *reinterpret_cast<uint2 *>(reinterpret_cast<uint16_t *>(dst[u]) + off) = w;
    }
  } else {
    *reinterpret_cast<float4 *>(reinterpret_cast<float *>(dq) + off) = aq;
    *reinterpret_cast<float4 *>(reinterpret_cast<float *>(dk) + off) = ak;
    *reinterpret_cast<float4 *>(reinterpret_cast<float *>(dv) + off) = av;
  }
}

}  // namespace

hipError_t launch_scatter(const Shape &s, const int *slot, const float *ot, void *o, int o_dtype, hipStream_t st) {
  const long long n = (long long)s.N * (s.d / 4);
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
  const long long n = (long long)s.N * (s.d / 4);
  dim3 grid((unsigned)((n + 255) / 256), s.BH);
  if (s.d == 128) k_pool_bwd<128><<<grid, 256, 0, st>>>(s, slot, dqt, dkt, dvt, dq, dk, dv, grad_dtype);
  else k_pool_bwd<64><<<grid, 256, 0, st>>>(s, slot, dqt, dkt, dvt, dq, dk, dv, grad_dtype);
  return hipGetLastError();
}

}  // namespace lh
