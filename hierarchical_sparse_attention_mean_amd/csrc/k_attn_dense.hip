// Row terms of the dense causal attention backward.
//
// "Long Context Pre-Training with Lighthouse Attention", Sec. 3.1 (Eq. 1) and
// Sec. 3.2: the attention of stage (iii) is plain causal softmax attention, so
// on full sequences (the dense baseline, S = N) its backward is the textbook
// one.  With P recomputed from the forward's LSE, the softmax-backward row term
// is delta_m = sum_d dO[m][d] O[m][d].  This kernel forms it (4 lanes per row,
// each D/4 columns, then two xor exchanges) and writes either the pair
// (LSE log2(e), delta) per row that the bf16 MFMA backward loads with each
// query tile, or delta alone for the fp32 kernels.
#include "lh_internal.h"

namespace lh {

namespace {

__device__ __forceinline__ float4 load4(const void *p, long long off, bool bf16) {
  if (bf16) {
    const uint2 w = *reinterpret_cast<const uint2 *>(reinterpret_cast<const uint16_t *>(p) + off);
    return make_float4(__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xFFFF0000u), __uint_as_float(w.y << 16),
                       __uint_as_float(w.y & 0xFFFF0000u));
  }
  return *reinterpret_cast<const float4 *>(reinterpret_cast<const float *>(p) + off);
}

template <int D>
__global__ __launch_bounds__(256) void k_attn_rowstats(int S, const void *__restrict__ dout, int dout_bf16,
                                                       const float *__restrict__ o, const float *__restrict__ lse,
                                                       float *__restrict__ pairs, float *__restrict__ delta) {
  constexpr int DP = D / 4;
  const int h = blockIdx.y;
  const int m = blockIdx.x * 64 + (threadIdx.x >> 2);
  const int part = threadIdx.x & 3;
  float dl = 0.f;
  if (m < S) {
    const long long base = ((long long)h * S + m) * D + part * DP;
#pragma unroll
    for (int e = 0; e < DP; e += 4) {
      const float4 g = load4(dout, base + e, dout_bf16 != 0);
      const float4 x = *reinterpret_cast<const float4 *>(o + base + e);
      dl = fmaf(g.x, x.x, dl);
      dl = fmaf(g.y, x.y, dl);
      dl = fmaf(g.z, x.z, dl);
      dl = fmaf(g.w, x.w, dl);
    }
  }
  dl += __shfl_xor(dl, 1);
  dl += __shfl_xor(dl, 2);
  if (m < S && part == 0) {
    const long long r = (long long)h * S + m;
    if (pairs) *reinterpret_cast<float2 *>(pairs + 2 * r) = make_float2(lse[r] * 1.4426950408889634f, dl);
    else delta[r] = dl;
  }
}

}  // namespace

hipError_t launch_attn_rowstats(int d, int BH, int S, const void *dout, int dout_bf16, const float *o,
                                const float *lse, float *pairs, float *delta, hipStream_t st) {
  dim3 grid((unsigned)((S + 63) / 64), BH);
  if (d == 128) lh::launch(k_attn_rowstats<128>, grid, 256, 0, st, S, dout, dout_bf16, o, lse, pairs, delta);
  else lh::launch(k_attn_rowstats<64>, grid, 256, 0, st, S, dout, dout_bf16, o, lse, pairs, delta);
  return hipGetLastError();
}

}  // namespace lh
