// Causal softmax attention over the gathered sub-sequence, fp32 vector-ALU
// kernels (the LH_F32 path): forward with online softmax, and the atomic-free
// backward (query-stationary dQ, key-stationary dK/dV).
//
// "Long Context Pre-Training with Lighthouse Attention", Sec. 3.5, Eq. (9): the
// gathered rows are attended with standard masked softmax attention (Sec. 3.1,
// Eq. 1, scale 1/sqrt(d)); after the topological sort the mask is the plain
// causal mask, row m sees rows m' <= m.
//
// Mapping: 64 query (or key) rows per work-group, 4 lanes per row, each lane
// owning D/4 consecutive dimensions; K/V (or Q/dO) tiles of 32 rows are staged
// in LDS as fp32.  Logits use exp2 with log2(e) folded into the scale.
#include "lh_internal.h"

namespace lh {

namespace {

constexpr int BM = 64;
constexpr int BN = 32;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

template <typename T, int D>
__device__ __forceinline__ void stage_rows(float (*dst)[D + 4], const T *src, long long row0, int nrows_valid) {
  // BN rows x D elements, 256 threads
  for (int idx = threadIdx.x; idx < BN * D; idx += 256) {
    const int r = idx / D, c = idx % D;
    dst[r][c] = (r < nrows_valid) ? IO<T>::ld(src, (row0 + r) * D + c) : 0.f;
  }
}

template <typename T, int D>
__global__ __launch_bounds__(256) void k_attn_fwd_valu(int S, int Sq, const T *__restrict__ qt, const T *__restrict__ kt,
                                                       const T *__restrict__ vt, float *__restrict__ ot,
                                                       float *__restrict__ lse) {
  constexpr int DP = D / 4;
  __shared__ float ks[BN][D + 4];
  __shared__ float vs[BN][D + 4];
  const int h = blockIdx.y;
  const int nqb = gridDim.x;
  const int qb = nqb - 1 - blockIdx.x;   // longest rows first
  const int q0 = qb * BM;
  const int r = threadIdx.x >> 2;
  const int part = threadIdx.x & 3;
  const int qi = q0 + r;
  const bool active = qi < S;
  const long long hb = (long long)h * S;    // O~, LSE, dO~, gradients: S rows per head
  const long long hq = (long long)h * Sq;   // gathered Q~, K~, V~: Sq rows per head
  const float scale = kLog2e / sqrtf((float)D);
  float qv[DP], o[DP];
#pragma unroll
  for (int e = 0; e < DP; ++e) {
    qv[e] = active ? IO<T>::ld(qt, (hq + qi) * D + part * DP + e) * scale : 0.f;
    o[e] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  const int kend = min(S, q0 + BM);
  for (int k0 = 0; k0 < kend; k0 += BN) {
    __syncthreads();
    stage_rows<T, D>(ks, kt + hq * D, k0, min(BN, S - k0));
    stage_rows<T, D>(vs, vt + hq * D, k0, min(BN, S - k0));
    __syncthreads();
    float sc[BN];
    float mt = m;
#pragma unroll
    for (int jj = 0; jj < BN; ++jj) {
      float dot = 0.f;
#pragma unroll
      for (int e = 0; e < DP; ++e) dot = fmaf(qv[e], ks[jj][part * DP + e], dot);
      dot += __shfl_xor(dot, 1);
      dot += __shfl_xor(dot, 2);
      sc[jj] = (k0 + jj <= qi) ? dot : -INFINITY;
      mt = fmaxf(mt, sc[jj]);
    }
    if (!active || mt == -INFINITY) continue;
    const float alpha = exp2f(m - mt);
    l *= alpha;
#pragma unroll
    for (int e = 0; e < DP; ++e) o[e] *= alpha;
#pragma unroll
    for (int jj = 0; jj < BN; ++jj) {
      const float pj = exp2f(sc[jj] - mt);
      l += pj;
#pragma unroll
      for (int e = 0; e < DP; ++e) o[e] = fmaf(pj, vs[jj][part * DP + e], o[e]);
    }
    m = mt;
  }
  if (!active) return;
  const float inv = 1.f / l;
#pragma unroll
  for (int e = 0; e < DP; ++e) ot[(hb + qi) * D + part * DP + e] = o[e] * inv;
  if (part == 0 && lse) lse[hb + qi] = (m + log2f(l)) * kLn2;
}

// dQ~ (query-stationary): dq_m = scale * sum_{m' <= m} P_mm' (dP_mm' - delta_m) K_m'
template <typename T, int D>
__global__ __launch_bounds__(256) void k_attn_dq_valu(int S, int Sq, const T *__restrict__ qt, const T *__restrict__ kt,
                                                      const T *__restrict__ vt, const float *__restrict__ lse,
                                                      const float *__restrict__ dot, const float *__restrict__ delta,
                                                      float *__restrict__ dqt) {
  constexpr int DP = D / 4;
  __shared__ float ks[BN][D + 4];
  __shared__ float vs[BN][D + 4];
  const int h = blockIdx.y;
  const int qb = gridDim.x - 1 - blockIdx.x;
  const int q0 = qb * BM;
  const int r = threadIdx.x >> 2;
  const int part = threadIdx.x & 3;
  const int qi = q0 + r;
  const bool active = qi < S;
  const long long hb = (long long)h * S;    // O~, LSE, dO~, gradients: S rows per head
  const long long hq = (long long)h * Sq;   // gathered Q~, K~, V~: Sq rows per head
  const float scale = 1.f / sqrtf((float)D);
  float qv[DP], gv[DP], acc[DP];
#pragma unroll
  for (int e = 0; e < DP; ++e) {
    qv[e] = active ? IO<T>::ld(qt, (hq + qi) * D + part * DP + e) * (scale * kLog2e) : 0.f;
    gv[e] = active ? dot[(hb + qi) * D + part * DP + e] : 0.f;
    acc[e] = 0.f;
  }
  const float lse2 = active ? lse[hb + qi] * kLog2e : 0.f;
  const float dl = active ? delta[hb + qi] : 0.f;
  const int kend = min(S, q0 + BM);
  for (int k0 = 0; k0 < kend; k0 += BN) {
    __syncthreads();
    stage_rows<T, D>(ks, kt + hq * D, k0, min(BN, S - k0));
    stage_rows<T, D>(vs, vt + hq * D, k0, min(BN, S - k0));
    __syncthreads();
#pragma unroll 4
    for (int jj = 0; jj < BN; ++jj) {
      float s2 = 0.f, dp = 0.f;
#pragma unroll
      for (int e = 0; e < DP; ++e) {
        s2 = fmaf(qv[e], ks[jj][part * DP + e], s2);
        dp = fmaf(gv[e], vs[jj][part * DP + e], dp);
      }
      s2 += __shfl_xor(s2, 1);
      s2 += __shfl_xor(s2, 2);
      dp += __shfl_xor(dp, 1);
      dp += __shfl_xor(dp, 2);
      const float pj = (k0 + jj <= qi) ? exp2f(s2 - lse2) : 0.f;
      const float ds = pj * (dp - dl);
#pragma unroll
      for (int e = 0; e < DP; ++e) acc[e] = fmaf(ds, ks[jj][part * DP + e], acc[e]);
    }
  }
  if (!active) return;
#pragma unroll
  for (int e = 0; e < DP; ++e) dqt[(hb + qi) * D + part * DP + e] = acc[e] * scale;
}

// dK~, dV~ (key-stationary): dv_j = sum_{m >= j} P_mj dO~_m ;
// dk_j = scale * sum_{m >= j} P_mj (dP_mj - delta_m) Q~_m
template <typename T, int D>
__global__ __launch_bounds__(256) void k_attn_dkv_valu(int S, int Sq, const T *__restrict__ qt, const T *__restrict__ kt,
                                                       const T *__restrict__ vt, const float *__restrict__ lse,
                                                       const float *__restrict__ dot, const float *__restrict__ delta,
                                                       float *__restrict__ dkt, float *__restrict__ dvt) {
  constexpr int DP = D / 4;
  __shared__ float qs[BN][D + 4];
  __shared__ float gs[BN][D + 4];
  __shared__ float ls[BN], dls[BN];
  const int h = blockIdx.y;
  const int kb = blockIdx.x;   // key blocks near the start see the most queries
  const int j0 = kb * BM;
  const int r = threadIdx.x >> 2;
  const int part = threadIdx.x & 3;
  const int kj = j0 + r;
  const bool active = kj < S;
  const long long hb = (long long)h * S;    // O~, LSE, dO~, gradients: S rows per head
  const long long hq = (long long)h * Sq;   // gathered Q~, K~, V~: Sq rows per head
  const float scale = 1.f / sqrtf((float)D);
  float kv[DP], vv[DP], adk[DP], adv[DP];
#pragma unroll
  for (int e = 0; e < DP; ++e) {
    kv[e] = active ? IO<T>::ld(kt, (hq + kj) * D + part * DP + e) * (scale * kLog2e) : 0.f;
    vv[e] = active ? IO<T>::ld(vt, (hq + kj) * D + part * DP + e) : 0.f;
    adk[e] = adv[e] = 0.f;
  }
  for (int m0 = j0; m0 < S; m0 += BN) {
    __syncthreads();
    stage_rows<T, D>(qs, qt + hq * D, m0, min(BN, S - m0));
    for (int idx = threadIdx.x; idx < BN * D; idx += 256) {
      const int rr = idx / D, c = idx % D;
      gs[rr][c] = (m0 + rr < S) ? dot[(hb + m0 + rr) * D + c] : 0.f;
    }
    if (threadIdx.x < BN) {
      const int mm = m0 + threadIdx.x;
      ls[threadIdx.x] = mm < S ? lse[hb + mm] * kLog2e : 0.f;
      dls[threadIdx.x] = mm < S ? delta[hb + mm] : 0.f;
    }
    __syncthreads();
#pragma unroll 4
    for (int ii = 0; ii < BN; ++ii) {
      float s2 = 0.f, dp = 0.f;
#pragma unroll
      for (int e = 0; e < DP; ++e) {
        s2 = fmaf(kv[e], qs[ii][part * DP + e], s2);
        dp = fmaf(vv[e], gs[ii][part * DP + e], dp);
      }
      s2 += __shfl_xor(s2, 1);
      s2 += __shfl_xor(s2, 2);
      dp += __shfl_xor(dp, 1);
      dp += __shfl_xor(dp, 2);
      const int mm = m0 + ii;
      const float pj = (mm >= kj && mm < S) ? exp2f(s2 - ls[ii]) : 0.f;
      const float ds = pj * (dp - dls[ii]);
#pragma unroll
      for (int e = 0; e < DP; ++e) {
        adv[e] = fmaf(pj, gs[ii][part * DP + e], adv[e]);
        adk[e] = fmaf(ds, qs[ii][part * DP + e], adk[e]);
      }
    }
  }
  if (!active) return;
#pragma unroll
  for (int e = 0; e < DP; ++e) {
    dkt[(hb + kj) * D + part * DP + e] = adk[e] * scale;
    dvt[(hb + kj) * D + part * DP + e] = adv[e];
  }
}

}  // namespace

hipError_t launch_attn_fwd_valu(int io, int d, int BH, int S, int Sq, const void *qt, const void *kt, const void *vt,
                                float *ot, float *lse, hipStream_t st) {
  dim3 grid((S + BM - 1) / BM, BH);
#define LH_FWD(T, D) lh::launch(k_attn_fwd_valu<T, D>, grid, 256, 0, st, S, Sq, (const T *)qt, (const T *)kt, (const T *)vt, ot, lse)
  if (io == LH_BF16) {
    if (d == 128) LH_FWD(uint16_t, 128);
    else LH_FWD(uint16_t, 64);
  } else {
    if (d == 128) LH_FWD(float, 128);
    else LH_FWD(float, 64);
  }
#undef LH_FWD
  return hipGetLastError();
}

hipError_t launch_attn_bwd_valu(int io, int d, int BH, int S, int Sq, const void *qt, const void *kt, const void *vt,
                                const float *ot, const float *lse, const float *dot, float *delta, float *dqt,
                                float *dkt, float *dvt, int part, hipStream_t st) {
  (void)ot;   // delta = rowsum(dO~ * O~) comes from the scatter adjoint
  dim3 grid((S + BM - 1) / BM, BH);
#define LH_BWD(T, D)                                                                                            \
  do {                                                                                                          \
    if (part == 0)                                                                                              \
      lh::launch(k_attn_dq_valu<T, D>, grid, 256, 0, st, S, Sq, (const T *)qt, (const T *)kt, (const T *)vt, lse, dot,     \
                                                 delta, dqt);                                                   \
    else                                                                                                        \
      lh::launch(k_attn_dkv_valu<T, D>, grid, 256, 0, st, S, Sq, (const T *)qt, (const T *)kt, (const T *)vt, lse, dot,    \
                                                  delta, dkt, dvt);                                             \
  } while (0)
  if (io == LH_BF16) {
    if (d == 128) LH_BWD(uint16_t, 128);
    else LH_BWD(uint16_t, 64);
  } else {
    if (d == 128) LH_BWD(float, 128);
    else LH_BWD(float, 64);
  }
#undef LH_BWD
  return hipGetLastError();
}

}  // namespace lh
