// Backward of the sub-sequence causal attention on bf16 MFMA (gfx950),
// atomic-free and deterministic.
//
// "Long Context Pre-Training with Lighthouse Attention", Sec. 3.2: gradients
// flow from the scattered output back through the dense sub-sequence attention
// (Eq. 9) into the gathered Q~, K~, V~; the selection is frozen.  With
// P = softmax(Q~ K~^T / sqrt(d) + causal) recomputed from the saved LSE,
// delta_m = rowsum(dO~ o O~) and dS = P o (dO~ V~^T - delta):
//   dV~ = P^T dO~,   dK~ = dS^T Q~ / sqrt(d),   dQ~ = dS K~ / sqrt(d).
//
// Two kernels, each owning its output rows (no floating-point atomics):
//   k_attn_bwd_dq    query-stationary: a wavefront holds 32 query rows of Q~ and
//                    dO~ as B operands; per key tile it forms S^T = K~ Q~^T and
//                    dP^T = V~ dO~^T (lane = one query), dS^T in registers, and
//                    accumulates dQ^T += K~^T dS^T with K~^T from LDS.
//   k_attn_bwd_dkdv  key-stationary: a wavefront holds 32 key rows of K~ and V~
//                    as B operands; per query tile it forms S = Q~ K~^T and
//                    dP = dO~ V~^T (lane = one key), and accumulates
//                    dV^T += dO~^T P and dK^T += Q~^T dS with the transposed
//                    query-side operands from LDS.
// The transposed operands (K~^T, Q~^T, dO~^T, row stride Sv) are written by the
// gather and by the scatter adjoint, so every LDS operand is read as rows.
#include "lh_internal.h"

namespace lh {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ bf16x8 lds_row8(const uint16_t *p) { return *reinterpret_cast<const bf16x8 *>(p); }

// two 4-element pieces 8 apart: the k-chunk mapping (h, j) -> 8 (j/4) + 4 h + j%4
__device__ __forceinline__ bf16x8 lds_split8(const uint16_t *p) {
  const bf16x4 lo = *reinterpret_cast<const bf16x4 *>(p);
  const bf16x4 hi = *reinterpret_cast<const bf16x4 *>(p + 8);
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// stage rows [r0, r0+R) of a [S][D] bf16 array into LDS with row stride LS
template <int R, int D, int LS>
__device__ __forceinline__ void stage_rows(uint16_t *dst, const uint16_t *src, int r0, int S) {
#pragma unroll
  for (int it = 0; it < (R * D) / (8 * 256); ++it) {
    const int idx = it * 256 + threadIdx.x;
    const int r = idx / (D / 8), cc = idx % (D / 8);
    uint4 val = make_uint4(0, 0, 0, 0);
    if (r0 + r < S) val = *reinterpret_cast<const uint4 *>(src + (long long)(r0 + r) * D + cc * 8);
    *reinterpret_cast<uint4 *>(&dst[r * LS + cc * 8]) = val;
  }
}

// stage columns [c0, c0+C) of a transposed [D][Sv] bf16 array into LDS [D][LS]
template <int C, int D, int LS>
__device__ __forceinline__ void stage_cols(uint16_t *dst, const uint16_t *src, int c0, int S, int Sv) {
#pragma unroll
  for (int it = 0; it < (C * D) / (8 * 256); ++it) {
    const int idx = it * 256 + threadIdx.x;
    const int r = idx / (C / 8), cc = idx % (C / 8);
    const int kk = c0 + cc * 8;
    uint4 val = make_uint4(0, 0, 0, 0);
    if (kk + 8 <= S) {
      val = *reinterpret_cast<const uint4 *>(src + (long long)r * Sv + kk);
    } else {
      uint16_t tmp[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) tmp[e] = (kk + e < S) ? src[(long long)r * Sv + kk + e] : (uint16_t)0;
      val = make_uint4(tmp[0] | (tmp[1] << 16), tmp[2] | (tmp[3] << 16), tmp[4] | (tmp[5] << 16),
                       tmp[6] | (tmp[7] << 16));
    }
    uint2 *d2 = reinterpret_cast<uint2 *>(&dst[r * LS + cc * 8]);
    d2[0] = make_uint2(val.x, val.y);
    d2[1] = make_uint2(val.z, val.w);
  }
}

template <int D>
__global__ __launch_bounds__(256, 2) void k_attn_bwd_dq(int S, int Sv, int BH, const uint16_t *__restrict__ qt,
                                                        const uint16_t *__restrict__ kt, const uint16_t *__restrict__ vt,
                                                        const uint16_t *__restrict__ ktt,
                                                        const uint16_t *__restrict__ dotb,
                                                        const float *__restrict__ lse, const float *__restrict__ delta,
                                                        float *__restrict__ dqt) {
  constexpr int BM = 128, BN = 64;
  constexpr int KC = D / 16, DB = D / 32;
  constexpr int KS = D + 8, TS = BN + 4;
  __shared__ __attribute__((aligned(16))) uint16_t ks[BN * KS];
  __shared__ __attribute__((aligned(16))) uint16_t vs[BN * KS];
  __shared__ __attribute__((aligned(16))) uint16_t kts[D * TS];
  const int nqb = (S + BM - 1) / BM;
  const int h = blockIdx.x % BH;
  const int qb = nqb - 1 - blockIdx.x / BH;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, ln = lane & 31, hf = lane >> 5;
  const int q0 = qb * BM, qw = q0 + 32 * w, qi = qw + ln;
  const long long hbS = (long long)h * S;
  const uint16_t *kh = kt + hbS * D;
  const uint16_t *vh = vt + hbS * D;
  const uint16_t *kth = ktt + (long long)h * D * Sv;
  bf16x8 qf[KC], gf[KC];
#pragma unroll
  for (int c = 0; c < KC; ++c) {
    if (qi < S) {
      qf[c] = *reinterpret_cast<const bf16x8 *>(qt + (hbS + qi) * D + 16 * c + 8 * hf);
      gf[c] = *reinterpret_cast<const bf16x8 *>(dotb + (hbS + qi) * D + 16 * c + 8 * hf);
    } else {
      qf[c] = (bf16x8){};
      gf[c] = (bf16x8){};
    }
  }
  const float c2 = kLog2e / sqrtf((float)D);
  const float lse2 = qi < S ? lse[hbS + qi] * kLog2e : 0.f;
  const float dl = qi < S ? delta[hbS + qi] : 0.f;
  f32x16 acc[DB];
#pragma unroll
  for (int b = 0; b < DB; ++b) acc[b] = (f32x16){};
  const int kend = min(S, q0 + BM);
  for (int k0 = 0; k0 < kend; k0 += BN) {
    __syncthreads();
    stage_rows<BN, D, KS>(ks, kh, k0, S);
    stage_rows<BN, D, KS>(vs, vh, k0, S);
    stage_cols<BN, D, TS>(kts, kth, k0, S, Sv);
    __syncthreads();
    if (k0 > qw + 31) continue;
    f32x16 st[2], dp[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      st[kb] = (f32x16){};
      dp[kb] = (f32x16){};
#pragma unroll
      for (int c = 0; c < KC; ++c) {
        st[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_row8(&ks[(32 * kb + ln) * KS + 16 * c + 8 * hf]), qf[c],
                                                         st[kb], 0, 0, 0);
        dp[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_row8(&vs[(32 * kb + ln) * KS + 16 * c + 8 * hf]), gf[c],
                                                         dp[kb], 0, 0, 0);
      }
    }
    bf16x8 dsf[4];
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int kb = c >> 1, i = 8 * (c & 1) + j;
        const int key = k0 + 32 * kb + 8 * (i >> 2) + 4 * hf + (i & 3);
        const float pj = (key <= qi) ? exp2f(fmaf(st[kb][i], c2, -lse2)) : 0.f;
        dsf[c][j] = (__bf16)(pj * (dp[kb][i] - dl));
      }
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int b = 0; b < DB; ++b)
        acc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_split8(&kts[(32 * b + ln) * TS + 16 * c + 4 * hf]), dsf[c],
                                                         acc[b], 0, 0, 0);
  }
  if (qi >= S) return;
  const float scale = 1.f / sqrtf((float)D);
  float *orow = dqt + (hbS + qi) * D;
#pragma unroll
  for (int b = 0; b < DB; ++b)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int dd = 32 * b + 8 * g + 4 * hf;
      *reinterpret_cast<float4 *>(orow + dd) = make_float4(acc[b][4 * g] * scale, acc[b][4 * g + 1] * scale,
                                                           acc[b][4 * g + 2] * scale, acc[b][4 * g + 3] * scale);
    }
}

template <int D>
__global__ __launch_bounds__(256, 1) void k_attn_bwd_dkdv(int S, int Sv, int BH, const uint16_t *__restrict__ qt,
                                                          const uint16_t *__restrict__ kt,
                                                          const uint16_t *__restrict__ vt,
                                                          const uint16_t *__restrict__ qtt,
                                                          const uint16_t *__restrict__ dotb,
                                                          const uint16_t *__restrict__ dott,
                                                          const float *__restrict__ lse,
                                                          const float *__restrict__ delta, float *__restrict__ dkt,
                                                          float *__restrict__ dvt) {
  constexpr int BK = 128, BQ = 32;
  constexpr int KC = D / 16, DB = D / 32;
  constexpr int QS = D + 8, TS = BQ + 4;
  __shared__ __attribute__((aligned(16))) uint16_t qs[BQ * QS];
  __shared__ __attribute__((aligned(16))) uint16_t gs[BQ * QS];
  __shared__ __attribute__((aligned(16))) uint16_t qts[D * TS];
  __shared__ __attribute__((aligned(16))) uint16_t gts[D * TS];
  __shared__ float ls[BQ], dls[BQ];
  const int h = blockIdx.x % BH;
  const int kb = blockIdx.x / BH;   // first key blocks see the most queries: launched first
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, ln = lane & 31, hf = lane >> 5;
  const int j0 = kb * BK, kw = j0 + 32 * w, kj = kw + ln;
  const long long hbS = (long long)h * S;
  const uint16_t *qh = qt + hbS * D;
  const uint16_t *gh = dotb + hbS * D;
  const uint16_t *qth = qtt + (long long)h * D * Sv;
  const uint16_t *gth = dott + (long long)h * D * Sv;
  bf16x8 kf[KC], vf[KC];
#pragma unroll
  for (int c = 0; c < KC; ++c) {
    if (kj < S) {
      kf[c] = *reinterpret_cast<const bf16x8 *>(kt + (hbS + kj) * D + 16 * c + 8 * hf);
      vf[c] = *reinterpret_cast<const bf16x8 *>(vt + (hbS + kj) * D + 16 * c + 8 * hf);
    } else {
      kf[c] = (bf16x8){};
      vf[c] = (bf16x8){};
    }
  }
  const float c2 = kLog2e / sqrtf((float)D);
  f32x16 adk[DB], adv[DB];
#pragma unroll
  for (int b = 0; b < DB; ++b) {
    adk[b] = (f32x16){};
    adv[b] = (f32x16){};
  }
  for (int q0 = j0; q0 < S; q0 += BQ) {
    __syncthreads();
    stage_rows<BQ, D, QS>(qs, qh, q0, S);
    stage_rows<BQ, D, QS>(gs, gh, q0, S);
    stage_cols<BQ, D, TS>(qts, qth, q0, S, Sv);
    stage_cols<BQ, D, TS>(gts, gth, q0, S, Sv);
    if (tid < BQ) {
      ls[tid] = (q0 + tid < S) ? lse[hbS + q0 + tid] * kLog2e : 0.f;
      dls[tid] = (q0 + tid < S) ? delta[hbS + q0 + tid] : 0.f;
    }
    __syncthreads();
    if (q0 + BQ - 1 < kw) continue;   // every query of the tile precedes this wavefront's keys
    f32x16 s = (f32x16){}, dp = (f32x16){};
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_row8(&qs[ln * QS + 16 * c + 8 * hf]), kf[c], s, 0, 0, 0);
      dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_row8(&gs[ln * QS + 16 * c + 8 * hf]), vf[c], dp, 0, 0, 0);
    }
    bf16x8 pf[2], dsf[2];
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int i = 8 * c + j;
        const int r = 8 * (i >> 2) + 4 * hf + (i & 3);
        const int q = q0 + r;
        const float pj = (q >= kj && q < S && kj < S) ? exp2f(fmaf(s[i], c2, -ls[r])) : 0.f;
        pf[c][j] = (__bf16)pj;
        dsf[c][j] = (__bf16)(pj * (dp[i] - dls[r]));
      }
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int b = 0; b < DB; ++b) {
        adv[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_split8(&gts[(32 * b + ln) * TS + 16 * c + 4 * hf]), pf[c],
                                                         adv[b], 0, 0, 0);
        adk[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_split8(&qts[(32 * b + ln) * TS + 16 * c + 4 * hf]),
                                                         dsf[c], adk[b], 0, 0, 0);
      }
  }
  if (kj >= S) return;
  const float scale = 1.f / sqrtf((float)D);
  float *krow = dkt + (hbS + kj) * D;
  float *vrow = dvt + (hbS + kj) * D;
#pragma unroll
  for (int b = 0; b < DB; ++b)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int dd = 32 * b + 8 * g + 4 * hf;
      *reinterpret_cast<float4 *>(krow + dd) = make_float4(adk[b][4 * g] * scale, adk[b][4 * g + 1] * scale,
                                                           adk[b][4 * g + 2] * scale, adk[b][4 * g + 3] * scale);
      *reinterpret_cast<float4 *>(vrow + dd) =
          make_float4(adv[b][4 * g], adv[b][4 * g + 1], adv[b][4 * g + 2], adv[b][4 * g + 3]);
    }
}

}  // namespace

hipError_t launch_attn_bwd_mfma(int d, int BH, int S, int Sv, const void *qt, const void *kt, const void *vt,
                                const void *qtt, const void *ktt, const void *dotb, const void *dott,
                                const float *lse, const float *delta, float *dqt, float *dkt, float *dvt,
                                hipStream_t st) {
  const uint16_t *q = (const uint16_t *)qt, *k = (const uint16_t *)kt, *v = (const uint16_t *)vt;
  const uint16_t *qT = (const uint16_t *)qtt, *kT = (const uint16_t *)ktt;
  const uint16_t *g = (const uint16_t *)dotb, *gT = (const uint16_t *)dott;
  dim3 gq(((S + 127) / 128) * BH), gk(((S + 127) / 128) * BH);
  if (d == 128) {
    k_attn_bwd_dq<128><<<gq, 256, 0, st>>>(S, Sv, BH, q, k, v, kT, g, lse, delta, dqt);
    k_attn_bwd_dkdv<128><<<gk, 256, 0, st>>>(S, Sv, BH, q, k, v, qT, g, gT, lse, delta, dkt, dvt);
  } else {
    k_attn_bwd_dq<64><<<gq, 256, 0, st>>>(S, Sv, BH, q, k, v, kT, g, lse, delta, dqt);
    k_attn_bwd_dkdv<64><<<gk, 256, 0, st>>>(S, Sv, BH, q, k, v, qT, g, gT, lse, delta, dkt, dvt);
  }
  return hipGetLastError();
}

}  // namespace lh
