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
//                    8 wavefronts, 256 queries per work-group.
//   k_attn_bwd_dkdv  key-stationary: a wavefront holds 32 key rows of K~ and V~
//                    as B operands; per query tile it forms S = Q~ K~^T and
//                    dP = dO~ V~^T (lane = one key), and accumulates
//                    dV^T += dO~^T P and dK^T += Q~^T dS with the transposed
//                    query-side operands from LDS.  4 wavefronts, 128 keys per
//                    work-group (the accumulators need the register file of a
//                    whole SIMD).
// Both stream their tiles through double-buffered LDS with the next tile's
// global loads in flight in registers.  The transposed operands (K~^T, Q~^T,
// dO~^T; row stride Sv, a multiple of 64, zero padded) are written by the
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

__device__ __forceinline__ void st_split8(uint16_t *p, uint4 v) {
  uint2 *d2 = reinterpret_cast<uint2 *>(p);
  d2[0] = make_uint2(v.x, v.y);
  d2[1] = make_uint2(v.z, v.w);
}

// ---------------------------------------------------------------------------
// dQ
// ---------------------------------------------------------------------------
constexpr int kDqWaves = 8;
constexpr int kDqThreads = 64 * kDqWaves;
constexpr int kDqBM = 32 * kDqWaves;
constexpr int kDqBN = 64;

template <int D>
struct DqTile {
  static constexpr int KS = D + 8;
  static constexpr int TS = kDqBN + 4;
  static constexpr int RCH = kDqBN * D / 8;          // 16-byte chunks of one row tile
  static constexpr int RPT = RCH / kDqThreads;       // per thread
  uint16_t k[kDqBN * KS];
  uint16_t v[kDqBN * KS];
  uint16_t kt[D * TS];
};

template <int D>
__global__ __launch_bounds__(kDqThreads, 1) void k_attn_bwd_dq(int S, int Sv, int BH, const uint16_t *__restrict__ qt,
                                                               const uint16_t *__restrict__ kt,
                                                               const uint16_t *__restrict__ vt,
                                                               const uint16_t *__restrict__ ktt,
                                                               const uint16_t *__restrict__ dotb,
                                                               const float *__restrict__ lse,
                                                               const float *__restrict__ delta,
                                                               float *__restrict__ dqt) {
  using Tile = DqTile<D>;
  constexpr int KC = D / 16, DB = D / 32;
  __shared__ __attribute__((aligned(16))) Tile buf[2];
  const int nqb = (S + kDqBM - 1) / kDqBM;
  const int h = blockIdx.x % BH;
  const int qb = nqb - 1 - blockIdx.x / BH;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, ln = lane & 31, hf = lane >> 5;
  const int q0 = qb * kDqBM, qw = q0 + 32 * w, qi = qw + ln;
  const long long hbS = (long long)h * S;
  const uint16_t *kh = kt + hbS * D;
  const uint16_t *vh = vt + hbS * D;
  const uint16_t *kth = ktt + (long long)h * D * Sv;

  uint4 rk[Tile::RPT], rv[Tile::RPT], rt[Tile::RPT];
  auto load_tile = [&](int k0) {
#pragma unroll
    for (int it = 0; it < Tile::RPT; ++it) {
      const int idx = it * kDqThreads + tid;
      const int r = idx / (D / 8), cc = idx % (D / 8);
      const bool ok = k0 + r < S;
      rk[it] = ok ? *reinterpret_cast<const uint4 *>(kh + (long long)(k0 + r) * D + cc * 8) : make_uint4(0, 0, 0, 0);
      rv[it] = ok ? *reinterpret_cast<const uint4 *>(vh + (long long)(k0 + r) * D + cc * 8) : make_uint4(0, 0, 0, 0);
      const int tr = idx / (kDqBN / 8), tc = idx % (kDqBN / 8);
      rt[it] = *reinterpret_cast<const uint4 *>(kth + (long long)tr * Sv + k0 + tc * 8);
    }
  };
  auto store_tile = [&](Tile &t) {
#pragma unroll
    for (int it = 0; it < Tile::RPT; ++it) {
      const int idx = it * kDqThreads + tid;
      const int r = idx / (D / 8), cc = idx % (D / 8);
      *reinterpret_cast<uint4 *>(&t.k[r * Tile::KS + cc * 8]) = rk[it];
      *reinterpret_cast<uint4 *>(&t.v[r * Tile::KS + cc * 8]) = rv[it];
      const int tr = idx / (kDqBN / 8), tc = idx % (kDqBN / 8);
      st_split8(&t.kt[tr * Tile::TS + tc * 8], rt[it]);
    }
  };

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

  const int kend = min(S, q0 + kDqBM);
  const int nt = (kend + kDqBN - 1) / kDqBN;
  load_tile(0);
  store_tile(buf[0]);
  __syncthreads();
  for (int t = 0; t < nt; ++t) {
    const int k0 = t * kDqBN;
    if (t + 1 < nt) load_tile(k0 + kDqBN);
    const Tile &cur = buf[t & 1];
    if (k0 <= qw + 31) {
      f32x16 st[2], dp[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        st[kb] = (f32x16){};
        dp[kb] = (f32x16){};
#pragma unroll
        for (int c = 0; c < KC; ++c) {
          st[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_row8(&cur.k[(32 * kb + ln) * Tile::KS + 16 * c + 8 * hf]),
                                                           qf[c], st[kb], 0, 0, 0);
          dp[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_row8(&cur.v[(32 * kb + ln) * Tile::KS + 16 * c + 8 * hf]),
                                                           gf[c], dp[kb], 0, 0, 0);
        }
      }
      const bool diag = k0 + kDqBN - 1 > qw;
      bf16x8 dsf[4];
#pragma unroll
      for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int kb = c >> 1, i = 8 * (c & 1) + j;
          const int key = k0 + 32 * kb + 8 * (i >> 2) + 4 * hf + (i & 3);
          float pj = __builtin_amdgcn_exp2f(fmaf(st[kb][i], c2, -lse2));
          if (diag && key > qi) pj = 0.f;
          dsf[c][j] = (__bf16)(pj * (dp[kb][i] - dl));
        }
#pragma unroll
      for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int b = 0; b < DB; ++b)
          acc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              lds_split8(&cur.kt[(32 * b + ln) * Tile::TS + 16 * c + 4 * hf]), dsf[c], acc[b], 0, 0, 0);
    }
    if (t + 1 < nt) store_tile(buf[(t + 1) & 1]);
    __syncthreads();
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

// ---------------------------------------------------------------------------
// dK, dV
// ---------------------------------------------------------------------------
constexpr int kKvWaves = 4;
constexpr int kKvThreads = 64 * kKvWaves;
constexpr int kKvBK = 32 * kKvWaves;
constexpr int kKvBQ = 32;

template <int D>
struct DkvTile {
  static constexpr int QS = D + 8;
  static constexpr int TS = kKvBQ + 4;
  static constexpr int RCH = kKvBQ * D / 8;
  static constexpr int RPT = RCH / kKvThreads;
  uint16_t q[kKvBQ * QS];
  uint16_t g[kKvBQ * QS];
  uint16_t qt[D * TS];
  uint16_t gt[D * TS];
  float ls[kKvBQ];
  float dl[kKvBQ];
};

template <int D>
__global__ __launch_bounds__(kKvThreads, 1) void k_attn_bwd_dkdv(int S, int Sv, int BH,
                                                                 const uint16_t *__restrict__ qt,
                                                                 const uint16_t *__restrict__ kt,
                                                                 const uint16_t *__restrict__ vt,
                                                                 const uint16_t *__restrict__ qtt,
                                                                 const uint16_t *__restrict__ dotb,
                                                                 const uint16_t *__restrict__ dott,
                                                                 const float *__restrict__ lse,
                                                                 const float *__restrict__ delta,
                                                                 float *__restrict__ dkt, float *__restrict__ dvt) {
  using Tile = DkvTile<D>;
  constexpr int KC = D / 16, DB = D / 32;
  __shared__ __attribute__((aligned(16))) Tile buf[2];
  const int h = blockIdx.x % BH;
  const int kb = blockIdx.x / BH;   // first key blocks see the most queries: launched first
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, ln = lane & 31, hf = lane >> 5;
  const int j0 = kb * kKvBK, kw = j0 + 32 * w, kj = kw + ln;
  const long long hbS = (long long)h * S;
  const uint16_t *qh = qt + hbS * D;
  const uint16_t *gh = dotb + hbS * D;
  const uint16_t *qth = qtt + (long long)h * D * Sv;
  const uint16_t *gth = dott + (long long)h * D * Sv;

  uint4 rq[Tile::RPT], rg[Tile::RPT], rqt[Tile::RPT], rgt[Tile::RPT];
  float rl = 0.f;
  auto load_tile = [&](int q0) {
#pragma unroll
    for (int it = 0; it < Tile::RPT; ++it) {
      const int idx = it * kKvThreads + tid;
      const int r = idx / (D / 8), cc = idx % (D / 8);
      const bool ok = q0 + r < S;
      rq[it] = ok ? *reinterpret_cast<const uint4 *>(qh + (long long)(q0 + r) * D + cc * 8) : make_uint4(0, 0, 0, 0);
      rg[it] = ok ? *reinterpret_cast<const uint4 *>(gh + (long long)(q0 + r) * D + cc * 8) : make_uint4(0, 0, 0, 0);
      const int tr = idx / (kKvBQ / 8), tc = idx % (kKvBQ / 8);
      rqt[it] = *reinterpret_cast<const uint4 *>(qth + (long long)tr * Sv + q0 + tc * 8);
      rgt[it] = *reinterpret_cast<const uint4 *>(gth + (long long)tr * Sv + q0 + tc * 8);
    }
    if (tid < 2 * kKvBQ) {
      const int r = tid & (kKvBQ - 1);
      rl = (q0 + r < S) ? (tid < kKvBQ ? lse[hbS + q0 + r] * kLog2e : delta[hbS + q0 + r]) : 0.f;
    }
  };
  auto store_tile = [&](Tile &t) {
#pragma unroll
    for (int it = 0; it < Tile::RPT; ++it) {
      const int idx = it * kKvThreads + tid;
      const int r = idx / (D / 8), cc = idx % (D / 8);
      *reinterpret_cast<uint4 *>(&t.q[r * Tile::QS + cc * 8]) = rq[it];
      *reinterpret_cast<uint4 *>(&t.g[r * Tile::QS + cc * 8]) = rg[it];
      const int tr = idx / (kKvBQ / 8), tc = idx % (kKvBQ / 8);
      st_split8(&t.qt[tr * Tile::TS + tc * 8], rqt[it]);
      st_split8(&t.gt[tr * Tile::TS + tc * 8], rgt[it]);
    }
    if (tid < kKvBQ) t.ls[tid] = rl;
    else if (tid < 2 * kKvBQ) t.dl[tid - kKvBQ] = rl;
  };

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
  const int nt = (S - j0 + kKvBQ - 1) / kKvBQ;   // query tiles from the block's first key to S
  load_tile(j0);
  store_tile(buf[0]);
  __syncthreads();
  for (int t = 0; t < nt; ++t) {
    const int q0 = j0 + t * kKvBQ;
    if (t + 1 < nt) load_tile(q0 + kKvBQ);
    const Tile &cur = buf[t & 1];
    if (q0 + kKvBQ - 1 >= kw) {   // otherwise every query of the tile precedes this wavefront's keys
      f32x16 s = (f32x16){}, dp = (f32x16){};
#pragma unroll
      for (int c = 0; c < KC; ++c) {
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_row8(&cur.q[ln * Tile::QS + 16 * c + 8 * hf]), kf[c], s, 0, 0,
                                                    0);
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_row8(&cur.g[ln * Tile::QS + 16 * c + 8 * hf]), vf[c], dp, 0,
                                                     0, 0);
      }
      const bool diag = q0 < kw + 31;   // some query of the tile precedes some key of the wavefront
      bf16x8 pf[2], dsf[2];
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int i = 8 * c + j;
          const int r = 8 * (i >> 2) + 4 * hf + (i & 3);
          float pj = __builtin_amdgcn_exp2f(fmaf(s[i], c2, -cur.ls[r]));
          if ((diag && q0 + r < kj) || q0 + r >= S || kj >= S) pj = 0.f;
          pf[c][j] = (__bf16)pj;
          dsf[c][j] = (__bf16)(pj * (dp[i] - cur.dl[r]));
        }
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int b = 0; b < DB; ++b) {
          adv[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              lds_split8(&cur.gt[(32 * b + ln) * Tile::TS + 16 * c + 4 * hf]), pf[c], adv[b], 0, 0, 0);
          adk[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              lds_split8(&cur.qt[(32 * b + ln) * Tile::TS + 16 * c + 4 * hf]), dsf[c], adk[b], 0, 0, 0);
        }
    }
    if (t + 1 < nt) store_tile(buf[(t + 1) & 1]);
    __syncthreads();
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
  dim3 gq(((S + kDqBM - 1) / kDqBM) * BH), gk(((S + kKvBK - 1) / kKvBK) * BH);
  if (d == 128) {
    k_attn_bwd_dq<128><<<gq, kDqThreads, 0, st>>>(S, Sv, BH, q, k, v, kT, g, lse, delta, dqt);
    k_attn_bwd_dkdv<128><<<gk, kKvThreads, 0, st>>>(S, Sv, BH, q, k, v, qT, g, gT, lse, delta, dkt, dvt);
  } else {
    k_attn_bwd_dq<64><<<gq, kDqThreads, 0, st>>>(S, Sv, BH, q, k, v, kT, g, lse, delta, dqt);
    k_attn_bwd_dkdv<64><<<gk, kKvThreads, 0, st>>>(S, Sv, BH, q, k, v, qT, g, gT, lse, delta, dkt, dvt);
  }
  return hipGetLastError();
}

}  // namespace lh
