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
//                    as B operands; per 32-query tile it forms S = Q~ K~^T and
//                    dP = dO~ V~^T (lane = one key), and accumulates
//                    dV^T += dO~^T P and dK^T += Q~^T dS with the transposed
//                    query-side operands from LDS.  4 wavefronts, 128 keys per
//                    work-group (the accumulators need the register file of a
//                    whole SIMD).
// Both stream their tiles through LDS filled by direct global->LDS loads
// (attn_tiles.h) while earlier tiles are computed; dK/dV software-pipelines
// the S/dP products of tile t+1 with the softmax of tile t (three buffers).  The
// transposed operands (K~^T, Q~^T, dO~^T; row stride Sv, a multiple of 64,
// zero padded, columns in perm16 order) are written by the gather and by the
// scatter adjoint, so every LDS operand is one 16-byte read per lane.  The
// row-major operands are padded with zero rows up to Sv, so no tile load needs a
// bounds check: a padding query or key contributes exactly 0.
#include "attn_tiles.h"

namespace lh {

namespace {

using tiles::bf16x8;
using tiles::f32x16;

constexpr float kLog2e = 1.4426950408889634f;

// ---------------------------------------------------------------------------
// dQ
// ---------------------------------------------------------------------------
constexpr int kDqWaves = 8;
constexpr int kDqThreads = 64 * kDqWaves;
constexpr int kDqBM = 32 * kDqWaves;
constexpr int kDqBN = 64;

template <int D>
struct DqTile {
  static constexpr int WR = 2 * D;       // bytes per K~ / V~ row
  static constexpr int WT = 2 * kDqBN;   // bytes per K~^T row
  char k[kDqBN * WR];
  char v[kDqBN * WR];
  char kt[D * WT];
};

template <int D>
__global__ __launch_bounds__(kDqThreads, 1) void k_attn_bwd_dq(int S, int Sv, int BH, const uint16_t *__restrict__ qt,
                                                               const uint16_t *__restrict__ kt,
                                                               const uint16_t *__restrict__ vt,
                                                               const uint16_t *__restrict__ ktt,
                                                               const uint16_t *__restrict__ dotb,
                                                               const float *__restrict__ rows,
                                                               float *__restrict__ dqt) {
  using Tile = DqTile<D>;
  constexpr int KC = D / 16, DB = D / 32;
  __shared__ __attribute__((aligned(1024))) Tile buf[2];
  const int nqb = (S + kDqBM - 1) / kDqBM;
  const int h = blockIdx.x % BH;
  const int qb = nqb - 1 - blockIdx.x / BH;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, ln = lane & 31, hf = lane >> 5;
  const int q0 = qb * kDqBM, qw = q0 + 32 * w, qi = qw + ln;
  const long long hbS = (long long)h * S;    // LSE, delta, dQ~: S rows per head
  const long long hbV = (long long)h * Sv;   // Q~, K~, V~, dO~: Sv rows per head (rows S..Sv-1 zero)
  const char *kh = reinterpret_cast<const char *>(kt + hbV * D);
  const char *vh = reinterpret_cast<const char *>(vt + hbV * D);
  const char *kth = reinterpret_cast<const char *>(ktt + (long long)h * D * Sv);

  // key tiles start below S and are 64 rows: they never pass the padded Sv rows
  auto fill = [&](Tile &t, int k0) {
    tiles::dma_tile<Tile::WR, kDqBN, kDqThreads>(t.k, kh + (long long)k0 * Tile::WR, Tile::WR, kDqBN - 1);
    tiles::dma_tile<Tile::WR, kDqBN, kDqThreads>(t.v, vh + (long long)k0 * Tile::WR, Tile::WR, kDqBN - 1);
    tiles::dma_tile<Tile::WT, D, kDqThreads>(t.kt, kth + 2LL * k0, 2LL * Sv, D - 1);
  };

  bf16x8 qf[KC], gf[KC];
#pragma unroll
  for (int c = 0; c < KC; ++c) {
    if (qi < Sv) {
      qf[c] = *reinterpret_cast<const bf16x8 *>(qt + (hbV + qi) * D + 16 * c + 8 * hf);
      gf[c] = *reinterpret_cast<const bf16x8 *>(dotb + (hbV + qi) * D + 16 * c + 8 * hf);
    } else {
      qf[c] = (bf16x8){};
      gf[c] = (bf16x8){};
    }
  }
  const float c2 = kLog2e / sqrtf((float)D);
  // (LSE log2(e), delta) of this lane's query (zero on the padding rows)
  const float2 rq = qi < Sv ? *reinterpret_cast<const float2 *>(rows + 2 * (hbV + qi)) : make_float2(0.f, 0.f);
  const float lse2 = rq.x, dl = rq.y;
  f32x16 acc[DB];
#pragma unroll
  for (int b = 0; b < DB; ++b) acc[b] = (f32x16){};

  const int kend = min(S, q0 + kDqBM);
  const int nt = (kend + kDqBN - 1) / kDqBN;
  fill(buf[0], 0);
  tiles::dma_wait();
  __syncthreads();
  for (int t = 0; t < nt; ++t) {
    const int k0 = t * kDqBN;
    if (t + 1 < nt) fill(buf[(t + 1) & 1], k0 + kDqBN);
    const Tile &cur = buf[t & 1];
    if (k0 <= qw + 31) {   // otherwise the tile is in this wavefront's future
      f32x16 st[2], dp[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        st[kb] = (f32x16){};
        dp[kb] = (f32x16){};
#pragma unroll
        for (int c = 0; c < KC; ++c) {
          const int off = tiles::tile_off<Tile::WR>(32 * kb + ln, 2 * c + hf);
          st[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tiles::lds_frag(cur.k, off), qf[c], st[kb], 0, 0, 0);
          dp[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tiles::lds_frag(cur.v, off), gf[c], dp[kb], 0, 0, 0);
        }
      }
      const bool diag = k0 + kDqBN - 1 > qw;   // causal mask (also masks the zero padding keys)
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
              tiles::lds_frag(cur.kt, tiles::tile_off<Tile::WT>(32 * b + ln, 2 * c + hf)), dsf[c], acc[b], 0, 0, 0);
    }
    tiles::dma_wait();
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
constexpr int kKvBQ = 32;   // query rows per tile
constexpr int kKvBufs = 4;  // tiles in LDS

// One query tile in LDS: Q~ and dO~ rows, their transposes, and the rows'
// (LSE log2(e), delta) pairs.
template <int D>
struct DkvTile {
  static constexpr int WR = 2 * D;       // bytes per Q~ / dO~ row
  static constexpr int WT = 2 * kKvBQ;   // bytes per Q~^T / dO~^T row
  static constexpr int Q = 0;
  static constexpr int G = Q + kKvBQ * WR;
  static constexpr int QT = G + kKvBQ * WR;
  static constexpr int GT = QT + D * WT;
  static constexpr int RS = GT + D * WT;
  static constexpr int BYTES = RS + 8 * kKvBQ;
};

template <bool B>
struct Flag {
  static constexpr bool value = B;
};

template <int D>
__global__ __launch_bounds__(kKvThreads, 1) void k_attn_bwd_dkdv(int S, int Sv, int BH,
                                                                 const uint16_t *__restrict__ qt,
                                                                 const uint16_t *__restrict__ kt,
                                                                 const uint16_t *__restrict__ vt,
                                                                 const uint16_t *__restrict__ qtt,
                                                                 const uint16_t *__restrict__ dotb,
                                                                 const uint16_t *__restrict__ dott,
                                                                 const float *__restrict__ rows,
                                                                 float *__restrict__ dkt, float *__restrict__ dvt) {
  using T = DkvTile<D>;
  constexpr int KC = D / 16, DB = D / 32;
  constexpr int NC = 4 * DB;   // dV/dK products per tile
  static_assert(NC == 2 * KC, "one S/dP operand read per dV/dK product");
  constexpr int EPS = 16 / KC;                                // softmax values per S/dP step
  constexpr int QBLK = kKvBQ * T::WR / 1024 / kKvWaves;       // 1 KB fill blocks per wavefront: Q~, dO~
  constexpr int TBLK = D * T::WT / 1024 / kKvWaves;           // ... Q~^T, dO~^T
  static_assert(QBLK * 1024 * kKvWaves == kKvBQ * T::WR && TBLK * 1024 * kKvWaves == D * T::WT, "fill blocks");
  // four tiles: t (softmax, dV/dK operands), t+1 (S/dP operands), t+2 and t+3
  // (filling: a fill has two iterations to land)
  __shared__ __attribute__((aligned(1024))) char lds[kKvBufs * T::BYTES];
  constexpr int kFillOps = 2 * QBLK + 2 * TBLK + 1;   // loads per wavefront per fill
  const int h = blockIdx.x % BH;
  const int kb = blockIdx.x / BH;   // first key blocks see the most queries: launched first
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, ln = lane & 31, hf = lane >> 5;
  const int wu = __builtin_amdgcn_readfirstlane(w);
  const int j0 = kb * kKvBK, kw = j0 + 32 * w, kj = kw + ln;
  const long long hbS = (long long)h * S;    // dK~, dV~: S rows per head
  const long long hbV = (long long)h * Sv;   // Q~, K~, V~, dO~, row pairs: Sv rows per head (rows S..Sv-1 zero)
  const char *qh = reinterpret_cast<const char *>(qt + hbV * D);
  const char *gh = reinterpret_cast<const char *>(dotb + hbV * D);
  const char *qth = reinterpret_cast<const char *>(qtt + (long long)h * D * Sv);
  const char *gth = reinterpret_cast<const char *>(dott + (long long)h * D * Sv);
  const char *rh = reinterpret_cast<const char *>(rows + 2 * hbV);
  const unsigned lbase = tiles::lds_addr(lds);

  // Fills: per-lane source offsets are loop invariant; the tile's base address
  // and the LDS destination are scalars.  Query tiles start below S and are 32
  // rows, so they never pass the padded Sv rows; a padding query (zero Q~, dO~,
  // LSE and delta) adds exactly 0.  Every wavefront issues the same 256-byte
  // fill of the row pairs (identical bytes), so the fill has no branch.
  unsigned vq[QBLK], vtr[TBLK];
#pragma unroll
  for (int i = 0; i < QBLK; ++i) vq[i] = tiles::dma_voff<T::WR>(wu + i * kKvWaves, T::WR);
#pragma unroll
  for (int i = 0; i < TBLK; ++i) vtr[i] = tiles::dma_voff<T::WT>(wu + i * kKvWaves, 2u * Sv);
  const unsigned vrs = 4u * lane;
  auto fill = [&](int jb, int q0) {
    const unsigned m = lbase + jb * T::BYTES;
#pragma unroll
    for (int i = 0; i < QBLK; ++i) {
      const unsigned blk = 1024u * (wu + i * kKvWaves);
      tiles::lds_load_s<16>(qh + (long long)q0 * T::WR, vq[i], m + T::Q + blk);
      tiles::lds_load_s<16>(gh + (long long)q0 * T::WR, vq[i], m + T::G + blk);
    }
#pragma unroll
    for (int i = 0; i < TBLK; ++i) {
      const unsigned blk = 1024u * (wu + i * kKvWaves);
      tiles::lds_load_s<16>(qth + 2LL * q0, vtr[i], m + T::QT + blk);
      tiles::lds_load_s<16>(gth + 2LL * q0, vtr[i], m + T::GT + blk);
    }
    tiles::lds_load_s<4>(rh + 8LL * q0, vrs, m + T::RS);
  };

  // per-lane LDS read offsets (loop invariant): S/dP operands (row ln, chunk
  // 2c+hf of a row-major tile) and dV/dK operands (row 32b+ln, chunk 2cc+hf of
  // a transposed tile, c = cc DB + b)
  int oq[KC], ot[KC];
#pragma unroll
  for (int c = 0; c < KC; ++c) {
    oq[c] = tiles::tile_off<T::WR>(ln, 2 * c + hf);
    ot[c] = tiles::tile_off<T::WT>(32 * (c % DB) + ln, 2 * (c / DB) + hf);
  }
  const int ors = T::RS + 32 * hf;   // row pairs 8 g4 + 4 hf + 0..3 at ors + 64 g4

  // K~, V~ rows of this lane's key: B operands of S and dP (keys past Sv read as zero)
  bf16x8 kf[KC], vf[KC];
#pragma unroll
  for (int c = 0; c < KC; ++c) {
    if (kj < Sv) {
      kf[c] = *reinterpret_cast<const bf16x8 *>(kt + (hbV + kj) * D + 16 * c + 8 * hf);
      vf[c] = *reinterpret_cast<const bf16x8 *>(vt + (hbV + kj) * D + 16 * c + 8 * hf);
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
  // dV/dK operands of the previous tile: P and dS (B operands, from the
  // softmax) and the dO~^T, Q~^T chunks (A operands, from LDS)
  bf16x8 pf[2], dsf[2], fgt[KC], fqt[KC];
#pragma unroll
  for (int c = 0; c < 2; ++c) pf[c] = dsf[c] = (bf16x8){};
#pragma unroll
  for (int c = 0; c < KC; ++c) fgt[c] = fqt[c] = (bf16x8){};
  // k-th dV/dK product of the previous tile
  auto dvdk = [&](int k) {
    const int c = k >> 1, cc = c / DB, b = c % DB;
    if (k & 1) adk[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fqt[c], dsf[cc], adk[b], 0, 0, 0);
    else adv[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fgt[c], pf[cc], adv[b], 0, 0, 0);
  };

  const int nt = (S - j0 + kKvBQ - 1) / kKvBQ;   // query tiles from the block's first key to S
  const int qlast = j0 + (nt - 1) * kKvBQ;       // first query of the last tile
  fill(0, j0);
  fill(1, min(j0 + kKvBQ, qlast));
  fill(2, min(j0 + 2 * kKvBQ, qlast));
  tiles::wait_fills_barrier<kFillOps>();   // tiles 0 and 1 landed
  // S = Q~ K~^T, dP = dO~ V~^T of the first tile (lane = one key, 16 query rows)
  f32x16 sv = (f32x16){}, dp = (f32x16){};
#pragma unroll
  for (int c = 0; c < KC; ++c) {
    sv = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tiles::lds_frag(lds + T::Q, oq[c]), kf[c], sv, 0, 0, 0);
    dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tiles::lds_frag(lds + T::G, oq[c]), vf[c], dp, 0, 0, 0);
  }

  // Iteration t.  One wavefront per SIMD has no other wavefront to hide its
  // latencies behind, so the body is one basic block in a fixed issue order:
  //  1. fill of tile t+3 (into the buffer tile t-1 used);
  //  2. LDS reads of tile t's row pairs;
  //  3. the NC dV/dK products of tile t-1 (operands already in registers),
  //     each followed by one LDS read of tile t+1's S/dP operands -- the
  //     products cover the read latency;
  //  4. KC steps, each issuing one S/dP product pair of tile t+1, the softmax
  //     of EPS of this lane's values of tile t (VALU work that runs while the
  //     products occupy the matrix core) and two LDS reads of tile t's dV/dK
  //     operands;
  //  5. wait for the fill of tile t+2 (issued one iteration earlier), barrier.
  // Every wavefront updates its accumulators on every tile; the causal mask is
  // applied on the first kKvBK/kKvBQ tiles only (on later tiles every query
  // follows every key of the block); the fill past the last tile repeats the
  // last tile and the S/dP products past it are dropped.
  auto iteration = [&](int t, auto mask) {
    constexpr bool MASK = decltype(mask)::value;
    const int q0 = j0 + t * kKvBQ;
    const int jc = t & (kKvBufs - 1), jn = (t + 1) & (kKvBufs - 1), jf = (t + 3) & (kKvBufs - 1);
    fill(jf, min(q0 + 3 * kKvBQ, qlast));
    const char *cur = lds + jc * T::BYTES;
    const char *nxt = lds + jn * T::BYTES;
    float4 r4[8];   // (LSE log2 e, delta) of rows 8 g4 + 4 hf + {0,1} and {2,3}
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      r4[2 * g4] = *reinterpret_cast<const float4 *>(cur + ors + 64 * g4);
      r4[2 * g4 + 1] = *reinterpret_cast<const float4 *>(cur + ors + 64 * g4 + 16);
    }
    bf16x8 fq[KC], fg[KC];
#pragma unroll
    for (int k = 0; k < NC; ++k) {
      dvdk(k);
      if (k & 1) fg[k >> 1] = tiles::lds_frag(nxt + T::G, oq[k >> 1]);
      else fq[k >> 1] = tiles::lds_frag(nxt + T::Q, oq[k >> 1]);
      __builtin_amdgcn_sched_barrier(0);
    }
    f32x16 sv_n = (f32x16){}, dp_n = (f32x16){};
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      sv_n = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fq[c], kf[c], sv_n, 0, 0, 0);
      dp_n = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fg[c], vf[c], dp_n, 0, 0, 0);
#pragma unroll
      for (int u = 0; u < EPS; ++u) {
        const int i = EPS * c + u;   // register of the 32x32 block: query row 8 g4 + 4 hf + e
        const int g4 = i >> 2, e = i & 3;
        const float4 &rp = r4[2 * g4 + (e >> 1)];
        const float ls = (e & 1) ? rp.z : rp.x;
        const float dl = (e & 1) ? rp.w : rp.y;
        float pj = __builtin_amdgcn_exp2f(fmaf(sv[i], c2, -ls));
        if constexpr (MASK) {
          if (q0 + 8 * g4 + 4 * hf + e < kj) pj = 0.f;
        }
        pf[i >> 3][i & 7] = (__bf16)pj;
        dsf[i >> 3][i & 7] = (__bf16)(pj * (dp[i] - dl));
      }
      fgt[c] = tiles::lds_frag(cur + T::GT, ot[c]);
      fqt[c] = tiles::lds_frag(cur + T::QT, ot[c]);
      __builtin_amdgcn_sched_barrier(0);
    }
    sv = sv_n;
    dp = dp_n;
    tiles::wait_fills_barrier<kFillOps>();   // tile t+2 landed; tile t+3 may be in flight
  };
  const int nm = min(nt, kKvBK / kKvBQ);
  for (int t = 0; t < nm; ++t) iteration(t, Flag<true>{});
  for (int t = nm; t < nt; ++t) iteration(t, Flag<false>{});
#pragma unroll
  for (int k = 0; k < NC; ++k) dvdk(k);
  tiles::dma_wait();   // the fills past the last tile, before the work-group exits

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
                                const float *rows, float *dqt, float *dkt, float *dvt, int part, hipStream_t st) {
  const uint16_t *q = (const uint16_t *)qt, *k = (const uint16_t *)kt, *v = (const uint16_t *)vt;
  const uint16_t *qT = (const uint16_t *)qtt, *kT = (const uint16_t *)ktt;
  const uint16_t *g = (const uint16_t *)dotb, *gT = (const uint16_t *)dott;
  dim3 gq(((S + kDqBM - 1) / kDqBM) * BH), gk(((S + kKvBK - 1) / kKvBK) * BH);
  if (part == 0) {   // dQ~
    if (d == 128) k_attn_bwd_dq<128><<<gq, kDqThreads, 0, st>>>(S, Sv, BH, q, k, v, kT, g, rows, dqt);
    else k_attn_bwd_dq<64><<<gq, kDqThreads, 0, st>>>(S, Sv, BH, q, k, v, kT, g, rows, dqt);
  } else {           // dK~, dV~
    if (d == 128) k_attn_bwd_dkdv<128><<<gk, kKvThreads, 0, st>>>(S, Sv, BH, q, k, v, qT, g, gT, rows, dkt, dvt);
    else k_attn_bwd_dkdv<64><<<gk, kKvThreads, 0, st>>>(S, Sv, BH, q, k, v, qT, g, gT, rows, dkt, dvt);
  }
  return hipGetLastError();
}

}  // namespace lh
