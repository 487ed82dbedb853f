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
//   k_attn_bwd_dkdv  key-stationary: the work of 32 keys is split over a pair
//                    of wavefronts on one SIMD.  The "P" wavefront holds the
//                    keys' K~ rows and dV~ accumulators: per 32-query tile it
//                    forms S = Q~ K~^T (lane = one key), P, and
//                    dV^T += dO~^T P.  The "dS" wavefront holds their V~ rows
//                    and dK~ accumulators: it forms dP = dO~ V~^T, takes P from
//                    its partner through LDS, and accumulates dK^T += Q~^T dS.
//                    The transposed query-side operands come from LDS.  4 pairs
//                    (8 wavefronts), 128 keys per work-group.
// Both stream their tiles through LDS filled by direct global->LDS loads
// (attn_tiles.h) while earlier tiles are computed.  Operands contracted over
// keys or queries (K~^T, Q~^T, dO~^T) come from the row-major tiles by
// transposing LDS reads.  The row-major operands are padded with zero rows up
// to Sv (a multiple of 64), so no tile load needs a bounds check: a padding
// query or key contributes exactly 0.
#include "attn_tiles.h"

namespace lh {

namespace {

using tiles::bf16x8;
using tiles::f32x16;

constexpr float kLog2e = 1.4426950408889634f;

template <bool B>
struct Flag {
  static constexpr bool value = B;
};

// ---------------------------------------------------------------------------
// dQ
// ---------------------------------------------------------------------------
// Query-stationary: a wavefront holds 32 query rows of Q~ and dO~ as B
// operands; per 64-key tile, for each half of 32 keys, it forms S^T = K~ Q~^T
// and dP^T = V~ dO~^T (lane = one query), dS^T = P^T o (dP^T - delta) in
// registers, and accumulates dQ~^T += K~^T dS^T, the K~^T operand coming from
// the row-major K~ tile by transposing reads.  8 wavefronts, 256 queries per
// work-group; tiles in a ring of four LDS buffers filled three tiles ahead; LDS
// operands streamed through a window of kDqWin fragments (as the forward).
constexpr int kDqWaves = 8;
constexpr int kDqThreads = 64 * kDqWaves;
constexpr int kDqBM = 32 * kDqWaves;
constexpr int kDqBN = 64;
constexpr int kDqBufs = 4;
constexpr int kDqWin = 8;

template <int D>
struct DqTile {
  static constexpr int WR = 2 * D;   // bytes per K~ / V~ row
  static constexpr int K = 0;
  static constexpr int V = kDqBN * WR;
  static constexpr int BYTES = 2 * kDqBN * WR;
};

template <int D>
__global__ __launch_bounds__(kDqThreads, 1) void k_attn_bwd_dq(int S, int Sv, int BH, const uint16_t *__restrict__ qt,
                                                               const uint16_t *__restrict__ kt,
                                                               const uint16_t *__restrict__ vt,
                                                               const uint16_t *__restrict__ dotb,
                                                               const float *__restrict__ rows,
                                                               float *__restrict__ dqt) {
  using T = DqTile<D>;
  constexpr int KC = D / 16, DB = D / 32;
  constexpr int NA = 2 * KC;          // S^T / dP^T fragments per 32-key half (K~, V~ alternating)
  constexpr int NH = NA + 2 * DB;     // ... plus the dQ fragments (K~^T) of the half
  constexpr int NF = 2 * NH;          // fragments per tile
  constexpr int KBLK = kDqBN * T::WR / 1024 / kDqWaves;   // 1 KB fill blocks per wavefront, K~ and V~ each
  static_assert(KBLK * 1024 * kDqWaves == kDqBN * T::WR, "fill blocks");
  constexpr int kFillOps = 2 * KBLK;
  __shared__ __attribute__((aligned(1024))) char lds[kDqBufs * T::BYTES];
  const int nqb = (S + kDqBM - 1) / kDqBM;
  const int h = blockIdx.x % BH;
  const int qb = nqb - 1 - blockIdx.x / BH;
  const int tid = threadIdx.x, lane = tid & 63, ln = lane & 31, hf = lane >> 5;
  const int wu = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int q0 = qb * kDqBM, qw = q0 + 32 * wu, qi = qw + ln;
  const long long hbS = (long long)h * S;    // dQ~: S rows per head
  const long long hbV = (long long)h * Sv;   // Q~, K~, V~, dO~, row pairs: Sv rows per head (rows S..Sv-1 zero)
  const char *kh = reinterpret_cast<const char *>(kt + hbV * D);
  const char *vh = reinterpret_cast<const char *>(vt + hbV * D);
  const unsigned lbase = tiles::lds_addr(lds);

  // fills: key tiles start below S and are 64 rows, so they never pass the Sv rows
  unsigned vo[KBLK];
#pragma unroll
  for (int i = 0; i < KBLK; ++i) vo[i] = tiles::dma_voff<T::WR>(wu + i * kDqWaves, T::WR);
  auto fill = [&](int jb, int k0) {
    const unsigned m = lbase + jb * T::BYTES;
#pragma unroll
    for (int i = 0; i < KBLK; ++i) {
      const unsigned blk = 1024u * (wu + i * kDqWaves);
      tiles::lds_load_s<16>(kh + (long long)k0 * T::WR, vo[i], m + T::K + blk);
      tiles::lds_load_s<16>(vh + (long long)k0 * T::WR, vo[i], m + T::V + blk);
    }
  };
  // fragment j of a tile (half kb = j / NH, r = j % NH): r < NA: K~ (r even) or
  // V~ (r odd) rows 32 kb + ln, chunk 2 (r/2) + hf; r >= NA: K~^T d rows
  // 32 b + ln over the 16 keys of chunk 2 kb + cc (r - NA = cc DB + b)
  int oq[KC], otr[DB][2];
#pragma unroll
  for (int c = 0; c < KC; ++c) oq[c] = tiles::tile_off<T::WR>(ln, 2 * c + hf);
#pragma unroll
  for (int b = 0; b < DB; ++b) {
    otr[b][0] = tiles::tr_off<T::WR>(0, 32 * b);
    otr[b][1] = tiles::tr_off<T::WR>(8, 32 * b);
  }
  auto frag = [&](const char *buf, int j) -> bf16x8 {
    const int kb = j / NH, r = j % NH;
    if (r < NA) return tiles::lds_frag(buf + ((r & 1) ? T::V : T::K) + 32 * kb * T::WR, oq[r >> 1]);
    const int cc = (r - NA) / DB, b = (r - NA) % DB;
    return tiles::tr_frag(buf + T::K + 16 * (2 * kb + cc) * T::WR, otr[b][0], otr[b][1]);
  };

  bf16x8 qf[KC], gf[KC];
#pragma unroll
  for (int c = 0; c < KC; ++c) {
    qf[c] = (qi < Sv) ? *reinterpret_cast<const bf16x8 *>(qt + (hbV + qi) * D + 16 * c + 8 * hf) : (bf16x8){};
    gf[c] = (qi < Sv) ? *reinterpret_cast<const bf16x8 *>(dotb + (hbV + qi) * D + 16 * c + 8 * hf) : (bf16x8){};
  }
  // (LSE log2(e), delta) of this lane's query (zero on the padding rows)
  const float2 rq = qi < Sv ? *reinterpret_cast<const float2 *>(rows + 2 * (hbV + qi)) : make_float2(0.f, 0.f);
  const float lse2 = rq.x, dl = rq.y;
  tiles::dma_wait();   // here, not inside the loop (see the forward)
  const float c2 = kLog2e / sqrtf((float)D);
  f32x16 acc[DB];
#pragma unroll
  for (int b = 0; b < DB; ++b) acc[b] = (f32x16){};

  const int kend = min(S, q0 + kDqBM);
  const int nt = (kend + kDqBN - 1) / kDqBN;
  const int klast = (nt - 1) * kDqBN;
  fill(0, 0);
  fill(1, min(kDqBN, klast));
  fill(2, min(2 * kDqBN, klast));
  tiles::wait_fills_barrier<kFillOps>();   // tiles 0 and 1 landed
  bf16x8 win[kDqWin];
#pragma unroll
  for (int j = 0; j < kDqWin; ++j) win[j] = frag(lds, j);

  auto iteration = [&](int t, auto mask) {
    constexpr bool MASK = decltype(mask)::value;
    const int k0 = t * kDqBN;
    fill((t + 3) & (kDqBufs - 1), min(k0 + 3 * kDqBN, klast));   // past the end: a repeat of the last tile
    const char *cur = lds + (t & (kDqBufs - 1)) * T::BYTES;
    const char *nxt = lds + ((t + 1) & (kDqBufs - 1)) * T::BYTES;
    auto next = [&](int j) {   // the window moves on (into the next tile near the end)
      win[j % kDqWin] = (j + kDqWin < NF) ? frag(cur, j + kDqWin) : frag(nxt, j + kDqWin - NF);
      __builtin_amdgcn_sched_barrier(0);
    };
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      f32x16 st = (f32x16){}, dp = (f32x16){};
      // the wavefronts of a SIMD alternate between runs of products and the dS
      // arithmetic; a run of products is issued at raised priority so that the
      // matrix core is kept fed while the other wavefront computes
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int c = 0; c < KC; ++c) {
        const int j = kb * NH + 2 * c;
        st = __builtin_amdgcn_mfma_f32_32x32x16_bf16(win[j % kDqWin], qf[c], st, 0, 0, 0);
        next(j);
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(win[(j + 1) % kDqWin], gf[c], dp, 0, 0, 0);
        next(j + 1);
      }
      __builtin_amdgcn_s_setprio(0);
      bf16x8 dsf[2];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float pj = __builtin_amdgcn_exp2f(fmaf(st[i], c2, -lse2));
        if constexpr (MASK) {
          const int key = k0 + 32 * kb + 8 * (i >> 2) + 4 * hf + (i & 3);
          if (key > qi) pj = 0.f;
        }
        dsf[i >> 3][i & 7] = (__bf16)(pj * (dp[i] - dl));
      }
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int r = 0; r < 2 * DB; ++r) {   // dQ~^T += K~^T dS^T over the half's two 16-key chunks
        const int j = kb * NH + NA + r;
        acc[r % DB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(win[j % kDqWin], dsf[r / DB], acc[r % DB], 0, 0, 0);
        next(j);
      }
    }
    __builtin_amdgcn_s_setprio(0);
    static_assert(kDqWin <= NA, "the reads kept in flight are single reads");
    tiles::wait_fills_barrier_keep<kFillOps, kDqWin>();   // tile t+2 landed; the window's reads (tile t+1) stay in flight
  };
  const int nu = max(0, nt - kDqBM / kDqBN);   // tiles before the block's first query: no mask
  for (int t = 0; t < nu; ++t) iteration(t, Flag<false>{});
  for (int t = nu; t < nt; ++t) iteration(t, Flag<true>{});
  tiles::dma_wait();   // the fills past the last tile, before the work-group exits

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
// Work-group: 128 keys, 4 pairs of wavefronts, one pair per 32 keys and per
// SIMD.  In a pair, the "P" wavefront holds the keys' K~ rows and the dV~
// accumulators, the "dS" wavefront their V~ rows and the dK~ accumulators (each
// needs half the registers of doing both, so two wavefronts fit on a SIMD and
// the hardware interleaves them).  Per 32-query tile t:
//   P  wavefront:  S = Q~ K~^T, P = exp2(S log2(e)/sqrt(d) - LSE log2(e))
//                  (causally masked), P -> LDS exchange (fp32),
//                  dV~^T += dO~^T P;
//   dS wavefront:  dP = dO~ V~^T for tile t, and for tile t-1 (one barrier
//                  behind, so P(t-1) is in the exchange):
//                  dS = P o (dP - delta), dK~^T += Q~^T dS.
// Each wavefront issues 16 of the tile's 32 MFMAs.  Only the row-major Q~ and
// dO~ tiles are streamed: the transposed operands dO~^T and Q~^T come from the
// same LDS tiles through transposing reads (attn_tiles.h), which halves the
// bytes per tile -- the kernel is otherwise bound by streaming the query tiles
// (1 KB per query per 128 keys).  Tiles go through a ring of four LDS buffers
// (t-1: dS side, t: both, t+1: landed, t+2: filling), the exchange is
// double-buffered by tile parity.
constexpr int kKvPairs = 4;
constexpr int kKvWaves = 2 * kKvPairs;
constexpr int kKvThreads = 64 * kKvWaves;
constexpr int kKvBK = 32 * kKvPairs;   // keys per work-group
constexpr int kKvBQ = 32;              // query rows per tile
constexpr int kKvBufs = 4;             // tiles in LDS
constexpr int kXBytes = 16 * 4 * 64;   // one pair's P: 16 fp32 per lane

// One query tile in LDS: Q~ and dO~ rows, LSE log2(e) and delta of the rows.
template <int D>
struct DkvTile {
  static constexpr int WR = 2 * D;   // bytes per Q~ / dO~ row
  static constexpr int Q = 0;
  static constexpr int G = Q + kKvBQ * WR;
  static constexpr int LS = G + kKvBQ * WR;
  static constexpr int DL = LS + 4 * kKvBQ;
  static constexpr int BYTES = DL + 4 * kKvBQ;
};

template <int D>
__global__ __launch_bounds__(kKvThreads, 1) void k_attn_bwd_dkdv(int S, int Sv, int BH,
                                                                 const uint16_t *__restrict__ qt,
                                                                 const uint16_t *__restrict__ kt,
                                                                 const uint16_t *__restrict__ vt,
                                                                 const uint16_t *__restrict__ dotb,
                                                                 const float *__restrict__ rows,
                                                                 float *__restrict__ dkt, float *__restrict__ dvt) {
  using T = DkvTile<D>;
  constexpr int KC = D / 16, DB = D / 32;
  static_assert(4 * DB == 2 * KC, "as many dV/dK products as S/dP products");
  constexpr int QB = kKvBQ * T::WR / 1024;   // 1 KB fill blocks of a Q~ or dO~ tile
  static_assert(QB * 1024 == kKvBQ * T::WR && (kKvWaves % QB == 0 || QB % kKvWaves == 0), "fill blocks");
  constexpr int QBLK = (QB + kKvWaves - 1) / kKvWaves;   // blocks per wavefront (duplicated if QB < 8)
  constexpr int kFillOps = 2 * QBLK + 1;                  // loads per wavefront per fill
  __shared__ __attribute__((aligned(1024))) char lds[kKvBufs * T::BYTES + 2 * kKvPairs * kXBytes];
  char *xch = lds + kKvBufs * T::BYTES;
  const int h = blockIdx.x % BH;
  const int kb = blockIdx.x / BH;   // first key blocks see the most queries: launched first
  const int tid = threadIdx.x, lane = tid & 63, ln = lane & 31, hf = lane >> 5;
  const int wu = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int pair = wu % kKvPairs;   // wavefronts w and w + 4 share a SIMD
  const bool dsw = wu >= kKvPairs;  // the dS wavefront of the pair
  const int j0 = kb * kKvBK, kw = j0 + 32 * pair, kj = kw + ln;
  const long long hbS = (long long)h * S;    // dK~, dV~: S rows per head
  const long long hbV = (long long)h * Sv;   // Q~, K~, V~, dO~, row pairs: Sv rows per head (rows S..Sv-1 zero)
  const char *qh = reinterpret_cast<const char *>(qt + hbV * D);
  const char *gh = reinterpret_cast<const char *>(dotb + hbV * D);
  const char *rh = reinterpret_cast<const char *>(rows + 2 * hbV);
  const unsigned lbase = tiles::lds_addr(lds);

  // Fills (every wavefront issues the same number of loads; with fewer blocks
  // than wavefronts some blocks are loaded twice, identical bytes).  Query
  // tiles start below S and are 32 rows, so they never pass the padded Sv
  // rows; a padding query (zero Q~, dO~, LSE and delta) adds exactly 0.  The
  // row pairs (LSE log2 e, delta) are split on the way in: lane l < 32 loads
  // the LSE of row l, lane 32 + l its delta, so LS and DL are adjacent arrays.
  unsigned vq[QBLK];
  int bq[QBLK];
#pragma unroll
  for (int i = 0; i < QBLK; ++i) {
    bq[i] = (wu + i * kKvWaves) % QB;
    vq[i] = tiles::dma_voff<T::WR>(bq[i], T::WR);
  }
  const unsigned vrs = 8u * ln + 4u * hf;
  auto fill = [&](int jb, int q0) {
    const unsigned m = lbase + jb * T::BYTES;
#pragma unroll
    for (int i = 0; i < QBLK; ++i) {
      tiles::lds_load_s<16>(qh + (long long)q0 * T::WR, vq[i], m + T::Q + 1024u * bq[i]);
      tiles::lds_load_s<16>(gh + (long long)q0 * T::WR, vq[i], m + T::G + 1024u * bq[i]);
    }
    tiles::lds_load_s<4>(rh + 8LL * q0, vrs, m + T::LS);
  };

  // per-lane LDS read offsets: row-major operands (row ln, chunk 2c+hf) and
  // the transposing reads of query chunk 0 (chunk cc adds 16 cc rows), d block b
  int oq[KC], otr[DB][2];
#pragma unroll
  for (int c = 0; c < KC; ++c) oq[c] = tiles::tile_off<T::WR>(ln, 2 * c + hf);
#pragma unroll
  for (int b = 0; b < DB; ++b) {
    otr[b][0] = tiles::tr_off<T::WR>(0, 32 * b);
    otr[b][1] = tiles::tr_off<T::WR>(8, 32 * b);
  }
  // this lane's part of its pair's exchange slot: 16 fp32 as 4 x 16 bytes,
  // [k][lane] so that consecutive lanes hit consecutive bank groups
  const int ox = pair * kXBytes + 16 * lane;

  // this lane's key row of K~ (P wavefront) or V~ (dS wavefront): B operand
  // of S = Q~ K~^T or dP = dO~ V~^T (keys past Sv read as zero)
  bf16x8 kv[KC];
  {
    const uint16_t *src = (dsw ? vt : kt) + (hbV + kj) * D + 8 * hf;
#pragma unroll
    for (int c = 0; c < KC; ++c) kv[c] = (kj < Sv) ? *reinterpret_cast<const bf16x8 *>(src + 16 * c) : (bf16x8){};
  }
  tiles::dma_wait();
  const float c2 = kLog2e / sqrtf((float)D);
  f32x16 acc[DB];   // dV~^T (P wavefront) or dK~^T (dS wavefront) of the pair's 32 keys
#pragma unroll
  for (int b = 0; b < DB; ++b) acc[b] = (f32x16){};

  const int nt = (S - j0 + kKvBQ - 1) / kKvBQ;   // query tiles from the block's first key to S
  const int qlast = j0 + (nt - 1) * kKvBQ;       // first query of the last tile
  fill(0, j0);
  fill(1, min(j0 + kKvBQ, qlast));
  tiles::wait_fills_barrier<kFillOps>();   // tile 0 landed

  // fragment reads of a phase are all issued before its first product, so
  // the LDS latency is paid once per phase rather than once per product
  auto rowfr = [&](const char *tile, bf16x8 (&f)[KC]) {
#pragma unroll
    for (int c = 0; c < KC; ++c) f[c] = tiles::lds_frag(tile, oq[c]);
  };
  auto colfr = [&](const char *tile, bf16x8 (&f)[KC]) {
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      const int cc = c / DB, b = c % DB;
      f[c] = tiles::tr_frag(tile + 16 * cc * T::WR, otr[b][0], otr[b][1]);
    }
  };
  // The P wavefront's runs of products are issued at raised wave priority (its
  // P feeds the dS wavefront one tile later); measured 3-4% faster than equal
  // priorities, while raising the dS wavefront's instead was slower.
  auto rowmm = [&](const bf16x8 (&f)[KC]) {
    f32x16 r = (f32x16){};
    if (!dsw) __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int c = 0; c < KC; ++c) r = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f[c], kv[c], r, 0, 0, 0);
    if (!dsw) __builtin_amdgcn_s_setprio(0);
    return r;
  };
  auto colmm = [&](const bf16x8 (&f)[KC], const bf16x8 *x) {
    if (!dsw) __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int c = 0; c < KC; ++c)
      acc[c % DB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f[c], x[c / DB], acc[c % DB], 0, 0, 0);
    if (!dsw) __builtin_amdgcn_s_setprio(0);
  };

  if (!dsw) {
    // ---- P wavefront: S, P, exchange, dV ----
    auto iter_p = [&](int t, auto mask) {
      constexpr bool MASK = decltype(mask)::value;
      const int q0 = j0 + t * kKvBQ;
      const char *cur = lds + (t % kKvBufs) * T::BYTES;
      fill((t + 2) % kKvBufs, min(q0 + 2 * kKvBQ, qlast));   // past the end: a repeat of the last tile
      bf16x8 fq[KC], fg[KC];
      rowfr(cur + T::Q, fq);
      float4 l4[4];   // LSE log2 e of rows 8 g4 + 4 hf + 0..3
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) l4[g4] = *reinterpret_cast<const float4 *>(cur + T::LS + 4 * (8 * g4 + 4 * hf));
      colfr(cur + T::G, fg);
      __builtin_amdgcn_sched_barrier(0);
      const f32x16 sv = rowmm(fq);
      float p[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int g4 = i >> 2, e = i & 3;
        const float ls = e == 0 ? l4[g4].x : e == 1 ? l4[g4].y : e == 2 ? l4[g4].z : l4[g4].w;
        p[i] = __builtin_amdgcn_exp2f(fmaf(sv[i], c2, -ls));
        if constexpr (MASK) {
          if (q0 + 8 * g4 + 4 * hf + e < kj) p[i] = 0.f;
        }
      }
      char *x = xch + (t & 1) * (kKvPairs * kXBytes) + ox;
#pragma unroll
      for (int k = 0; k < 4; ++k)
        *reinterpret_cast<float4 *>(x + 1024 * k) = make_float4(p[4 * k], p[4 * k + 1], p[4 * k + 2], p[4 * k + 3]);
      bf16x8 pf[2];
#pragma unroll
      for (int i = 0; i < 16; ++i) pf[i >> 3][i & 7] = (__bf16)p[i];
      colmm(fg, pf);   // dV~^T += dO~^T P
      tiles::wait_fills_barrier<kFillOps>();   // tile t+1 landed
    };
    const int nm = min(nt, kKvBK / kKvBQ);   // tiles that reach below some key of the block: masked
    for (int t = 0; t < nm; ++t) iter_p(t, Flag<true>{});
    for (int t = nm; t < nt; ++t) iter_p(t, Flag<false>{});
  } else {
    // ---- dS wavefront: dP of tile t; dS and dK of tile t-1 ----
    f32x16 dpp = (f32x16){};   // dP of the previous tile
    auto ds_dk = [&](int t, const bf16x8 (&fq)[KC], const float4 (&p4)[4], const float4 (&d4)[4]) {
      bf16x8 dsf[2];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int g4 = i >> 2, e = i & 3;
        const float pj = e == 0 ? p4[g4].x : e == 1 ? p4[g4].y : e == 2 ? p4[g4].z : p4[g4].w;
        const float dl = e == 0 ? d4[g4].x : e == 1 ? d4[g4].y : e == 2 ? d4[g4].z : d4[g4].w;
        dsf[i >> 3][i & 7] = (__bf16)(pj * (dpp[i] - dl));
      }
      colmm(fq, dsf);   // dK~^T += Q~^T dS
    };
    auto ds_reads = [&](int t, bf16x8 (&fq)[KC], float4 (&p4)[4], float4 (&d4)[4]) {
      const char *tb = lds + (t % kKvBufs) * T::BYTES;
      const char *x = xch + (t & 1) * (kKvPairs * kXBytes) + ox;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        p4[k] = *reinterpret_cast<const float4 *>(x + 1024 * k);
        d4[k] = *reinterpret_cast<const float4 *>(tb + T::DL + 4 * (8 * k + 4 * hf));
      }
      colfr(tb + T::Q, fq);
    };
    for (int t = 0; t < nt; ++t) {
      const int q0 = j0 + t * kKvBQ;
      const char *cur = lds + (t % kKvBufs) * T::BYTES;
      fill((t + 2) % kKvBufs, min(q0 + 2 * kKvBQ, qlast));
      bf16x8 fq[KC], fg[KC];
      float4 p4[4], d4[4];
      if (t > 0) ds_reads(t - 1, fq, p4, d4);
      rowfr(cur + T::G, fg);
      __builtin_amdgcn_sched_barrier(0);
      if (t > 0) ds_dk(t - 1, fq, p4, d4);
      dpp = rowmm(fg);   // dP = dO~ V~^T
      tiles::wait_fills_barrier<kFillOps>();
    }
    {
      bf16x8 fq[KC];
      float4 p4[4], d4[4];
      ds_reads(nt - 1, fq, p4, d4);
      ds_dk(nt - 1, fq, p4, d4);
    }
  }
  tiles::dma_wait();   // the fills past the last tile, before the work-group exits

  if (kj >= S) return;
  const float scale = dsw ? 1.f / sqrtf((float)D) : 1.f;
  float *orow = (dsw ? dkt : dvt) + (hbS + kj) * D;
#pragma unroll
  for (int b = 0; b < DB; ++b)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int dd = 32 * b + 8 * g + 4 * hf;
      *reinterpret_cast<float4 *>(orow + dd) = make_float4(acc[b][4 * g] * scale, acc[b][4 * g + 1] * scale,
                                                           acc[b][4 * g + 2] * scale, acc[b][4 * g + 3] * scale);
    }
}

}  // namespace

hipError_t launch_attn_bwd_mfma(int d, int BH, int S, int Sv, const void *qt, const void *kt, const void *vt,
                                const void *dotb, const float *rows, float *dqt, float *dkt, float *dvt, int part,
                                hipStream_t st) {
  const uint16_t *q = (const uint16_t *)qt, *k = (const uint16_t *)kt, *v = (const uint16_t *)vt;
  const uint16_t *g = (const uint16_t *)dotb;
  dim3 gq(((S + kDqBM - 1) / kDqBM) * BH), gk(((S + kKvBK - 1) / kKvBK) * BH);
  if (part == 0) {   // dQ~
    if (d == 128) lh::launch(k_attn_bwd_dq<128>, gq, kDqThreads, 0, st, S, Sv, BH, q, k, v, g, rows, dqt);
    else lh::launch(k_attn_bwd_dq<64>, gq, kDqThreads, 0, st, S, Sv, BH, q, k, v, g, rows, dqt);
  } else {           // dK~, dV~
    if (d == 128) lh::launch(k_attn_bwd_dkdv<128>, gk, kKvThreads, 0, st, S, Sv, BH, q, k, v, g, rows, dkt, dvt);
    else lh::launch(k_attn_bwd_dkdv<64>, gk, kKvThreads, 0, st, S, Sv, BH, q, k, v, g, rows, dkt, dvt);
  }
  return hipGetLastError();
}

}  // namespace lh
