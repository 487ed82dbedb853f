// Causal softmax attention over the gathered sub-sequence on bf16 MFMA (gfx950).
//
// "Long Context Pre-Training with Lighthouse Attention", Sec. 3.5, Eq. (9):
// plain masked softmax attention on the topologically sorted sub-sequence; the
// mask is the standard causal one and the scale is 1/sqrt(d) (Sec. 3.1, Eq. 1).
// The paper hands this step to stock FlashAttention; this is a hand-written
// gfx950 kernel with the same online-softmax structure.
//
// Orientation.  Each wavefront owns 32 query rows and computes the transposed
// logits S^T = K~ Q~^T with v_mfma_f32_32x32x16_bf16: in the 32x32 result a lane
// holds one query column and 16 key rows, so the softmax max / sum over keys is
// in-lane plus one exchange between the two half-waves.  The probabilities P^T
// (converted to bf16) are then the B operand, straight from registers, of
// O^T += V~^T P^T, whose result again gives each lane one query column -- the
// running max, sum and rescale factor are per-lane scalars.  Both K~ and V~
// are staged as row-major tiles; the V~^T operand comes from the V~ tile by
// transposing LDS reads in the key order of the probability registers
// (attn_tiles.h).
//
// Work-group: 8 wavefronts x 32 queries = 256 query rows (one work-group per
// CU); key/value tiles of 64 rows in a ring of four LDS buffers filled by
// direct global->LDS loads (attn_tiles.h) three tiles ahead, so a fill has two
// tiles' time to land.  Each wavefront streams its LDS operands through a
// window of W fragments in registers: every MFMA consumes the oldest and the
// read of the fragment W places later is issued right after it, in a fixed
// order (scheduling barriers), so the LDS latency is covered by W products;
// near a tile's end the window already reads the next tile, whose fill has
// landed.  The loop body has no branch except the rescale.
// Softmax: exp2 with log2(e)/sqrt(d) folded into one FMA; the accumulators are
// rescaled only on tiles where some lane's running max grows (after the first
// few tiles most do not).  The running max is kept exact, so each row's
// largest probability is exactly 1 and is not perturbed by the bf16 rounding
// of P.  The causal mask is applied on the last four tiles of a work-group
// only (the tiles that reach its first query); tiles past a wavefront's own
// queries are computed fully masked (probabilities exactly 0).  Work-groups
// are numbered head-fastest (block b -> head b mod BH) and longest query
// blocks first: with BH a multiple of 8 a head's blocks share one XCD's L2,
// and the causal tail is balanced.
#include "attn_tiles.h"

namespace lh {

namespace {

using tiles::bf16x8;
using tiles::f32x16;

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int BM = 32 * kWaves;   // query rows per work-group
constexpr int BN = 64;            // key rows per tile
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

constexpr int kFwdBufs = 4;   // key/value tiles in LDS
constexpr int kWin = 8;       // LDS operand fragments in flight per wavefront

// One key/value tile in LDS: K~ rows, then V~ rows.
template <int D>
struct FwdTile {
  static constexpr int WK = 2 * D;   // bytes per K~ / V~ row
  static constexpr int K = 0;
  static constexpr int V = BN * WK;
  static constexpr int BYTES = 2 * BN * WK;
};

template <bool B>
struct Flag {
  static constexpr bool value = B;
};

template <int D>
__global__ __launch_bounds__(kThreads, 1) void k_attn_fwd_mfma(int S, int Sq, int BH,
                                                               const uint16_t *__restrict__ qt,
                                                               const uint16_t *__restrict__ kt,
                                                               const uint16_t *__restrict__ vt,
                                                               float *__restrict__ ot, float *__restrict__ lse) {
  using T = FwdTile<D>;
  constexpr int KC = D / 16;          // 16-wide d chunks of the Q.K contraction
  constexpr int DB = D / 32;          // 32-row d blocks of O^T
  constexpr int NS = 2 * KC;          // S^T products (= K~ fragments) per tile
  constexpr int NF = NS + 4 * DB;     // LDS operand fragments per tile: K~, then V~^T
  static_assert(NS + kWin <= NF, "the window reaches the next tile only in the O^T phase");
  constexpr int KBLK = BN * T::WK / 1024 / kWaves;   // 1 KB fill blocks per wavefront, K~ and V~ each
  static_assert(KBLK * 1024 * kWaves == BN * T::WK, "fill blocks");
  constexpr int kFillOps = 2 * KBLK;                 // loads per wavefront per fill
  __shared__ __attribute__((aligned(1024))) char lds[kFwdBufs * T::BYTES];

  const int nqb = (S + BM - 1) / BM;
  const int h = blockIdx.x % BH;
  const int qb = nqb - 1 - blockIdx.x / BH;
  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, ln = lane & 31, hf = lane >> 5;
  const int wu = __builtin_amdgcn_readfirstlane(w);
  const int q0 = qb * BM;
  const int qw = q0 + 32 * w;   // first query of this wavefront
  const int qi = qw + ln;       // this lane's query
  const long long hbS = (long long)h * S;   // O~, LSE: S rows per head
  const uint16_t *qh = qt + (long long)h * Sq * D;   // Q~, K~, V~: Sq rows per head
  const char *kh = reinterpret_cast<const char *>(kt + (long long)h * Sq * D);
  const char *vh = reinterpret_cast<const char *>(vt + (long long)h * Sq * D);
  const unsigned lbase = tiles::lds_addr(lds);

  // Fills.  K~ and V~ rows past S are clamped to row S-1 (finite; those keys
  // are causally masked: probability exactly 0).
  int kr[KBLK];
  unsigned kc[KBLK];
#pragma unroll
  for (int i = 0; i < KBLK; ++i) {
    const int byte = (wu + i * kWaves) * 1024 + 16 * lane;
    kr[i] = byte / T::WK;
    kc[i] = 16u * (((byte % T::WK) / 16) ^ tiles::swz<T::WK>(kr[i]));
  }
  auto fill = [&](int jb, int k0) {
    const unsigned m = lbase + jb * T::BYTES;
    const int rclamp = S - 1 - k0;
#pragma unroll
    for (int i = 0; i < KBLK; ++i) {
      const unsigned vo = (unsigned)min(kr[i], rclamp) * T::WK + kc[i];
      tiles::lds_load_s<16>(kh + (long long)k0 * T::WK, vo, m + T::K + 1024u * (wu + i * kWaves));
      tiles::lds_load_s<16>(vh + (long long)k0 * T::WK, vo, m + T::V + 1024u * (wu + i * kWaves));
    }
  };

  // LDS operand fragment j of a tile: K~ rows 32 kb + ln, chunk 2c + hf
  // (j = kb KC + c; the swizzle of row 32 x + ln equals that of row ln, so the
  // per-lane offset depends on c only), then V~^T d rows 32 b + ln over the 16
  // keys of chunk c (j = NS + c DB + b): two transposing reads of the V~ tile.
  int ok[KC], ov[DB][2];
#pragma unroll
  for (int c = 0; c < KC; ++c) ok[c] = tiles::tile_off<T::WK>(ln, 2 * c + hf);
#pragma unroll
  for (int b = 0; b < DB; ++b) {
    ov[b][0] = tiles::tr_off<T::WK>(0, 32 * b);
    ov[b][1] = tiles::tr_off<T::WK>(8, 32 * b);
  }
  auto frag = [&](const char *buf, int j) -> bf16x8 {
    if (j < NS) return tiles::lds_frag(buf + T::K + 32 * (j / KC) * T::WK, ok[j % KC]);
    const int jj = j - NS, c = jj / DB, b = jj % DB;
    return tiles::tr_frag(buf + T::V + 16 * c * T::WK, ov[b][0], ov[b][1]);
  };

  // Q~ fragment: B operand of S^T = K~ Q~^T (lane: query qi, d = 16c + 8hf .. +7)
  bf16x8 qf[KC];
#pragma unroll
  for (int c = 0; c < KC; ++c)
    qf[c] = (qi < S) ? *reinterpret_cast<const bf16x8 *>(qh + (long long)qi * D + 16 * c + 8 * hf) : (bf16x8){};
  // wait for them here: first used inside the loop, they would otherwise make
  // the compiler wait for every outstanding load (the fills) on each iteration
  tiles::dma_wait();
  f32x16 acc[DB];
#pragma unroll
  for (int b = 0; b < DB; ++b) acc[b] = (f32x16){};
  const float c2 = kLog2e / sqrtf((float)D);
  float m = -INFINITY;   // running max of the scaled logits (log2 units)
  float l = 0.f;         // running sum of this half-wave's probabilities

  const int kend = min(S, q0 + BM);
  const int nt = (kend + BN - 1) / BN;
  const int klast = (nt - 1) * BN;
  fill(0, 0);
  fill(1, min(BN, klast));
  fill(2, min(2 * BN, klast));
  tiles::wait_fills_barrier<kFillOps>();   // tiles 0 and 1 landed
  bf16x8 win[kWin];
#pragma unroll
  for (int j = 0; j < kWin; ++j) win[j] = frag(lds, j);

  auto iteration = [&](int t, auto mask) {
    constexpr bool MASK = decltype(mask)::value;
    const int k0 = t * BN;
    fill((t + 3) & (kFwdBufs - 1), min(k0 + 3 * BN, klast));   // past the end: a repeat of the last tile
    const char *cur = lds + (t & (kFwdBufs - 1)) * T::BYTES;
    const char *nxt = lds + ((t + 1) & (kFwdBufs - 1)) * T::BYTES;
    // S^T = K~ Q~^T for the 64 keys of the tile (lane = query, 2 x 16 keys)
    f32x16 st[2] = {(f32x16){}, (f32x16){}};
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      st[j / KC] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(win[j % kWin], qf[j % KC], st[j / KC], 0, 0, 0);
      win[j % kWin] = frag(cur, j + kWin);
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (MASK) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = k0 + 32 * kb + 8 * (i >> 2) + 4 * hf + (i & 3);
          if (key > qi) st[kb][i] = -INFINITY;
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, st[kb][i]);
    mx = fmaxf(mx, __shfl_xor(mx, 32)) * c2;
    // rescale only if some lane's running max grows
    const bool grow = mx > m;
    if (__ballot(grow)) {
      const float mnew = grow ? mx : m;
      const float alpha = __builtin_amdgcn_exp2f(m - mnew);   // 0 when m = -inf, 1 when unchanged
      m = mnew;
      l *= alpha;
#pragma unroll
      for (int b = 0; b < DB; ++b) acc[b] *= alpha;
    }
    // probabilities, bf16 B operand chunks of 16 keys (fully masked keys: exactly 0)
    bf16x8 pf[4];
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float pj = __builtin_amdgcn_exp2f(fmaf(st[c >> 1][8 * (c & 1) + j], c2, -m));
        l += pj;
        pf[c][j] = (__bf16)pj;
      }
    // O^T += V~^T P^T; the window moves on into the next tile
#pragma unroll
    for (int j = NS; j < NF; ++j) {
      const int jj = j - NS;
      acc[jj % DB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(win[j % kWin], pf[jj / DB], acc[jj % DB], 0, 0, 0);
      win[j % kWin] = (j + kWin < NF) ? frag(cur, j + kWin) : frag(nxt, j + kWin - NF);
      __builtin_amdgcn_sched_barrier(0);
    }
    // tile t+2 landed; tile t+3 in flight; the window's reads (tile t+1) stay in flight
    tiles::wait_fills_barrier_keep<kFillOps, kWin>();
  };
  const int nu = max(0, nt - BM / BN);   // tiles before the block's first query: no mask
  for (int t = 0; t < nu; ++t) iteration(t, Flag<false>{});
  for (int t = nu; t < nt; ++t) iteration(t, Flag<true>{});
  tiles::dma_wait();   // the fills past the last tile, before the work-group exits

  if (qi >= S) return;
  const float lt = l + __shfl_xor(l, 32);
  const float inv = 1.f / lt;
  float *orow = ot + (hbS + qi) * D;
#pragma unroll
  for (int b = 0; b < DB; ++b)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int dd = 32 * b + 8 * g + 4 * hf;
      *reinterpret_cast<float4 *>(orow + dd) =
          make_float4(acc[b][4 * g] * inv, acc[b][4 * g + 1] * inv, acc[b][4 * g + 2] * inv, acc[b][4 * g + 3] * inv);
    }
  if (hf == 0 && lse) lse[hbS + qi] = (m + __log2f(lt)) * kLn2;
}

}  // namespace

hipError_t launch_attn_fwd_mfma(int d, int BH, int S, int Sq, const void *qt, const void *kt, const void *vt,
                                float *ot, float *lse, hipStream_t st) {
  const int nqb = (S + BM - 1) / BM;
  dim3 grid(nqb * BH);
  if (d == 128)
    lh::launch(k_attn_fwd_mfma<128>, grid, kThreads, 0, st, S, Sq, BH, (const uint16_t *)qt, (const uint16_t *)kt,
                                                    (const uint16_t *)vt, ot, lse);
  else
    lh::launch(k_attn_fwd_mfma<64>, grid, kThreads, 0, st, S, Sq, BH, (const uint16_t *)qt, (const uint16_t *)kt,
                                                   (const uint16_t *)vt, ot, lse);
  return hipGetLastError();
}

}  // namespace lh
