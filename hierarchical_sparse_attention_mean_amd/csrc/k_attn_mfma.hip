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
// running max, sum and rescale factor are per-lane scalars.  V~^T comes
// pre-transposed from the gather ([d][Sv], Sv a multiple of 64, zero padded,
// columns in the perm16 order of attn_tiles.h) so both LDS operands are single
// 16-byte reads per lane.
//
// Work-group: 8 wavefronts x 32 queries = 256 query rows (one work-group per
// CU); key/value tiles of 64 rows, double-buffered in LDS and filled by direct
// global->LDS loads (attn_tiles.h): the next tile streams in while the current
// one is computed, with no registers spent on it.
// Softmax: exp2 with log2(e)/sqrt(d) folded into one FMA; the accumulators are
// rescaled only on tiles where some lane's running max grows (after the first
// few tiles most do not).  The running max is kept exact, so each row's
// largest probability is exactly 1 and is not perturbed by the bf16 rounding
// of P.  Work-groups are numbered head-fastest (block b -> head b mod BH)
// and longest query blocks first: with BH a multiple of 8 a head's blocks share
// one XCD's L2, and the causal tail is balanced.
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

template <int D>
struct FwdTile {
  static constexpr int WK = 2 * D;    // bytes per K~ row
  static constexpr int WV = 2 * BN;   // bytes per V~^T row
  char k[BN * WK];
  char v[D * WV];
};

template <int D>
__global__ __launch_bounds__(kThreads, 1) void k_attn_fwd_mfma(int S, int Sq, int Sv, int BH,
                                                               const uint16_t *__restrict__ qt,
                                                               const uint16_t *__restrict__ kt,
                                                               const uint16_t *__restrict__ vtt,
                                                               float *__restrict__ ot, float *__restrict__ lse) {
  using Tile = FwdTile<D>;
  constexpr int KC = D / 16;   // 16-wide d chunks of the Q.K contraction
  constexpr int DB = D / 32;   // 32-row d blocks of O^T
  __shared__ __attribute__((aligned(1024))) Tile buf[2];

  const int nqb = (S + BM - 1) / BM;
  const int h = blockIdx.x % BH;
  const int qb = nqb - 1 - blockIdx.x / BH;
  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, ln = lane & 31, hf = lane >> 5;
  const int q0 = qb * BM;
  const int qw = q0 + 32 * w;   // first query of this wavefront
  const int qi = qw + ln;       // this lane's query
  const long long hbS = (long long)h * S;   // O~, LSE: S rows per head
  const uint16_t *qh = qt + (long long)h * Sq * D;   // Q~, K~: Sq rows per head
  const char *kh = reinterpret_cast<const char *>(kt + (long long)h * Sq * D);
  const char *vh = reinterpret_cast<const char *>(vtt + (long long)h * D * Sv);

  // K~ rows past S are clamped to row S-1 (finite; those keys are causally masked);
  // V~^T columns past S are the zero padding up to Sv.
  auto fill = [&](Tile &t, int k0) {
    tiles::dma_tile<Tile::WK, BN, kThreads>(t.k, kh + (long long)k0 * Tile::WK, Tile::WK, S - 1 - k0);
    tiles::dma_tile<Tile::WV, D, kThreads>(t.v, vh + 2LL * k0, 2LL * Sv, D - 1);
  };

  // Q~ fragment: B operand of S^T = K~ Q~^T (lane: query qi, d = 16c + 8hf .. +7)
  bf16x8 qf[KC];
#pragma unroll
  for (int c = 0; c < KC; ++c)
    qf[c] = (qi < S) ? *reinterpret_cast<const bf16x8 *>(qh + (long long)qi * D + 16 * c + 8 * hf) : (bf16x8){};
  f32x16 acc[DB];
#pragma unroll
  for (int b = 0; b < DB; ++b) acc[b] = (f32x16){};
  const float c2 = kLog2e / sqrtf((float)D);
  float m = -INFINITY;   // running max of the scaled logits (log2 units)
  float l = 0.f;         // running sum of this half-wave's probabilities

  const int kend = min(S, q0 + BM);
  const int nt = (kend + BN - 1) / BN;
  fill(buf[0], 0);
  tiles::dma_wait();
  __syncthreads();
  for (int t = 0; t < nt; ++t) {
    const int k0 = t * BN;
    if (t + 1 < nt) fill(buf[(t + 1) & 1], k0 + BN);   // streams in while this tile is computed
    const Tile &cur = buf[t & 1];
    if (k0 <= qw + 31) {   // otherwise the whole tile is in this wavefront's future
      f32x16 st[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        st[kb] = (f32x16){};
#pragma unroll
        for (int c = 0; c < KC; ++c)
          st[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              tiles::lds_frag(cur.k, tiles::tile_off<Tile::WK>(32 * kb + ln, 2 * c + hf)), qf[c], st[kb], 0, 0, 0);
      }
      if (k0 + BN - 1 > qw) {   // tile reaches past this wavefront's first query: causal mask
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
      // probabilities, bf16 B operand chunks of 16 keys
      bf16x8 pf[4];
#pragma unroll
      for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float pj = __builtin_amdgcn_exp2f(fmaf(st[c >> 1][8 * (c & 1) + j], c2, -m));
          l += pj;
          pf[c][j] = (__bf16)pj;
        }
      // O^T += V~^T P^T
#pragma unroll
      for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int b = 0; b < DB; ++b)
          acc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              tiles::lds_frag(cur.v, tiles::tile_off<Tile::WV>(32 * b + ln, 2 * c + hf)), pf[c], acc[b], 0, 0, 0);
    }
    tiles::dma_wait();
    __syncthreads();
  }
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

hipError_t launch_attn_fwd_mfma(int d, int BH, int S, int Sq, int vstride, const void *qt, const void *kt, const void *vtt,
                                float *ot, float *lse, hipStream_t st) {
  const int nqb = (S + BM - 1) / BM;
  dim3 grid(nqb * BH);
  if (d == 128)
    k_attn_fwd_mfma<128><<<grid, kThreads, 0, st>>>(S, Sq, vstride, BH, (const uint16_t *)qt, (const uint16_t *)kt,
                                                    (const uint16_t *)vtt, ot, lse);
  else
    k_attn_fwd_mfma<64><<<grid, kThreads, 0, st>>>(S, Sq, vstride, BH, (const uint16_t *)qt, (const uint16_t *)kt,
                                                   (const uint16_t *)vtt, ot, lse);
  return hipGetLastError();
}

}  // namespace lh
