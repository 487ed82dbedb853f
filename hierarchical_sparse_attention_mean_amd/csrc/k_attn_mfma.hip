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
// pre-transposed from the gather ([d][Sv], Sv a multiple of 64, zero padded) so
// both LDS operands are read as contiguous rows.
//
// Work-group: 8 wavefronts x 32 queries = 256 query rows (one work-group per
// CU); key/value tiles of 64 rows, double-buffered in LDS, the next tile's
// global loads in flight in registers while the current tile is computed.
// Softmax: exp2 with log2(e)/sqrt(d) folded into one FMA; the accumulators are
// rescaled only on tiles where some lane's running max grows (after the first
// few tiles most do not).  The running max is kept exact, so each row's
// largest probability is exactly 1 and is not perturbed by the bf16 rounding
// of P.  Work-groups are numbered head-fastest (block b -> head b mod BH)
// and longest query blocks first: with BH a multiple of 8 a head's blocks share
// one XCD's L2, and the causal tail is balanced.
#include "lh_internal.h"

namespace lh {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int BM = 32 * kWaves;   // query rows per work-group
constexpr int BN = 64;            // key rows per tile
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

template <int D>
struct FwdTile {
  static constexpr int KS = D + 8;              // padded K~ row stride (bf16)
  static constexpr int VS = BN + 4;             // padded V~^T row stride (bf16)
  static constexpr int KCH = BN * D / 8;        // 16-byte chunks per K~ tile
  static constexpr int VCH = D * BN / 8;        // 16-byte chunks per V~^T tile
  static constexpr int KPT = KCH / kThreads;    // chunks per thread
  static constexpr int VPT = VCH / kThreads;
  uint16_t k[BN * KS];
  uint16_t v[D * VS];
};

template <int D>
__global__ __launch_bounds__(kThreads, 1) void k_attn_fwd_mfma(int S, int Sv, int BH, const uint16_t *__restrict__ qt,
                                                               const uint16_t *__restrict__ kt,
                                                               const uint16_t *__restrict__ vtt,
                                                               float *__restrict__ ot, float *__restrict__ lse) {
  using Tile = FwdTile<D>;
  constexpr int KC = D / 16;   // 16-wide d chunks of the Q.K contraction
  constexpr int DB = D / 32;   // 32-row d blocks of O^T
  __shared__ __attribute__((aligned(16))) Tile buf[2];

  const int nqb = (S + BM - 1) / BM;
  const int h = blockIdx.x % BH;
  const int qb = nqb - 1 - blockIdx.x / BH;
  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, ln = lane & 31, hf = lane >> 5;
  const int q0 = qb * BM;
  const int qw = q0 + 32 * w;   // first query of this wavefront
  const int qi = qw + ln;       // this lane's query
  const long long hbS = (long long)h * S;
  const uint16_t *qh = qt + hbS * D;
  const uint16_t *kh = kt + hbS * D;
  const uint16_t *vh = vtt + (long long)h * D * Sv;

  // global -> registers for one tile (rows past S read as zero)
  uint4 kreg[Tile::KPT], vreg[Tile::VPT];
  auto load_tile = [&](int k0) {
#pragma unroll
    for (int it = 0; it < Tile::KPT; ++it) {
      const int idx = it * kThreads + tid;
      const int r = idx / (D / 8), cc = idx % (D / 8);
      kreg[it] = (k0 + r < S) ? *reinterpret_cast<const uint4 *>(kh + (long long)(k0 + r) * D + cc * 8)
                              : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int it = 0; it < Tile::VPT; ++it) {
      const int idx = it * kThreads + tid;
      const int r = idx / (BN / 8), cc = idx % (BN / 8);   // r = d row, cc = 8-key chunk
      vreg[it] = *reinterpret_cast<const uint4 *>(vh + (long long)r * Sv + k0 + cc * 8);
    }
  };
  auto store_tile = [&](Tile &t) {
#pragma unroll
    for (int it = 0; it < Tile::KPT; ++it) {
      const int idx = it * kThreads + tid;
      const int r = idx / (D / 8), cc = idx % (D / 8);
      *reinterpret_cast<uint4 *>(&t.k[r * Tile::KS + cc * 8]) = kreg[it];
    }
#pragma unroll
    for (int it = 0; it < Tile::VPT; ++it) {
      const int idx = it * kThreads + tid;
      const int r = idx / (BN / 8), cc = idx % (BN / 8);
      uint2 *dst = reinterpret_cast<uint2 *>(&t.v[r * Tile::VS + cc * 8]);
      dst[0] = make_uint2(vreg[it].x, vreg[it].y);
      dst[1] = make_uint2(vreg[it].z, vreg[it].w);
    }
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
  load_tile(0);
  store_tile(buf[0]);
  __syncthreads();
  for (int t = 0; t < nt; ++t) {
    const int k0 = t * BN;
    if (t + 1 < nt) load_tile(k0 + BN);
    const Tile &cur = buf[t & 1];
    if (k0 <= qw + 31) {   // otherwise the whole tile is in this wavefront's future
      f32x16 st[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        st[kb] = (f32x16){};
#pragma unroll
        for (int c = 0; c < KC; ++c) {
          const bf16x8 a = *reinterpret_cast<const bf16x8 *>(&cur.k[(32 * kb + ln) * Tile::KS + 16 * c + 8 * hf]);
          st[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[c], st[kb], 0, 0, 0);
        }
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
        for (int b = 0; b < DB; ++b) {
          const uint16_t *row = &cur.v[(32 * b + ln) * Tile::VS + 16 * c + 4 * hf];
          const bf16x4 lo = *reinterpret_cast<const bf16x4 *>(row);
          const bf16x4 hi = *reinterpret_cast<const bf16x4 *>(row + 8);
          const bf16x8 a = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
          acc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[c], acc[b], 0, 0, 0);
        }
    }
    if (t + 1 < nt) store_tile(buf[(t + 1) & 1]);
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

hipError_t launch_attn_fwd_mfma(int d, int BH, int S, int vstride, const void *qt, const void *kt, const void *vtt,
                                float *ot, float *lse, hipStream_t st) {
  const int nqb = (S + BM - 1) / BM;
  dim3 grid(nqb * BH);
  if (d == 128)
    k_attn_fwd_mfma<128><<<grid, kThreads, 0, st>>>(S, vstride, BH, (const uint16_t *)qt, (const uint16_t *)kt,
                                                    (const uint16_t *)vtt, ot, lse);
  else
    k_attn_fwd_mfma<64><<<grid, kThreads, 0, st>>>(S, vstride, BH, (const uint16_t *)qt, (const uint16_t *)kt,
                                                   (const uint16_t *)vtt, ot, lse);
  return hipGetLastError();
}

}  // namespace lh
