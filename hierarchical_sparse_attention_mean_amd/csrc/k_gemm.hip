// Dense products of the projection-inclusive layer ("Long Context Pre-Training
// with Lighthouse Attention", Sec. 3.1: Q, K and V are the per-head projections
// X W_Q, X W_K, X W_V of the layer input; Sec. 3.2: the gradient reaches the
// projections through the attention, so the backward needs dX and every dW):
//
//   C[m][n] = sum_k A[m][k] B[k][n]      (fp32 accumulation)
//
// over matrices addressed through MatView (lh_internal.h), so that the head
// layout [B][H][N][d] of Q, K, V, O and their gradients is read and written in
// place as the [N][H d] matrix of the layer, and the three projection matrices
// act as one [d_model][3 H d] matrix.  Operands come in two memory orders:
// "k-major" (the contraction index is the contiguous one: X as the left factor
// of X W, W_O^T, W^T) and "mn-major" (the output index is contiguous: W, and X
// and dQ as the factors of X^T dQ).  No operand is ever transposed in memory.
//
// bf16 (k_gemm_mfma): v_mfma_f32_32x32x16_bf16 on 256 x 256 output tiles, 8
//   wavefronts of 128 (n) x 64 (m) each.  The product is formed transposed,
//   D = C^T (A slot: rows n of B^T, B slot: columns m of A^T), so that each lane
//   holds one output row m and four consecutive n per store.  Tiles of 32
//   contraction steps go global -> LDS by direct loads (global_load_lds, no
//   registers) through a ring of four stages filled three ahead.  k-major tiles
//   are 256 rows of 64 bytes (operand reads ds_read_b128); mn-major tiles are
//   four 32 x 64 sub-tiles of 128-byte rows read with transposing reads
//   (ds_read_b64_tr_b16), two per operand, each giving 4 consecutive k.  Both
//   read kinds hand an MFMA lane the 8 consecutive contraction indices
//   16 kk + 8 hf + 0..7, so k-major and mn-major operands mix freely.
//   Work-groups are numbered XCD-aware: work-group i runs on XCD i mod 8, and
//   the tiles an XCD runs at one time share rows of A and columns of B in its L2.
// fp32 (k_gemm_f32): a plain LDS-tiled vector-ALU product, for the fp32 layer.
// Split-K (the weight gradients contract over all B N tokens): each split writes
// an fp32 partial product, and k_split_reduce adds the partials in split order
// -- deterministic, no atomics.
#include "attn_tiles.h"

namespace lh {

namespace {

using tiles::bf16x8;
using tiles::f32x16;

constexpr int kGThreads = 512;                 // 8 wavefronts
constexpr int kGBM = 256, kGBN = 256;          // output tile
constexpr int kGBK = 32;                       // contraction steps per stage
constexpr int kGStages = 4;                    // LDS ring
constexpr int kGOpBytes = kGBM * kGBK * 2;     // one operand's tile: 16 KB
constexpr int kGStageBytes = 2 * kGOpBytes;    // A then B
constexpr int kGFillOps = 4;                   // 1 KB loads per wavefront per stage (2 per operand)
constexpr int kGGroup = 4;                     // m-tiles an XCD walks together over all n-tiles
static_assert(kGOpBytes / 1024 == 2 * (kGThreads / 64), "two 1 KB blocks per wavefront per operand");

// A view's three base pointers as wave-uniform values: held in scalar
// registers, so that choosing one per stage is a select, not a reload from the
// kernel arguments (a scalar load, whose wait would also wait for every LDS read
// in flight).
// A pointer that is the same in every lane, as a scalar-register value (the
// compiler may form uniform 64-bit address arithmetic on the vector ALUs; the
// DMA's base operand must be scalar registers).
__device__ __forceinline__ const char *uniform_ptr(const void *q) {
  const unsigned long long a = (unsigned long long)q;
  const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)a);
  const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)(a >> 32));
  return reinterpret_cast<const char *>(((unsigned long long)hi << 32) | lo);
}

// (Three members rather than an array: an array indexed by a computed value
// would be placed in scratch memory.)
struct Bases {
  const char *p0, *p1, *p2;
  __device__ __forceinline__ explicit Bases(const MatView &v)
      : p0(uniform_ptr(v.p[0])), p1(uniform_ptr(v.p[1])), p2(uniform_ptr(v.p[2])) {}
  __device__ __forceinline__ const char *pick(unsigned which) const {
    return which == 0 ? p0 : which == 1 ? p1 : p2;
  }
};

// The global-memory address space, so that stores through computed pointers are
// global stores (not flat ones, which would also count as LDS operations).
typedef __attribute__((address_space(1))) char gchar;
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Byte pointer of view element (r, c) of batch element b (c inside one column
// block of the view; all arguments the same in every lane).
template <int ES>
__device__ __forceinline__ const char *vptr(const MatView &v, const Bases &bs, int b, long long r, unsigned c) {
  const unsigned which = c / (unsigned)v.seg, cc = c - which * (unsigned)v.seg;
  const unsigned h = cc / (unsigned)v.hd, j = cc - h * (unsigned)v.hd;
  return bs.pick(which) + (long long)ES * ((long long)b * v.bstride + (long long)h * v.hstride + r * v.ld + (long long)j);
}

// Per-lane byte offset, in a tile of W-byte bf16 rows, of the transposing read
// that gives lane (ln, hf) column c0 + ln of rows r0 + 8 hf + 0..3 (lanes
// 4k + m of each 16-lane group address row r0 + 8 hf + k, columns
// c0 + 16 (group & 1) + 4 m .. +3).  The read at rows +4 (offset tr_seq_off of
// r0 + 4) gives rows r0 + 8 hf + 4..7: together 8 consecutive contraction rows.
template <int W>
__device__ __forceinline__ int tr_seq_off(int r0, int c0) {
  const int l = threadIdx.x & 63, li = l & 15;
  const int r = r0 + 8 * (l >> 5) + (li >> 2);
  const int col = c0 + 16 * ((l >> 4) & 1) + 4 * (li & 3);
  return r * W + 16 * ((col >> 3) ^ tiles::swz<W>(r)) + 2 * (col & 7);
}

__device__ __forceinline__ bf16x8 tr_seq(const char *tile, int lo, int hi) {
  const tiles::s16x8 v = __builtin_shufflevector(tiles::lds_tr4(tile + lo), tiles::lds_tr4(tile + hi), 0, 1, 2, 3, 4,
                                                 5, 6, 7);
  return __builtin_bit_cast(bf16x8, v);
}

// One operand of the bf16 product: where its two 1 KB blocks per wavefront
// come from, and where its MFMA fragments are read.
//   KM = true : k-major, view (r, c) = (m or n, k); tile rows = m or n.
//   KM = false: mn-major, view (r, c) = (k, m or n); tile rows = k.
// NB = fragments per k16 step (2 for A: 64 m per wavefront; 4 for B: 128 n).
template <bool KM, int NB>
struct Operand {
  Bases bs;
  unsigned voff[2];      // per-lane source offset of each block (k-major: fixed; mn-major: without the k-tail clamp)
  int rrow[2];           // mn-major: tile row (k) of this lane in each block
  unsigned lc16[2];      // mn-major: 16 * logical chunk of this lane in each block
  const char *colbase[2];   // mn-major: base of the sub-tile's columns (k = 0)
  int frag[2][NB][2];    // LDS offsets of the fragment reads [kk][block][lo/hi]

  __device__ __forceinline__ explicit Operand(const MatView &v) : bs(v) {}

  // Sources of this wavefront's fills for a tile: w = wavefront, mn0 = first m
  // (or n) of the tile, MN = its extent.
  __device__ __forceinline__ void init_fill(const MatView &v, int b, int w, int mn0, int MN) {
    const int l = threadIdx.x & 63;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int blk = w + 8 * i;
      if constexpr (KM) {
        const int r = 16 * blk + (l >> 2);                      // tile row
        const int lc = (l & 3) ^ tiles::swz<64>(r);
        const int rr = min(mn0 + r, MN - 1) - mn0;              // rows past the extent repeat the last
        voff[i] = (unsigned)(rr * v.ld * 2 + 16 * lc);
      } else {
        const int s = blk >> 2;                                 // sub-tile: columns 64 s .. 64 s + 63
        const int r = 8 * (blk & 3) + (l >> 3);
        rrow[i] = r;
        lc16[i] = 16u * (unsigned)((l & 7) ^ tiles::swz<128>(r));
        const int c0 = min(mn0 + 64 * s, MN - 64);              // sub-tiles past the extent repeat the last
        colbase[i] = vptr<2>(v, bs, b, 0, (unsigned)c0);
      }
    }
  }

  // LDS offsets of this lane's fragment reads; wpos = first m (or n) of the
  // wavefront's fragments inside the tile (the same for every tile).
  __device__ __forceinline__ void init_frag(int wpos) {
    const int l = threadIdx.x & 63, ln = l & 31, hf = l >> 5;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int f = 0; f < NB; ++f) {
        const int p = wpos + 32 * f;                            // first m (n) of fragment f
        if constexpr (KM) {
          frag[kk][f][0] = tiles::tile_off<64>(p + ln, 2 * kk + hf);
          frag[kk][f][1] = 0;
        } else {
          const int s = p >> 6, c0 = p & 63;
          frag[kk][f][0] = 4096 * s + tr_seq_off<128>(16 * kk, c0);
          frag[kk][f][1] = 4096 * s + tr_seq_off<128>(16 * kk + 4, c0);
        }
      }
  }

  // Issue this wavefront's two blocks of the stage with contraction rows
  // k0 .. k0 + 31 (rows >= kend repeat row kend - 1) into LDS tile `dst`.
  __device__ __forceinline__ void fill(const MatView &v, int b, int mn0, int k0, int kend, char *dst, int w) {
    if constexpr (KM) {
      const char *base = uniform_ptr(vptr<2>(v, bs, b, mn0, (unsigned)k0));
#pragma unroll
      for (int i = 0; i < 2; ++i)
        tiles::lds_load_s<16>(base, voff[i], tiles::lds_addr(dst + 1024 * (w + 8 * i)));
    } else {
      const int kmax = kend - 1 - k0;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const char *base = uniform_ptr(colbase[i] + 2LL * k0 * v.ld);
        const unsigned off = (unsigned)(min(rrow[i], kmax) * v.ld * 2) + lc16[i];
        tiles::lds_load_s<16>(base, off, tiles::lds_addr(dst + 1024 * (w + 8 * i)));
      }
    }
  }

  __device__ __forceinline__ bf16x8 read(const char *tile, int kk, int f) const {
    if constexpr (KM) return tiles::lds_frag(tile, frag[kk][f][0]);
    else return tr_seq(tile, frag[kk][f][0], frag[kk][f][1]);
  }
};

template <bool B> struct Flag { static constexpr bool value = B; };

// One stage (32 contraction steps) of a wavefront's 128 x 64 block: operands
// from ring slot `ta`; kstage = first contraction index of the stage.  TAIL:
// the stage reaches past kend, whose A entries (repeats) are zeroed.
template <bool TAIL, bool AKM, bool BKM>
__device__ __forceinline__ void mfma_stage(f32x16 (&acc)[4][2], const Operand<AKM, 2> &A, const Operand<BKM, 4> &Bo,
                                           const char *ta, int kstage, int kend) {
  const char *tb = ta + kGOpBytes;
  const int hf = (threadIdx.x & 63) >> 5;
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
    bf16x8 af[2], bfr[4];
#pragma unroll
    for (int f = 0; f < 2; ++f) af[f] = A.read(ta, kk, f);
#pragma unroll
    for (int f = 0; f < 4; ++f) bfr[f] = Bo.read(tb, kk, f);
    if constexpr (TAIL) {
      const int kfirst = kstage + 16 * kk + 8 * hf;
#pragma unroll
      for (int f = 0; f < 2; ++f)
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (kfirst + e >= kend) af[f][e] = (__bf16)0.f;
    }
#pragma unroll
    for (int fn = 0; fn < 4; ++fn)
#pragma unroll
      for (int fm = 0; fm < 2; ++fm)
        acc[fn][fm] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[fn], af[fm], acc[fn][fm], 0, 0, 0);
  }
}

// Stores of a wavefront's block.  D[n][m] = C[m][n]: lane (ln, hf) of fragment
// (fn, fm) holds m = m0 + 64 wm + 32 fm + ln and n = n0 + 128 wn + 32 fn + 8 q +
// 4 hf + 0..3 in acc[fn][fm][4 q .. 4 q + 3].  FULL: the tile lies inside C.
template <int OUT, bool FULL>
__device__ __forceinline__ void store_block(const f32x16 (&acc)[4][2], const GemmArgs &g, int b, int z, int m0, int n0,
                                            int wm, int wn) {
  const int l = threadIdx.x & 63, ln = l & 31, hf = l >> 5;
  constexpr int ES = OUT == LH_BF16 ? 2 : 4;
  const Bases cb(g.c);
#pragma unroll
  for (int fn = 0; fn < 4; ++fn) {
    const int nb = n0 + 128 * wn + 32 * fn;
    if (!FULL && nb >= g.N) continue;
    gchar *base = (gchar *)(vptr<ES>(g.c, cb, b, 0, (unsigned)nb)) + (long long)ES * z * g.zstride;
#pragma unroll
    for (int fm = 0; fm < 2; ++fm) {
      const int m = m0 + 64 * wm + 32 * fm + ln;
      if (!FULL && m >= g.M) continue;
      gchar *row = base + (long long)ES * ((long long)m * g.c.ld + 4 * hf);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f32x16 &a = acc[fn][fm];
        if constexpr (OUT == LH_BF16) {
          const unsigned lo = f32_to_bf16_rne(a[4 * q]) | ((unsigned)f32_to_bf16_rne(a[4 * q + 1]) << 16);
          const unsigned hi = f32_to_bf16_rne(a[4 * q + 2]) | ((unsigned)f32_to_bf16_rne(a[4 * q + 3]) << 16);
          *reinterpret_cast<__attribute__((address_space(1))) u32x2 *>(row + 2 * 8 * q) = (u32x2){lo, hi};
        } else {
          *reinterpret_cast<__attribute__((address_space(1))) f32x4 *>(row + 4 * 8 * q) =
              (f32x4){a[4 * q], a[4 * q + 1], a[4 * q + 2], a[4 * q + 3]};
        }
      }
    }
  }
}

__device__ __forceinline__ void zero(f32x16 (&acc)[4][2]) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = (f32x16){};
}

// One work-group per tile.  AKM / BKM: A / B k-major.  OUT: lh_dtype of C.
template <bool AKM, bool BKM, int OUT>
__global__ __launch_bounds__(kGThreads, 1) void k_gemm_mfma(GemmArgs g) {
  __shared__ __attribute__((aligned(1024))) char lds[kGStages * kGStageBytes];
  const int nm = (g.M + kGBM - 1) / kGBM, nn = (g.N + kGBN - 1) / kGBN;
  // XCD-aware numbering: XCD x = blockIdx.x % 8 runs m-tiles (or splits) = x mod 8
  const int x = blockIdx.x & 7, sidx = blockIdx.x >> 3;
  int mt, nt, z;
  if (g.splits > 1) {   // split-K: an XCD runs whole splits, one tile after the other
    const int T = nm * nn;
    z = 8 * (sidx / T) + x;
    mt = (sidx % T) / nn;
    nt = (sidx % T) % nn;
    if (z >= g.splits) return;
  } else {              // groups of kGGroup of the XCD's m-tiles walk all n-tiles together
    const int grp = sidx / (kGGroup * nn), within = sidx % (kGGroup * nn);
    nt = within / kGGroup;
    mt = 8 * (grp * kGGroup + within % kGGroup) + x;
    z = 0;
    if (mt >= nm) return;
  }
  const int b = blockIdx.y;
  const int m0 = mt * kGBM, n0 = nt * kGBN;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wn = w & 1, wm = w >> 1;
  const int kbeg = z * g.kchunk, kend = min(g.K, kbeg + g.kchunk);
  const int nk = kend > kbeg ? (kend - kbeg + kGBK - 1) / kGBK : 0;

  Operand<AKM, 2> A(g.a);
  Operand<BKM, 4> Bo(g.b);
  A.init_fill(g.a, b, w, m0, g.M);
  A.init_frag(64 * wm);
  Bo.init_fill(g.b, b, w, n0, g.N);
  Bo.init_frag(128 * wn);
  f32x16 acc[4][2];
  zero(acc);

  auto fill = [&](int t) {   // stage t (clamped to the last) into ring slot t % kGStages
    const int k0 = kbeg + kGBK * min(t, nk - 1);
    char *dst = lds + (t % kGStages) * kGStageBytes;
    A.fill(g.a, b, m0, k0, kend, dst, w);
    Bo.fill(g.b, b, n0, k0, kend, dst + kGOpBytes, w);
  };
  if (nk > 0) {
    fill(0);
    fill(1);
    fill(2);
    tiles::wait_fills_barrier<2 * kGFillOps>();   // stage 0 landed
    const bool tail = (kend - kbeg) % kGBK != 0;
    const int nfull = tail ? nk - 1 : nk;
    for (int t = 0; t < nfull; ++t) {
      fill(t + 3);   // ring slot of stage t - 1, which every wavefront has finished
      mfma_stage<false>(acc, A, Bo, lds + (t % kGStages) * kGStageBytes, kbeg + kGBK * t, kend);
      tiles::wait_fills_barrier<2 * kGFillOps>();
    }
    if (tail) mfma_stage<true>(acc, A, Bo, lds + ((nk - 1) % kGStages) * kGStageBytes, kbeg + kGBK * (nk - 1), kend);
    tiles::dma_wait();   // the fills past the last stage
  }
  store_block<OUT, false>(acc, g, b, z, m0, n0, wm, wn);
}

// ---------------------------------------------------------------------------
// fp32 operands: 64 x 64 tile per 256 threads, 4 x 4 outputs per thread,
// contraction in steps of 16 through LDS.  Element access goes through the
// view per element (this path serves the fp32 layer, not the bf16 hot path).
// ---------------------------------------------------------------------------
constexpr int kFT = 64, kFK = 16;

__device__ __forceinline__ float vload_f32(const MatView &v, int b, long long r, long long c) {
  const long long which = c / v.seg, cc = c - which * v.seg;
  const long long h = cc / v.hd, j = cc - h * v.hd;
  const float *p = reinterpret_cast<const float *>(which == 0 ? v.p[0] : which == 1 ? v.p[1] : v.p[2]);
  return p[b * v.bstride + h * v.hstride + r * v.ld + j];
}

template <bool AKM, bool BKM, int OUT>
__global__ __launch_bounds__(256) void k_gemm_f32(GemmArgs g) {
  __shared__ float As[kFK][kFT + 1], Bs[kFK][kFT + 1];
  const int nn = (g.N + kFT - 1) / kFT;
  const int m0 = (blockIdx.x / nn) * kFT, n0 = (blockIdx.x % nn) * kFT;
  const int b = blockIdx.y, z = blockIdx.z;
  const int kbeg = z * g.kchunk, kend = min(g.K, kbeg + g.kchunk);
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  float acc[4][4] = {};
  for (int k0 = kbeg; k0 < kend; k0 += kFK) {
    for (int e = threadIdx.x; e < kFK * kFT; e += 256) {
      const int kk = e / kFT, mm = e % kFT;
      const int k = k0 + kk, m = m0 + mm, n = n0 + mm;
      float av = 0.f, bv = 0.f;
      if (k < kend && m < g.M) av = AKM ? vload_f32(g.a, b, m, k) : vload_f32(g.a, b, k, m);
      if (k < kend && n < g.N) bv = BKM ? vload_f32(g.b, b, n, k) : vload_f32(g.b, b, k, n);
      As[kk][mm] = av;
      Bs[kk][mm] = bv;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < kFK; ++kk)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(As[kk][ty + 16 * i], Bs[kk][tx + 16 * j], acc[i][j]);
    __syncthreads();
  }
  for (int i = 0; i < 4; ++i)
    for (int j = 0; j < 4; ++j) {
      const int m = m0 + ty + 16 * i, n = n0 + tx + 16 * j;
      if (m >= g.M || n >= g.N) continue;
      const long long which = n / g.c.seg, cc = n - which * g.c.seg;
      const long long h = cc / g.c.hd, jj = cc - h * g.c.hd;
      const long long o = (long long)b * g.c.bstride + h * g.c.hstride + (long long)m * g.c.ld + jj + z * g.zstride;
      void *p = const_cast<void *>(which == 0 ? g.c.p[0] : which == 1 ? g.c.p[1] : g.c.p[2]);
      if constexpr (OUT == LH_BF16) reinterpret_cast<uint16_t *>(p)[o] = f32_to_bf16_rne(acc[i][j]);
      else reinterpret_cast<float *>(p)[o] = acc[i][j];
    }
}

// out(r, c) = sum over the nparts partials [nparts][M][N] (fp32, in order), four
// columns per thread.
__global__ __launch_bounds__(256) void k_split_reduce(const float *__restrict__ part, int nparts, int M, int N,
                                                      MatView out) {
  const long long i4 = (long long)blockIdx.x * 256 + threadIdx.x;
  const long long MN = (long long)M * N;
  if (4 * i4 >= MN) return;
  const int m = (int)(4 * i4 / N), n = (int)(4 * i4 % N);
  float4 s = *reinterpret_cast<const float4 *>(part + 4 * i4);
  for (int z = 1; z < nparts; ++z) {
    const float4 t = *reinterpret_cast<const float4 *>(part + z * MN + 4 * i4);
    s.x += t.x;
    s.y += t.y;
    s.z += t.z;
    s.w += t.w;
  }
  const unsigned which = (unsigned)n / (unsigned)out.seg, cc = (unsigned)n - which * (unsigned)out.seg;
  const unsigned h = cc / (unsigned)out.hd, j = cc - h * (unsigned)out.hd;
  float *p = reinterpret_cast<float *>(const_cast<void *>(which == 0 ? out.p[0] : which == 1 ? out.p[1] : out.p[2]));
  *reinterpret_cast<float4 *>(p + (long long)h * out.hstride + (long long)m * out.ld + j) = s;
}

}  // namespace

int gemm_blocks(const GemmArgs &g, int io) {
  if (io == LH_BF16) {
    const int nm = (g.M + kGBM - 1) / kGBM, nn = (g.N + kGBN - 1) / kGBN;
    if (g.splits > 1) return 8 * nm * nn * ((g.splits + 7) / 8);
    const int groups = (nm + 8 * kGGroup - 1) / (8 * kGGroup);
    return 8 * groups * kGGroup * nn;
  }
  return ((g.M + kFT - 1) / kFT) * ((g.N + kFT - 1) / kFT);
}

template <bool AKM, bool BKM>
void launch_kinds(const GemmArgs &g, int io, int out_dtype, const dim3 &grid, hipStream_t st) {
  if (io == LH_BF16) {
    if (out_dtype == LH_BF16) lh::launch(k_gemm_mfma<AKM, BKM, LH_BF16>, grid, kGThreads, 0, st, g);
    else lh::launch(k_gemm_mfma<AKM, BKM, LH_F32>, grid, kGThreads, 0, st, g);
  } else {
    if (out_dtype == LH_BF16) lh::launch(k_gemm_f32<AKM, BKM, LH_BF16>, grid, 256, 0, st, g);
    else lh::launch(k_gemm_f32<AKM, BKM, LH_F32>, grid, 256, 0, st, g);
  }
}

// Preconditions (checked by the caller on the host): a k-major operand needs
// K and kchunk to be multiples of 32; an mn-major operand needs its extent (M or
// N) to be a multiple of 64; every column block of a view (hd, seg) is a
// multiple of 64; N is a multiple of 32; pointers are 16-byte aligned.
hipError_t launch_gemm(const GemmArgs &g, bool akm, bool bkm, int io, int out_dtype, int batch, hipStream_t st) {
  const dim3 grid(gemm_blocks(g, io), batch, io == LH_BF16 ? 1 : g.splits);
  if (akm && !bkm) launch_kinds<true, false>(g, io, out_dtype, grid, st);
  else if (akm && bkm) launch_kinds<true, true>(g, io, out_dtype, grid, st);
  else if (!akm && !bkm) launch_kinds<false, false>(g, io, out_dtype, grid, st);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_split_reduce(const float *part, int nparts, int M, int N, const MatView &out, hipStream_t st) {
  const long long n4 = (long long)M * N / 4;
  lh::launch(k_split_reduce, (unsigned)((n4 + 255) / 256), 256, 0, st, part, nparts, M, N, out);
  return hipGetLastError();
}

}  // namespace lh
