// Topological compaction and gather of the selected triples.
//
// "Long Context Pre-Training with Lighthouse Attention", Sec. 3.5: the selected
// (Q, K, V) triples form a contiguous sub-sequence sorted topologically by
// pyramid coordinate, so that the mask of the sub-sequence attention (Eq. 9) is
// the plain S x S causal mask.  Order used: base position of an entry = last
// token of its window, end(l, i) = (i+1) p^l - 1, ascending; finer level first
// among equal ends.  Position t is the end of (0, t) and of (l, (t+1)/p^l - 1)
// for every l >= 1 with p^l | t+1, so the slot of an entry is a prefix sum over
// base positions of "selected entries ending here".
//
//   k_compact_count   per tile of base positions: number of selected entries
//                     ending in the tile.
//   k_compact_gather  tile offset = sum of the earlier tiles' counts; block scan
//                     inside the tile; writes the slot map (-1 for unselected
//                     entries), the sorted flat coordinates, and copies the rows
//                     of Q~, K~, V~ into place (head stride Sv = S rounded up to
//                     a multiple of 64, rows S..Sv-1 zero).
#include "lh_internal.h"

namespace lh {

namespace {

constexpr int kThreads = 256;
constexpr int kPer = kCompactTile / kThreads;   // positions per thread

__device__ __forceinline__ int count_at(const Shape &s, const uint8_t *fl, int t) {
  int c = fl[t];
  for (int l = 1; l < s.L; ++l) {
    if ((t + 1) % s.pw[l] != 0) break;
    c += fl[s.off[l] + (t + 1) / s.pw[l] - 1];
  }
  return c;
}

__device__ __forceinline__ int block_sum(int v, int *red) {
  const int t = threadIdx.x;
  for (int m = 32; m > 0; m >>= 1) v += __shfl_xor(v, m);
  if ((t & 63) == 0) red[t >> 6] = v;
  __syncthreads();
  int tot = 0;
  for (int i = 0; i < kThreads / 64; ++i) tot += red[i];
  __syncthreads();
  return tot;
}

__global__ __launch_bounds__(kThreads) void k_compact_count(Shape s, const uint8_t *__restrict__ flags,
                                                            int *__restrict__ tilecount) {
  __shared__ int red[kThreads / 64];
  const int h = blockIdx.y;
  const uint8_t *fl = flags + (long long)h * s.P;
  const int t0 = blockIdx.x * kCompactTile + threadIdx.x * kPer;
  int c = 0;
  for (int e = 0; e < kPer; ++e)
    if (t0 + e < s.N) c += count_at(s, fl, t0 + e);
  const int tot = block_sum(c, red);
  if (threadIdx.x == 0) tilecount[(long long)h * s.ntile + blockIdx.x] = tot;
}

template <typename T, int D>
__global__ __launch_bounds__(kThreads) void k_compact_gather(Shape s, const T *__restrict__ q, const T *__restrict__ k,
                                                            const T *__restrict__ v, const char *__restrict__ ws,
                                                            FwdWs w, const uint8_t *__restrict__ flags,
                                                            const int *__restrict__ tilecount, int *__restrict__ slot,
                                                            int *__restrict__ coords, T *__restrict__ qt,
                                                            T *__restrict__ kt, T *__restrict__ vt) {
  __shared__ int red[kThreads / 64];
  __shared__ int scan[kThreads / 64];   // wavefront totals
  __shared__ int lflat[kCompactTile * 2];     // flat indices of this tile's slots (spills to global if more)
  const int h = blockIdx.y;
  const int tile = blockIdx.x;
  const int tid = threadIdx.x;
  const uint8_t *fl = flags + (long long)h * s.P;
  // offset of this tile in the sub-sequence
  int pre = 0;
  for (int i = tid; i < tile; i += kThreads) pre += tilecount[(long long)h * s.ntile + i];
  const int m0 = block_sum(pre, red);
  // per-thread counts of its kPer positions, exclusive scan over the block
  const int t0 = tile * kCompactTile + tid * kPer;
  int cnt[kPer];
  int mine = 0;
  for (int e = 0; e < kPer; ++e) {
    cnt[e] = (t0 + e < s.N) ? count_at(s, fl, t0 + e) : 0;
    mine += cnt[e];
  }
  // exclusive scan over the block: inclusive scan within each wavefront by
  // shuffles, then the wavefront totals (one barrier)
  const int lane = tid & 63, wv = tid >> 6;
  int incl = mine;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(incl, off);
    if (lane >= off) incl += y;
  }
  if (lane == 63) scan[wv] = incl;
  __syncthreads();
  int wbase = 0, ntot = 0;
#pragma unroll
  for (int i = 0; i < kThreads / 64; ++i) {
    wbase += i < wv ? scan[i] : 0;
    ntot += scan[i];
  }
  int m = m0 + wbase + incl - mine;
  int *sl = slot + (long long)h * s.P;
  int *co = coords + (long long)h * s.S;
  for (int e = 0; e < kPer; ++e) {
    const int t = t0 + e;
    if (t >= s.N) break;
    // entries ending at t, finer level first
    {
      const int f = t;
      if (fl[f]) {
        sl[f] = m;
        co[m] = f;
        if (m - m0 < kCompactTile * 2) lflat[m - m0] = f;
        ++m;
      } else {
        sl[f] = -1;
      }
    }
    for (int l = 1; l < s.L; ++l) {
      if ((t + 1) % s.pw[l] != 0) break;
      const int f = s.off[l] + (t + 1) / s.pw[l] - 1;
      if (fl[f]) {
        sl[f] = m;
        co[m] = f;
        if (m - m0 < kCompactTile * 2) lflat[m - m0] = f;
        ++m;
      } else {
        sl[f] = -1;
      }
    }
  }
  __syncthreads();
  // row copies: CH threads per row, 8 elements each
  constexpr int CH = D / 8;
  constexpr int RPI = kThreads / CH;   // rows per iteration
  const int j = tid % CH;
  const int rr = tid / CH;
  const long long hS = (long long)h * s.Sv;   // gathered rows: head stride Sv
  for (int mm = rr; mm < ntot; mm += RPI) {
    const int f = (mm < kCompactTile * 2) ? lflat[mm] : co[m0 + mm];
    int l = 0;
    while (l + 1 < s.L && f >= s.off[l + 1]) ++l;
    const int i = f - s.off[l];
    const T *sq, *sk, *sv;
    if (l == 0) {
      const long long base = ((long long)h * s.N + i) * D;
      sq = q + base;
      sk = k + base;
      sv = v + base;
    } else {
      const long long base = ((long long)h * s.n[l] + i) * D;
      sq = reinterpret_cast<const T *>(ws + w.lev[l][0]) + base;
      sk = reinterpret_cast<const T *>(ws + w.lev[l][1]) + base;
      sv = reinterpret_cast<const T *>(ws + w.lev[l][2]) + base;
    }
    const long long dst = (hS + m0 + mm) * D + j * 8;
    if constexpr (sizeof(T) == 2) {
      const uint4 a = *reinterpret_cast<const uint4 *>(sq + j * 8);
      const uint4 b = *reinterpret_cast<const uint4 *>(sk + j * 8);
      const uint4 c = *reinterpret_cast<const uint4 *>(sv + j * 8);
      *reinterpret_cast<uint4 *>(qt + dst) = a;
      *reinterpret_cast<uint4 *>(kt + dst) = b;
      *reinterpret_cast<uint4 *>(vt + dst) = c;
    } else {
#pragma unroll
      for (int hlf = 0; hlf < 2; ++hlf) {
        const float4 a = *reinterpret_cast<const float4 *>(sq + j * 8 + hlf * 4);
        const float4 b = *reinterpret_cast<const float4 *>(sk + j * 8 + hlf * 4);
        const float4 c = *reinterpret_cast<const float4 *>(sv + j * 8 + hlf * 4);
        *reinterpret_cast<float4 *>(qt + dst + hlf * 4) = a;
        *reinterpret_cast<float4 *>(kt + dst + hlf * 4) = b;
        *reinterpret_cast<float4 *>(vt + dst + hlf * 4) = c;
      }
    }
  }
  // zero the padding rows S..Sv-1 of the gathered rows
  if (tile == s.ntile - 1) {
    const int pad = s.Sv - s.S;
    for (int idx = tid; idx < D * pad; idx += kThreads) {
      const long long o = (hS + s.S) * D + idx;
      qt[o] = T(0);
      kt[o] = T(0);
      vt[o] = T(0);
    }
  }
}

}  // namespace

hipError_t launch_compact_gather(const Shape &s, const void *q, const void *k, const void *v, void *ws,
                                 const FwdWs &w, const uint8_t *flags, int *slot, int *coords, void *qt,
                                 void *kt, void *vt, hipStream_t st) {
  char *wsb = reinterpret_cast<char *>(ws);
  int *tc = reinterpret_cast<int *>(wsb + w.tilecount);
  dim3 grid(s.ntile, s.BH);
  lh::launch(k_compact_count, grid, kThreads, 0, st, s, flags, tc);
#define LH_GATHER(T, D)                                                                                         \
  lh::launch(k_compact_gather<T, D>, grid, kThreads, 0, st, s, (const T *)q, (const T *)k, (const T *)v, wsb, w, flags, \
                                                    tc, slot, coords, (T *)qt, (T *)kt, (T *)vt)
  if (s.io == LH_BF16) {
    if (s.d == 128) LH_GATHER(uint16_t, 128);
    else LH_GATHER(uint16_t, 64);
  } else {
    if (s.d == 128) LH_GATHER(float, 128);
    else LH_GATHER(float, 64);
  }
#undef LH_GATHER
  return hipGetLastError();
}

}  // namespace lh
