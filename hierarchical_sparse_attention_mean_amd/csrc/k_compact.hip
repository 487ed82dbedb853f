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
//                     ending in the tile (one wavefront per tile).
//   k_compact_slots   tile offset = sum of the earlier tiles' counts; block scan
//                     inside the tile; writes the slot map (-1 for unselected
//                     entries) and the sorted flat coordinates.
//   k_gather_rows     one thread per 8-element piece of a gathered row: copies
//                     the rows of Q~, K~, V~ named by the coordinates into place
//                     (head stride Sv = S rounded up to a multiple of 64, rows
//                     S..Sv-1 zero).  A flat grid over the rows, so the copy
//                     keeps every compute unit busy at any tile count.
#include <type_traits>

#include "lh_internal.h"

namespace lh {

namespace {

constexpr int kThreads = 256;
constexpr int kRowsPerThread = 1;   // gathered rows copied per thread

// One wavefront per tile [T0, T1) of base positions.  The entries of level l
// ending in the tile are the contiguous run i in [T0 / p^l, T1 / p^l) (integer
// division), so the count is a sum of flag bytes over one run per level; the
// level-0 run of a whole, 16-byte aligned tile is read 16 flags per lane
// (flags are 0 or 1, so a popcount of the 16 bytes counts them).
constexpr int kCountWaves = kThreads / 64;   // tiles per work-group

__global__ __launch_bounds__(kThreads) void k_compact_count(Shape s, const uint8_t *__restrict__ flags,
                                                            int *__restrict__ tilecount) {
  static_assert(kCompactTile == 64 * 16, "16 level-0 flags per lane");
  const int h = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int tile = blockIdx.x * kCountWaves + (threadIdx.x >> 6);
  if (tile >= s.ntile) return;
  const uint8_t *fl = flags + (long long)h * s.P;
  const int T0 = tile * kCompactTile, T1 = min(s.N, T0 + kCompactTile);
  int c = 0;
  if (T1 - T0 == kCompactTile && (reinterpret_cast<uintptr_t>(fl + T0) & 15) == 0) {
    const uint4 f4 = *reinterpret_cast<const uint4 *>(fl + T0 + 16 * lane);
    c = __popc(f4.x) + __popc(f4.y) + __popc(f4.z) + __popc(f4.w);
  } else {
    for (int t = T0 + lane; t < T1; t += 64) c += fl[t];
  }
  for (int l = 1; l < s.L; ++l) {
    const int a = T0 / s.pw[l], b = T1 / s.pw[l];
    for (int i = a + lane; i < b; i += 64) c += fl[s.off[l] + i];
  }
#pragma unroll
  for (int m = 32; m > 0; m >>= 1) c += __shfl_xor(c, m);
  if (lane == 0) tilecount[(long long)h * s.ntile + tile] = c;
}

// One work-group per tile, kPer = 4 base positions per thread.  The entries of
// level l >= 1 ending at the thread's positions [t0, t1) are the run
// i in [t0 / p^l, t1 / p^l), at most two entries (p >= 2); the thread loads its
// level-0 flags and each level's run once, as bits, together with its share of
// the earlier tiles' counts (the tile's offset).  One block sum and one block
// scan then give each thread its first slot, and the thread walks its
// positions in order (finer level first at each) writing the slot map and the
// coordinates from those bits.
constexpr int kPer = kCompactTile / kThreads;   // positions per thread
static_assert(kPer == 4, "four level-0 flags per thread, at most two entries of a coarser level");

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

__global__ __launch_bounds__(kThreads) void k_compact_slots(Shape s, const uint8_t *__restrict__ flags,
                                                            const int *__restrict__ tilecount, int *__restrict__ slot,
                                                            int *__restrict__ coords) {
  static_assert(2 * (LH_MAX_LEVELS - 1) <= 64, "two bits per coarser level");
  __shared__ int red[kThreads / 64];
  __shared__ int scan[kThreads / 64];   // wavefront totals
  const int h = blockIdx.y;
  const int tile = blockIdx.x;
  const int tid = threadIdx.x;
  const uint8_t *fl = flags + (long long)h * s.P;
  const int t0 = tile * kCompactTile + tid * kPer;
  const int t1 = min(s.N, t0 + kPer);   // the thread's positions [t0, t1), possibly empty
  // level-0 flags: byte e of f0 is the flag of t0 + e
  unsigned int f0 = 0;
  if (t1 - t0 == kPer && (reinterpret_cast<uintptr_t>(fl + t0) & 3) == 0) {
    f0 = *reinterpret_cast<const unsigned int *>(fl + t0);
  } else {
    for (int e = 0; e < t1 - t0; ++e) f0 |= (unsigned int)fl[t0 + e] << (8 * e);
  }
  // coarser levels: bits 2(l-1) and 2(l-1)+1 are the flags of the run's entries
  unsigned long long cf = 0;
  for (int l = 1; l < s.L; ++l) {
    const int a = t0 / s.pw[l], b = t0 < t1 ? t1 / s.pw[l] : a;
    const unsigned int x0 = a < b ? fl[s.off[l] + a] : 0u;
    const unsigned int x1 = a + 1 < b ? fl[s.off[l] + a + 1] : 0u;
    cf |= (unsigned long long)(x0 | (x1 << 1)) << (2 * (l - 1));
  }
  const int mine = __popc(f0) + __popcll(cf);
  int pre = 0;
  for (int i = tid; i < tile; i += kThreads) pre += tilecount[(long long)h * s.ntile + i];
  const int m0 = block_sum(pre, red);
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
  int wbase = 0;
#pragma unroll
  for (int i = 0; i < kThreads / 64; ++i) wbase += i < wv ? scan[i] : 0;
  int m = m0 + wbase + incl - mine;
  int *sl = slot + (long long)h * s.P;
  int *co = coords + (long long)h * s.S;
  int v0[kPer];   // level-0 slot-map entries of the thread's positions
#pragma unroll
  for (int e = 0; e < kPer; ++e) {
    const int t = t0 + e;
    v0[e] = -1;
    if (t >= t1) continue;
    // entries ending at t, finer level first
    if ((f0 >> (8 * e)) & 1u) {
      v0[e] = m;
      co[m++] = t;
    }
    for (int l = 1; l < s.L; ++l) {
      if ((t + 1) % s.pw[l] != 0) break;
      const int i = (t + 1) / s.pw[l] - 1;
      const int f = s.off[l] + i;
      if ((cf >> (2 * (l - 1) + (i - t0 / s.pw[l]))) & 1ull) {
        sl[f] = m;
        co[m++] = f;
      } else {
        sl[f] = -1;
      }
    }
  }
  if (t1 - t0 == kPer && (reinterpret_cast<uintptr_t>(sl + t0) & 15) == 0) {
    *reinterpret_cast<int4 *>(sl + t0) = make_int4(v0[0], v0[1], v0[2], v0[3]);
  } else {
#pragma unroll
    for (int e = 0; e < kPer; ++e)
      if (t0 + e < t1) sl[t0 + e] = v0[e];
  }
}

// Row copies: gathered row m of head h is the pyramid entry coords[m] (rows
// S..Sv-1 are written as zeros).  A thread copies one piece of 8 elements of
// the row, the same piece of Q~, K~ and V~; CH = D / 8 threads per row.  The
// level of an entry and the start of its level's rows are selected from the
// shape by an unrolled scan over the levels (uniform in l, so the offsets stay
// scalar).
template <typename T, int D>
__global__ __launch_bounds__(kThreads) void k_gather_rows(Shape s, const T *__restrict__ q, const T *__restrict__ k,
                                                          const T *__restrict__ v, const char *__restrict__ ws,
                                                          FwdWs w, const int *__restrict__ coords,
                                                          T *__restrict__ qt, T *__restrict__ kt,
                                                          T *__restrict__ vt) {
  constexpr int CH = D / 8;
  constexpr int RPB = kThreads / CH;   // rows per work-group and pass
  using V8 = typename std::conditional<sizeof(T) == 2, uint4, float4>::type;
  constexpr int NV = sizeof(T) == 2 ? 1 : 2;   // 16-byte vectors per piece
  const int h = blockIdx.y;
  const int j = threadIdx.x % CH;
  V8 a[kRowsPerThread][NV], b[kRowsPerThread][NV], c[kRowsPerThread][NV];
  // all rows' loads first, then all stores
#pragma unroll
  for (int u = 0; u < kRowsPerThread; ++u) {
    const int m = (blockIdx.x * kRowsPerThread + u) * RPB + threadIdx.x / CH;
#pragma unroll
    for (int x = 0; x < NV; ++x) a[u][x] = b[u][x] = c[u][x] = V8{};
    if (m >= s.S) continue;   // rows S..Sv-1: zeros
    const int f = coords[(long long)h * s.S + m];
    const T *bq = q, *bk = k, *bv = v;
    long long r = (long long)h * s.N + f;
#pragma unroll
    for (int l = 1; l < LH_MAX_LEVELS; ++l) {
      if (l >= s.L) break;
      if (f >= s.off[l]) {
        bq = reinterpret_cast<const T *>(ws + w.lev[l][0]);
        bk = reinterpret_cast<const T *>(ws + w.lev[l][1]);
        bv = reinterpret_cast<const T *>(ws + w.lev[l][2]);
        r = (long long)h * s.n[l] + (f - s.off[l]);
      }
    }
    const long long src = r * D + j * 8;
#pragma unroll
    for (int x = 0; x < NV; ++x) {
      a[u][x] = reinterpret_cast<const V8 *>(bq + src)[x];
      b[u][x] = reinterpret_cast<const V8 *>(bk + src)[x];
      c[u][x] = reinterpret_cast<const V8 *>(bv + src)[x];
    }
  }
#pragma unroll
  for (int u = 0; u < kRowsPerThread; ++u) {
    const int m = (blockIdx.x * kRowsPerThread + u) * RPB + threadIdx.x / CH;
    if (m >= s.Sv) continue;
    const long long dst = ((long long)h * s.Sv + m) * D + j * 8;
#pragma unroll
    for (int x = 0; x < NV; ++x) {
      reinterpret_cast<V8 *>(qt + dst)[x] = a[u][x];
      reinterpret_cast<V8 *>(kt + dst)[x] = b[u][x];
      reinterpret_cast<V8 *>(vt + dst)[x] = c[u][x];
    }
  }
}

}  // namespace

hipError_t launch_compact_gather(const Shape &s, const void *q, const void *k, const void *v, void *ws,
                                 const FwdWs &w, const uint8_t *flags, int *slot, int *coords, void *qt,
                                 void *kt, void *vt, hipStream_t st) {
  char *wsb = reinterpret_cast<char *>(ws);
  int *tc = reinterpret_cast<int *>(wsb + w.tilecount);
  lh::launch(k_compact_count, dim3((s.ntile + kCountWaves - 1) / kCountWaves, s.BH), kThreads, 0, st, s, flags, tc);
  lh::launch(k_compact_slots, dim3(s.ntile, s.BH), kThreads, 0, st, s, flags, (const int *)tc, slot, coords);
  const int rows = kRowsPerThread * kThreads / (s.d / 8);   // rows per row-copy work-group
  const dim3 rgrid((s.Sv + rows - 1) / rows, s.BH);
#define LH_GATHER(T, D)                                                                                          \
  lh::launch(k_gather_rows<T, D>, rgrid, kThreads, 0, st, s, (const T *)q, (const T *)k, (const T *)v,          \
             (const char *)wsb, w, (const int *)coords, (T *)qt, (T *)kt, (T *)vt)
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
