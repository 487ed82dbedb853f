// Exact joint top-k over all non-coarsest pyramid levels and both score streams.
//
// "Long Context Pre-Training with Lighthouse Attention", Sec. 3.4: selection
// runs jointly over the concatenated QK and KQ streams across levels; the
// coarsest level is always kept; Sec. 3.5: the non-coarsest levels contribute
// B = (L-1) p k entries (here min(B, |E|), distinct entries).  The 64-bit key of
// a candidate, formed from its two scores (make_key), is unique and orders the
// entries by (score desc, stream index asc), so the selection is exactly "the B
// largest keys".
//
// The paper's kernel keeps a per-chunk top-m buffer by bitonic merging.  Here
// the same exact set is found in three passes whose number does not depend on k
// (the pool+score kernel before them has cleared the per-head state and
// histogram and recorded each of its work-groups' score ranges):
//   1. k_topk_hist    one pass over the scores: the head's score range from the
//                     pool+score records, then an LDS histogram of a 12-bit digit
//                     of the score bits rescaled to that range, merged into the
//                     head's global histogram with atomics (kHistBlocks
//                     work-groups per head keep the merges few).
//   2. k_topk_filter  one pass over the scores: every work-group finds the
//                     boundary bin once (a block-wide suffix scan of the merged
//                     histogram); keys above it are flagged, keys in it are
//                     appended to the work-group's own region of the candidate
//                     list (an LDS counter: no global atomics); the coarsest
//                     level is flagged.
//   3. k_topk_refine  the candidates' ranks among themselves, counted in LDS by
//                     kRefineBlocks work-groups per head: a candidate is selected
//                     if fewer than `need` candidates are larger.  A candidate list
//                     longer than LDS holds takes 8-bit radix passes over global
//                     memory instead (one work-group per head).
#include "lh_internal.h"

namespace lh {

namespace {

constexpr int kPerRound = kTopkRound;   // scores per thread and stream loaded ahead of their use
constexpr int kRefineThreads = 512;
constexpr int kRefineBlocks = 32;    // refine work-groups per head
constexpr int kRankLds = 16384;      // candidates ranked in LDS (128 KB)

__device__ __forceinline__ int digit_shift(unsigned int umin, unsigned int umax) {
  const unsigned int range = umax - umin;
  int sh = 0;
  while ((range >> sh) >= (unsigned int)kHistBins) ++sh;
  return sh;
}

__device__ __forceinline__ int key_digit(unsigned long long key, unsigned int umin, int sh) {
  const unsigned int hi = (unsigned int)(key >> 32);
  return (int)((hi - umin) >> sh);
}

__device__ __forceinline__ int key_flat(unsigned long long key, int P) {
  const unsigned int g = 0xFFFFFFFFu - (unsigned int)(key & 0xFFFFFFFFull);
  return (int)(g >= (unsigned int)P ? g - (unsigned int)P : g);
}

// Entries [i0, i1) of a head handled by work-group b of nb (topk_chunk).
__device__ __forceinline__ void chunk_of(long long n, int b, int nb, long long &i0, long long &i1) {
  const long long per = topk_chunk(n, nb);
  i0 = (long long)b * per;
  i1 = min(n, i0 + per);
}

// Block-wide min / max of the pool+score work-groups' ranges of head h (both
// streams); every thread gets the result.
__device__ void head_range(const uint2 *br, int n, unsigned int &umin, unsigned int &umax) {
  __shared__ unsigned int smin[kTopkThreads / 64], smax[kTopkThreads / 64];
  unsigned int mn = 0xFFFFFFFFu, mx = 0u;
  for (int i = threadIdx.x; i < n; i += kTopkThreads) {
    const uint2 r = br[i];
    mn = min(mn, r.x);
    mx = max(mx, r.y);
  }
#pragma unroll
  for (int m = 32; m > 0; m >>= 1) {
    mn = min(mn, (unsigned int)__shfl_xor((int)mn, m));
    mx = max(mx, (unsigned int)__shfl_xor((int)mx, m));
  }
  if ((threadIdx.x & 63) == 0) {
    smin[threadIdx.x >> 6] = mn;
    smax[threadIdx.x >> 6] = mx;
  }
  __syncthreads();
  mn = smin[0];
  mx = smax[0];
#pragma unroll
  for (int wv = 1; wv < kTopkThreads / 64; ++wv) {
    mn = min(mn, smin[wv]);
    mx = max(mx, smax[wv]);
  }
  umin = mn;
  umax = mx;
}

// One round of a pass: the scores of entries i0 + r*kTopkThreads + tid,
// r < kPerRound, of both streams (entries >= i1 read as 0 and are not used).
struct Round {
  float qk[kPerRound], kq[kPerRound];
  __device__ __forceinline__ void load(const float *q, const float *k, long long i0, long long i1) {
#pragma unroll
    for (int r = 0; r < kPerRound; ++r) {
      const long long i = i0 + (long long)r * kTopkThreads + threadIdx.x;
      qk[r] = i < i1 ? q[i] : 0.f;
      kq[r] = i < i1 ? k[i] : 0.f;
    }
  }
};

__global__ __launch_bounds__(kTopkThreads) void k_topk_hist(Shape s, char *__restrict__ ws, FwdWs w,
                                                            const float *__restrict__ scores) {
  __shared__ unsigned int hist[kHistBins];
  const int h = blockIdx.y;
  const float *qk = scores + (long long)h * 2 * s.P, *kq = qk + s.P;
  long long i0, i1;
  chunk_of(s.E, blockIdx.x, gridDim.x, i0, i1);
  Round cur;
  cur.load(qk, kq, i0, i1);   // in flight while the range is formed
  for (int i = threadIdx.x; i < kHistBins; i += kTopkThreads) hist[i] = 0;
  unsigned int umin, umax;
  head_range(reinterpret_cast<const uint2 *>(ws + w.brange) + (long long)h * 2 * s.npool, 2 * s.npool, umin, umax);
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    TopkState *st = reinterpret_cast<TopkState *>(ws + w.state) + h;
    st->umin = umin;
    st->umax = umax;
  }
  const int sh = digit_shift(umin, umax);
  for (long long r0 = i0; r0 < i1; r0 += (long long)kPerRound * kTopkThreads) {
    Round nxt;
    const long long n0 = r0 + (long long)kPerRound * kTopkThreads;
    if (n0 < i1) nxt.load(qk, kq, n0, i1);
#pragma unroll
    for (int r = 0; r < kPerRound; ++r) {
      const long long i = r0 + (long long)r * kTopkThreads + threadIdx.x;
      if (i < i1) atomicAdd(&hist[key_digit(make_key(cur.qk[r], cur.kq[r], (int)i, s.P), umin, sh)], 1u);
    }
    cur = nxt;
  }
  __syncthreads();
  unsigned int *gh = reinterpret_cast<unsigned int *>(ws + w.hist) + (long long)h * kHistBins;
  for (int i = threadIdx.x; i < kHistBins; i += kTopkThreads)
    if (hist[i]) atomicAdd(&gh[i], hist[i]);
}

// Boundary bin b* of the head's merged histogram gh: count(digit > b*) < Bsel
// <= count(digit >= b*).  Returns b* and writes the count above it.  1024
// threads, 4 bins each: a suffix scan within each wavefront (shuffles), then
// across the 16 wavefronts.
__device__ int find_boundary(const unsigned int *gh, long long Bsel, long long *above_out) {
  static_assert(kHistBins == 4 * kTopkThreads, "4 bins per thread");
  constexpr int NW = kTopkThreads / 64;
  __shared__ unsigned int wtot[NW];
  __shared__ int bstar_s;
  __shared__ long long above_s;
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  const uint4 c = reinterpret_cast<const uint4 *>(gh)[t];   // bins 4t .. 4t+3
  const unsigned int mine = c.x + c.y + c.z + c.w;          // <= |E| < 2^31
  unsigned int suf = mine;                                  // bins >= 4t within the wavefront
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const unsigned int v = (unsigned int)__shfl_down((int)suf, o);
    if (lane + o < 64) suf += v;
  }
  if (lane == 0) wtot[wv] = suf;
  if (t == 0) {
    bstar_s = -1;
    above_s = 0;
  }
  __syncthreads();
  unsigned long long later = 0;   // bins of the wavefronts above this one
  for (int u = wv + 1; u < NW; ++u) later += wtot[u];
  const unsigned long long incl = later + suf;   // bins >= 4t
  const unsigned long long excl = incl - mine;   // bins >  4t + 3
  if (excl < (unsigned long long)Bsel && (unsigned long long)Bsel <= incl) {
    const unsigned int cb[4] = {c.x, c.y, c.z, c.w};
    unsigned long long acc = excl;
    for (int i = 3; i >= 0; --i) {
      if (acc + cb[i] >= (unsigned long long)Bsel) {
        bstar_s = 4 * t + i;
        above_s = (long long)acc;
        break;
      }
      acc += cb[i];
    }
  }
  __syncthreads();
  *above_out = above_s;
  return bstar_s;
}

__global__ __launch_bounds__(kTopkThreads) void k_topk_filter(Shape s, char *__restrict__ ws, FwdWs w,
                                                              const float *__restrict__ scores,
                                                              uint8_t *__restrict__ flags) {
  const int h = blockIdx.y;
  const float *qk = scores + (long long)h * 2 * s.P, *kq = qk + s.P;
  long long i0, i1;
  chunk_of(s.P, blockIdx.x, gridDim.x, i0, i1);
  const long long c1 = min(i1, (long long)s.E);   // candidates of the chunk: [i0, c1)
  Round cur;
  cur.load(qk, kq, i0, c1);   // in flight while the boundary is found
  TopkState *stp = reinterpret_cast<TopkState *>(ws + w.state) + h;
  int bstar;
  long long above = 0;
  unsigned int umin = 0;
  int sh = 0;
  if (s.Bsel == 0) {
    bstar = kHistBins;          // nothing selected
  } else if (s.Bsel == s.E) {
    bstar = -1;                 // everything selected
  } else {
    umin = stp->umin;
    sh = digit_shift(umin, stp->umax);
    bstar = find_boundary(reinterpret_cast<const unsigned int *>(ws + w.hist) + (long long)h * kHistBins, s.Bsel,
                          &above);
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    stp->bstar = (unsigned int)bstar;
    stp->need = (bstar < 0 || bstar >= kHistBins) ? 0 : (long long)s.Bsel - above;
  }
  // this work-group's region of the candidate list, filled through an LDS counter
  unsigned long long *cand = reinterpret_cast<unsigned long long *>(ws + w.cand) + (long long)h * w.cstride + i0;
  __shared__ unsigned int ncand;
  if (threadIdx.x == 0) ncand = 0;
  __syncthreads();
  uint8_t *fl = flags + (long long)h * s.P;
  const int lane = threadIdx.x & 63;
  for (long long r0 = i0; r0 < i1; r0 += (long long)kPerRound * kTopkThreads) {
    Round nxt;
    const long long n0 = r0 + (long long)kPerRound * kTopkThreads;
    if (n0 < c1) nxt.load(qk, kq, n0, c1);
#pragma unroll
    for (int r = 0; r < kPerRound; ++r) {
      const long long i = r0 + (long long)r * kTopkThreads + threadIdx.x;
      bool boundary = false;
      unsigned long long key = 0;
      if (i < c1) {
        key = make_key(cur.qk[r], cur.kq[r], (int)i, s.P);
        const int dg = (bstar < 0) ? kHistBins : (bstar >= kHistBins ? -1 : key_digit(key, umin, sh));
        fl[i] = (uint8_t)(dg > bstar ? 1 : 0);
        boundary = (dg == bstar);
      } else if (i < i1) {
        fl[i] = 1;   // coarsest level: always in the index set
      }
      const unsigned long long m = __ballot(boundary);
      if (m) {
        unsigned int base = 0;
        const int leader = __ffsll((long long)m) - 1;
        if (lane == leader) base = atomicAdd(&ncand, (unsigned int)__popcll(m));
        base = __shfl(base, leader);
        if (boundary) cand[base + __popcll(m & ((1ull << lane) - 1ull))] = key;
      }
    }
    cur = nxt;
  }
  __syncthreads();
  if (threadIdx.x == 0) reinterpret_cast<unsigned int *>(ws + w.ccount)[h * kFilterBlocks + blockIdx.x] = ncand;
}

// The candidate list of a head: the filter work-groups' regions (region b at
// b * per holds cnt[b] keys) seen as one list through the prefix table pre[]
// (pre[b] = keys before region b, pre[nb] = all).
struct Cands {
  const unsigned long long *base;
  const unsigned int *pre;
  long long per;
  int nb;
  __device__ __forceinline__ unsigned long long operator[](long long i) const {
    int lo = 0, hi = nb - 1;   // the region b with pre[b] <= i < pre[b + 1]
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if ((long long)pre[mid] <= i) lo = mid;
      else hi = mid - 1;
    }
    return base[(long long)lo * per + (i - pre[lo])];
  }
};

// Radix select of the need-th largest of the C candidates (global memory), by
// one work-group: 8-bit digits from the top; keys are unique, so the threshold
// is exact.  Flags every key >= the threshold.
__device__ void radix_select(const Cands &cand, long long C, long long need, uint8_t *fl, int P) {
  __shared__ unsigned int hist[256];
  __shared__ unsigned long long sel_prefix;
  __shared__ long long sel_need;
  __shared__ int sel_done;
  const int tid = threadIdx.x;
  unsigned long long prefix = 0, mask = 0;
  for (int shift = 56; shift >= 0; shift -= 8) {
    for (int i = tid; i < 256; i += kRefineThreads) hist[i] = 0;
    __syncthreads();
    for (long long i = tid; i < C; i += kRefineThreads) {
      const unsigned long long key = cand[i];
      if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 255], 1u);
    }
    __syncthreads();
    if (tid == 0) {
      long long acc = 0;
      int b = 255;
      for (; b >= 0; --b) {
        if (acc + (long long)hist[b] >= need) break;
        acc += hist[b];
      }
      sel_need = need - acc;
      sel_prefix = prefix | ((unsigned long long)b << shift);
      sel_done = ((long long)hist[b] == need - acc) ? 1 : 0;
    }
    __syncthreads();
    need = sel_need;
    prefix = sel_prefix;
    mask |= 255ull << shift;
    const int done = sel_done;
    __syncthreads();
    if (done) break;
  }
  // every key >= prefix (all keys of the final bucket are taken) is selected
  for (long long i = tid; i < C; i += kRefineThreads) {
    const unsigned long long key = cand[i];
    if (key >= prefix) fl[key_flat(key, P)] = 1;
  }
}

__global__ __launch_bounds__(kRefineThreads) void k_topk_refine(Shape s, char *__restrict__ ws, FwdWs w,
                                                                uint8_t *__restrict__ flags) {
  __shared__ unsigned long long keys[kRankLds];
  __shared__ unsigned int pre[kFilterBlocks + 1];
  const int h = blockIdx.y;
  const long long need = reinterpret_cast<const TopkState *>(ws + w.state)[h].need;
  if (need <= 0) return;
  const int nbf = topk_blocks(s.P, kFilterBlocks);   // filter work-groups per head
  const int tid = threadIdx.x;
  const unsigned int *cnt = reinterpret_cast<const unsigned int *>(ws + w.ccount) + h * kFilterBlocks;
  if (tid < 64) {   // prefix table of the regions' counts (one wavefront, inclusive scan by shuffles)
    const unsigned int c = tid < nbf ? cnt[tid] : 0u;
    unsigned int incl = c;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const unsigned int v = (unsigned int)__shfl_up((int)incl, o);
      if (tid >= o) incl += v;
    }
    if (tid < nbf) pre[tid] = incl - c;
    if (tid == nbf - 1) pre[nbf] = incl;   // all keys
  }
  __syncthreads();
  const long long C = pre[nbf];
  const long long per = topk_chunk(s.P, nbf);
  const unsigned long long *base = reinterpret_cast<const unsigned long long *>(ws + w.cand) + (long long)h * w.cstride;
  const Cands cand{base, pre, per, nbf};
  uint8_t *fl = flags + (long long)h * s.P;
  if (need >= C) {   // the whole boundary bin
    for (long long i = (long long)blockIdx.x * kRefineThreads + tid; i < C; i += (long long)gridDim.x * kRefineThreads)
      fl[key_flat(cand[i], s.P)] = 1;
    return;
  }
  if (C > kRankLds) {
    if (blockIdx.x == 0) radix_select(cand, C, need, fl, s.P);
    return;
  }
  // Rank counting.  The head's kRefineBlocks x kRefineThreads lanes are spread
  // over the C candidates, `lpc` lanes per candidate (a power of two, so that a
  // lane group lies within a wavefront), each lane counting the larger keys
  // among every lpc-th candidate; neighbouring lanes of a group read
  // neighbouring keys, so a read is a few broadcasts without bank conflicts.
  int lpc = 1;
  while (lpc < 64 && (long long)(2 * lpc) * C <= (long long)kRefineBlocks * kRefineThreads) lpc <<= 1;
  const int group = kRefineThreads / lpc;   // candidates per work-group per round
  const long long first = (long long)blockIdx.x * group;
  if (first >= C) return;
  const int n = (int)C;
  // stage the list in LDS: 8 lanes per region (region b at b * per holds
  // pre[b+1] - pre[b] keys), each issuing its loads before storing any
  static_assert(kRefineThreads / 8 >= kFilterBlocks, "8 lanes per filter region");
  {
    const int b = tid >> 3, r = tid & 7;
    if (b < nbf) {
      const int nkeys = (int)(pre[b + 1] - pre[b]);
      const unsigned long long *src = base + (long long)b * per;
      unsigned long long *dst = keys + pre[b];
      for (int i0 = r; i0 < nkeys; i0 += 64) {
        unsigned long long v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = i0 + 8 * u < nkeys ? src[i0 + 8 * u] : 0ull;
#pragma unroll
        for (int u = 0; u < 8; ++u)
          if (i0 + 8 * u < nkeys) dst[i0 + 8 * u] = v[u];
      }
    }
  }
  __syncthreads();
  const int q = tid & (lpc - 1);
  for (long long j0 = first; j0 < C; j0 += (long long)gridDim.x * group) {
    const long long j = j0 + tid / lpc;
    const unsigned long long key = j < C ? keys[j] : ~0ull;
    unsigned int c = 0;
    int m = q;
    for (; m + 3 * lpc < n; m += 4 * lpc) {
      c += keys[m] > key;
      c += keys[m + lpc] > key;
      c += keys[m + 2 * lpc] > key;
      c += keys[m + 3 * lpc] > key;
    }
    for (; m < n; m += lpc) c += keys[m] > key;
    for (int o = 1; o < lpc; o <<= 1) c += (unsigned int)__shfl_xor((int)c, o);
    if (j < C && q == 0 && (long long)c < need) fl[key_flat(key, s.P)] = 1;
  }
}

}  // namespace

hipError_t launch_topk(const Shape &s, void *ws, const FwdWs &w, const float *scores, uint8_t *flags,
                       hipStream_t st) {
  char *wsb = reinterpret_cast<char *>(ws);
  const bool partial = s.Bsel > 0 && s.Bsel < s.E;
  if (partial) lh::launch(k_topk_hist, dim3(topk_blocks(s.E, kHistBlocks), s.BH), kTopkThreads, 0, st, s, wsb, w, scores);
  lh::launch(k_topk_filter, dim3(topk_blocks(s.P, kFilterBlocks), s.BH), kTopkThreads, 0, st, s, wsb, w, scores, flags);
  if (partial) lh::launch(k_topk_refine, dim3(kRefineBlocks, s.BH), kRefineThreads, 0, st, s, wsb, w, flags);
  return hipGetLastError();
}

}  // namespace lh
