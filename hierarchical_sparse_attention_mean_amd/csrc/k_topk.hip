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
// the same exact set is found in a bounded number of passes that do not depend
// on k:
//   1. k_topk_hist    one pass over the scores: LDS histogram of a 12-bit digit of
//                     the score bits, rescaled to the per-head [min, max] range
//                     that the score kernel recorded; merged with global atomics.
//   2. k_topk_filter  one pass over the scores: every work-group finds the boundary
//                     bin from the histogram; keys above it are flagged, keys in
//                     it are appended to a per-head candidate list.
//   3. k_topk_refine  one work-group per head takes the `need` largest of the
//                     candidates: radix passes over the list while it is larger
//                     than LDS, else a bitonic sort of the next power-of-two size
//                     staged in registers (in-thread and cross-lane shuffle stages)
//                     and LDS (cross-wave stages).
// Flags of the coarsest level are set to 1 by the filter.
#include <type_traits>

#include "lh_internal.h"

namespace lh {

namespace {

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

__global__ __launch_bounds__(256) void k_topk_hist(Shape s, char *__restrict__ ws, FwdWs w,
                                                   const float *__restrict__ scores) {
  __shared__ unsigned int hist[kHistBins];
  const int h = blockIdx.y;
  for (int i = threadIdx.x; i < kHistBins; i += 256) hist[i] = 0;
  const TopkState st = reinterpret_cast<const TopkState *>(ws + w.state)[h];
  const int sh = digit_shift(st.umin, st.umax);
  __syncthreads();
  const float *qk = scores + (long long)h * 2 * s.P, *kq = qk + s.P;
  for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < s.E; i += (long long)gridDim.x * 256)
    atomicAdd(&hist[key_digit(make_key(qk[i], kq[i], (int)i, s.P), st.umin, sh)], 1u);
  __syncthreads();
  unsigned int *gh = reinterpret_cast<unsigned int *>(ws + w.hist) + (long long)h * kHistBins;
  for (int i = threadIdx.x; i < kHistBins; i += 256)
    if (hist[i]) atomicAdd(&gh[i], hist[i]);
}

// Boundary bin b* of head h: count(digit > b*) < Bsel <= count(digit >= b*).
// Returns b* and writes the count above it.  256 threads, 16 bins each.
__device__ int find_boundary(const unsigned int *gh, long long Bsel, long long *above_out) {
  __shared__ unsigned long long part[256];
  __shared__ int bstar_s;
  __shared__ unsigned long long above_s;
  constexpr int PER = kHistBins / 256;
  const int t = threadIdx.x;
  unsigned long long mine = 0;
  unsigned int c[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    c[i] = gh[t * PER + i];
    mine += c[i];
  }
  part[t] = mine;
  if (t == 0) {
    bstar_s = -1;
    above_s = 0;
  }
  __syncthreads();
  // suffix sums over threads (higher threads hold higher bins)
  for (int off = 1; off < 256; off <<= 1) {
    unsigned long long add = (t + off < 256) ? part[t + off] : 0;
    __syncthreads();
    part[t] += add;
    __syncthreads();
  }
  const unsigned long long incl = part[t];          // bins >= t*PER
  const unsigned long long excl = incl - mine;      // bins >  t*PER+PER-1
  if (excl < (unsigned long long)Bsel && (unsigned long long)Bsel <= incl) {
    unsigned long long acc = excl;
    for (int i = PER - 1; i >= 0; --i) {
      if (acc + c[i] >= (unsigned long long)Bsel) {
        bstar_s = t * PER + i;
        above_s = acc;
        break;
      }
      acc += c[i];
    }
  }
  __syncthreads();
  *above_out = (long long)above_s;
  return bstar_s;
}

__global__ __launch_bounds__(256) void k_topk_filter(Shape s, char *__restrict__ ws, FwdWs w,
                                                     const float *__restrict__ scores, uint8_t *__restrict__ flags) {
  const int h = blockIdx.y;
  TopkState *stp = reinterpret_cast<TopkState *>(ws + w.state) + h;
  const TopkState st = *stp;
  int bstar;
  long long above = 0;
  if (s.Bsel == 0) {
    bstar = kHistBins;          // nothing selected
  } else if (s.Bsel == s.E) {
    bstar = -1;                 // everything selected
  } else {
    bstar = find_boundary(reinterpret_cast<const unsigned int *>(ws + w.hist) + (long long)h * kHistBins,
                          s.Bsel, &above);
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    stp->bstar = (unsigned int)bstar;
    stp->need = (bstar < 0 || bstar >= kHistBins) ? 0 : (long long)s.Bsel - above;
  }
  const int sh = digit_shift(st.umin, st.umax);
  const float *qk = scores + (long long)h * 2 * s.P, *kq = qk + s.P;
  unsigned long long *cand = reinterpret_cast<unsigned long long *>(ws + w.cand) + (long long)h * s.E;
  uint8_t *fl = flags + (long long)h * s.P;
  const int lane = threadIdx.x & 63;
  for (long long i0 = (long long)blockIdx.x * 256; i0 < s.P; i0 += (long long)gridDim.x * 256) {
    const long long i = i0 + threadIdx.x;
    bool boundary = false;
    unsigned long long key = 0;
    if (i < s.E) {
      key = make_key(qk[i], kq[i], (int)i, s.P);
      const int dg = (bstar < 0) ? kHistBins : (bstar >= kHistBins ? -1 : key_digit(key, st.umin, sh));
      fl[i] = (uint8_t)(dg > bstar ? 1 : 0);
      boundary = (dg == bstar);
    } else if (i < s.P) {
      fl[i] = 1;   // coarsest level: always in the index set
    }
    const unsigned long long m = __ballot(boundary);
    if (m) {
      unsigned int base = 0;
      const int leader = __ffsll((long long)m) - 1;
      if (lane == leader) base = atomicAdd(&stp->cand_count, (unsigned int)__popcll(m));
      base = __shfl(base, leader);
      if (boundary) {
        const unsigned long long below = m & ((1ull << lane) - 1ull);
        cand[base + __popcll(below)] = key;
      }
    }
  }
}

// Bitonic sort (descending) of NT*PER keys: element e = slot*NT + tid lives in
// register slot `slot` of thread `tid`.  Partners at distance j >= NT are in the
// same thread; 64 <= j < NT go through LDS; j < 64 are in the same wavefront and
// are exchanged with shuffles.
template <int NT, int PER>
__device__ void bitonic_sort_desc(unsigned long long (&x)[PER], unsigned long long *lds) {
  constexpr int n = NT * PER;
  const int tid = threadIdx.x;
  for (int k = 2; k <= n; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      if (j >= NT) {
        const int js = j / NT;
#pragma unroll
        for (int sl = 0; sl < PER; ++sl) {
          const int partner = sl ^ js;
          if (partner > sl) {
            const int e = sl * NT + tid;
            const bool desc = (e & k) == 0;
            const unsigned long long a = x[sl], b = x[partner];
            const bool swap = desc ? (a < b) : (a > b);
            if (swap) {
              x[sl] = b;
              x[partner] = a;
            }
          }
        }
      } else if (j >= 64) {
#pragma unroll
        for (int sl = 0; sl < PER; ++sl) lds[sl * NT + tid] = x[sl];
        __syncthreads();
#pragma unroll
        for (int sl = 0; sl < PER; ++sl) {
          const int e = sl * NT + tid;
          const unsigned long long y = lds[e ^ j];
          const bool lo = (e & j) == 0;
          const bool desc = (e & k) == 0;
          const unsigned long long mx = x[sl] > y ? x[sl] : y;
          const unsigned long long mn = x[sl] > y ? y : x[sl];
          x[sl] = (lo == desc) ? mx : mn;
        }
        __syncthreads();
      } else {
#pragma unroll
        for (int sl = 0; sl < PER; ++sl) {
          const int e = sl * NT + tid;
          const unsigned long long y = __shfl_xor(x[sl], j);
          const bool lo = (e & j) == 0;
          const bool desc = (e & k) == 0;
          const unsigned long long mx = x[sl] > y ? x[sl] : y;
          const unsigned long long mn = x[sl] > y ? y : x[sl];
          x[sl] = (lo == desc) ? mx : mn;
        }
      }
    }
  }
}

constexpr int kRefineThreads = 1024;

__global__ __launch_bounds__(kRefineThreads) void k_topk_refine(Shape s, char *__restrict__ ws, FwdWs w,
                                                                 uint8_t *__restrict__ flags) {
  constexpr int PER = kTopkCandLds / kRefineThreads;
  __shared__ unsigned long long lds[kTopkCandLds];
  __shared__ unsigned int hist[256];
  __shared__ unsigned long long sel_prefix;
  __shared__ long long sel_need;
  __shared__ int sel_done;
  const int h = blockIdx.x;
  const TopkState st = reinterpret_cast<const TopkState *>(ws + w.state)[h];
  const long long C = st.cand_count;
  long long need = st.need;
  if (need <= 0 || C == 0) return;
  const unsigned long long *cand = reinterpret_cast<const unsigned long long *>(ws + w.cand) + (long long)h * s.E;
  uint8_t *fl = flags + (long long)h * s.P;
  const int tid = threadIdx.x;
  if (need >= C) {
    for (long long i = tid; i < C; i += kRefineThreads) fl[key_flat(cand[i], s.P)] = 1;
    return;
  }
  // the candidates, padded with zeros to the next sort size (1024 .. kTopkCandLds
  // keys: one to PER per thread), sorted in registers and LDS; the first
  // `need` are selected
  auto sort_select = [&](auto per) {
    constexpr int R = decltype(per)::value;
    unsigned long long x[R];
#pragma unroll
    for (int sl = 0; sl < R; ++sl) {
      const long long e = (long long)sl * kRefineThreads + tid;
      x[sl] = e < C ? cand[e] : 0ull;   // 0 is below every real key (its low half is never 0)
    }
    bitonic_sort_desc<kRefineThreads, R>(x, lds);
#pragma unroll
    for (int sl = 0; sl < R; ++sl) {
      const long long e = (long long)sl * kRefineThreads + tid;
      if (e < need) fl[key_flat(x[sl], s.P)] = 1;
    }
  };
  static_assert(PER == 8, "sort sizes below");
  if (C <= kRefineThreads) return sort_select(std::integral_constant<int, 1>{});
  if (C <= 2 * kRefineThreads) return sort_select(std::integral_constant<int, 2>{});
  if (C <= 4 * kRefineThreads) return sort_select(std::integral_constant<int, 4>{});
  if (C <= kTopkCandLds) return sort_select(std::integral_constant<int, 8>{});
  // Radix select of the need-th largest key over the list in global memory:
  // 8-bit digits from the top; keys are unique, so the threshold is exact.
  unsigned long long prefix = 0, mask = 0;
  if (tid == 0) sel_done = 0;
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
    if (key >= prefix) fl[key_flat(key, s.P)] = 1;
  }
}

__global__ void k_topk_init(int BH, char *__restrict__ ws, FwdWs w) {
  // TopkState words: umin = ~0, everything else 0; then the histogram, all 0
  const long long nstate = (long long)BH * (sizeof(TopkState) / 4);
  const long long n = nstate + (long long)BH * kHistBins;
  unsigned int *st = reinterpret_cast<unsigned int *>(ws + w.state);
  unsigned int *hist = reinterpret_cast<unsigned int *>(ws + w.hist);
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (long long)gridDim.x * blockDim.x) {
    if (i < nstate) st[i] = (i % (sizeof(TopkState) / 4) == 0) ? 0xFFFFFFFFu : 0u;
    else hist[i - nstate] = 0u;
  }
}

}  // namespace

hipError_t launch_topk_init(const Shape &s, void *ws, const FwdWs &w, hipStream_t st) {
  const long long n = (long long)s.BH * (sizeof(TopkState) / 4 + kHistBins);
  int blocks = (int)((n + 255) / 256);
  if (blocks > 1024) blocks = 1024;
  k_topk_init<<<blocks, 256, 0, st>>>(s.BH, reinterpret_cast<char *>(ws), w);
  return hipGetLastError();
}

hipError_t launch_topk(const Shape &s, void *ws, const FwdWs &w, const float *scores, uint8_t *flags,
                       hipStream_t st) {
  char *wsb = reinterpret_cast<char *>(ws);
  const bool partial = s.Bsel > 0 && s.Bsel < s.E;
  if (partial) {
    const int nb = (int)((s.E + 256 * 16 - 1) / (256 * 16));
    k_topk_hist<<<dim3(nb, s.BH), 256, 0, st>>>(s, wsb, w, scores);
  }
  const int nbf = (int)((s.P + 256 * 8 - 1) / (256 * 8));
  k_topk_filter<<<dim3(nbf, s.BH), 256, 0, st>>>(s, wsb, w, scores, flags);
  if (partial) k_topk_refine<<<dim3(s.BH), kRefineThreads, 0, st>>>(s, wsb, w, flags);
  return hipGetLastError();
}

}  // namespace lh
