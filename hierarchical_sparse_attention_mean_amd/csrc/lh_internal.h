// Internal declarations shared by the HIP sources of liblighthouse.so.
// Shape arithmetic follows "Long Context Pre-Training with Lighthouse
// Attention": pyramid levels (Sec. 3.3), selection budget and sub-sequence
// length (Sec. 3.5, Eq. 8).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/lighthouse.h"

#define LH_MAX_LEVELS 24

namespace lh {

// Everything a kernel needs to know about one problem; passed by value.
struct Shape {
  int BH;                    // heads (B*H), processed independently
  int N;                     // base positions per head
  int d;                     // head dimension
  int L, p;                  // levels, pooling factor
  int io;                    // lh_dtype of q, k, v and of the pyramid / gathered rows
  int64_t topk;
  int n[LH_MAX_LEVELS];      // entries of level l: N / p^l
  int off[LH_MAX_LEVELS];    // flat offset of level l (level-major, finest first)
  int pw[LH_MAX_LEVELS];     // p^l
  int P;                     // pyramid entries per head
  int E;                     // candidates per head (levels 0..L-2)
  int Bsel;                  // selected candidates per head
  int S;                     // gathered length per head
  int Sv;                    // row stride of the transposed copies: S rounded up to a multiple of 64
  int ntile;                 // compaction tiles per head
  int npool;                 // pool+score work-groups per head and tensor (coarsest windows / windows per work-group)
};

// Pool+score work-groups of 256 threads: a row of d elements is spread over
// d / EL lanes (EL = 8 up to five levels, 4 beyond), so a work-group has
// 256 / (d / EL) row-groups.  A row-group walks one coarsest window, or, at
// five levels when p divides the row-group count, one of the p sub-windows of
// a coarsest window (pool_score_split).
__host__ __device__ inline int pool_score_rowgroups(int d, int L) { return 256 / (d / (L <= 5 ? 8 : 4)); }
__host__ __device__ inline bool pool_score_split(int d, int L, int p) {
  return L == 5 && pool_score_rowgroups(d, L) % p == 0;
}
// Coarsest windows per pool+score work-group.
__host__ __device__ inline int pool_score_windows(int d, int L, int p) {
  return pool_score_split(d, L, p) ? pool_score_rowgroups(d, L) / p : pool_score_rowgroups(d, L);
}

constexpr int kCompactTile = 1024;   // base positions per compaction work-group
constexpr int kHistBins = 4096;      // first radix-select digit of the top-k

// Work split of the top-k's histogram and filter passes over n entries of a
// head: up to maxb work-groups (kHistBlocks, kFilterBlocks) of kTopkThreads
// threads, each taking an equal chunk (a whole number of work-group widths) in
// rounds of kTopkRound entries per thread.
constexpr int kTopkThreads = 1024;
constexpr int kHistBlocks = 32;     // few work-groups: each merges its histogram with global atomics
constexpr int kFilterBlocks = 64;   // two per compute unit at 8 heads
constexpr int kTopkRound = 8;
__host__ __device__ inline int topk_blocks(long long n, int maxb) {
  const long long r = (long long)kTopkRound * kTopkThreads;
  const long long b = (n + r - 1) / r;
  return (int)(b < 1 ? 1 : (b > maxb ? maxb : b));
}
__host__ __device__ inline long long topk_chunk(long long n, int nb) {
  return ((n + nb - 1) / nb + kTopkThreads - 1) / kTopkThreads * kTopkThreads;
}

// Per-head state of the top-k (in the forward workspace).  The pool+score
// kernel clears it (and the histogram); the histogram pass writes the score
// range, the filter pass the boundary bin and `need`.
struct TopkState {
  unsigned int umin;        // min over candidates of the score bits (upper key half)
  unsigned int umax;        // max of the same
  unsigned int bstar;       // boundary bin
  unsigned int pad0;
  long long need;           // keys still to take from the boundary bin
  long long pad1;
};

// Forward workspace layout (byte offsets).
struct FwdWs {
  size_t lev[LH_MAX_LEVELS][3];  // pooled Q, K, V of level l >= 1 ([BH][n_l][d], io dtype)
  size_t brange;                 // uint2 [BH][2][npool]: (min, max) of each pool+score work-group's candidate score bits
  size_t state;                  // TopkState [BH]
  size_t hist;                   // uint32 [BH][kHistBins]
  size_t cand;                   // uint64 [BH][cstride]: boundary-bin keys, filter work-group b's at b * chunk
  size_t ccount;                 // uint32 [BH][kFilterBlocks]: keys each filter work-group wrote
  size_t tilecount;              // int32 [BH][ntile]
  long long cstride;             // candidate slots per head: filter work-groups x chunk (>= P)
  size_t total;
};

// Backward workspace layout.
struct BwdWs {
  size_t dot;     // fp32 [BH][S][d]  gradient of O~ (LH_F32 mode)
  size_t dotb;    // bf16 [BH][Sv][d] gradient of O~ (LH_BF16 mode); rows S..Sv-1 zero
  size_t delta;   // fp32 [BH][S]     rowsum(dO~ * O~) (LH_F32 mode)
  size_t rows;    // fp32 [BH][Sv][2] (LSE log2(e), rowsum(dO~ * O~)) per row (LH_BF16 mode); rows S..Sv-1 zero
  size_t dqt;     // fp32 [BH][S][d]
  size_t dkt;     // fp32 [BH][S][d]
  size_t dvt;     // fp32 [BH][S][d]
  size_t total;
};

// Matrix view for the layer's products: element (r, c) of a matrix whose column
// index c runs over up to three stored matrices side by side (which = c / seg),
// each made of column blocks of width hd stored hstride elements apart:
//   elem(b, r, c) = p[which] + b bstride + (cc / hd) hstride + r ld + cc % hd,   cc = c % seg.
// Row-major [R][C]: seg = hd = C, hstride = 0, ld = C.  Head layout [B][H][N][d]
// seen as the [N][H d] matrix of a layer: seg = H d, hd = d, hstride = N d, ld = d,
// bstride = H N d.  Element offsets, not bytes.
struct MatView {
  const void *p[3];
  long long seg, hd, hstride, ld, bstride;
};

// C[m][n] = sum_k A[m][k] B[k][n] for m < M, n < N, k < K, per batch element.
// Split-K: split z covers k in [z kchunk, min(K, (z+1) kchunk)) and writes its
// partial product at C + z zstride (elements).
struct GemmArgs {
  int M, N, K;
  MatView a, b, c;
  int kchunk, splits;
  long long zstride;
};

// ---- bf16 helpers (storage is raw uint16 bit patterns) ----
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(((unsigned int)b) << 16);
}
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  unsigned int u = __float_as_uint(f);
  u = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
  return (uint16_t)u;
}

template <typename T> struct IO;
template <> struct IO<float> {
  static __device__ __forceinline__ float ld(const float *p, long long i) { return p[i]; }
  static __device__ __forceinline__ void st(float *p, long long i, float v) { p[i] = v; }
};
template <> struct IO<uint16_t> {
  static __device__ __forceinline__ float ld(const uint16_t *p, long long i) { return bf16_to_f32(p[i]); }
  static __device__ __forceinline__ void st(uint16_t *p, long long i, float v) { p[i] = f32_to_bf16_rne(v); }
};

// 64-bit selection key of candidate f (flat index) from its two scores:
//   key = bits(max(QK, KQ)) << 32 | (0xFFFFFFFF - g),
// g = f if QK >= KQ else P + f (stream index of the larger score).  Scores are
// non-negative, so the float bits order like the values, and "larger key"
// means "larger score, then lower stream index": the order of the joint
// selection over the concatenated QK || KQ stream.  Keys are unique.
__device__ __forceinline__ unsigned long long make_key(float qk, float kq, int f, int P) {
  const float r = fmaxf(qk, kq);
  const unsigned int g = (qk >= kq) ? (unsigned int)f : (unsigned int)(P + f);
  return ((unsigned long long)__float_as_uint(r) << 32) | (unsigned long long)(0xFFFFFFFFu - g);
}

// ---- kernel launches ----
// Stage timing of the calling host thread: while a timed stage is open (see
// lh_timing_begin), every launch carries the stage's stop event and the first
// one also its start event, recorded by the kernel dispatches themselves
// (hipExtLaunchKernel), so timing adds no packets between the kernels.
struct LaunchTiming {
  hipEvent_t start, stop;
  bool started;   // a launch has carried the start event
};
extern thread_local LaunchTiming *t_launch_timing;   // null unless a timed stage is open

template <typename... KArgs, typename... Args>
inline void launch(void (*kernel)(KArgs...), dim3 grid, dim3 block, unsigned shmem, hipStream_t st, Args... args) {
  static_assert(sizeof...(KArgs) == sizeof...(Args), "kernel arguments");
  LaunchTiming *lt = t_launch_timing;
  if (!lt) {
    hipLaunchKernelGGL(kernel, grid, block, shmem, st, static_cast<KArgs>(args)...);
    return;
  }
  hipExtLaunchKernelGGL(kernel, grid, block, shmem, st, lt->started ? nullptr : lt->start, lt->stop, 0,
                        static_cast<KArgs>(args)...);
  lt->started = true;
}

// ---- launchers (each enqueues on `st`, returns hipGetLastError()) ----
hipError_t launch_pool_score(const Shape &s, const void *q, const void *k, const void *v, void *ws,
                             const FwdWs &w, float *scores, hipStream_t st);
hipError_t launch_topk(const Shape &s, void *ws, const FwdWs &w, const float *scores, uint8_t *flags,
                       hipStream_t st);
hipError_t launch_compact_gather(const Shape &s, const void *q, const void *k, const void *v, void *ws,
                                 const FwdWs &w, const uint8_t *flags, int *slot, int *coords,
                                 void *qt, void *kt, void *vt, hipStream_t st);
hipError_t launch_scatter(const Shape &s, const int *slot, const int *coords, const float *ot, void *o,
                          int o_dtype, hipStream_t st);
hipError_t launch_scatter_bwd(const Shape &s, const void *dout, int dout_dtype, const int *slot, const int *coords,
                              const float *ot, const float *lse, float *dot32, uint16_t *dotb, float *delta,
                              float *rows, hipStream_t st);
hipError_t launch_pool_bwd(const Shape &s, const int *slot, const float *dqt, const float *dkt,
                           const float *dvt, void *dq, void *dk, void *dv, int grad_dtype, hipStream_t st);
// akm / bkm: A / B k-major (view (r, c) = (m, k) / (n, k)), else mn-major ((k, m) / (k, n)).
// io: operand dtype (LH_BF16: MFMA; LH_F32: vector ALU).  grid.y = batch.
int gemm_blocks(const GemmArgs &g, int io);
hipError_t launch_gemm(const GemmArgs &g, bool akm, bool bkm, int io, int out_dtype, int batch, hipStream_t st);
// out(r, c) (fp32) = sum over the nparts fp32 partials [nparts][M][N], in order.
hipError_t launch_split_reduce(const float *part, int nparts, int M, int N, const MatView &out, hipStream_t st);

}  // namespace lh
