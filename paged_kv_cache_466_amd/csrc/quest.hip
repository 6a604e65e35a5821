// Query-aware page selection for gfx950 ("KV Cache Engineering for LLM
// Serving", section 7 "Query-aware sparse reads"): a page is one physical
// block; it keeps the elementwise minimum and maximum of its keys; a query
// scores a page by the sum over dimensions of max(q * min, q * max), the
// largest q . k any key inside the page's box can reach; the highest-scoring
// pages of each (sequence, KV head) are read, every entry stays stored.
//
// Kernels:
//  * quest_summarize_kernel - minimum / maximum per (block, KV head, dim)
//    over the block's written rows, stored in the cache's 16-bit type (exact:
//    both are stored values).  Layout [NB][Hkv][2][D].
//  * quest_score_kernel - the score of every page of every (sequence, KV
//    head): the largest over the group's query heads, in fp64 (each product
//    of two 16-bit values is exact there), stored as an order-preserving
//    64-bit key.  One lane per page, 64 pages per wave; the query parts
//    are held in LDS and reach the FMAs by DPP row broadcasts.
//  * quest_select_kernel - per (sequence, KV head), the `budget` largest
//    keys by a radix select (11-bit digits from the highest bit where keys
//    differ, stopping once a digit's bin is kept whole) over the keys held
//    in LDS (LDS histograms), ties to the lower page, written in logical
//    order as (physical block, logical block).
#include <hip/hip_runtime.h>

#include <type_traits>

#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {

namespace {

constexpr int kBS = 16;

__device__ __forceinline__ int clamp_len_q(int L, int mbs) {
  const int cap = mbs * kBS;
  return L < 0 ? 0 : (L > cap ? cap : L);
}

__device__ __forceinline__ int table_pb(const int32_t* bt, int mbs, int s, int lb, int num_blocks) {
  const int pb = bt[(size_t)s * mbs + lb];
  return (pb < 0 || pb >= num_blocks) ? 0 : pb;   // a bad table must not leave the arrays
}

template <typename T>
__device__ __forceinline__ float ld16(const uint16_t* p, size_t i) {
  return std::is_same<T, BF16>::value ? bf16_to_f32(p[i]) : f16_to_f32(p[i]);
}
template <typename T>
__device__ __forceinline__ float cvt16(uint16_t b) {
  return std::is_same<T, BF16>::value ? bf16_to_f32(b) : f16_to_f32(b);
}
template <typename T>
__device__ __forceinline__ uint16_t st16(float x) {
  return std::is_same<T, BF16>::value ? f32_to_bf16(x) : f32_to_f16(x);
}

// grid (S, blocks per sequence or 1), 256 threads: one (sequence, logical
// block), all KV heads and dimensions.
template <typename T>
__global__ __launch_bounds__(256) void quest_summarize_kernel(const uint16_t* __restrict__ k_cache,
                                                              uint16_t* __restrict__ summ,
                                                              const int32_t* __restrict__ bt, int mbs,
                                                              const int32_t* __restrict__ lens, int num_blocks,
                                                              int Hkv, int D, int last_only) {
  const int s = blockIdx.x;
  const int L = clamp_len_q(lens[s], mbs);
  const int nb = (L + kBS - 1) / kBS;
  const int lb = last_only ? nb - 1 : (int)blockIdx.y;
  if (lb < 0 || lb >= nb) return;
  const int pb = table_pb(bt, mbs, s, lb, num_blocks);
  const int rows = min(kBS, L - lb * kBS);
  const int row_elems = Hkv * D;
  for (int i = threadIdx.x; i < row_elems; i += 256) {
    float mn = INFINITY, mx = -INFINITY;
    for (int r = 0; r < rows; ++r) {
      const float v = ld16<T>(k_cache, ((size_t)pb * kBS + r) * row_elems + i);
      mn = fminf(mn, v);
      mx = fmaxf(mx, v);
    }
    const int h = i / D, d = i - h * D;
    uint16_t* o = summ + ((size_t)pb * Hkv + h) * 2 * D;
    o[d] = st16<T>(mn);
    o[D + d] = st16<T>(mx);
  }
}

// Order-preserving map of a double onto uint64 (larger value, larger key).
__device__ __forceinline__ uint64_t order_key(double x) {
  const uint64_t b = __builtin_bit_cast(uint64_t, x);
  return (b >> 63) ? ~b : (b | (1ull << 63));
}

// Query heads of a group padded to a power of two (at most 16); the padded
// heads repeat the last one, so the largest score over them is unchanged.
__host__ __device__ constexpr int padded_group(int G) { return G <= 1 ? 1 : G <= 2 ? 2 : G <= 4 ? 4 : G <= 8 ? 8 : 16; }

// The query parts of one (sequence, KV head) as doubles in LDS, in the
// order the scoring stages use them: stage st pairs the minima (st even,
// with q- = min(q, 0)) or the maxima (st odd, with q+ = max(q, 0)) of
// dimensions 64 (st / 2) .. +63 with the parts of all GP (padded) heads;
// value f = st * 64 GP + i GP + g (dimension 64 (st / 2) + i, head g, both
// parts exact) is entry f % 16 of register pair f / 16 of a 16-lane row.
// Pairs are stored two at a time per row position: pair v, position n at
// byte ((v / 2) * 16 + n) * 16 + (v % 2) * 8, so that lane n of a row
// reads pairs v and v + 1 with one 16-byte load.
__host__ __device__ constexpr int quest_q_bytes(int D, int GP) { return D * 2 * GP * 8; }
__device__ __forceinline__ int quest_q_offset(int f) { return ((f >> 5) * 16 + (f & 15)) * 16 + ((f >> 4) & 1) * 8; }

// acc[i] += (entry B + i of q's row) * x for i < N: v_fmac_f64 with a DPP
// row broadcast of its first operand.  The leading s_nop covers the two
// wait states a DPP read needs after a VALU write of its source.
template <int N, int B>
__device__ __forceinline__ void fmac_row_bcast(double* acc, double q, double x);
template <int B>
__device__ __forceinline__ void fmac_row_bcast1(double* a, double q, double x) {
  asm volatile(
      "s_nop 1\n"
      "v_fmac_f64_dpp %0, %1, %2 row_newbcast:%3 row_mask:0xf bank_mask:0xf"
      : "+v"(a[0])
      : "v"(q), "v"(x), "n"(B));
}
template <int B>
__device__ __forceinline__ void fmac_row_bcast2(double* a, double q, double x) {
  asm volatile(
      "s_nop 1\n"
      "v_fmac_f64_dpp %0, %2, %3 row_newbcast:%4 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %1, %2, %3 row_newbcast:%5 row_mask:0xf bank_mask:0xf"
      : "+v"(a[0]), "+v"(a[1])
      : "v"(q), "v"(x), "n"(B), "n"(B + 1));
}
template <int B>
__device__ __forceinline__ void fmac_row_bcast4(double* a, double q, double x) {
  asm volatile(
      "s_nop 1\n"
      "v_fmac_f64_dpp %0, %4, %5 row_newbcast:%6 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %1, %4, %5 row_newbcast:%7 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %2, %4, %5 row_newbcast:%8 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %3, %4, %5 row_newbcast:%9 row_mask:0xf bank_mask:0xf"
      : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3])
      : "v"(q), "v"(x), "n"(B), "n"(B + 1), "n"(B + 2), "n"(B + 3));
}
template <int B>
__device__ __forceinline__ void fmac_row_bcast8(double* a, double q, double x) {
  asm volatile(
      "s_nop 1\n"
      "v_fmac_f64_dpp %0, %8, %9 row_newbcast:%10 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %1, %8, %9 row_newbcast:%11 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %2, %8, %9 row_newbcast:%12 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %3, %8, %9 row_newbcast:%13 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %4, %8, %9 row_newbcast:%14 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %5, %8, %9 row_newbcast:%15 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %6, %8, %9 row_newbcast:%16 row_mask:0xf bank_mask:0xf\n"
      "v_fmac_f64_dpp %7, %8, %9 row_newbcast:%17 row_mask:0xf bank_mask:0xf"
      : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]), "+v"(a[4]), "+v"(a[5]), "+v"(a[6]), "+v"(a[7])
      : "v"(q), "v"(x), "n"(B), "n"(B + 1), "n"(B + 2), "n"(B + 3), "n"(B + 4), "n"(B + 5), "n"(B + 6),
        "n"(B + 7));
}
template <int N, int B>
__device__ __forceinline__ void fmac_row_bcast(double* acc, double q, double x) {
  if constexpr (N == 1) fmac_row_bcast1<B>(acc, q, x);
  else if constexpr (N == 2) fmac_row_bcast2<B>(acc, q, x);
  else if constexpr (N == 4) fmac_row_bcast4<B>(acc, q, x);
  else fmac_row_bcast8<B>(acc, q, x);
}

constexpr int kScorePages = 64;   // pages per scoring wave: one per lane
constexpr int kScoreWaves = 4;    // waves per scoring workgroup
constexpr int kScoreStageDims = 64;   // dimensions of a stage (one 128-byte line of minima or maxima)

template <typename T>
__device__ __forceinline__ double cvt_d(uint32_t w, int upper) {
  if constexpr (std::is_same<T, BF16>::value)
    return (double)__builtin_bit_cast(float, upper ? (w & 0xffff0000u) : (w << 16));
  else
    return (double)f16_to_f32((uint16_t)(upper ? w >> 16 : w));
}

// acc[g] += (part of head g for dimension i) * x for the GP heads; qv: the
// register pairs of query parts from the one holding dimension 0 on.
template <int GP>
__device__ __forceinline__ void score_dim(double* acc, const double* qv, int i, double x) {
  if constexpr (GP == 16) {
    fmac_row_bcast<8, 0>(acc, qv[i], x);
    fmac_row_bcast<8, 8>(acc + 8, qv[i], x);
  } else {
    constexpr int PER = 16 / GP;   // dimensions per register pair
    const double q = qv[i / PER];
    switch (i % PER) {   // a constant after unrolling
#define PKV_SCORE_DIM(R)                                        \
  case R:                                                       \
    if constexpr (R < PER) fmac_row_bcast<GP, R * GP>(acc, q, x); \
    break;
      PKV_SCORE_DIM(0) PKV_SCORE_DIM(1) PKV_SCORE_DIM(2) PKV_SCORE_DIM(3)
      PKV_SCORE_DIM(4) PKV_SCORE_DIM(5) PKV_SCORE_DIM(6) PKV_SCORE_DIM(7)
      PKV_SCORE_DIM(8) PKV_SCORE_DIM(9) PKV_SCORE_DIM(10) PKV_SCORE_DIM(11)
      PKV_SCORE_DIM(12) PKV_SCORE_DIM(13) PKV_SCORE_DIM(14) PKV_SCORE_DIM(15)
#undef PKV_SCORE_DIM
    }
  }
}

// grid (S * Hkv, ceil(mbs / 256)), 4 waves: lane i of wave w scores page
// lb0 + 64 w + i.  With q+ = max(q, 0) and q- = min(q, 0), max(q * min, q *
// max) = q+ * max + q- * min (min <= max), so a head's score is two fp64
// dot products of exact products, one over the page's minima and one over
// its maxima.  The workgroup first writes its query group's parts to LDS
// (layout above); they reach the FMAs by DPP row broadcasts.  Each lane
// reads its own page's summary in stages of one 128-byte line (64 minima
// or 64 maxima), two stages in flight.
template <typename T, int D, int GP>
__global__ __launch_bounds__(64 * kScoreWaves) void quest_score_kernel(const uint16_t* __restrict__ query,
                                                                       const uint16_t* __restrict__ summ,
                                                                       const int32_t* __restrict__ bt, int mbs,
                                                                       const int32_t* __restrict__ lens,
                                                                       int num_blocks, int Hq, int Hkv,
                                                                       uint64_t* __restrict__ keys) {
  constexpr int NST = 2 * D / kScoreStageDims;     // stages: minima and maxima of each 64 dimensions
  constexpr int PPS = kScoreStageDims * GP / 16;   // register pairs of query parts per stage
  constexpr int QPIECES = GP * D / 8;              // 8-dimension pieces of the (padded) query group
  static_assert(NST >= 2 && QPIECES <= 64 * kScoreWaves, "shape");
  __shared__ __attribute__((aligned(16))) uint8_t qs[quest_q_bytes(D, GP)];
  const int sk = blockIdx.x, s = sk / Hkv, kvh = sk - s * Hkv;
  const int L = clamp_len_q(lens[s], mbs);
  const int nb = (L + kBS - 1) / kBS;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int lb0 = (blockIdx.y * kScoreWaves + wave) * kScorePages;
  if (blockIdx.y * kScoreWaves * kScorePages >= nb) return;
  // thread t < QPIECES: dimensions 8 (t % (D / 8)) .. +7 of (padded) head
  // t / (D / 8); heads past the group repeat its last one
  const int G = Hq / Hkv;
  const int qg = threadIdx.x / (D / 8), qd8 = threadIdx.x % (D / 8);
  uint4 qraw = make_uint4(0, 0, 0, 0);
  if (threadIdx.x < QPIECES)
    qraw = *reinterpret_cast<const uint4*>(query + ((size_t)s * Hq + kvh * G + min(qg, G - 1)) * D + 8 * qd8);
  // a wave past the last page scores copies of it (nothing is stored)
  const int pb = table_pb(bt, mbs, s, min(lb0 + lane, nb - 1), num_blocks);
  if (threadIdx.x < QPIECES) {
    const uint32_t w[4] = {qraw.x, qraw.y, qraw.z, qraw.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const double x = cvt_d<T>(w[e >> 1], e & 1);
      const int d = 8 * qd8 + e;
      const int fmin = 2 * (d / kScoreStageDims) * kScoreStageDims * GP + (d % kScoreStageDims) * GP + qg;
      *reinterpret_cast<double*>(qs + quest_q_offset(fmin)) = x < 0.0 ? x : 0.0;
      *reinterpret_cast<double*>(qs + quest_q_offset(fmin + kScoreStageDims * GP)) = x > 0.0 ? x : 0.0;
    }
  }
  // stage st: 8 pieces of 16 bytes of the minima (st even) or maxima (st odd)
  const uint4* page = reinterpret_cast<const uint4*>(summ + ((size_t)pb * Hkv + kvh) * 2 * D);
  auto piece = [&](int st, int c) { return page[(st & 1) * (D / 8) + (st >> 1) * 8 + c]; };
  __builtin_amdgcn_sched_barrier(0);
  uint4 ra[8], rb[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) ra[c] = piece(0, c);
#pragma unroll
  for (int c = 0; c < 8; ++c) rb[c] = piece(1, c);
  __builtin_amdgcn_sched_barrier(0);
  // lgkmcnt(0): this wave's query stores are done (the stage loads stay in
  // flight; __syncthreads() would wait for them too)
  __builtin_amdgcn_s_waitcnt(0xC07F);
  asm volatile("s_barrier" ::: "memory");
  const int qrow = (lane & 15) * 16;   // this lane's row position in qs
  // one sum per head over both parts (every product is exact, so the order
  // of the additions does not change it)
  double acc[GP];
#pragma unroll
  for (int h = 0; h < GP; ++h) acc[h] = 0.0;
#pragma unroll
  for (int st = 0; st < NST; ++st) {
    const uint4* r = (st & 1) ? rb : ra;
    // the stage's query parts half at a time (32 dimensions), so that four
    // waves fit on a SIMD
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      constexpr int HP = PPS / 2;   // register pairs per half stage
      double qv[HP];
#pragma unroll
      for (int i = 0; i < HP; i += 2) {
        const double2 t = *reinterpret_cast<const double2*>(qs + ((st * PPS + half * HP + i) / 2) * 256 + qrow);
        qv[i] = t.x;
        qv[i + 1] = t.y;
      }
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const uint4 p4 = r[4 * half + c];
        const uint32_t w[4] = {p4.x, p4.y, p4.z, p4.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) score_dim<GP>(acc, qv, 8 * c + e, cvt_d<T>(w[e >> 1], e & 1));
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // the next stage into this stage's registers (kept in this order)
    if (st + 2 < NST) {
      uint4* rr = (st & 1) ? rb : ra;
#pragma unroll
      for (int c = 0; c < 8; ++c) rr[c] = piece(st + 2, c);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  double best = acc[0];
#pragma unroll
  for (int h = 1; h < GP; ++h) best = fmax(best, acc[h]);
  if (lb0 + lane < nb) keys[(size_t)sk * mbs + lb0 + lane] = order_key(best);
}

constexpr int kSelThreads = 1024;   // threads of a selection workgroup (16 waves)
constexpr int kSelLoad = 4;          // key loads in flight per thread
constexpr int kDigitBits = 11;       // radix digits: 11, 11, 11, 11, 11, 9 bits
constexpr int kBins = 1 << kDigitBits;

// Exclusive scan over a kSelThreads-thread workgroup; returns the thread's
// prefix and writes the total to *total.
__device__ __forceinline__ int block_scan(int x, int* tmp, int* total) {
  constexpr int W = kSelThreads / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = x;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(incl, o, 64);
    if (lane >= o) incl += y;
  }
  if (lane == 63) tmp[wave] = incl;
  __syncthreads();
  int base = 0, all = 0;
#pragma unroll
  for (int w = 0; w < W; ++w) {
    base += w < wave ? tmp[w] : 0;
    all += tmp[w];
  }
  *total = all;
  __syncthreads();
  return base + incl - x;
}

// OR of x over a kSelThreads-thread workgroup.
__device__ __forceinline__ uint64_t block_or(uint64_t x, uint64_t* tmp64) {
  constexpr int W = kSelThreads / 64;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x |= __shfl_xor(x, o, 64);
  if ((threadIdx.x & 63) == 0) tmp64[threadIdx.x >> 6] = x;
  __syncthreads();
  uint64_t all = 0;
#pragma unroll
  for (int w = 0; w < W; ++w) all |= tmp64[w];
  __syncthreads();
  return all;
}

// grid (S * Hkv), kSelThreads threads.  IN_LDS: the keys of the (sequence,
// KV head) are first copied to LDS; otherwise every pass reads them from
// global memory.  Thread t owns the contiguous run of keys [t * per,
// (t + 1) * per).  Radix select of the budget-th largest key, 11 bits at a
// time from the highest bit where the keys differ, with LDS histogram
// atomics, stopping early once the digit's whole bin is kept; then every
// larger key is kept, and the first keys equal to it in page order until
// the budget is met.
template <bool IN_LDS>
__global__ __launch_bounds__(kSelThreads) void quest_select_kernel(const uint64_t* __restrict__ keys,
                                                                   const int32_t* __restrict__ bt, int mbs,
                                                                   const int32_t* __restrict__ lens,
                                                                   int num_blocks, int Hkv, int budget,
                                                                   int32_t* __restrict__ selected) {
  extern __shared__ uint64_t kl[];
  __shared__ int hist[kBins];
  __shared__ int pick[3];
  __shared__ int tmp[kSelThreads / 64];
  __shared__ uint64_t tmp64[kSelThreads / 64];
  const int tid = threadIdx.x;
  const int s = blockIdx.x / Hkv;
  const int L = clamp_len_q(lens[s], mbs);
  const int nb = (L + kBS - 1) / kBS;
  int2* out = reinterpret_cast<int2*>(selected) + (size_t)blockIdx.x * budget;
  if (nb <= budget) {
    for (int i = tid; i < nb; i += kSelThreads) out[i] = make_int2(table_pb(bt, mbs, s, i, num_blocks), i);
    return;
  }
  const uint64_t* kg = keys + (size_t)blockIdx.x * mbs;
  if constexpr (IN_LDS) {
    for (int i0 = 0; i0 < nb; i0 += kSelThreads * kSelLoad) {
      uint64_t v[kSelLoad];
#pragma unroll
      for (int u = 0; u < kSelLoad; ++u) v[u] = kg[min(i0 + u * kSelThreads + tid, nb - 1)];
#pragma unroll
      for (int u = 0; u < kSelLoad; ++u)
        if (i0 + u * kSelThreads + tid < nb) kl[i0 + u * kSelThreads + tid] = v[u];
    }
    __syncthreads();
  }
  auto key_at = [&](int i) { return IN_LDS ? kl[i] : kg[i]; };
  const int per = (nb + kSelThreads - 1) / kSelThreads;
  const int r0 = min(nb, tid * per), r1 = min(nb, r0 + per);
  // bits every key shares need no pass (their digits would all fall in one
  // bin): start below the highest bit where two keys differ
  const uint64_t k0 = key_at(0);
  uint64_t dif = 0;
  for (int i = r0; i < r1; ++i) dif |= key_at(i) ^ k0;
  dif = block_or(dif, tmp64);
  int top = dif ? 64 - __clzll((long long)dif) : 0;
  uint64_t mask = top >= 64 ? 0 : ~0ull << top;
  uint64_t prefix = k0 & mask;
  int remaining = budget;   // keys still to take among those whose masked bits equal prefix
  while (top > 0) {
    const int bits = top < kDigitBits ? top : kDigitBits;
    const int shift = top - bits;
    const int dmask = (1 << bits) - 1;
    for (int b = tid; b < kBins; b += kSelThreads) hist[b] = 0;
    __syncthreads();
    for (int st0 = 0; st0 < per; st0 += kSelLoad) {
      uint64_t v[kSelLoad];
#pragma unroll
      for (int u = 0; u < kSelLoad; ++u) v[u] = key_at(min(r0 + st0 + u, nb - 1));
#pragma unroll
      for (int u = 0; u < kSelLoad; ++u) {
        if (r0 + st0 + u < r1 && (v[u] & mask) == prefix) atomicAdd(&hist[(int)((v[u] >> shift) & dmask)], 1);
      }
    }
    __syncthreads();
    // thread t holds digits (kBins-1 - 2t) and (kBins-2 - 2t), largest first;
    // the digit where the count of larger keys first reaches `remaining`
    constexpr int BPT = kBins / kSelThreads;
    int c[BPT], sum = 0;
#pragma unroll
    for (int u = 0; u < BPT; ++u) {
      c[u] = hist[kBins - 1 - (tid * BPT + u)];
      sum += c[u];
    }
    int unused;
    int above = block_scan(sum, tmp, &unused);
#pragma unroll
    for (int u = 0; u < BPT; ++u) {
      if (above < remaining && above + c[u] >= remaining) {
        pick[0] = kBins - 1 - (tid * BPT + u);
        pick[1] = remaining - above;
        pick[2] = c[u];
      }
      above += c[u];
    }
    __syncthreads();
    prefix |= (uint64_t)pick[0] << shift;
    mask |= (uint64_t)dmask << shift;
    remaining = pick[1];
    top = shift;
    const bool whole_bin = pick[2] == remaining;   // every key in the digit's bin is kept
    __syncthreads();
    if (whole_bin) break;
  }
  // kept: keys whose masked bits exceed prefix, and the first `remaining`
  // (in page order) of those equal to it
  int eq = 0;
  for (int i = r0; i < r1; ++i) eq += (key_at(i) & mask) == prefix;
  int unused;
  int eq_seen = block_scan(eq, tmp, &unused);
  int nsel = 0;
  for (int i = r0; i < r1; ++i) {
    const uint64_t key = key_at(i) & mask;
    if (key > prefix) ++nsel;
    else if (key == prefix) nsel += (eq_seen++ < remaining);
  }
  int pos = block_scan(nsel, tmp, &unused);
  eq_seen -= eq;
  for (int i = r0; i < r1; ++i) {
    const uint64_t key = key_at(i) & mask;
    bool sel = key > prefix;
    if (key == prefix) sel = eq_seen++ < remaining;
    if (sel) out[pos++] = make_int2(table_pb(bt, mbs, s, i, num_blocks), i);
  }
}

}  // namespace

int launch_quest_summarize(const void* k_cache, int kv_dtype, void* k_summary, const int32_t* block_tables,
                           int max_blocks_per_seq, const int32_t* seq_lens, int num_seqs, int num_blocks,
                           int num_kv_heads, int head_dim, int last_only, void* stream) {
  const dim3 grid(num_seqs, last_only ? 1 : max_blocks_per_seq);
  hipStream_t st = (hipStream_t)stream;
  auto k = reinterpret_cast<const uint16_t*>(k_cache);
  auto o = reinterpret_cast<uint16_t*>(k_summary);
  if (kv_dtype == PKV_BF16)
    quest_summarize_kernel<BF16><<<grid, 256, 0, st>>>(k, o, block_tables, max_blocks_per_seq, seq_lens, num_blocks,
                                                       num_kv_heads, head_dim, last_only);
  else
    quest_summarize_kernel<F16><<<grid, 256, 0, st>>>(k, o, block_tables, max_blocks_per_seq, seq_lens, num_blocks,
                                                      num_kv_heads, head_dim, last_only);
  return hipGetLastError();
}

int launch_quest_select(const void* query, int q_dtype, const void* k_summary, const int32_t* block_tables,
                        int max_blocks_per_seq, const int32_t* seq_lens, int num_seqs, int num_q_heads,
                        int num_kv_heads, int head_dim, int num_blocks, int budget, int32_t* selected,
                        void* scratch, void* stream) {
  hipStream_t st = (hipStream_t)stream;
  auto q = reinterpret_cast<const uint16_t*>(query);
  auto sm = reinterpret_cast<const uint16_t*>(k_summary);
  auto keys = reinterpret_cast<uint64_t*>(scratch);
  const int GP = padded_group(num_q_heads / num_kv_heads);
  constexpr int kWgPages = kScorePages * kScoreWaves;
  const dim3 sgrid(num_seqs * num_kv_heads, (max_blocks_per_seq + kWgPages - 1) / kWgPages);
#define PKV_SCORE(T, D, G)                                                                              \
  quest_score_kernel<T, D, G><<<sgrid, 64 * kScoreWaves, 0, st>>>(q, sm, block_tables, max_blocks_per_seq, \
                                                                  seq_lens, num_blocks, num_q_heads, num_kv_heads, keys)
#define PKV_SCORE_G(T, D)              \
  switch (GP) {                        \
    case 1: PKV_SCORE(T, D, 1); break; \
    case 2: PKV_SCORE(T, D, 2); break; \
    case 4: PKV_SCORE(T, D, 4); break; \
    case 8: PKV_SCORE(T, D, 8); break; \
    default: PKV_SCORE(T, D, 16); break; \
  }
  if (q_dtype == PKV_BF16) {
    if (head_dim == 64) PKV_SCORE_G(BF16, 64) else PKV_SCORE_G(BF16, 128)
  } else {
    if (head_dim == 64) PKV_SCORE_G(F16, 64) else PKV_SCORE_G(F16, 128)
  }
#undef PKV_SCORE_G
#undef PKV_SCORE
  const int e = hipGetLastError();
  if (e != hipSuccess) return e;
  // keys in LDS: up to 16384 pages (128 KiB), enough for 256K-token
  // sequences; longer bounds read them from global memory
  constexpr int kMaxLdsKeys = 16384;
  const dim3 grid(num_seqs * num_kv_heads);
  if (max_blocks_per_seq <= kMaxLdsKeys) {
    static std::atomic<bool> lds_set[64];
    const hipError_t e2 =
        set_lds_limit_once(reinterpret_cast<const void*>(quest_select_kernel<true>), kMaxLdsKeys * 8, lds_set);
    if (e2 != hipSuccess) return e2;
    quest_select_kernel<true><<<grid, kSelThreads, (size_t)max_blocks_per_seq * 8, st>>>(
        keys, block_tables, max_blocks_per_seq, seq_lens, num_blocks, num_kv_heads, budget, selected);
  } else {
    quest_select_kernel<false><<<grid, kSelThreads, 0, st>>>(keys, block_tables, max_blocks_per_seq, seq_lens, num_blocks,
                                                     num_kv_heads, budget, selected);
  }
  return hipGetLastError();
}

}  // namespace pkv
