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
// Tables up to kPickMaxPages blocks wide take a shorter road to the same
// pages:
//  * quest_bound_kernel - every page's score on the matrix cores (16-bit
//    products exact in fp32, fp32 sums) with a bound on its error, stored
//    as a (lower, upper) pair per page.
//  * quest_pick_kernel - per (sequence, KV head), thresholds from the bounds
//    that settle most pages (surely kept, surely not), the exact fp64 score
//    of the few others, and the budget largest, ties to the lower page.
#include <hip/hip_runtime.h>

#include <algorithm>
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

constexpr int kSelThreads = 1024;   // threads of the exact-key selection workgroup (16 waves)
constexpr int kSelLoad = 4;          // key loads in flight per thread
constexpr int kDigitBits = 11;       // radix digits of 11 bits (the last one shorter)
constexpr int kBins = 1 << kDigitBits;

// Exclusive scan over an NT-thread workgroup; returns the thread's prefix
// and writes the total to *total.
template <int NT>
__device__ __forceinline__ int block_scan(int x, int* tmp, int* total) {
  constexpr int W = NT / 64;
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

// OR of x over an NT-thread workgroup.
template <int NT, typename K>
__device__ __forceinline__ K block_or(K x, K* tmpk) {
  constexpr int W = NT / 64;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x |= __shfl_xor(x, o, 64);
  if ((threadIdx.x & 63) == 0) tmpk[threadIdx.x >> 6] = x;
  __syncthreads();
  K all = 0;
#pragma unroll
  for (int w = 0; w < W; ++w) all |= tmpk[w];
  __syncthreads();
  return all;
}

// Sum of x over a wave.
__device__ __forceinline__ int wave_sum(int x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

// Lanes below this one whose bit is set in a wave-wide ballot.
__device__ __forceinline__ int lanes_below(uint64_t b) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(b >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)b, 0));
}

// Inclusive sum over the lanes up to this one: shifts by 1, 2, 4, 8 within
// each 16-lane row, then row 0's total into row 1 and row 2's into row 3
// (broadcast of lane 15 of each row), then lane 31's into rows 2 and 3.
__device__ __forceinline__ int wave_incl_scan(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);   // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);   // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);   // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);   // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);   // row_bcast:15 into rows 1, 3
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);   // row_bcast:31 into rows 2, 3
  return x;
}

// Radix select of the k-th largest (1 <= k <= n) of the keys key_at(0 ..
// n - 1) by an NT-thread workgroup.  Wave w sweeps the run [w * per, (w +
// 1) * per) (per a multiple of 64), lane l every 64th key from w * per + l,
// so a sweep reads consecutive keys across a wave.  Digits of kDigitBits
// from the highest bit where two keys differ, counted in LDS histograms;
// it stops early once the digit's whole bin is among the k largest.  On
// return fewer than k keys have (key & mask) > prefix, the k-th largest has
// (key & mask) == prefix, and the first `remaining` keys (in index order)
// with (key & mask) == prefix complete the k largest.
template <int NT, typename K, typename Get>
__device__ void radix_select(Get key_at, int n, int per, int k, int* hist, int* tmp, K* tmpk, int* pick,
                             K& prefix, K& mask, int& remaining) {
  constexpr int KB = 8 * (int)sizeof(K);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int r0 = min(n, wave * per), r1 = min(n, r0 + per);
  // bits every key shares need no pass (their digits would all fall in one
  // bin): start below the highest bit where two keys differ
  const K k0 = key_at(0);
  K dif = 0;
  for (int i = r0 + lane; i < r1; i += 64) dif |= key_at(i) ^ k0;
  dif = block_or<NT, K>(dif, tmpk);
  int top = 0;
  if (dif) top = KB - (sizeof(K) == 8 ? __clzll((long long)dif) : __clz((int)dif));
  mask = top >= KB ? K(0) : (K)(~K(0) << top);
  prefix = k0 & mask;
  remaining = k;   // keys still to take among those whose masked bits equal prefix
  while (top > 0) {
    const int bits = top < kDigitBits ? top : kDigitBits;
    const int shift = top - bits;
    const int dmask = (1 << bits) - 1;
    for (int b = tid; b < kBins; b += NT) hist[b] = 0;
    __syncthreads();
    for (int i0 = r0 + lane; i0 < r1; i0 += 64 * kSelLoad) {
      K v[kSelLoad];
#pragma unroll
      for (int u = 0; u < kSelLoad; ++u) v[u] = key_at(min(i0 + 64 * u, n - 1));
#pragma unroll
      for (int u = 0; u < kSelLoad; ++u) {
        if (i0 + 64 * u < r1 && (v[u] & mask) == prefix) atomicAdd(&hist[(int)((v[u] >> shift) & dmask)], 1);
      }
    }
    __syncthreads();
    // thread t holds digits kBins-1 - BPT t .. -(BPT-1), largest first; the
    // digit where the count of larger keys first reaches `remaining`
    constexpr int BPT = kBins / NT;
    int c[BPT], sum = 0;
#pragma unroll
    for (int u = 0; u < BPT; ++u) {
      c[u] = hist[kBins - 1 - (tid * BPT + u)];
      sum += c[u];
    }
    int unused;
    int above = block_scan<NT>(sum, tmp, &unused);
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
    prefix |= (K)pick[0] << shift;
    mask |= (K)dmask << shift;
    remaining = pick[1];
    top = shift;
    const bool whole_bin = pick[2] == remaining;   // every key in the digit's bin is kept
    __syncthreads();
    if (whole_bin) break;
  }
}

// grid (S * Hkv), kSelThreads threads: the budget largest of the exact
// keys the scoring kernel wrote.  IN_LDS: the keys of the (sequence, KV
// head) are first copied to LDS; otherwise every pass reads them from
// global memory.  Every larger key is kept, and the first keys equal to the
// budget-th largest in page order until the budget is met; written in page
// order, a wave keeping page order by ballots over its run.
template <bool IN_LDS>
__global__ __launch_bounds__(kSelThreads) void quest_select_kernel(const uint64_t* __restrict__ keys,
                                                                   const int32_t* __restrict__ bt, int mbs,
                                                                   const int32_t* __restrict__ lens,
                                                                   int num_blocks, int Hkv, int budget,
                                                                   int32_t* __restrict__ selected) {
  constexpr int W = kSelThreads / 64;
  extern __shared__ uint64_t kl[];
  __shared__ int hist[kBins];
  __shared__ int pick[3];
  __shared__ int tmp[W];
  __shared__ int cnt[2][W];
  __shared__ uint64_t tmp64[W];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
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
  const int per = (nb + 64 * W - 1) / (64 * W) * 64;
  const int r0 = min(nb, wave * per), r1 = min(nb, r0 + per);
  uint64_t prefix, mask;
  int remaining;
  radix_select<kSelThreads, uint64_t>(key_at, nb, per, budget, hist, tmp, tmp64, pick, prefix, mask, remaining);
  // per wave, the keys above and equal to prefix give its first output slot
  // and its first equal key's rank
  int gt = 0, eq = 0;
  for (int i = r0 + lane; i < r1; i += 64) {
    const uint64_t key = key_at(i) & mask;
    gt += key > prefix;
    eq += key == prefix;
  }
  gt = wave_sum(gt);
  eq = wave_sum(eq);
  if (lane == 0) {
    cnt[0][wave] = gt;
    cnt[1][wave] = eq;
  }
  __syncthreads();
  int pos = 0, eq_seen = 0;
  for (int w = 0; w < wave; ++w) {
    const int e = cnt[1][w];
    pos += cnt[0][w] + min(max(remaining - eq_seen, 0), e);
    eq_seen += e;
  }
  for (int i0 = r0; i0 < r1; i0 += 64) {
    const int i = i0 + lane;
    const uint64_t key = key_at(min(i, nb - 1)) & mask;
    const bool is_eq = i < r1 && key == prefix;
    const uint64_t be = __ballot(is_eq);
    const bool sel = i < r1 && (key > prefix || (is_eq && eq_seen + lanes_below(be) < remaining));
    const uint64_t bs = __ballot(sel);
    if (sel) out[pos + lanes_below(bs)] = make_int2(table_pb(bt, mbs, s, i, num_blocks), i);
    pos += __popcll(bs);
    eq_seen += __popcll(be);
  }
}

// ---------------------------------------------------------------------------
// Bounded selection (block tables up to kPickMaxPages wide): every page is
// scored once on MFMA in fp32 with a bound on the error, and only the pages
// whose place against the cut the bounds leave open are scored exactly.
// The pages chosen are those of the exact scores (the same as above).
// ---------------------------------------------------------------------------

constexpr int kBoundWaves = 4;    // waves per bounding workgroup
constexpr int kBoundGroups = 2;   // 16-page groups per wave, all loads issued first
constexpr int kBoundPages = 16 * kBoundGroups * kBoundWaves;   // pages per workgroup
constexpr int kPickMaxPages = 9216;                           // widest table taken here
constexpr int kPickWide = 4096;   // tables wider than this are picked by 1024 threads, others by 512

// Order-preserving map of a float onto uint32 (larger value, larger key).
__device__ __forceinline__ uint32_t order_key32(float x) {
  const uint32_t b = __builtin_bit_cast(uint32_t, x);
  return (b >> 31) ? ~b : (b | 0x80000000u);
}

// 0xffff in each 16-bit half of w whose sign bit is set.
__device__ __forceinline__ uint32_t sign_halves(uint32_t w) { return ((w >> 15) & 0x00010001u) * 0xffffu; }

// grid (S * Hkv, ceil(mbs / kBoundPages)), 4 waves: for every page, a lower
// and an upper bound of its score, stored as order keys (lower, upper).  A
// wave loads kBoundGroups groups of 16 pages, then bounds them.
//
// For a group of 16 pages: v_mfma_f32_16x16x32 with the query group
// as the A operand (row g: head min(g, G - 1), so padded rows repeat the
// last head) and the pages' summaries as the B operand (column c: page c;
// k < D the minima against q- = min(q, 0), k >= D the maxima against q+ =
// max(q, 0)), so a lane's B operand is 16 contiguous bytes of one summary
// and 4 lanes read 64 contiguous bytes.  A second product of the absolute
// values gives A_h = sum |products|.  Each product of two 16-bit values is
// exact in fp32; the sums round.  A fp32 sum of n terms in any order, with
// any rounding of each addition to 24 bits, or with the terms aligned to
// the largest and cut to 24 bits, is off by less than about n 2^-23 times
// the sum of the terms' magnitudes, at most 2^-15 A_h here (n <= 2 D + 1 =
// 257); the bound taken is 2^-13 A_h (4 times that, so it also covers the
// rounding of A_h and of the bound's own arithmetic) plus an absolute term
// for terms that underflow or are flushed: 2^-99 (bf16: a flushed denormal
// summary value, below 2^-126, times a query value of at most 2^18 over
// 256 terms, and sums below 2^-126 flushed), plus 2^-13 sum |q| for f16
// (flushed denormal summary values, below 2^-14).  A sum
// that is not finite gives no bound (lower -inf, upper +inf), and a query
// with a denormal element, or (bf16) one above 2^18, voids every bound of
// its (sequence, KV head) (the picking kernel checks it): such pages are
// scored exactly.  The page's bounds are the largest over the heads.
template <typename T, int D>
__global__ __launch_bounds__(64 * kBoundWaves) void quest_bound_kernel(const uint16_t* __restrict__ query,
                                                                       const uint16_t* __restrict__ summ,
                                                                       const int32_t* __restrict__ bt, int mbs,
                                                                       const int32_t* __restrict__ lens,
                                                                       int num_blocks, int Hq, int Hkv, int budget,
                                                                       uint2* __restrict__ bounds) {
  typedef Mfma<T> M;
  typedef typename M::vec8 V8;
  constexpr bool kBF = std::is_same<T, BF16>::value;
  constexpr int NT = D / 16;   // k steps of 32 over a page's 2 D summary values
  const int sk = blockIdx.x, s = sk / Hkv, kvh = sk - s * Hkv;
  const int L = clamp_len_q(lens[s], mbs);
  const int nb = (L + kBS - 1) / kBS;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int p0 = (blockIdx.y * kBoundWaves + wave) * 16 * kBoundGroups;
  if (nb <= budget || p0 >= nb) return;   // every page kept, or past the end (no barriers below)
  const int G = Hq / Hkv;
  const int col = lane & 15, kq = lane >> 4;
  // pages first: their loads are the long wait; B operand of step t:
  // elements 32 t + 8 kq .. +7 of page p0 + 16 g + col
  uint4 x[kBoundGroups][NT];
#pragma unroll
  for (int g = 0; g < kBoundGroups; ++g) {
    const int lb = min(p0 + 16 * g + col, nb - 1);
    const int pb = table_pb(bt, mbs, s, lb, num_blocks);
    const uint4* page = reinterpret_cast<const uint4*>(summ + ((size_t)pb * Hkv + kvh) * 2 * D);
#pragma unroll
    for (int t = 0; t < NT; ++t) x[g][t] = page[4 * t + kq];
  }
  // A operand of step t: elements k = 32 t + 8 kq .. +7 of row col
  const uint4* qrow = reinterpret_cast<const uint4*>(query + ((size_t)s * Hq + kvh * G + min(col, G - 1)) * D);
  uint4 qa[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int k0 = 32 * t + 8 * kq;   // k0 < D for every lane of a step, or for none
    const uint4 w = qrow[(k0 % D) / 8];
    uint32_t ww[4] = {w.x, w.y, w.z, w.w}, pa[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t m = sign_halves(ww[e]);
      pa[e] = (32 * t < D) ? (ww[e] & m) : (ww[e] & ~m);
    }
    qa[t] = make_uint4(pa[0], pa[1], pa[2], pa[3]);
  }
  auto absv = [](const uint4& v) {
    return make_uint4(v.x & 0x7fff7fffu, v.y & 0x7fff7fffu, v.z & 0x7fff7fffu, v.w & 0x7fff7fffu);
  };
  // f16: sum |q| per head (rows 4 kq + i of a ones column)
  floatx4 qn = {0.f, 0.f, 0.f, 0.f};
  if constexpr (!kBF) {
    const uint4 ones = make_uint4(0x3c003c00u, 0x3c003c00u, 0x3c003c00u, 0x3c003c00u);
#pragma unroll
    for (int t = 0; t < NT; ++t)
      qn = M::qk(__builtin_bit_cast(V8, absv(qa[t])), __builtin_bit_cast(V8, ones), qn);
  }
#pragma unroll
  for (int g = 0; g < kBoundGroups; ++g) {
    const int pg = p0 + 16 * g;
    if (pg >= nb) break;
    floatx4 acc = {0.f, 0.f, 0.f, 0.f}, aab = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      acc = M::qk(__builtin_bit_cast(V8, qa[t]), __builtin_bit_cast(V8, x[g][t]), acc);
      aab = M::qk(__builtin_bit_cast(V8, absv(qa[t])), __builtin_bit_cast(V8, absv(x[g][t])), aab);
    }
    // lane: page col, heads 4 kq .. +3
    float lo = -INFINITY, hi = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float b = fmaf(qn[i], 0x1p-13f, fmaf(aab[i], 0x1p-13f, 0x1p-99f));   // qn = 0 for bf16
      float l = acc[i] - b, h = acc[i] + b;
      if (!(b <= 3.0e38f) || acc[i] != acc[i]) {
        l = -INFINITY;
        h = INFINITY;
      }
      lo = fmaxf(lo, l);
      hi = fmaxf(hi, h);
    }
    lo = fmaxf(lo, __shfl_xor(lo, 16, 64));
    hi = fmaxf(hi, __shfl_xor(hi, 16, 64));
    lo = fmaxf(lo, __shfl_xor(lo, 32, 64));
    hi = fmaxf(hi, __shfl_xor(hi, 32, 64));
    if (lane < 16 && pg + lane < nb)
      bounds[(size_t)sk * mbs + pg + lane] = make_uint2(order_key32(lo), order_key32(hi));
  }
}

constexpr int kPairMax = 256;   // open pages ranked pairwise; more take a radix select
constexpr int kPickBin = 8;     // keys a threshold's bin may keep before the digits stop

// grid (S * Hkv), kPickThreads threads (512, or 1024 for tables wider than
// kPickWide): the budget pages of the largest exact scores from the bounds.
// theta, at most the budget-th largest lower bound, and ucut, at least the
// (budget + 1)-th largest upper bound, are narrowed down together one radix
// digit at a time (from the highest bit where two bounds differ) until the
// bin holding each has at most kPickBin keys: theta is the lower edge of its
// bin, ucut the upper edge of its.  At least budget pages have lower bounds
// >= theta, so a page whose upper bound is below theta is not among the
// budget best; at most budget pages have upper bounds > ucut, so a page
// whose lower bound is above ucut is (at most budget - 1 others can reach
// its score).  The others ("open" pages) get their exact fp64 score, as the
// scoring kernel computes it, and the budget - (sure pages) largest of those
// are kept, equal scores to the lower page; all written in page order.  A
// query the bounds do not hold for (a denormal element, or for bf16 one
// above 2^18) opens every page.
//
// Wave w owns pages [w * per, (w + 1) * per), lane l of it pages w * per + l
// + 64 j for j < per / 64 <= JMAX; the sweeps are unrolled to JMAX with
// their loads unconditional (clamped), so that they issue together.
// LDS: [mbs] 8-byte words: the bounds of every page, then the open pages'
// physical blocks and then their exact keys (by rank in page order), then
// the kept pages in page order (16-bit); [mbs] 16-bit open pages (bit 15
// set once a page is chosen).
template <typename T, int D, int GP, int kPickThreads>
__global__ __launch_bounds__(kPickThreads) __attribute__((amdgpu_waves_per_eu(4))) void quest_pick_kernel(
    const uint16_t* __restrict__ query, const uint16_t* __restrict__ summ, const int32_t* __restrict__ bt, int mbs,
    const int32_t* __restrict__ lens, int num_blocks, int Hq, int Hkv, int budget, const uint2* __restrict__ bounds,
    int32_t* __restrict__ selected) {
  constexpr int W = kPickThreads / 64;
  constexpr int JMAX = (kPickThreads == 512 ? kPickWide : kPickMaxPages) / kPickThreads;
  constexpr bool kBF = std::is_same<T, BF16>::value;
  extern __shared__ uint64_t pk_lds[];
  __shared__ int hist[2][kBins];
  __shared__ int pick[6];
  __shared__ int tmp[W];
  __shared__ int cnt[2][W];
  __shared__ uint64_t tmp64[W];
  __shared__ __attribute__((aligned(16))) float qs[GP * D];   // query group (padded heads repeat the last), exact
  uint2* kb = reinterpret_cast<uint2*>(pk_lds);
  uint64_t* kex = pk_lds;
  uint16_t* kept = reinterpret_cast<uint16_t*>(pk_lds);
  uint16_t* open = reinterpret_cast<uint16_t*>(pk_lds + mbs);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int sk = blockIdx.x, s = sk / Hkv, kvh = sk - s * Hkv;
  const int L = clamp_len_q(lens[s], mbs);
  const int nb = (L + kBS - 1) / kBS;
  const int G = Hq / Hkv;
  int2* out = reinterpret_cast<int2*>(selected) + (size_t)sk * budget;
  if (nb <= budget) {
    for (int i = tid; i < nb; i += kPickThreads) out[i] = make_int2(table_pb(bt, mbs, s, i, num_blocks), i);
    return;
  }
  const int nj = (nb + 64 * W - 1) / (64 * W);   // pages per lane (at most JMAX)
  const int r0 = wave * nj * 64 + lane;           // the lane's first page
  auto page_of = [&](int j) { return r0 + 64 * j; };
  const uint2* bg = bounds + (size_t)sk * mbs;
  const uint32_t k0 = bg[0].x;
  uint32_t dif = 0;
  {
    uint2 v[JMAX];
#pragma unroll
    for (int j = 0; j < JMAX; ++j)
      if (j < nj) v[j] = bg[min(page_of(j), nb - 1)];
#pragma unroll
    for (int j = 0; j < JMAX; ++j)
      if (j < nj) {
        dif |= (v[j].x ^ k0) | (v[j].y ^ k0);   // a clamped copy of page nb - 1 changes nothing
        if (page_of(j) < nb) kb[page_of(j)] = v[j];
      }
  }
  for (int b = tid; b < 2 * kBins; b += kPickThreads) hist[b / kBins][b % kBins] = 0;
  // the query group to LDS, and the elements the bounds assume
  bool odd = false;
  for (int i = tid; i < GP * D; i += kPickThreads) {
    const int h = i / D;
    const uint16_t raw = query[((size_t)s * Hq + kvh * G + min(h, G - 1)) * D + (i - h * D)];
    qs[i] = cvt16<T>(raw);
    const uint32_t v = raw & 0x7fffu;
    odd |= kBF ? ((v != 0 && v < 0x0080u) || v > ((127u + 18u) << 7 | 0x7fu)) : (v != 0 && v < 0x0400u);
  }
  // one reduction: the bits where bounds differ, and bit 32 for the query
  const uint64_t both = block_or<kPickThreads, uint64_t>((uint64_t)dif | ((uint64_t)odd << 32), tmp64);
  dif = (uint32_t)both;
  const bool all_open = (both >> 32) != 0;
  // theta's bin (pl, m) and ucut's bin (pu, m), narrowed in step
  int top = dif ? 32 - __clz((int)dif) : 0;
  uint32_t m = top >= 32 ? 0u : (~0u << top);
  uint32_t pl = k0 & m, pu = k0 & m;
  int rl = budget, ru = budget + 1;   // ranks still to place inside the bins
  // the bins are zero here (cleared above, then as each pass reads them)
  while (top > 0) {
    const int bits = top < kDigitBits ? top : kDigitBits, shift = top - bits;
    const uint32_t dmask = (1u << bits) - 1u;
    {
      uint2 v[JMAX];
#pragma unroll
      for (int j = 0; j < JMAX; ++j)
        if (j < nj) v[j] = kb[min(page_of(j), nb - 1)];
#pragma unroll
      for (int j = 0; j < JMAX; ++j)
        if (j < nj && page_of(j) < nb) {
          if ((v[j].x & m) == pl) atomicAdd(&hist[0][(v[j].x >> shift) & dmask], 1);
          if ((v[j].y & m) == pu) atomicAdd(&hist[1][(v[j].y >> shift) & dmask], 1);
        }
    }
    __syncthreads();
    // thread t holds digits kBins-1 - BPT t .. -(BPT-1), largest first; both
    // counts in one word (each at most nb < 2^16)
    constexpr int BPT = kBins / kPickThreads;
    int c0[BPT], c1[BPT], sum = 0;
#pragma unroll
    for (int u = 0; u < BPT; ++u) {
      const int d = kBins - 1 - (tid * BPT + u);
      c0[u] = hist[0][d];
      c1[u] = hist[1][d];
      hist[0][d] = 0;
      hist[1][d] = 0;
      sum += c0[u] + (c1[u] << 16);
    }
    const int incl = wave_incl_scan(sum);
    if (lane == 63) tmp[wave] = incl;
    __syncthreads();
    int above = incl - sum;
#pragma unroll
    for (int w = 0; w < W; ++w) above += w < wave ? tmp[w] : 0;
    int a0 = above & 0xffff, a1 = above >> 16;
#pragma unroll
    for (int u = 0; u < BPT; ++u) {
      const int d = kBins - 1 - (tid * BPT + u);
      if (a0 < rl && a0 + c0[u] >= rl) {
        pick[0] = d;
        pick[1] = rl - a0;
        pick[2] = c0[u];
      }
      if (a1 < ru && a1 + c1[u] >= ru) {
        pick[3] = d;
        pick[4] = ru - a1;
        pick[5] = c1[u];
      }
      a0 += c0[u];
      a1 += c1[u];
    }
    __syncthreads();
    pl |= (uint32_t)pick[0] << shift;
    pu |= (uint32_t)pick[3] << shift;
    m |= dmask << shift;
    rl = pick[1];
    ru = pick[4];
    top = shift;
    if (pick[2] <= kPickBin && pick[5] <= kPickBin) break;
    // pick[] is rewritten only after the next pass's first barrier
  }
  uint32_t theta = pl, ucut = pu | ~m;
  if (all_open) {
    theta = 0u;
    ucut = ~0u;
  }
  // bit j of sure / opn: page_of(j)
  uint32_t sure = 0, opn = 0;
  {
    uint2 v[JMAX];
#pragma unroll
    for (int j = 0; j < JMAX; ++j)
      if (j < nj) v[j] = kb[min(page_of(j), nb - 1)];
#pragma unroll
    for (int j = 0; j < JMAX; ++j)
      if (j < nj && page_of(j) < nb) {
        if (v[j].x > ucut) sure |= 1u << j;
        else if (v[j].y >= theta) opn |= 1u << j;
      }
  }
  const int n_sure = wave_sum(__popc(sure)), n_open = wave_sum(__popc(opn));
  if (lane == 0) {
    cnt[0][wave] = n_sure;
    cnt[1][wave] = n_open;
  }
  __syncthreads();
  int sure_all = 0, open_all = 0, open_before = 0;
#pragma unroll
  for (int w = 0; w < W; ++w) {
    open_before += w < wave ? cnt[1][w] : 0;
    sure_all += cnt[0][w];
    open_all += cnt[1][w];
  }
  {
    int o = open_before;
#pragma unroll
    for (int j = 0; j < JMAX; ++j) {
      if (j < nj) {
        const bool mine = (opn >> j) & 1u;
        const uint64_t bo = __ballot(mine);
        if (mine) open[o + lanes_below(bo)] = (uint16_t)page_of(j);
        o += __popcll(bo);
      }
    }
  }
  __syncthreads();   // the bounds are read; their words take the open pages' blocks
  for (int i = tid; i < open_all; i += kPickThreads) kex[i] = (uint64_t)table_pb(bt, mbs, s, open[i], num_blocks);
  __syncthreads();
  // exact scores of the open pages: kSplit lanes per (page, head), each a
  // kSplit-th of the dimensions, the loads issued first
  constexpr int kSplit = 4;
  for (int jj = tid; jj < open_all * GP * kSplit; jj += kPickThreads) {
    const int slot = jj / (kSplit * GP), h = (jj / kSplit) % GP, part = jj % kSplit;
    const int pb = (int)kex[slot];
    constexpr int C = D / (8 * kSplit);   // 8-dimension chunks of a part
    const uint4* pg = reinterpret_cast<const uint4*>(summ + ((size_t)pb * Hkv + kvh) * 2 * D) + part * C;
    uint4 mn[C], mx[C];
#pragma unroll
    for (int c = 0; c < C; ++c) {
      mn[c] = pg[c];
      mx[c] = pg[D / 8 + c];
    }
    const float4* qh = reinterpret_cast<const float4*>(qs + h * D + part * (8 * C));
    double acc0 = 0.0, acc1 = 0.0;
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const float4 q0 = qh[2 * c], q1 = qh[2 * c + 1];
      const float qv[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
      const uint32_t lo[4] = {mn[c].x, mn[c].y, mn[c].z, mn[c].w}, hi[4] = {mx[c].x, mx[c].y, mx[c].z, mx[c].w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const double q = (double)qv[e];
        acc0 = fma(q < 0.0 ? q : 0.0, cvt_d<T>(lo[e >> 1], e & 1), acc0);
        acc1 = fma(q > 0.0 ? q : 0.0, cvt_d<T>(hi[e >> 1], e & 1), acc1);
      }
      __builtin_amdgcn_sched_barrier(0);   // converted values stay chunk by chunk
    }
    double acc = acc0 + acc1;
#pragma unroll
    for (int o = 1; o < kSplit; o <<= 1) acc += __shfl_xor(acc, o, 64);
#pragma unroll
    for (int o = kSplit; o < kSplit * GP; o <<= 1) acc = fmax(acc, __shfl_xor(acc, o, 64));
    if ((jj & (kSplit * GP - 1)) == 0) kex[slot] = order_key(acc);
  }
  __syncthreads();
  // the `need` largest exact keys among the open pages, equal keys to the
  // lower slot (slots are in page order): bit 15 of open[slot]
  const int need = budget - sure_all;   // 0 <= need <= open_all
  if (open_all <= kPairMax) {
    if (tid < open_all) {
      const uint64_t kp = kex[tid];
      int rank = 0;
#pragma unroll 8
      for (int q = 0; q < open_all; ++q) {
        const uint64_t kq = kex[q];
        rank += (kq > kp) || (kq == kp && q < tid);
      }
      if (rank < need) open[tid] |= 0x8000u;
    }
  } else if (need > 0) {
    const int per_o = (open_all + 64 * W - 1) / (64 * W) * 64;
    uint64_t kp, km;
    int remaining;
    radix_select<kPickThreads, uint64_t>([&](int i) { return kex[i]; }, open_all, per_o, need, hist[0], tmp, tmp64,
                                         pick, kp, km, remaining);
    const int o0 = min(open_all, wave * per_o), o1 = min(open_all, o0 + per_o);
    int eq = 0;
    for (int i = o0 + lane; i < o1; i += 64) eq += (kex[i] & km) == kp;
    eq = wave_sum(eq);
    if (lane == 0) tmp[wave] = eq;
    __syncthreads();
    int eq_seen = 0;
    for (int w = 0; w < wave; ++w) eq_seen += tmp[w];
    for (int i0 = o0; i0 < o1; i0 += 64) {
      const int i = i0 + lane;
      const uint64_t key = kex[min(i, open_all - 1)] & km;
      const bool is_eq = i < o1 && key == kp;
      const uint64_t be = __ballot(is_eq);
      if (i < o1 && (key > kp || (is_eq && eq_seen + lanes_below(be) < remaining))) open[i] |= 0x8000u;
      eq_seen += __popcll(be);
    }
  }
  __syncthreads();
  // the kept pages in page order: the chosen open pages join the sure ones
  uint32_t sel = sure;
  {
    int o = open_before;
#pragma unroll
    for (int j = 0; j < JMAX; ++j) {
      if (j < nj) {
        const bool mine = (opn >> j) & 1u;
        const uint64_t bo = __ballot(mine);
        if (mine && (open[o + lanes_below(bo)] & 0x8000u)) sel |= 1u << j;
        o += __popcll(bo);
      }
    }
  }
  const int n_sel = wave_sum(__popc(sel));
  if (lane == 0) cnt[0][wave] = n_sel;
  __syncthreads();   // also: the exact keys are read, their words take the kept pages
  int pos = 0;
  for (int w = 0; w < wave; ++w) pos += cnt[0][w];
#pragma unroll
  for (int j = 0; j < JMAX; ++j) {
    if (j < nj) {
      const bool mine = (sel >> j) & 1u;
      const uint64_t bs = __ballot(mine);
      if (mine && pos + lanes_below(bs) < budget) kept[pos + lanes_below(bs)] = (uint16_t)page_of(j);
      pos += __popcll(bs);
    }
  }
  __syncthreads();
  for (int i = tid; i < budget; i += kPickThreads) {
    const int lb = kept[i];
    out[i] = make_int2(table_pb(bt, mbs, s, lb, num_blocks), lb);
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
  const int GP = padded_group(num_q_heads / num_kv_heads);
  const int mbs = max_blocks_per_seq;
  if (mbs <= kPickMaxPages) {
    // bounds on MFMA, then exact scores of the open pages only
    auto bounds = reinterpret_cast<uint2*>(scratch);
    const dim3 bgrid(num_seqs * num_kv_heads, (mbs + kBoundPages - 1) / kBoundPages);
#define PKV_BOUND(T, D)                                                                                       \
  quest_bound_kernel<T, D><<<bgrid, 64 * kBoundWaves, 0, st>>>(q, sm, block_tables, mbs, seq_lens, num_blocks, \
                                                               num_q_heads, num_kv_heads, budget, bounds)
    if (q_dtype == PKV_BF16) {
      if (head_dim == 64) PKV_BOUND(BF16, 64); else PKV_BOUND(BF16, 128);
    } else {
      if (head_dim == 64) PKV_BOUND(F16, 64); else PKV_BOUND(F16, 128);
    }
#undef PKV_BOUND
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const size_t lds = (size_t)mbs * 10 + 8;
    static std::atomic<bool> lds_set[2][2][5][2][64];
    const bool wide = mbs > kPickWide;
#define PKV_PICK_N(T, D, G, TI, DI, GI, NT, NI)                                                                  \
  do {                                                                                                          \
    e = set_lds_limit_once(reinterpret_cast<const void*>(quest_pick_kernel<T, D, G, NT>), kPickMaxPages * 10 + 8, \
                           lds_set[TI][DI][GI][NI]);                                                            \
    if (e != hipSuccess) return e;                                                                              \
    quest_pick_kernel<T, D, G, NT><<<num_seqs * num_kv_heads, NT, lds, st>>>(                                    \
        q, sm, block_tables, mbs, seq_lens, num_blocks, num_q_heads, num_kv_heads, budget, bounds, selected);   \
  } while (0)
#define PKV_PICK(T, D, G, TI, DI, GI)                        \
  do {                                                       \
    if (wide) PKV_PICK_N(T, D, G, TI, DI, GI, 1024, 1);      \
    else PKV_PICK_N(T, D, G, TI, DI, GI, 512, 0);            \
  } while (0)
#define PKV_PICK_G(T, D, TI, DI)                     \
  switch (GP) {                                      \
    case 1: PKV_PICK(T, D, 1, TI, DI, 0); break;     \
    case 2: PKV_PICK(T, D, 2, TI, DI, 1); break;     \
    case 4: PKV_PICK(T, D, 4, TI, DI, 2); break;     \
    case 8: PKV_PICK(T, D, 8, TI, DI, 3); break;     \
    default: PKV_PICK(T, D, 16, TI, DI, 4); break;   \
  }
    if (q_dtype == PKV_BF16) {
      if (head_dim == 64) PKV_PICK_G(BF16, 64, 0, 0) else PKV_PICK_G(BF16, 128, 0, 1)
    } else {
      if (head_dim == 64) PKV_PICK_G(F16, 64, 1, 0) else PKV_PICK_G(F16, 128, 1, 1)
    }
#undef PKV_PICK_G
#undef PKV_PICK
#undef PKV_PICK_N
    return hipGetLastError();
  }
  auto keys = reinterpret_cast<uint64_t*>(scratch);
  constexpr int kWgPages = kScorePages * kScoreWaves;
  const dim3 sgrid(num_seqs * num_kv_heads, (mbs + kWgPages - 1) / kWgPages);
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
  if (mbs <= kMaxLdsKeys) {
    static std::atomic<bool> lds_set[64];
    const hipError_t e2 =
        set_lds_limit_once(reinterpret_cast<const void*>(quest_select_kernel<true>), kMaxLdsKeys * 8, lds_set);
    if (e2 != hipSuccess) return e2;
    quest_select_kernel<true><<<grid, kSelThreads, (size_t)mbs * 8, st>>>(
        keys, block_tables, mbs, seq_lens, num_blocks, num_kv_heads, budget, selected);
  } else {
    quest_select_kernel<false><<<grid, kSelThreads, 0, st>>>(keys, block_tables, mbs, seq_lens, num_blocks,
                                                             num_kv_heads, budget, selected);
  }
  return hipGetLastError();
}

}  // namespace pkv
