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
//    64-bit key.  16 lanes per page, 8 (or 4) dimensions per lane, 64
//    pages per workgroup.
//  * quest_select_kernel - per (sequence, KV head), the `budget` largest
//    keys by a 6-pass radix select (11-bit digits) over the keys held in LDS
//    (LDS histograms), ties to the lower page, written in logical order as
//    (physical block, logical block).
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

// x of the lane `o` places further along its row of 16 lanes (DPP row
// rotation), for a double.
__device__ __forceinline__ double row_ror(double x, int o) {
  const uint64_t b = __builtin_bit_cast(uint64_t, x);
  int lo = (int)(uint32_t)b, hi = (int)(uint32_t)(b >> 32);
  switch (o) {
    case 8:
      lo = __builtin_amdgcn_mov_dpp(lo, 0x128, 0xF, 0xF, false);
      hi = __builtin_amdgcn_mov_dpp(hi, 0x128, 0xF, 0xF, false);
      break;
    case 4:
      lo = __builtin_amdgcn_mov_dpp(lo, 0x124, 0xF, 0xF, false);
      hi = __builtin_amdgcn_mov_dpp(hi, 0x124, 0xF, 0xF, false);
      break;
    case 2:
      lo = __builtin_amdgcn_mov_dpp(lo, 0x122, 0xF, 0xF, false);
      hi = __builtin_amdgcn_mov_dpp(hi, 0x122, 0xF, 0xF, false);
      break;
    default:
      lo = __builtin_amdgcn_mov_dpp(lo, 0x121, 0xF, 0xF, false);
      hi = __builtin_amdgcn_mov_dpp(hi, 0x121, 0xF, 0xF, false);
      break;
  }
  return __builtin_bit_cast(double, ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo);
}

// Order-preserving map of a double onto uint64 (larger value, larger key).
__device__ __forceinline__ uint64_t order_key(double x) {
  const uint64_t b = __builtin_bit_cast(uint64_t, x);
  return (b >> 63) ? ~b : (b | (1ull << 63));
}

constexpr int kScorePagesPerGroup = 64;   // pages per scoring workgroup: 4 rounds of 16

// grid (S * Hkv, ceil(mbs / 64)), 256 threads: 16 lanes per page, 16 pages
// a round, 4 rounds.  The table entries of all rounds are requested
// together, then all summaries together with the query group.  With
// q+ = max(q, 0) and q- = min(q, 0), max(q * min, q * max) = q+ * max +
// q- * min (min <= max), so a head's score is two fp64 dot products; every
// product is exact, and the 16-lane sums of 4 heads are reduced together
// by DPP row rotations.
template <typename T, int D>
__global__ __launch_bounds__(256) void quest_score_kernel(const uint16_t* __restrict__ query,
                                                          const uint16_t* __restrict__ summ,
                                                          const int32_t* __restrict__ bt, int mbs,
                                                          const int32_t* __restrict__ lens, int num_blocks,
                                                          int Hq, int Hkv, uint64_t* __restrict__ keys) {
  constexpr int DPL = D / 16;   // dimensions per lane: 16 bytes of 16-bit values at D = 128
  constexpr int R = kScorePagesPerGroup / 16;
  typedef uint16_t u16xN __attribute__((ext_vector_type(DPL)));
  __shared__ float qp[16 * D], qn[16 * D];   // q+ and q- of the group's heads (exact)
  const int s = blockIdx.x / Hkv, kvh = blockIdx.x % Hkv;
  const int G = Hq / Hkv;
  const int L = clamp_len_q(lens[s], mbs);
  const int nb = (L + kBS - 1) / kBS;
  const int lb0 = blockIdx.y * kScorePagesPerGroup;
  if (lb0 >= nb) return;
  const int j = threadIdx.x & 15;
  int pb[R];
#pragma unroll
  for (int r = 0; r < R; ++r) pb[r] = table_pb(bt, mbs, s, min(lb0 + r * 16 + (int)threadIdx.x / 16, nb - 1), num_blocks);
  u16xN mn[R], mx[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const uint16_t* o = summ + ((size_t)pb[r] * Hkv + kvh) * 2 * D + j * DPL;
    mn[r] = *reinterpret_cast<const u16xN*>(o);
    mx[r] = *reinterpret_cast<const u16xN*>(o + D);
  }
  {
    // the group's G * D query values as 8-element pieces (index clamped)
    typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));
    constexpr int PPT = (16 * D / 8 + 255) / 256;   // pieces per thread
    const u16x8* q8 = reinterpret_cast<const u16x8*>(query + ((size_t)s * Hq + kvh * G) * D);
    u16x8 qv[PPT];
#pragma unroll
    for (int u = 0; u < PPT; ++u) qv[u] = q8[min(u * 256 + (int)threadIdx.x, G * D / 8 - 1)];
#pragma unroll
    for (int u = 0; u < PPT; ++u) {
      const int piece = u * 256 + threadIdx.x;
      if (piece < 16 * D / 8) {   // within the arrays (pieces past G * D repeat the last)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float x = cvt16<T>(qv[u][e]);
          qp[piece * 8 + e] = fmaxf(x, 0.f);
          qn[piece * 8 + e] = fminf(x, 0.f);
        }
      }
    }
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < R; ++r) {
    double lo[DPL], hi[DPL];
#pragma unroll
    for (int k = 0; k < DPL; ++k) {
      lo[k] = cvt16<T>(mn[r][k]);
      hi[k] = cvt16<T>(mx[r][k]);
    }
    double best = -INFINITY;
    for (int g0 = 0; g0 < G; g0 += 4) {
      double acc[4];
#pragma unroll
      for (int gg = 0; gg < 4; ++gg) {
        const int g = min(g0 + gg, G - 1);   // heads past G repeat the last one
        const float* a = qp + g * D + j * DPL;
        const float* b = qn + g * D + j * DPL;
        double t = 0.0;
#pragma unroll
        for (int k = 0; k < DPL; ++k) t = fma((double)a[k], hi[k], fma((double)b[k], lo[k], t));
        acc[gg] = t;
      }
      // sum over the page's 16 lanes: rotations within a row of 16 lanes
#pragma unroll
      for (int o = 8; o >= 1; o >>= 1) {
#pragma unroll
        for (int gg = 0; gg < 4; ++gg) acc[gg] += row_ror(acc[gg], o);
      }
#pragma unroll
      for (int gg = 0; gg < 4; ++gg) best = fmax(best, acc[gg]);
    }
    const int lb = lb0 + r * 16 + threadIdx.x / 16;
    if (lb < nb && j == 0) keys[((size_t)s * Hkv + kvh) * mbs + lb] = order_key(best);
  }
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

// grid (S * Hkv), kSelThreads threads.  IN_LDS: the keys of the (sequence,
// KV head) are first copied to LDS; otherwise every pass reads them from
// global memory.  Thread t owns the contiguous run of keys [t * per,
// (t + 1) * per).  Radix select of the budget-th largest key, 11 bits at a
// time from the top, with LDS histogram atomics; then every larger key is
// kept, and the first keys equal to it in page order until the budget is
// met.
template <bool IN_LDS>
__global__ __launch_bounds__(kSelThreads) void quest_select_kernel(const uint64_t* __restrict__ keys,
                                                                   const int32_t* __restrict__ bt, int mbs,
                                                                   const int32_t* __restrict__ lens,
                                                                   int num_blocks, int Hkv, int budget,
                                                                   int32_t* __restrict__ selected) {
  extern __shared__ uint64_t kl[];
  __shared__ int hist[kBins];
  __shared__ int pick[2];
  __shared__ int tmp[kSelThreads / 64];
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
  uint64_t prefix = 0, mask = 0;
  int remaining = budget;   // keys still to take at or below the current prefix
  for (int top = 64; top > 0; top -= kDigitBits) {
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
      }
      above += c[u];
    }
    __syncthreads();
    prefix |= (uint64_t)pick[0] << shift;
    mask |= (uint64_t)dmask << shift;
    remaining = pick[1];
    __syncthreads();
  }
  int eq = 0;
  for (int i = r0; i < r1; ++i) eq += key_at(i) == prefix;
  int unused;
  int eq_seen = block_scan(eq, tmp, &unused);
  int nsel = 0;
  for (int i = r0; i < r1; ++i) {
    const uint64_t key = key_at(i);
    if (key > prefix) ++nsel;
    else if (key == prefix) nsel += (eq_seen++ < remaining);
  }
  int pos = block_scan(nsel, tmp, &unused);
  eq_seen -= eq;
  for (int i = r0; i < r1; ++i) {
    const uint64_t key = key_at(i);
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
  const dim3 sgrid(num_seqs * num_kv_heads, (max_blocks_per_seq + kScorePagesPerGroup - 1) / kScorePagesPerGroup);
#define PKV_SCORE(T, D)                                                                                        \
  quest_score_kernel<T, D><<<sgrid, 256, 0, st>>>(q, sm, block_tables, max_blocks_per_seq, seq_lens, num_blocks, \
                                                 num_q_heads, num_kv_heads, keys)
  if (q_dtype == PKV_BF16) {
    if (head_dim == 64) PKV_SCORE(BF16, 64);
    else PKV_SCORE(BF16, 128);
  } else {
    if (head_dim == 64) PKV_SCORE(F16, 64);
    else PKV_SCORE(F16, 128);
  }
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
