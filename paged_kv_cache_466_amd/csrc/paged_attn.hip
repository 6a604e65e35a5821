// Paged decode attention for gfx950.
//
// One workgroup per (KV partition, KV head, sequence).  The workgroup walks
// the partition's physical blocks through the sequence's block table, in
// logical order ("Chapter 18", "How PagedAttention Works"; Learning-AI topic
// t13_4, block table; "KV Cache Engineering", section 10), computes the
// grouped query heads' scores against each block's keys (GQA, "KV Cache
// Engineering" section 1: the G = Hq/Hkv query heads of a group read the
// same KV head), keeps an online softmax, and accumulates P.V.  Partitions
// either write the final output (one partition per sequence) or fp32
// partials (m, l, acc) that a merge kernel combines by log-sum-exp.
//
// Two kernels:
//  * paged_attn_mfma_kernel - bf16 / f16 caches and INT8 / FP8-E4M3 codes
//    (converted to the query's 16-bit type in registers).  Per 16-token block
//    and wave: S^T = K Q^T on v_mfma_f32_16x16x32 (K rows go straight from
//    HBM into the A operand; the query group, padded to 16 heads, is the B
//    operand), then out^T += V^T P^T on v_mfma_f32_16x16x16 where the score
//    tile is already in the B-operand layout and V^T is read from an LDS
//    copy of the block with ds_read_b64_tr_b16.
//  * paged_attn_simple_kernel - fp32 caches (and any group size): scores in
//    LDS, plain fp32 FMAs.  Exact fp32 arithmetic, for the fp32 path.
//
// Scores are kept in the log2 domain: s2 = (q.k) * sm_scale * log2(e), so
// exp(s - m) = exp2(s2 - m2).
#include <hip/hip_runtime.h>

#include <type_traits>

#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {

constexpr int kBS = 16;                     // tokens per block
constexpr float kLog2e = 1.4426950408889634f;

struct AttnParams {
  void* out;
  const void* query;
  const void* k_cache;
  const void* v_cache;
  const float* k_scales;
  const float* v_scales;
  const int32_t* block_tables;
  const int32_t* seq_lens;
  float* ws_m;
  float* ws_l;
  float* ws_acc;
  int mbs, num_q_heads, num_kv_heads, num_blocks;
  int partition_size, num_partitions;
  int sink, window;
  float scale_log2;   // sm_scale * log2(e)
};

__device__ __forceinline__ int clamp_len(int L, int mbs) {
  const int cap = mbs * kBS;
  return L < 0 ? 0 : (L > cap ? cap : L);
}

// Is logical token t taken into attention for a sequence of length L?
__device__ __forceinline__ bool kept(int t, int L, int sink, int window) {
  if (t >= L) return false;
  if (sink == 0 && window == 0) return true;
  return t < sink || t >= L - window;
}

// Does block lb (tokens 16lb .. 16lb+15) hold at least one kept token?
__device__ __forceinline__ bool block_needed(int lb, int L, int sink, int window) {
  const int t0 = lb * kBS;
  if (t0 >= L) return false;
  if (sink == 0 && window == 0) return true;
  return t0 < sink || t0 + kBS - 1 >= L - window;
}

__device__ __forceinline__ int table_entry(const AttnParams& p, int s, int lb) {
  int pb = p.block_tables[(size_t)s * p.mbs + lb];
  // a bad table must not make the kernel leave the cache arrays
  return (pb < 0 || pb >= p.num_blocks) ? 0 : pb;
}

// ===========================================================================
// MFMA kernel
// ===========================================================================

// 16-bit MFMA element type of the query (bf16 or f16) and the converted KV.
template <typename QT> struct Mfma;
template <> struct Mfma<BF16> {
  typedef bf16x8 vec8;
  __device__ static floatx4 qk(const vec8& a, const vec8& b, const floatx4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  __device__ static floatx4 pv(const shortx4& a, const shortx4& b, const floatx4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
  }
  __device__ static uint32_t pack2(float x, float y) {
    return (uint32_t)f32_to_bf16(x) | ((uint32_t)f32_to_bf16(y) << 16);
  }
  __device__ static shortx4 tr_read(const void* lds) {
    bf16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
        (__attribute__((address_space(3))) bf16x4*)(lds));
    return __builtin_bit_cast(shortx4, v);
  }
};
template <> struct Mfma<F16> {
  typedef f16x8 vec8;
  __device__ static floatx4 qk(const vec8& a, const vec8& b, const floatx4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
  __device__ static floatx4 pv(const shortx4& a, const shortx4& b, const floatx4& c) {
    typedef _Float16 h4 __attribute__((ext_vector_type(4)));
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(h4, a), __builtin_bit_cast(h4, b), c, 0,
                                                 0, 0);
  }
  __device__ static uint32_t pack2(float x, float y) {
    return (uint32_t)f32_to_f16(x) | ((uint32_t)f32_to_f16(y) << 16);
  }
  __device__ static shortx4 tr_read(const void* lds) {
    fp16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4f16((__attribute__((address_space(3))) fp16x4*)(lds));
    return __builtin_bit_cast(shortx4, v);
  }
};

template <typename QT>
__device__ __forceinline__ uint32_t pack_q(float a, float b) { return Mfma<QT>::pack2(a, b); }

// 8 codes -> 8 elements of the query's 16-bit type, exactly (every INT8 and
// FP8-E4M3 value is a bf16 and an f16 value).
template <typename QT, typename KVT>
__device__ __forceinline__ uint4 to16(const uint2& c) {
  float f[8];
  if constexpr (std::is_same<KVT, I8>::value) {
    const uint32_t w[2] = {c.x, c.y};
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int b = 0; b < 4; ++b) f[4 * i + b] = (float)(int8_t)((w[i] >> (8 * b)) & 0xFF);
  } else {
    const uint32_t w[2] = {c.x, c.y};
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      floatx2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(w[i], false);
      floatx2 hi = __builtin_amdgcn_cvt_pk_f32_fp8(w[i], true);
      f[4 * i] = lo[0]; f[4 * i + 1] = lo[1]; f[4 * i + 2] = hi[0]; f[4 * i + 3] = hi[1];
    }
  }
  return make_uint4(pack_q<QT>(f[0], f[1]), pack_q<QT>(f[2], f[3]), pack_q<QT>(f[4], f[5]),
                    pack_q<QT>(f[6], f[7]));
}

// d-offset (elements) of the 8-element k-chunk that lane group `kg` feeds to
// MFMA number `c` of the q.K product.  Any assignment works as long as K and
// Q use the same one; it is chosen so that each load instruction reads long
// contiguous runs: 16-bit rows read 64 contiguous bytes per row per
// instruction, 8-bit rows let one lane read 32 contiguous bytes.
template <typename KVT, int D>
__device__ __forceinline__ int qk_doff(int c, int kg) {
  if constexpr (KVT::bytes == 2) return 32 * c + 8 * kg;
  else return (D / 4) * kg + 8 * c;
}

template <typename QT, typename KVT, int D, int WAVES>
__global__ __launch_bounds__(64 * WAVES) void paged_attn_mfma_kernel(AttnParams p) {
  constexpr int NC = D / 32;                 // q.K MFMAs per block (k = 32)
  constexpr int NN = D / 16;                 // P.V MFMAs per block (n = 16)
  constexpr int VROW = D * 2 + 16;           // LDS bytes per staged V row (16-bit, padded)
  constexpr int ACC_STRIDE = D + 4;          // floats per head row of the merge buffer
  constexpr int WAVE_LDS = 16 * ACC_STRIDE * 4;
  static_assert(kBS * VROW <= WAVE_LDS, "V staging must fit the per-wave region");
  constexpr bool kCodes = KVT::bytes == 1;
  constexpr int KCH = kCodes ? NC / 2 : NC;            // 16-byte K loads per lane per block
  constexpr int ROW_BYTES = D * KVT::bytes;
  constexpr int LANES_PER_ROW = ROW_BYTES / 16;
  constexpr int ROWS_PER_PASS = 64 / LANES_PER_ROW;
  constexpr int VCH = kBS / ROWS_PER_PASS;             // 16-byte V loads per lane per block
  // Scores may exceed the running max by this much (log2 units) before the
  // accumulators are rescaled: probabilities stay below 2^8.
  constexpr float kSlack = 8.0f;
  typedef Mfma<QT> M;

  __shared__ __attribute__((aligned(16))) uint8_t lds[WAVES * WAVE_LDS + WAVES * 16 * 2 * 4];
  // kvh fastest: the KV heads of one block are dispatched together, so the
  // block's 16 x Hkv x D rows are read from HBM close together in time.
  const int kvh = blockIdx.x, part = blockIdx.y, s = blockIdx.z;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int G = p.num_q_heads / p.num_kv_heads;
  const int L = clamp_len(p.seq_lens[s], p.mbs);
  const bool single = p.num_partitions == 1;
  const int t_begin = part * p.partition_size;
  const bool windowed = p.sink != 0 || p.window != 0;

  if (t_begin >= L) {
    if (single && part == 0) {
      // empty sequence: zeros
      for (int i = threadIdx.x; i < G * D; i += 64 * WAVES)
        store_out<QT>(p.out, ((size_t)s * p.num_q_heads + kvh * G) * D + i, 0.f);
    }
    return;
  }
  const int t_end = min(t_begin + p.partition_size, L);
  const int lb_begin = t_begin / kBS, lb_end = (t_end + kBS - 1) / kBS;

  const int g = lane & 15;       // query head in the group (column of S^T / out^T)
  const int kg = lane >> 4;      // lane group: k-chunk of the operands, 4-row slab of outputs

  // ---- query group as the B operand of S^T = K Q^T (zero rows for g >= G) --
  typename M::vec8 qop[NC];
  {
    const size_t qrow = ((size_t)s * p.num_q_heads + kvh * G + g) * D;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      uint4 w = make_uint4(0, 0, 0, 0);
      if (g < G) w = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(p.query) + qrow +
                                                    qk_doff<KVT, D>(c, kg));
      qop[c] = __builtin_bit_cast(typename M::vec8, w);
    }
  }

  // ---- this wave's blocks: lb = first + j * WAVES, j < nwb ------------------
  const int first = lb_begin + wave;
  const int nwb = first < lb_end ? (lb_end - first + WAVES - 1) / WAVES : 0;
  // lane i holds the table entry of wave block (chunk * 64 + i)
  int chunk = 0;
  int pbv = lane < nwb ? table_entry(p, s, first + lane * WAVES) : 0;

  auto block_needed_j = [&](int j) { return block_needed(first + j * WAVES, L, p.sink, p.window); };
  auto next_needed = [&](int j) {
    while (j < nwb && !block_needed_j(j)) ++j;
    return j;
  };
  auto entry = [&](int j) {
    if ((j >> 6) != chunk) {               // wave-uniform; once per 64 blocks
      chunk = j >> 6;
      const int jj = chunk * 64 + lane;
      pbv = jj < nwb ? table_entry(p, s, first + jj * WAVES) : 0;
    }
    return __builtin_amdgcn_readlane(pbv, j & 63);
  };

  struct Tile {
    uint4 k[KCH];
    uint4 v[VCH];
    int pb;
    float ks, vs;
  };
  const size_t row_elems = (size_t)p.num_kv_heads * D;   // elements between token rows
  auto load_tile = [&](Tile& t, int j) {
    const int pb = entry(j);
    t.pb = pb;
    const size_t tile = ((size_t)pb * kBS * p.num_kv_heads + kvh) * D;   // element offset of row 0
    const uint8_t* kbase = reinterpret_cast<const uint8_t*>(p.k_cache) +
                           (tile + (size_t)(lane & 15) * row_elems) * KVT::bytes;
    if constexpr (!kCodes) {
#pragma unroll
      for (int c = 0; c < NC; ++c) t.k[c] = *reinterpret_cast<const uint4*>(kbase + qk_doff<KVT, D>(c, kg) * 2);
    } else {
#pragma unroll
      for (int c2 = 0; c2 < KCH; ++c2) t.k[c2] = *reinterpret_cast<const uint4*>(kbase + (D / 4) * kg + 16 * c2);
    }
    const uint8_t* vbase = reinterpret_cast<const uint8_t*>(p.v_cache) + tile * KVT::bytes;
#pragma unroll
    for (int pass = 0; pass < VCH; ++pass) {
      const int r = pass * ROWS_PER_PASS + lane / LANES_PER_ROW;
      t.v[pass] = *reinterpret_cast<const uint4*>(vbase + (size_t)r * row_elems * KVT::bytes +
                                                  (lane % LANES_PER_ROW) * 16);
    }
    if constexpr (kCodes) {
      t.ks = p.k_scales[(size_t)pb * p.num_kv_heads + kvh];
      t.vs = p.v_scales[(size_t)pb * p.num_kv_heads + kvh];
    } else {
      t.ks = t.vs = 1.f;
    }
  };

  float m2 = -INFINITY;          // running max (log2 domain) of head g, same in all lane groups
  float lsum = 0.f;              // this lane's share of the softmax denominator
  floatx4 acc[NN];
#pragma unroll
  for (int n = 0; n < NN; ++n) acc[n] = floatx4{0.f, 0.f, 0.f, 0.f};
  uint8_t* vstage = lds + wave * WAVE_LDS;

  auto process = [&](const Tile& t, int j) {
    const int lb = first + j * WAVES;
    const int t0 = lb * kBS;
    // every token of the block is kept: no masking work
    const bool full = t0 + kBS <= L && (!windowed || t0 + kBS <= p.sink || t0 >= L - p.window);

    // ---- V rows -> LDS (masked rows as zeros: 0 * NaN must not reach acc) --
#pragma unroll
    for (int pass = 0; pass < VCH; ++pass) {
      const int r = pass * ROWS_PER_PASS + lane / LANES_PER_ROW;
      const int cchunk = lane % LANES_PER_ROW;
      uint4 w = t.v[pass];
      if constexpr (!kCodes) {
        if (!full && !kept(t0 + r, L, p.sink, p.window)) w = make_uint4(0, 0, 0, 0);
        *reinterpret_cast<uint4*>(vstage + r * VROW + cchunk * 16) = w;
      } else {
        uint4 lo = to16<QT, KVT>(make_uint2(w.x, w.y));
        uint4 hi = to16<QT, KVT>(make_uint2(w.z, w.w));
        if (!full && !kept(t0 + r, L, p.sink, p.window)) lo = hi = make_uint4(0, 0, 0, 0);
        *reinterpret_cast<uint4*>(vstage + r * VROW + cchunk * 32) = lo;
        *reinterpret_cast<uint4*>(vstage + r * VROW + cchunk * 32 + 16) = hi;
      }
    }

    // ---- S^T = K Q^T --------------------------------------------------------
    floatx4 sacc = floatx4{0.f, 0.f, 0.f, 0.f};
    if constexpr (!kCodes) {
#pragma unroll
      for (int c = 0; c < NC; ++c) sacc = M::qk(__builtin_bit_cast(typename M::vec8, t.k[c]), qop[c], sacc);
    } else {
#pragma unroll
      for (int c2 = 0; c2 < KCH; ++c2) {
        const uint4 lo = to16<QT, KVT>(make_uint2(t.k[c2].x, t.k[c2].y));
        const uint4 hi = to16<QT, KVT>(make_uint2(t.k[c2].z, t.k[c2].w));
        sacc = M::qk(__builtin_bit_cast(typename M::vec8, lo), qop[2 * c2], sacc);
        sacc = M::qk(__builtin_bit_cast(typename M::vec8, hi), qop[2 * c2 + 1], sacc);
      }
    }
    const float factor = p.scale_log2 * t.ks;
    // lane holds tokens 4*kg + i of this block for head g
    float sc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) sc[i] = sacc[i] * factor;
    if (!full) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (!kept(t0 + 4 * kg + i, L, p.sink, p.window)) sc[i] = -INFINITY;
    }
    const float lm = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
    // ---- online softmax, rescaling only when a score passes m2 + slack -----
    if (__ballot(lm > m2 + kSlack)) {
      float bmax = fmaxf(lm, __shfl_xor(lm, 16, 64));
      bmax = fmaxf(bmax, __shfl_xor(bmax, 32, 64));
      const float mnew = fmaxf(m2, bmax);
      const float alpha = __builtin_amdgcn_exp2f(m2 - mnew);   // 0 while m2 = -inf
      lsum *= alpha;
#pragma unroll
      for (int n = 0; n < NN; ++n) acc[n] *= alpha;
      m2 = mnew;
    }
    float pr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      pr[i] = __builtin_amdgcn_exp2f(sc[i] - m2);
      lsum += pr[i];
    }
    // P^T as the B operand (tokens 4kg..4kg+3 of head g), V scale folded in
    const uint32_t p01 = M::pack2(pr[0] * t.vs, pr[1] * t.vs);
    const uint32_t p23 = M::pack2(pr[2] * t.vs, pr[3] * t.vs);
    const shortx4 pop = __builtin_bit_cast(shortx4, make_uint2(p01, p23));

    // ---- out^T += V^T P^T: V^T chunks through the transposing LDS read ----
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    {
      // lane i of each 16-lane group reads row 4kg + i/4, columns 4(i%4)..+3
      const uint8_t* rd = vstage + (4 * kg + (g >> 2)) * VROW + (g & 3) * 8;
#pragma unroll
      for (int n = 0; n < NN; ++n) {
        const shortx4 vop = M::tr_read(rd + n * 32);
        acc[n] = M::pv(vop, pop, acc[n]);
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };

  // ---- main loop: block j+1's loads are in flight while block j computes --
  {
    Tile ta, tb;
    int j = next_needed(0);
    if (j < nwb) load_tile(ta, j);
    while (j < nwb) {
      int jn = next_needed(j + 1);
      if (jn < nwb) load_tile(tb, jn);
      process(ta, j);
      j = jn;
      if (j >= nwb) break;
      jn = next_needed(j + 1);
      if (jn < nwb) load_tile(ta, jn);
      process(tb, j);
      j = jn;
    }
  }

  // ---- this wave's softmax state -> LDS; combine the waves -----------------
  lsum += __shfl_xor(lsum, 16, 64);
  lsum += __shfl_xor(lsum, 32, 64);
  float* accbuf = reinterpret_cast<float*>(lds + wave * WAVE_LDS);
  float* mlbuf = reinterpret_cast<float*>(lds + WAVES * WAVE_LDS);
  __syncthreads();   // every wave is done with its V staging area
#pragma unroll
  for (int n = 0; n < NN; ++n)
    *reinterpret_cast<floatx4*>(accbuf + g * ACC_STRIDE + 16 * n + 4 * kg) = acc[n];
  if (kg == 0) {
    mlbuf[(wave * 16 + g) * 2] = m2;
    mlbuf[(wave * 16 + g) * 2 + 1] = lsum;
  }
  __syncthreads();

  const size_t head0 = (size_t)s * p.num_q_heads + kvh * G;
  for (int i = threadIdx.x; i < G * D; i += 64 * WAVES) {
    const int gg = i / D, d = i % D;
    float Mx = -INFINITY;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) Mx = fmaxf(Mx, mlbuf[(w * 16 + gg) * 2]);
    float num = 0.f, den = 0.f;
    if (Mx != -INFINITY) {
#pragma unroll
      for (int w = 0; w < WAVES; ++w) {
        const float mw = mlbuf[(w * 16 + gg) * 2];
        if (mw == -INFINITY) continue;
        const float e = exp2f(mw - Mx);
        num += e * reinterpret_cast<float*>(lds + w * WAVE_LDS)[gg * ACC_STRIDE + d];
        den += e * mlbuf[(w * 16 + gg) * 2 + 1];
      }
    }
    if (single) {
      store_out<QT>(p.out, (head0 + gg) * D + d, den > 0.f ? num / den : 0.f);
    } else {
      const size_t pi = (head0 + gg) * p.num_partitions + part;
      p.ws_acc[pi * D + d] = num;
      if (d == 0) {
        p.ws_m[pi] = Mx;
        p.ws_l[pi] = den;
      }
    }
  }
}

// ===========================================================================
// Simple fp32 kernel: scores in LDS, fp32 FMAs, chunks of 256 tokens with an
// online softmax across chunks.  Any group size with G * D <= 2048.
// ===========================================================================
template <typename QT, typename KVT, int D>
__global__ __launch_bounds__(256) void paged_attn_simple_kernel(AttnParams p) {
  constexpr int CH = 256;
  constexpr int MAXG = 16;
  constexpr int MAXPAIRS = MAXG * D / 256;
  __shared__ float qs[MAXG * D];
  __shared__ float sc[MAXG * CH];
  __shared__ float mrow[MAXG], lrow[MAXG], arow[MAXG];
  const int kvh = blockIdx.x, part = blockIdx.y, s = blockIdx.z;
  const int tid = threadIdx.x;
  const int G = p.num_q_heads / p.num_kv_heads;
  const int L = clamp_len(p.seq_lens[s], p.mbs);
  const bool single = p.num_partitions == 1;
  const int t_begin = part * p.partition_size;
  const size_t head0 = (size_t)s * p.num_q_heads + kvh * G;
  if (t_begin >= L) {
    if (single && part == 0)
      for (int i = tid; i < G * D; i += 256) store_out<QT>(p.out, head0 * D + i, 0.f);
    return;
  }
  const int t_end = min(t_begin + p.partition_size, L);
  for (int i = tid; i < G * D; i += 256) qs[i] = load_elem<QT>(p.query, head0 * D + i);
  if (tid < G) {
    mrow[tid] = -INFINITY;
    lrow[tid] = 0.f;
  }
  float acc[MAXPAIRS];
#pragma unroll
  for (int k = 0; k < MAXPAIRS; ++k) acc[k] = 0.f;
  __syncthreads();

  const size_t row_elems = (size_t)p.num_kv_heads * D;
  for (int c0 = t_begin; c0 < t_end; c0 += CH) {
    // scores of this chunk
    {
      const int t = c0 + tid;
      if (t < t_end && kept(t, L, p.sink, p.window)) {
        const int pb = table_entry(p, s, t / kBS);
        const size_t row = ((size_t)pb * kBS + t % kBS) * row_elems + (size_t)kvh * D;
        float f = 1.f;
        if (KVT::bytes == 1) f = p.k_scales[(size_t)pb * p.num_kv_heads + kvh];
        for (int gg = 0; gg < G; ++gg) {
          float dot = 0.f;
          for (int d = 0; d < D; ++d) dot = fmaf(qs[gg * D + d], load_elem<KVT>(p.k_cache, row + d), dot);
          sc[gg * CH + tid] = dot * f * p.scale_log2;
        }
      } else {
        for (int gg = 0; gg < G; ++gg) sc[gg * CH + tid] = -INFINITY;
      }
    }
    __syncthreads();
    // chunk max, new running max, probabilities, chunk sum (one wave per head)
    {
      const int wv = tid >> 6, ln = tid & 63;
      for (int gg = wv; gg < G; gg += 4) {
        float mx = -INFINITY;
        for (int i = ln; i < CH; i += 64) mx = fmaxf(mx, sc[gg * CH + i]);
        mx = wave_max(mx);
        const float mold = mrow[gg];
        const float mnew = fmaxf(mold, mx);
        float sum = 0.f;
        for (int i = ln; i < CH; i += 64) {
          const float e = mnew == -INFINITY ? 0.f : exp2f(sc[gg * CH + i] - mnew);
          sc[gg * CH + i] = e;
          sum += e;
        }
        sum = wave_sum(sum);
        if (ln == 0) {
          const float a = mnew == -INFINITY ? 1.f : exp2f(mold - mnew);
          arow[gg] = a;
          lrow[gg] = lrow[gg] * a + sum;
          mrow[gg] = mnew;
        }
      }
    }
    __syncthreads();
    // P.V for the (head, dim) pairs this thread owns
#pragma unroll
    for (int k = 0; k < MAXPAIRS; ++k) {
      const int i = tid + 256 * k;
      if (i >= G * D) break;
      const int gg = i / D, d = i % D;
      float a = acc[k] * arow[gg];
      const int n = min(CH, t_end - c0);
      for (int j = 0; j < n; ++j) {
        const float pj = sc[gg * CH + j];
        if (pj == 0.f) continue;
        const int t = c0 + j;
        const int pb = table_entry(p, s, t / kBS);
        const size_t row = ((size_t)pb * kBS + t % kBS) * row_elems + (size_t)kvh * D;
        float v = load_elem<KVT>(p.v_cache, row + d);
        if (KVT::bytes == 1) v *= p.v_scales[(size_t)pb * p.num_kv_heads + kvh];
        a = fmaf(pj, v, a);
      }
      acc[k] = a;
    }
    __syncthreads();
  }
#pragma unroll
  for (int k = 0; k < MAXPAIRS; ++k) {
    const int i = tid + 256 * k;
    if (i >= G * D) break;
    const int gg = i / D, d = i % D;
    const float den = lrow[gg];
    if (single) {
      store_out<QT>(p.out, (head0 + gg) * D + d, den > 0.f ? acc[k] / den : 0.f);
    } else {
      const size_t pi = (head0 + gg) * p.num_partitions + part;
      p.ws_acc[pi * D + d] = acc[k];
      if (d == 0) {
        p.ws_m[pi] = mrow[gg];
        p.ws_l[pi] = den;
      }
    }
  }
}

// ===========================================================================
// Merge: out = sum_p 2^(m_p - M) acc_p / sum_p 2^(m_p - M) l_p
// One workgroup per (query head, sequence); 8 partition rows in flight, each
// read by D/4 threads with 16-byte loads.
// ===========================================================================
template <typename QT, int D>
__global__ __launch_bounds__(256) void paged_attn_merge_kernel(void* out, const int32_t* seq_lens,
                                                               const float* ws_m, const float* ws_l,
                                                               const float* ws_acc, int num_q_heads,
                                                               int num_partitions, int partition_size,
                                                               int max_len) {
  constexpr int TPR = D / 4;               // threads per partition row
  constexpr int ROWS = 256 / TPR;
  __shared__ float red[256];
  __shared__ floatx4 part_num[ROWS][TPR];
  __shared__ float part_den[ROWS];
  const int h = blockIdx.x, s = blockIdx.y;
  const int tid = threadIdx.x;
  int L = seq_lens[s];
  L = L < 0 ? 0 : (L > max_len ? max_len : L);
  const int np = (L + partition_size - 1) / partition_size;
  const size_t base = ((size_t)s * num_q_heads + h) * num_partitions;
  float mx = -INFINITY;
  for (int i = tid; i < np; i += 256) mx = fmaxf(mx, ws_m[base + i]);
  red[tid] = mx;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (tid < o) red[tid] = fmaxf(red[tid], red[tid + o]);
    __syncthreads();
  }
  const float M = red[0];
  const int row = tid / TPR, c = tid % TPR;
  floatx4 num = floatx4{0.f, 0.f, 0.f, 0.f};
  float den = 0.f;
  if (M != -INFINITY) {
    for (int i = row; i < np; i += ROWS) {
      const float mi = ws_m[base + i];
      if (mi == -INFINITY) continue;
      const float e = exp2f(mi - M);
      const floatx4 a = *reinterpret_cast<const floatx4*>(ws_acc + (base + i) * D + 4 * c);
      num += e * a;
      den += e * ws_l[base + i];
    }
  }
  part_num[row][c] = num;
  if (c == 0) part_den[row] = den;
  __syncthreads();
  if (tid < TPR) {
    floatx4 n = floatx4{0.f, 0.f, 0.f, 0.f};
    float dn = 0.f;
    for (int r = 0; r < ROWS; ++r) {
      n += part_num[r][tid];
      dn += part_den[r];
    }
    const size_t o = ((size_t)s * num_q_heads + h) * D + 4 * tid;
#pragma unroll
    for (int k = 0; k < 4; ++k) store_out<QT>(out, o + k, dn > 0.f ? n[k] / dn : 0.f);
  }
}

// ===========================================================================
// launchers
// ===========================================================================
static AttnParams make_params(const AttnArgs& a) {
  AttnParams p;
  p.out = a.out;
  p.query = a.query;
  p.k_cache = a.k_cache;
  p.v_cache = a.v_cache;
  p.k_scales = a.k_scales;
  p.v_scales = a.v_scales;
  p.block_tables = a.block_tables;
  p.seq_lens = a.seq_lens;
  p.ws_m = a.ws_m;
  p.ws_l = a.ws_l;
  p.ws_acc = a.ws_acc;
  p.mbs = a.max_blocks_per_seq;
  p.num_q_heads = a.num_q_heads;
  p.num_kv_heads = a.num_kv_heads;
  p.num_blocks = a.num_blocks;
  p.partition_size = a.partition_size;
  p.num_partitions = a.num_partitions;
  p.sink = a.sink_tokens;
  p.window = a.window_tokens;
  p.scale_log2 = a.sm_scale * kLog2e;
  return p;
}

constexpr int kWaves = 4;

template <typename QT, typename KVT, int D>
static int launch_mfma(const AttnParams& p, dim3 grid, hipStream_t st) {
  paged_attn_mfma_kernel<QT, KVT, D, kWaves><<<grid, 64 * kWaves, 0, st>>>(p);
  return hipGetLastError();
}

template <typename QT, typename KVT>
static int launch_mfma_d(const AttnParams& p, int D, dim3 grid, hipStream_t st) {
  return D == 64 ? launch_mfma<QT, KVT, 64>(p, grid, st) : launch_mfma<QT, KVT, 128>(p, grid, st);
}

template <typename QT, typename KVT, int D>
static int launch_simple(const AttnParams& p, dim3 grid, hipStream_t st) {
  paged_attn_simple_kernel<QT, KVT, D><<<grid, 256, 0, st>>>(p);
  return hipGetLastError();
}

int launch_paged_attn_partition(const AttnArgs& a) {
  const AttnParams p = make_params(a);
  const dim3 grid(a.num_kv_heads, a.num_partitions, a.num_seqs);
  hipStream_t st = (hipStream_t)a.stream;
  const int D = a.head_dim;
  if (a.num_seqs == 0) return hipSuccess;
  if (a.kv_dtype == PKV_F32) {
    return D == 64 ? launch_simple<F32, F32, 64>(p, grid, st) : launch_simple<F32, F32, 128>(p, grid, st);
  }
  if (a.q_dtype == PKV_BF16) {
    switch (a.kv_dtype) {
      case PKV_BF16: return launch_mfma_d<BF16, BF16>(p, D, grid, st);
      case PKV_I8: return launch_mfma_d<BF16, I8>(p, D, grid, st);
      default: return launch_mfma_d<BF16, FP8>(p, D, grid, st);
    }
  }
  switch (a.kv_dtype) {
    case PKV_F16: return launch_mfma_d<F16, F16>(p, D, grid, st);
    case PKV_I8: return launch_mfma_d<F16, I8>(p, D, grid, st);
    default: return launch_mfma_d<F16, FP8>(p, D, grid, st);
  }
}

int launch_paged_attn_merge(const AttnArgs& a) {
  if (a.num_partitions <= 1 || a.num_seqs == 0) return hipSuccess;
  const dim3 grid(a.num_q_heads, a.num_seqs);
  hipStream_t st = (hipStream_t)a.stream;
  const int max_len = a.max_blocks_per_seq * a.block_size;
#define PKV_MERGE(QT, D)                                                                               \
  paged_attn_merge_kernel<QT, D><<<grid, 256, 0, st>>>(a.out, a.seq_lens, a.ws_m, a.ws_l, a.ws_acc,    \
                                                      a.num_q_heads, a.num_partitions, a.partition_size, \
                                                      max_len)
  if (a.head_dim == 64) {
    if (a.q_dtype == PKV_F32) PKV_MERGE(F32, 64);
    else if (a.q_dtype == PKV_BF16) PKV_MERGE(BF16, 64);
    else PKV_MERGE(F16, 64);
  } else {
    if (a.q_dtype == PKV_F32) PKV_MERGE(F32, 128);
    else if (a.q_dtype == PKV_BF16) PKV_MERGE(BF16, 128);
    else PKV_MERGE(F16, 128);
  }
#undef PKV_MERGE
  return hipGetLastError();
}

}  // namespace pkv
