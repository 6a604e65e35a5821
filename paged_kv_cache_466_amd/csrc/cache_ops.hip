// Cache-write kernels: slot mapping, the slot write (reshape_and_cache),
// whole-block copy-on-write, and absmax block quantisation.
//
// All four are memory-bound streams over short rows; each thread moves 16
// bytes per access so that a wave touches whole 64-byte segments.
#include <hip/hip_runtime.h>

#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {

// ---------------------------------------------------------------------------
// slot = table[s][p / bs] * bs + p % bs   (t13_4 block table; Chapter 18,
// "How PagedAttention Works")
// ---------------------------------------------------------------------------
__global__ void slot_mapping_kernel(int32_t* __restrict__ slots, const int32_t* __restrict__ tables,
                                    int mbs, const int32_t* __restrict__ seq_ids,
                                    const int32_t* __restrict__ positions, int num_tokens,
                                    int num_seqs, int bs, int num_blocks) {
  const int j = blockIdx.x * blockDim.x + threadIdx.x;
  if (j >= num_tokens) return;
  const int s = seq_ids ? seq_ids[j] : j;
  const int p = positions[j];
  int32_t slot = -1;
  if (s >= 0 && s < num_seqs && p >= 0) {
    const int lb = p / bs;
    if (lb < mbs) {
      const int32_t pb = tables[(size_t)s * mbs + lb];
      if (pb >= 0 && pb < num_blocks) slot = pb * bs + p % bs;
    }
  }
  slots[j] = slot;
}

int launch_slot_mapping(int32_t* slot_mapping, const int32_t* block_tables, int max_blocks_per_seq,
                        const int32_t* seq_ids, const int32_t* positions, int num_tokens, int num_seqs,
                        int block_size, int num_blocks, void* stream) {
  if (num_tokens == 0) return hipSuccess;
  const int threads = 256;
  const int grid = (num_tokens + threads - 1) / threads;
  slot_mapping_kernel<<<grid, threads, 0, (hipStream_t)stream>>>(
      slot_mapping, block_tables, max_blocks_per_seq, seq_ids, positions, num_tokens, num_seqs,
      block_size, num_blocks);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// reshape_and_cache: token j's [Hkv, D] row goes to cache row slot_mapping[j].
// A cache row for slot `slot` starts at slot * row_bytes because a block is
// [bs][Hkv][D] and blocks are consecutive.
// ---------------------------------------------------------------------------
__global__ void reshape_and_cache_kernel(const uint4* __restrict__ key, const uint4* __restrict__ value,
                                         uint4* __restrict__ kc, uint4* __restrict__ vc,
                                         const int32_t* __restrict__ slots, int num_tokens,
                                         int chunks_per_row, long long num_slots) {
  const long long total = (long long)num_tokens * chunks_per_row;
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (long long)gridDim.x * blockDim.x) {
    const int j = (int)(i / chunks_per_row);
    const int c = (int)(i - (long long)j * chunks_per_row);
    const long long slot = slots[j];
    if (slot < 0 || slot >= num_slots) continue;
    const long long dst = slot * chunks_per_row + c;
    kc[dst] = key[i];
    vc[dst] = value[i];
  }
}

int launch_reshape_and_cache(const void* key, const void* value, void* k_cache, void* v_cache,
                             int elem_bytes, const int32_t* slot_mapping, int num_tokens,
                             int num_blocks, int block_size, int num_kv_heads, int head_dim,
                             void* stream) {
  if (num_tokens == 0) return hipSuccess;
  const int chunks_per_row = num_kv_heads * head_dim * elem_bytes / 16;
  const long long total = (long long)num_tokens * chunks_per_row;
  const int threads = 256;
  long long grid = (total + threads - 1) / threads;
  if (grid > 65536) grid = 65536;
  reshape_and_cache_kernel<<<(int)grid, threads, 0, (hipStream_t)stream>>>(
      (const uint4*)key, (const uint4*)value, (uint4*)k_cache, (uint4*)v_cache, slot_mapping,
      num_tokens, chunks_per_row, (long long)num_blocks * block_size);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// append_kv: slot mapping and slot write in one pass.  Thread group of token
// j computes its slot from the table (as slot_mapping_kernel), optionally
// records it, and copies the token's K and V rows there.
// ---------------------------------------------------------------------------
__global__ void append_kv_kernel(const uint4* __restrict__ key, const uint4* __restrict__ value,
                                 uint4* __restrict__ kc, uint4* __restrict__ vc,
                                 const int32_t* __restrict__ tables, int mbs, const int32_t* __restrict__ seq_ids,
                                 const int32_t* __restrict__ positions, int32_t* __restrict__ slots_out,
                                 int num_tokens, int num_seqs, int bs, int num_blocks, int chunks_per_row) {
  const int j = blockIdx.x;
  if (j >= num_tokens) return;
  const int s = seq_ids ? seq_ids[j] : j;
  const int pos = positions[j];
  long long slot = -1;
  if (s >= 0 && s < num_seqs && pos >= 0) {
    const int lb = pos / bs;
    if (lb < mbs) {
      const int32_t pb = tables[(size_t)s * mbs + lb];
      if (pb >= 0 && pb < num_blocks) slot = (long long)pb * bs + pos % bs;
    }
  }
  if (slots_out && threadIdx.x == 0) slots_out[j] = (int32_t)slot;
  if (slot < 0) return;
  const long long src = (long long)j * chunks_per_row, dst = slot * chunks_per_row;
  for (int c = threadIdx.x; c < chunks_per_row; c += blockDim.x) {
    kc[dst + c] = key[src + c];
    vc[dst + c] = value[src + c];
  }
}

int launch_append_kv(const void* key, const void* value, void* k_cache, void* v_cache, int elem_bytes,
                     const int32_t* block_tables, int max_blocks_per_seq, const int32_t* seq_ids,
                     const int32_t* positions, int32_t* slot_mapping, int num_tokens, int num_seqs,
                     int num_blocks, int block_size, int num_kv_heads, int head_dim, void* stream) {
  if (num_tokens == 0) return hipSuccess;
  const int chunks_per_row = num_kv_heads * head_dim * elem_bytes / 16;
  int threads = 64;
  while (threads < chunks_per_row && threads < 256) threads *= 2;
  append_kv_kernel<<<num_tokens, threads, 0, (hipStream_t)stream>>>(
      (const uint4*)key, (const uint4*)value, (uint4*)k_cache, (uint4*)v_cache, block_tables, max_blocks_per_seq,
      seq_ids, positions, slot_mapping, num_tokens, num_seqs, block_size, num_blocks, chunks_per_row);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// copy_blocks: duplicate whole blocks (K, V and their scale rows).
// ---------------------------------------------------------------------------
__global__ void copy_blocks_kernel(uint4* __restrict__ kc, uint4* __restrict__ vc,
                                   float* __restrict__ ks, float* __restrict__ vs,
                                   const int32_t* __restrict__ src_dst, int chunks_per_block,
                                   int num_blocks, int num_kv_heads) {
  const int pair = blockIdx.x;
  const int src = src_dst[2 * pair];
  const int dst = src_dst[2 * pair + 1];
  if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks) return;
  const long long s0 = (long long)src * chunks_per_block;
  const long long d0 = (long long)dst * chunks_per_block;
  for (int c = blockIdx.y * blockDim.x + threadIdx.x; c < chunks_per_block; c += gridDim.y * blockDim.x) {
    kc[d0 + c] = kc[s0 + c];
    vc[d0 + c] = vc[s0 + c];
  }
  if (blockIdx.y == 0 && ks) {
    for (int h = threadIdx.x; h < num_kv_heads; h += blockDim.x) {
      ks[(size_t)dst * num_kv_heads + h] = ks[(size_t)src * num_kv_heads + h];
      vs[(size_t)dst * num_kv_heads + h] = vs[(size_t)src * num_kv_heads + h];
    }
  }
}

int launch_copy_blocks(void* k_cache, void* v_cache, float* k_scales, float* v_scales,
                       const int32_t* src_dst, int n, int elem_bytes, int num_blocks, int block_size,
                       int num_kv_heads, int head_dim, void* stream) {
  if (n == 0) return hipSuccess;
  const int chunks_per_block = block_size * num_kv_heads * head_dim * elem_bytes / 16;
  const int threads = 256;
  int gy = (chunks_per_block + threads - 1) / threads;
  if (gy > 64) gy = 64;
  copy_blocks_kernel<<<dim3(n, gy), threads, 0, (hipStream_t)stream>>>(
      (uint4*)k_cache, (uint4*)v_cache, k_scales, v_scales, src_dst, chunks_per_block, num_blocks,
      num_kv_heads);
  return hipGetLastError();
}

// Code type of the quantisers: INT8, FP8-E4M3 or packed INT4.
enum CodeKind { kCodeI8 = 0, kCodeFP8 = 1, kCodeI4 = 2, kCodeBF8 = 3 };

template <int CODE> struct CodeTraits;
template <> struct CodeTraits<kCodeI8> { static constexpr float qmax = 127.f; static constexpr int bits = 8; };
template <> struct CodeTraits<kCodeFP8> { static constexpr float qmax = 448.f; static constexpr int bits = 8; };
template <> struct CodeTraits<kCodeBF8> { static constexpr float qmax = 57344.f; static constexpr int bits = 8; };
template <> struct CodeTraits<kCodeI4> { static constexpr float qmax = 7.f; static constexpr int bits = 4; };

// Codes of N values x with scale sc ("KV Cache Engineering", section 8:
// x / scale rounded half to even and clipped to the largest code; FP8
// rounds to the E4M3 grid), stored at dst as N * bits / 8 bytes (INT4:
// element 2i in the low nibble of byte i).
template <int CODE, int N>
__device__ __forceinline__ void encode_store(const float* x, const float* sc, uint8_t* dst) {
  constexpr float qmax = CodeTraits<CODE>::qmax;
  uint8_t codes[N];
#pragma unroll
  for (int i = 0; i < N; ++i) {
    if (sc[i] == 0.f) {
      codes[i] = 0;
    } else {
      const float y = __fdiv_rn(x[i], sc[i]);
      if constexpr (CODE == kCodeFP8) {
        codes[i] = (uint8_t)f32_to_e4m3(y);
      } else if constexpr (CODE == kCodeBF8) {
        codes[i] = (uint8_t)f32_to_e5m2(y);
      } else {
        float r = rintf(y);
        r = fminf(fmaxf(r, -qmax), qmax);
        codes[i] = (uint8_t)(int8_t)(int)r;
      }
    }
  }
  if constexpr (CODE == kCodeI4) {
    constexpr int NB = N / 2;   // bytes
    uint32_t w[NB / 4];
#pragma unroll
    for (int k = 0; k < NB / 4; ++k) {
      w[k] = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        w[k] |= (uint32_t)((codes[8 * k + 2 * j] & 0xF) | ((codes[8 * k + 2 * j + 1] & 0xF) << 4)) << (8 * j);
    }
    if constexpr (NB == 16) *reinterpret_cast<uint4*>(dst) = make_uint4(w[0], w[1], w[2], w[3]);
    else *reinterpret_cast<uint2*>(dst) = make_uint2(w[0], w[1]);
  } else {
#pragma unroll
    for (int c = 0; c < N / 16; ++c) {
      uint32_t w[4];
#pragma unroll
      for (int k = 0; k < 4; ++k)
        w[k] = (uint32_t)codes[c * 16 + 4 * k] | ((uint32_t)codes[c * 16 + 4 * k + 1] << 8) |
               ((uint32_t)codes[c * 16 + 4 * k + 2] << 16) | ((uint32_t)codes[c * 16 + 4 * k + 3] << 24);
      reinterpret_cast<uint4*>(dst)[c] = make_uint4(w[0], w[1], w[2], w[3]);
    }
  }
}

// ---------------------------------------------------------------------------
// quantize_kv: one wave per (block, KV head) tile of [BS=16][D].
// Lane l reads token row l/4, quarter l%4 of the head dimension.
// "KV Cache Engineering", section 8: scale = absmax / largest code, codes
// rounded half to even and clipped.
// ---------------------------------------------------------------------------
template <typename SRC, int D, int CODE>
__global__ __launch_bounds__(64) void quantize_kv_kernel(
    const typename SRC::raw* __restrict__ src, void* __restrict__ dst, float* __restrict__ scales,
    const int32_t* __restrict__ block_ids, int num_blocks, int num_kv_heads) {
  constexpr int BS = 16;
  constexpr int ELEMS = D / 4;                 // per lane
  constexpr int SRC_CHUNKS = ELEMS * SRC::bytes / 16;
  constexpr int EL16 = 16 / SRC::bytes;
  constexpr int ROWB = D * CodeTraits<CODE>::bits / 8;   // code bytes per row
  const int b = block_ids ? block_ids[blockIdx.x] : (int)blockIdx.x;
  const int h = blockIdx.y;
  if (b < 0 || b >= num_blocks) return;
  const int lane = threadIdx.x;
  const int t = lane >> 2, q = lane & 3;
  const size_t row = ((size_t)b * BS + t) * num_kv_heads + h;   // element row index
  const uint4* p = reinterpret_cast<const uint4*>(src + row * D + q * ELEMS);
  float x[ELEMS];
#pragma unroll
  for (int c = 0; c < SRC_CHUNKS; ++c) {
    uint4 v = p[c];
    decode16<SRC>(v, x + c * EL16);
  }
  float a = 0.f;
#pragma unroll
  for (int i = 0; i < ELEMS; ++i) a = fmaxf(a, fabsf(x[i]));
  a = wave_max(a);
  const float sc = __fdiv_rn(a, CodeTraits<CODE>::qmax);
  float scv[ELEMS];
#pragma unroll
  for (int i = 0; i < ELEMS; ++i) scv[i] = sc;
  encode_store<CODE, ELEMS>(x, scv, reinterpret_cast<uint8_t*>(dst) + row * ROWB + q * (ROWB / 4));
  if (lane == 0) scales[(size_t)b * num_kv_heads + h] = sc;
}

// ---------------------------------------------------------------------------
// Grouped scales ("KV Cache Engineering", section 8, the KIVI paragraph:
// keys grouped by channel, values by token), each group inside one block
// tile: with quantize_kv's lane layout (lane l: token row t = l/4, quarter
// q = l%4 of the head dimension), channel q * D/4 + i of a tile lives in
// lanes q, q + 4, ..., q + 60, and token row t in lanes 4t .. 4t + 3.
// Sets each element's group scale (group absmax / largest code) and returns
// the tile's largest group scale (uniform).
// ---------------------------------------------------------------------------
enum GroupKind { kGroupChannel = 0, kGroupToken = 1 };

template <int CODE, int GROUP, int ELEMS>
__device__ __forceinline__ float group_scales(const float* x, float* sc) {
  constexpr float qmax = CodeTraits<CODE>::qmax;
  float smax;
  if constexpr (GROUP == kGroupChannel) {
    smax = 0.f;
#pragma unroll
    for (int i = 0; i < ELEMS; ++i) {
      float a = fabsf(x[i]);
#pragma unroll
      for (int o = 4; o < 64; o <<= 1) a = fmaxf(a, __shfl_xor(a, o, 64));
      sc[i] = __fdiv_rn(a, qmax);
      smax = fmaxf(smax, sc[i]);
    }
    smax = fmaxf(smax, __shfl_xor(smax, 1, 64));
    smax = fmaxf(smax, __shfl_xor(smax, 2, 64));
  } else {
    float a = 0.f;
#pragma unroll
    for (int i = 0; i < ELEMS; ++i) a = fmaxf(a, fabsf(x[i]));
    a = fmaxf(a, __shfl_xor(a, 1, 64));
    a = fmaxf(a, __shfl_xor(a, 2, 64));
    const float st = __fdiv_rn(a, qmax);
#pragma unroll
    for (int i = 0; i < ELEMS; ++i) sc[i] = st;
    smax = wave_max(st);
  }
  return smax;
}

// Writes the group scales of one tile: channel scales [D] (row-0 lanes, a
// quarter each) or token scales [16] (one lane per row).
template <int GROUP, int D>
__device__ __forceinline__ void store_group_scales(float* gs_tile, const float* sc, int t, int q) {
  constexpr int ELEMS = D / 4;
  if constexpr (GROUP == kGroupChannel) {
    if (t == 0) {
#pragma unroll
      for (int i = 0; i < ELEMS; i += 4)
        *reinterpret_cast<float4*>(gs_tile + q * ELEMS + i) = make_float4(sc[i], sc[i + 1], sc[i + 2], sc[i + 3]);
    }
  } else {
    if (q == 0) gs_tile[t] = sc[0];
  }
}

template <typename SRC, int D, int CODE, int GROUP>
__global__ __launch_bounds__(64) void quantize_kv_grouped_kernel(
    const typename SRC::raw* __restrict__ src, void* __restrict__ dst, float* __restrict__ tile_scales,
    float* __restrict__ gscales, const int32_t* __restrict__ block_ids, int num_blocks, int num_kv_heads) {
  constexpr int BS = 16;
  constexpr int ELEMS = D / 4;                 // per lane
  constexpr int SRC_CHUNKS = ELEMS * SRC::bytes / 16;
  constexpr int EL16 = 16 / SRC::bytes;
  constexpr int ROWB = D * CodeTraits<CODE>::bits / 8;   // code bytes per row
  constexpr int GS = GROUP == kGroupChannel ? D : BS;    // group scales per tile
  const int b = block_ids ? block_ids[blockIdx.x] : (int)blockIdx.x;
  const int h = blockIdx.y;
  if (b < 0 || b >= num_blocks) return;
  const int lane = threadIdx.x;
  const int t = lane >> 2, q = lane & 3;
  const size_t row = ((size_t)b * BS + t) * num_kv_heads + h;   // element row index
  const uint4* p = reinterpret_cast<const uint4*>(src + row * D + q * ELEMS);
  float x[ELEMS];
#pragma unroll
  for (int c = 0; c < SRC_CHUNKS; ++c) decode16<SRC>(p[c], x + c * EL16);
  float sc[ELEMS];
  const float smax = group_scales<CODE, GROUP, ELEMS>(x, sc);
  encode_store<CODE, ELEMS>(x, sc, reinterpret_cast<uint8_t*>(dst) + row * ROWB + q * (ROWB / 4));
  store_group_scales<GROUP, D>(gscales + ((size_t)b * num_kv_heads + h) * GS, sc, t, q);
  if (lane == 0 && tile_scales) tile_scales[(size_t)b * num_kv_heads + h] = smax;
}

template <typename SRC, int D>
static int launch_q(const void* src, void* dst, int code_dtype, float* scales, const int32_t* ids,
                    int n_blocks, int num_blocks, int num_kv_heads, hipStream_t st) {
  dim3 grid(n_blocks, num_kv_heads);
  typedef typename SRC::raw R;
  if (code_dtype == PKV_FP8E4M3)
    quantize_kv_kernel<SRC, D, kCodeFP8><<<grid, 64, 0, st>>>((const R*)src, dst, scales, ids, num_blocks,
                                                              num_kv_heads);
  else if (code_dtype == PKV_FP8E5M2)
    quantize_kv_kernel<SRC, D, kCodeBF8><<<grid, 64, 0, st>>>((const R*)src, dst, scales, ids, num_blocks,
                                                              num_kv_heads);
  else if (code_dtype == PKV_I4)
    quantize_kv_kernel<SRC, D, kCodeI4><<<grid, 64, 0, st>>>((const R*)src, dst, scales, ids, num_blocks,
                                                             num_kv_heads);
  else
    quantize_kv_kernel<SRC, D, kCodeI8><<<grid, 64, 0, st>>>((const R*)src, dst, scales, ids, num_blocks,
                                                             num_kv_heads);
  return hipGetLastError();
}

template <typename SRC, int D, int GROUP>
static int launch_qg(const void* src, void* dst, int code_dtype, float* tile_scales, float* gscales,
                     const int32_t* ids, int n_blocks, int num_blocks, int num_kv_heads, hipStream_t st) {
  dim3 grid(n_blocks, num_kv_heads);
  typedef typename SRC::raw R;
#define PKV_QG(CODE)                                                                                   \
  quantize_kv_grouped_kernel<SRC, D, CODE, GROUP><<<grid, 64, 0, st>>>((const R*)src, dst, tile_scales, \
                                                                      gscales, ids, num_blocks, num_kv_heads)
  switch (code_dtype) {
    case PKV_FP8E4M3: PKV_QG(kCodeFP8); break;
    case PKV_FP8E5M2: PKV_QG(kCodeBF8); break;
    case PKV_I4: PKV_QG(kCodeI4); break;
    default: PKV_QG(kCodeI8); break;
  }
#undef PKV_QG
  return hipGetLastError();
}

int launch_quantize_kv_grouped(const void* src_cache, int src_dtype, void* dst_codes, int code_dtype,
                               float* tile_scales, float* group_scales, int group, const int32_t* block_ids,
                               int n_blocks, int num_blocks, int num_kv_heads, int head_dim, void* stream) {
  if (n_blocks == 0) return hipSuccess;
  hipStream_t st = (hipStream_t)stream;
#define PKV_QGD(SRC, D)                                                                                    \
  return group == PKV_GROUP_CHANNEL                                                                        \
             ? launch_qg<SRC, D, kGroupChannel>(src_cache, dst_codes, code_dtype, tile_scales, group_scales, \
                                                block_ids, n_blocks, num_blocks, num_kv_heads, st)          \
             : launch_qg<SRC, D, kGroupToken>(src_cache, dst_codes, code_dtype, tile_scales, group_scales,   \
                                              block_ids, n_blocks, num_blocks, num_kv_heads, st)
#define PKV_QGS(SRC)                 \
  if (head_dim == 64) PKV_QGD(SRC, 64); \
  PKV_QGD(SRC, 128)
  switch (src_dtype) {
    case PKV_F32: { PKV_QGS(F32); }
    case PKV_BF16: { PKV_QGS(BF16); }
    default: { PKV_QGS(F16); }
  }
#undef PKV_QGS
#undef PKV_QGD
}

int launch_quantize_kv(const void* src_cache, int src_dtype, void* dst_codes, int code_dtype,
                       float* dst_scales, const int32_t* block_ids, int n_blocks, int num_blocks,
                       int block_size, int num_kv_heads, int head_dim, void* stream) {
  (void)block_size;
  if (n_blocks == 0) return hipSuccess;
  hipStream_t st = (hipStream_t)stream;
#define PKV_Q(SRC)                                                                                  \
  return head_dim == 64 ? launch_q<SRC, 64>(src_cache, dst_codes, code_dtype, dst_scales, block_ids, \
                                            n_blocks, num_blocks, num_kv_heads, st)                 \
                        : launch_q<SRC, 128>(src_cache, dst_codes, code_dtype, dst_scales, block_ids, \
                                             n_blocks, num_blocks, num_kv_heads, st)
  switch (src_dtype) {
    case PKV_F32: PKV_Q(F32);
    case PKV_BF16: PKV_Q(BF16);
    default: PKV_Q(F16);
  }
#undef PKV_Q
}

// ---------------------------------------------------------------------------
// append_kv_quantized: the new token of each sequence goes into the
// sequence's tail (the source values of its partial last block), and the
// block is quantised again from the tail, its unwritten rows taken as
// zeros.  One wave per (sequence, KV head, K or V), with quantize_kv's lane
// layout (lane l: token row l/4, quarter l%4 of the head dimension) and the
// same arithmetic, so a full block ends with exactly quantize_kv's codes.
// GRP: grouped scales (keys per channel into k_group and their largest into
// k_scales, values per token into v_group), quantize_kv_grouped's arithmetic.
// ---------------------------------------------------------------------------
template <typename SRC, int D, int CODE, bool GRP>
__global__ __launch_bounds__(64) void append_quantized_kernel(
    const typename SRC::raw* __restrict__ key, const typename SRC::raw* __restrict__ value,
    typename SRC::raw* __restrict__ k_tail, typename SRC::raw* __restrict__ v_tail, uint8_t* __restrict__ k_codes,
    uint8_t* __restrict__ v_codes, float* __restrict__ k_scales, float* __restrict__ v_scales,
    float* __restrict__ k_group, float* __restrict__ v_group, const int32_t* __restrict__ tables, int mbs,
    const int32_t* __restrict__ positions, int num_blocks, int num_kv_heads) {
  constexpr int BS = 16;
  constexpr int ELEMS = D / 4;                 // per lane
  constexpr int SRC_CHUNKS = ELEMS * SRC::bytes / 16;
  constexpr int EL16 = 16 / SRC::bytes;
  constexpr int ROWB = D * CodeTraits<CODE>::bits / 8;   // code bytes per row
  const int s = blockIdx.x, h = blockIdx.y;
  const bool is_v = blockIdx.z != 0;
  const int pos = positions[s];
  if (pos < 0 || pos / BS >= mbs) return;
  const int row = pos % BS;
  const int b = tables[(size_t)s * mbs + pos / BS];
  if (b < 0 || b >= num_blocks) return;
  const int lane = threadIdx.x;
  const int t = lane >> 2, q = lane & 3;
  typename SRC::raw* tail = (is_v ? v_tail : k_tail) + (((size_t)s * BS + t) * num_kv_heads + h) * D + q * ELEMS;
  float x[ELEMS];
  if (t < row) {
    const uint4* p = reinterpret_cast<const uint4*>(tail);
#pragma unroll
    for (int c = 0; c < SRC_CHUNKS; ++c) decode16<SRC>(p[c], x + c * EL16);
  } else if (t == row) {
    const typename SRC::raw* src = (is_v ? value : key) + ((size_t)s * num_kv_heads + h) * D + q * ELEMS;
    const uint4* p = reinterpret_cast<const uint4*>(src);
#pragma unroll
    for (int c = 0; c < SRC_CHUNKS; ++c) {
      const uint4 v = p[c];
      reinterpret_cast<uint4*>(tail)[c] = v;
      decode16<SRC>(v, x + c * EL16);
    }
  } else {
#pragma unroll
    for (int i = 0; i < ELEMS; ++i) x[i] = 0.f;
  }
  uint8_t* dst = is_v ? v_codes : k_codes;
  float scv[ELEMS];
  if constexpr (GRP) {
    const size_t tile = (size_t)b * num_kv_heads + h;
    if (is_v) {
      (void)group_scales<CODE, kGroupToken, ELEMS>(x, scv);
      store_group_scales<kGroupToken, D>(v_group + tile * BS, scv, t, q);
    } else {
      const float smax = group_scales<CODE, kGroupChannel, ELEMS>(x, scv);
      store_group_scales<kGroupChannel, D>(k_group + tile * D, scv, t, q);
      if (lane == 0) k_scales[tile] = smax;
    }
    encode_store<CODE, ELEMS>(x, scv, dst + (((size_t)b * BS + t) * num_kv_heads + h) * ROWB + q * (ROWB / 4));
  } else {
    float a = 0.f;
#pragma unroll
    for (int i = 0; i < ELEMS; ++i) a = fmaxf(a, fabsf(x[i]));
    a = wave_max(a);
    const float sc = __fdiv_rn(a, CodeTraits<CODE>::qmax);
#pragma unroll
    for (int i = 0; i < ELEMS; ++i) scv[i] = sc;
    encode_store<CODE, ELEMS>(x, scv, dst + (((size_t)b * BS + t) * num_kv_heads + h) * ROWB + q * (ROWB / 4));
    if (lane == 0) (is_v ? v_scales : k_scales)[(size_t)b * num_kv_heads + h] = sc;
  }
}

template <typename SRC, int D, bool GRP>
static int launch_aq(const void* key, const void* value, void* k_tail, void* v_tail, void* k_codes, void* v_codes,
                     int code_dtype, float* k_scales, float* v_scales, float* k_group, float* v_group,
                     const int32_t* tables, int mbs, const int32_t* positions, int num_seqs, int num_blocks,
                     int num_kv_heads, hipStream_t st) {
  typedef typename SRC::raw R;
  const dim3 grid(num_seqs, num_kv_heads, 2);
#define PKV_AQK(CODE)                                                                                      \
  append_quantized_kernel<SRC, D, CODE, GRP><<<grid, 64, 0, st>>>(                                         \
      (const R*)key, (const R*)value, (R*)k_tail, (R*)v_tail, (uint8_t*)k_codes, (uint8_t*)v_codes, k_scales, \
      v_scales, k_group, v_group, tables, mbs, positions, num_blocks, num_kv_heads)
  if (code_dtype == PKV_FP8E4M3) PKV_AQK(kCodeFP8);
  else if (code_dtype == PKV_FP8E5M2) PKV_AQK(kCodeBF8);
  else if (code_dtype == PKV_I4) PKV_AQK(kCodeI4);
  else PKV_AQK(kCodeI8);
#undef PKV_AQK
  return hipGetLastError();
}

// k_group / v_group non-null: grouped scales (k_scales takes the tiles'
// largest channel scales, v_scales is unused).
int launch_append_quantized(const void* key, const void* value, int src_dtype, void* k_tail, void* v_tail,
                            void* k_codes, void* v_codes, int code_dtype, float* k_scales, float* v_scales,
                            float* k_group, float* v_group, const int32_t* block_tables, int max_blocks_per_seq,
                            const int32_t* positions, int num_seqs, int num_blocks, int num_kv_heads, int head_dim,
                            void* stream) {
  hipStream_t st = (hipStream_t)stream;
#define PKV_AQD(SRC, D, GRP)                                                                                  \
  return launch_aq<SRC, D, GRP>(key, value, k_tail, v_tail, k_codes, v_codes, code_dtype, k_scales, v_scales, \
                                k_group, v_group, block_tables, max_blocks_per_seq, positions, num_seqs,      \
                                num_blocks, num_kv_heads, st)
#define PKV_AQ(SRC)                                  \
  if (k_group) {                                     \
    if (head_dim == 64) PKV_AQD(SRC, 64, true);      \
    PKV_AQD(SRC, 128, true);                         \
  }                                                  \
  if (head_dim == 64) PKV_AQD(SRC, 64, false);       \
  PKV_AQD(SRC, 128, false)
  switch (src_dtype) {
    case PKV_F32: { PKV_AQ(F32); }
    case PKV_BF16: { PKV_AQ(BF16); }
    default: { PKV_AQ(F16); }
  }
#undef PKV_AQ
#undef PKV_AQD
}

// ---------------------------------------------------------------------------
// Streaming-read probe: workgroup w reads the w-th contiguous chunk of the
// buffer, each thread keeping 8 16-byte non-temporal loads in flight, and
// folds what it read into one word per workgroup.
// ---------------------------------------------------------------------------
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4* __restrict__ src, size_t n16,
                                                          uint32_t* __restrict__ sink) {
  constexpr int U = 8;
  const size_t per = (n16 + gridDim.x - 1) / gridDim.x;
  const size_t lo = (size_t)blockIdx.x * per;
  const size_t hi = lo + per < n16 ? lo + per : n16;
  uint32_t acc = 0;
  size_t i = lo + threadIdx.x;
  for (; i + (U - 1) * 256 < hi; i += U * 256) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(src + i + u * 256);
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  for (; i < hi; i += 256) {
    const u32x4 v = __builtin_nontemporal_load(src + i);
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  __shared__ uint32_t red[256];
  red[threadIdx.x] = acc;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (threadIdx.x < o) red[threadIdx.x] ^= red[threadIdx.x + o];
    __syncthreads();
  }
  if (threadIdx.x == 0) sink[blockIdx.x] = red[0];
}

int launch_stream_read(const void* src, size_t bytes, uint32_t* sink, void* stream) {
  stream_read_kernel<<<kStreamReadBlocks, 256, 0, (hipStream_t)stream>>>((const u32x4*)src, bytes / 16, sink);
  return hipGetLastError();
}

}  // namespace pkv
