// Device helpers for gfx950: storage-type conversions, 16-byte vector
// access and wave64 reductions.
#ifndef PKV_DEVICE_H_
#define PKV_DEVICE_H_

#include <hip/hip_runtime.h>

#include <atomic>
#include <stdint.h>

namespace pkv {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __fp16 fp16x4 __attribute__((__vector_size__(4 * sizeof(__fp16))));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx2 __attribute__((ext_vector_type(2)));
typedef short shortx4 __attribute__((ext_vector_type(4)));

// Storage tags: each holds raw bits; `Elems16` elements fill 16 bytes.
struct F32 { typedef float raw; static constexpr int bytes = 4; static constexpr int bits = 32; };
struct BF16 { typedef uint16_t raw; static constexpr int bytes = 2; static constexpr int bits = 16; };
struct F16 { typedef uint16_t raw; static constexpr int bytes = 2; static constexpr int bits = 16; };
struct I8 { typedef int8_t raw; static constexpr int bytes = 1; static constexpr int bits = 8; };
struct FP8 { typedef uint8_t raw; static constexpr int bytes = 1; static constexpr int bits = 8; };
// OCP FP8 E5M2 codes
struct BF8 { typedef uint8_t raw; static constexpr int bytes = 1; static constexpr int bits = 8; };
// two signed 4-bit codes per byte: element 2i in the low nibble
struct I4 { typedef uint8_t raw; static constexpr int bytes = 1; static constexpr int bits = 4; };

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }
__device__ __forceinline__ float f16_to_f32(uint32_t bits16) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
}

// Round-to-nearest-even float -> bf16 bits (hardware v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint16_t f32_to_bf16(float x) {
  return __builtin_bit_cast(uint16_t, (__bf16)x);
}
__device__ __forceinline__ uint16_t f32_to_f16(float x) {
  return __builtin_bit_cast(uint16_t, (_Float16)x);
}

// Decode the 16 bytes `v` holding 16/bytes elements of storage type T into
// `out` as float.  Exact for every storage type (codes decode to the code's
// own value; the scale is applied by the caller).
template <typename T> __device__ __forceinline__ void decode16(const uint4& v, float* out);

template <> __device__ __forceinline__ void decode16<F32>(const uint4& v, float* out) {
  out[0] = __uint_as_float(v.x); out[1] = __uint_as_float(v.y);
  out[2] = __uint_as_float(v.z); out[3] = __uint_as_float(v.w);
}
template <> __device__ __forceinline__ void decode16<BF16>(const uint4& v, float* out) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    out[2 * i] = __uint_as_float(w[i] << 16);
    out[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}
template <> __device__ __forceinline__ void decode16<F16>(const uint4& v, float* out) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    out[2 * i] = f16_to_f32(w[i] & 0xFFFFu);
    out[2 * i + 1] = f16_to_f32(w[i] >> 16);
  }
}
template <> __device__ __forceinline__ void decode16<I8>(const uint4& v, float* out) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int b = 0; b < 4; ++b) out[4 * i + b] = (float)(int8_t)((w[i] >> (8 * b)) & 0xFF);
  }
}
// OCP FP8-E4M3 -> fp32 via the gfx950 converter (exact).
template <> __device__ __forceinline__ void decode16<FP8>(const uint4& v, float* out) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    floatx2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(w[i], false);
    floatx2 hi = __builtin_amdgcn_cvt_pk_f32_fp8(w[i], true);
    out[4 * i + 0] = lo[0]; out[4 * i + 1] = lo[1];
    out[4 * i + 2] = hi[0]; out[4 * i + 3] = hi[1];
  }
}

// Store helpers for the output types.
template <typename T> __device__ __forceinline__ void store_out(void* base, size_t idx, float x);
template <> __device__ __forceinline__ void store_out<F32>(void* base, size_t idx, float x) {
  reinterpret_cast<float*>(base)[idx] = x;
}
template <> __device__ __forceinline__ void store_out<BF16>(void* base, size_t idx, float x) {
  reinterpret_cast<uint16_t*>(base)[idx] = f32_to_bf16(x);
}
template <> __device__ __forceinline__ void store_out<F16>(void* base, size_t idx, float x) {
  reinterpret_cast<uint16_t*>(base)[idx] = f32_to_f16(x);
}

template <typename T> __device__ __forceinline__ float load_elem(const void* base, size_t idx);
template <> __device__ __forceinline__ float load_elem<F32>(const void* base, size_t idx) {
  return reinterpret_cast<const float*>(base)[idx];
}
template <> __device__ __forceinline__ float load_elem<BF16>(const void* base, size_t idx) {
  return bf16_to_f32(reinterpret_cast<const uint16_t*>(base)[idx]);
}
template <> __device__ __forceinline__ float load_elem<F16>(const void* base, size_t idx) {
  return f16_to_f32(reinterpret_cast<const uint16_t*>(base)[idx]);
}

// ---------------------------------------------------------------------------
// wave64 reductions (butterfly over all 64 lanes)
// ---------------------------------------------------------------------------
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

// DPP quad permutes: exchange with lane ^1 / ^2 inside groups of four lanes.
__device__ __forceinline__ float dpp_xor1(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, true));
}
__device__ __forceinline__ float dpp_xor2(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, true));
}

// ---------------------------------------------------------------------------
// FP8-E4M3 (OCP "fn") encoder: round to nearest, ties to even, saturating at
// +-448, sign of zero kept.  Integer arithmetic on the fp32 bit pattern.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t f32_to_e4m3(float x) {
  const uint32_t u = __float_as_uint(x);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7FFFFFFFu;
  uint32_t code;
  if (a > 0x43E00000u) {                 // |x| > 448: saturate
    code = 0x7E;
  } else if (a >= 0x3C800000u) {         // |x| >= 2^-6: normal range
    // keep exponent and top 3 mantissa bits, round the 20 dropped bits
    uint32_t q = a >> 20;
    const uint32_t rem = a & 0xFFFFFu;
    if (rem > 0x80000u || (rem == 0x80000u && (q & 1u))) q += 1;
    code = q - (120u << 3);              // rebias exponent 127 -> 7
    if (code > 0x7E) code = 0x7E;
  } else {                               // subnormal: value = m * 2^-9
    const float y = __uint_as_float(a) * 512.0f;   // exact power-of-two scaling
    code = (uint32_t)rintf(y);                     // 0..8; 8 is the smallest normal
  }
  return code | sign;
}

// ---------------------------------------------------------------------------
// FP8-E5M2 (OCP) encoder: round to nearest, ties to even, saturating at
// +-57344 (no infinity is produced), sign of zero kept.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t f32_to_e5m2(float x) {
  const uint32_t u = __float_as_uint(x);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7FFFFFFFu;
  uint32_t code;
  if (a > 0x47600000u) {                 // |x| > 57344: saturate
    code = 0x7B;
  } else if (a >= 0x38800000u) {         // |x| >= 2^-14: normal range
    // keep exponent and top 2 mantissa bits, round the 21 dropped bits
    uint32_t q = a >> 21;
    const uint32_t rem = a & 0x1FFFFFu;
    if (rem > 0x100000u || (rem == 0x100000u && (q & 1u))) q += 1;
    code = q - (112u << 2);              // rebias exponent 127 -> 15
    if (code > 0x7B) code = 0x7B;
  } else {                               // subnormal: value = m * 2^-16
    const float y = __uint_as_float(a) * 65536.0f;   // exact power-of-two scaling
    code = (uint32_t)rintf(y);                       // 0..4; 4 is the smallest normal
  }
  return code | sign;
}

// ---------------------------------------------------------------------------
// buffer loads and the 16-bit MFMA operand helpers shared by the attention
// kernels
// ---------------------------------------------------------------------------
// Raw buffer resource over `nbytes` bytes from `base` (gfx9 descriptor word 3).
// A load whose offset + size exceeds nbytes returns zeros and reads nothing.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int nbytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, nbytes, 0x00020000);
}
// POL: cache-policy bits of the load (gfx950: 2 = nt, non-temporal).
template <int POL = 0>
__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, int voff) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, POL));
}
constexpr int kPolicyStream = 2;   // non-temporal: streamed data does not evict reused data
__device__ __forceinline__ float buf_load4(__amdgpu_buffer_rsrc_t r, int voff, int soff = 0) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0));
}
constexpr int kOutOfRange = 0x40000000;    // buffer offset that is always out of range

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
  // two values rounded to nearest even, packed (one v_cvt_pk_bf16_f32)
  __device__ static uint32_t pack2(float x, float y) {
    typedef __bf16 b2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((floatx2){x, y}, b2));
  }
  // c plus the two packed values (one v_dot2_f32_bf16 against (1, 1))
  __device__ static float acc2(uint32_t w, float c) {
    typedef __bf16 b2 __attribute__((ext_vector_type(2)));
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(b2, w), (b2){(__bf16)1.0f, (__bf16)1.0f}, c, false);
  }
  // two FP8-E4M3 codes (byte pair `hi` of w) -> two values, exactly
  template <bool HI> __device__ static uint32_t fp8x2(uint32_t w) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
  }
  template <bool HI> __device__ static uint32_t bf8x2(uint32_t w) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(w, 1.0f, HI));
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
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((floatx2){x, y}, h2));
  }
  __device__ static float acc2(uint32_t w, float c) {
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(h2, w), (h2){(_Float16)1.0f, (_Float16)1.0f}, c, false);
  }
  template <bool HI> __device__ static uint32_t fp8x2(uint32_t w) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, HI));
  }
  template <bool HI> __device__ static uint32_t bf8x2(uint32_t w) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_bf8(w, 1.0f, HI));
  }
  __device__ static shortx4 tr_read(const void* lds) {
    fp16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4f16((__attribute__((address_space(3))) fp16x4*)(lds));
    return __builtin_bit_cast(shortx4, v);
  }
};

// Raises a kernel's dynamic-LDS limit to `bytes` once per device (the
// attribute is set with the device current; devices up to 64 are tracked,
// others set it on every call).  `done` is the kernel's own flag array.
inline hipError_t set_lds_limit_once(const void* kernel, int bytes, std::atomic<bool>* done) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev >= 0 && dev < 64 && done[dev].load(std::memory_order_acquire)) return hipSuccess;
  e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess && dev >= 0 && dev < 64) done[dev].store(true, std::memory_order_release);
  return e;
}

}  // namespace pkv

#endif  // PKV_DEVICE_H_
