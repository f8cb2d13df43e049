// Device helpers shared by the ZHA kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace zha {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

struct bf16_t {
  uint16_t bits;
};

template <typename T>
struct Elem;
template <>
struct Elem<float> {
  static constexpr int size = 4;
  static constexpr int per16 = 4;  // elements per 16-byte piece
};
template <>
struct Elem<bf16_t> {
  static constexpr int size = 2;
  static constexpr int per16 = 8;
};

__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }
// 16-byte load with the nontemporal hint (a streamed operand read once,
// whole 128-byte lines per instruction)
__device__ __forceinline__ uint4 ld16_nt(const void* p) {
  typedef unsigned int u32x4_nt __attribute__((ext_vector_type(4)));
  const u32x4_nt v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_nt*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// Raw buffer loads: the base is wave-uniform, offsets are bytes, and a load
// at an offset past `bytes` returns zeros (no branch, no fault), so masked
// loads need no control flow.  kOffNone is such an offset.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr uint32_t kOffNone = 0x80000000u;
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  // base and size are wave-uniform by contract: take lane 0's so that they
  // live in scalar registers whatever the compiler proved
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  void* p = reinterpret_cast<void*>(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(p, (short)0, (int)__builtin_amdgcn_readfirstlane(bytes), 0x00020000);
}
// Cache policy of streamed operands (each byte read once per call, each
// 128-byte line by one instruction): the nontemporal bit, which lifts a plain
// read stream from about 6.1 to 7.1 TB/s on MI355X.  Loads that split a line
// over two instructions (MFMA operand layouts) and re-read data use 0.
constexpr int kStream = 2;
template <int AUX = kStream>
__device__ __forceinline__ uint4 bld16(rsrc_t r, uint32_t off) {
  typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;
  const u32x4 v = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, AUX));
  return make_uint4(v[0], v[1], v[2], v[3]);
}
template <int AUX = kStream>
__device__ __forceinline__ float bld4f(rsrc_t r, uint32_t off) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, AUX));
}
__device__ __forceinline__ void st16(void* p, uint4 v) { *reinterpret_cast<uint4*>(p) = v; }
// Nontemporal stores for streams written once and read by a later kernel:
// on MI355X, tiles that read 64 KiB and write 16 KiB move about 4% more
// bytes per second with them than with plain stores.
__device__ __forceinline__ void st16_nt(float* p, float a, float b, float c, float d) {
  __builtin_nontemporal_store(f32x4{a, b, c, d}, reinterpret_cast<f32x4*>(p));
}
__device__ __forceinline__ void st4_nt(float* p, float a) { __builtin_nontemporal_store(a, p); }

// Unpack one 16-byte piece into fp32 values.
__device__ __forceinline__ void unpack(const uint4& v, float* out, bf16_t) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    out[2 * i] = __uint_as_float(w[i] << 16);
    out[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}
__device__ __forceinline__ void unpack(const uint4& v, float* out, float) {
  out[0] = __uint_as_float(v.x);
  out[1] = __uint_as_float(v.y);
  out[2] = __uint_as_float(v.z);
  out[3] = __uint_as_float(v.w);
}

// Round fp32 to bf16 (round to nearest even, hardware conversion).
__device__ __forceinline__ uint32_t bf16_bits(float x) {
  __bf16 b = (__bf16)x;
  return (uint32_t)__builtin_bit_cast(uint16_t, b);
}

// Two fp32 values rounded to bf16 (nearest even) by one packed conversion:
// a in the low half, b in the high half.
typedef float f32x2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t bf16_pair(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2v{a, b}, bf16x2v));
}
// Sum of v over the lanes l, l + 4, l + 8 and l + 12 of each 16-lane row (the
// four lanes whose indexes agree in bits 0-1 and differ in bits 2-3), in
// every lane: two DPP row rotations (by 4, then by 8) feed the adds, so no
// LDS permute is involved.
__device__ __forceinline__ float row_sum_stride4(float v) {
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x124, 0xf, 0xf, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x128, 0xf, 0xf, false));
  return v;
}
// The rounded values of a bf16_pair word as fp32.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
// x rounded to bf16 (nearest even), as fp32.
__device__ __forceinline__ float round_bf16f(float x) { return bf16_lo(bf16_pair(x, 0.f)); }
// Four bf16 values (two bf16_pair words, low word first) as the operand of
// a K = 16 bf16 MFMA.
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ s16x4 pack_s16x4(uint32_t lo, uint32_t hi) {
  return __builtin_bit_cast(s16x4, u32x2v{lo, hi});
}

// Pack fp32 values of one piece, rounding to the storage type; also returns
// the rounded values as fp32 in `rounded`.
__device__ __forceinline__ uint4 pack(const float* x, float* rounded, bf16_t) {
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    w[i] = bf16_pair(x[2 * i], x[2 * i + 1]);
    rounded[2 * i] = bf16_lo(w[i]);
    rounded[2 * i + 1] = bf16_hi(w[i]);
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}
__device__ __forceinline__ uint4 pack(const float* x, float* rounded, float) {
#pragma unroll
  for (int i = 0; i < 4; ++i) rounded[i] = x[i];
  return make_uint4(__float_as_uint(x[0]), __float_as_uint(x[1]), __float_as_uint(x[2]),
                    __float_as_uint(x[3]));
}

__device__ __forceinline__ bf16x8 as_bf16x8(const uint4& v) { return __builtin_bit_cast(bf16x8, v); }

// Monotone map of a float to uint32: larger float -> larger key (-inf lowest
// of the non-NaN values).
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_to_float(uint32_t k) {
  uint32_t u = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
  return __uint_as_float(u);
}

__device__ __forceinline__ float wave_max_xor(float v, int from, int to) {
  for (int o = from; o < to; o <<= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ float wave_sum_xor(float v, int from, int to) {
  for (int o = from; o < to; o <<= 1) v += __shfl_xor(v, o);
  return v;
}

constexpr float kNegInf = -__builtin_huge_valf();

// Wave-scope barrier for LDS regions private to one wave.
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

}  // namespace zha
