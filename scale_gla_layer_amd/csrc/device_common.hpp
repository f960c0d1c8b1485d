// Device helpers shared by the MS-GLA kernels (gfx950 / CDNA4, wave64).
//
// Every contraction in this library is expressed as a sequence of 64-byte
// "k-slabs": for a 16 x 16 output tile, lane l supplies 16 bytes of the A row
// (l % 16) and 16 bytes of the B column (l % 16), taken at byte offset
// 16 * (l / 16) of the slab.  For bfloat16 one slab is 32 k-values and one
// v_mfma_f32_16x16x32_bf16; for fp32 it is 16 k-values and four
// v_mfma_f32_16x16x4_f32 (element j of every lane in the j-th instruction).
// The k ordering inside a slab is irrelevant to a contraction as long as A and
// B use the same one.  The 16 x 16 fp32 result lives in 4 registers per lane:
// lane l holds rows 4 * (l / 16) + i, i = 0..3, of column l % 16.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "layout.hpp"

namespace msgla {

typedef __bf16 bf16;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;
typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2;

constexpr int WAVE = 64;

template <typename T> struct ElemTraits;
template <> struct ElemTraits<float> { static constexpr int PER16 = 4; };
template <> struct ElemTraits<bf16> { static constexpr int PER16 = 8; };

// number of T elements in 16 bytes / in a 64-byte slab / in a 128-byte row segment
template <typename T> constexpr int per16() { return ElemTraits<T>::PER16; }
template <typename T> constexpr int slab_elems() { return 4 * ElemTraits<T>::PER16; }

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// One 64-byte k-slab of a 16x16 tile: acc += A_slab * B_slab.
template <typename T> __device__ __forceinline__ f32x4 mma_slab(u32x4 a, u32x4 b, f32x4 acc);

template <> __device__ __forceinline__ f32x4 mma_slab<bf16>(u32x4 a, u32x4 b, f32x4 acc) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
}

// (Vector elements are copied to scalars first: __builtin_bit_cast applied
// directly to a vector-element lvalue reads element 0 with this compiler.)
__device__ __forceinline__ float u2f(uint32_t u) { return __builtin_bit_cast(float, u); }
__device__ __forceinline__ uint32_t f2u(float f) { return __builtin_bit_cast(uint32_t, f); }

template <> __device__ __forceinline__ f32x4 mma_slab<float>(u32x4 a, u32x4 b, f32x4 acc) {
  const f32x4 af = __builtin_bit_cast(f32x4, a), bf = __builtin_bit_cast(f32x4, b);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(af[0], bf[0], acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(af[1], bf[1], acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(af[2], bf[2], acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(af[3], bf[3], acc, 0, 0, 0);
  return acc;
}

// ---- conversions between 16-byte packets of T and fp32 lanes ------------------

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(bf16 v) { return (float)v; }
template <typename T> __device__ __forceinline__ T from_f32(float v) { return (T)v; }

// Unpack a 16-byte packet into PER16 floats.
template <typename T> __device__ __forceinline__ void unpack16(u32x4 p, float* out);
template <> __device__ __forceinline__ void unpack16<float>(u32x4 p, float* out) {
  const f32x4 f = __builtin_bit_cast(f32x4, p);
  out[0] = f[0];
  out[1] = f[1];
  out[2] = f[2];
  out[3] = f[3];
}
template <> __device__ __forceinline__ void unpack16<bf16>(u32x4 p, float* out) {
  const uint32_t w[4] = {p[0], p[1], p[2], p[3]};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    out[2 * i] = u2f(w[i] << 16);
    out[2 * i + 1] = u2f(w[i] & 0xffff0000u);
  }
}

// Pack PER16 floats into a 16-byte packet (round to nearest even for bf16).
template <typename T> __device__ __forceinline__ u32x4 pack16(const float* in);
template <> __device__ __forceinline__ u32x4 pack16<float>(const float* in) {
  return u32x4{f2u(in[0]), f2u(in[1]), f2u(in[2]), f2u(in[3])};
}
template <> __device__ __forceinline__ u32x4 pack16<bf16>(const float* in) {
  bf16x8 v;
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = (bf16)in[i];
  return __builtin_bit_cast(u32x4, v);
}

// 8-byte packets (4 bf16 or 2 fp32)
template <typename T> __device__ __forceinline__ u32x2 pack8(const float* in);
template <> __device__ __forceinline__ u32x2 pack8<float>(const float* in) {
  return u32x2{f2u(in[0]), f2u(in[1])};
}
template <> __device__ __forceinline__ u32x2 pack8<bf16>(const float* in) {
  bf16x4 v;
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = (bf16)in[i];
  return __builtin_bit_cast(u32x2, v);
}

// v = hi + lo with hi = bf16(v) and lo = bf16(v - hi), 8 values per packet.
__device__ __forceinline__ void split_bf16(const float* v, u32x4& hi, u32x4& lo) {
  float h[8], r[8];
  hi = pack16<bf16>(v);
  unpack16<bf16>(hi, h);
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = v[i] - h[i];
  lo = pack16<bf16>(r);
}

__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }
__device__ __forceinline__ u32x2 ld8(const void* p) { return *reinterpret_cast<const u32x2*>(p); }
__device__ __forceinline__ void st8(void* p, u32x2 v) { *reinterpret_cast<u32x2*>(p) = v; }

__device__ __forceinline__ u32x4 zero16() { return u32x4{0u, 0u, 0u, 0u}; }

// ---- XCD-aware block remap --------------------------------------------------
// MI355X dispatches consecutive workgroups round-robin over its 8 XCDs, each
// with its own L2.  remap_xcd turns the hardware block id into a work index
// such that each XCD receives one contiguous range of the work list, so
// neighbouring tiles (which share operands) share an L2.
__device__ __forceinline__ int remap_xcd(int bid, int per_xcd) {
  return (bid % N_XCD) * per_xcd + bid / N_XCD;
}

// True when a forward may read its state_in (no entry state, or its header
// passed the device-side check).
__device__ __forceinline__ bool state_in_ok(const StateCheck* chk) { return !chk || chk->status == 0; }

// Numerically safe log(sigmoid(z)) = min(z, 0) - log1p(exp(-|z|)).
__device__ __forceinline__ float logsigmoid_f(float z) {
  return fminf(z, 0.f) - log1pf(__expf(-fabsf(z)));
}

}  // namespace msgla
