// Device helpers shared by the gfx950 kernels of libswa.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "swa_internal.h"

namespace swa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
// 16-byte register piece of a K/V row: a native vector, so arrays of them stay in VGPRs (HIP's
// uint4 is a struct whose copies lower to memcpy and can pin an array to scratch)
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Word 3 of a raw buffer resource on gfx9-family parts (32-bit data format, no swizzle); with a
// stride of 0 the resource's record count is its size in bytes and out-of-range reads return 0.
constexpr int kBufferRsrcWord3 = 0x00020000;

#define SWA_LDS __attribute__((address_space(3)))

__device__ __forceinline__ float bf2f(uint16_t x) { return __uint_as_float((uint32_t)x << 16); }

// float -> bf16, round to nearest even (the hardware conversion on gfx950).
__device__ __forceinline__ uint16_t f2bf(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Value of `x` held by lane (lane ^ 32) of the wave (1-D workgroups of whole waves, so bit 5 of
// the work-item id is bit 5 of the lane; read through the builtin, not a device-library call).
__device__ __forceinline__ float other_half(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float((__builtin_amdgcn_workitem_id_x() & 32) ? r[0] : r[1]);
}

// 16 E4M3 codes (one u32x4, code i in byte i) to 16 bf16 values times a power-of-two scale
// (exact): v_cvt_scalef32_pk_bf16_fp8 converts two codes and multiplies by 2^exponent(scale).
__device__ __forceinline__ void e4m3x16_to_bf16(u32x4 in, float scale, bf16x8 &lo, bf16x8 &hi) {
  bf16x2 p[8];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    p[2 * j] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(in[j], scale, false);     // bytes 0, 1
    p[2 * j + 1] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(in[j], scale, true);  // bytes 2, 3
  }
  lo = bf16x8{p[0][0], p[0][1], p[1][0], p[1][1], p[2][0], p[2][1], p[3][0], p[3][1]};
  hi = bf16x8{p[4][0], p[4][1], p[5][0], p[5][1], p[6][0], p[6][1], p[7][0], p[7][1]};
}

// 8 E4M3 codes (one uint2, code i in byte i) to 8 bf16 values (as one 16-byte u32x4) times a
// power-of-two scale (exact).
__device__ __forceinline__ u32x4 e4m3x8_to_bf16(uint2 in, float scale) {
  const bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(in.x, scale, false);
  const bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(in.x, scale, true);
  const bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(in.y, scale, false);
  const bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(in.y, scale, true);
  return u32x4{__builtin_bit_cast(uint32_t, p0), __builtin_bit_cast(uint32_t, p1), __builtin_bit_cast(uint32_t, p2),
               __builtin_bit_cast(uint32_t, p3)};
}

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// LDS transposing read: in each group of 16 lanes, lane i receives element (i % 4) of the 8-byte
// chunks addressed by lanes i/4, i/4+4, i/4+8, i/4+12 of its group (checked on gfx950).
__device__ __forceinline__ bf16x4 lds_read_tr(const uint16_t *p) {
  i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((SWA_LDS i16x4 *)(p));
  return __builtin_bit_cast(bf16x4, v);
}

__device__ __forceinline__ bf16x8 cat(bf16x4 a, bf16x4 b) {
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

// ---- RoPE (RoFormer, Su et al. 2021, §3.2-§3.4): pair i of a head vector turns by p * theta_i at
// position p.  The angle comes from two fp32 (cos, sin) tables built on the host in float64:
// lo[l][i] for l * theta_i (l < 2048) and hi[h][i] for h * 2048 * theta_i; p = h * 2048 + l turns by
// the product of the two rotations.  Every RoPE path (the standalone kernel and the fused loads and
// commits) uses these helpers, so they all round the same way.
__device__ __forceinline__ float2 rope_cs(float2 lo, float2 hi) {  // (cos, sin) of the summed angle
  return make_float2(fmaf(hi.x, lo.x, -hi.y * lo.y), fmaf(hi.y, lo.x, hi.x * lo.y));
}
__device__ __forceinline__ void rope_turn(float &x, float &y, float2 cs) {  // (x + iy) * (c + is)
  const float nx = fmaf(x, cs.x, -y * cs.y);
  const float ny = fmaf(x, cs.y, y * cs.x);
  x = nx;
  y = ny;
}
// (cos, sin) of pairs i0 .. i0+N-1 (N even, i0 even) at position p
template <int N>
__device__ __forceinline__ void rope_angles(const float2 *lo_tab, const float2 *hi_tab, int half, int64_t p, int i0,
                                            float2 (&cs)[N]) {
  const float4 *lt = reinterpret_cast<const float4 *>(lo_tab + (p & (kRopeLo - 1)) * half + i0);
  const float4 *ht = reinterpret_cast<const float4 *>(hi_tab + (p >> kRopeLoBits) * half + i0);
#pragma unroll
  for (int j = 0; j < N / 2; ++j) {
    const float4 l = lt[j], h = ht[j];
    cs[2 * j] = rope_cs(make_float2(l.x, l.y), make_float2(h.x, h.y));
    cs[2 * j + 1] = rope_cs(make_float2(l.z, l.w), make_float2(h.z, h.w));
  }
}
__device__ __forceinline__ float bf_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }
__device__ __forceinline__ uint32_t bf_pack(float lo, float hi) {
  return (uint32_t)f2bf(lo) | ((uint32_t)f2bf(hi) << 16);
}
// 8 bf16 of the pairs layout: pairs i0 .. i0+3 as (x, y) neighbours, rotated at position p
__device__ __forceinline__ u32x4 rope_pairs8(u32x4 u, const float2 *lo_tab, const float2 *hi_tab, int half,
                                             int64_t p, int i0) {
  float2 cs[4];
  rope_angles<4>(lo_tab, hi_tab, half, p, i0, cs);
  u32x4 r;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    float x = bf_lo(u[j]), y = bf_hi(u[j]);
    rope_turn(x, y, cs[j]);
    r[j] = bf_pack(x, y);
  }
  return r;
}
// halves layout: ux holds the first coordinates of pairs i0 .. i0+7, uy the second ones
__device__ __forceinline__ void rope_halves8(u32x4 &ux, u32x4 &uy, const float2 *lo_tab, const float2 *hi_tab,
                                             int half, int64_t p, int i0) {
  float2 cs[8];
  rope_angles<8>(lo_tab, hi_tab, half, p, i0, cs);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    float x0 = bf_lo(ux[j]), x1 = bf_hi(ux[j]), y0 = bf_lo(uy[j]), y1 = bf_hi(uy[j]);
    rope_turn(x0, y0, cs[2 * j]);
    rope_turn(x1, y1, cs[2 * j + 1]);
    ux[j] = bf_pack(x0, x1);
    uy[j] = bf_pack(y0, y1);
  }
}
// the same 16 bytes held by lane (lane ^ 32)
__device__ __forceinline__ u32x4 lane32_swap(u32x4 u) {
  u32x4 r;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    auto t = __builtin_amdgcn_permlane32_swap(u[j], u[j], false, false);
    r[j] = (__builtin_amdgcn_workitem_id_x() & 32) ? t[0] : t[1];
  }
  return r;
}

// Key and value row of position `j` (< prior) of sequence `seq` for KV head `h` in the pool.
template <typename T>
__device__ __forceinline__ void pool_rows(const LayerView &L, int32_t seq, int32_t h, int64_t j,
                                          const T *&krow, const T *&vrow) {
  const int64_t d = L.d;
  if (!L.is_full) {
    const T *ring = reinterpret_cast<const T *>(L.ring_base + (int64_t)seq * L.ring_seq_stride);
    const int64_t slot = j % L.w;
    krow = ring + ((int64_t)h * L.w + slot) * d;
    vrow = ring + ((int64_t)L.hkv * L.w + (int64_t)h * L.w + slot) * d;
  } else {
    const int32_t page = L.tables[(int64_t)seq * L.table_stride + (j >> 4)];
    const T *pb = reinterpret_cast<const T *>(L.page_base) + (int64_t)page * (2LL * L.hkv * kPageTokens * d);
    const int64_t r = j & (kPageTokens - 1);
    krow = pb + ((int64_t)h * kPageTokens + r) * d;
    vrow = pb + ((int64_t)L.hkv * kPageTokens + (int64_t)h * kPageTokens + r) * d;
  }
}

}  // namespace swa
