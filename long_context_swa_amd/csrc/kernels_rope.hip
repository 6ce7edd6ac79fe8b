// RoPE (rotary position embedding) of a call's queries and keys, in place, at the positions the
// pool gives them.
//
// RoFormer (Su et al., 2021) §3.2-§3.4: pair i of a head vector is turned by the angle
// p * theta_i at position p, theta_i = base^(-2i/d), as the complex number x + iy times
// e^(i p theta_i).  Pair i is coordinates (2i, 2i+1) ("pairs") or (i, i + d/2) ("halves").
//
// Angles are never formed in fp32 (p * theta_i loses all accuracy near a million positions).
// The host fills two tables of (cos, sin) in float64 and stores them as fp32: `lo` for angles
// l * theta_i, l < 2048, and `hi` for h * 2048 * theta_i.  A position p = h * 2048 + l turns by the
// product of the two rotations (angle addition), so the kernel's error is a few fp32 ulps.
//
// Each thread rotates four pairs of one (token, head) row: 16 contiguous bytes of a bf16 row in
// the pairs layout, or 8 bytes from each half in the halves layout, so lanes of a wave cover
// contiguous runs of a row.  Query rows of a token come first, then its key rows; both share the
// token's table entries.

#include "dev_common.h"

namespace swa {

template <int ES, int STYLE>
__global__ void __launch_bounds__(256) rope_kernel(RopeArgs a) {
  const int cpr = a.d / 8;  // threads per row: 4 pairs each
  const int heads = a.hq + a.hkv;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (int64_t)a.tokens * heads * cpr) return;
  const int c = (int)(idx % cpr);
  const int64_t rest = idx / cpr;
  const int h = (int)(rest % heads);
  const int64_t tok = rest / heads;
  const int64_t p = (a.ent ? a.ent[tok / a.n].prior : a.pos0) + tok % a.n;
  char *row = h < a.hq ? a.q + ((tok * a.hq + h) * a.d) * ES : a.k + ((tok * a.hkv + (h - a.hq)) * a.d) * ES;

  // angle tables: pairs 4c .. 4c+3 of the position's two parts
  const int half = a.d / 2;
  const float4 *lt = reinterpret_cast<const float4 *>(a.lo_tab + (p & (kRopeLo - 1)) * half + 4 * c);
  const float4 *ht = reinterpret_cast<const float4 *>(a.hi_tab + (p >> kRopeLoBits) * half + 4 * c);
  const float4 l01 = lt[0], l23 = lt[1], h01 = ht[0], h23 = ht[1];
  const float lc[4] = {l01.x, l01.z, l23.x, l23.z}, ls[4] = {l01.y, l01.w, l23.y, l23.w};
  const float hc[4] = {h01.x, h01.z, h23.x, h23.z}, hs[4] = {h01.y, h01.w, h23.y, h23.w};

  // the four pairs (x_j, y_j)
  float x[4], y[4];
  char *px, *py;  // pairs: one 16/32-byte piece; halves: a piece in each half
  if (STYLE == 0) {
    px = row + 8 * c * ES;
    py = px;
  } else {
    px = row + 4 * c * ES;
    py = row + (half + 4 * c) * ES;
  }
  if (ES == 2) {
    if (STYLE == 0) {
      const u32x4 u = *reinterpret_cast<const u32x4 *>(px);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        x[j] = __uint_as_float(u[j] << 16);
        y[j] = __uint_as_float(u[j] & 0xffff0000u);
      }
    } else {
      const uint2 ux = *reinterpret_cast<const uint2 *>(px), uy = *reinterpret_cast<const uint2 *>(py);
      const uint32_t wx[2] = {ux.x, ux.y}, wy[2] = {uy.x, uy.y};
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        x[2 * j] = __uint_as_float(wx[j] << 16);
        x[2 * j + 1] = __uint_as_float(wx[j] & 0xffff0000u);
        y[2 * j] = __uint_as_float(wy[j] << 16);
        y[2 * j + 1] = __uint_as_float(wy[j] & 0xffff0000u);
      }
    }
  } else {
    if (STYLE == 0) {
      const float4 f0 = reinterpret_cast<const float4 *>(px)[0], f1 = reinterpret_cast<const float4 *>(px)[1];
      x[0] = f0.x; y[0] = f0.y; x[1] = f0.z; y[1] = f0.w;
      x[2] = f1.x; y[2] = f1.y; x[3] = f1.z; y[3] = f1.w;
    } else {
      const float4 fx = *reinterpret_cast<const float4 *>(px), fy = *reinterpret_cast<const float4 *>(py);
      x[0] = fx.x; x[1] = fx.y; x[2] = fx.z; x[3] = fx.w;
      y[0] = fy.x; y[1] = fy.y; y[2] = fy.z; y[3] = fy.w;
    }
  }

  float ox[4], oy[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    // rotation by (h * 2048 + l) * theta = rotation by h * 2048 * theta, then by l * theta
    const float cs = fmaf(hc[j], lc[j], -hs[j] * ls[j]);
    const float sn = fmaf(hs[j], lc[j], hc[j] * ls[j]);
    ox[j] = fmaf(x[j], cs, -y[j] * sn);
    oy[j] = fmaf(x[j], sn, y[j] * cs);
  }

  if (ES == 2) {
    if (STYLE == 0) {
      u32x4 u;
#pragma unroll
      for (int j = 0; j < 4; ++j) u[j] = (uint32_t)f2bf(ox[j]) | ((uint32_t)f2bf(oy[j]) << 16);
      *reinterpret_cast<u32x4 *>(px) = u;
    } else {
      uint2 ux, uy;
      ux.x = (uint32_t)f2bf(ox[0]) | ((uint32_t)f2bf(ox[1]) << 16);
      ux.y = (uint32_t)f2bf(ox[2]) | ((uint32_t)f2bf(ox[3]) << 16);
      uy.x = (uint32_t)f2bf(oy[0]) | ((uint32_t)f2bf(oy[1]) << 16);
      uy.y = (uint32_t)f2bf(oy[2]) | ((uint32_t)f2bf(oy[3]) << 16);
      *reinterpret_cast<uint2 *>(px) = ux;
      *reinterpret_cast<uint2 *>(py) = uy;
    }
  } else {
    if (STYLE == 0) {
      reinterpret_cast<float4 *>(px)[0] = make_float4(ox[0], oy[0], ox[1], oy[1]);
      reinterpret_cast<float4 *>(px)[1] = make_float4(ox[2], oy[2], ox[3], oy[3]);
    } else {
      *reinterpret_cast<float4 *>(px) = make_float4(ox[0], ox[1], ox[2], ox[3]);
      *reinterpret_cast<float4 *>(py) = make_float4(oy[0], oy[1], oy[2], oy[3]);
    }
  }
}

hipError_t launch_rope(const RopeArgs &a, int es, hipStream_t s) {
  const int64_t total = (int64_t)a.tokens * (a.hq + a.hkv) * (a.d / 8);
  const int64_t blocks = (total + 255) / 256;
  if (blocks == 0) return hipSuccess;
  if (blocks > INT32_MAX) return hipErrorInvalidValue;
  const dim3 g((unsigned)blocks), b(256);
  if (es == 2) {
    if (a.style == 0) hipLaunchKernelGGL((rope_kernel<2, 0>), g, b, 0, s, a);
    else hipLaunchKernelGGL((rope_kernel<2, 1>), g, b, 0, s, a);
  } else {
    if (a.style == 0) hipLaunchKernelGGL((rope_kernel<4, 0>), g, b, 0, s, a);
    else hipLaunchKernelGGL((rope_kernel<4, 1>), g, b, 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace swa
