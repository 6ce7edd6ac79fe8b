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
// token's table entries.  Rotated keys go back into k, or to a separate buffer (kout: the rotated
// chunk keys a fused-RoPE prefill reads).  The arithmetic is the helpers' in dev_common.h, shared
// with the fused paths.

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
  const bool is_q = h < a.hq;
  const int64_t roff = (is_q ? (tok * a.hq + h) : (tok * a.hkv + (h - a.hq))) * a.d * ES;
  const char *row = (is_q ? a.q : a.k) + roff;
  char *orow = (is_q || !a.kout ? (is_q ? a.q : a.k) : a.kout) + roff;
  const int half = a.d / 2;
  // pairs: one 16-byte (bf16) or 32-byte (fp32) piece holding pairs 4c .. 4c+3 as neighbours;
  // halves: the first and the second coordinates of pairs 4c .. 4c+3, one piece in each half
  const int64_t ox = STYLE == 0 ? 8 * c * ES : 4 * c * ES, oy = STYLE == 0 ? ox : (half + 4 * c) * ES;
  if (ES == 2 && STYLE == 0) {
    const u32x4 u = *reinterpret_cast<const u32x4 *>(row + ox);
    *reinterpret_cast<u32x4 *>(orow + ox) = rope_pairs8(u, a.lo_tab, a.hi_tab, half, p, 4 * c);
    return;
  }
  float2 cs[4];
  rope_angles<4>(a.lo_tab, a.hi_tab, half, p, 4 * c, cs);
  float x[4], y[4];
  if (ES == 2) {
    const uint2 ux = *reinterpret_cast<const uint2 *>(row + ox), uy = *reinterpret_cast<const uint2 *>(row + oy);
    x[0] = bf_lo(ux.x); x[1] = bf_hi(ux.x); x[2] = bf_lo(ux.y); x[3] = bf_hi(ux.y);
    y[0] = bf_lo(uy.x); y[1] = bf_hi(uy.x); y[2] = bf_lo(uy.y); y[3] = bf_hi(uy.y);
  } else if (STYLE == 0) {
    const float4 f0 = reinterpret_cast<const float4 *>(row + ox)[0], f1 = reinterpret_cast<const float4 *>(row + ox)[1];
    x[0] = f0.x; y[0] = f0.y; x[1] = f0.z; y[1] = f0.w;
    x[2] = f1.x; y[2] = f1.y; x[3] = f1.z; y[3] = f1.w;
  } else {
    const float4 fx = *reinterpret_cast<const float4 *>(row + ox), fy = *reinterpret_cast<const float4 *>(row + oy);
    x[0] = fx.x; x[1] = fx.y; x[2] = fx.z; x[3] = fx.w;
    y[0] = fy.x; y[1] = fy.y; y[2] = fy.z; y[3] = fy.w;
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) rope_turn(x[j], y[j], cs[j]);
  if (ES == 2) {
    *reinterpret_cast<uint2 *>(orow + ox) = make_uint2(bf_pack(x[0], x[1]), bf_pack(x[2], x[3]));
    *reinterpret_cast<uint2 *>(orow + oy) = make_uint2(bf_pack(y[0], y[1]), bf_pack(y[2], y[3]));
  } else if (STYLE == 0) {
    reinterpret_cast<float4 *>(orow + ox)[0] = make_float4(x[0], y[0], x[1], y[1]);
    reinterpret_cast<float4 *>(orow + ox)[1] = make_float4(x[2], y[2], x[3], y[3]);
  } else {
    *reinterpret_cast<float4 *>(orow + ox) = make_float4(x[0], x[1], x[2], x[3]);
    *reinterpret_cast<float4 *>(orow + oy) = make_float4(y[0], y[1], y[2], y[3]);
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
