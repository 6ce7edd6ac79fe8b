// fp32 attention: one wave per query row (sequence, query, q head), keys 64 at a time, online
// softmax.  Serves fp32 pools for every layer kind and both prefill and decode/verify; the
// small, latency-bound fp32 workloads need no tiling.
//
// Row at absolute position i sees keys W(i) = {max(0, i-w+1) .. i} in an SWA layer and {0 .. i}
// in a full layer ([SWA-theory] §数学的定義 Eq.(1)); score q·k/sqrt(d) (Eq.(3)), softmax (Eq.(4)),
// weighted sum of values (Eq.(5)).  Keys below the committed length come from the pool, the rest
// from the new tokens passed with the call.

#include "dev_common.h"

namespace swa {

__device__ __forceinline__ float wave_max(float x) {
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

__global__ void __launch_bounds__(64) attn_f32_kernel(F32AttnArgs a) {
  const int lane = threadIdx.x;
  const int64_t row = blockIdx.x;
  const int hq = a.hq, ql = a.q_len;
  const int h = (int)(row % hq);
  const int t = (int)((row / hq) % ql);
  const int si = (int)(row / ((int64_t)hq * ql));
  int32_t seq;
  int64_t prior;
  if (a.seqs) { seq = a.seqs[si].seq; prior = a.seqs[si].prior; }
  else { seq = a.seq; prior = a.prior; }
  const LayerView &L = a.L;
  const int d = L.d, hkv = L.hkv;
  const int g = h / (hq / hkv);
  const int64_t i = prior + t;
  const int64_t lo = L.is_full ? 0 : (i - L.w + 1 > 0 ? i - L.w + 1 : 0);

  // pool rows are 16-byte aligned (d is 64 or 128); the call's new-token rows are when its k
  // tensor is (rows are d floats apart)
  const bool vec = (reinterpret_cast<uintptr_t>(a.k_new) & 15) == 0;
  __shared__ __attribute__((aligned(16))) float qs[128];
  __shared__ float ps[64];
  const float *qrow = a.q + (((int64_t)si * ql + t) * hq + h) * d;
  for (int c = lane; c < d; c += 64) qs[c] = qrow[c];
  __syncthreads();

  float m = -INFINITY, l = 0.f, o0 = 0.f, o1 = 0.f;
  const float c2 = a.scale_log2;
  auto rows_of = [&](int64_t j, const float *&kr, const float *&vr) {
    if (j < prior) {
      pool_rows<float>(L, seq, g, j, kr, vr);
    } else {
      const int64_t r = ((int64_t)si * ql + (j - prior)) * hkv + g;
      kr = a.k_new + r * d;
      vr = a.v_new + r * d;
    }
  };
  for (int64_t base = lo; base <= i; base += 64) {
    const int64_t j = base + lane;
    float s = -INFINITY;
    const float *vr = nullptr;  // this lane's key's V row, handed to every lane for the PV sum
    if (j <= i) {
      const float *kr;
      rows_of(j, kr, vr);
      float acc = 0.f;
      if (vec) {  // 16-byte loads of the key row (same fma order as the scalar loop)
        const float4 *k4 = reinterpret_cast<const float4 *>(kr);
        const float4 *q4 = reinterpret_cast<const float4 *>(qs);
#pragma unroll 4
        for (int c = 0; c < d / 4; ++c) {
          const float4 kv = k4[c], qv = q4[c];
          acc = fmaf(qv.x, kv.x, acc);
          acc = fmaf(qv.y, kv.y, acc);
          acc = fmaf(qv.z, kv.z, acc);
          acc = fmaf(qv.w, kv.w, acc);
        }
      } else {
        for (int c = 0; c < d; ++c) acc = fmaf(qs[c], kr[c], acc);
      }
      s = acc * c2;  // log2-domain score
    }
    const float mx = wave_max(s);
    const float mn = fmaxf(m, mx);
    const float alpha = exp2_fast(m - mn);  // m = -inf on the first block: alpha = 0
    const float p = (j <= i) ? exp2_fast(s - mn) : 0.f;
    l = l * alpha + wave_sum(p);
    o0 *= alpha;
    o1 *= alpha;
    m = mn;
    ps[lane] = p;
    __syncthreads();
    const int cnt = (int)((i - base + 1) < 64 ? (i - base + 1) : 64);
    const uint64_t vaddr = reinterpret_cast<uint64_t>(vr);
    const int vlo = (int)(uint32_t)vaddr, vhi = (int)(uint32_t)(vaddr >> 32);
    for (int jj = 0; jj < cnt; ++jj) {  // jj is uniform: the V row address of key base + jj by readlane
      const uint64_t a64 = (uint64_t)(uint32_t)__builtin_amdgcn_readlane(vlo, jj) |
                           ((uint64_t)(uint32_t)__builtin_amdgcn_readlane(vhi, jj) << 32);
      const float *vj = reinterpret_cast<const float *>(a64);
      const float pj = ps[jj];
      o0 = fmaf(pj, vj[lane], o0);
      if (d > 64) o1 = fmaf(pj, vj[lane + 64], o1);
    }
    __syncthreads();
  }
  float *orow = a.out + (((int64_t)si * ql + t) * hq + h) * d;
  const float inv = 1.f / l;
  orow[lane] = o0 * inv;
  if (d > 64) orow[lane + 64] = o1 * inv;
}

hipError_t launch_attn_f32(const F32AttnArgs &a, hipStream_t s) {
  const int64_t rows = (int64_t)a.n_seqs * a.q_len * a.hq;
  if (rows == 0) return hipSuccess;
  hipLaunchKernelGGL(attn_f32_kernel, dim3((unsigned)rows), dim3(64), 0, s, a);
  return hipGetLastError();
}

}  // namespace swa
