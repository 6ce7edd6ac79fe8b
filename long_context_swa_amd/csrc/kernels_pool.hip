// Pool kernels: commit of new tokens into the rings / pages (plain copies, or E4M3 quantisation
// for FP8 pools), and the copies behind a fork.
//
// Commit ([SWA-theory] §Rolling Buffer KV Cache, Eq.(7)): the token at position p goes to ring
// slot p mod w of an SWA layer, or to row p % 16 of page table[p / 16] of a full layer.  Each
// thread moves one 16-byte piece of one (token, KV head) row of K and the same piece of V; lanes
// of a wave cover consecutive pieces, so reads and writes are contiguous runs of d elements.
// Fused-RoPE pools receive unrotated keys and turn them here, at their positions, as they store.

#include "dev_common.h"

namespace swa {

// The K pieces (16 bytes: 8 bf16) a commit thread stores for piece c of a row of cpr pieces at
// position p: piece c as passed, or, for fused-RoPE pools, rotated at p (pairs layout: pairs
// 4c .. 4c+3 inside the piece; halves layout: the thread with c < cpr/2 turns pairs 8c .. 8c+7,
// whose coordinates sit in pieces c and c + cpr/2, and stores both; the other thread stores no K).
// Returns the number of pieces; their indices go to pc, their values to val.
__device__ __forceinline__ int commit_k_pieces(const LayerView &L, const char *krow, int c, int cpr, int64_t p,
                                               int (&pc)[2], u32x4 (&val)[2]) {
  pc[0] = c;
  val[0] = *reinterpret_cast<const u32x4 *>(krow + 16 * c);
  if (!L.rope_fused) return 1;
  if (L.rope_style == 0) {
    val[0] = rope_pairs8(val[0], L.rope_lo, L.rope_hi, L.d / 2, p, 4 * c);
    return 1;
  }
  if (c >= cpr / 2) return 0;
  pc[1] = c + cpr / 2;
  val[1] = *reinterpret_cast<const u32x4 *>(krow + 16 * pc[1]);
  rope_halves8(val[0], val[1], L.rope_lo, L.rope_hi, L.d / 2, p, 8 * c);
  return 2;
}

template <int ES>
__global__ void __launch_bounds__(256) append_kernel(LayerView L, int32_t seq, const char *__restrict__ k,
                                                     const char *__restrict__ v, int32_t row0,
                                                     int32_t n_write, int64_t pos0) {
  const int cpr = L.d * ES / 16;  // 16-byte pieces per row
  const int64_t total = (int64_t)n_write * L.hkv * cpr;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= total) return;
  const int c = (int)(idx % cpr);
  const int64_t rest = idx / cpr;
  const int h = (int)(rest % L.hkv);
  const int64_t t = rest / L.hkv;
  const int64_t p = pos0 + row0 + t;
  const int64_t row_bytes = (int64_t)L.d * ES;
  const int64_t src = ((row0 + t) * L.hkv + h) * row_bytes + 16 * c;
  char *kd, *vd;
  if (!L.is_full) {
    char *ring = L.ring_base + (int64_t)seq * L.ring_seq_stride;
    const int64_t slot = p % L.w;
    kd = ring + ((int64_t)h * L.w + slot) * row_bytes;
    vd = ring + ((int64_t)L.hkv * L.w + (int64_t)h * L.w + slot) * row_bytes;
  } else {
    const int32_t page = L.tables[(int64_t)seq * L.table_stride + (p >> 4)];
    char *pb = L.page_base + (int64_t)page * (2LL * L.hkv * kPageTokens * row_bytes);
    const int64_t r = p & (kPageTokens - 1);
    kd = pb + ((int64_t)h * kPageTokens + r) * row_bytes;
    vd = pb + ((int64_t)L.hkv * kPageTokens + (int64_t)h * kPageTokens + r) * row_bytes;
  }
  if (ES == 2) {  // fused RoPE pools are bf16 or FP8
    int pc[2];
    u32x4 kv[2];
    const int np = commit_k_pieces(L, k + src - 16 * c, c, cpr, p, pc, kv);
    for (int i = 0; i < np; ++i) *reinterpret_cast<u32x4 *>(kd + 16 * pc[i]) = kv[i];
  } else {
    *reinterpret_cast<uint4 *>(kd + 16 * c) = *reinterpret_cast<const uint4 *>(k + src);
  }
  *reinterpret_cast<uint4 *>(vd + 16 * c) = *reinterpret_cast<const uint4 *>(v + src);
}

template <int ES>
__global__ void __launch_bounds__(256) append_batch_kernel(LayerView L, const SeqEntry *__restrict__ ent,
                                                           int32_t n_seqs, const char *__restrict__ k,
                                                           const char *__restrict__ v, int32_t n,
                                                           int32_t row0, int32_t n_write) {
  const int cpr = L.d * ES / 16;
  const int64_t per_seq = (int64_t)n_write * L.hkv * cpr;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= per_seq * n_seqs) return;
  const int si = (int)(idx / per_seq);
  const int64_t r = idx - (int64_t)si * per_seq;
  const int c = (int)(r % cpr);
  const int h = (int)((r / cpr) % L.hkv);
  const int64_t t = r / ((int64_t)cpr * L.hkv);
  const int32_t seq = ent[si].seq;
  const int64_t p = ent[si].prior + row0 + t;
  const int64_t row_bytes = (int64_t)L.d * ES;
  const int64_t src = (((int64_t)si * n + row0 + t) * L.hkv + h) * row_bytes + 16 * c;
  char *kd, *vd;
  if (!L.is_full) {
    char *ring = L.ring_base + (int64_t)seq * L.ring_seq_stride;
    const int64_t slot = p % L.w;
    kd = ring + ((int64_t)h * L.w + slot) * row_bytes;
    vd = ring + ((int64_t)L.hkv * L.w + (int64_t)h * L.w + slot) * row_bytes;
  } else {
    const int32_t page = L.tables[(int64_t)seq * L.table_stride + (p >> 4)];
    char *pb = L.page_base + (int64_t)page * (2LL * L.hkv * kPageTokens * row_bytes);
    const int64_t rr = p & (kPageTokens - 1);
    kd = pb + ((int64_t)h * kPageTokens + rr) * row_bytes;
    vd = pb + ((int64_t)L.hkv * kPageTokens + (int64_t)h * kPageTokens + rr) * row_bytes;
  }
  if (ES == 2) {  // fused RoPE pools are bf16 or FP8
    int pc[2];
    u32x4 kv[2];
    const int np = commit_k_pieces(L, k + src - 16 * c, c, cpr, p, pc, kv);
    for (int i = 0; i < np; ++i) *reinterpret_cast<u32x4 *>(kd + 16 * pc[i]) = kv[i];
  } else {
    *reinterpret_cast<uint4 *>(kd + 16 * c) = *reinterpret_cast<const uint4 *>(k + src);
  }
  *reinterpret_cast<uint4 *>(vd + 16 * c) = *reinterpret_cast<const uint4 *>(v + src);
}

// ---- FP8 pools.  Each thread quantises one 16-byte piece (8 bf16 elements) of a (token, KV head)
// row into 8 E4M3 codes: x * inv_scale (exact, a power of two), clamped to +-448, then rounded to
// the nearest code with ties to even (v_cvt_pk_fp8_f32), so out-of-range values saturate.  A NaN
// input is stored as the code 0x7F (S.1111.111 with S = 0, the format's NaN), whatever its sign:
// the clamp alone would turn it into -448.
__device__ __forceinline__ uint2 quant8_e4m3(u32x4 in, float inv) {
  uint32_t w[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    float y[4];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const uint32_t u = in[2 * h + j];
      y[2 * j] = __uint_as_float(u << 16) * inv;
      y[2 * j + 1] = __uint_as_float(u & 0xffff0000u) * inv;
    }
    uint32_t nan_bytes = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      nan_bytes |= (y[j] != y[j]) ? 0xffu << (8 * j) : 0u;
      y[j] = fminf(fmaxf(y[j], -448.f), 448.f);
    }
    int r = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);  // bytes 0, 1
    r = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], r, true);       // bytes 2, 3
    w[h] = ((uint32_t)r & ~nan_bytes) | (0x7f7f7f7fu & nan_bytes);
  }
  return make_uint2(w[0], w[1]);
}

// destination rows of position p, KV head h in the pool (K row; V row is `vshift` bytes further)
__device__ __forceinline__ char *fp8_row(const LayerView &L, int32_t seq, int64_t p, int h) {
  const int64_t row_bytes = L.d;  // 1 byte per element
  if (!L.is_full) {
    char *ring = L.ring_base + (int64_t)seq * L.ring_seq_stride;
    return ring + ((int64_t)h * L.w + p % L.w) * row_bytes;
  }
  const int32_t page = L.tables[(int64_t)seq * L.table_stride + (p >> 4)];
  char *pb = L.page_base + (int64_t)page * (2LL * L.hkv * kPageTokens * row_bytes);
  return pb + ((int64_t)h * kPageTokens + (p & (kPageTokens - 1))) * row_bytes;
}

__global__ void __launch_bounds__(256) append_fp8_kernel(LayerView L, int32_t seq, const char *__restrict__ k,
                                                         const char *__restrict__ v, int32_t row0,
                                                         int32_t n_write, int64_t pos0) {
  const int cpr = L.d / 8;  // 16-byte bf16 input pieces per row
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (int64_t)n_write * L.hkv * cpr) return;
  const int c = (int)(idx % cpr);
  const int64_t rest = idx / cpr;
  const int h = (int)(rest % L.hkv);
  const int64_t t = rest / L.hkv;
  const int64_t src = ((row0 + t) * L.hkv + h) * (int64_t)L.d * 2 + 16 * c;
  const int64_t vshift = L.is_full ? (int64_t)L.hkv * kPageTokens * L.d : (int64_t)L.hkv * L.w * L.d;
  const int64_t p = pos0 + row0 + t;
  char *kd = fp8_row(L, seq, p, h);
  int pc[2];
  u32x4 kv[2];
  const int np = commit_k_pieces(L, k + src - 16 * c, c, cpr, p, pc, kv);
  for (int i = 0; i < np; ++i) *reinterpret_cast<uint2 *>(kd + 8 * pc[i]) = quant8_e4m3(kv[i], L.k_inv);
  *reinterpret_cast<uint2 *>(kd + vshift + 8 * c) = quant8_e4m3(*reinterpret_cast<const u32x4 *>(v + src), L.v_inv);
}

__global__ void __launch_bounds__(256) append_batch_fp8_kernel(LayerView L, const SeqEntry *__restrict__ ent,
                                                               int32_t n_seqs, const char *__restrict__ k,
                                                               const char *__restrict__ v, int32_t n,
                                                               int32_t row0, int32_t n_write) {
  const int cpr = L.d / 8;
  const int64_t per_seq = (int64_t)n_write * L.hkv * cpr;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= per_seq * n_seqs) return;
  const int si = (int)(idx / per_seq);
  const int64_t r = idx - (int64_t)si * per_seq;
  const int c = (int)(r % cpr);
  const int h = (int)((r / cpr) % L.hkv);
  const int64_t t = r / ((int64_t)cpr * L.hkv);
  const int64_t src = (((int64_t)si * n + row0 + t) * L.hkv + h) * (int64_t)L.d * 2 + 16 * c;
  const int64_t vshift = L.is_full ? (int64_t)L.hkv * kPageTokens * L.d : (int64_t)L.hkv * L.w * L.d;
  const int64_t p = ent[si].prior + row0 + t;
  char *kd = fp8_row(L, ent[si].seq, p, h);
  int pc[2];
  u32x4 kv[2];
  const int np = commit_k_pieces(L, k + src - 16 * c, c, cpr, p, pc, kv);
  for (int i = 0; i < np; ++i) *reinterpret_cast<uint2 *>(kd + 8 * pc[i]) = quant8_e4m3(kv[i], L.k_inv);
  *reinterpret_cast<uint2 *>(kd + vshift + 8 * c) = quant8_e4m3(*reinterpret_cast<const u32x4 *>(v + src), L.v_inv);
}

__global__ void __launch_bounds__(256) table_patch_kernel(int32_t *tables, const TablePatch *patches, int32_t n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) tables[patches[i].index] = patches[i].value;
}

__global__ void __launch_bounds__(256) copy_list_kernel(char *arena, CopyList jobs) {
  const CopyJob j = jobs.job[blockIdx.y];
  const int64_t n16 = j.bytes / 16;
  const uint4 *src = reinterpret_cast<const uint4 *>(arena + j.src_off);
  uint4 *dst = reinterpret_cast<uint4 *>(arena + j.dst_off);
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += (int64_t)gridDim.x * 256)
    dst[i] = src[i];
}

// Clock measurement aid: one lane reads the shader-clock counter (s_memtime) and the fixed-rate
// wall clock (s_memrealtime) before and after sleeping until `ticks` wall-clock ticks have passed;
// the ratio of the two differences times the wall clock's rate is the shader clock over that span.
// out[0..1] shader clock at start / end, out[2..3] wall clock at start / end, out[4] wall rate (kHz).
__global__ void __launch_bounds__(64) clock_probe_kernel(int64_t *out, int64_t ticks, int64_t wall_khz) {
  if (__builtin_amdgcn_workitem_id_x() != 0) return;
  const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
  const uint64_t t0 = __builtin_amdgcn_s_memtime();
  uint64_t r = r0;
  while ((int64_t)(r - r0) < ticks) {  // ends: the wall clock only advances
    __builtin_amdgcn_s_sleep(8);
    r = __builtin_amdgcn_s_memrealtime();
  }
  const uint64_t t1 = __builtin_amdgcn_s_memtime();
  out[0] = (int64_t)t0;
  out[1] = (int64_t)t1;
  out[2] = (int64_t)r0;
  out[3] = (int64_t)r;
  out[4] = wall_khz;
}

hipError_t launch_append(const LayerView &L, int32_t seq, const void *k, const void *v,
                         int32_t src_row0, int32_t n_write, int64_t pos0, int es, hipStream_t s) {
  const int64_t total = (int64_t)n_write * L.hkv * (L.d * es / 16);
  const int64_t blocks = (total + 255) / 256;
  if (blocks == 0) return hipSuccess;
  if (L.kv_fp8) {
    if (es != 2) return hipErrorInvalidValue;
    hipLaunchKernelGGL(append_fp8_kernel, dim3((unsigned)blocks), dim3(256), 0, s, L, seq,
                       static_cast<const char *>(k), static_cast<const char *>(v), src_row0, n_write, pos0);
    return hipGetLastError();
  }
  if (es == 2)
    hipLaunchKernelGGL(append_kernel<2>, dim3((unsigned)blocks), dim3(256), 0, s, L, seq,
                       static_cast<const char *>(k), static_cast<const char *>(v), src_row0, n_write, pos0);
  else
    hipLaunchKernelGGL(append_kernel<4>, dim3((unsigned)blocks), dim3(256), 0, s, L, seq,
                       static_cast<const char *>(k), static_cast<const char *>(v), src_row0, n_write, pos0);
  return hipGetLastError();
}

hipError_t launch_append_batch(const LayerView &L, const SeqEntry *entries, int32_t n_seqs, const void *k,
                               const void *v, int32_t n, int32_t src_row0, int32_t n_write, int es,
                               hipStream_t s) {
  const int64_t total = (int64_t)n_seqs * n_write * L.hkv * (L.d * es / 16);
  const int64_t blocks = (total + 255) / 256;
  if (blocks == 0) return hipSuccess;
  if (L.kv_fp8) {
    if (es != 2) return hipErrorInvalidValue;
    hipLaunchKernelGGL(append_batch_fp8_kernel, dim3((unsigned)blocks), dim3(256), 0, s, L, entries, n_seqs,
                       static_cast<const char *>(k), static_cast<const char *>(v), n, src_row0, n_write);
    return hipGetLastError();
  }
  if (es == 2)
    hipLaunchKernelGGL(append_batch_kernel<2>, dim3((unsigned)blocks), dim3(256), 0, s, L, entries, n_seqs,
                       static_cast<const char *>(k), static_cast<const char *>(v), n, src_row0, n_write);
  else
    hipLaunchKernelGGL(append_batch_kernel<4>, dim3((unsigned)blocks), dim3(256), 0, s, L, entries, n_seqs,
                       static_cast<const char *>(k), static_cast<const char *>(v), n, src_row0, n_write);
  return hipGetLastError();
}

hipError_t launch_table_patch(int32_t *tables, const TablePatch *patches, int32_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(table_patch_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, tables, patches, n);
  return hipGetLastError();
}

hipError_t launch_copy_list(char *arena, const CopyList &jobs, hipStream_t s) {
  if (jobs.n == 0) return hipSuccess;
  int64_t mx = 0;
  for (int i = 0; i < jobs.n; ++i) mx = jobs.job[i].bytes > mx ? jobs.job[i].bytes : mx;
  int64_t bx = (mx / 16 + 255) / 256;
  if (bx > 1024) bx = 1024;
  if (bx < 1) bx = 1;
  hipLaunchKernelGGL(copy_list_kernel, dim3((unsigned)bx, (unsigned)jobs.n), dim3(256), 0, s, arena, jobs);
  return hipGetLastError();
}

hipError_t launch_clock_probe(int64_t *out, int64_t ticks, int64_t wall_khz, hipStream_t s) {
  hipLaunchKernelGGL(clock_probe_kernel, dim3(1), dim3(64), 0, s, out, ticks, wall_khz);
  return hipGetLastError();
}

}  // namespace swa
