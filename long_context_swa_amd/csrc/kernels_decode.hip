// bf16 decode / multi-token verify over the pool, split over keys, then a log-sum-exp merge.
//
// Each work item is (sequence, KV head, range of prior keys): an SWA item walks the ring's w slots
// ([SWA-theory] §Rolling Buffer KV Cache, Eq.(7)); a full-layer item walks a range of pages.  The
// item's query rows are the G query heads of that KV head times q_len new positions (<= 32 rows),
// so every K/V byte read from HBM serves all of them.  Rows at position L+t see pool keys with
// position >= L+t-w+1 (SWA; the one stale slot, position L-w, is masked by position) or all of
// them (full), plus the new tokens L..L+t passed with the call ([SWA-theory] Eq.(1)).
//
// A wave owns one item: S^T = K·Q^T (32 keys x 32 rows) on v_mfma_f32_32x32x16_bf16 with K loaded
// straight from HBM into A-operand registers (16 contiguous bytes per lane), online softmax in
// fp32, and O^T += V^T·P^T with V staged row-major in the wave's LDS slice and read back
// transposed (ds_read_b64_tr_b16).  The next 32 keys are loaded while the current ones compute.
// Items that cover a whole row write normalised bf16 output; split rows write (m, l, o) partials
// that the combine kernel merges:  o = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s,  which is
// the same softmax (Eq.(4)-(5)) regrouped.

#include "dev_common.h"

namespace swa {

namespace {

constexpr int WAVES = 4;
constexpr int KSTEP = 32;

template <int D, bool FULL>
__global__ void __launch_bounds__(64 * WAVES, 1) decode_bf16_kernel(const DecodeArgs a) {
  constexpr int VS = D + 16;          // LDS row stride (elements)
  constexpr int NC = D / 16;          // S^T k-steps over d
  constexpr int ND = D / 32;          // O^T d-blocks
  constexpr int VP = KSTEP * D / 8 / 64;  // 16-byte V pieces per lane per step
  __shared__ __attribute__((aligned(16))) uint16_t vsm[WAVES][KSTEP * VS];

  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int idx = blockIdx.x * WAVES + wv;
  if (idx >= a.n_items) return;
  const WorkItem it = a.items[idx];
  const SeqEntry se = a.seqs[it.si];
  const LayerView &L = a.L;
  const int hkv = L.hkv, W = L.w;
  const int G = a.hq / hkv, ql = a.q_len, rows = G * ql;
  const int64_t Lp = se.prior;
  const int seq = se.seq, head = it.head;
  uint16_t *vw = vsm[wv];

  const int ncol = lane & 31, hh = lane >> 5;
  const int t = ncol / G, gh = ncol - (ncol / G) * G;
  const bool row_ok = ncol < rows;
  const int64_t qpos = Lp + t;
  const int64_t qrow_idx = ((int64_t)it.si * ql + t) * a.hq + head * G + gh;

  bf16x8 qf[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    if (row_ok) qf[c] = *reinterpret_cast<const bf16x8 *>(a.q + qrow_idx * D + 16 * c + 8 * hh);
    else qf[c] = bf16x8{};
  }

  const uint16_t *ring = nullptr;
  if (!FULL) ring = reinterpret_cast<const uint16_t *>(L.ring_base + (int64_t)seq * L.ring_seq_stride);
  const int32_t *table = FULL ? L.tables + (int64_t)seq * L.table_stride : nullptr;
  const uint16_t *pages = FULL ? reinterpret_cast<const uint16_t *>(L.page_base) : nullptr;

  // steps: prior keys [k_begin, k_end) in chunks of 32 (k_begin is page-aligned for full
  // layers, so a step spans exactly two pages), then (if with_new) one step of new keys
  const int64_t kb0 = it.k_begin, kb1 = it.k_end;
  const int n_prior_steps = (int)((kb1 - kb0 + KSTEP - 1) / KSTEP);
  const int n_steps = n_prior_steps + (it.with_new ? 1 : 0);

  // Base of key row 0 of the step's 16-key group `grp` (K); V rows are `voff` elements further.
  // Key r of the group is at base + r * D.
  const int64_t voff = FULL ? (int64_t)hkv * kPageTokens * D : (int64_t)hkv * W * D;
  auto group_base = [&](int st, int grp) -> const uint16_t * {
    const int64_t k0 = kb0 + (int64_t)st * KSTEP + 16 * grp;
    if (FULL) {
      const int64_t pi = k0 >> 4;
      const int32_t page = (k0 < kb1) ? table[pi] : 0;
      return pages + (int64_t)page * (2LL * hkv * kPageTokens * D) + (int64_t)head * kPageTokens * D;
    }
    return ring + ((int64_t)head * W + k0) * D;
  };

  bf16x8 kreg[NC];
  u32x4 vreg[VP];
  auto load_step = [&](int st) {
    const bool is_new = st >= n_prior_steps;
    const uint16_t *gb0, *gb1;
    int nvalid;  // keys of this step that exist
    if (!is_new) {
      gb0 = group_base(st, 0);
      gb1 = group_base(st, 1);
      const int64_t left = kb1 - (kb0 + (int64_t)st * KSTEP);
      nvalid = left < KSTEP ? (int)left : KSTEP;
    } else {
      gb0 = gb1 = a.k_new + ((int64_t)it.si * ql * hkv + head) * D;
      nvalid = ql;
    }
    // row pointer of key `key` of the step (K); V is voff further (pool) or in v_new (new keys)
    auto krow = [&](int key) -> const uint16_t * {
      if (is_new) return gb0 + (int64_t)key * hkv * D;
      return (key < 16 ? gb0 : gb1) + (int64_t)(key & 15) * D;
    };
    auto vrow = [&](int key) -> const uint16_t * {
      if (is_new) return a.v_new + ((int64_t)(it.si * ql + key) * hkv + head) * D;
      return (key < 16 ? gb0 : gb1) + voff + (int64_t)(key & 15) * D;
    };
    if (ncol < nvalid) {
      const uint16_t *kr = krow(ncol);
#pragma unroll
      for (int c = 0; c < NC; ++c) kreg[c] = *reinterpret_cast<const bf16x8 *>(kr + 16 * c + 8 * hh);
    } else {
#pragma unroll
      for (int c = 0; c < NC; ++c) kreg[c] = bf16x8{};
    }
#pragma unroll
    for (int i = 0; i < VP; ++i) {
      const int pc = lane + 64 * i;
      const int key = pc / (D / 8), col = pc % (D / 8);
      u32x4 vv = {0, 0, 0, 0};
      if (key < nvalid) vv = *reinterpret_cast<const u32x4 *>(vrow(key) + 8 * col);
      vreg[i] = vv;
    }
  };

  f32x16 o[ND];
#pragma unroll
  for (int db = 0; db < ND; ++db) o[db] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;
  const float c2 = a.scale_log2;
  const int g16 = lane >> 4, s16 = lane & 15;

  if (n_steps > 0) load_step(0);
  for (int st = 0; st < n_steps; ++st) {
    // stage this step's V in the wave's LDS slice
#pragma unroll
    for (int i = 0; i < VP; ++i) {
      const int pc = lane + 64 * i;
      const int key = pc / (D / 8), col = pc % (D / 8);
      *reinterpret_cast<u32x4 *>(&vw[key * VS + 8 * col]) = vreg[i];
    }
    f32x16 s = f32x16{};
#pragma unroll
    for (int c = 0; c < NC; ++c) s = mfma32(kreg[c], qf[c], s);
    // the next step's loads overlap this step's softmax and PV work
    if (st + 1 < n_steps) load_step(st + 1);

    // mask: S^T row (key) 8*(rr/4) + 4*hh + rr%4 of the step against this lane's query
    const bool is_new = st >= n_prior_steps;
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) {
      const int key = 8 * (rr >> 2) + 4 * hh + (rr & 3);
      bool ok = row_ok;
      if (!is_new) {
        const int64_t kidx = kb0 + (int64_t)st * KSTEP + key;
        ok = ok && kidx < kb1;
        if (!FULL) {
          // slot kidx holds the latest position p = kidx (mod W) with p < Lp
          const int64_t p = Lp - 1 - ((Lp - 1 - kidx) % W);
          ok = ok && p > qpos - W;
        }
      } else {
        ok = ok && key <= t && (FULL || key > t - W);
      }
      if (!ok) s[rr] = -INFINITY;
    }

    float mx = -INFINITY;
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) mx = fmaxf(mx, s[rr]);
    mx = fmaxf(mx, other_half(mx));
    const float m_new = fmaxf(m_run, mx);
    if (__builtin_amdgcn_ballot_w64(m_new > m_run) != 0) {
      const float alpha = m_new > m_run ? exp2_fast((m_run - m_new) * c2) : 1.f;
#pragma unroll
      for (int db = 0; db < ND; ++db) o[db] *= alpha;
      l_run *= alpha;
      m_run = m_new;
    }
    const float msc = (m_run == -INFINITY) ? 0.f : m_run * c2;
    bf16x8 pf[2];
    float lsum = 0.f;
#pragma unroll
    for (int half = 0; half < 2; ++half)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float p = exp2_fast(fmaf(s[8 * half + e], c2, -msc));
        lsum += p;
        pf[half][e] = (__bf16)p;
      }
    l_run += lsum;

#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const uint16_t *vp = &vw[(16 * k + 4 * hh + (s16 >> 2)) * VS + 16 * (g16 & 1) + 4 * (s16 & 3)];
#pragma unroll
      for (int db = 0; db < ND; ++db) {
        const bf16x4 lo = lds_read_tr(vp + 32 * db);
        const bf16x4 hi = lds_read_tr(vp + 8 * VS + 32 * db);
        o[db] = mfma32(cat(lo, hi), pf[k], o[db]);
      }
    }
  }

  const float l_tot = l_run + other_half(l_run);
  if (!row_ok) return;
  if (it.part < 0) {
    const float inv = 1.f / l_tot;
    uint16_t *orow = a.out + qrow_idx * D;
#pragma unroll
    for (int db = 0; db < ND; ++db)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int dd = 32 * db + 8 * q4 + 4 * hh;
        uint2 w;
        w.x = (uint32_t)f2bf(o[db][4 * q4 + 0] * inv) | ((uint32_t)f2bf(o[db][4 * q4 + 1] * inv) << 16);
        w.y = (uint32_t)f2bf(o[db][4 * q4 + 2] * inv) | ((uint32_t)f2bf(o[db][4 * q4 + 3] * inv) << 16);
        *reinterpret_cast<uint2 *>(orow + dd) = w;
      }
  } else {
    const int64_t prow = (int64_t)it.part * rows + ncol;
    float *po = a.part_o + prow * D;
#pragma unroll
    for (int db = 0; db < ND; ++db)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int dd = 32 * db + 8 * q4 + 4 * hh;
        *reinterpret_cast<float4 *>(po + dd) =
            make_float4(o[db][4 * q4 + 0], o[db][4 * q4 + 1], o[db][4 * q4 + 2], o[db][4 * q4 + 3]);
      }
    if (hh == 0) {
      a.part_ml[prow * 2 + 0] = (m_run == -INFINITY) ? -INFINITY : m_run * c2;
      a.part_ml[prow * 2 + 1] = l_tot;
    }
  }
}

// Merge the partials of every split (sequence, KV head, query row): one workgroup per row.  The
// row's reference max M over the partials is found by a block reduction; then thread dd sums
// 2^(m_s - M) o_s[dd] and 2^(m_s - M) l_s over the partials (coalesced over dd).
template <int D>
__global__ void __launch_bounds__(256) combine_kernel(const DecodeArgs a) {
  const int hkv = a.L.hkv;
  const int G = a.hq / hkv, ql = a.q_len, rows = G * ql;
  const int pair = blockIdx.x / rows, n = blockIdx.x % rows;
  const int si = pair / hkv, head = pair % hkv;
  const CombineEntry ce = a.combine[pair];
  if (ce.count == 0) return;
  __shared__ float red[256];
  float M = -INFINITY;
  for (int s = threadIdx.x; s < ce.count; s += 256)
    M = fmaxf(M, a.part_ml[((int64_t)(ce.first + s) * rows + n) * 2]);
  red[threadIdx.x] = M;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (threadIdx.x < o) red[threadIdx.x] = fmaxf(red[threadIdx.x], red[threadIdx.x + o]);
    __syncthreads();
  }
  M = red[0];
  // threads [0, D) own one output dim each; with D < 256 the other threads split the partials
  constexpr int SPLIT = 256 / D;
  const int dd = threadIdx.x % D, part = threadIdx.x / D;
  float num = 0.f, den = 0.f;
  for (int s = part; s < ce.count; s += SPLIT) {
    const int64_t pr = (int64_t)(ce.first + s) * rows + n;
    const float ms = a.part_ml[pr * 2];
    const float f = ms == -INFINITY ? 0.f : exp2_fast(ms - M);
    num = fmaf(f, a.part_o[pr * D + dd], num);
    den = fmaf(f, a.part_ml[pr * 2 + 1], den);
  }
  __shared__ float nsum[256], dsum[256];
  nsum[threadIdx.x] = num;
  dsum[threadIdx.x] = den;
  __syncthreads();
  if (threadIdx.x < D) {
    for (int k = 1; k < SPLIT; ++k) {
      num += nsum[threadIdx.x + k * D];
      den += dsum[threadIdx.x + k * D];
    }
    const int t = n / G, gh = n % G;
    const int64_t qrow_idx = ((int64_t)si * ql + t) * a.hq + head * G + gh;
    a.out[qrow_idx * D + dd] = f2bf(num / den);
  }
}

}  // namespace

hipError_t launch_decode_bf16(const DecodeArgs &a, hipStream_t s) {
  if (a.hq / a.L.hkv * a.q_len > 32) return hipErrorInvalidValue;
  if (a.n_items > 0) {
    const dim3 grid((unsigned)((a.n_items + WAVES - 1) / WAVES)), block(64 * WAVES);
    if (a.L.d == 128) {
      if (a.L.is_full) hipLaunchKernelGGL((decode_bf16_kernel<128, true>), grid, block, 0, s, a);
      else hipLaunchKernelGGL((decode_bf16_kernel<128, false>), grid, block, 0, s, a);
    } else {
      if (a.L.is_full) hipLaunchKernelGGL((decode_bf16_kernel<64, true>), grid, block, 0, s, a);
      else hipLaunchKernelGGL((decode_bf16_kernel<64, false>), grid, block, 0, s, a);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (a.n_parts > 0) {
    const int rows = a.hq / a.L.hkv * a.q_len;
    const dim3 grid((unsigned)(a.n_seqs * a.L.hkv * rows)), block(256);
    if (a.L.d == 128) hipLaunchKernelGGL(combine_kernel<128>, grid, block, 0, s, a);
    else hipLaunchKernelGGL(combine_kernel<64>, grid, block, 0, s, a);
    return hipGetLastError();
  }
  return hipSuccess;
}

}  // namespace swa
