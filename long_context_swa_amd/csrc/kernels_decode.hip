// bf16 decode / multi-token verify over the pool, split over keys, then a log-sum-exp merge.
//
// Each work item is (sequence, KV head, range of prior keys).  A full-layer item walks a range of
// pages and runs on one 4-wave workgroup whose waves split the range and merge in LDS; an SWA item
// walks the ring's w slots ([SWA-theory] §Rolling Buffer KV Cache, Eq.(7)) on a single wave, four
// items per workgroup, with no merge, when the call has enough items to fill the chip that way;
// small calls (a single sequence's verify, a few sequences) split each SWA item over a workgroup's
// four waves like a full-layer item, which cuts the serial 32-key steps per wave to about a
// quarter.  The
// item's query rows are the G query heads of that KV head times q_len new positions, 32 of them
// per item, so every K/V byte read from HBM serves up to 32 rows (more rows, up to 128, take
// several items over the same keys, adjacent in the work list so the repeat reads meet L2).  Rows at position L+t see pool keys with
// position >= L+t-w+1 (SWA; the one stale slot, position L-w, is masked by position) or all of
// them (full), plus the new tokens L..L+t passed with the call ([SWA-theory] Eq.(1)).
//
// Per wave: S^T = K·Q^T (32 keys x 32 rows) on v_mfma_f32_32x32x16_bf16 with K loaded
// straight from HBM into A-operand registers (one contiguous half row per lane), online softmax
// in fp32, and O^T += V^T·P^T with V staged row-major in the wave's LDS slice and read back
// transposed (ds_read_b64_tr_b16).  The next 32 keys are loaded while the current ones compute;
// keys past the item's end are clamped onto its last key and masked, so loads never branch.
// Two waves per SIMD keep twice the bytes in flight.
// Items that cover a whole row write normalised bf16 output; split rows write (m, l, o) partials
// that the combine kernel merges:  o = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s,  which is
// the same softmax (Eq.(4)-(5)) regrouped.

#include "dev_common.h"

#include <type_traits>

namespace swa {

namespace {

constexpr int WAVES = 4;
constexpr int KSTEP = 32;

// SWA calls with at most this many items split every item over a workgroup's four waves: the
// split grid (four waves per item) then still fits in one pass at two waves per SIMD
constexpr int kSwaSplitMaxItems = 512;

// ONE: one item per wave (SWA layers only), four items per workgroup; otherwise one item per
// workgroup, its keys split over the four waves
template <int D, bool FULL, bool F8, bool ONE>
__global__ void __launch_bounds__(64 * WAVES, 2) decode_bf16_kernel(const DecodeArgs a) {
  static_assert(!(FULL && ONE), "full-layer items always split over the workgroup");
  // V row stride in LDS (elements): rows 16 banks apart, so the 4 rows a 32-lane transposing
  // read covers fall on disjoint banks
  constexpr int VS = D + 32;
  constexpr int NC = D / 16;              // S^T k-steps over d
  constexpr int ND = D / 32;              // O^T d-blocks
  constexpr int CPR = D / 8;              // 16-byte pieces per row
  constexpr int VP = KSTEP * CPR / 64;    // 16-byte V pieces per lane per step
  constexpr int HALF = D / 2;
  // FP8 pools: a lane's K half row is HALF codes (KRAW 16-byte loads); a step's V tile is VRAW
  // 16-code pieces per lane
  constexpr int KRAW = HALF / 16;
  constexpr int VRAW = KSTEP * D / 16 / 64;
  using KT = std::conditional_t<F8, uint8_t, uint16_t>;  // pool element
  __shared__ __attribute__((aligned(16))) uint16_t vsm[WAVES][KSTEP * VS];

  const int tid = (int)__builtin_amdgcn_workitem_id_x();
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int item_idx = ONE ? (int)__builtin_amdgcn_workgroup_id_x() * WAVES + wv : (int)__builtin_amdgcn_workgroup_id_x();
  if (ONE && item_idx >= a.n_items) return;  // no workgroup barrier in this mode
  const WorkItem it = a.items[item_idx];
  const LayerView &L = a.L;
  const int hkv = L.hkv, W = L.w;
  const int G = a.hq / hkv, ql = a.q_len, rows = G * ql;
  const int64_t Lp = it.prior;
  const int seq = it.seq, head = it.head;
  uint16_t *vw = vsm[wv];

  const int ncol = lane & 31, hh = lane >> 5;
  const int r = it.row0 + ncol;  // this lane's query row: token t of query head gh of the group
  const int t = r / G, gh = r - (r / G) * G;
  const bool row_ok = r < rows;
  const int64_t qrow_idx = ((int64_t)it.si * ql + t) * a.hq + head * G + gh;

  // Q^T and K operands use one permutation of the contraction index (any bijection common to A
  // and B leaves the dot products unchanged): k-step c, lane half hh holds d-elements
  // HALF*hh + 8c .. +8, so every lane loads one contiguous HALF-element run of its K row.
  bf16x8 qf[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c)
    qf[c] = row_ok ? *reinterpret_cast<const bf16x8 *>(a.q + qrow_idx * D + HALF * hh + 8 * c) : bf16x8{};
  // fused RoPE: turn a fragment set of this layout (elements HALF*hh + 8c .. +7 of a row) at
  // position `pos`: pairs (D/4)hh + 4c .. +3 as neighbours, or (halves) the first coordinates of
  // pairs 8c .. 8c+7 in lane half 0 and their second coordinates in lane half 1 (swapped across)
  auto rope_frags = [&](bf16x8 (&f)[NC], int64_t pos) __attribute__((always_inline)) {
    if (L.rope_style == 0) {
#pragma unroll
      for (int c = 0; c < NC; ++c)
        f[c] = __builtin_bit_cast(bf16x8, rope_pairs8(__builtin_bit_cast(u32x4, f[c]), L.rope_lo, L.rope_hi, HALF, pos,
                                                      (D / 4) * hh + 4 * c));
    } else {
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const u32x4 mine = __builtin_bit_cast(u32x4, f[c]), other = lane32_swap(mine);
        u32x4 x = hh ? other : mine, y = hh ? mine : other;
        rope_halves8(x, y, L.rope_lo, L.rope_hi, HALF, pos, 8 * c);
        f[c] = __builtin_bit_cast(bf16x8, hh ? y : x);
      }
    }
  };
  // (rows past the item's last hold zeros; they turn at Lp so every table read stays in range)
  if (L.rope_fused) rope_frags(qf, Lp + (row_ok ? t : 0));

  const KT *ring = nullptr;
  if (!FULL) ring = reinterpret_cast<const KT *>(L.ring_base + (int64_t)seq * L.ring_seq_stride);
  const int32_t *table = FULL ? L.tables + (int64_t)seq * L.table_stride : nullptr;
  const KT *pages = FULL ? reinterpret_cast<const KT *>(L.page_base) : nullptr;
  const int64_t page_elems = 2LL * hkv * kPageTokens * D;
  // in the pool, a key's V row sits `voff` elements after its K row
  const int64_t voff = FULL ? (int64_t)hkv * kPageTokens * D : (int64_t)hkv * W * D;

  // Split items: the item's prior keys are split into WAVES consecutive ranges of a multiple of 32
  // keys (each starts on a page boundary for full layers: items start at multiples of 128); wave wv walks
  // [kb0, kb1) in steps of 32 (for SWA layers the keys are ring slots), and the last wave also
  // takes the call's new tokens.  Keys past kb1 are clamped to kb1-1 (a valid row, masked below).
  const int per_wave = ONE ? it.k_end - it.k_begin
                          : (it.k_end - it.k_begin + WAVES * KSTEP - 1) / (WAVES * KSTEP) * KSTEP;
  const int kb0 = ONE ? it.k_begin : min(it.k_begin + wv * per_wave, it.k_end);
  const int kb1 = ONE ? it.k_end : min(kb0 + per_wave, it.k_end);
  const bool do_new = it.with_new && (ONE || wv == WAVES - 1);
  const int n_prior = kb1 > kb0 ? (kb1 - kb0 + KSTEP - 1) / KSTEP : 0;
  // SWA: ring slot e holds the newest prior token; slot s holds position Lp-1-(e-s) for s <= e and
  // Lp-1-(e-s+W) for s > e, i.e. Lp-1+rel with rel = s-e (s <= e) or s-e-W (s > e).  Query t
  // (position Lp+t) sees positions >= Lp+t-W+1, i.e. rel >= t-W+2: one modulo per item.
  const int e_slot = (!FULL && Lp > 0) ? (int)((Lp - 1) % W) : 0;

  // K row of the step's 16-key group g (full layers: the group's page; uniform per group)
  auto group_base = [&](int st, int g) -> const KT * {
    const int k0 = min(kb0 + st * KSTEP + 16 * g, kb1 - 1);
    if (FULL) return pages + (int64_t)table[k0 >> 4] * page_elems + (int64_t)head * kPageTokens * D;
    return ring + (int64_t)head * W * D;
  };
  // row offset (elements) of key `key` of the step inside its group's base
  auto key_off = [&](int st, int key) -> int64_t {
    const int kidx = min(kb0 + st * KSTEP + key, kb1 - 1);
    return (int64_t)(FULL ? (kidx & (kPageTokens - 1)) : kidx) * D;
  };

  bf16x8 kreg[NC];
  u32x4 vreg[VP];
  u32x4 kraw[F8 ? KRAW : 1], vraw[F8 ? VRAW : 1];  // FP8 pools: the prior step's raw codes
  auto load_prior = [&](int st) {
    const KT *gb0 = group_base(st, 0), *gb1 = group_base(st, 1);
    const KT *kr = (ncol < 16 ? gb0 : gb1) + key_off(st, ncol) + HALF * hh;
    if constexpr (F8) {
#pragma unroll
      for (int j = 0; j < KRAW; ++j) kraw[j] = *reinterpret_cast<const u32x4 *>(kr + 16 * j);
#pragma unroll
      for (int i = 0; i < VRAW; ++i) {
        const int pc = lane + 64 * i, key = pc / (D / 16), col = pc % (D / 16);  // key >> 4 uniform per i
        vraw[i] = *reinterpret_cast<const u32x4 *>((key < 16 ? gb0 : gb1) + voff + key_off(st, key) + 16 * col);
      }
    } else {
#pragma unroll
      for (int c = 0; c < NC; ++c) kreg[c] = *reinterpret_cast<const bf16x8 *>(kr + 8 * c);
#pragma unroll
      for (int i = 0; i < VP; ++i) {
        const int pc = lane + 64 * i, key = pc / CPR, col = pc % CPR;  // key >> 4 is uniform per i
        vreg[i] = *reinterpret_cast<const u32x4 *>((key < 16 ? gb0 : gb1) + voff + key_off(st, key) + 8 * col);
      }
    }
  };
  // the call's new tokens (q_len <= 4): K/V rows of key j at ((si*ql + j)*hkv + head)*D (fused
  // RoPE turns the keys, at their positions L + j, right before their S^T product)
  auto load_new_into = [&](bf16x8 (&kd)[NC], u32x4 (&vd)[VP]) __attribute__((always_inline)) {
    const int64_t base = ((int64_t)it.si * ql * hkv + head) * D;
    const int kj = min(ncol, ql - 1);
#pragma unroll
    for (int c = 0; c < NC; ++c)
      kd[c] = *reinterpret_cast<const bf16x8 *>(a.k_new + base + (int64_t)kj * hkv * D + HALF * hh + 8 * c);
#pragma unroll
    for (int i = 0; i < VP; ++i) {
      const int pc = lane + 64 * i, key = min(pc / CPR, ql - 1), col = pc % CPR;
      vd[i] = *reinterpret_cast<const u32x4 *>(a.v_new + base + (int64_t)key * hkv * D + 8 * col);
    }
  };
  auto load_new = [&]() __attribute__((always_inline)) { load_new_into(kreg, vreg); };

  f32x16 o[ND];
#pragma unroll
  for (int db = 0; db < ND; ++db) o[db] = f32x16{};
  // m_ref: reference max in log2 units, raised only when a step's max exceeds it by more than 8
  // (a factor 2^8), so the accumulators are rescaled rarely and every p stays <= 2^8
  float m_ref = -INFINITY, l_run = 0.f;
  const float c2 = a.scale_log2;
  const int g16 = lane >> 4, s16 = lane & 15;

  auto stage_v = [&]() {
#pragma unroll
    for (int i = 0; i < VP; ++i) {
      const int pc = lane + 64 * i, key = pc / CPR, col = pc % CPR;
      *reinterpret_cast<u32x4 *>(&vw[key * VS + 8 * col]) = vreg[i];
    }
  };
  auto compute_s = [&]() {
    f32x16 s = f32x16{};
#pragma unroll
    for (int c = 0; c < NC; ++c) s = mfma32(kreg[c], qf[c], s);
    return s;
  };
  // FP8 pools: the prior step's V codes, dequantised into the wave's LDS slice as bf16
  auto stage_v_raw = [&]() {
#pragma unroll
    for (int i = 0; i < VRAW; ++i) {
      const int pc = lane + 64 * i, key = pc / (D / 16), col = pc % (D / 16);
      bf16x8 lo, hi;
      e4m3x16_to_bf16(vraw[i], L.v_scale, lo, hi);
      *reinterpret_cast<bf16x8 *>(&vw[key * VS + 16 * col]) = lo;
      *reinterpret_cast<bf16x8 *>(&vw[key * VS + 16 * col + 8]) = hi;
    }
  };
  // FP8 pools: S^T of the prior step from its K codes, dequantised into MFMA operands
  auto compute_s_raw = [&]() {
    f32x16 s = f32x16{};
#pragma unroll
    for (int j = 0; j < KRAW; ++j) {
      bf16x8 k0, k1;
      e4m3x16_to_bf16(kraw[j], L.k_scale, k0, k1);
      s = mfma32(k0, qf[2 * j], s);
      s = mfma32(k1, qf[2 * j + 1], s);
    }
    return s;
  };
  // softmax of one masked step and O^T += V^T P^T from the wave's LDS slice
  auto softmax_pv = [&](f32x16 &s) {
    float mx = -INFINITY;
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) mx = fmaxf(mx, s[rr]);
    mx = fmaxf(mx, other_half(mx)) * c2;
    const bool raise = mx > m_ref + 8.f;
    if (__builtin_amdgcn_ballot_w64(raise) != 0) {
      const float alpha = raise ? exp2_fast(m_ref - mx) : 1.f;  // 0 when m_ref was -inf
#pragma unroll
      for (int db = 0; db < ND; ++db) o[db] *= alpha;
      l_run *= alpha;
      m_ref = raise ? mx : m_ref;
    }
    const float msc = (m_ref == -INFINITY) ? 0.f : m_ref;
    bf16x8 pf[2];
#pragma unroll
    for (int half = 0; half < 2; ++half)
#pragma unroll
      for (int e = 0; e < 8; ++e) pf[half][e] = (__bf16)exp2_fast(fmaf(s[8 * half + e], c2, -msc));
    // row sum of the bf16-rounded P, the values the PV product multiplies (as in the prefill
    // kernel), two per v_dot2_f32_bf16
    float ps[4] = {0.f, 0.f, 0.f, 0.f};
    const bf16x2 one2 = {(__bf16)1.f, (__bf16)1.f};
#pragma unroll
    for (int half = 0; half < 2; ++half)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        ps[j] = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pf[half][2 * j], pf[half][2 * j + 1]}, one2, ps[j], false);
    l_run += (ps[0] + ps[1]) + (ps[2] + ps[3]);
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
  };

  // the call's new tokens as one more step (keys loaded in kreg/vreg beforehand): V staged before
  // the keys turn (fused RoPE), so the V registers are free again during the rotation
  auto new_step = [&]() __attribute__((always_inline)) {
    stage_v();
    if (L.rope_fused) rope_frags(kreg, Lp + min(ncol, ql - 1));
    f32x16 s = compute_s();
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) {
      const int key = 8 * (rr >> 2) + 4 * hh + (rr & 3);
      const bool ok = row_ok & (key <= t) & (FULL | (key > t - W));
      s[rr] = ok ? s[rr] : -INFINITY;
    }
    softmax_pv(s);
  };
  // mask: S^T row (key) 8*(rr/4) + 4*hh + rr%4 of prior step st against this lane's query
  // (bitwise &/| and one select per element: straight-line code, no short-circuit branches)
  auto mask_prior = [&](f32x16 &s, int st) __attribute__((always_inline)) {
    const int kbase = kb0 + st * KSTEP;
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) {
      const int kidx = kbase + 8 * (rr >> 2) + 4 * hh + (rr & 3);
      // SWA: age of the slot relative to the newest one, in (-W, 0]
      const int rel = kidx - e_slot - (kidx > e_slot ? W : 0);
      const bool ok = row_ok & (kidx < kb1) & (FULL | (rel >= t - W + 2));
      s[rr] = ok ? s[rr] : -INFINITY;
    }
  };
  // A split-form SWA wave with one prior step and the new tokens (the last wave of an item at
  // w <= 128) issues both loads at once, the new tokens into a set of their own, so their latency
  // overlaps the prior step's instead of following it.
  constexpr bool ONE_STEP_FORM = !FULL && !F8 && !ONE;
  if (ONE_STEP_FORM && do_new && n_prior == 1) {
    bf16x8 knew[NC];
    u32x4 vnew[VP];
    load_prior(0);
    load_new_into(knew, vnew);
    stage_v();
    f32x16 s = compute_s();
    mask_prior(s, 0);
    softmax_pv(s);
#pragma unroll
    for (int c = 0; c < NC; ++c) kreg[c] = knew[c];
#pragma unroll
    for (int i = 0; i < VP; ++i) vreg[i] = vnew[i];
    new_step();
  } else {
    if (n_prior > 0) load_prior(0);
    else if (do_new) load_new();
    // FP8 pools take the new tokens (bf16, in the bf16 registers) first, while the first prior
    // step's codes load: after the loop their registers would be live beside the prior step's
    if constexpr (F8) {
      if (do_new && n_prior > 0) {
        load_new();
        new_step();
      }
    }
    for (int st = 0; st < n_prior; ++st) {
      // after this step's PV the wave reads the slice again only after the next store
      f32x16 s;
      if constexpr (F8) {
        stage_v_raw();
        s = compute_s_raw();
      } else {
        stage_v();
        s = compute_s();
      }
      // the next step's loads overlap this step's softmax and PV work (FP8 pools took the new
      // tokens before the loop)
      if (st + 1 < n_prior) load_prior(st + 1);
      else if (!F8 && do_new) load_new();
      mask_prior(s, st);
      softmax_pv(s);
    }
    if (do_new && !(F8 && n_prior > 0)) new_step();
  }

  // ---- merge the four waves' (m_ref, l, O) in LDS (the V slices are free now): waves 1 and 3
  // into 0 and 2, then 2 into 0.  O and l are relative to 2^m_ref, so a merge rescales both
  // sides to the larger reference.  Slot layout [register][lane]: each store is 256 contiguous
  // bytes.
  constexpr int SLOT = ND * 16 * 64 + 2 * 64;  // floats
  float *mrg = reinterpret_cast<float *>(&vsm[0][0]);
  auto put = [&](float *p) {
#pragma unroll
    for (int db = 0; db < ND; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) p[(db * 16 + r) * 64 + lane] = o[db][r];
    p[ND * 16 * 64 + lane] = m_ref;
    p[ND * 16 * 64 + 64 + lane] = l_run;
  };
  auto take = [&](const float *p) {
    const float m2 = p[ND * 16 * 64 + lane], l2 = p[ND * 16 * 64 + 64 + lane];
    const float M = fmaxf(m_ref, m2);
    const float a1 = m_ref == -INFINITY ? 0.f : exp2_fast(m_ref - M);
    const float a2 = m2 == -INFINITY ? 0.f : exp2_fast(m2 - M);
#pragma unroll
    for (int db = 0; db < ND; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[db][r] = a1 * o[db][r] + a2 * p[(db * 16 + r) * 64 + lane];
    l_run = a1 * l_run + a2 * l2;
    m_ref = M;
  };
  if constexpr (!ONE) {
    __syncthreads();  // every wave is done with its V slice
    if (wv & 1) put(mrg + (wv >> 1) * SLOT);
    __syncthreads();
    if (!(wv & 1)) take(mrg + (wv >> 1) * SLOT);
    __syncthreads();
    if (wv == 2) put(mrg);
    __syncthreads();
    if (wv != 0) return;
    take(mrg);
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
    const int64_t prow = (int64_t)it.part * rows + r;
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
      a.part_ml[prow * 2 + 0] = m_ref;  // o and l are relative to 2^m_ref (-inf: no valid key)
      a.part_ml[prow * 2 + 1] = l_tot;
    }
  }
}

// Merge the partials of every split (sequence, KV head, query row): one workgroup per row, in one
// pass.  Thread (pl, c4) owns 4 output dims (one float4 of each partial it reads) and the partials
// pl, pl + PL, ...; it loads them UNR at a time (a batch's loads are all in flight together, so a
// row with hundreds of partials, as in a 1M-token verify, waits out about one memory latency) and
// folds each batch into its running (M, num, den): M rises to the batch max first, the sums are
// rescaled by 2^(M_old - M), then num += 2^(m_s - M) o_s and den += 2^(m_s - M) l_s.  The PL
// running states of a column then merge pairwise in LDS by the same rule, and
// o = num / den  -- the softmax of Eq.(4)-(5) regrouped over the splits.
template <int D, int NT, int UNR>
__global__ void __launch_bounds__(NT) combine_kernel(const DecodeArgs a) {
  constexpr int C4 = D / 4;    // float4 columns of a row
  constexpr int PL = NT / C4;  // partials read in parallel
  const int hkv = a.L.hkv;
  const int G = a.hq / hkv, ql = a.q_len, rows = G * ql;
  const int pair = blockIdx.x / rows, n = blockIdx.x % rows;
  const int si = pair / hkv, head = pair % hkv;
  const CombineEntry ce = a.combine[pair];
  if (ce.count == 0) return;
  const int tid = threadIdx.x, c4 = tid % C4, pl = tid / C4;
  float M = -INFINITY, den = 0.f;
  float4 num = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s0 = pl; s0 < ce.count; s0 += UNR * PL) {
    float ms[UNR], ls[UNR];
    float4 ov[UNR];
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      ms[u] = -INFINITY;
      ls[u] = 0.f;
      ov[u] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (s0 + u * PL < ce.count) {
        const int64_t pr = (int64_t)(ce.first + s0 + u * PL) * rows + n;
        ms[u] = a.part_ml[pr * 2];
        ls[u] = a.part_ml[pr * 2 + 1];
        ov[u] = *reinterpret_cast<const float4 *>(a.part_o + pr * D + 4 * c4);
      }
    }
    float mb = M;
#pragma unroll
    for (int u = 0; u < UNR; ++u) mb = fmaxf(mb, ms[u]);
    if (mb > M) {  // M == -inf leaves num = den = 0, which any factor keeps
      const float f = M == -INFINITY ? 0.f : exp2_fast(M - mb);
      num.x *= f;
      num.y *= f;
      num.z *= f;
      num.w *= f;
      den *= f;
      M = mb;
    }
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const float f = ms[u] == -INFINITY ? 0.f : exp2_fast(ms[u] - M);  // a split with no valid key adds 0
      num.x = fmaf(f, ov[u].x, num.x);
      num.y = fmaf(f, ov[u].y, num.y);
      num.z = fmaf(f, ov[u].z, num.z);
      num.w = fmaf(f, ov[u].w, num.w);
      den = fmaf(f, ls[u], den);
    }
  }
  __shared__ float4 nsum[NT];
  __shared__ float dsum[NT], msum[NT];
  nsum[tid] = num;
  dsum[tid] = den;
  msum[tid] = M;
  __syncthreads();
#pragma unroll
  for (int h = PL / 2; h > 0; h >>= 1) {
    if (pl < h) {
      const float m2 = msum[tid + h * C4], d2 = dsum[tid + h * C4];
      const float4 n2 = nsum[tid + h * C4];
      const float Mx = fmaxf(M, m2);
      const float f1 = M == -INFINITY ? 0.f : exp2_fast(M - Mx);
      const float f2 = m2 == -INFINITY ? 0.f : exp2_fast(m2 - Mx);
      num.x = f1 * num.x + f2 * n2.x;
      num.y = f1 * num.y + f2 * n2.y;
      num.z = f1 * num.z + f2 * n2.z;
      num.w = f1 * num.w + f2 * n2.w;
      den = f1 * den + f2 * d2;
      M = Mx;
      nsum[tid] = num;
      dsum[tid] = den;
      msum[tid] = M;
    }
    __syncthreads();
  }
  if (pl == 0) {
    const float inv = 1.f / den;
    const int t = n / G, gh = n % G;
    const int64_t qrow_idx = ((int64_t)si * ql + t) * a.hq + head * G + gh;
    uint2 w;
    w.x = (uint32_t)f2bf(num.x * inv) | ((uint32_t)f2bf(num.y * inv) << 16);
    w.y = (uint32_t)f2bf(num.z * inv) | ((uint32_t)f2bf(num.w * inv) << 16);
    *reinterpret_cast<uint2 *>(a.out + qrow_idx * D + 4 * c4) = w;
  }
}

}  // namespace

hipError_t launch_decode_bf16(const DecodeArgs &a, hipStream_t s) {
  if (a.hq / a.L.hkv * a.q_len > 128) return hipErrorInvalidValue;
  if (a.n_items > 0) {
    const bool f8 = a.L.kv_fp8 != 0, full = a.L.is_full != 0;
    // SWA layers run one item per wave unless the call is small enough to split every item
    const bool one = !full && a.n_items > kSwaSplitMaxItems;
    const dim3 grid((unsigned)(one ? (a.n_items + WAVES - 1) / WAVES : a.n_items)), block(64 * WAVES);
#define SWA_DECODE(D_, FULL_, F8_, ONE_) hipLaunchKernelGGL((decode_bf16_kernel<D_, FULL_, F8_, ONE_>), grid, block, 0, s, a)
#define SWA_DECODE_D(D_)                                                                      \
    do {                                                                                        \
      if (full) { if (f8) SWA_DECODE(D_, true, true, false); else SWA_DECODE(D_, true, false, false); } \
      else if (one) { if (f8) SWA_DECODE(D_, false, true, true); else SWA_DECODE(D_, false, false, true); } \
      else { if (f8) SWA_DECODE(D_, false, true, false); else SWA_DECODE(D_, false, false, false); } \
    } while (0)
    if (a.L.d == 128) SWA_DECODE_D(128);
    else SWA_DECODE_D(64);
#undef SWA_DECODE_D
#undef SWA_DECODE
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (a.n_parts > 0) {
    const int rows = a.hq / a.L.hkv * a.q_len;
    const dim3 grid((unsigned)(a.n_seqs * a.L.hkv * rows));
    // rows with more partials than a 256-thread batch holds (8 partials per thread in parallel)
    // take 1024 threads, so even a 1M-token verify's ~400 partials load in one batch
    const bool wide = a.max_split > 256 / (a.L.d / 4) * 8;
    if (a.L.d == 128) {
      if (wide) hipLaunchKernelGGL((combine_kernel<128, 1024, 12>), grid, dim3(1024), 0, s, a);
      else hipLaunchKernelGGL((combine_kernel<128, 256, 8>), grid, dim3(256), 0, s, a);
    } else {
      if (wide) hipLaunchKernelGGL((combine_kernel<64, 1024, 12>), grid, dim3(1024), 0, s, a);
      else hipLaunchKernelGGL((combine_kernel<64, 256, 8>), grid, dim3(256), 0, s, a);
    }
    return hipGetLastError();
  }
  return hipSuccess;
}

}  // namespace swa
