// bf16 prefill attention on gfx950 MFMA: a chunk of n queries at positions L .. L+n-1 of one
// sequence against the keys W(i) of each query ([SWA-theory] §数学的定義 Eq.(1)-(5)), with the
// keys below L read from the pool (ring for SWA layers, pages for full layers) and the chunk's own
// keys from the call's k/v.  fp32 accumulation and softmax; P is rounded to bf16 for the PV
// product; the output is rounded to bf16 (RNE).
//
// Work decomposition
//   * A workgroup (8 waves, two per SIMD, one workgroup per CU) owns one KV head and a block of
//     P positions; its 256 query rows are the G = Hq/Hkv query heads sharing that KV head times
//     P positions (P = 256/G), so each K/V tile staged in LDS serves every query head of the
//     group, and the global loads and LDS stores of a tile are spread over 8 waves.
//   * Keys are processed in tiles of 64 absolute positions.  Tiles wholly outside the block's
//     band [i0-w+1, i1] are never visited; tiles wholly inside it run without a mask; the few
//     tiles crossing the band edge mask per element (the whole-tile skip of the FlashAttention-2
//     style kernels the page mentions in §発展的な話題, done here on absolute positions).
//   * Each wave computes S^T = K·Q^T for its 32 rows with v_mfma_f32_32x32x16_bf16, so one lane
//     owns one query column and 16 keys of it: the row max and sum are in-lane plus one
//     permlane32 swap.  P^T leaves the accumulator registers directly as the B operand of
//     O^T += V^T·P^T; V^T's A operand comes from the row-major V tile in LDS through the gfx950
//     transposing LDS read (ds_read_b64_tr_b16), so no transpose is ever written.  LDS reads are
//     issued ahead of their MFMAs: K fragments through a 4-deep register ring, the first V^T step
//     right after the S^T product so it arrives during the softmax.
//   * K/V tiles are double-buffered in LDS and staged through two register sets: a tile's global
//     loads are issued two tiles ahead and held in VGPRs (native vector types, so they never go
//     through scratch) until its LDS store at the end of the preceding tile, so the store rarely
//     waits on its loads; out-of-band keys are clamped, not branched around.
//   * The row max and the row sum run with the IEEE mode bit off (build flag of this file), so
//     an fmax of an MFMA result needs no quieting first.
//   * Workgroup ids are remapped so each XCD (ids round-robin over 8) gets a contiguous range of
//     (KV head, block) pairs: neighbouring blocks share most of their band, which then stays in
//     that XCD's L2.  Blocks run last-first where their key counts grow along the chunk (full
//     layers; a window wider than the prefix by more than 8 blocks), so the longest start first and
//     the short ones fill the tail; otherwise every block has the same keys and they run in order.

#include "dev_common.h"

#include <type_traits>

namespace swa {

namespace {

constexpr int BN = 64;             // keys per tile
constexpr int WG = 512;            // threads per workgroup: 8 waves, two per SIMD
constexpr int ROWS = WG / 2;       // query rows per workgroup (32 per wave)
constexpr int NKB = BN / 32;       // 32-key blocks of S^T per tile

template <int D>
struct Tile {
  static constexpr int KS = D + 8;    // K row stride in LDS (elements): 272 B / 144 B
  // V row stride in LDS (elements): 320 B / 192 B.  A transposing read by 32 lanes covers 4 rows
  // of 64 B; with rows 16 banks apart (mod 64) they fall on disjoint banks.
  static constexpr int VS = D + 32;
  static constexpr int PIECES = BN * D / 8;       // 16-byte pieces per K (or V) tile
  static constexpr int PER_THREAD = PIECES / WG;  // 2 (D=128) or 1 (D=64)
  static constexpr int NC = D / 16;               // MFMA k-steps over d for S^T
  static constexpr int ND = D / 32;               // 32-wide d blocks of O^T
};

__device__ __forceinline__ int clamp_i(int x, int lo, int hi) { return min(max(x, lo), hi); }  // v_med3_i32

template <int D, bool FULL, bool F8>
__global__ void __launch_bounds__(WG, 1)
prefill_bf16_kernel(const PrefillArgs a, int G, int P, int nb, int n_wg) {
  using T = Tile<D>;
  using KT = std::conditional_t<F8, uint8_t, uint16_t>;  // pool element (FP8 pools: E4M3 codes)
  __shared__ __attribute__((aligned(16))) uint16_t ks[2][BN * T::KS];
  __shared__ __attribute__((aligned(16))) uint16_t vs[2][BN * T::VS];

  // ---- XCD-contiguous remap of the workgroup id
  const int x = (int)__builtin_amdgcn_workgroup_id_x();  // builtins: no device-library call
  const int q8 = n_wg >> 3, rem = n_wg & 7, xcd = x & 7;
  const int logical = xcd * q8 + (xcd < rem ? xcd : rem) + (x >> 3);
  const int head = logical / nb;
  const int bi = logical - head * nb;
  const bool last_first = FULL || a.prior + 8LL * P < (int64_t)a.L.w;  // uniform over the grid
  const int b = last_first ? nb - 1 - bi : bi;

  const LayerView &L = a.L;
  const int hkv = L.hkv, W = L.w;
  const int64_t L0 = a.prior;
  const int64_t i0 = L0 + (int64_t)b * P;
  const int64_t i_last = L0 + a.n - 1;
  const int64_t i1 = (i0 + P - 1 < i_last) ? i0 + P - 1 : i_last;
  const int64_t k_lo = FULL ? 0 : (i0 - W + 1 > 0 ? i0 - W + 1 : 0);
  const int64_t k_hi = i1;

  const int tid = (int)__builtin_amdgcn_workitem_id_x(), lane = tid & 63, wv = tid >> 6;
  const int ncol = lane & 31, hh = lane >> 5;

  // ---- this lane's query column: row r = pp*G + gh (consecutive rows are adjacent in memory)
  const int r = wv * 32 + ncol;
  const int pp = r / G, gh = r - (r / G) * G;
  const int64_t ipos = i0 + pp;
  const bool row_ok = ipos <= i1;
  const int qh = head * G + gh;
  const uint16_t *qrow = a.q + ((ipos - L0) * a.hq + qh) * D;

  bf16x8 qf[T::NC];
#pragma unroll
  for (int c = 0; c < T::NC; ++c) {
    if (row_ok) qf[c] = *reinterpret_cast<const bf16x8 *>(qrow + 16 * c + 8 * hh);
    else qf[c] = bf16x8{};
  }

  // ---- tile loader.  Thread `tid` moves pieces i = 0..PER_THREAD-1 of each K and V tile: key
  // kq + KPI*i, 16-byte column tid % CPR (16 consecutive threads cover one 256-byte row).  The
  // source of a tile is decided once per tile (uniform): all keys in the chunk, all in the pool,
  // or straddling L (rare: per-key choice).  Keys of a tile outside the block's band
  // [k_lo, k_hi] are clamped into it rather than branched around: they load a valid duplicate
  // row, whose scores the edge mask sets to -inf and whose V rows meet p = 0, so every value the
  // MFMAs see stays finite.
  constexpr int CPR = D / 8, KPI = WG / CPR;
  const int kq = tid / CPR, col8 = (tid % CPR) * 8;
  u32x4 kreg[2][T::PER_THREAD], vreg[2][T::PER_THREAD];  // two staging sets: loads run two tiles ahead
  const KT *ring = nullptr;
  if (!FULL) ring = reinterpret_cast<const KT *>(L.ring_base + (int64_t)a.seq * L.ring_seq_stride);
  const int32_t *table = FULL ? L.tables + (int64_t)a.seq * L.table_stride : nullptr;
  const KT *pages = FULL ? reinterpret_cast<const KT *>(L.page_base) : nullptr;
  // one 8-element piece of a pool row as 8 bf16 (FP8 pools: 8 codes dequantised with `scale`)
  auto pool_piece = [&](const KT *row8, float scale) -> u32x4 {
    if constexpr (F8) return e4m3x8_to_bf16(*reinterpret_cast<const uint2 *>(row8), scale);
    else return *reinterpret_cast<const u32x4 *>(row8);
  };
  const int64_t page_elems = 2LL * hkv * kPageTokens * D;
  const int64_t chunk_row = (int64_t)hkv * D;  // elements between consecutive chunk positions
  // in the pool, a key's V row sits `pool_vshift` elements after its K row
  const int64_t pool_vshift = FULL ? (int64_t)hkv * kPageTokens * D : (int64_t)hkv * W * D;
  auto load_tile = [&](int64_t tbase, int ss) {
    // band-relative clamp bounds of this tile's keys (uniform; every visited tile meets the band)
    const int lo_c = (int)(k_lo - tbase > 0 ? k_lo - tbase : 0);
    const int hi_c = (int)(k_hi - tbase < BN - 1 ? k_hi - tbase : BN - 1);
    if (tbase >= L0) {  // every key of the tile is a chunk token
      // buffer loads: the tile's (uniform) base goes into a buffer resource, each piece needs
      // only a 32-bit in-tile byte offset (no per-lane 64-bit address arithmetic)
      const int64_t toff = (tbase - L0) * chunk_row + (int64_t)head * D;
      const auto rk = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(a.k + toff), 0, BN * (int)chunk_row * 2, kBufferRsrcWord3);
      const auto rv = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(a.v + toff), 0, BN * (int)chunk_row * 2, kBufferRsrcWord3);
#pragma unroll
      for (int i = 0; i < T::PER_THREAD; ++i) {
        const int bo = (clamp_i(kq + KPI * i, lo_c, hi_c) * (int)chunk_row + col8) * 2;
        kreg[ss][i] = __builtin_amdgcn_raw_buffer_load_b128(rk, bo, 0, 0);
        vreg[ss][i] = __builtin_amdgcn_raw_buffer_load_b128(rv, bo, 0, 0);
      }
    } else if (tbase + BN <= L0 && (FULL || W >= BN)) {  // pool tile, fast form
      if (FULL) {
        // tiles start on page boundaries: key tbase + k sits in page (tbase + k) / 16, row k % 16.
        // Pool tiles of a full layer lie wholly inside [0, L) and are never clipped.
#pragma unroll
        for (int i = 0; i < T::PER_THREAD; ++i) {
          const int key = kq + KPI * i;
          const KT *kr = pages + (int64_t)table[(tbase + key) >> 4] * page_elems +
                         ((int64_t)head * kPageTokens + (key & (kPageTokens - 1))) * D + col8;
          kreg[ss][i] = pool_piece(kr, L.k_scale);
          vreg[ss][i] = pool_piece(kr + pool_vshift, L.v_scale);
        }
      } else {
        const int sbase = (int)(tbase % W);  // one modulo per tile; slots then advance with one wrap
        const KT *hb = ring + (int64_t)head * W * D + col8;
#pragma unroll
        for (int i = 0; i < T::PER_THREAD; ++i) {
          int slot = sbase + clamp_i(kq + KPI * i, lo_c, hi_c);
          slot = slot >= W ? slot - W : slot;
          const KT *kr = hb + (int64_t)slot * D;
          kreg[ss][i] = pool_piece(kr, L.k_scale);
          vreg[ss][i] = pool_piece(kr + pool_vshift, L.v_scale);
        }
      }
    } else {  // straddles L, or a small ring / narrow pages: choose per key (selects, no branch)
#pragma unroll
      for (int i = 0; i < T::PER_THREAD; ++i) {
        const int64_t j = tbase + clamp_i(kq + KPI * i, lo_c, hi_c);
        const int64_t jp = j < L0 ? j : L0 - 1;  // pool row address (valid when j < L)
        const int64_t jc = j < L0 ? L0 : j;      // chunk row address (valid when j >= L)
        const KT *pr = FULL ? pages + (int64_t)table[jp >> 4] * page_elems +
                                  ((int64_t)head * kPageTokens + (jp & (kPageTokens - 1))) * D
                            : ring + ((int64_t)head * W + jp % W) * D;
        const int64_t ce = (jc - L0) * chunk_row + (int64_t)head * D + col8;
        const bool in_pool = j < L0;
        kreg[ss][i] = in_pool ? pool_piece(pr + col8, L.k_scale) : *reinterpret_cast<const u32x4 *>(a.k + ce);
        vreg[ss][i] = in_pool ? pool_piece(pr + pool_vshift + col8, L.v_scale) : *reinterpret_cast<const u32x4 *>(a.v + ce);
      }
    }
  };
  auto store_tile = [&](int buf, int ss) {
#pragma unroll
    for (int i = 0; i < T::PER_THREAD; ++i) {
      const int key = kq + KPI * i;
      *reinterpret_cast<u32x4 *>(&ks[buf][key * T::KS + col8]) = kreg[ss][i];
      *reinterpret_cast<u32x4 *>(&vs[buf][key * T::VS + col8]) = vreg[ss][i];
    }
  };

  f32x16 o[T::ND];
#pragma unroll
  for (int db = 0; db < T::ND; ++db) o[db] = f32x16{};
  float m_ref = -INFINITY, l_run = 0.f;  // m_ref: reference max, already scaled to log2 units
  const float c2 = a.scale_log2;

  const int64_t t_first = k_lo / BN, t_last = k_hi / BN;
  // Tile u is staged in register set (u - t_first) & 1 and LDS buffer (u - t_first) & 1.  Its
  // loads are issued two tiles ahead (at the top of iteration u - 2) and its LDS store happens at
  // the end of iteration u - 1, so a store rarely waits for its loads.
  load_tile(t_first * BN, 0);
  store_tile(0, 0);
  if (t_first < t_last) load_tile((t_first + 1) * BN, 1);
  __syncthreads();

  auto iteration = [&](int64_t t, auto set_c) {
    constexpr int SS = decltype(set_c)::value;   // staging set of tile t (free: stored already)
    const int buf = SS;
    const int64_t tbase = t * BN;
    if (t + 1 < t_last) load_tile(tbase + 2 * BN, SS);

    // band class of this tile for the whole block (uniform across the workgroup)
    const bool inner = (tbase + BN - 1 <= i0) && (FULL || tbase >= i1 - W + 1);

    // S^T = K Q^T for keys [tbase, tbase+BN): NKB 32-key blocks.  K fragments (32 keys x 16 d)
    // come from LDS through a ring of KD registers, each read KD fragments before its MFMA; the
    // group barriers keep that order (left alone, the scheduler sinks each read next to its use
    // and every pair of MFMAs waits out a full LDS latency).
    f32x16 s[NKB];
    {
      constexpr int NF = NKB * T::NC, KD = 4;
      const uint16_t *kp0 = &ks[buf][ncol * T::KS + 8 * hh];
      auto kfrag = [&](int f) {
        return *reinterpret_cast<const bf16x8 *>(kp0 + (f / T::NC) * 32 * T::KS + 16 * (f % T::NC));
      };
      bf16x8 kr[KD];
#pragma unroll
      for (int f = 0; f < KD; ++f) kr[f] = kfrag(f);
      __builtin_amdgcn_sched_group_barrier(0x100, KD, 0);
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        const int kb = f / T::NC, c = f % T::NC;
        s[kb] = mfma32(kr[f % KD], qf[c], c == 0 ? f32x16{} : s[kb]);
        if (f + KD < NF) kr[f % KD] = kfrag(f + KD);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (f + KD < NF) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
    }
    // V^T fragments of the first 16-key step, read now so they arrive during the softmax
    const int g16 = lane >> 4, s16 = lane & 15;
    auto vfrag = [&](int k, int db) {
      const uint16_t *vp = &vs[buf][(16 * k + 4 * hh + (s16 >> 2)) * T::VS + 16 * (g16 & 1) + 4 * (s16 & 3)] + 32 * db;
      return cat(lds_read_tr(vp), lds_read_tr(vp + 8 * T::VS));
    };
    bf16x8 v0[T::ND];
#pragma unroll
    for (int db = 0; db < T::ND; ++db) v0[db] = vfrag(0, db);
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * T::ND, 0);
    // mask on edge tiles: key tbase+koff (row of S^T) is valid for this lane's query iff
    // koff <= ipos - tbase and (full layer or koff > ipos - W - tbase); 32-bit offsets
    if (!inner) {
      // an empty volatile asm keeps this block a real branch: without it the compiler turns the
      // per-element selects into unconditional ones, ~100 VALU ops on every (mostly inner) tile
      __asm__ volatile("");
      const int64_t dh = ipos - tbase;
      const int hi_k = row_ok ? (int)(dh < 127 ? (dh > -2 ? dh : -2) : 127) : -2;
      const int64_t dl = ipos - W - tbase;
      const int lo_k = FULL ? -1 : (int)(dl < 127 ? (dl > -2 ? dl : -2) : 127);
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
          const int koff = kb * 32 + 8 * (rr >> 2) + 4 * hh + (rr & 3);
          s[kb][rr] = ((koff <= hi_k) & (koff > lo_k)) ? s[kb][rr] : -INFINITY;
        }
    }
    // online softmax in the log2 domain; lane pair (l, l^32) owns one query.  The reference max
    // m_ref is raised only when the tile max exceeds it by more than 8 (a factor 2^8), so the
    // accumulators are rescaled rarely (typically once) and every p stays <= 2^8: exact softmax
    // after the final division, with no overflow risk in fp32 or bf16.
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) mx = fmaxf(mx, s[kb][rr]);
    mx = fmaxf(mx, other_half(mx)) * c2;
    const bool raise = mx > m_ref + 8.f;
    if (__builtin_amdgcn_ballot_w64(raise) != 0) {
      const float alpha = raise ? exp2_fast(m_ref - mx) : 1.f;  // 0 when m_ref was -inf
#pragma unroll
      for (int db = 0; db < T::ND; ++db) o[db] *= alpha;
      l_run *= alpha;
      m_ref = raise ? mx : m_ref;
    }
    const float msc = (m_ref == -INFINITY) ? 0.f : m_ref;
    bf16x8 pf[2 * NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int half = 0; half < 2; ++half)
#pragma unroll
        for (int e = 0; e < 8; ++e) pf[kb * 2 + half][e] = (__bf16)exp2_fast(fmaf(s[kb][8 * half + e], c2, -msc));
    // row sum of the bf16-rounded P (the values the PV product uses), two per v_dot2_f32_bf16
    float ps[4] = {0.f, 0.f, 0.f, 0.f};
    const bf16x2 one2 = {(__bf16)1.f, (__bf16)1.f};
#pragma unroll
    for (int k = 0; k < 2 * NKB; ++k)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        ps[j] = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pf[k][2 * j], pf[k][2 * j + 1]}, one2, ps[j], false);
    l_run += (ps[0] + ps[1]) + (ps[2] + ps[3]);

    // O^T += V^T P^T: BN/16 16-key steps x D/32 d-blocks; V^T via transposing LDS reads (the
    // first step's fragments were read before the softmax)
#pragma unroll
    for (int k = 0; k < 2 * NKB; ++k) {
#pragma unroll
      for (int db = 0; db < T::ND; ++db) o[db] = mfma32(k == 0 ? v0[db] : vfrag(k, db), pf[k], o[db]);
    }

    // Buffer buf^1 was last read in iteration t-1, which every wave finished before the barrier
    // that closed it; one barrier after the store publishes tile t+1.
    if (t < t_last) {
      store_tile(buf ^ 1, SS ^ 1);
      __syncthreads();
    }
  };
  for (int64_t t = t_first; t <= t_last; t += 2) {
    iteration(t, std::integral_constant<int, 0>{});
    if (t + 1 <= t_last) iteration(t + 1, std::integral_constant<int, 1>{});
  }

  // ---- normalise and write: lane holds query ncol, dims 32*db + 8*(rr/4) + 4*hh + rr%4
  const float l_tot = l_run + other_half(l_run);
  if (row_ok) {
    const float inv = 1.f / l_tot;
    uint16_t *orow = a.out + ((ipos - L0) * a.hq + qh) * D;
#pragma unroll
    for (int db = 0; db < T::ND; ++db)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int dd = 32 * db + 8 * q4 + 4 * hh;
        uint2 w;
        w.x = (uint32_t)f2bf(o[db][4 * q4 + 0] * inv) | ((uint32_t)f2bf(o[db][4 * q4 + 1] * inv) << 16);
        w.y = (uint32_t)f2bf(o[db][4 * q4 + 2] * inv) | ((uint32_t)f2bf(o[db][4 * q4 + 3] * inv) << 16);
        *reinterpret_cast<uint2 *>(orow + dd) = w;
      }
  }
}

}  // namespace

hipError_t launch_prefill_bf16(const PrefillArgs &a, hipStream_t s) {
  const int G = a.hq / a.L.hkv;
  const int P = ROWS / G;
  const int nb = (a.n + P - 1) / P;
  const int64_t n_wg = (int64_t)nb * a.L.hkv;
  if (n_wg == 0) return hipSuccess;
  if (n_wg > INT32_MAX) return hipErrorInvalidValue;
  const dim3 grid((unsigned)n_wg), block(WG);
#define SWA_PREFILL(D_, FULL_, F8_) \
  hipLaunchKernelGGL((prefill_bf16_kernel<D_, FULL_, F8_>), grid, block, 0, s, a, G, P, nb, (int)n_wg)
  const bool f8 = a.L.kv_fp8 != 0, full = a.L.is_full != 0;
  if (a.L.d == 128) {
    if (full) { if (f8) SWA_PREFILL(128, true, true); else SWA_PREFILL(128, true, false); }
    else { if (f8) SWA_PREFILL(128, false, true); else SWA_PREFILL(128, false, false); }
  } else {
    if (full) { if (f8) SWA_PREFILL(64, true, true); else SWA_PREFILL(64, true, false); }
    else { if (f8) SWA_PREFILL(64, false, true); else SWA_PREFILL(64, false, false); }
  }
#undef SWA_PREFILL
  return hipGetLastError();
}

}  // namespace swa
