// Internal declarations shared by the host library and the kernel launchers of libswa.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace swa {

constexpr int kPageTokens = 16;

// Device-side view of one pool layer, enough for any kernel to find a position's key and value.
//   SWA layer  : ring of `w` slots per (seq, kv head).  K [Hkv][w][d] then V [Hkv][w][d].
//   Full layer : 16-token pages.  K [Hkv][16][d] then V [Hkv][16][d] per page; per-sequence
//                page tables (int32) in the arena, row `seq` of `table_stride` entries.
struct LayerView {
  char *ring_base;        // SWA: ring block of seq 0 for this layer
  int64_t ring_seq_stride;  // bytes between consecutive sequences' rings of this layer
  char *page_base;        // full: page 0 of this layer
  const int32_t *tables;  // full: page table row of seq 0
  int64_t table_stride;   // entries per sequence row
  int32_t w;              // ring slots (SWA) / window (0 = full attention)
  int32_t is_full;
  int32_t hkv, d;
  // FP8 pools: rows hold E4M3 codes (1 byte per element) read as code * scale; the scales are
  // powers of two, so inv = 1/scale is exact
  int32_t kv_fp8;
  float k_scale, v_scale, k_inv, v_inv;
  // Fused RoPE (rope_fused pools): queries and the call's new keys arrive unrotated and are turned
  // by the kernels at their positions; angle tables as for RopeArgs
  int32_t rope_fused, rope_style;  // style 0: pairs (2i, 2i+1), 1: halves (i, i + d/2)
  const float2 *rope_lo, *rope_hi;
};

// Per-sequence entry of a decode call (uploaded to the workspace).
struct SeqEntry {
  int32_t seq;       // pool sequence id
  int32_t pad;
  int64_t prior;     // committed length L (queries sit at L .. L+q_len-1)
};

// One split-K work item of a decode call: KV head `head` of call sequence `si`, prior keys
// [k_begin, k_end) (page-aligned, except the end), plus the new tokens if `with_new`, for the
// query rows row0 .. row0+31 of the (sequence, KV head) (rows = G query heads x q_len tokens;
// more than 32 rows take several items over the same keys).  The item carries its sequence's pool
// id and committed length too, so a kernel reads them with the item instead of after it.
struct WorkItem {
  int32_t si;
  int32_t head;
  int32_t k_begin;
  int32_t k_end;
  int32_t part;      // partial-result slot, or -1: this item covers the whole row, write `out`
  int32_t with_new;
  int32_t row0 = 0;
  int32_t seq = 0;   // pool sequence id of call sequence si
  int64_t prior = 0; // its committed length L
};

// Combine table: for (si, head), partials [first, first + count).
struct CombineEntry {
  int32_t first;
  int32_t count;
};

// Page-table entry to set on the device: tables[index] = value (index into the arena's tables).
struct TablePatch {
  int64_t index;
  int32_t value;
  int32_t pad;
};

struct CopyJob {
  int64_t src_off, dst_off, bytes;  // byte offsets into the arena; bytes % 16 == 0
};
constexpr int kMaxCopyJobs = 96;  // a fork of a 60-SWA-layer stack (60 rings + partial pages) in one launch
struct CopyList {
  CopyJob job[kMaxCopyJobs];
  int32_t n;
};

// Record `msg` as the calling thread's last error (swa_last_error) and return `code`.
int set_error(int code, const char *msg);

// ------------------------------------------------------------------------------ launchers

hipError_t launch_copy_list(char *arena, const CopyList &jobs, hipStream_t s);
hipError_t launch_clock_probe(int64_t *out, int64_t ticks, int64_t wall_khz, hipStream_t s);
hipError_t launch_table_patch(int32_t *tables, const TablePatch *patches, int32_t n, hipStream_t s);

// Batched commit: sequence entries[i] takes rows [i*n + src_row0, i*n + src_row0 + n_write) of
// k/v ([n_seqs * n][Hkv][d]) at positions prior_i + src_row0 + t.  `es` is the element size of
// k/v (4: fp32, 2: bf16); FP8 pools (L.kv_fp8) take bf16 and quantise.
hipError_t launch_append_batch(const LayerView &L, const SeqEntry *entries, int32_t n_seqs, const void *k,
                               const void *v, int32_t n, int32_t src_row0, int32_t n_write, int es,
                               hipStream_t s);

// Append tokens [src_row0, src_row0 + n_write) of k/v ([n][Hkv][d]) at positions pos0 + row
// (`es` and FP8 as above).
hipError_t launch_append(const LayerView &L, int32_t seq, const void *k, const void *v,
                         int32_t src_row0, int32_t n_write, int64_t pos0, int es,
                         hipStream_t s);

// RoPE of a call's q and k rows, in place (RoFormer rotation, angle tables built on the host).
// Token r of the call sits at position (ent ? ent[r / n].prior : pos0) + r % n.
constexpr int kRopeLoBits = 11;
constexpr int64_t kRopeLo = 1 << kRopeLoBits;  // rows of the low-angle table
struct RopeArgs {
  char *q, *k;            // [tokens][hq][d] and [tokens][hkv][d] in the activation dtype
  char *kout;             // rotated keys go here ([tokens][hkv][d]) instead of back into k, or nullptr
  const SeqEntry *ent;    // per-sequence first position, or nullptr (one sequence at pos0)
  int64_t pos0;
  const float2 *lo_tab;   // [kRopeLo][d/2] (cos, sin) of l * theta_i
  const float2 *hi_tab;   // [..][d/2] (cos, sin) of h * kRopeLo * theta_i
  int32_t tokens, n;      // rows per tensor, tokens per sequence
  int32_t hq, hkv, d;     // hq = 0 / hkv = 0 when q / k is absent
  int32_t style;          // 0: pairs (2i, 2i+1), 1: halves (i, i + d/2)
};
hipError_t launch_rope(const RopeArgs &a, int es, hipStream_t s);

// fp32 generic attention (prefill of one sequence or decode of many; direct, no split).
struct F32AttnArgs {
  LayerView L;
  const float *q, *k_new, *v_new;
  float *out;
  const SeqEntry *seqs;  // device (decode) or nullptr (prefill: single sequence)
  int32_t seq;           // prefill: the sequence; decode: unused
  int64_t prior;         // prefill: committed length
  int32_t n_seqs, q_len, hq;
  float scale_log2;      // log2(e) / sqrt(d)
};
hipError_t launch_attn_f32(const F32AttnArgs &a, hipStream_t s);

// bf16 MFMA prefill (one sequence, chunk of n tokens at positions prior .. prior+n-1).
struct PrefillArgs {
  LayerView L;
  const uint16_t *q, *k, *v;
  uint16_t *out;
  int32_t seq;
  int64_t prior;
  int32_t n, hq;
  float scale_log2;
  int32_t n_cu;  // compute units of the device (sizes the band form's grid)
};
hipError_t launch_prefill_bf16(const PrefillArgs &a, hipStream_t s);

// bf16 MFMA decode over a work list, then (if any item is split) the log-sum-exp combine.
struct DecodeArgs {
  LayerView L;
  const uint16_t *q, *k_new, *v_new;
  uint16_t *out;
  const SeqEntry *seqs;
  const WorkItem *items;
  const CombineEntry *combine;
  float *part_o;   // [n_parts][rows][d]
  float *part_ml;  // [n_parts][rows][2]
  int32_t n_items, n_parts, n_seqs, q_len, hq;
  int32_t max_split;  // most partials of any (sequence, KV head): sizes the combine's workgroups
  float scale_log2;
};
hipError_t launch_decode_bf16(const DecodeArgs &a, hipStream_t s);

}  // namespace swa
