// Internal declarations shared by the library's HIP sources (not installed).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "kvq.h"

namespace kvq {

constexpr int kHeadDim = 128;
constexpr int kGroup = 128;
constexpr int kGqa = 4;            // query heads per KV head
constexpr int kPage = 64;          // tokens per page
constexpr int kSplitQuantum = 256; // split lengths are multiples of this
constexpr int kChunkTokens = 2048;    // decode prologue chunk: fold operands in LDS
constexpr int kComputeUnits = 256;    // MI355X

// ---- LDS poison fill (debug build) -----------------------------------------
// Built with KVQ_POISON_LDS defined, each kernel fills its LDS with all-ones
// bytes (NaN in binary16, bf16 and fp32; the largest code in a code byte)
// before its first write, and again at the top of every pass of a
// work-group-uniform loop that reuses the LDS. A read of a byte that the
// kernel (or that pass) did not write first then shows up in the output.
// Every thread of the work-group must make the call: it holds two barriers.
// In a normal build it compiles to nothing.
template <int THREADS>
__device__ __forceinline__ void poison_lds(void* p, int bytes) {
#ifdef KVQ_POISON_LDS
  __syncthreads();  // earlier readers of this LDS are done
  uint32_t* w = (uint32_t*)p;
  for (int i = (int)__builtin_amdgcn_workitem_id_x(); i < bytes / 4; i += THREADS) w[i] = ~0u;
  __syncthreads();
#else
  (void)p;
  (void)bytes;
#endif
}

// Resident 256-thread decode work-groups per CU that the register allocation
// targets (the kernels' launch bounds; 4 leave 128 VGPRs per lane, 3 leave
// 168): INT2 fits in 128 (with channel-wise V, whose per-group partials take
// a second set of accumulator tiles, by folding them in two halves of 4
// tiles; a few set-up values of the channel-wise-K and paged variants then
// live in scratch from the prologue to the final merge, outside the loops);
// INT4 holds twice the codes. The split planner sizes grids by the same
// numbers.
constexpr int groups_per_cu(int bits, int /*v_axis*/) { return bits == 2 ? 4 : 3; }
// Token-wise groups of 32 / 64 channels: INT2 with two groups per token fits
// in 128 VGPRs (4 per CU); INT2 with four groups and INT4 with two take 3;
// INT4 with four groups per token, whose per-group accumulators need the 256
// VGPRs of 2, takes 2.
constexpr int tg_groups_per_cu(int bits, int ng) {
  return bits == 2 ? (ng == 2 ? 4 : 3) : (ng == 4 ? 2 : 3);
}

// Code positions inside a 64-token block (layout_version 2). The decode
// kernels load a block as 1 KB pieces, lane l taking bytes 16 l .. 16 l + 15
// of each piece, and these maps put there what lane l needs: the K row of
// the token its MFMA row handles, and the V words of its channels.
// Lane of token u (0..63) in the K loads: 16 floor(u / 16) + rho(u mod 16).
__host__ __device__ constexpr int k_lane_of(int bits, int u) {
  const int v = u & 15;
  const int rho = bits == 4 ? 8 * (v >> 3) + 2 * (v & 3) + ((v >> 2) & 1) : 2 * (v & 7) + (v >> 3);
  return 16 * (u >> 4) + rho;
}
// Byte offset in the block of byte o of token u's K row.
__host__ __device__ constexpr int k_block_byte(int bits, int u, int o) {
  return 1024 * (o >> 4) + 16 * k_lane_of(bits, u) + (o & 15);
}
// Word offset in the block of the V word of word-row r (tokens tpw r ..
// tpw r + tpw - 1), channel d: lane 16 (r mod 4) + floor(d / 8) holds
// channels 8 floor(d / 8) .. + 7 of rows r and r + 4.
__host__ __device__ constexpr int v_block_word(int r, int d) {
  return 512 * (r >> 2) + 256 * ((d >> 2) & 1) + 64 * (r & 3) + 4 * (d >> 3) + (d & 3);
}

// Launch arguments of the append (one new token per sequence, one layer).
struct AppendArgs {
  const uint16_t* k_new;   // bf16 [B][Hkv][D]
  const uint16_t* v_new;
  const int32_t* seq_lens; // tokens before the append
  const int32_t* page_table;
  int max_pages;
  int batch;
  int max_len;
  int num_kv_heads;
  int bits;
  int k_axis;
  int v_axis;
  int paged;
  int padded_len;
  int ng;                  // token-wise (s, z) pairs per token: 128 / group
  uint16_t* k_win;         // bf16 [B][Hkv][128][D]
  uint16_t* v_win;
  uint8_t* k_codes;
  uint32_t* v_words;
  uint16_t* k_sz;
  uint16_t* v_sz;
};

// Work-groups of a decode launch: ns splits of each of the B H rows (row =
// b H + h), on a 1-D grid. Work-groups are dealt to the 8 XCDs in turn, so the
// one at launch index i runs on XCD i mod 8. Index i is read as position
// p = i / 8 in the queue of XCD k = i mod 8, and that queue takes rows k, k + 8,
// k + 16, ..., the ns splits of a row one after another. Every XCD then gets
// the same number of rows (with 8 KV heads, one head of every sequence: the
// same work even when the lengths are ragged), while a (split, head, sequence)
// grid with the split fastest would put split s of every row on XCD
// (s + X r) mod 8 for X columns, the same few XCDs for the rows' first splits
// whenever X is even. Index counts are padded to whole rounds of 8 rows; the
// padding work-groups return at once.
inline long decode_grid_blocks(long rows, int ns) { return ((rows + 7) / 8) * 8 * (long)ns; }
constexpr long kMaxGridBlocks = 1L << 24;  // 256-thread work-groups: a grid must stay below it (32-bit work-item count)
struct WorkItem {
  int sp, h, b;
  bool live;
};
__device__ inline WorkItem work_item(unsigned i, unsigned H, unsigned B, unsigned ns) {
  const unsigned k = i & 7u, p = i >> 3;
  const unsigned row = k + 8u * (p / ns);
  return WorkItem{(int)(p % ns), (int)(row % H), (int)(row / H), row < H * B};
}

// ---- the auto plan from the lengths (num_splits = 0) ----------------------
// When the max_len plan splits the rows (fewer (sequence, KV head) rows than
// resident work-group slots), the quantised decode with num_splits = 0 plans
// on the device, from the lengths in seq_lens, with no host synchronisation:
// every work-group derives the same plan. The split is
//   * with lengths about equal (longest <= 1.5 x mean, or all empty): the
//     max_len plan's split `auto_tokens`, on the max_len plan's grid;
//   * otherwise H sum(L) / (2 slots) tokens rounded up to whole 2048-token
//     chunks (about two splits per resident work-group slot, so that the
//     longest sequences leave no tail), when that is below auto_tokens; the
//     work-items (one per work-group) run over the sequences, then their KV
//     heads, then a row's splits.
// The grid covers both: max(the max_len grid, 2 slots + rows); with the
// length split S >= H sum(L) / (2 slots), sum_b H ceil(L_b / S) <= 2 slots +
// rows. Work-groups past the plan's items return at once.
__host__ __device__ inline int lengths_split(long long total, int longest, int batch, int heads,
                                             long long slots, int auto_tokens) {
  if (total <= 0 || 2LL * longest * batch <= 3LL * total) return auto_tokens;
  const long long den = 2LL * slots;
  const long long t = ((long long)heads * total + den - 1) / den;
  long long k = (t + kChunkTokens - 1) / kChunkTokens;
  if (k < 1) k = 1;
  return k * kChunkTokens < auto_tokens ? (int)(k * kChunkTokens) : auto_tokens;
}
inline long plan_item_bound(long rows, int ns_auto, long slots) {
  const long by_grid = decode_grid_blocks(rows, ns_auto), by_slots = 2 * slots + rows;
  return by_grid > by_slots ? by_grid : by_slots;
}

// Launch arguments of the quantised decode (one layer).
struct DecodeArgs {
  const uint16_t* q;       // bf16 [B][Hq][D]
  const uint8_t* k_codes;
  const uint32_t* v_words;
  const uint16_t* k_sz;
  const uint16_t* v_sz;
  const int32_t* seq_lens;
  const int32_t* page_table;
  int max_pages;
  int batch;
  int num_kv_heads;
  int max_len;             // sequence lengths are clamped to [0, max_len]
  int padded_len;          // contiguous Lp
  int split_tokens;        // multiple of kSplitQuantum
  int num_splits;
  float scale_log2;        // softmax_scale * log2(e)
  float* part_o;           // [B][Hq][part_stride][D]   (partials)
  float* part_ml;          // [B][Hq][part_stride][2]
  void* out;               // final output when direct_out
  int out_bf16;
  int direct_out;          // 1: one split, write out; 0: write partial slot part_base + split
  int part_stride;         // partial slots per (sequence, query head)
  int part_base;
  int len_mode;            // 0: L = seq_lens[b]; 1: L rounded down to whole 128-token groups
  int fp8_qk;              // 1: q.K^T on fp8 (E4M3) operands, hi/lo query parts
  // the auto plan on the device (dev_plan = 1): split_tokens / num_splits are
  // the max_len plan's, the grid has plan_items work-groups; partials are
  // [row][num_splits] (plan mode 0) or per work-item (mode 1), part_o
  // [item][4][D], part_ml [item][4][2]
  int dev_plan;
  int plan_items;
  int plan_slots;          // resident work-group slots of the kernel on the chip
  int* plan_hdr;           // [0]: the split chosen, [1]: plan mode (written by work-group 0)
  int* row_first;          // [B][Hkv]: item of a row's first split (mode 1, rows with >= 2 splits)
};

struct Bf16Args {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const int32_t* seq_lens;
  const int32_t* page_table;
  int max_pages;
  int batch;
  int num_kv_heads;
  int max_len;
  int page_size;
  int split_tokens;
  int num_splits;
  float scale_log2;
  float* part_o;
  float* part_ml;
  void* out;
  int out_bf16;
  int direct_out;          // as DecodeArgs
  int part_stride;
  int part_base;
  int len_mode;            // 0: L = seq_lens[b]; 2: L mod 128 (the tokens of a residual window)
};

struct PackArgs {
  const float* k;
  const float* v;
  const int32_t* seq_lens;
  const int32_t* page_table;
  int max_pages;
  int batch;
  int max_len;
  int num_kv_heads;
  int bits;
  int k_axis;
  int v_axis;
  int paged;
  int padded_len;
  int ng;                  // token-wise (s, z) pairs per token: 128 / group
  uint8_t* k_codes;
  uint32_t* v_words;
  uint16_t* k_sz;
  uint16_t* v_sz;
};

// Kernel launchers (return the hipError_t of the launch).
hipError_t launch_pack(const PackArgs& a, hipStream_t s);
hipError_t launch_decode_quant(const kvq_format& f, const DecodeArgs& a, hipStream_t s);
// token-wise K and V with 32 or 64 channels per group (contiguous caches)
hipError_t launch_decode_quant_tg(const kvq_format& f, const DecodeArgs& a, hipStream_t s);
hipError_t launch_decode_bf16(const Bf16Args& a, hipStream_t s);
hipError_t launch_combine(const float* part_o, const float* part_ml, int rows, int num_splits,
                          void* out, int out_bf16, hipStream_t s);
// merge of a device-planned call: every (sequence, query head) row with two or
// more splits; zeros for empty rows (rows with one split were written by the decode)
hipError_t launch_combine_plan(const DecodeArgs& a, hipStream_t s);

hipError_t launch_append(const AppendArgs& a, hipStream_t s);
// Reads bytes (a multiple of 16) once; the HBM read reference for measurement.
hipError_t launch_stream_read(const void* data, size_t bytes, uint32_t* sink, hipStream_t s);
hipError_t launch_issue_probe(int mode, int iters, int blocks, float* out, hipStream_t s);

}  // namespace kvq
