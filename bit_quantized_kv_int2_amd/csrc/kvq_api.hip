// Host side of the C ABI: argument checks (before any HIP call), split
// planning, workspace carving and kernel launches on the caller's stream.
#include <math.h>
#include <string.h>

#include <mutex>

#include "kvq_internal.h"

using namespace kvq;

static thread_local int32_t g_last_hip_error = 0;

static kvq_status hip_status(hipError_t e) {
  if (e == hipSuccess) return KVQ_OK;
  g_last_hip_error = (int32_t)e;
  return KVQ_ERR_HIP;
}

// Per-thread HIP error code set by kvq_debug_inject_hip_error (0: none).
static thread_local int32_t g_inject_hip_error = 0;

// Every entry point calls this once its host checks have passed, right before
// its first HIP call. The launches below report hipGetLastError() after each
// kernel. That state is per thread and shared with every other HIP user in the
// process, so a failure another library left unread (a device query, say)
// would be blamed on this call's launch: it is cleared here. With an injected
// code set, no HIP call is made and the entry point fails with that code.
static kvq_status begin_hip() {
  if (g_inject_hip_error != 0) return hip_status((hipError_t)g_inject_hip_error);
  (void)hipGetLastError();
  return KVQ_OK;
}

static bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// ---- the scratch of decode_attention_quant_noalloc ------------------------
// The split partials (m, l, O) of the allocation-free entry point live in
// this file-scope device array, one copy per GPU, held until the process
// ends. In host code `scratch` names a host-side stand-in, not the device
// copy: its device address comes from hipGetSymbolAddress, resolved once per
// device with that device current, and only that address is ever used.
static __device__ __align__(256) unsigned char scratch[KVQ_NOALLOC_SCRATCH_BYTES];
constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kMaxDevices];

static kvq_status scratch_address(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e);
  if (dev < 0 || dev >= kMaxDevices) return hip_status(hipErrorInvalidDevice);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e);
    if (!p) return hip_status(hipErrorInvalidSymbol);
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return KVQ_OK;
}

extern "C" {

const char* kvq_status_string(kvq_status s) {
  switch (s) {
    case KVQ_OK: return "ok";
    case KVQ_ERR_NULL_POINTER: return "null pointer";
    case KVQ_ERR_BAD_FORMAT: return "unsupported format";
    case KVQ_ERR_BAD_SHAPE: return "bad shape";
    case KVQ_ERR_MISALIGNED: return "device pointer not 16-byte aligned";
    case KVQ_ERR_WORKSPACE: return "workspace too small";
    case KVQ_ERR_HIP: return "HIP launch failed";
  }
  return "unknown status";
}

int32_t kvq_last_hip_error(void) { return g_last_hip_error; }

void kvq_debug_inject_hip_error(int32_t hip_error) { g_inject_hip_error = hip_error; }

uint32_t kvq_build_flags(void) {
#ifdef KVQ_POISON_LDS
  return KVQ_BUILD_POISON_LDS;
#else
  return 0;
#endif
}

uint32_t kvq_layout_version(void) { return KVQ_LAYOUT_VERSION; }

kvq_status kvq_check_format(const kvq_format* f) {
  if (!f) return KVQ_ERR_NULL_POINTER;
  if (f->layout_version != KVQ_LAYOUT_VERSION) return KVQ_ERR_BAD_FORMAT;
  if (f->bits != 2 && f->bits != 4) return KVQ_ERR_BAD_FORMAT;
  if (f->k_axis != KVQ_TOKEN_WISE && f->k_axis != KVQ_CHANNEL_WISE) return KVQ_ERR_BAD_FORMAT;
  if (f->v_axis != KVQ_TOKEN_WISE && f->v_axis != KVQ_CHANNEL_WISE) return KVQ_ERR_BAD_FORMAT;
  if (f->head_dim != kHeadDim) return KVQ_ERR_BAD_FORMAT;
  // 128 everywhere; 32 or 64 channels per group when both axes are token-wise
  // (the one group size then counts channels for K and V; a token's pairs
  // sit with the token, in its page for a paged cache)
  if (f->group != kGroup) {
    if (f->group != 32 && f->group != 64) return KVQ_ERR_BAD_FORMAT;
    if (f->k_axis != KVQ_TOKEN_WISE || f->v_axis != KVQ_TOKEN_WISE) return KVQ_ERR_BAD_FORMAT;
  }
  if (f->num_kv_heads < 1 || f->num_kv_heads > 65535) return KVQ_ERR_BAD_FORMAT;
  if (f->num_q_heads != kGqa * f->num_kv_heads) return KVQ_ERR_BAD_FORMAT;
  if (f->page_size != 0 && f->page_size != kPage) return KVQ_ERR_BAD_FORMAT;
  return KVQ_OK;
}

static int padded_len(int max_len) { return ((max_len + kGroup - 1) / kGroup) * kGroup; }

kvq_status kvq_cache_sizes(const kvq_format* f, int32_t batch, int32_t max_len,
                           int32_t num_pages, size_t bytes[4]) {
  kvq_status st = kvq_check_format(f);
  if (st != KVQ_OK) return st;
  if (!bytes) return KVQ_ERR_NULL_POINTER;
  const size_t H = (size_t)f->num_kv_heads, D = kHeadDim, b = (size_t)f->bits;
  size_t tokens;  // token rows per head-slot array
  size_t groups;  // channel-wise pair rows
  if (f->page_size == 0) {
    if (batch < 0 || max_len < 0) return KVQ_ERR_BAD_SHAPE;
    tokens = (size_t)batch * H * (size_t)padded_len(max_len);
    groups = (size_t)batch * H * (size_t)(padded_len(max_len) / kGroup);
  } else {
    if (num_pages < 0) return KVQ_ERR_BAD_SHAPE;
    tokens = (size_t)num_pages * H * kPage;
    groups = (size_t)num_pages * H;
  }
  bytes[0] = tokens * D * b / 8;
  bytes[1] = tokens * D * b / 8;
  const size_t ng = (size_t)(kHeadDim / f->group);  // token-wise groups per token
  bytes[2] = (f->k_axis == KVQ_TOKEN_WISE ? tokens * ng * 4 : groups * D * 4);
  bytes[3] = (f->v_axis == KVQ_TOKEN_WISE ? tokens * ng * 4 : groups * D * 4);
  return KVQ_OK;
}

// Token split per (sequence, KV head): a multiple of kSplitQuantum tokens.
// A decode work-group walks its split in chunks of kChunkTokens (the fold
// operands of one chunk sit in LDS), so a split may span the whole sequence.
// The automatic plan splits only as far as needed to give the chip one full
// round of resident work-groups (`slots`): a second, partial round of short
// splits costs more than it balances.
static constexpr long kBf16Slots = 1024;

static long quant_slots(const kvq_format* f) {
  const int per_cu = f->group == kGroup ? groups_per_cu(f->bits, f->v_axis) : tg_groups_per_cu(f->bits, kHeadDim / f->group);
  return (long)kComputeUnits * per_cu;
}

static int plan_split_tokens(long slots, int batch, int num_kv_heads, int max_len,
                             int num_splits) {
  if (max_len <= 0) return kSplitQuantum;
  const int quanta = (max_len + kSplitQuantum - 1) / kSplitQuantum;
  if (num_splits <= 0) {
    const long units = (long)batch * num_kv_heads;
    long ns = units > 0 ? (slots + units - 1) / units : 1;
    if (ns > quanta) ns = quanta;
    num_splits = (int)ns;
  }
  const int q_per = (quanta + num_splits - 1) / num_splits;
  return q_per * kSplitQuantum;
}

static int splits_for(int max_len, int split_tokens) {
  if (max_len <= 0) return 1;
  return (max_len + split_tokens - 1) / split_tokens;
}

kvq_status kvq_plan_splits(const kvq_format* f, int32_t batch, int32_t max_len,
                           int32_t* num_splits) {
  kvq_status st = kvq_check_format(f);
  if (st != KVQ_OK) return st;
  if (!num_splits) return KVQ_ERR_NULL_POINTER;
  if (batch < 0 || max_len < 0) return KVQ_ERR_BAD_SHAPE;
  *num_splits = splits_for(max_len, plan_split_tokens(quant_slots(f), batch, f->num_kv_heads,
                                                       max_len, 0));
  return KVQ_OK;
}

// ---- length-aware split plan -------------------------------------------
// The auto plan splits every sequence into about slots / (B H) pieces of
// max_len / that many tokens, which fills the chip exactly when the lengths
// are equal. In a ragged batch (longest > 1.5 x mean), the longest sequence's
// pieces then set the call time while most slots idle. There the split is
// sized to about half the mean work per work-group slot, H sum(L) / (2 slots)
// tokens, in whole 2048-token chunks (at least one, at most the auto plan's
// split): enough pieces that the long sequences leave no tail, few enough that
// the per-split query load, merge and partial write stay small. Among that
// chunk count and its neighbours, a split count that is odd (else 2 mod 4) is
// preferred: an XCD deals its work-groups in turn over its parts, and with a
// count divisible by 4 every row's first split, the one short rows keep busy,
// lands on the same part. (Measured on the 64-sequence log-uniform [1K, 128K]
// paged batch: 15 splits 214 us, 30 splits 224 us, 20 splits 241 us, 12
// splits 259 us for INT2; the auto plan's 2 splits 504 us.)
kvq_status kvq_plan_splits_for_lengths(const kvq_format* f, int32_t batch, int32_t max_len,
                                       const int32_t* seq_lens_host, int32_t* num_splits) {
  kvq_status st = kvq_check_format(f);
  if (st != KVQ_OK) return st;
  if (!num_splits || (batch > 0 && !seq_lens_host)) return KVQ_ERR_NULL_POINTER;
  if (batch < 0 || max_len < 0) return KVQ_ERR_BAD_SHAPE;
  const long slots = quant_slots(f);
  const int auto_tokens = plan_split_tokens(slots, batch, f->num_kv_heads, max_len, 0);
  *num_splits = splits_for(max_len, auto_tokens);
  long total = 0, longest = 0;
  for (int b = 0; b < batch; ++b) {
    long L = seq_lens_host[b] < 0 ? 0 : seq_lens_host[b];
    if (L > max_len) L = max_len;
    total += L;
    if (L > longest) longest = L;
  }
  if (total == 0 || 2 * longest * batch <= 3 * total) return KVQ_OK;  // lengths about equal
  const double target = (double)f->num_kv_heads * (double)total / (2.0 * (double)slots);
  long k0 = (long)(target / kChunkTokens + 0.5);
  if (k0 < 1) k0 = 1;
  const int quanta = (max_len + kSplitQuantum - 1) / kSplitQuantum;
  // chunk counts k0, k0 + 1, k0 - 1: the first with an odd split count, else
  // the first with one that is 2 mod 4, else k0
  int best = -1, best_rank = 3;
  const long ks[3] = {k0, k0 + 1, k0 - 1};
  for (long k : ks) {
    if (k < 1 || k * kChunkTokens >= auto_tokens) continue;
    const int per = (int)(k * kChunkTokens / kSplitQuantum);
    const int req = (quanta + per - 1) / per;
    const int ns = splits_for(max_len, plan_split_tokens(slots, batch, f->num_kv_heads, max_len, req));
    const int rank = ns % 2 ? 0 : (ns % 4 == 2 ? 1 : 2);
    if (rank < best_rank) {
      best_rank = rank;
      best = ns;
    }
  }
  if (best > 0) *num_splits = best;
  return KVQ_OK;
}

static kvq_status resolve_splits(const kvq_format* f, long slots, int batch, int max_len, int req,
                                 int* split_tokens, int* nsplit) {
  if (req < 0) return KVQ_ERR_BAD_SHAPE;
  int quanta = max_len > 0 ? (max_len + kSplitQuantum - 1) / kSplitQuantum : 1;
  if (req > quanta) return KVQ_ERR_BAD_SHAPE;
  *split_tokens = plan_split_tokens(slots, batch, f->num_kv_heads, max_len, req);
  *nsplit = splits_for(max_len, *split_tokens);
  if (decode_grid_blocks((long)batch * f->num_kv_heads, *nsplit) >= kMaxGridBlocks) return KVQ_ERR_BAD_SHAPE;
  return KVQ_OK;
}

// The combine kernel runs batch * Hq work-groups of kHeadDim work-items; the
// whole grid must count its work-items in 32 bits.
static bool combine_grid_fits(const kvq_format* f, int batch) {
  return (long)batch * f->num_q_heads * kHeadDim < (1L << 32);
}

static size_t workspace_bytes_for(const kvq_format* f, int batch, int nsplit) {
  if (nsplit <= 1) return 0;
  const size_t rows = (size_t)batch * f->num_q_heads;
  return rows * nsplit * (kHeadDim + 2) * sizeof(float);
}

// The auto plan of the quantised decode runs on the device (lengths_split)
// when the max_len plan splits the rows (ns_auto >= 2); with one split per
// row (a batch that fills the chip by its rows) the decode keeps that plan.
// The host fixes the device plan's grid and workspace from batch and max_len
// alone. Workspace: a 16-byte header (the split chosen, the plan mode), the
// first work-item of each (sequence, KV head) row, then per work-item
// partials O [4][D] and (m, l) [4] (mode 0 uses them as [row][ns_auto]).
struct AutoPlan {
  int auto_tokens;  // the max_len plan's split
  int ns_auto;      // its split count
  bool device;      // the plan is made on the device
  long items;       // grid (device plan: a bound on the plan's work-items)
  size_t bytes;     // workspace
  size_t row_first_off, part_o_off, part_ml_off;
};

static kvq_status auto_plan_for(const kvq_format* f, int batch, int max_len, AutoPlan* p) {
  const long slots = quant_slots(f);
  p->auto_tokens = plan_split_tokens(slots, batch, f->num_kv_heads, max_len, 0);
  p->ns_auto = splits_for(max_len, p->auto_tokens);
  const long rows = (long)batch * f->num_kv_heads;
  p->device = p->ns_auto >= 2;
  p->items = p->device ? plan_item_bound(rows, p->ns_auto, slots) : decode_grid_blocks(rows, p->ns_auto);
  if (p->items >= kMaxGridBlocks) return KVQ_ERR_BAD_SHAPE;
  p->row_first_off = 16;
  p->part_o_off = p->row_first_off + (((size_t)rows * 4 + 15) / 16) * 16;
  p->part_ml_off = p->part_o_off + (size_t)p->items * kGqa * kHeadDim * sizeof(float);
  p->bytes = p->device ? p->part_ml_off + (size_t)p->items * kGqa * 2 * sizeof(float) : 0;
  return KVQ_OK;
}

kvq_status kvq_auto_plan(const kvq_format* f, int32_t batch, int32_t max_len,
                         const int32_t* seq_lens_host, int32_t* split_tokens, int32_t* items,
                         int32_t* grid) {
  kvq_status st = kvq_check_format(f);
  if (st != KVQ_OK) return st;
  if (!split_tokens || !items || !grid || (batch > 0 && !seq_lens_host)) return KVQ_ERR_NULL_POINTER;
  if (batch < 0 || max_len < 0) return KVQ_ERR_BAD_SHAPE;
  AutoPlan p;
  st = auto_plan_for(f, batch, max_len, &p);
  if (st != KVQ_OK) return st;
  long long total = 0;
  int longest = 0;
  for (int b = 0; b < batch; ++b) {
    int L = seq_lens_host[b] < 0 ? 0 : (seq_lens_host[b] > max_len ? max_len : seq_lens_host[b]);
    total += L;
    if (L > longest) longest = L;
  }
  const int S = p.device ? lengths_split(total, longest, batch, f->num_kv_heads, quant_slots(f), p.auto_tokens)
                         : p.auto_tokens;
  long n = 0;
  for (int b = 0; b < batch; ++b) {
    int L = seq_lens_host[b] < 0 ? 0 : (seq_lens_host[b] > max_len ? max_len : seq_lens_host[b]);
    n += L > 0 ? (long)f->num_kv_heads * ((L + S - 1) / S) : 0;
  }
  *split_tokens = S;
  *items = (int32_t)n;
  *grid = (int32_t)p.items;
  return KVQ_OK;
}

kvq_status kvq_workspace_size(const kvq_format* f, int32_t batch, int32_t max_len,
                              int32_t num_splits, size_t* bytes) {
  kvq_status st = kvq_check_format(f);
  if (st != KVQ_OK) return st;
  if (!bytes) return KVQ_ERR_NULL_POINTER;
  if (batch < 0 || max_len < 0) return KVQ_ERR_BAD_SHAPE;
  // enough for either decode: the quantised and the bf16 plans may differ
  int split_tokens, nq, nb;
  st = resolve_splits(f, quant_slots(f), batch, max_len, num_splits, &split_tokens, &nq);
  if (st != KVQ_OK) return st;
  st = resolve_splits(f, kBf16Slots, batch, max_len, num_splits, &split_tokens, &nb);
  if (st != KVQ_OK) return st;
  *bytes = workspace_bytes_for(f, batch, nq > nb ? nq : nb);
  if (num_splits == 0) {  // the quantised decode's plan on the device
    AutoPlan p;
    st = auto_plan_for(f, batch, max_len, &p);
    if (st != KVQ_OK) return st;
    if (p.bytes > *bytes) *bytes = p.bytes;
  }
  return KVQ_OK;
}

static kvq_status check_cache_ptrs(const kvq_cache* c) {
  if (!c) return KVQ_ERR_NULL_POINTER;
  if (!c->k_codes || !c->v_codes || !c->k_scale_offset || !c->v_scale_offset)
    return KVQ_ERR_NULL_POINTER;
  if (!aligned16(c->k_codes) || !aligned16(c->v_codes) || !aligned16(c->k_scale_offset) ||
      !aligned16(c->v_scale_offset))
    return KVQ_ERR_MISALIGNED;
  return KVQ_OK;
}

static kvq_status check_common(const kvq_format* f, const int32_t* seq_lens,
                               const int32_t* page_table, int32_t max_pages, int32_t batch,
                               int32_t max_len) {
  if (!seq_lens) return KVQ_ERR_NULL_POINTER;
  if (!aligned16(seq_lens)) return KVQ_ERR_MISALIGNED;
  if (batch < 0 || batch > 65535 || max_len < 0 || max_len > (1 << 30)) return KVQ_ERR_BAD_SHAPE;
  if (f->page_size != 0) {
    if (!page_table) return KVQ_ERR_NULL_POINTER;
    if (!aligned16(page_table)) return KVQ_ERR_MISALIGNED;
    if (max_pages < (max_len + kPage - 1) / kPage || max_pages < 1) return KVQ_ERR_BAD_SHAPE;
  }
  return KVQ_OK;
}

kvq_status kv_quantize_pack(const kvq_format* f, const float* k, const float* v,
                            const int32_t* seq_lens, const int32_t* page_table,
                            int32_t max_pages_per_seq, int32_t batch, int32_t max_len,
                            const kvq_cache* out, void* stream) {
  kvq_status st = kvq_check_format(f);
  if (st != KVQ_OK) return st;
  if (!k || !v) return KVQ_ERR_NULL_POINTER;
  if (!aligned16(k) || !aligned16(v)) return KVQ_ERR_MISALIGNED;
  st = check_cache_ptrs(out);
  if (st != KVQ_OK) return st;
  st = check_common(f, seq_lens, page_table, max_pages_per_seq, batch, max_len);
  if (st != KVQ_OK) return st;
  if (batch == 0 || max_len == 0) return KVQ_OK;
  // one work-group per 128-token tile of a (sequence, KV head), counted in 31
  // bits (2^31 tiles would be 128 TiB of fp32 input per tensor)
  if ((long)batch * f->num_kv_heads * (padded_len(max_len) / kGroup) >= (1L << 31))
    return KVQ_ERR_BAD_SHAPE;
  PackArgs a;
  memset(&a, 0, sizeof a);
  a.k = k;
  a.v = v;
  a.seq_lens = seq_lens;
  a.page_table = f->page_size ? page_table : nullptr;
  a.max_pages = max_pages_per_seq;
  a.batch = batch;
  a.max_len = max_len;
  a.num_kv_heads = f->num_kv_heads;
  a.bits = f->bits;
  a.k_axis = f->k_axis;
  a.v_axis = f->v_axis;
  a.paged = f->page_size != 0;
  a.padded_len = padded_len(max_len);
  a.ng = kHeadDim / f->group;
  a.k_codes = (uint8_t*)out->k_codes;
  a.v_words = (uint32_t*)out->v_codes;
  a.k_sz = (uint16_t*)out->k_scale_offset;
  a.v_sz = (uint16_t*)out->v_scale_offset;
  st = begin_hip();
  if (st != KVQ_OK) return st;
  return hip_status(launch_pack(a, (hipStream_t)stream));
}

static kvq_status check_out(const void* q, void* out, int32_t out_dtype) {
  if (!q || !out) return KVQ_ERR_NULL_POINTER;
  if (!aligned16(q) || !aligned16(out)) return KVQ_ERR_MISALIGNED;
  if (out_dtype != KVQ_OUT_F32 && out_dtype != KVQ_OUT_BF16) return KVQ_ERR_BAD_FORMAT;
  return KVQ_OK;
}

static kvq_status decode_quant_impl(const kvq_format* f, const void* q, const kvq_cache* cache,
                                    const int32_t* seq_lens, const int32_t* page_table,
                                    int32_t max_pages_per_seq, int32_t batch, int32_t max_len,
                                    float softmax_scale, void* out, int32_t out_dtype,
                                    int32_t num_splits, void* workspace, size_t workspace_bytes,
                                    void* stream, int fp8_qk, bool use_scratch = false) {
  kvq_status st = kvq_check_format(f);
  if (st != KVQ_OK) return st;
  if (fp8_qk && f->group != kGroup) return KVQ_ERR_BAD_FORMAT;
  st = check_out(q, out, out_dtype);
  if (st != KVQ_OK) return st;
  st = check_cache_ptrs(cache);
  if (st != KVQ_OK) return st;
  st = check_common(f, seq_lens, page_table, max_pages_per_seq, batch, max_len);
  if (st != KVQ_OK) return st;
  if (!(softmax_scale == softmax_scale) || isinf(softmax_scale)) return KVQ_ERR_BAD_SHAPE;
  int split_tokens, nsplit;
  st = resolve_splits(f, quant_slots(f), batch, max_len, num_splits, &split_tokens, &nsplit);
  if (st != KVQ_OK) return st;
  AutoPlan ap;
  bool dev_plan = false;
  if (num_splits == 0) {
    st = auto_plan_for(f, batch, max_len, &ap);
    if (st != KVQ_OK) return st;
    dev_plan = ap.device;
  }
  if ((dev_plan || nsplit > 1) && !combine_grid_fits(f, batch)) return KVQ_ERR_BAD_SHAPE;
  size_t need = dev_plan ? ap.bytes : workspace_bytes_for(f, batch, nsplit);
  if (use_scratch) {
    // every check above is host-only; the scratch address is the first HIP call
    if (need > KVQ_NOALLOC_SCRATCH_BYTES) return KVQ_ERR_WORKSPACE;
    if (batch == 0) return KVQ_OK;
    if (need > 0) {
      st = begin_hip();
      if (st != KVQ_OK) return st;
      st = scratch_address(&workspace);
      if (st != KVQ_OK) return st;
      workspace_bytes = KVQ_NOALLOC_SCRATCH_BYTES;
    }
  }
  if (need > 0) {
    if (!workspace || workspace_bytes < need) return KVQ_ERR_WORKSPACE;
    if (!aligned16(workspace)) return KVQ_ERR_MISALIGNED;
  }
  if (batch == 0) return KVQ_OK;
  DecodeArgs a;
  memset(&a, 0, sizeof a);
  a.q = (const uint16_t*)q;
  a.k_codes = (const uint8_t*)cache->k_codes;
  a.v_words = (const uint32_t*)cache->v_codes;
  a.k_sz = (const uint16_t*)cache->k_scale_offset;
  a.v_sz = (const uint16_t*)cache->v_scale_offset;
  a.seq_lens = seq_lens;
  a.page_table = f->page_size ? page_table : nullptr;
  a.max_pages = max_pages_per_seq;
  a.batch = batch;
  a.num_kv_heads = f->num_kv_heads;
  a.max_len = max_len;
  a.padded_len = padded_len(max_len);
  a.split_tokens = split_tokens;
  a.num_splits = nsplit;
  a.scale_log2 = softmax_scale * 1.4426950408889634f;
  a.out = out;
  a.out_bf16 = out_dtype == KVQ_OUT_BF16;
  a.direct_out = nsplit == 1;
  a.part_stride = nsplit;
  a.fp8_qk = fp8_qk;
  if (dev_plan) {
    unsigned char* w = (unsigned char*)workspace;
    a.dev_plan = 1;
    a.split_tokens = ap.auto_tokens;
    a.num_splits = ap.ns_auto;
    a.plan_items = (int)ap.items;
    a.plan_slots = (int)quant_slots(f);
    a.plan_hdr = (int*)w;
    a.row_first = (int*)(w + ap.row_first_off);
    a.part_o = (float*)(w + ap.part_o_off);
    a.part_ml = (float*)(w + ap.part_ml_off);
  } else if (nsplit > 1) {
    const size_t rows = (size_t)batch * f->num_q_heads;
    a.part_o = (float*)workspace;
    a.part_ml = a.part_o + rows * nsplit * kHeadDim;
  }
  hipStream_t s = (hipStream_t)stream;
  st = begin_hip();
  if (st != KVQ_OK) return st;
  st = hip_status(launch_decode_quant(*f, a, s));
  if (st != KVQ_OK) return st;
  if (dev_plan) return hip_status(launch_combine_plan(a, s));
  if (nsplit == 1) return st;
  return hip_status(launch_combine(a.part_o, a.part_ml, batch * f->num_q_heads, nsplit, out,
                                   a.out_bf16, s));
}

kvq_status decode_attention_quant(const kvq_format* f, const void* q, const kvq_cache* cache,
                                  const int32_t* seq_lens, const int32_t* page_table,
                                  int32_t max_pages_per_seq, int32_t batch, int32_t max_len,
                                  float softmax_scale, void* out, int32_t out_dtype,
                                  int32_t num_splits, void* workspace, size_t workspace_bytes,
                                  void* stream) {
  return decode_quant_impl(f, q, cache, seq_lens, page_table, max_pages_per_seq, batch, max_len,
                           softmax_scale, out, out_dtype, num_splits, workspace, workspace_bytes,
                           stream, 0);
}

kvq_status decode_attention_quant_fp8(const kvq_format* f, const void* q, const kvq_cache* cache,
                                      const int32_t* seq_lens, const int32_t* page_table,
                                      int32_t max_pages_per_seq, int32_t batch, int32_t max_len,
                                      float softmax_scale, void* out, int32_t out_dtype,
                                      int32_t num_splits, void* workspace,
                                      size_t workspace_bytes, void* stream) {
  return decode_quant_impl(f, q, cache, seq_lens, page_table, max_pages_per_seq, batch, max_len,
                           softmax_scale, out, out_dtype, num_splits, workspace, workspace_bytes,
                           stream, 1);
}

kvq_status decode_attention_quant_noalloc(const kvq_format* f, const void* q,
                                          const kvq_cache* cache, const int32_t* seq_lens,
                                          const int32_t* page_table, int32_t max_pages_per_seq,
                                          int32_t batch, int32_t max_len, float softmax_scale,
                                          void* out, int32_t out_dtype, int32_t num_splits,
                                          void* stream) {
  return decode_quant_impl(f, q, cache, seq_lens, page_table, max_pages_per_seq, batch, max_len,
                           softmax_scale, out, out_dtype, num_splits, nullptr, 0, stream, 0, true);
}

kvq_status decode_attention_bf16(const kvq_format* f, const void* q, const void* k,
                                 const void* v, const int32_t* seq_lens,
                                 const int32_t* page_table, int32_t max_pages_per_seq,
                                 int32_t batch, int32_t max_len, float softmax_scale, void* out,
                                 int32_t out_dtype, int32_t num_splits, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  kvq_status st = kvq_check_format(f);
  if (st != KVQ_OK) return st;
  st = check_out(q, out, out_dtype);
  if (st != KVQ_OK) return st;
  if (!k || !v) return KVQ_ERR_NULL_POINTER;
  if (!aligned16(k) || !aligned16(v)) return KVQ_ERR_MISALIGNED;
  st = check_common(f, seq_lens, page_table, max_pages_per_seq, batch, max_len);
  if (st != KVQ_OK) return st;
  if (!(softmax_scale == softmax_scale) || isinf(softmax_scale)) return KVQ_ERR_BAD_SHAPE;
  int split_tokens, nsplit;
  st = resolve_splits(f, kBf16Slots, batch, max_len, num_splits, &split_tokens, &nsplit);
  if (st != KVQ_OK) return st;
  if (nsplit > 1 && !combine_grid_fits(f, batch)) return KVQ_ERR_BAD_SHAPE;
  size_t need = workspace_bytes_for(f, batch, nsplit);
  if (need > 0) {
    if (!workspace || workspace_bytes < need) return KVQ_ERR_WORKSPACE;
    if (!aligned16(workspace)) return KVQ_ERR_MISALIGNED;
  }
  if (batch == 0) return KVQ_OK;
  Bf16Args a;
  memset(&a, 0, sizeof a);
  a.q = (const uint16_t*)q;
  a.k = (const uint16_t*)k;
  a.v = (const uint16_t*)v;
  a.seq_lens = seq_lens;
  a.page_table = f->page_size ? page_table : nullptr;
  a.max_pages = max_pages_per_seq;
  a.batch = batch;
  a.num_kv_heads = f->num_kv_heads;
  a.max_len = max_len;
  a.page_size = f->page_size;
  a.split_tokens = split_tokens;
  a.num_splits = nsplit;
  a.scale_log2 = softmax_scale * 1.4426950408889634f;
  a.out = out;
  a.out_bf16 = out_dtype == KVQ_OUT_BF16;
  a.direct_out = nsplit == 1;
  a.part_stride = nsplit;
  if (nsplit > 1) {
    const size_t rows = (size_t)batch * f->num_q_heads;
    a.part_o = (float*)workspace;
    a.part_ml = a.part_o + rows * nsplit * kHeadDim;
  }
  hipStream_t s = (hipStream_t)stream;
  st = begin_hip();
  if (st != KVQ_OK) return st;
  st = hip_status(launch_decode_bf16(a, s));
  if (st != KVQ_OK || nsplit == 1) return st;
  return hip_status(launch_combine(a.part_o, a.part_ml, batch * f->num_q_heads, nsplit, out,
                                   a.out_bf16, s));
}

kvq_status kv_append(const kvq_format* f, const void* k_new, const void* v_new,
                     const int32_t* seq_lens, const int32_t* page_table, int32_t max_pages_per_seq,
                     int32_t batch, int32_t max_len, const kvq_cache* cache, void* k_window,
                     void* v_window, void* stream) {
  kvq_status st = kvq_check_format(f);
  if (st != KVQ_OK) return st;
  if (!k_new || !v_new || !k_window || !v_window) return KVQ_ERR_NULL_POINTER;
  if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_window) || !aligned16(v_window))
    return KVQ_ERR_MISALIGNED;
  st = check_cache_ptrs(cache);
  if (st != KVQ_OK) return st;
  st = check_common(f, seq_lens, page_table, max_pages_per_seq, batch, max_len);
  if (st != KVQ_OK) return st;
  if (batch == 0 || max_len == 0) return KVQ_OK;
  AppendArgs a;
  memset(&a, 0, sizeof a);
  a.k_new = (const uint16_t*)k_new;
  a.v_new = (const uint16_t*)v_new;
  a.seq_lens = seq_lens;
  a.page_table = f->page_size ? page_table : nullptr;
  a.max_pages = max_pages_per_seq;
  a.batch = batch;
  a.max_len = max_len;
  a.num_kv_heads = f->num_kv_heads;
  a.bits = f->bits;
  a.k_axis = f->k_axis;
  a.v_axis = f->v_axis;
  a.paged = f->page_size != 0;
  a.padded_len = padded_len(max_len);
  a.ng = kHeadDim / f->group;
  a.k_win = (uint16_t*)k_window;
  a.v_win = (uint16_t*)v_window;
  a.k_codes = (uint8_t*)cache->k_codes;
  a.v_words = (uint32_t*)cache->v_codes;
  a.k_sz = (uint16_t*)cache->k_scale_offset;
  a.v_sz = (uint16_t*)cache->v_scale_offset;
  st = begin_hip();
  if (st != KVQ_OK) return st;
  return hip_status(launch_append(a, (hipStream_t)stream));
}

static size_t window_workspace_bytes(const kvq_format* f, int batch, int nsplit) {
  return (size_t)batch * f->num_q_heads * (nsplit + 1) * (kHeadDim + 2) * sizeof(float);
}

kvq_status kvq_window_workspace_size(const kvq_format* f, int32_t batch, int32_t max_len,
                                     int32_t num_splits, size_t* bytes) {
  kvq_status st = kvq_check_format(f);
  if (st != KVQ_OK) return st;
  if (!bytes) return KVQ_ERR_NULL_POINTER;
  if (batch < 0 || max_len < 0) return KVQ_ERR_BAD_SHAPE;
  int split_tokens, nsplit;
  st = resolve_splits(f, quant_slots(f), batch, max_len, num_splits, &split_tokens, &nsplit);
  if (st != KVQ_OK) return st;
  *bytes = window_workspace_bytes(f, batch, nsplit);
  return KVQ_OK;
}

kvq_status decode_attention_quant_window(const kvq_format* f, const void* q,
                                         const kvq_cache* cache, const void* k_window,
                                         const void* v_window, const int32_t* seq_lens,
                                         const int32_t* page_table, int32_t max_pages_per_seq,
                                         int32_t batch, int32_t max_len, float softmax_scale,
                                         void* out, int32_t out_dtype, int32_t num_splits,
                                         void* workspace, size_t workspace_bytes, void* stream) {
  kvq_status st = kvq_check_format(f);
  if (st != KVQ_OK) return st;
  st = check_out(q, out, out_dtype);
  if (st != KVQ_OK) return st;
  st = check_cache_ptrs(cache);
  if (st != KVQ_OK) return st;
  if (!k_window || !v_window) return KVQ_ERR_NULL_POINTER;
  if (!aligned16(k_window) || !aligned16(v_window)) return KVQ_ERR_MISALIGNED;
  st = check_common(f, seq_lens, page_table, max_pages_per_seq, batch, max_len);
  if (st != KVQ_OK) return st;
  if (!(softmax_scale == softmax_scale) || isinf(softmax_scale)) return KVQ_ERR_BAD_SHAPE;
  int split_tokens, nsplit;
  st = resolve_splits(f, quant_slots(f), batch, max_len, num_splits, &split_tokens, &nsplit);
  if (st != KVQ_OK) return st;
  if (!combine_grid_fits(f, batch)) return KVQ_ERR_BAD_SHAPE;  // the window path always merges
  const size_t need = window_workspace_bytes(f, batch, nsplit);
  if (!workspace || workspace_bytes < need) return KVQ_ERR_WORKSPACE;
  if (!aligned16(workspace)) return KVQ_ERR_MISALIGNED;
  if (batch == 0) return KVQ_OK;
  const size_t rows = (size_t)batch * f->num_q_heads;
  const int slots = nsplit + 1;  // the quantised splits, then the window
  float* part_o = (float*)workspace;
  float* part_ml = part_o + rows * slots * kHeadDim;
  const float scale_log2 = softmax_scale * 1.4426950408889634f;
  hipStream_t s = (hipStream_t)stream;

  DecodeArgs a;
  memset(&a, 0, sizeof a);
  a.q = (const uint16_t*)q;
  a.k_codes = (const uint8_t*)cache->k_codes;
  a.v_words = (const uint32_t*)cache->v_codes;
  a.k_sz = (const uint16_t*)cache->k_scale_offset;
  a.v_sz = (const uint16_t*)cache->v_scale_offset;
  a.seq_lens = seq_lens;
  a.page_table = f->page_size ? page_table : nullptr;
  a.max_pages = max_pages_per_seq;
  a.batch = batch;
  a.num_kv_heads = f->num_kv_heads;
  a.max_len = max_len;
  a.padded_len = padded_len(max_len);
  a.split_tokens = split_tokens;
  a.num_splits = nsplit;
  a.scale_log2 = scale_log2;
  a.part_o = part_o;
  a.part_ml = part_ml;
  a.part_stride = slots;
  a.len_mode = 1;  // whole groups from the cache
  st = begin_hip();
  if (st != KVQ_OK) return st;
  st = hip_status(launch_decode_quant(*f, a, s));
  if (st != KVQ_OK) return st;

  Bf16Args w;
  memset(&w, 0, sizeof w);
  w.q = (const uint16_t*)q;
  w.k = (const uint16_t*)k_window;
  w.v = (const uint16_t*)v_window;
  w.seq_lens = seq_lens;
  w.batch = batch;
  w.num_kv_heads = f->num_kv_heads;
  w.max_len = kGroup;  // window rows per (sequence, KV head)
  w.page_size = 0;
  w.split_tokens = kGroup;
  w.num_splits = 1;
  w.scale_log2 = scale_log2;
  w.part_o = part_o;
  w.part_ml = part_ml;
  w.part_stride = slots;
  w.part_base = nsplit;
  w.len_mode = 2;  // the tokens past the last whole group
  st = hip_status(launch_decode_bf16(w, s));
  if (st != KVQ_OK) return st;
  return hip_status(launch_combine(part_o, part_ml, (int)rows, slots, out,
                                   out_dtype == KVQ_OUT_BF16, s));
}

kvq_status kvq_stream_read(const void* data, size_t bytes, uint32_t* sink, void* stream) {
  if (!data || !sink) return KVQ_ERR_NULL_POINTER;
  if (!aligned16(data) || ((uintptr_t)sink & 3u)) return KVQ_ERR_MISALIGNED;
  if (bytes % 16 != 0) return KVQ_ERR_BAD_SHAPE;
  if (bytes == 0) return KVQ_OK;
  kvq_status st = begin_hip();
  if (st != KVQ_OK) return st;
  return hip_status(launch_stream_read(data, bytes, sink, (hipStream_t)stream));
}

kvq_status kvq_issue_probe(int mode, int iters, int blocks, float* out, void* stream) {
  if (!out) return KVQ_ERR_NULL_POINTER;
  if ((uintptr_t)out & 3u) return KVQ_ERR_MISALIGNED;
  if (mode < 0 || mode > 3 || iters < 1 || blocks < 1 || blocks > 65535) return KVQ_ERR_BAD_SHAPE;
  kvq_status st = begin_hip();
  if (st != KVQ_OK) return st;
  return hip_status(launch_issue_probe(mode, iters, blocks, out, (hipStream_t)stream));
}

}  // extern "C"
