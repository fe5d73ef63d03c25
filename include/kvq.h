/*
 * kvq.h -- C ABI of the MI355X (gfx950) INT2/INT4 decode-attention library.
 *
 * Single-token decode attention, softmax(scale * q.K^T) . V with grouped
 * query heads, read directly from KV caches quantised to 2 or 4 bits with a
 * per-group scale s and offset z (x ~ s*c + z), groups token-wise or
 * channel-wise independently for K and V. The scale and offset are folded
 * into the other operand or the partial products instead of dequantising
 * each element (FOSCAR, arXiv:2611.09722: abstract; grafy.ai "What is FOSCAR
 * and how does it work?"; rag-lover.com explainer on acc-fold/operand-fold).
 *
 * Conventions shared by every entry point
 *   - Device pointers are plain device addresses (hipMalloc or a framework's
 *     allocator), 16-byte aligned. The caller owns every buffer; the library
 *     never allocates or frees device memory.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Calls are asynchronous on that stream and never synchronise it.
 *   - All argument checks are synchronous, run on the host before any HIP
 *     call, and launch nothing on failure. A failed launch returns
 *     KVQ_ERR_HIP (kvq_last_hip_error() gives the hipError_t of the calling
 *     thread). A device fault shows up at the caller's next synchronisation.
 *   - seq_lens lives in device memory; max_len (host) is an upper bound,
 *     0 <= seq_lens[b] <= max_len. A length of 0 gives a zero output row.
 *   - No state is kept between calls except the thread-local last HIP error
 *     (and, for decode_attention_quant_noalloc only, its per-GPU scratch).
 *
 * Cache layout (layout_version 2; little-endian; D = head_dim = 128, b = bits,
 * G = group, tpw = 32/b tokens per V word, Lp = max_len rounded up to a
 * multiple of 128; paged caches use 64-token pages):
 *   Codes are stored in 64-token blocks: one page, or tokens 64k .. 64k + 63
 *   of a contiguous sequence. Within a block, u = token index (0..63).
 *   K codes   contiguous [B][Hkv][Lp/64][64*D*b/8] bytes; paged [P][Hkv][64*D*b/8].
 *             Token u's row of D*b/8 bytes holds channel d at bit b*d. Byte o
 *             of that row sits at block offset
 *               1024*floor(o/16) + 16*lambda(u) + (o mod 16),
 *               lambda(u) = 16*floor(u/16) + rho(u mod 16),
 *               INT4: rho(v) = 8*floor(v/8) + 2*(v mod 4) + (floor(v/4) mod 2)
 *               INT2: rho(v) = 2*(v mod 8) + floor(v/8)
 *             (each 16-byte piece goes where one 64-lane load of 1 KB finds it).
 *   V codes   contiguous [B][Hkv][Lp/64][(64/tpw)*D] uint32; paged
 *             [P][Hkv][(64/tpw)*D]. Word-row r of a block holds tokens
 *             tpw*r .. tpw*r + tpw - 1; its word for channel d holds token
 *             tpw*r + j at bit b*j and sits at block word
 *               512*floor(r/4) + 256*(floor(d/4) mod 2) + 64*(r mod 4)
 *               + 4*floor(d/8) + (d mod 4).
 *   (s, z)    binary16 pairs, s first.
 *             token-wise:   contiguous [B][Hkv][Lp][D/G][2]; paged [P][Hkv][64][D/G][2]
 *             channel-wise: contiguous [B][Hkv][Lp/G][D][2]; paged [P][Hkv][D][2],
 *                           a 128-token group's pairs in the page that holds
 *                           its first token (the other page's slot is unused).
 *   Quantisation of a group: s = fp16((max - min) / (2^b - 1)) with an fp32
 *   division, z = fp16(min), c = clamp(rint((x - z) / s), 0, 2^b - 1) in fp32
 *   with the stored s and z (c = 0 when s == 0); min and max order -0 below
 *   +0, and the values are finite. Codes of tokens at or past a
 *   sequence's length, within the written extent, are 0.
 */
#ifndef KVQ_H
#define KVQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KVQ_LAYOUT_VERSION 2u

typedef enum {
  KVQ_OK = 0,
  KVQ_ERR_NULL_POINTER = 1, /* a required pointer is NULL */
  KVQ_ERR_BAD_FORMAT = 2,   /* unsupported bits/axes/group/head_dim/heads/page size/version */
  KVQ_ERR_BAD_SHAPE = 3,    /* batch, max_len, pages or splits out of range */
  KVQ_ERR_MISALIGNED = 4,   /* a device pointer is not 16-byte aligned */
  KVQ_ERR_WORKSPACE = 5,    /* workspace missing or smaller than kvq_workspace_size() */
  KVQ_ERR_HIP = 6           /* a HIP launch failed; see kvq_last_hip_error() */
} kvq_status;

typedef enum { KVQ_TOKEN_WISE = 0, KVQ_CHANNEL_WISE = 1 } kvq_axis;
typedef enum { KVQ_OUT_F32 = 0, KVQ_OUT_BF16 = 1 } kvq_out_dtype;

typedef struct {
  int32_t bits;         /* 2 or 4 */
  int32_t k_axis;       /* kvq_axis of K's groups */
  int32_t v_axis;       /* kvq_axis of V's groups */
  int32_t group;        /* 128; or 32 / 64 channels per group when K and V are
                           both token-wise (contiguous or paged) */
  int32_t head_dim;     /* 128 */
  int32_t num_kv_heads; /* >= 1 */
  int32_t num_q_heads;  /* 4 * num_kv_heads (query head hq reads KV head hq / 4) */
  int32_t page_size;    /* 0 = contiguous cache, 64 = paged cache */
  uint32_t layout_version; /* must be KVQ_LAYOUT_VERSION */
} kvq_format;

/* Device pointers to one layer's packed cache (layout above). */
typedef struct {
  void* k_codes;
  void* v_codes;
  void* k_scale_offset;
  void* v_scale_offset;
} kvq_cache;

/* Host-only helpers (no GPU needed). */
const char* kvq_status_string(kvq_status s);
int32_t kvq_last_hip_error(void);
uint32_t kvq_layout_version(void);

/* Test hook for the failure path, usable without a GPU. While hip_error is
 * non-zero, every entry point that would call HIP runs its host checks as
 * usual and then, in place of its first HIP call, returns KVQ_ERR_HIP with
 * kvq_last_hip_error() == hip_error; it makes no HIP call and launches
 * nothing. Argument errors still come first. 0 switches the hook off (the
 * default). Per calling thread. The pages define no failure handling; this
 * only exercises the library's own error reporting. */
void kvq_debug_inject_hip_error(int32_t hip_error);

/* Build variant bits (host-only). KVQ_BUILD_POISON_LDS: the debug build in
 * which every kernel fills its LDS with all-ones bytes before first use, so a
 * read of LDS that the kernel did not write first turns its output into
 * NaN or wrong codes; it computes the same results as the normal build. */
#define KVQ_BUILD_POISON_LDS 1u
uint32_t kvq_build_flags(void);

/* Checks a format; KVQ_OK if the library supports it. */
kvq_status kvq_check_format(const kvq_format* fmt);

/* Byte sizes of the four cache arrays (k_codes, v_codes, k_scale_offset,
 * v_scale_offset). Contiguous caches use batch and max_len; paged caches use
 * num_pages (pool slots of 64 tokens each). */
kvq_status kvq_cache_sizes(const kvq_format* fmt, int32_t batch, int32_t max_len,
                           int32_t num_pages, size_t bytes[4]);

/* Split-KV plan from batch and max_len alone: the number of token splits per
 * (sequence, KV head) that fills the chip when every sequence is max_len long.
 * decode_attention_bf16 uses it for num_splits = 0; the quantised decode's
 * auto plan (kvq_auto_plan) starts from it. */
kvq_status kvq_plan_splits(const kvq_format* fmt, int32_t batch, int32_t max_len,
                           int32_t* num_splits);

/* Split-KV plan for a batch whose sequence lengths the caller knows on the
 * host (a serving engine's scheduler does): the num_splits to pass to
 * decode_attention_quant. Part of the decode's scheduling step: the pages put
 * the kernel into a serving engine whose batches mix long and short contexts
 * (FOSCAR arXiv:2611.09722; grafy.ai "How can developers integrate FOSCAR").
 * The auto plan sizes splits from max_len alone, which fills the chip when the
 * lengths are equal, and this returns the auto plan's count then. When the
 * longest length exceeds 1.5x the mean, it returns a count whose splits are
 * whole 2048-token chunks, about H * sum(len) / (2 * work-group slots) tokens
 * long (the chunk count k0 nearest that, or k0 +- 1 where that makes the split
 * count odd, else 2 mod 4; never longer than the auto plan's split), so that
 * the longest sequences do not set the call time. seq_lens_host: [batch] int32
 * in host memory (entries clamped to [0, max_len]); may be NULL when
 * batch == 0. Pure host computation: no GPU call, no allocation. Errors:
 * KVQ_ERR_NULL_POINTER, KVQ_ERR_BAD_SHAPE, or the format's. */
kvq_status kvq_plan_splits_for_lengths(const kvq_format* fmt, int32_t batch, int32_t max_len,
                                       const int32_t* seq_lens_host, int32_t* num_splits);

/* The quantised decode's auto plan (num_splits = 0), which the decode derives
 * on the device from the lengths in seq_lens, with no host synchronisation
 * (a drop-in decode step: grafy.ai "How can developers integrate FOSCAR into
 * their LLM serving stacks?"). Every (sequence, KV head) row is cut into
 * splits of split_tokens tokens:
 *   - lengths about equal (the longest at most 1.5x the mean, or all 0): the
 *     split of kvq_plan_splits (batch, max_len);
 *   - otherwise H * sum(len) / (2 * work-group slots) tokens rounded up to
 *     whole 2048-token chunks, when shorter than that split: the longest
 *     sequences then do not set the call time.
 * The plan is made on the device when the kvq_plan_splits count is 2 or more
 * (fewer (sequence, KV head) rows than resident work-groups); with one split
 * per row the rows alone fill the chip and the decode keeps that plan (no
 * merge step, no workspace). A row with one split writes its output in the
 * decode; rows with more are merged by a second kernel. This host copy of the
 * rule reports the plan for
 * lengths known on the host: split_tokens, items (the splits, summed over
 * rows) and grid (the work-groups the call launches, a bound on items that
 * depends on batch and max_len only). seq_lens_host: [batch] int32 in host
 * memory, entries clamped to [0, max_len]; may be NULL when batch == 0. Pure
 * host computation. Errors: KVQ_ERR_NULL_POINTER, KVQ_ERR_BAD_SHAPE, or the
 * format's. */
kvq_status kvq_auto_plan(const kvq_format* fmt, int32_t batch, int32_t max_len,
                         const int32_t* seq_lens_host, int32_t* split_tokens, int32_t* items,
                         int32_t* grid);

/* Workspace bytes decode_attention_quant / decode_attention_bf16 need for a
 * given split count (0 = the auto plan; when the quantised decode plans on
 * the device: a 16-byte header, one int32 per (sequence, KV head) and per
 * work-item partials, grid x 4 x (128 + 2) floats). */
kvq_status kvq_workspace_size(const kvq_format* fmt, int32_t batch, int32_t max_len,
                              int32_t num_splits, size_t* bytes);

/*
 * kv_quantize_pack -- quantise and pack one layer's K and V into the cache.
 * Producer side of the format the decode reads (grafy.ai "How can developers
 * integrate": the cache must be quantised with the required group-wise
 * scale/offset layout; the grouping choices follow rag-lover.com
 * "conditions of use").
 *   k, v        device fp32 [batch][Hkv][max_len][D], row-major.
 *   seq_lens    device int32 [batch].
 *   page_table  device int32 [batch][max_pages_per_seq] (physical page of each
 *               64-token logical page) for paged formats, NULL for contiguous.
 *   out         cache to write: every token row / word / pair of every page a
 *               sequence references (contiguous: its whole padded extent),
 *               zeros past the sequence length.
 * Bit-exact with the documented quantisation rule.
 */
kvq_status kv_quantize_pack(const kvq_format* fmt, const float* k, const float* v,
                            const int32_t* seq_lens, const int32_t* page_table,
                            int32_t max_pages_per_seq, int32_t batch, int32_t max_len,
                            const kvq_cache* out, void* stream);

/*
 * decode_attention_quant -- one query token per sequence against the packed
 * cache, with the affine folds (token-wise K: scale the partial q.K^T and add
 * z times the query sum; channel-wise K: fold s into q and add the offset
 * after the product; token-wise V: fold s into P with a per-head offset;
 * channel-wise V: scale each 128-token group's partial P.V, never across
 * groups -- rag-lover.com explainer and limits section).
 *   q           device bf16 [batch][Hq][D].
 *   cache       packed cache in fmt's layout.
 *   softmax_scale  multiplies q.K^T (e.g. 1/sqrt(D)).
 *   out         device [batch][Hq][D], fp32 or bf16 per out_dtype.
 *   num_splits  token splits per (sequence, KV head); 0 = the auto plan,
 *               made on the device from seq_lens (kvq_auto_plan).
 *   workspace   device scratch of at least kvq_workspace_size() bytes.
 */
kvq_status decode_attention_quant(const kvq_format* fmt, const void* q, const kvq_cache* cache,
                                  const int32_t* seq_lens, const int32_t* page_table,
                                  int32_t max_pages_per_seq, int32_t batch, int32_t max_len,
                                  float softmax_scale, void* out, int32_t out_dtype,
                                  int32_t num_splits, void* workspace, size_t workspace_bytes,
                                  void* stream);

/*
 * decode_attention_quant_fp8 -- decode_attention_quant on fp8 / fp4 matrix
 * operands (v_mfma_scale_f32_16x16x128_f8f6f4), the analogue of the pages'
 * Blackwell path that injects codes into the low bits of E4M3 / E2M1
 * (rag-lover.com explainer). A 2- or 4-bit code masked into its byte is the
 * E4M3 value code * 2^-9 (exact, codes < 16), a 2-bit code masked into its
 * nibble the E2M1 value code / 2 (INT2 K codes take this form), so one
 * 128-deep product takes 32 channels of a token (q.K^T) or 16 tokens of two
 * channels (P.V); codes enter the product exactly.
 *   q.K^T: the query side is an E4M3 pair hi + lo / 16 of q * s
 *   (channel-wise K) or q (token-wise K): at least 8 significant bits
 *   (relative error <= 2^-8, the precision of a bf16 operand), exactly q for
 *   token-wise K; the channel-wise-K offset sum uses the same rounded pair.
 *   P.V: the probabilities (P * s for token-wise V, P for channel-wise V)
 *   are E4M3 pairs hi + lo / 16 in the rows of the product (hi and lo rows
 *   summed once at the end). Token-wise V: the offset sum over tokens from the
 *   rounded pair. Channel-wise V: each 64-token step's products are folded
 *   with its group's scale and offset, the offset weighted by the sum of the
 *   same rounded pairs (a fifth product against code 1).
 * Numeric bound: the output meets rel-L2 <= 4e-3 and max-abs <= 2e-2 against
 * the fp64 oracle, the same gate as decode_attention_quant.
 *   Formats with groups of 128 only (others: KVQ_ERR_BAD_FORMAT); all other
 *   arguments, workspace and split plan as decode_attention_quant.
 */
kvq_status decode_attention_quant_fp8(const kvq_format* fmt, const void* q,
                                      const kvq_cache* cache, const int32_t* seq_lens,
                                      const int32_t* page_table, int32_t max_pages_per_seq,
                                      int32_t batch, int32_t max_len, float softmax_scale,
                                      void* out, int32_t out_dtype, int32_t num_splits,
                                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * decode_attention_quant_noalloc -- decode_attention_quant for callers that
 * cannot allocate device memory or pass a workspace (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation). The
 * per-split partials go to a device array of KVQ_NOALLOC_SCRATCH_BYTES that
 * the library holds on every GPU it runs on until the process ends; the call
 * itself allocates nothing (no hipMalloc, no allocating library routine).
 *   Arguments as decode_attention_quant without the workspace; the current
 *   device must be the one the stream runs on.
 *   Limit: the split partials must fit, batch * Hq * splits * (D + 2) * 4
 *   bytes <= KVQ_NOALLOC_SCRATCH_BYTES (kvq_workspace_size() gives the
 *   figure); larger calls return KVQ_ERR_WORKSPACE before any HIP call. One
 *   split needs no scratch.
 *   The array keeps the last call's contents; nothing in it needs clearing
 *   (every split writes its partial before the merge reads it). Calls on
 *   one GPU share the array: calls that may overlap in time (different
 *   streams, or threads) race and must be serialised by the caller.
 *   Errors as decode_attention_quant; KVQ_ERR_HIP also if the array's device
 *   address cannot be resolved (first call on a device).
 */
#define KVQ_NOALLOC_SCRATCH_BYTES (32u << 20)
kvq_status decode_attention_quant_noalloc(const kvq_format* fmt, const void* q,
                                          const kvq_cache* cache, const int32_t* seq_lens,
                                          const int32_t* page_table, int32_t max_pages_per_seq,
                                          int32_t batch, int32_t max_len, float softmax_scale,
                                          void* out, int32_t out_dtype, int32_t num_splits,
                                          void* stream);

/*
 * decode_attention_bf16 -- the same decode over an unquantised bf16 cache:
 * the BF16-cache decode the pages measure the quantised kernels against
 * (rag-lover.com 既存手法との違い; grafy.ai "What performance gains does
 * FOSCAR deliver?"). Bits and axes of fmt are ignored.
 *   k, v        device bf16: contiguous [batch][Hkv][max_len][D], paged
 *               [P][Hkv][64][D].
 *   other arguments as decode_attention_quant.
 */
kvq_status decode_attention_bf16(const kvq_format* fmt, const void* q, const void* k,
                                 const void* v, const int32_t* seq_lens,
                                 const int32_t* page_table, int32_t max_pages_per_seq,
                                 int32_t batch, int32_t max_len, float softmax_scale, void* out,
                                 int32_t out_dtype, int32_t num_splits, void* workspace,
                                 size_t workspace_bytes, void* stream);

/*
 * kv_append -- decode-time quantise-on-write of one new token per sequence.
 * A serving engine fills the cache as tokens are generated (grafy.ai "How can
 * developers integrate FOSCAR into their LLM serving stacks?"); a channel-wise
 * group needs all of its 128 tokens before its (s, z) exist (rag-lover.com
 * "conditions of use": each group shares one s and z), so the tokens past the
 * last whole group stay in a bf16 residual window and a group is quantised
 * when its last token arrives. The pages do not describe this step; the
 * residual window is this library's reading.
 *   k_new, v_new  device bf16 [batch][Hkv][D]: the new token of every sequence.
 *   seq_lens      device int32 [batch]: tokens BEFORE this append; the new token
 *                 gets index seq_lens[b] (the caller then increments it).
 *                 Sequences with seq_lens[b] >= max_len are left untouched.
 *   k_window, v_window  device bf16 [batch][Hkv][128][D]: token t of a sequence
 *                 lives in row t % 128 while t >= 128 * floor(len / 128).
 *   cache         packed cache (fmt's layout, contiguous or paged): when index
 *                 seq_lens[b] completes a 128-token group, that group's codes and
 *                 (s, z) are written, bit-identical to kv_quantize_pack applied to
 *                 the window's bf16 values; nothing else in the cache changes.
 * Whole groups of a prompt may be written with kv_quantize_pack (lengths rounded
 * down to a multiple of 128) and its remaining tokens appended one by one.
 */
kvq_status kv_append(const kvq_format* fmt, const void* k_new, const void* v_new,
                     const int32_t* seq_lens, const int32_t* page_table,
                     int32_t max_pages_per_seq, int32_t batch, int32_t max_len,
                     const kvq_cache* cache, void* k_window, void* v_window, void* stream);

/* Workspace bytes decode_attention_quant_window needs (its quantised splits
 * plus one slot for the window). */
kvq_status kvq_window_workspace_size(const kvq_format* fmt, int32_t batch, int32_t max_len,
                                     int32_t num_splits, size_t* bytes);

/*
 * decode_attention_quant_window -- decode over a cache filled by kv_append:
 * tokens [0, L - L % 128) from the packed cache with the affine folds (as
 * decode_attention_quant), tokens [L - L % 128, L) from the bf16 window (as
 * decode_attention_bf16), merged with the same log-sum-exp combine.
 *   seq_lens      device int32 [batch]: total tokens L (cache + window).
 *   workspace     at least kvq_window_workspace_size() bytes (always needed).
 *   other arguments as decode_attention_quant.
 */
kvq_status decode_attention_quant_window(const kvq_format* fmt, const void* q,
                                         const kvq_cache* cache, const void* k_window,
                                         const void* v_window, const int32_t* seq_lens,
                                         const int32_t* page_table, int32_t max_pages_per_seq,
                                         int32_t batch, int32_t max_len, float softmax_scale,
                                         void* out, int32_t out_dtype, int32_t num_splits,
                                         void* workspace, size_t workspace_bytes, void* stream);

/*
 * kvq_stream_read -- measurement reference, not part of the method: reads
 * `bytes` of device memory once with 128-bit non-temporal loads (up to 1024
 * work-groups, each a contiguous range) and nothing else, giving the
 * practical HBM read rate that the decode kernels' effective rates are
 * compared with (the pages compare against the chip's peak bandwidth:
 * grafy.ai "What performance gains does FOSCAR deliver?"; rag-lover.com
 * TL;DR).
 *   data   device pointer, 16-byte aligned; bytes a multiple of 16.
 *   sink   device uint32; written only if the XOR of all words read equals
 *          0x9E3779B9 (it exists so the loads cannot be elided).
 * Returns KVQ_ERR_NULL_POINTER / KVQ_ERR_MISALIGNED / KVQ_ERR_BAD_SHAPE on bad
 * arguments (nothing launched), KVQ_ERR_HIP on a failed launch.
 */
kvq_status kvq_stream_read(const void* data, size_t bytes, uint32_t* sink, void* stream);

/*
 * kvq_issue_probe -- measurement, not part of the method: whether a SIMD
 * overlaps matrix products with vector instructions. It decides how the
 * decode kernels trade one for the other (an extra 16x16x32 product against
 * a few fmas). `blocks` work-groups of 256 work-items (1024 = four per CU,
 * four waves per SIMD) each run `iters` steps of
 *   mode 0: 8 independent v_mfma_f32_16x16x32_f16 per wave,
 *   mode 1: 32 fp32 fmas (8 independent chains) per wave,
 *   mode 2: both in every wave, 4 fmas before each product,
 *   mode 3: mode 0 in even waves, mode 1 in odd waves.
 *   out    device float[blocks * 256], written once per work-item (a sum that
 *          keeps the work alive).
 * Time it with events around the call. Returns KVQ_ERR_NULL_POINTER /
 * KVQ_ERR_MISALIGNED / KVQ_ERR_BAD_SHAPE (mode outside 0..3, iters < 1,
 * blocks outside 1..65535) with nothing launched, KVQ_ERR_HIP on a failed
 * launch.
 */
kvq_status kvq_issue_probe(int mode, int iters, int blocks, float* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* KVQ_H */
