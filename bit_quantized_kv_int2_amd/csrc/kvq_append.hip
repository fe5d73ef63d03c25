// Decode-time append: one new token per sequence goes into a bf16 residual
// window of up to 128 tokens per (sequence, KV head). When a token completes
// a 128-token group, the work-group of that (sequence, KV head) quantises the
// whole window into the cache with the bulk pack's rule (kvq_quant.h), so the
// cache only ever holds whole groups and the decode reads the window's tokens
// in bf16.
#include "kvq_internal.h"
#include "kvq_quant.h"

namespace kvq {
namespace {

constexpr int kAppendThreads = 256;
typedef uint32_t u4 __attribute__((ext_vector_type(4)));

__device__ inline float bf16_f32(uint16_t u) { return __builtin_bit_cast(float, (uint32_t)u << 16); }

__global__ void __launch_bounds__(kAppendThreads) append_kernel(AppendArgs a) {
  const int h = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int H = a.num_kv_heads;
  const int L = a.seq_lens[b];          // index of the new token
  if (L < 0 || L >= a.max_len) return;  // no room: nothing is written (uniform in the work-group)
  const long unit = (long)b * H + h;
  const int slot = L % kGroup;
  uint16_t* kw = a.k_win + unit * kGroup * kHeadDim;
  uint16_t* vw = a.v_win + unit * kGroup * kHeadDim;
  if (tid < kHeadDim) kw[slot * kHeadDim + tid] = a.k_new[unit * kHeadDim + tid];
  else vw[slot * kHeadDim + tid - kHeadDim] = a.v_new[unit * kHeadDim + tid - kHeadDim];
  if (slot != kGroup - 1) return;  // the group is not complete yet
  __syncthreads();                 // every row of the window, the new one included, is visible

  Geo g;
  g.H = H;
  g.Lp = a.padded_len;
  g.max_pages = a.max_pages;
  g.paged = a.paged;
  g.table = a.page_table;
  const int g0 = L + 1 - kGroup;  // first token of the completed group
  const int qmax = (1 << a.bits) - 1, per = 32 / a.bits;
  // one (s, z) per token and channel group (token-wise, ng groups of G
  // channels) or per channel (channel-wise)
  const int ng = a.ng, G = kHeadDim / ng;
  __shared__ float S[kGroup * 4], Z[kGroup * 4];
  // the window of one tensor, staged in LDS with whole 16-byte loads: the
  // min/max and encode loops below read each value once or twice at scattered
  // places, which from global memory is a chain of cache-latency loads
  __shared__ __attribute__((aligned(16))) uint16_t win[kGroup * kHeadDim];

  for (int is_k = 1; is_k >= 0; --is_k) {
    poison_lds<kAppendThreads>(S, sizeof S);
    poison_lds<kAppendThreads>(Z, sizeof Z);
    poison_lds<kAppendThreads>(win, sizeof win);
    {
      const u4* src = (const u4*)(is_k ? kw : vw);
      for (int i = tid; i < kGroup * kHeadDim / 8; i += kAppendThreads) ((u4*)win)[i] = src[i];
    }
    __syncthreads();
    const uint16_t* w = win;
    const int axis = is_k ? a.k_axis : a.v_axis;
    uint16_t* sz = is_k ? a.k_sz : a.v_sz;
    const int ngroups = axis == KVQ_TOKEN_WISE ? kGroup * ng : kHeadDim;
    for (int gi = tid; gi < ngroups; gi += kAppendThreads) {
      float mn, mx;
      long p;
      if (axis == KVQ_TOKEN_WISE) {  // group = channels [jG, jG + G) of token t
        const int t = gi / ng, j = gi % ng;
        const uint16_t* row = w + t * kHeadDim + j * G;
        // start each thread's walk along its row at its own offset, so that
        // the threads of a wave read different LDS banks at each step
        mn = mx = bf16_f32(row[gi % G]);
        for (int e = 1; e < G; ++e) {
          const float v = bf16_f32(row[(gi + e) % G]);
          mn = __builtin_elementwise_minimum(mn, v);
          mx = __builtin_elementwise_maximum(mx, v);
        }
        p = pair_token(g, b, h, g0 + t, j, ng);
      } else {  // group = channel gi over the 128 tokens
        mn = mx = bf16_f32(w[gi]);
        for (int t = 1; t < kGroup; ++t) {
          const float v = bf16_f32(w[t * kHeadDim + gi]);
          mn = __builtin_elementwise_minimum(mn, v);
          mx = __builtin_elementwise_maximum(mx, v);
        }
        p = pair_channel(g, b, h, g0, gi);
      }
      const uint16_t s16 = f16_bits(__fdiv_rn(mx - mn, (float)qmax)), z16 = f16_bits(mn);
      sz[p] = s16;
      sz[p + 1] = z16;
      S[gi] = f16_val(s16);
      Z[gi] = f16_val(z16);
    }
    __syncthreads();
    if (is_k) {  // K: one word = 32/b consecutive channels of a token row
      const int words = kHeadDim / per;
      for (int i = tid; i < kGroup * words; i += kAppendThreads) {
        const int t = i / words, j = i % words;
        uint32_t wd = 0;
        for (int e = 0; e < per; ++e) {
          const int d = j * per + e;
          const int gi = axis == KVQ_TOKEN_WISE ? t * ng + d / G : d;
          wd |= (uint32_t)encode(bf16_f32(w[t * kHeadDim + d]), S[gi], Z[gi], qmax) << (a.bits * e);
        }
        const int tt = g0 + t;
        const long blk = g.chunk(b, h, tt) * (long)(kPage * words * 4);
        *(uint32_t*)(a.k_codes + blk + k_block_byte(a.bits, tt % kPage, 4 * j)) = wd;
      }
    } else {  // V: one word = 32/b consecutive tokens of a channel
      const int nw = kGroup / per;
      for (int i = tid; i < nw * kHeadDim; i += kAppendThreads) {
        const int d = i % kHeadDim, t0 = (i / kHeadDim) * per;
        uint32_t wd = 0;
        for (int e = 0; e < per; ++e) {
          const int t = t0 + e;
          const int gi = axis == KVQ_TOKEN_WISE ? t * ng + d / G : d;
          wd |= (uint32_t)encode(bf16_f32(w[t * kHeadDim + d]), S[gi], Z[gi], qmax) << (a.bits * e);
        }
        const int tt = g0 + t0;
        const long blk = g.chunk(b, h, tt) * (long)((kPage / per) * kHeadDim);
        a.v_words[blk + v_block_word((tt % kPage) / per, d)] = wd;
      }
    }
    __syncthreads();  // S and Z are reused for V
  }
}

}  // namespace

hipError_t launch_append(const AppendArgs& a, hipStream_t s) {
  append_kernel<<<dim3(a.num_kv_heads, a.batch), kAppendThreads, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace kvq
