// Quantise + pack one layer's K and V into the documented cache layout.
//
// Each group shares one scale s and offset z (x ~ s*c + z); groups run along
// tokens or along channels, chosen separately for K and V (FOSCAR pages:
// grafy.ai "What is FOSCAR and how does it work?", rag-lover.com
// "conditions of use"). The rule is fixed bit for bit: min/max in fp32,
// s = fp16((max - min) / (2^b - 1)) with an IEEE fp32 division, z =
// fp16(min), code = clamp(rint((x - z) / s), 0, 2^b - 1) in fp32 from the
// stored fp16 s and z, code 0 when s == 0.
//
// Two passes: one thread per group computes (s, z); then one thread per
// packed 32-bit word recomputes its codes from the stored pairs. K words
// hold 32/b consecutive channels of a token; V words hold 32/b consecutive
// tokens of a channel. Words go to their place in the 64-token block
// (k_block_byte, v_block_word).
#include "kvq_internal.h"
#include "kvq_quant.h"

namespace kvq {
namespace {

// ---- pass 1: scale/offset per group -----------------------------------

__global__ void __launch_bounds__(256) sz_token_kernel(PackArgs a, Geo g, int is_k) {
  const float* x = is_k ? a.k : a.v;
  uint16_t* sz = is_k ? a.k_sz : a.v_sz;
  const int qmax = (1 << a.bits) - 1;
  const int ng = a.ng, G = kHeadDim / ng;  // one pair per G consecutive channels of a token
  const long total = (long)a.batch * a.num_kv_heads * a.padded_len * ng;
  for (long i = blockIdx.x * (long)blockDim.x + threadIdx.x; i < total;
       i += (long)gridDim.x * blockDim.x) {
    const int j = (int)(i % ng);
    const long r = i / ng;
    int t = (int)(r % a.padded_len);
    long bh = r / a.padded_len;
    int h = (int)(bh % a.num_kv_heads), b = (int)(bh / a.num_kv_heads);
    int L = min(max(a.seq_lens[b], 0), a.max_len);
    if (t >= g.extent(L)) continue;
    uint16_t s16 = 0, z16 = 0;
    if (t < L) {
      const float4* row = (const float4*)(x + ((bh * a.max_len) + t) * (long)kHeadDim + j * G);
      float4 v0 = row[0];
      float mn = fminf(fminf(v0.x, v0.y), fminf(v0.z, v0.w));
      float mx = fmaxf(fmaxf(v0.x, v0.y), fmaxf(v0.z, v0.w));
      for (int c = 1; c < G / 4; ++c) {
        float4 v = row[c];
        mn = fminf(mn, fminf(fminf(v.x, v.y), fminf(v.z, v.w)));
        mx = fmaxf(mx, fmaxf(fmaxf(v.x, v.y), fmaxf(v.z, v.w)));
      }
      s16 = f16_bits(__fdiv_rn(mx - mn, (float)qmax));
      z16 = f16_bits(mn);
    }
    long p = pair_token(g, b, h, t, j, ng);
    sz[p] = s16;
    sz[p + 1] = z16;
  }
}

__global__ void __launch_bounds__(256) sz_channel_kernel(PackArgs a, Geo g, int is_k) {
  const float* x = is_k ? a.k : a.v;
  uint16_t* sz = is_k ? a.k_sz : a.v_sz;
  const int qmax = (1 << a.bits) - 1;
  const int ngroups = a.padded_len / kGroup;
  const long total = (long)a.batch * a.num_kv_heads * ngroups * kHeadDim;
  for (long i = blockIdx.x * (long)blockDim.x + threadIdx.x; i < total;
       i += (long)gridDim.x * blockDim.x) {
    int d = (int)(i % kHeadDim);
    long r = i / kHeadDim;
    int gi = (int)(r % ngroups);
    long bh = r / ngroups;
    int h = (int)(bh % a.num_kv_heads), b = (int)(bh / a.num_kv_heads);
    int L = min(max(a.seq_lens[b], 0), a.max_len);
    int t0 = gi * kGroup;
    if (t0 >= g.extent(L)) continue;
    uint16_t s16 = 0, z16 = 0;
    if (t0 < L) {
      int n = min(kGroup, L - t0);
      const float* col = x + (bh * a.max_len + t0) * (long)kHeadDim + d;
      float mn = col[0], mx = col[0];
      for (int t = 1; t < n; ++t) {
        float v = col[(long)t * kHeadDim];
        mn = fminf(mn, v);
        mx = fmaxf(mx, v);
      }
      s16 = f16_bits(__fdiv_rn(mx - mn, (float)qmax));
      z16 = f16_bits(mn);
    }
    long p = pair_channel(g, b, h, t0, d);
    sz[p] = s16;
    sz[p + 1] = z16;
  }
}

// ---- pass 2: codes -------------------------------------------------------

// K: one thread per 32-bit word of a token row (32/b consecutive channels).
__global__ void __launch_bounds__(256) k_codes_kernel(PackArgs a, Geo g) {
  const int bits = a.bits, qmax = (1 << bits) - 1, per = 32 / bits;
  const int words = kHeadDim / per;
  const long total = (long)a.batch * a.num_kv_heads * a.padded_len * words;
  for (long i = blockIdx.x * (long)blockDim.x + threadIdx.x; i < total;
       i += (long)gridDim.x * blockDim.x) {
    int j = (int)(i % words);
    long r = i / words;
    int t = (int)(r % a.padded_len);
    long bh = r / a.padded_len;
    int h = (int)(bh % a.num_kv_heads), b = (int)(bh / a.num_kv_heads);
    int L = min(max(a.seq_lens[b], 0), a.max_len);
    if (t >= g.extent(L)) continue;
    uint32_t w = 0;
    if (t < L) {
      const float* xr = a.k + (bh * a.max_len + t) * (long)kHeadDim + j * per;
      float S = 0.f, Z = 0.f;
      if (a.k_axis == KVQ_TOKEN_WISE) {  // a word's channels lie in one group (32/b <= 16 <= G)
        long p = pair_token(g, b, h, t, (j * per) / (kHeadDim / a.ng), a.ng);
        S = f16_val(a.k_sz[p]);
        Z = f16_val(a.k_sz[p + 1]);
      }
      for (int e = 0; e < per; ++e) {
        int d = j * per + e;
        if (a.k_axis == KVQ_CHANNEL_WISE) {
          long p = pair_channel(g, b, h, t, d);
          S = f16_val(a.k_sz[p]);
          Z = f16_val(a.k_sz[p + 1]);
        }
        w |= (uint32_t)encode(xr[e], S, Z, qmax) << (bits * e);
      }
    }
    // bytes 4 j .. 4 j + 3 of the row stay inside one 16-byte piece
    const long blk = g.chunk(b, h, t) * (long)(kPage * words * 4);
    *(uint32_t*)(a.k_codes + blk + k_block_byte(bits, t % kPage, 4 * j)) = w;
  }
}

// V: one thread per word = 32/b consecutive tokens of one channel.
__global__ void __launch_bounds__(256) v_codes_kernel(PackArgs a, Geo g) {
  const int bits = a.bits, qmax = (1 << bits) - 1, per = 32 / bits;
  const int nw = a.padded_len / per;
  const long total = (long)a.batch * a.num_kv_heads * nw * kHeadDim;
  for (long i = blockIdx.x * (long)blockDim.x + threadIdx.x; i < total;
       i += (long)gridDim.x * blockDim.x) {
    int d = (int)(i % kHeadDim);
    long r = i / kHeadDim;
    int wi = (int)(r % nw);
    long bh = r / nw;
    int h = (int)(bh % a.num_kv_heads), b = (int)(bh / a.num_kv_heads);
    int L = min(max(a.seq_lens[b], 0), a.max_len);
    int t0 = wi * per;
    if (t0 >= g.extent(L)) continue;
    uint32_t w = 0;
    for (int e = 0; e < per; ++e) {
      int t = t0 + e;
      if (t >= L) break;
      long p = (a.v_axis == KVQ_TOKEN_WISE) ? pair_token(g, b, h, t, d / (kHeadDim / a.ng), a.ng)
                                            : pair_channel(g, b, h, t, d);
      float S = f16_val(a.v_sz[p]), Z = f16_val(a.v_sz[p + 1]);
      float xv = a.v[(bh * a.max_len + t) * (long)kHeadDim + d];
      w |= (uint32_t)encode(xv, S, Z, qmax) << (bits * e);
    }
    const long blk = g.chunk(b, h, t0) * (long)((kPage / per) * kHeadDim);
    a.v_words[blk + v_block_word((t0 % kPage) / per, d)] = w;
  }
}

int grid_for(long total) {
  long blocks = (total + 255) / 256;
  if (blocks > 256 * 64) blocks = 256 * 64;
  if (blocks < 1) blocks = 1;
  return (int)blocks;
}

}  // namespace

hipError_t launch_pack(const PackArgs& a, hipStream_t s) {
  Geo g{a.num_kv_heads, a.padded_len, a.max_pages, a.paged, a.page_table};
  const long tok = (long)a.batch * a.num_kv_heads * a.padded_len;
  const long grp = (long)a.batch * a.num_kv_heads * (a.padded_len / kGroup) * kHeadDim;
  for (int is_k = 1; is_k >= 0; --is_k) {
    int axis = is_k ? a.k_axis : a.v_axis;
    if (axis == KVQ_TOKEN_WISE)
      sz_token_kernel<<<grid_for(tok * a.ng), 256, 0, s>>>(a, g, is_k);
    else
      sz_channel_kernel<<<grid_for(grp), 256, 0, s>>>(a, g, is_k);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int per = 32 / a.bits;
  k_codes_kernel<<<grid_for(tok * (kHeadDim / per)), 256, 0, s>>>(a, g);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  v_codes_kernel<<<grid_for(tok / per * kHeadDim), 256, 0, s>>>(a, g);
  return hipGetLastError();
}

}  // namespace kvq
