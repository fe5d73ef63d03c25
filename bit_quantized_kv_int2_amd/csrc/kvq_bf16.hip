// Split-KV decode attention over an unquantised bf16 KV cache (the
// comparison baseline for the quantised path; same split plan, same LSE
// combine). gfx950, v_mfma_f32_16x16x32_bf16.
//
// Per wave iteration of 32 tokens:
//   * K: two 16-token tiles; lane (row i, group g) loads 16 B of its token's
//     row per k-step (channels 32 s + 8 g .. +7); tile rows map to tokens so
//     that the QK^T accumulator is already the PV B operand.
//   * V: lane (i, g) loads channels 8i..8i+7 of the 8 tokens 8g..8g+7 (each
//     load instruction covers four whole 256-byte rows) and v_perm-packs
//     token pairs of one channel into the A operand of 8 channel tiles.
//   * Online softmax with a lazily moved maximum; the normaliser is summed
//     from the rounded bf16 probabilities that feed the PV product.
//   * K and V loads are non-temporal: the cache is streamed once, and such
//     streams read HBM faster when they do not allocate in the caches (each
//     K load still covers whole 64-byte halves of the rows it touches).
#include <math.h>

#include "kvq_internal.h"

namespace kvq {
namespace {

typedef __bf16 b8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr int kThr = 8;
constexpr int kTit = 32;

__device__ inline f4 mfma_bf(u4 a, u4 b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(b8, a), __builtin_bit_cast(b8, b), c,
                                                 0, 0, 0);
}
__device__ inline float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ inline uint32_t pack_bf16x2(float lo, float hi) {
  __bf16 a = (__bf16)lo, b = (__bf16)hi;
  return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}
__device__ inline float bflo(uint32_t u) { return __builtin_bit_cast(float, u << 16); }
__device__ inline float bfhi(uint32_t u) { return __builtin_bit_cast(float, u & 0xFFFF0000u); }

template <bool PAGED>
__global__ void __launch_bounds__(kThreads) bf16_kernel(Bf16Args a) {
  __shared__ __attribute__((aligned(16))) float mo[kWaves * 4 * 128];
  __shared__ float ml[kWaves * 4 * 2];
  poison_lds<kThreads>(mo, sizeof mo);
  poison_lds<kThreads>(ml, sizeof ml);

  const WorkItem wi = work_item(blockIdx.x, a.num_kv_heads, a.batch, a.num_splits);
  if (!wi.live) return;  // padding to whole rounds of 8 rows
  const int sp = wi.sp, h = wi.h, b = wi.b;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int H = a.num_kv_heads, Hq = H * kGqa;
  int L = max(a.seq_lens[b], 0);
  if (a.len_mode == 2) L %= kGroup;  // the residual window holds the tokens past the last whole group
  L = min(L, a.max_len);  // contract: 0 <= len <= max_len
  const int tb = sp * a.split_tokens;
  const int te = min(tb + a.split_tokens, L);
  const long row0 = (long)b * Hq + (long)h * kGqa;
  if (te <= tb) {
    for (int e = tid; e < kGqa * kHeadDim; e += kThreads) {
      int hh = e / kHeadDim, d = e % kHeadDim;
      if (a.direct_out) {
        if (a.out_bf16) ((uint16_t*)a.out)[(row0 + hh) * kHeadDim + d] = 0;
        else ((float*)a.out)[(row0 + hh) * kHeadDim + d] = 0.f;
      } else {
        const long pr = (row0 + hh) * a.part_stride + a.part_base + sp;
        a.part_o[pr * kHeadDim + d] = 0.f;
        if (d == 0) {
          a.part_ml[pr * 2] = -INFINITY;
          a.part_ml[pr * 2 + 1] = 0.f;
        }
      }
    }
    return;
  }
  const int n = lane & 15, g = lane >> 4, hh = n & 3, ri = lane & 15;
  const long unit = (long)b * H + h;
  auto row_of = [&](int t) -> long {  // row index of token t in the [..][D] arrays
    t = min(t, L - 1);  // rows past the sequence are never read; masked below
    if (!PAGED) return unit * a.max_len + t;
    return ((long)a.page_table[(long)b * a.max_pages + t / kPage] * H + h) * kPage + t % kPage;
  };

  // B operand of q^T: lane (n, g), k-step s: q[head n&3][32 s + 8 g .. +7]
  u4 bq[4];
  {
    const uint16_t* qp = a.q + (row0 + hh) * kHeadDim;
#pragma unroll
    for (int s = 0; s < 4; ++s) bq[s] = *(const u4*)(qp + 32 * s + 8 * g);
  }

  struct Tile {
    u4 k[2][4];
    u4 v[8];
  };
  auto load = [&](int t0, Tile& x) {
#pragma unroll
    for (int T = 0; T < 2; ++T) {
      const long r = row_of(t0 + 8 * (ri >> 2) + 4 * T + (ri & 3));
#pragma unroll
      for (int s = 0; s < 4; ++s) x.k[T][s] = __builtin_nontemporal_load((const u4*)(a.k + r * kHeadDim + 32 * s + 8 * g));
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const long r = row_of(t0 + 8 * g + j);
      x.v[j] = __builtin_nontemporal_load((const u4*)(a.v + r * kHeadDim + 8 * ri));
    }
  };

  f4 O[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) O[c] = f4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, lsum = 0.f;
  const float alpha = a.scale_log2;

  Tile cur;
  {
    const int t0 = tb + wv * kTit;
    if (t0 < te) load(t0, cur);
  }
  for (int it = wv;; it += kWaves) {
    const int t0 = tb + it * kTit;
    if (t0 >= te) break;
    Tile nxt;
    if (t0 + kWaves * kTit < te) load(t0 + kWaves * kTit, nxt);
    float S[2][4];
#pragma unroll
    for (int T = 0; T < 2; ++T) {
      f4 c4 = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s) c4 = mfma_bf(cur.k[T][s], bq[s], c4);
#pragma unroll
      for (int j = 0; j < 4; ++j) S[T][j] = c4[j] * alpha;
    }
    if (t0 + kTit > te) {
#pragma unroll
      for (int T = 0; T < 2; ++T)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (t0 + 8 * g + 4 * T + j >= te) S[T][j] = -INFINITY;
    }
    float mx = S[0][0];
#pragma unroll
    for (int T = 0; T < 2; ++T)
#pragma unroll
      for (int j = 0; j < 4; ++j) mx = fmaxf(mx, S[T][j]);
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    if (__any(mx > m_run + (float)kThr)) {
      const float mn = fmaxf(m_run, mx);
      const float sc = exp2_fast(m_run - mn);
#pragma unroll
      for (int c = 0; c < 8; ++c) O[c] *= sc;
      lsum *= sc;
      m_run = mn;
    }
    u4 bp;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      uint32_t pk = pack_bf16x2(exp2_fast(S[0][m] - m_run), exp2_fast(S[1][m] - m_run));
      bp[m] = pk;
      lsum += bflo(pk) + bfhi(pk);
    }
    // A operand of channel tile c: VGPR m = (V[8g+m][8i+c], V[8g+4+m][8i+c])
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      u4 av;
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const uint32_t x0 = cur.v[m][c >> 1], x1 = cur.v[m + 4][c >> 1];
        // pick the 16-bit half (c & 1) of each and pack (x0 half, x1 half)
        av[m] = (c & 1) ? __builtin_amdgcn_perm(x1, x0, 0x07060302u)
                        : __builtin_amdgcn_perm(x1, x0, 0x05040100u);
      }
      O[c] = mfma_bf(av, bp, O[c]);
    }
    cur = nxt;
  }
  lsum += __shfl_xor(lsum, 16);
  lsum += __shfl_xor(lsum, 32);

  // merge the four waves
  if (n < 4 && g == 0) ml[(wv * 4 + n) * 2] = m_run;
  __syncthreads();
  float mall = -INFINITY;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) mall = fmaxf(mall, ml[(w * 4 + hh) * 2]);
  const float f = (m_run == -INFINITY) ? 0.f : exp2_fast(m_run - mall);
  __syncthreads();
  if (n < 4) {
    float* dst = mo + (wv * 4 + n) * kHeadDim;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int c = 0; c < 8; ++c) dst[8 * (4 * g + j) + c] = O[c][j] * f;
    if (g == 0) {
      ml[(wv * 4 + n) * 2 + 1] = lsum * f;
      ml[(wv * 4 + n) * 2] = mall;
    }
  }
  __syncthreads();
  const int qh = tid >> 6, d = (tid & 63) * 2;
  float n0 = 0.f, n1 = 0.f, lt = 0.f;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    n0 += mo[(w * 4 + qh) * kHeadDim + d];
    n1 += mo[(w * 4 + qh) * kHeadDim + d + 1];
    lt += ml[(w * 4 + qh) * 2 + 1];
  }
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  const float o0 = n0 * inv, o1 = n1 * inv;
  const long row = row0 + qh;
  if (a.direct_out) {
    if (a.out_bf16) *(uint32_t*)((uint16_t*)a.out + row * kHeadDim + d) = pack_bf16x2(o0, o1);
    else *(float2*)((float*)a.out + row * kHeadDim + d) = make_float2(o0, o1);
  } else {
    const long pr = row * a.part_stride + a.part_base + sp;
    *(float2*)(a.part_o + pr * kHeadDim + d) = make_float2(o0, o1);
    if (d == 0) {
      a.part_ml[pr * 2] = ml[qh * 2];
      a.part_ml[pr * 2 + 1] = lt;
    }
  }
}

}  // namespace

hipError_t launch_decode_bf16(const Bf16Args& a, hipStream_t s) {
  dim3 grid((unsigned)decode_grid_blocks((long)a.batch * a.num_kv_heads, a.num_splits));
  if (a.page_size) bf16_kernel<true><<<grid, kThreads, 0, s>>>(a);
  else bf16_kernel<false><<<grid, kThreads, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace kvq
