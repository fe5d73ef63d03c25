// Quantise + pack one layer's K and V into the documented cache layout.
//
// Each group shares one scale s and offset z (x ~ s*c + z); groups run along
// tokens or along channels, chosen separately for K and V (FOSCAR pages:
// grafy.ai "What is FOSCAR and how does it work?", rag-lover.com
// "conditions of use"). The rule is fixed bit for bit: min/max in fp32 (a
// total order with -0 < +0), s = fp16((max - min) / (2^b - 1)) with an IEEE
// fp32 division, z = fp16(min), code = clamp(rint((x - z) / s), 0, 2^b - 1)
// in fp32 from the stored fp16 s and z, code 0 when s == 0.
//
// One pass, one work-group per (tensor, sequence, KV head, 128-token tile).
// The tile's 64 KB of fp32 is read once, as 16-byte loads: thread (k, c)
// holds tokens 16k .. 16k + 15 of channels 4c .. 4c + 3, a 32-lane half-wave
// covering whole 512-byte token rows. Then
//   * channel-wise groups (a channel over the tile's 128 tokens): min/max
//     over the thread's 16 tokens, across the two half-waves
//     (v_permlane32_swap) and across the four waves (LDS);
//   * token-wise groups (G channels of a token): min/max over the thread's 4
//     channels, then across the G/4 lanes of the group (DPP within rows of 16
//     lanes, v_permlane16_swap across the two rows of a half-wave);
//   * codes: (x - z) * (1/s), rounded, is the code of (x - z) / s except
//     close to a half-integer, where the two roundings could part; those rare
//     elements take the IEEE division (code_of states the bound);
//   * V words (32/b consecutive tokens of a channel) form in the thread's
//     registers and go out as 16-byte stores (4 channels side by side in the
//     layout); K rows (a token's channels across 32 lanes) and token-wise
//     (s, z) pairs are assembled in LDS and written as whole 16-byte pieces.
// Only 64-token blocks inside the written extent are stored (paged: the
// pages the sequence references). Input and output are touched once:
// non-temporal loads and stores keep them from displacing other data in the
// caches (measured 4-9% faster than plain ones at 32K tokens x 1024 heads).
#include "kvq_internal.h"
#include "kvq_quant.h"

namespace kvq {
namespace {

constexpr int kPackThreads = 256;
typedef uint32_t u4v __attribute__((ext_vector_type(4)));
typedef float f4v __attribute__((ext_vector_type(4)));

__device__ inline float vmin(float a, float b) { return __builtin_elementwise_minimum(a, b); }
__device__ inline float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }

// x from lane (l xor m) within rows of 16 lanes (DPP quad_perm / mirrors)
template <int CTRL>
__device__ inline float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL,
                                                               0xF, 0xF, false));
}
constexpr int kQuadXor1 = 0xB1;    // quad_perm [1, 0, 3, 2]
constexpr int kQuadXor2 = 0x4E;    // quad_perm [2, 3, 0, 1]
constexpr int kRowHalfMirror = 0x141;
constexpr int kRowMirror = 0x140;

// Min or max of v over lane pairs (l, l xor 16) or (l, l xor 32), from one
// row swap of v with itself: v_permlane16_swap exchanges the odd 16-lane rows
// of its first operand with the even rows of its second, so the two results
// hold rows (v0, v0, v2, v2) and (v1, v1, v3, v3); v_permlane32_swap
// exchanges the upper half of the first with the lower half of the second,
// giving halves (lo, lo) and (hi, hi). Each result is converted to a scalar
// before the bit cast: a bit cast of a vector element read in place takes
// element 0 whatever the index.
template <int WIDTH, bool MAX>
__device__ inline float pair_reduce(float v) {
  const unsigned u = __builtin_bit_cast(unsigned, v);
  auto r = WIDTH == 16 ? __builtin_amdgcn_permlane16_swap(u, u, false, false)
                       : __builtin_amdgcn_permlane32_swap(u, u, false, false);
  const float x = __builtin_bit_cast(float, (unsigned)r[0]);
  const float y = __builtin_bit_cast(float, (unsigned)r[1]);
  return MAX ? vmax(x, y) : vmin(x, y);
}

// min and max over the 2^steps lanes of an aligned group (steps 3, 4 or 5)
__device__ inline void lane_minmax(float& mn, float& mx, int steps) {
  mn = vmin(mn, dpp<kQuadXor1>(mn));
  mx = vmax(mx, dpp<kQuadXor1>(mx));
  mn = vmin(mn, dpp<kQuadXor2>(mn));
  mx = vmax(mx, dpp<kQuadXor2>(mx));
  mn = vmin(mn, dpp<kRowHalfMirror>(mn));  // lane i of 8 meets lane 7 - i: the other quad
  mx = vmax(mx, dpp<kRowHalfMirror>(mx));
  if (steps >= 4) {
    mn = vmin(mn, dpp<kRowMirror>(mn));    // lane i of 16 meets lane 15 - i: the other half-row
    mx = vmax(mx, dpp<kRowMirror>(mx));
  }
  if (steps >= 5) {  // rows 0 <-> 1 and 2 <-> 3
    mn = pair_reduce<16, false>(mn);
    mx = pair_reduce<16, true>(mx);
  }
}


struct Quant {
  float S, R, Z;     // stored scale and offset as fp32, R ~ 1 / S (0 when S == 0)
  uint32_t pair;     // s bits | z bits << 16
};

// s = fp16(RN32((max - min) / qmax)): the fp64 product (max - min) *
// RN64(1 / qmax), rounded to fp32, is that quotient. A quotient exact in fp32
// is reached within 2^-53 of itself; any other has the repeating binary
// expansion of a ratio with denominator 3 or 15, which stays more than 2^-30
// (relative) away from every fp32 rounding boundary, far beyond the product's
// error. 1 / s comes from v_rcp_f32 (within one ulp).
template <int BITS>
__device__ inline Quant make_quant(float mn, float mx) {
  Quant q;
  float s32 = (float)((double)(mx - mn) * (1.0 / (double)((1 << BITS) - 1)));
  // kept in a register: otherwise the two roundings (fp64 -> fp32 -> fp16)
  // are merged into one direct fp64 -> fp16 conversion, which differs at ties
  asm("" : "+v"(s32));
  const uint16_t s16 = f16_bits(s32);
  const uint16_t z16 = f16_bits(mn);
  q.S = f16_val(s16);
  q.Z = f16_val(z16);
  q.R = q.S != 0.0f ? __builtin_amdgcn_rcpf(q.S) : 0.0f;
  q.pair = (uint32_t)s16 | ((uint32_t)z16 << 16);
  return q;
}

// clamp(rint((x - Z) / S), 0, qmax) bit for bit, mostly without the division:
// with R within one ulp of 1 / S, t = (x - Z) * R is within |t| 2^-22.4 of
// the exact quotient; when |t - rint(t)| + |t| 2^-20 < 1/2 no rounding
// boundary (a half-integer) lies between t, the exact quotient and its fp32
// rounding, so all three round to the same integer. Otherwise (or when t is
// not finite) the IEEE division decides.
template <int BITS>
__device__ inline uint32_t code_of(float x, const Quant& q) {
  const float d = x - q.Z;
  float t = d * q.R;
  float r = rintf(t);
  if (!(fmaf(fabsf(t), 0x1p-20f, fabsf(t - r)) < 0.5f)) {
    t = q.S != 0.0f ? __fdiv_rn(d, q.S) : 0.0f;
    r = rintf(t);
  }
  return (uint32_t)__builtin_amdgcn_fmed3f(r, 0.0f, (float)((1 << BITS) - 1));
}

template <int BITS, bool ISV, int AXIS>
__global__ void __launch_bounds__(kPackThreads) pack_kernel(PackArgs a, Geo g, int tiles) {
  constexpr int kRowBytes = kHeadDim * BITS / 8;      // one token's K row
  constexpr int kBlockBytes = kPage * kRowBytes;      // one 64-token block of K codes
  constexpr int kTpw = 32 / BITS;                     // tokens per V word
  constexpr int kBlockWords = (kPage / kTpw) * kHeadDim;
  const float* x = ISV ? a.v : a.k;
  uint16_t* sz = ISV ? a.v_sz : a.k_sz;
  const int tid = threadIdx.x, c = tid & 31, kq = tid >> 5, wave = tid >> 6;
  const int ngroups = a.padded_len / kGroup;
  const int ng = a.ng;
  const int gl = (kHeadDim / ng) / 4;  // lanes per token-wise group

  __shared__ float4 red[2][4][32];                               // channel-wise [min|max][wave][quad]
  __shared__ __attribute__((aligned(16))) uint8_t krow[2 * kBlockBytes];  // K codes of the tile
  __shared__ __attribute__((aligned(16))) uint32_t pairs[kGroup * 4];     // token-wise (s, z)

  for (int tile = blockIdx.x; tile < tiles; tile += gridDim.x) {
    const int gi = tile % ngroups;
    const int bh = tile / ngroups;
    const int h = bh % a.num_kv_heads, b = bh / a.num_kv_heads;
    const int L = min(max(a.seq_lens[b], 0), a.max_len);
    const int t0 = gi * kGroup;
    const int E = g.extent(L);
    if (t0 >= E) continue;  // uniform: nothing of this tile is written
    poison_lds<kPackThreads>(red, sizeof red);
    poison_lds<kPackThreads>(krow, sizeof krow);
    poison_lds<kPackThreads>(pairs, sizeof pairs);
    const int n = L - t0;   // valid rows of the tile (may be <= 0 or > 128)

    float4 v[16];
    if (n > 0) {
      // rows past the sequence repeat its last row: in bounds, and they
      // leave a channel's min/max unchanged; their codes are masked below
      const float* src = x + ((long)bh * a.max_len + t0) * kHeadDim + 4 * c;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int r = min(16 * kq + i, n - 1);
        const f4v t = __builtin_nontemporal_load((const f4v*)(src + (long)r * kHeadDim));
        v[i] = float4{t.x, t.y, t.z, t.w};
      }
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) v[i] = float4{0.f, 0.f, 0.f, 0.f};
    }

    uint32_t words[4][16 / kTpw > 0 ? 16 / kTpw : 1];  // V: [channel][word-row of the thread]
    if (ISV) {
#pragma unroll
      for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int j = 0; j < 16 / kTpw; ++j) words[e][j] = 0;
    }

    if (AXIS == KVQ_CHANNEL_WISE) {
      float mn[4], mx[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float lo = v[0][e], hi = v[0][e];
#pragma unroll
        for (int i = 1; i < 16; ++i) {
          lo = vmin(lo, v[i][e]);
          hi = vmax(hi, v[i][e]);
        }
        mn[e] = pair_reduce<32, false>(lo);
        mx[e] = pair_reduce<32, true>(hi);
      }
      if ((tid & 32) == 0) {
        red[0][wave][c] = float4{mn[0], mn[1], mn[2], mn[3]};
        red[1][wave][c] = float4{mx[0], mx[1], mx[2], mx[3]};
      }
      __syncthreads();
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float4 lo = red[0][w][c], hi = red[1][w][c];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          mn[e] = vmin(mn[e], lo[e]);
          mx[e] = vmax(mx[e], hi[e]);
        }
      }
      Quant q[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) q[e] = make_quant<BITS>(mn[e], mx[e]);
      if (tid < 32) {  // the tile's 128 pairs: 512 contiguous bytes
        const long p = pair_channel(g, b, h, t0, 4 * c);
        __builtin_nontemporal_store(u4v{q[0].pair, q[1].pair, q[2].pair, q[3].pair}, (u4v*)(sz + p));
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const bool ok = 16 * kq + i < n;
        uint32_t cd[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) cd[e] = ok ? code_of<BITS>(v[i][e], q[e]) : 0u;
        if (ISV) {
#pragma unroll
          for (int e = 0; e < 4; ++e) words[e][i / kTpw] |= cd[e] << (BITS * (i % kTpw));
        } else {
          const int t = 16 * kq + i;
          const int off = (t >> 6) * kBlockBytes;
          if (BITS == 2)
            krow[off + k_block_byte(2, t & 63, c)] =
                (uint8_t)(cd[0] | (cd[1] << 2) | (cd[2] << 4) | (cd[3] << 6));
          else
            *(uint16_t*)(krow + off + k_block_byte(4, t & 63, 2 * c)) =
                (uint16_t)(cd[0] | (cd[1] << 4) | (cd[2] << 8) | (cd[3] << 12));
        }
      }
    } else {  // token-wise: G = 128 / ng channels of a token per group
      const int steps = gl == 32 ? 5 : gl == 16 ? 4 : 3;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int t = 16 * kq + i;
        const bool ok = t < n;
        float mn = vmin(vmin(v[i].x, v[i].y), vmin(v[i].z, v[i].w));
        float mx = vmax(vmax(v[i].x, v[i].y), vmax(v[i].z, v[i].w));
        lane_minmax(mn, mx, steps);
        Quant q = make_quant<BITS>(mn, mx);
        if (!ok) {  // past the sequence: pair (0, 0), every code 0
          q.S = q.R = q.Z = 0.0f;
          q.pair = 0;
        }
        if (c % gl == 0) pairs[t * ng + c / gl] = q.pair;
        uint32_t cd[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) cd[e] = ok ? code_of<BITS>(v[i][e], q) : 0u;
        if (ISV) {
#pragma unroll
          for (int e = 0; e < 4; ++e) words[e][i / kTpw] |= cd[e] << (BITS * (i % kTpw));
        } else {
          const int off = (t >> 6) * kBlockBytes;
          if (BITS == 2)
            krow[off + k_block_byte(2, t & 63, c)] =
                (uint8_t)(cd[0] | (cd[1] << 2) | (cd[2] << 4) | (cd[3] << 6));
          else
            *(uint16_t*)(krow + off + k_block_byte(4, t & 63, 2 * c)) =
                (uint16_t)(cd[0] | (cd[1] << 4) | (cd[2] << 8) | (cd[3] << 12));
        }
      }
    }

    if (ISV) {
      // thread's tokens 16 kq .. 16 kq + 15 lie in block kq / 4; word-row r
      // of channel 4c + e sits at 512 (r / 4) + 256 (c mod 2) + 64 (r mod 4)
      // + 4 (c / 2) + e: the 4 channels are one 16-byte piece
      const int t = t0 + 16 * kq;
      if (t < E) {
        uint32_t* blk = a.v_words + g.chunk(b, h, t) * (long)kBlockWords;
#pragma unroll
        for (int j = 0; j < 16 / kTpw; ++j) {
          const int r = ((16 * kq) & 63) / kTpw + j;
          __builtin_nontemporal_store(u4v{words[0][j], words[1][j], words[2][j], words[3][j]},
                                      (u4v*)(blk + v_block_word(r, 4 * c)));
        }
      }
    }
    if (!ISV || AXIS == KVQ_TOKEN_WISE) {
      __syncthreads();  // K rows and token-wise pairs complete in LDS
      if (!ISV) {
        constexpr int kPieces = 2 * kBlockBytes / 16;
#pragma unroll
        for (int p = tid; p < kPieces; p += kPackThreads) {
          const int blk = p / (kBlockBytes / 16);
          const int t = t0 + kPage * blk;
          if (t < E)
            __builtin_nontemporal_store(((const u4v*)krow)[p],
                                        (u4v*)(a.k_codes + g.chunk(b, h, t) * (long)kBlockBytes +
                                               (p % (kBlockBytes / 16)) * 16));
        }
      }
      if (AXIS == KVQ_TOKEN_WISE) {
        const int per_blk = kPage * ng / 4;  // 16-byte pieces of one block's pairs
        if (tid < 2 * per_blk) {
          const int blk = tid / per_blk;
          const int t = t0 + kPage * blk;
          if (t < E)
            __builtin_nontemporal_store(((const u4v*)pairs)[tid],
                                        (u4v*)(sz + pair_token(g, b, h, t, 0, ng) + (tid % per_blk) * 8));
        }
      }
    }
    __syncthreads();  // LDS free for the next tile
  }
}

template <int BITS, bool ISV>
hipError_t launch_one(const PackArgs& a, const Geo& g, int tiles, int grid, hipStream_t s) {
  const int axis = ISV ? a.v_axis : a.k_axis;
  if (axis == KVQ_TOKEN_WISE)
    pack_kernel<BITS, ISV, KVQ_TOKEN_WISE><<<grid, kPackThreads, 0, s>>>(a, g, tiles);
  else
    pack_kernel<BITS, ISV, KVQ_CHANNEL_WISE><<<grid, kPackThreads, 0, s>>>(a, g, tiles);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_pack(const PackArgs& a, hipStream_t s) {
  Geo g{a.num_kv_heads, a.padded_len, a.max_pages, a.paged, a.page_table};
  // the entry point keeps the tile count below 2^31
  const int tiles = (int)((long)a.batch * a.num_kv_heads * (a.padded_len / kGroup));
  if (tiles <= 0) return hipSuccess;
  const int grid = tiles < (1 << 20) ? tiles : (1 << 20);
  hipError_t e;
  if (a.bits == 2) {
    e = launch_one<2, false>(a, g, tiles, grid, s);
    if (e == hipSuccess) e = launch_one<2, true>(a, g, tiles, grid, s);
  } else {
    e = launch_one<4, false>(a, g, tiles, grid, s);
    if (e == hipSuccess) e = launch_one<4, true>(a, g, tiles, grid, s);
  }
  return e;
}

}  // namespace kvq
