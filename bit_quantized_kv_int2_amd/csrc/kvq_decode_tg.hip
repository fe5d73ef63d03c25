// Decode attention over INT2/INT4 caches whose K and V groups are both
// token-wise with G = 128 / NG channels per group (NG = 2: G = 64, NG = 4:
// G = 32), gfx950. A token has NG (s, z) pairs per tensor.
//
// Folds (rag-lover.com explainer; limits section: an acc-fold partial is
// scaled per quantisation group and never accumulated across groups):
//   q.K^T, acc-fold per channel group j:
//     S_t = sum_j [ s_{t,j} (q_j . c_{t,j}) + z_{t,j} sum_{d in j} q_d ]
//     one MFMA accumulator per group; the 16 k-steps fall into NG blocks of
//     16 / NG consecutive k-steps, one per group.
//   P.V, operand-fold per channel group:
//     O_d = sum_t (P_t s_{t,j(d)}) c_{t,d} + sum_t P_t z_{t,j(d)}
//     every 16-channel tile lies in one group (tile c = channels 16c..16c+15)
//     and takes that group's P'' operand, as the compressed A operand of the
//     2:4-sparse 16x16x64 product (the V codes its dense B; one product per
//     tile and iteration); the offset sum of each group runs on the vector
//     unit over the same rounded P'' (four fmas per group and iteration in
//     place of two matrix products, which the vector unit would wait out on
//     gfx950).
// Everything else (block-diagonal dense QK^T, token maps, subnormal operands,
// consistent offsets, lazy softmax, wave-local chunks) is as in the G = 128
// kernel; a chunk holds 2048 / NG tokens so its fold operands fit the same LDS.
#include "kvq_internal.h"
#include "kvq_decode_common.h"

namespace kvq {
namespace {

template <int BITS, int NG>
struct TgLds {
  static constexpr int CHUNK = kChunkTokens / NG;           // tokens per chunk
  static constexpr int HEAD_STRIDE = 288;                    // q'' of one head: 16 k-steps + padding
  static constexpr int QS = 0;                               // float q [4][128]
  static constexpr int QB = QS + 4 * 128 * 4;                // u4 q'' [4 heads][18]
  static constexpr int QZ = QB + 4 * HEAD_STRIDE + 16;       // 256 B of zeros, 16 B into a 128-byte line
  static constexpr int KB = QZ + 256 + 112;                  // float2 (s', z'') [CHUNK tokens][NG], skewed
  static constexpr int KB_BYTES = CHUNK * NG * 8 + CHUNK;    // + 16 B per 16-token run
  static constexpr int VA = KB + KB_BYTES;                   // float coef [NG][CHUNK], pairs XOR-permuted
  static constexpr int VA_GROUP = CHUNK * 4;
  static constexpr int VR = VA + NG * VA_GROUP;              // float w * rho [NG][CHUNK], addressed like coef
  static constexpr int RED = VR + NG * VA_GROUP;             // float [32]: q max per head, q sums per (head, group)
  static constexpr int TOTAL = RED + 32 * 4;
  static constexpr int MO = 0;                               // merge area (after the main loop)
  static constexpr int ML = MO + 4 * 4 * 128 * 4;
  static_assert(ML + 4 * 4 * 2 * 4 <= RED, "merge area overlaps reductions");
  static_assert(QB % 128 == 0 && (QZ - QB) % 128 == 16, "bank layout");
  static_assert(KB % 16 == 0 && VA % 16 == 0 && VR % 16 == 0, "alignment");
  static_assert(3 * TOTAL <= 160 * 1024, "three work-groups per CU");
  // byte offset of token t's NG (s', z'') pairs: each run of 16 tokens starts
  // 16 B further into the bank rotation than the last, so the two tokens 16
  // apart that one 8-lane group of a 128-bit read fetches use different banks
  __device__ static inline int kb_off(int t) { return t * NG * 8 + 16 * (t >> 4); }
};

template <int BITS, int NG, bool PAGED>
__global__ void __launch_bounds__(kThreads, tg_groups_per_cu(BITS, NG)) decode_tg_kernel(DecodeArgs a) {
  using C = Cfg<BITS>;
  using M = TgLds<BITS, NG>;
  constexpr int G = kHeadDim / NG;   // channels per group
  constexpr int TPG = 8 / NG;        // 16-channel PV tiles per group
  constexpr int NV = BITS == 2 ? 8 : 16;
  __shared__ __attribute__((aligned(16))) unsigned char lds[M::TOTAL];
  float* qs = (float*)(lds + M::QS);
  float* red = (float*)(lds + M::RED);

  static_assert(M::TOTAL >= (8 + kThreads) * 4, "find_split borrows the start of the LDS");
  poison_lds<kThreads>(lds, M::TOTAL);
  const Split ws = find_split(a, (int*)lds);
  if (!ws.live) return;  // padding, or past the plan's work-items
  const int sp = ws.sp, h = ws.h, b = ws.b;
  const int tid = __builtin_amdgcn_workitem_id_x(), lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int H = a.num_kv_heads, Hq = H * kGqa;
  int L = min(max(a.seq_lens[b], 0), a.max_len);
  if (a.len_mode == 1) L -= L % kGroup;
  const int tb = sp * ws.S;
  const int te = min(tb + ws.S, L);
  const long row0 = (long)b * Hq + (long)h * kGqa;

  if (te <= tb) {  // nothing in this split (or an empty sequence)
    for (int e = tid; e < kGqa * kHeadDim; e += kThreads) {
      int hh = e / kHeadDim, d = e % kHeadDim;
      if (ws.direct) {
        if (a.out_bf16) ((uint16_t*)a.out)[(row0 + hh) * kHeadDim + d] = 0;
        else ((float*)a.out)[(row0 + hh) * kHeadDim + d] = 0.f;
      } else {
        const long pr = ws.pbase + hh * ws.pmul;
        a.part_o[pr * kHeadDim + d] = 0.f;
        if (d == 0) {
          a.part_ml[pr * 2] = -INFINITY;
          a.part_ml[pr * 2 + 1] = 0.f;
        }
      }
    }
    return;
  }
  const float alpha = a.scale_log2;

  // ---- cache addressing ---------------------------------------------------
  const long unit = (long)b * H + h;
  auto chunk_of = [&](int t) -> long {  // 64-token block of token t
    if (!PAGED) return unit * (a.padded_len / kPage) + t / kPage;
    return (long)a.page_table[(long)b * a.max_pages + t / kPage] * H + h;
  };

  const int n = lane & 15, g = lane >> 4, hh = n & 3;
  const int ri = lane & 15;

  // ---- code loads for one 64-token iteration ---------------------------
  // An iteration is one 64-token block (block order as in the G = 128
  // kernel). K as there: lane l = 16 g + ri gets the row of token
  // tok(g, ri>>2, ri&3) from 1 KB whole-line loads. V: lane (ri, g) loads, for
  // each 16-channel tile c, the word of channel 16c + ri in word row g (INT2)
  // or rows g and g + 4 (INT4; k-step k = row g + 4k); in block order that
  // word sits at v_block_word(g + 4k, 16c + ri) = lane base + 512 k + 8 c.
  struct Codes {
    u4 k[C::KDW / 4];
    uint32_t v[NV];
  };
  auto lane_koff = [](int lg, int lr) { return (uint32_t)(16 * (16 * lg + lr)); };
  auto load_block = [&](long ch, Codes& cd, uint32_t koff, int lg, int lr) {
    const unsigned char* kb = a.k_codes + ch * (kPage * C::KROW) + koff;
#pragma unroll
    for (int e = 0; e < C::KDW / 4; ++e) cd.k[e] = __builtin_nontemporal_load((const u4*)(kb + 1024 * e));
    const uint32_t* vb = a.v_words + ch * ((kPage / C::TPW) * kHeadDim) + v_block_word(lg, lr);
#pragma unroll
    for (int e = 0; e < NV; ++e) cd.v[e] = vb[512 * (e >> 3) + 8 * (e & 7)];
  };
  // Paged caches: the physical page of a wave's next iteration is read one
  // iteration before its codes (as in the G = 128 kernel), so the code loads
  // never wait on a page-table read. A wave's next iteration is 64 tokens on
  // within its 128-token block, else 448 tokens on.
  auto next_it = [](int t) { return t + (((t >> 6) & 1) ? 7 : 1) * C::TIT; };
  auto page_at = [&](int t) -> int {  // (through a vector register: see the G = 128 kernel)
    int z = 0;
    asm volatile("" : "+v"(z));
    return a.page_table[(long)b * a.max_pages + t / kPage + z];
  };

  // wave wv owns the 128-token groups wv, wv + 4, ... (iterations 2G, 2G + 1)
  Codes cur;
  int pg_next = 0;  // paged: physical page of this wave's next iteration
  {
    const int t0 = tb + 2 * wv * C::TIT;
    if (t0 < te) load_block(chunk_of(t0), cur, lane_koff(g, ri), g, ri);
    if (PAGED && next_it(t0) < te) pg_next = page_at(next_it(t0));
  }

  // ---- query: once per split -------------------------------------------------
  {
    const int d = lane * 2;  // wave wv loads query head wv
    const uint32_t qq = *(const uint32_t*)(a.q + (row0 + wv) * kHeadDim + d);
    const float q0 = bf16val((uint16_t)(qq & 0xFFFF)), q1 = bf16val((uint16_t)(qq >> 16));
    const float m = wave_max_dpp(fmaxf(fabsf(q0), fabsf(q1)));
    qs[wv * 128 + d] = q0;
    qs[wv * 128 + d + 1] = q1;
    // sum of q over each channel group: G / 2 lanes (one DPP row for G = 32,
    // two rows for G = 64)
    float gs = row_sum(q0 + q1);
    if (NG == 2) gs = swap16_sum(gs);
    if ((lane % (G / 2)) == 0) red[16 + wv * 4 + lane / (G / 2)] = gs;
    if (lane == 0) red[wv] = m;
  }
  if (tid < 16) ((u4*)(lds + M::QZ))[tid] = u4{0u, 0u, 0u, 0u};
  __syncthreads();
  // q'' = q * 2^-E / w (max |q''| < 2^14), shared by all waves and groups
  const float qmax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const int E = exp_above(qmax) - 14;
  if (tid < 64) {
    const float two_mE = ldexpf(1.f, -E);
    const int s = tid & 15, qh = tid >> 4;
    uint32_t wds[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      float v0 = qs[qh * 128 + C::k_run(s, 0) + m] * two_mE * C::inv_w(m);
      float v1 = qs[qh * 128 + C::k_run(s, 1) + m] * two_mE * C::inv_w(m);
      wds[m] = pack_f16x2(v0, v1);
    }
    ((u4*)(lds + M::QB + qh * M::HEAD_STRIDE))[s] = u4{wds[0], wds[1], wds[2], wds[3]};
  }
  __syncthreads();
  const float ktok_sc = alpha * ldexpf(1.f, E + 24);

  f4 O[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) O[c] = f4{0.f, 0.f, 0.f, 0.f};
  float X[NG];  // this lane's part of its head's offset sum, per group
#pragma unroll
  for (int j = 0; j < NG; ++j) X[j] = 0.f;
  float m_run = -INFINITY;
  float mneg = 0.f;  // -m_run once the first scores are in (0 before)
  float lsum = 0.f;
  int F = 0;  // P'' = P * s * 2^-F / w, running per wave
  float kseed = 0.f;  // the running output's start value (kSeedV), scaled along
  // P.V on the 2:4-sparse 16x16x64 product (P'' its compressed A, the
  // V codes its dense B); tile c of lane (g, n) then holds head g, channel
  // 16 c + n, in rows 0 and 1 (two replicas that split the tokens; rows 2 and
  // 3 repeat them and are never read)
  constexpr bool SPV = true;

  // ---- (s, z) rows of a chunk: lane l takes TPL = 8 / NG consecutive tokens
  // of this wave's blocks (128-token blocks wv, wv + 4, .. of the chunk), all
  // NG channel groups of each: one contiguous 4 NG-byte (s, z) row per token
  // and tensor. The lane's first token t0 is a multiple of TPL, so a token's
  // code slot within its 4-token run is (t0 & 3) + u. Where the registers
  // allow (G = 32), the next chunk's rows are loaded during this chunk's main
  // loop, so the next prologue does not wait for them.
  constexpr int TPL = 8 / NG;
  constexpr bool PREFETCH = NG == 4;
  typedef uint32_t row_t __attribute__((ext_vector_type(NG)));
  auto lane_t0 = [&]() {  // from a laundered lane id: nothing of it stays live
    int pl = lane;
    asm volatile("" : "+v"(pl));
    const int tw = pl * TPL;  // index into the wave's tokens of the chunk
    return 128 * (wv + 4 * (tw >> 7)) + (tw & 127);
  };
  auto load_rows = [&](int cbx, row_t* kz, row_t* vz) {
    const int t0 = lane_t0();
    const int ntok = min(cbx + M::CHUNK, te) - cbx;
    // the chunk's rows sit at a base shared by the wave plus a 32-bit lane
    // offset (token ta of that base). In a paged cache a lane's TPL tokens lie
    // in one page: the base is that page's block (the page of the chunk's
    // last token for a lane wholly past the end, whose loads are masked), so
    // every page-table read is of a token inside the sequence.
    long szb = (unit * a.padded_len + cbx) * (long)(4 * NG);
    int ta = t0;
    if (PAGED) {
      szb = (chunk_of(cbx + min(t0, ntok - 1)) * kPage) * (long)(4 * NG);
      ta = t0 % kPage;  // (chunks start at multiples of 64 tokens)
    }
    const unsigned char* krow = (const unsigned char*)a.k_sz + szb;
    const unsigned char* vrow = (const unsigned char*)a.v_sz + szb;
    if (ntok == M::CHUNK) {  // a whole chunk: no token past the end
#pragma unroll
      for (int u = 0; u < TPL; ++u) {
        kz[u] = *(const row_t*)(krow + (uint32_t)(4 * NG * (ta + u)));
        vz[u] = *(const row_t*)(vrow + (uint32_t)(4 * NG * (ta + u)));
      }
    } else {  // tokens past the end read as (0, 0)
#pragma unroll
      for (int u = 0; u < TPL; ++u) {
        kz[u] = row_t(0u);
        vz[u] = row_t(0u);
        if (t0 + u < ntok) {
          kz[u] = *(const row_t*)(krow + (uint32_t)(4 * NG * (ta + u)));
          vz[u] = *(const row_t*)(vrow + (uint32_t)(4 * NG * (ta + u)));
        }
      }
    }
  };
  row_t kz[TPL], vz[TPL];
  if constexpr (PREFETCH) load_rows(tb, kz, vz);

  for (int cb = tb; cb < te; cb += M::CHUNK) {
    const int ce = min(cb + M::CHUNK, te);

    // ---- prologue
    if constexpr (!PREFETCH) load_rows(cb, kz, vz);
    const int t0 = lane_t0();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    {
      // every scale of this wave's tokens < 2^Fs (scales of 0 count as 1)
      uint32_t mb = 0, smin = 0x7FFFu;
#pragma unroll
      for (int u = 0; u < TPL; ++u)
#pragma unroll
        for (int j = 0; j < NG; ++j) {
          mb = max(mb, (uint32_t)vz[u][j] & 0x7FFFu);
          smin = min(smin, (uint32_t)vz[u][j] & 0x7FFFu);
        }
      mb = wave_max_u(mb);
      // sigma = s, or 1 where s == 0 (a constant token group, or the (0, 0)
      // read past the end): patched into the words by the rare waves that
      // hold one, so the common formulas need no selects
      if (__any(smin == 0u)) {
#pragma unroll
        for (int u = 0; u < TPL; ++u)
#pragma unroll
          for (int j = 0; j < NG; ++j) {
            const uint32_t w = vz[u][j];
            if ((w & 0x7FFFu) == 0u) vz[u][j] = (w & 0xFFFF0000u) | 0x3C00u;
          }
      }
      const int Fc = max((int)(mb >> 10) - 14, 1) + kThr - 14;
      if (cb == tb) {
        F = Fc;
      } else if (Fc > F) {
        const float sc = ldexpf(1.f, F - Fc);
#pragma unroll
        for (int c = 0; c < 8; ++c) O[c] *= sc;
#pragma unroll
        for (int j = 0; j < NG; ++j) X[j] *= sc;
        kseed *= sc;
        F = Fc;
      }
      // slot weight of token t0 + u: 2^(BITS ((t0 & 3) + u) % SLOTS)); with
      // two tokens per lane (INT2) the lane's pair sits at slots 0, 1 or 2, 3
      // (powers of two: the divisions by lw are multiplications by 1 / lw)
      const bool hi_pair = BITS == 2 && TPL == 2 && (t0 & 2);
      const float lw = hi_pair ? 16.f : 1.f, inv_lw = hi_pair ? 0.0625f : 1.f;
      const float two_mF = ldexpf(1.f, -F) * inv_lw;
      float cf[NG][TPL], rw[NG][TPL];
#pragma unroll
      for (int u = 0; u < TPL; ++u) {
        const float wu = (float)(1 << (BITS * (u % C::SLOTS)));  // weight / lw
        // tokens of the odd slots (u odd) enter mirrored: scale negated,
        // offset z + qmax s; wt / sigma as the reciprocal of sigma / wt
        const bool mir = u & 1;
#pragma unroll
        for (int j = 0; j < NG; ++j) {
          // products of a binary16 value as fma with a zero addend: one
          // mixed-precision instruction each (sigma > 0, so no signed zero)
          const float sg = f16lo(vz[u][j]), zv = f16hi(vz[u][j]);
          cf[j][u] = fmaf(sg, (mir ? -1.f : 1.f) * (two_mF / wu), 0.f);
          const float rs = __builtin_amdgcn_rcpf(fmaf(sg, (1.f / wu) * inv_lw, 0.f));
          rw[j][u] = fmaf(zv, mir ? -rs : rs, mir ? -(float)((1 << BITS) - 1) * wu * lw : 0.f);
        }
      }
      // coefficient pairs (t0 + u, t0 + u + 1) of each group: TPL / 2 adjacent pairs
#pragma unroll
      for (int j = 0; j < NG; ++j) {
        unsigned char* coef = lds + M::VA + j * M::VA_GROUP + coef_off<BITS>(t0 / 2);
        unsigned char* rwp = lds + M::VR + j * M::VA_GROUP + coef_off<BITS>(t0 / 2);
        if constexpr (TPL == 4) {
          *(float4*)coef = make_float4(cf[j][0], cf[j][1], cf[j][2], cf[j][3]);
          *(float4*)rwp = make_float4(rw[j][0], rw[j][1], rw[j][2], rw[j][3]);
        } else {
          *(float2*)coef = make_float2(cf[j][0], cf[j][1]);
          *(float2*)rwp = make_float2(rw[j][0], rw[j][1]);
        }
      }
      // token-wise K: (s', z'') of (token, group), the NG groups of a token adjacent
#pragma unroll
      for (int u = 0; u < TPL; ++u) {
        float2 kv[NG];
#pragma unroll
        for (int j = 0; j < NG; ++j)  // (a zero offset may lose its sign: it only ever is added)
          kv[j] = make_float2(fmaf(f16lo(kz[u][j]), ktok_sc, 0.f), fmaf(f16hi(kz[u][j]), alpha, 0.f));
        float4* kd = (float4*)(lds + M::KB + M::kb_off(t0 + u));
#pragma unroll
        for (int j2 = 0; j2 < NG; j2 += 2) kd[j2 / 2] = make_float4(kv[j2].x, kv[j2].y, kv[j2 + 1].x, kv[j2 + 1].y);
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");

    // ---- per-lane constants of the main loop: hoisted out of the chunk loop
    // where the registers allow (chunks of 512 tokens are 2 iterations per
    // wave, so rebuilding them per chunk costs ~20 VALU per iteration); INT2
    // with G = 64 fits its 4 work-groups per CU only when they are rebuilt
    // from a laundered lane id, so none of them is live through the prologue
    int mlane = lane;
    if (BITS == 2 && NG == 2) asm volatile("" : "+v"(mlane));
    const int mn_ = mlane & 15, mg = mlane >> 4, mhh = mn_ & 3, mnq = mn_ >> 2;
    const uint32_t koff = lane_koff(mg, mn_);
    const int tk0 = C::tok(mnq, mg, 0);
    const bool qlive = mg == mnq;
    int src[2][2];
#pragma unroll
    for (int k = 0; k < 2; ++k)
#pragma unroll
      for (int m2 = 0; m2 < 2; ++m2) {
        const int sq = BITS == 2 ? mg : 2 * k + (mg >> 1);
        const int sg = BITS == 2 ? 2 * k + m2 : 2 * (mg & 1) + m2;
        src[k][m2] = 4 * (mhh + 4 * sq + 16 * sg);
      }
    // sparse P.V: A row mn_ = 4 x + r holds head x, replica r & 1; its
    // compressed dword p pairs with B group m = 2 (g >> 1) + (p & 1) of word
    // row rw = 2 (g & 1) + (p >> 1): (VGPR m of unpack half 0, VGPR m ^ 2 of
    // half 1), where the index picks replica r & 1's VGPR mr = m ^ 2 (r & 1):
    // the P'' pair of tokens 16 rw + 4 (r & 1) + mr and + 8, held by score lane
    // (2 (r & 1) + (mr >> 1), x + 4 rw) in pk[p & 1]; the replicas' source
    // lanes are 16 apart, on different permute banks
    // (INT4: word rows g and g + 4 in unpack halves 0 and 1, VGPR m of a word
    // codes m and m + 4: replica r's pair of word row 2 (g & 1) + (p >> 1) + 4 r
    // sits in score lane (2 (p >> 1) + (mr >> 1), x + 4 (g & 1) + 8 r))
    int sadr[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int rw = 2 * (mg & 1) + (p >> 1);
      sadr[p] = BITS == 2 ? 4 * ((mnq + 4 * rw) + 16 * (2 * (mhh & 1) + ((mg >> 1) ^ (mhh & 1))))
                          : 4 * ((mnq + 4 * (mg & 1) + 8 * (mhh & 1)) + 16 * (2 * (p >> 1) + ((mg >> 1) ^ (mhh & 1))));
    }
    const int sidx = (mhh & 1) ? (int)0xEEEEEEEEu : 0x44444444;
    // byte offsets of the lane's coefficient pairs within an iteration
    // (iterations start at multiples of 64 tokens: pair rel / 2 + r sits at
    // 4 rel + the offset of pair r, r < 32)
    static_assert(C::TIT == 64, "coefficient pair blocks");
    const int cfo0 = coef_off<BITS>(tk0 / 2), cfo1 = coef_off<BITS>((tk0 + C::D2) / 2);
    float Qs[NG];
#pragma unroll
    for (int j = 0; j < NG; ++j) Qs[j] = red[16 + mhh * 4 + j];

    row_t nkz[TPL], nvz[TPL];

    for (int jj = 0;; ++jj) {
      const int it = 2 * (wv + 4 * (jj >> 1)) + (jj & 1);
      const int t0 = cb + it * C::TIT;
      if (t0 >= ce) break;
      // the next chunk's rows, issued with the first iteration's code loads:
      // waited for one iteration later, not by this iteration's first product.
      // A next chunk exists only after a whole one, and in a whole chunk every
      // wave has an iteration jj = 0, so the rows passed on are always loaded.
      static_assert(M::CHUNK >= 4 * 2 * C::TIT, "every wave iterates in a whole chunk");
      if constexpr (PREFETCH) {
        if (jj == 0 && cb + M::CHUNK < te) load_rows(cb + M::CHUNK, nkz, nvz);
      }
      Codes nxt;
      const int t1 = t0 + ((jj & 1) ? 7 : 1) * C::TIT;  // this wave's next iteration
      if (PAGED) {
        if (t1 < te) {
          load_block((long)pg_next * H + h, nxt, koff, mg, mn_);
          if (next_it(t1) < te) pg_next = page_at(next_it(t1));
        }
      } else if (t1 < te) {
        load_block(chunk_of(t1), nxt, koff, mg, mn_);
      }
      const int rel = t0 - cb;

      // QK^T: k-step s belongs to channel group s * NG / 16; consecutive
      // MFMAs go to different groups' accumulators
      float S[4];
      {
        const u4* qb = (const u4*)(lds + (qlive ? M::QB + mhh * M::HEAD_STRIDE : M::QZ));
        f4 acc[NG];
#pragma unroll
        for (int j = 0; j < NG; ++j) acc[j] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ss = 0; ss < 16; ++ss) {
          const int j = ss % NG, s = j * (16 / NG) + ss / NG;
          const uint32_t w = BITS == 4 ? cur.k[s >> 2][s & 3] : cur.k[s >> 3][(s >> 1) & 3];
          const u4 av = BITS == 4 ? unpack4(w) : unpack2(w, s & 1);
          acc[j] = mfma(av, qb[s], acc[j]);
        }
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int t = rel + tk0 + (q4 >> 1) + C::D2 * (q4 & 1);  // S[q4]'s token
          const float4* kt = (const float4*)(lds + M::KB + M::kb_off(t));  // two groups per float4
          float sv = mneg;  // the score less the running maximum
#pragma unroll
          for (int j2 = 0; j2 < NG; j2 += 2) {
            const float4 p = kt[j2 / 2];
            sv = fmaf(acc[j2][q4], p.x, fmaf(p.y, Qs[j2], sv));
            sv = fmaf(acc[j2 + 1][q4], p.z, fmaf(p.w, Qs[j2 + 1], sv));
          }
          S[q4] = sv;
        }
      }
      if (t0 + C::TIT > te) {  // the split's partial last iteration only
        asm volatile("");  // keeps this a branch (see the quantised decode kernel)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (t0 + tk0 + (j >> 1) + C::D2 * (j & 1) >= te) S[j] = -INFINITY;
      }
      // m_run is the same in all lanes of a head, so a lane's own maximum
      // past m_run + kThr is the same test as its head's: the cross-lane
      // reduction is needed only when the running maximum moves, and for
      // the wave's first scores
      const float lmx = fmaxf(fmaxf(S[0], S[1]), fmaxf(S[2], S[3]));
      if (m_run == -INFINITY || __any(lmx > (float)kThr)) {
        float Sr[4];  // the scores (to the rounding of S - mneg); masked stay -inf
#pragma unroll
        for (int j = 0; j < 4; ++j) Sr[j] = S[j] == -INFINITY ? -INFINITY : S[j] - mneg;
        const float mn = fmaxf(m_run, head_max(fmaxf(fmaxf(Sr[0], Sr[1]), fmaxf(Sr[2], Sr[3]))));
#pragma unroll
        for (int j = 0; j < 4; ++j) S[j] = Sr[j] - mn;
        mneg = -mn;
        const float sc = exp2_fast(m_run - mn);
        // the first scores of this wave (sc = 0) plant the seed
        const float k0 = m_run == -INFINITY ? kSeedV : 0.f;
        // sparse P.V: lane (g, n)'s tiles hold head g, whose scale score lane g has
        const float so = SPV ? __shfl(sc, mg) : sc, ko = SPV ? __shfl(k0, mg) : k0;
#pragma unroll
        for (int c = 0; c < 8; ++c)
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) O[c][q4] = fmaf(O[c][q4], so, ko);
#pragma unroll
        for (int j = 0; j < NG; ++j) X[j] *= sc;
        kseed = fmaf(kseed, sc, k0);
        lsum *= sc;
        m_run = mn;
      }
      float P[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) P[j] = exp2_fast(S[j]);
      lsum += (P[0] + P[1]) + (P[2] + P[3]);

      // PV, one channel group at a time: its P'' operand, its tiles, its offset tile
#pragma unroll
      for (int j = 0; j < NG; ++j) {
        const unsigned char* cf = lds + M::VA + j * M::VA_GROUP;
        const float2 c0 = *(const float2*)(cf + 4 * rel + cfo0);
        const float2 c1 = *(const float2*)(cf + 4 * rel + cfo1);
        uint32_t pk[2];
        pk[0] = pack_f16x2(P[0] * c0.x, P[1] * c1.x);
        pk[1] = pack_f16x2(P[2] * c0.y, P[3] * c1.y);
        {  // the group's offset sum over the same rounded P''
          const unsigned char* rb = lds + M::VR + j * M::VA_GROUP;
          const float2 r0 = *(const float2*)(rb + 4 * rel + cfo0);
          const float2 r1 = *(const float2*)(rb + 4 * rel + cfo1);
          float ox = X[j];
          ox = fmaf(f16lo(pk[0]), r0.x, ox);  // token tk0
          ox = fmaf(f16hi(pk[0]), r1.x, ox);  // tk0 + D2
          ox = fmaf(f16lo(pk[1]), r0.y, ox);  // tk0 + 1
          ox = fmaf(f16hi(pk[1]), r1.y, ox);  // tk0 + D2 + 1
          X[j] = ox;
        }
        if (SPV) {
          // 4 permutes, then one sparse product of 64 tokens per tile; B group
          // m = (VGPR m of unpack half 0, VGPR m ^ 2 of half 1) of the lane's word
          u4 ap;
#pragma unroll
          for (int p = 0; p < 4; ++p) ap[p] = (uint32_t)__builtin_amdgcn_ds_bpermute(sadr[p], (int)pk[p & 1]);
#pragma unroll
          for (int ct = 0; ct < TPG; ++ct) {
            const int c = j * TPG + ct;
            const uint32_t w = cur.v[c];
            const u4 h0 = BITS == 4 ? unpack4v(w) : unpack2v(w, 0);
            const u4 h1 = BITS == 4 ? unpack4v(cur.v[8 + c]) : unpack2v(w, 1);
            O[c] = smfmac(ap, u8v{h0[0], h1[2], h0[1], h1[3], h0[2], h1[0], h0[3], h1[1]}, O[c], sidx);
          }
          continue;
        }
        u4 bp[2];
#pragma unroll
        for (int k = 0; k < 2; ++k)
#pragma unroll
          for (int m = 0; m < 4; ++m)
            bp[k][m] = (uint32_t)__builtin_amdgcn_ds_bpermute(src[k][m >> 1], (int)pk[m & 1]);
#pragma unroll
        for (int k = 0; k < 2; ++k) {
#pragma unroll
          for (int ct = 0; ct < TPG; ++ct) {
            const int c = j * TPG + ct;
            const uint32_t w = BITS == 4 ? cur.v[8 * k + c] : cur.v[c];
            const u4 av = BITS == 4 ? unpack4v(w) : unpack2v(w, k);
            O[c] = mfma(av, bp[k], O[c]);
          }
        }
      }
      cur = nxt;
    }
    if constexpr (PREFETCH) {
#pragma unroll
      for (int u = 0; u < TPL; ++u) {
        kz[u] = nkz[u];
        vz[u] = nvz[u];
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  }

  // ---- per-wave result ----------------------------------------------------
  lsum = head_sum(lsum);
  {
    const float s24 = ldexpf(1.f, F + 24), sF = ldexpf(1.f, F);
#pragma unroll
    for (int j = 0; j < NG; ++j) {
      const float off = head_sum(X[j]);  // head n & 3's offset sum of group j
      if (SPV) {
        // head g's two replica rows, each started from the seed
        const float offk = __shfl(fmaf(-2.f * kseed, s24, off * sF), g);
#pragma unroll
        for (int ct = 0; ct < TPG; ++ct) {
          f4& o = O[j * TPG + ct];
          o[0] = fmaf(o[0] + o[1], s24, offk);
        }
        continue;
      }
      const float offk = fmaf(-kseed, s24, off * sF);    // (O - kseed) 2^(F + 24) + off 2^F
#pragma unroll
      for (int ct = 0; ct < TPG; ++ct)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) O[j * TPG + ct][q4] = fmaf(O[j * TPG + ct][q4], s24, offk);
    }
  }

  // ---- merge the four waves --------------------------------------------
  __syncthreads();
  float* mo = (float*)(lds + M::MO);
  float* ml = (float*)(lds + M::ML);
  if (n < 4 && g == 0) ml[(wv * 4 + n) * 2] = m_run;
  __syncthreads();
  float mall = -INFINITY;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) mall = fmaxf(mall, ml[(w * 4 + hh) * 2]);
  const float f = (m_run == -INFINITY) ? 0.f : exp2_fast(m_run - mall);
  __syncthreads();
  if (SPV) {
    const float fo = __shfl(f, g);  // head g's factor
    float* dst = mo + (wv * 4 + g) * kHeadDim + n;
#pragma unroll
    for (int c = 0; c < 8; ++c) dst[16 * c] = O[c][0] * fo;
    if (n < 4 && g == 0) ml[(wv * 4 + n) * 2 + 1] = lsum * f;
  } else if (n < 4) {
    // lane (n, g) holds rows 4g .. 4g + 3 of every tile: channels 16c + 4g + q4
    float* dst = mo + (wv * 4 + n) * kHeadDim + 4 * g;
#pragma unroll
    for (int c = 0; c < 8; ++c)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) dst[16 * c + q4] = O[c][q4] * f;
    if (g == 0) ml[(wv * 4 + n) * 2 + 1] = lsum * f;
  }
  if (n < 4 && g == 0) ml[(wv * 4 + n) * 2] = mall;
  __syncthreads();
  {
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
    if (ws.direct) {
      if (a.out_bf16) {
        __bf16 b0 = (__bf16)o0, b1 = (__bf16)o1;
        uint32_t pk = (uint32_t)__builtin_bit_cast(uint16_t, b0) |
                      ((uint32_t)__builtin_bit_cast(uint16_t, b1) << 16);
        *(uint32_t*)((uint16_t*)a.out + row * kHeadDim + d) = pk;
      } else {
        *(float2*)((float*)a.out + row * kHeadDim + d) = make_float2(o0, o1);
      }
    } else {
      const long pr = ws.pbase + qh * ws.pmul;
      *(float2*)(a.part_o + pr * kHeadDim + d) = make_float2(o0, o1);
      if (d == 0) {
        a.part_ml[pr * 2] = ml[(0 * 4 + qh) * 2];
        a.part_ml[pr * 2 + 1] = lt;
      }
    }
  }
}

template <int BITS, int NG>
hipError_t launch_tg(const DecodeArgs& a, hipStream_t s) {
  dim3 grid((unsigned)(a.dev_plan ? a.plan_items : decode_grid_blocks((long)a.batch * a.num_kv_heads, a.num_splits)));
  if (a.page_table) decode_tg_kernel<BITS, NG, true><<<grid, kThreads, 0, s>>>(a);
  else decode_tg_kernel<BITS, NG, false><<<grid, kThreads, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_quant_tg(const kvq_format& f, const DecodeArgs& a, hipStream_t s) {
  if (f.group == 64) return f.bits == 4 ? launch_tg<4, 2>(a, s) : launch_tg<2, 2>(a, s);
  return f.bits == 4 ? launch_tg<4, 4>(a, s) : launch_tg<2, 4>(a, s);
}

}  // namespace kvq
