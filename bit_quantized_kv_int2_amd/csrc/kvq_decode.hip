// Split-KV decode attention over INT2/INT4 quantised KV caches, gfx950.
//
// Method (FOSCAR, arXiv:2611.09722; rag-lover.com explainer, limits section):
// the per-group affine map x = s*c + z is never applied per element.
//   q.K^T contracts over channels:
//     token-wise K   (acc-fold):     S_t = s_t * (q . c_t) + z_t * sum(q)
//     channel-wise K (operand-fold): S_t = (q*s_i) . c_t + sum_d q_d z_{i,d}
//   P.V contracts over tokens:
//     token-wise V   (operand-fold): O   = sum_t (P_t s_t) c_t + sum_t P_t z_t
//     channel-wise V (acc-fold):     O_d = sum_i s_{i,d} (sum_{t in i} P_t c_{t,d})
//                                          + z_{i,d} sum_{t in i} P_t,
//                                    scaled per 128-token group, never across groups.
//
// gfx950 mapping
//   * Matrix unit. Dense form v_mfma_f32_16x16x32_f16 (INT4 q.K^T, INT4
//     channel-wise-V P.V, the fp8 variants use scaled fp8 products): A =
//     codes (16 rows x 32 k), B = folded query / probabilities; in q.K^T the
//     B columns are 4 heads x 4 token quarters (block diagonal over k). Sparse
//     form v_smfmac_f32_16x16x64_f16 (INT2 q.K^T and P.V, INT4 token-wise-V
//     P.V): the block-diagonal operand, q'' or P'', becomes the 2:4-sparse A
//     (its two nonzeros of every four k and their index) and the codes the
//     dense B, at twice the multiply-adds per issue slot.
//   * Operand construction: a 2- or 4-bit code ANDed out of its packed 32-bit
//     word, left at its bit offset inside a 16-bit lane with every other bit
//     zero, is the binary16 subnormal c * 2^k * 2^-24 (k = the code's bit
//     offset within its byte). Unpacking costs one AND per two codes plus one
//     shift per word: 5 ops per 8 INT4 codes, 9 per 16 INT2 codes, no base
//     constant to cancel later. The 2^k weight is divided out of the other
//     operand (an exact power of two).
//   * Consistent offsets: every offset term is computed from the rounded
//     fp16 operand the matrix unit actually consumed, so rounding q*s or P*s
//     to fp16 perturbs only the weights, not the cancellation between the
//     code term and the offset term.
//   * Token <-> lane maps are chosen so that each score lane's probability
//     pairs are the token pairs of one packed V VGPR: P'' reaches the P.V
//     operand with one ds_bpermute per operand dword.
//   * A work-group takes one split (a multiple of 256 tokens) of one
//     (sequence, KV head) row, in the per-XCD order of work_item, and walks it
//     in 2048-token chunks. Per chunk, each wave builds the fold operands of
//     its own 128-token groups in LDS: q*s per K group (channel-wise K) or q
//     (token-wise K), per-token or per-group V coefficients. The four waves
//     then stream 64 tokens per iteration each: whole-line 1 KB wave loads of
//     the codes one iteration ahead, online softmax with a lazily moved
//     maximum; the (m, l, O) of the four waves are merged through LDS.
//   * Offset terms from the same rounded P that feeds the code tiles:
//     token-wise V sums P''_t (w rho)_t on the vector unit (four fmas per
//     lane and iteration; on gfx950 a matrix product and vector work do not
//     overlap, so an extra tile would cost more); channel-wise V takes
//     sum_t P''_t from one more product against a fixed "code 1" pattern.
#include <math.h>

#include "kvq_internal.h"
#include "kvq_decode_common.h"

namespace kvq {
namespace {


template <int BITS, int KAX, int VAX, bool PAGED, bool FP8>
__global__ void __launch_bounds__(kThreads, groups_per_cu(BITS, VAX)) decode_kernel(DecodeArgs a) {
  using C = Cfg<BITS>;
  // fp8 operands for P.V too: O[0..3] are the four 128-deep products'
  // accumulators; token-wise V: X[0] the offset sum
  constexpr bool PV8 = FP8;
  using M = Lds<KAX, VAX>;
  __shared__ __attribute__((aligned(16))) unsigned char lds[M::TOTAL];
  float* qs = (float*)(lds + M::QS);
  float* red = (float*)(lds + M::RED);
  unsigned* redu = (unsigned*)red;

  // work-item and work-group ids straight from the builtins: this file is
  // built with the IEEE mode bit cleared, which keeps the device library's
  // id helpers from being inlined
  static_assert(M::TOTAL >= (8 + kThreads) * 4, "find_split borrows the start of the LDS");
  poison_lds<kThreads>(lds, M::TOTAL);
  const Split ws = find_split(a, (int*)lds);
  if (!ws.live) return;  // padding, or past the plan's work-items
  const int sp = ws.sp, h = ws.h, b = ws.b;
  const int tid = __builtin_amdgcn_workitem_id_x(), lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: keeps addressing scalar
  const int H = a.num_kv_heads, Hq = H * kGqa;
  int L = min(max(a.seq_lens[b], 0), a.max_len);  // contract: 0 <= len <= max_len
  if (a.len_mode == 1) L -= L % kGroup;  // whole groups only (the rest is a residual window)
  const int tb = sp * ws.S;
  const int te = min(tb + ws.S, L);
  const long row0 = (long)b * Hq + (long)h * kGqa;  // first query head row of this KV head

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

  // ---- cache addressing -------------------------------------------------
  const long unit = (long)b * H + h;
  auto chunk_of = [&](int t) -> long {  // 64-token chunk of token t
    if (!PAGED) return unit * (a.padded_len / kPage) + t / kPage;
    return (long)a.page_table[(long)b * a.max_pages + t / kPage] * H + h;
  };
  auto ksz_chan = [&](int t0, int d) -> const uint16_t* {  // pair of (group of t0, channel d)
    if (!PAGED) return a.k_sz + ((unit * (a.padded_len / kGroup) + t0 / kGroup) * kHeadDim + d) * 2;
    return a.k_sz + (chunk_of(t0) * kHeadDim + d) * 2;
  };
  auto vsz_chan = [&](int t0, int d) -> const uint16_t* {
    if (!PAGED) return a.v_sz + ((unit * (a.padded_len / kGroup) + t0 / kGroup) * kHeadDim + d) * 2;
    return a.v_sz + (chunk_of(t0) * kHeadDim + d) * 2;
  };
  auto ksz_tok = [&](int t) -> const uint16_t* { return a.k_sz + (chunk_of(t) * kPage + t % kPage) * 2; };
  auto vsz_tok = [&](int t) -> const uint16_t* { return a.v_sz + (chunk_of(t) * kPage + t % kPage) * 2; };

  // lane roles: C/B layout column n = head (n & 3) + 4 q, lane group g;
  // A layout row ri
  const int n = lane & 15, g = lane >> 4, hh = n & 3, nq = n >> 2;
  // INT2 fp16 q.K^T on the 2:4-sparse product (SQK): the score registers
  // that lane L holds with the dense product sit in lane perm(L), perm
  // swapping lane bits 5:4 and 1:0; sl is this lane's index in the dense
  // layout, and everything that follows the scores uses it
  constexpr bool SQK = BITS == 2 && !FP8;
  auto perm = [](int l) { return ((l & 3) << 4) | (l & 12) | (l >> 4); };
  // and lane 16 a + b loads the K row that dense-layout lane 16 (b >> 2) +
  // 4 (b & 3) + a loads (the token of score slot a in its column b)
  auto kperm = [](int l) { return ((l & 12) << 2) | ((l & 3) << 2) | (l >> 4); };
  const int kl = SQK ? kperm(lane) : lane;
  const int sl = SQK ? perm(lane) : lane;
  const int sn = sl & 15, sg = sl >> 4, shh = sn & 3;
  const int ri = lane & 15;

  // ---- code loads for one 64-token iteration ---------------------------
  // An iteration is one 64-token block of the cache (iterations start at
  // multiples of 64). The block order puts in bytes 16 l .. 16 l + 15 of each
  // 1 KB piece what lane l = 16 g + ri needs: for K the row of token
  // tok(g, ri>>2, ri&3), 16 bytes per piece; for V the words of channels
  // 8 ri .. 8 ri + 7 of word rows g (pieces 0, 1) and 4 + g (INT4: 2, 3).
  // Every load is a whole-line 1 KB wave access, issued non-temporal: the
  // codes are read once, and such streams read HBM faster when they do not
  // allocate in the caches.
  struct Codes {
    u4 k[C::KDW / 4];
    u4 v[C::NVW];
  };
  auto lane_koff = [](int lg, int lr) { return (uint32_t)(16 * (16 * lg + lr)); };  // bytes
  auto lane_voff = [](int lg, int lr) { return (uint32_t)(4 * (16 * lg + lr)); };   // words
  auto load_block = [&](long ch, Codes& cd, uint32_t koff, uint32_t voff) {
    const unsigned char* kb = a.k_codes + ch * (kPage * C::KROW) + koff;
#pragma unroll
    for (int e = 0; e < C::KDW / 4; ++e) cd.k[e] = __builtin_nontemporal_load((const u4*)(kb + 1024 * e));
    const uint32_t* vb = a.v_words + ch * ((kPage / C::TPW) * kHeadDim) + voff;
#pragma unroll
    for (int e = 0; e < C::NVW; ++e) cd.v[e] = __builtin_nontemporal_load((const u4*)(vb + 256 * e));
  };
  auto load_codes = [&](int t0, Codes& cd, uint32_t koff, uint32_t voff) {
    load_block(chunk_of(t0), cd, koff, voff);
  };
  // Paged caches: the physical page of a wave's next iteration is loaded one
  // iteration before its codes, so the code loads never wait on a page-table
  // read; the load's wait falls in with the code loads' own at the end of the
  // iteration. A wave's next iteration is 64 tokens on within a 128-token group
  // (iterations start at multiples of 64, and groups at multiples of 128), else
  // 448 tokens on, in its next group of the same or the next chunk.
  auto next_it = [](int t) { return t + (((t >> 6) & 1) ? 7 : 1) * C::TIT; };
  // (the index is passed through a vector register so that the loaded page
  // stays in one too: taken as wave-uniform, it would be moved to a scalar
  // register, and waited for, right after the load)
  auto page_at = [&](int t) -> int {
    int z = 0;
    asm volatile("" : "+v"(z));
    return a.page_table[(long)b * a.max_pages + t / kPage + z];
  };

  // Wave wv owns the 128-token groups wv, wv + 4, wv + 8, ... of the split
  // (64-token iterations 2G and 2G + 1 of each such group G). It builds the
  // fold operands of exactly those groups into LDS slots no other wave reads,
  // so after the query is shared the waves never wait for each other until
  // the final merge.
  // The first iteration's codes go out before anything else; later
  // iterations (also across chunk boundaries) are loaded one ahead.
  Codes cur;
  int pg_next = 0;  // paged: physical page of this wave's next iteration
  {
    const int t0 = tb + 2 * wv * C::TIT;
    if (t0 < te) load_codes(t0, cur, lane_koff(kl >> 4, kl & 15), lane_voff(g, ri));
    if (PAGED && next_it(t0) < te) pg_next = page_at(next_it(t0));
  }

  // q'' row of one head, 16 B per dense k-step s (piece s >> 3, dword
  // (s >> 1) & 3, unpack half s & 1; VGPR m = 0..3). Sparse q.K^T reads it as
  // the compressed A operand of product s & 7: A lane group g takes VGPRs
  // 2 (g >> 1) and + 1 of piece 0, then of piece 1, so a k-step's 16 B go to
  // two 8-byte places in the 32 B of that product
  auto put_qrow = [&](unsigned char* row, int ks, u4 w) {
    if (SQK) {
      *(u2*)(row + 32 * (ks & 7) + 8 * (ks >> 3)) = u2{w[0], w[1]};
      *(u2*)(row + 32 * (ks & 7) + 16 + 8 * (ks >> 3)) = u2{w[2], w[3]};
    } else {
      ((u4*)row)[ks] = w;
    }
  };

  // ---- query: once per split -------------------------------------------------
  {
    const int d = lane * 2;  // wave wv loads query head wv
    const uint32_t qq = *(const uint32_t*)(a.q + (row0 + wv) * kHeadDim + d);
    const float q0 = bf16val((uint16_t)(qq & 0xFFFF)), q1 = bf16val((uint16_t)(qq >> 16));
    const float m = wave_max_dpp(fmaxf(fabsf(q0), fabsf(q1)));
    if (KAX == KVQ_CHANNEL_WISE) {
      // q * 2^-Eq / w(d) in binary16 (|.| < 1; exact: a bf16 value scaled by
      // powers of two), stored in B-operand order for the per-group products
      const int Eq = exp_above(m);
      const float t = ldexpf(1.f, -Eq);
      _Float16* qh = (_Float16*)(lds + M::QS) + wv * 128;
      if (FP8) {  // fp8 / fp4 QK^T: positions of the codes' A elements
        qh[C::qpos8(d)] = (_Float16)(q0 * t / C::w8(d));
        qh[C::qpos8(d + 1)] = (_Float16)(q1 * t / C::w8(d + 1));
      } else {
        qh[C::qpos(d)] = (_Float16)(q0 * t * C::inv_wd(d));
        qh[C::qpos(d + 1)] = (_Float16)(q1 * t * C::inv_wd(d + 1));
      }
      if (lane == 0) redu[wv] = (unsigned)Eq;
    } else {
      qs[wv * 128 + d] = q0;
      qs[wv * 128 + d + 1] = q1;
      const float sum = wave_sum_dpp(q0 + q1);
      if (lane == 0) { red[wv] = m; red[20 + wv] = sum; }
    }
  }
  if (tid < M::QZ_BYTES / 16) ((u4*)(lds + M::QZ))[tid] = u4{0u, 0u, 0u, 0u};
  __syncthreads();
  if (KAX == KVQ_TOKEN_WISE) {
    // token-wise K: q'' = q * 2^-E / w (max |q''| < 2^14), shared by all waves
    const float qmax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    const int E = exp_above(qmax) - 14;
    if (tid < 64 && FP8) {
      // fp8: q * 2^-(E + 6) / w8 (< 2^8) as an E4M3 pair hi + lo / 16, hi in
      // bytes 0-127 and lo in 128-255 of the head's row; a bf16 q needs at
      // most 8 significant bits, so hi + lo / 16 is q exactly
      const float two_mE6 = ldexpf(1.f, -E - 6);
      const int ck = tid & 15, qh = tid >> 4;
      uint32_t hw[2], lw[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        float x[4];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const int d = C::ch8(ck, t, b);
          x[b] = qs[qh * 128 + d] * two_mE6 / C::w8(d);
        }
        hw[t] = cvt_fp8x2<true>(x[2], x[3], cvt_fp8x2<false>(x[0], x[1], any_u32()));
        const f2 h01 = fp8x2_val<false>(hw[t]), h23 = fp8x2_val<true>(hw[t]);
        lw[t] = cvt_fp8x2<true>((x[2] - h23.x) * 16.f, (x[3] - h23.y) * 16.f,
                                cvt_fp8x2<false>((x[0] - h01.x) * 16.f, (x[1] - h01.y) * 16.f, any_u32()));
      }
      *(u2*)(lds + M::QB + qh * M::HEAD_STRIDE + 8 * ck) = u2{hw[0], hw[1]};
      *(u2*)(lds + M::QB + qh * M::HEAD_STRIDE + 128 + 8 * ck) = u2{lw[0], lw[1]};
    } else if (tid < 64) {
      const float two_mE = ldexpf(1.f, -E);
      const int s = tid & 15, qh = tid >> 4;
      uint32_t wds[4];
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        float v0 = qs[qh * 128 + C::k_run(s, 0) + m] * two_mE * C::inv_w(m);
        float v1 = qs[qh * 128 + C::k_run(s, 1) + m] * two_mE * C::inv_w(m);
        wds[m] = pack_f16x2(v0, v1);
      }
      put_qrow(lds + M::QB + qh * M::HEAD_STRIDE, s, u4{wds[0], wds[1], wds[2], wds[3]});
    }
    __syncthreads();
  }
  const float ktok_sc = KAX == KVQ_TOKEN_WISE
      ? alpha * ldexpf(1.f, exp_above(fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]))) - 14 + (FP8 ? 6 : 24))
      : 0.f;

  // accumulators: O and X in units of 2^-F, m_run in log2 units
  f4 O[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) O[c] = f4{0.f, 0.f, 0.f, 0.f};
  // token-wise V: this lane's part of its head's offset sum, in X[0] (held as
  // a 4-vector: with a scalar the INT4 fp8 kernels' registers spill)
  f4 X = f4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY;
  float lsum = 0.f;
  // fp16 token-wise V: the running output starts from kSeedV (set when the
  // first scores arrive), scaled along with it; kseed is its current value
  constexpr bool SEED = !PV8 && VAX == KVQ_TOKEN_WISE;
  // fp16 token-wise V: P.V on the 2:4-sparse 16x16x64 product, with P'' as
  // its compressed A operand and the V codes as its dense B. Accumulator
  // tile c of lane (g, n) then holds head g, channel 8 n + c, in rows 0 and 1
  // (two replicas that split the tokens; rows 2 and 3 repeat them and are
  // never read)
  constexpr bool SPV = SEED;
  // INT2 channel-wise V on the sparse product too (SPVC): scalar outputs Oc
  // (head g, channel 8 n + c of lane (g, n)), folded per iteration; lsum then
  // follows the tiles' head
  constexpr bool SPVC = !PV8 && VAX == KVQ_CHANNEL_WISE && BITS == 2;
  float Oc[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) Oc[c] = 0.f;
  float kseed = 0.f;
  // P'' = P * coef * 2^-F with max P'' < 2^14. Token-wise V: F follows the
  // largest scale this wave has seen and only grows (the accumulators are
  // rescaled by the exact power of two when it does); channel-wise V: constant.
  int F = kThr - 14 + (PV8 ? 6 : 0);

  // ---- chunks of up to kChunkTokens tokens: prologue, then the main loop ----
  for (int cb = tb; cb < te; cb += kChunkTokens) {
    const int ce = min(cb + kChunkTokens, te);
    const int ntok = ce - cb;
    const int ng = (ntok + kGroup - 1) / kGroup;

    // Per-lane prologue indices are derived from a copy of the lane id that
    // the compiler must treat as new in every chunk: otherwise it hoists them
    // (and the addresses built from them) out of the chunk loop and keeps
    // them live through the main loop, which costs registers and occupancy.
    int pl = lane;
    asm volatile("" : "+v"(pl));
    // lane l serves group gl = wv + 4 (l / 16) of the chunk: the 16 lanes of
    // a DPP row share a group
    const int gl = wv + 4 * (pl >> 4);
    const bool glive = gl < ng;
    // token-wise (s, z): the wave's 4 groups are 128 runs of 4 tokens (32
    // per group); lane l takes runs l and l + 64, tokens tb_run[r] .. +3.
    // Consecutive lanes then load consecutive 16-byte (s, z) runs and store
    // consecutive 16-byte coefficient slots (no two lanes on one bank).
    // Runs start at multiples of 4 tokens: a run's token e sits in code slot
    // e % SLOTS.
    int tb_run[2];
#pragma unroll
    for (int rr = 0; rr < 2; ++rr) {
      const int r = pl + 64 * rr;
      tb_run[rr] = kGroup * (wv + 4 * (r >> 5)) + 4 * (r & 31);
    }
    const int ck_s = pl & 15;  // channel-wise K: k-step of group gl; channel-wise V: channels 8 ck_s ..

    // ---- prologue: (s, z) loads -------------------------------------------
    // Contiguous caches: (s, z) pairs of one (sequence, KV head) are one run
    // per token (token-wise) or per (group, channel) (channel-wise), so the
    // chunk's pairs sit at a base shared by the wave plus a 32-bit lane offset
    // (groups start at multiples of 128 tokens: the chunk's first group is
    // cb / 128)
    const long gbase = (unit * (a.padded_len / kGroup) + cb / kGroup) * (long)kHeadDim;
    const unsigned char* ksz_c = (const unsigned char*)a.k_sz + 4 * (KAX == KVQ_TOKEN_WISE ? unit * a.padded_len + cb : gbase);
    const unsigned char* vsz_c = (const unsigned char*)a.v_sz + 4 * (VAX == KVQ_TOKEN_WISE ? unit * a.padded_len + cb : gbase);
    // byte offsets within the chunk's run fit 32 bits (a wave-shared base plus
    // one offset register per load)
    auto ksz_tok_c = [&](int r) -> const void* { return PAGED ? (const void*)ksz_tok(cb + r) : ksz_c + (uint32_t)(4 * r); };
    auto vsz_tok_c = [&](int r) -> const void* { return PAGED ? (const void*)vsz_tok(cb + r) : vsz_c + (uint32_t)(4 * r); };
    // channel-wise (s, z): lanes of groups past the end (a partial chunk)
    // read the chunk's last group instead, so every lane loads and none needs
    // a mask; only the lanes of live groups write fold operands
    const int glc = min(gl, ng - 1);
    auto ksz_chan_c = [&](int d) -> const void* {  // group glc of the chunk, channel d
      return PAGED ? (const void*)ksz_chan(cb + glc * kGroup, d) : ksz_c + (uint32_t)(4 * (glc * kHeadDim + d));
    };
    auto vsz_chan_c = [&](int d) -> const void* {
      return PAGED ? (const void*)vsz_chan(cb + glc * kGroup, d) : vsz_c + (uint32_t)(4 * (glc * kHeadDim + d));
    };
    u4 vz[2];  // V (s, z): 2 runs of 4 tokens, or 8 pairs
    u4 kz[2];  // K (s, z): 2 runs of 4 tokens, or 8 channels
    // FULL: a whole chunk (every token run of the lane is inside the split,
    // no masks); otherwise token runs past the end read as (0, 0)
    auto load_sz = [&](auto full_c) {
      constexpr bool FULL = decltype(full_c)::value;
      if (!FULL) {
        vz[0] = vz[1] = u4{0u, 0u, 0u, 0u};
        kz[0] = kz[1] = u4{0u, 0u, 0u, 0u};
      }
      if (VAX == KVQ_TOKEN_WISE) {
#pragma unroll
        for (int rr = 0; rr < 2; ++rr) {
          if (FULL || tb_run[rr] < ntok) {
            vz[rr] = *(const u4*)vsz_tok_c(tb_run[rr]);
            if (!FULL && tb_run[rr] + 4 > ntok) {  // tokens past the end contribute (s, z) = (0, 0)
#pragma unroll
              for (int e = 1; e < 4; ++e)
                if (tb_run[rr] + e >= ntok) vz[rr][e] = 0u;
            }
          }
        }
      } else {
        const u4* p = (const u4*)vsz_chan_c(8 * ck_s);
        vz[0] = p[0];
        vz[1] = p[1];
      }
      if (KAX == KVQ_TOKEN_WISE) {
#pragma unroll
        for (int rr = 0; rr < 2; ++rr)
          if (FULL || tb_run[rr] < ntok) kz[rr] = *(const u4*)ksz_tok_c(tb_run[rr]);
      } else if (FP8) {
        // the 8 channels of B-operand positions 8 ck_s .. + 7: pair e = 2 b + t
        // is channel ch8(ck_s, t, b)
        if (BITS == 4) {
#pragma unroll
          for (int hf = 0; hf < 2; ++hf) kz[hf] = *(const u4*)ksz_chan_c(8 * ck_s + 4 * hf);
        } else {  // every other channel of 16
#pragma unroll
          for (int e = 0; e < 8; ++e) kz[e >> 2][e & 3] = *(const uint32_t*)ksz_chan_c(C::ch8(ck_s, e & 1, e >> 1));
        }
      } else {
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) kz[hf] = *(const u4*)ksz_chan_c(C::k_run(ck_s, hf));
      }
    };
    if (ntok == kChunkTokens) load_sz(BoolC<true>{});
    else load_sz(BoolC<false>{});

    // Scales of 0 (a constant group or token, or the (0, 0) read for what
    // lies past the end) stand for a stand-in scale in the fold formulas. The
    // waves that hold one patch it into the (s, z) words before the common
    // formulas, which then need no selects; smallest_s is the lane's smallest
    // scale bit pattern (sign cleared) over its 8 words.
    auto smallest_s = [](const u4 (&z)[2]) {
      uint32_t m = 0x7FFFu;
#pragma unroll
      for (int e = 0; e < 8; ++e) m = min(m, z[e >> 2][e & 3] & 0x7FFFu);
      return m;
    };
    auto patch_zero_s = [](u4 (&z)[2], uint32_t one) {  // one: binary16 bits of the stand-in
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t u = z[e >> 2][e & 3];
        if ((u & 0x7FFFu) == 0u) z[e >> 2][e & 3] = (u & 0xFFFF0000u) | one;
      }
    };
    // the channel-wise stand-in 2^(es - 1), es = ((max scale bits) >> 10) - 14:
    // binary16 exponent field (max bits) >> 10, or 2^-15 (0x0200) below the
    // normal range
    auto half_top_s = [](uint32_t mb) { return (mb & 0x7C00u) ? (mb & 0x7C00u) : 0x0200u; };

    // ---- prologue: fold operands into this wave's LDS slots -----------------
    // the previous chunk's main loop of this wave has issued all its reads
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    // V first: its (s, z) registers are free before the K part needs its own
    if (VAX == KVQ_TOKEN_WISE) {
      // every scale of this wave's tokens < 2^Fs (scales of 0 are replaced by
      // 1, hence Fs >= 1; bit patterns of scales >= 0 order as values)
      uint32_t smax = 0u, smin = 0x7FFFu;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t sb = vz[e >> 2][e & 3] & 0x7FFFu;
        smax = max(smax, sb);
        smin = min(smin, sb);
      }
      const uint32_t mb = wave_max_u(smax);
      // sigma = s, or 1 where s == 0 (a constant token, or the (0, 0) of a
      // token past the end): the rare waves that hold such a scale patch it
      // to 1 here, so the common path needs no selects
      if (__any(smin == 0u)) patch_zero_s(vz, 0x3C00u);
      // (fp8 P.V: P'' < 2^8 for E4M3, six binades lower)
      const int Fc = max((int)(mb >> 10) - 14, 1) + kThr - 14 + (PV8 ? 6 : 0);
      if (cb == tb) {
        F = Fc;
      } else if (Fc > F) {
        const float sc = ldexpf(1.f, F - Fc);
#pragma unroll
        for (int c = 0; c < 8; ++c) O[c] *= sc;
        X *= sc;
        if (SEED) kseed *= sc;
        F = Fc;
      }
      const float two_mF = ldexpf(1.f, -F);
      // coef[t] = sigma * 2^-F / w(t) and the offset weight w(t) * rho in fp32
      // (sigma = s, or 1 where s == 0; rho = z / sigma). Runs start at a
      // multiple of 4 tokens, so token e of a run has slot e % SLOTS.
      unsigned char* coef = lds + M::VA;
      float rw[2][4];
#pragma unroll
      for (int rr = 0; rr < 2; ++rr) {
        float cf[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          // weight of the token's code: fp16 subnormal slot, or (fp8 P.V)
          // its E4M3 byte's bit offset (INT2 tokens 4b + 1, 4b + 3: 4)
          const float wt = PV8 ? ((BITS == 2 && (e & 1)) ? 4.f : 1.f)
                               : (float)(1 << (BITS * (e % C::SLOTS)));
          const float sg = f16lo(vz[rr][e]), zv = f16hi(vz[rr][e]);
          // fp16 P.V: tokens of the odd slots (e odd) enter mirrored, with
          // the scale negated and the offset z + qmax s. wt / sigma is the
          // reciprocal of sigma / wt (a power-of-two scaling: the same bits
          // as the reciprocal of sigma times wt)
          const bool mir = !PV8 && (e & 1);
          cf[e] = sg * ((mir ? -1.f : 1.f) * (two_mF / wt));
          const float rs = __builtin_amdgcn_rcpf(sg * (1.f / wt));
          // (a product as an fma with +0 added: read straight from the binary16
          // z; only the sign of a zero product can differ, which no sum sees)
          rw[rr][e] = fmaf(zv, mir ? -rs : rs, mir ? -(float)((1 << BITS) - 1) * wt : 0.f);
        }
        *(float4*)(coef + coef_off<BITS>(tb_run[rr] / 2)) = make_float4(cf[0], cf[1], cf[2], cf[3]);
        // fp32 w * rho per token, addressed like coef
        *(float4*)(lds + M::VR + coef_off<BITS>(tb_run[rr] / 2)) = make_float4(rw[rr][0], rw[rr][1], rw[rr][2], rw[rr][3]);
      }
    } else {
      // (sigma, rho) of two channels per float4 (sigma = s, or 1 where s == 0;
      // rho = z / sigma); fp16 P.V takes rho - kKappa (the products start
      // from kKappa * sum P'')
      if (__any(smallest_s(vz) == 0u)) patch_zero_s(vz, 0x3C00u);
      const float kap = PV8 ? 0.f : kKappa;
      if (glive) {
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const uint32_t p0 = vz[e >> 2][e & 3], p1 = vz[e >> 2][(e + 1) & 3];
          const float s0 = f16lo(p0), z0 = f16hi(p0), s1 = f16lo(p1), z1 = f16hi(p1);
          *(float4*)(lds + M::VA + vg_off<KAX, VAX>(gl, 8 * ck_s + e)) =
              make_float4(s0, z0 * __builtin_amdgcn_rcpf(s0) - kap, s1, z1 * __builtin_amdgcn_rcpf(s1) - kap);
        }
      }
    }
    if (KAX == KVQ_CHANNEL_WISE && FP8) {
      // fp8 QK^T: x = q 2^-Eq / w8 * s 2^(8 - es) (< 2^8; s == 0 counts as
      // 2^(es - 1), offset weight adjusted to match) as E4M3 hi + lo / 16;
      // rho8 = w8 (z / s) 2^(es - 8); the offset sum uses the rounded pair,
      // and S = alpha 2^(es + Eq - 8) acc + alpha 2^Eq sum (hi + lo/16) rho8.
      const uint32_t mb = row_max_u(max_lo16(kz[0], kz[1]));
      const int es = (int)(mb >> 10) - 14;
      if (__any(smallest_s(kz) == 0u)) patch_zero_s(kz, half_top_s(mb));
      const float up = ldexpf(1.f, 8 - es), dn = ldexpf(1.f, es - 8);
      float sp[8], rho[8];  // index e = 2 b + t
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t pr = kz[e >> 2][e & 3];
        const float sv = f16lo(pr), zv = f16hi(pr);
        const float wt = C::w8(C::ch8(ck_s, e & 1, e >> 1));
        sp[e] = sv * up;
        rho[e] = fmaf(zv, __builtin_amdgcn_rcpf(sv) * (wt * dn), 0.f);
      }
      float2* kb = (float2*)(lds + M::KB);
      const u4* qh = (const u4*)(lds + M::QS);
      float hb = 0.f;  // lanes ck_s < 4: the bias sum of head ck_s (every lane of a row holds each sum)
#pragma unroll 1
      for (int qh_i = 0; qh_i < 4; ++qh_i) {
        const u4 qv = qh[qh_i * 16 + ck_s];  // positions 8 ck_s + 4 t + b
        uint32_t hw[2], lw[2];
        float bias = 0.f;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          float x[4];
#pragma unroll
          for (int b = 0; b < 4; ++b) {
            const uint32_t hv = qv[2 * t + (b >> 1)];
            x[b] = ((b & 1) ? f16hi(hv) : f16lo(hv)) * sp[2 * b + t];
          }
          hw[t] = cvt_fp8x2<true>(x[2], x[3], cvt_fp8x2<false>(x[0], x[1], any_u32()));
          const f2 h01 = fp8x2_val<false>(hw[t]), h23 = fp8x2_val<true>(hw[t]);
          lw[t] = cvt_fp8x2<true>((x[2] - h23.x) * 16.f, (x[3] - h23.y) * 16.f,
                                  cvt_fp8x2<false>((x[0] - h01.x) * 16.f, (x[1] - h01.y) * 16.f, any_u32()));
          const f2 l01 = fp8x2_val<false>(lw[t]), l23 = fp8x2_val<true>(lw[t]);
          bias = fmaf(fmaf(l01.x, 0.0625f, h01.x), rho[t], bias);
          bias = fmaf(fmaf(l01.y, 0.0625f, h01.y), rho[2 + t], bias);
          bias = fmaf(fmaf(l23.x, 0.0625f, h23.x), rho[4 + t], bias);
          bias = fmaf(fmaf(l23.y, 0.0625f, h23.y), rho[6 + t], bias);
        }
        if (glive) {
          unsigned char* qrow = lds + M::QB + gl * M::GROUP_STRIDE + qh_i * M::HEAD_STRIDE;
          *(u2*)(qrow + 8 * ck_s) = u2{hw[0], hw[1]};
          *(u2*)(qrow + 128 + 8 * ck_s) = u2{lw[0], lw[1]};
        }
        bias = row_sum(bias);
        hb = ck_s == qh_i ? bias : hb;
      }
      if (glive && ck_s < 4) {
        const int Eq = (int)redu[ck_s];
        kb[gl * 4 + ck_s] = make_float2(alpha * ldexpf(1.f, es + Eq - 8), alpha * ldexpf(hb, Eq));
      }
    } else if (KAX == KVQ_CHANNEL_WISE) {
      // s' = s * 2^(14 - es) with every s of the group < 2^es (s' < 2^14), and
      // the offset weight rho' = w * (z / s) * 2^(es - 14); a channel with
      // s == 0 (all codes 0) takes s' = 2^13 and rho' = w * z * 2^-13, which
      // gives the same offset. q'' = (q 2^-Eq / w) * s' is rounded once to
      // binary16 (one packed multiply per two channels), and
      // S = alpha 2^(10 + es + Eq) acc + alpha 2^Eq sum q'' rho' uses the
      // rounded q'' in both terms, so rounding moves only the weight of x^.
      const uint32_t mb = row_max_u(max_lo16(kz[0], kz[1]));
      const int es = (int)(mb >> 10) - 14;
      if (__any(smallest_s(kz) == 0u)) patch_zero_s(kz, half_top_s(mb));
      const float up = ldexpf(1.f, 14 - es), dn = ldexpf(1.f, es - 14);
      uint32_t spk[4];
      float rho[8];
      {
        float sp8[8];
#pragma unroll
        for (int hf = 0; hf < 2; ++hf)
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            const float sv = f16lo(kz[hf][m]), zv = f16hi(kz[hf][m]);
            sp8[4 * hf + m] = sv * up;
            rho[4 * hf + m] = fmaf(zv, __builtin_amdgcn_rcpf(sv) * (C::w(m) * dn), 0.f);  // product, from binary16 z
          }
#pragma unroll
        for (int m = 0; m < 4; ++m) spk[m] = pack_f16x2(sp8[m], sp8[4 + m]);
      }
      float2* kb = (float2*)(lds + M::KB);
      const u4* qh = (const u4*)(lds + M::QS);
      float hb = 0.f;  // lanes ck_s < 4: the bias sum of head ck_s (every lane of a row holds each sum)
#pragma unroll 1
      for (int qh_i = 0; qh_i < 4; ++qh_i) {  // one head at a time keeps few registers live
        const u4 qv = qh[qh_i * 16 + ck_s];
        u4 wds;
        float bias = 0.f;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          wds[m] = mul_f16x2(qv[m], spk[m]);
          bias = fmaf(f16lo(wds[m]), rho[m], fmaf(f16hi(wds[m]), rho[4 + m], bias));
        }
        if (glive) put_qrow(lds + M::QB + gl * M::GROUP_STRIDE + qh_i * M::HEAD_STRIDE, ck_s, wds);
        bias = row_sum(bias);
        hb = ck_s == qh_i ? bias : hb;
      }
      if (glive && ck_s < 4) {
        const int Eq = (int)redu[ck_s];
        kb[gl * 4 + ck_s] = make_float2(alpha * ldexpf(1.f, 10 + es + Eq), alpha * ldexpf(hb, Eq));
      }
    } else {
      float4* ktok = (float4*)(lds + M::KB);  // (s', z'') of two tokens per float4
#pragma unroll
      for (int rr = 0; rr < 2; ++rr) {
        const int t4 = tb_run[rr];  // 4 tokens
#pragma unroll
        for (int e = 0; e < 4; e += 2) {
          const bool v0 = t4 + e < ntok, v1 = t4 + e + 1 < ntok;
          const uint32_t p0 = kz[rr][e], p1 = kz[rr][e + 1];
          ktok[(t4 + e) / 2] = make_float4(v0 ? f16lo(p0) * ktok_sc : 0.f, v0 ? f16hi(p0) * alpha : 0.f,
                                           v1 ? f16lo(p1) * ktok_sc : 0.f, v1 ? f16hi(p1) * alpha : 0.f);
        }
      }
    }
    // LDS operations of one wave complete in order; the fence keeps the
    // compiler from moving the main loop's reads above the writes
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");

    // ---- per-lane constants of the main loop, rebuilt per chunk from a
    // laundered lane id so that none of them is live through the prologue
    int mlane = lane;
    asm volatile("" : "+v"(mlane));
    const int mn_ = mlane & 15, mg = mlane >> 4, mhh = mn_ & 3, mnq = mn_ >> 2;
    // the same in the dense score layout (sparse q.K^T: of the permuted lane)
    const int msl = SQK ? perm(mlane) : mlane;
    const int smn = msl & 15, smg = msl >> 4, smhh = smn & 3, smnq = smn >> 2;
    const int mkl = SQK ? kperm(mlane) : mlane;
    const uint32_t koff = lane_koff(mkl >> 4, mkl & 15), voff = lane_voff(mg, mn_);
    // compact scores: score lane (n, g) holds tokens tk0 + {0, D2, 1, D2 + 1} (j = 0..3)
    const int tk0 = C::tok(smnq, smg, 0);
    // B operand of QK^T is block diagonal: column (head, q) is nonzero only in
    // k-group q, so only lanes with g == q read q''; the others read zeros
    // (sparse q.K^T: A row mn_ = 4 x + slot is head x, token slot mhh, whose
    // tokens lane group g holds when slot >> 1 == g & 1; the others read zeros)
    const bool qlive = SQK ? (mhh >> 1) == (mg & 1) : mg == mnq;
    // PV B operand VGPR m of k-step k comes from lane src[k][m >> 1], register pk[m & 1]
    int src[2][2];
#pragma unroll
    for (int k = 0; k < 2; ++k)
#pragma unroll
      for (int m2 = 0; m2 < 2; ++m2) {
        const int sq = BITS == 2 ? mg : 2 * k + (mg >> 1);
        const int sg = BITS == 2 ? 2 * k + m2 : 2 * (mg & 1) + m2;
        src[k][m2] = 4 * (mhh + 4 * sq + 16 * sg);  // byte address for ds_bpermute
      }
    // sparse P.V: A row mn_ = 4 x + r holds head x, replica r & 1. Its
    // compressed dword p pairs with B group m = 2 (g >> 1) + (p & 1) of word
    // row rw = 2 (g & 1) + (p >> 1): (VGPR m of unpack half 0, VGPR m ^ 2 of
    // half 1), of which the index picks one (positions 0, 1 or 2, 3), replica
    // r & 1 the VGPR mr = m ^ 2 (r & 1) of half r & 1. That is the P'' pair
    // of tokens 16 rw + 4 (r & 1) + mr and + 8, which score lane
    // (2 (r & 1) + (mr >> 1), x + 4 rw) holds in pk[p & 1] (mr and m share
    // their parity). The two replicas of a 32-lane half then read source lanes
    // 16 apart, on different banks of the permute (32 apart would share one)
    // INT4: B lane g holds word rows g (unpack half 0) and g + 4 (half 1),
    // VGPR m of a word codes m and m + 4; replica r's VGPR mr of word row
    // wr = 2 (g & 1) + (p >> 1) + 4 r is the pair of tokens 8 wr + mr and + 4,
    // which score lane (2 (p >> 1) + (mr >> 1), x + 4 (g & 1) + 8 r) holds in
    // pk[p & 1]; sources again 16 apart per 32-lane half
    int sadr[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int rw = 2 * (mg & 1) + (p >> 1);
      const int sd = BITS == 2 ? (mnq + 4 * rw) + 16 * (2 * (mhh & 1) + ((mg >> 1) ^ (mhh & 1)))
                               : (mnq + 4 * (mg & 1) + 8 * (mhh & 1)) + 16 * (2 * (p >> 1) + ((mg >> 1) ^ (mhh & 1)));
      sadr[p] = 4 * (SQK ? perm(sd) : sd);  // the score lane's actual index
    }
    const int sidx = (mhh & 1) ? (int)0xEEEEEEEEu : 0x44444444;
    // fp8 P.V: this lane's A row r = mn_ holds head r & 3 for the channel half
    // (r >> 2) & 1, part hi (r < 8) or lo; its 16 probability bytes come from
    // four score lanes (ds_bpermute byte addresses asrc), two per dword
    const int arow_j = (mn_ >> 2) & 1, arow_lo = mn_ >> 3;
    const int ascale = arow_lo ? kE8M0One - 4 : kE8M0One;
    // v_perm selectors of the A row's two halves: byte-interleave two
    // gathered dwords (even / odd A dwords), or 0x0C (a zero byte) in every
    // position for the half of the other channel
    // INT4: lane groups 1 and 3 gather the dwords of each pair in the other
    // order (qd ^ 1). Their sources then lie 16 lanes from those of lane
    // groups 0 and 2 instead of 32, on other banks of the permute; the swap
    // exchanges the two inputs of each v_perm below, which bit 2 of every
    // live selector byte undoes
    const int qsw = BITS == 4 ? (mg & 1) : 0;
    const uint32_t sflip = qsw ? 0x04040404u : 0u;
    uint32_t asel[2][2];
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      asel[hf][0] = hf == arow_j ? 0x05010400u ^ sflip : 0x0C0C0C0Cu;
      asel[hf][1] = hf == arow_j ? 0x07030602u ^ sflip : 0x0C0C0C0Cu;
    }
    int asrc[4];
#pragma unroll
    for (int qd = 0; qd < 4; ++qd) {
      int ls;
      if (BITS == 2) {
        const int gi = (qd >> 1) | ((qd & 1) << 1);  // 0, 2, 1, 3
        ls = (mhh + 4 * mg) + 16 * gi;
      } else {
        const int qs = qd ^ qsw;
        const int gi = 2 * (mg & 1) + (qs & 1), nq = (mg >> 1) + 2 * (qs >> 1);
        ls = (mhh + 4 * nq) + 16 * gi;
      }
      asrc[qd] = 4 * ls;
    }
    // channel-wise V with fp8 P.V: 2^-F / E4M3 weight of the even / odd tokens
    const float cw8[2] = {ldexpf(1.f, -F), ldexpf(1.f, -F) / (BITS == 2 ? 4.f : 1.f)};
    float cw[2];  // channel-wise V: 2^-F / weight of the compact values' tokens
#pragma unroll
    for (int aa = 0; aa < 2; ++aa) {
      // tk0 is even: aa = 1 is an odd slot, whose codes enter mirrored
      const int slot = (tk0 + aa) % C::TPW;
      cw[aa] = (aa ? -1.f : 1.f) * ldexpf(1.f, -F) / (float)(1 << (BITS * (slot % C::SLOTS)));
    }
    const float Qh = KAX == KVQ_TOKEN_WISE ? red[20 + smhh] : 0.f;
    // token-wise V: byte offsets of this lane's coefficient pairs within an
    // iteration. An iteration starts at a multiple of 64 tokens (32 pairs,
    // two whole 16-pair blocks), so pair rel / 2 + r sits at 4 rel + the
    // offset of pair r, and r < 32 for both of the lane's pairs
    static_assert(C::TIT == 64, "coefficient pair blocks");  // tk0 + D2 < 64: r < 32
    const int cfo0 = coef_off<BITS>(tk0 / 2), cfo1 = coef_off<BITS>((tk0 + C::D2) / 2);

    // ---- main loop over this wave's iterations of the chunk: the next
    // iteration's codes are in flight while this one is computed
    for (int jj = 0;; ++jj) {
      const int it = 2 * (wv + 4 * (jj >> 1)) + (jj & 1);
      const int t0 = cb + it * C::TIT;
      if (t0 >= ce) break;
      Codes nxt;
      const int t1 = t0 + ((jj & 1) ? 7 : 1) * C::TIT;  // this wave's next iteration
      if (PAGED) {
        if (t1 < te) {
          load_block((long)pg_next * H + h, nxt, koff, voff);
          if (next_it(t1) < te) pg_next = page_at(next_it(t1));
        }
      } else if (t1 < te) {
        load_codes(t1, nxt, koff, voff);
      }
      const int rel = t0 - cb;
      const int gi = rel / kGroup;

      // QK^T over 16 k-steps of 8 channels per k-group: 64 tokens x 4 heads
      float S[4];
      f4 acc;
      float2 sb;       // channel-wise K: the group's (scale, bias)
      float4 p0, p1;   // token-wise K: (s', z'') of the lane's tokens
      {
        const u4* qb = (const u4*)(lds + (qlive ? M::QB + (KAX == KVQ_CHANNEL_WISE ? gi : 0) * M::GROUP_STRIDE +
                                                      mhh * M::HEAD_STRIDE
                                                : M::QZ));
        f4 c0 = f4{0.f, 0.f, 0.f, 0.f}, c1 = f4{0.f, 0.f, 0.f, 0.f};
        if (FP8 && BITS == 2) {
          // E2M1 codes: the 32 channels of A lane group g pair with the E4M3
          // bytes of half g >> 1 of lane groups 2 (g & 1) and 2 (g & 1) + 1.
          // So column (head, q) takes 16 bytes of its q'' row (offset
          // 16 (mg & 1) in each 32-channel run) into half q >> 1 when
          // mg >> 1 == q & 1, and zeros everywhere else. One read of the wave
          // then fetches 8 distinct live 16-byte chunks, on 8 consecutive
          // 16-byte bank quads (of the 256-byte bank period) starting at the
          // group's row base, and 2 zero chunks. The zero chunks are placed on
          // two of the other 8 quads: a 128-bit read is conflict-free only
          // when the wave's distinct chunks fall on different quads.
          const bool live = (mg >> 1) == (mnq & 1);
          const int qbase = M::QB + (KAX == KVQ_CHANNEL_WISE ? gi : 0) * M::GROUP_STRIDE;
          const unsigned char* qrow = lds + qbase + mhh * M::HEAD_STRIDE + 16 * (mg & 1);
          const int zq = (qbase / 16 + 8 + (mg & 1) - M::QZ / 16) & 15;  // zero row quad offset
          const unsigned char* zrow = lds + M::QZ + 16 * zq;
          const u4* b0 = (const u4*)(live && mnq < 2 ? qrow : zrow);
          const u4* b1 = (const u4*)(live && mnq >= 2 ? qrow : zrow);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const v8i av = unpack_k8<BITS>(cur.k, j);
            c0 = mfma4k(av, cat8(b0[2 * j], b1[2 * j]), c0, kE8M0One);
            c1 = mfma4k(av, cat8(b0[8 + 2 * j], b1[8 + 2 * j]), c1, kE8M0One - 4);
          }
        } else if (FP8) {
          // 4 MFMAs of 32 channels per k-group, hi and lo (scale 2^-4) parts
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const v8i av = unpack_k8<BITS>(cur.k, j);
            c0 = mfma8(av, cat8(qb[2 * j], qb[2 * j + 1]), c0, kE8M0One);
            c1 = mfma8(av, cat8(qb[8 + 2 * j], qb[9 + 2 * j]), c1, kE8M0One - 4);
          }
        } else if (SQK) {
          // 8 sparse products of 16 channels x 4 tokens per column. Lane group
          // pairs (0, 1) and (2, 3) trade halves (odd rows of the piece-0
          // dwords with even rows of the piece-1 dwords): then rows 0 and 2
          // hold piece 0 and rows 1 and 3 piece 1 of two tokens, x (the even
          // row's, slots 0 and 2) and y (the odd row's, slots 1 and 3); B group
          // m is (VGPR m of x, VGPR m of y), and the index takes x or y
          u4 kx, ky;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const auto r = __builtin_amdgcn_permlane16_swap(cur.k[0][i], cur.k[1][i], false, false);
            kx[i] = (uint32_t)r[0];
            ky[i] = (uint32_t)r[1];
          }
          const int qbase = M::QB + (KAX == KVQ_CHANNEL_WISE ? gi : 0) * M::GROUP_STRIDE;
          // read s's 8 live 16-byte chunks fill 8 consecutive bank quads from
          // the group's base + 2 s; the zero row sits 8 quads on, at zero-region
          // quad zq + 2 s (zq < 16 and s < 8 stay inside the region)
          const int zq = (qbase / 16 + 8 - M::QZ / 16) & 15;
          const unsigned char* abase = qlive ? lds + qbase + mnq * M::HEAD_STRIDE + 16 * (mg >> 1)
                                             : lds + M::QZ + 16 * zq;
#pragma unroll
          for (int s = 0; s < 8; ++s) {
            const u4 av = *(const u4*)(abase + 32 * s);
            const u4 x = unpack2(kx[s >> 1], s & 1), y = unpack2(ky[s >> 1], s & 1);
            const u8v bv = u8v{x[0], y[0], x[1], y[1], x[2], y[2], x[3], y[3]};
            if (s & 1) c1 = smfmac(av, bv, c1, sidx);
            else c0 = smfmac(av, bv, c0, sidx);
          }
        } else {
#pragma unroll
          for (int s = 0; s < 16; ++s) {
            const uint32_t w = BITS == 4 ? cur.k[s >> 2][s & 3] : cur.k[s >> 3][(s >> 1) & 3];
            const u4 av = BITS == 4 ? unpack4(w) : unpack2(w, s & 1);
            if (s & 1) c1 = mfma(av, qb[s], c1);
            else c0 = mfma(av, qb[s], c0);
          }
        }
        acc = c0 + c1;
        // S[j]: the score less the running maximum, the subtraction folded
        // into the score's affine map (one add per iteration, not four);
        // score(j) is the score itself, for the rare moves of the maximum
        if (KAX == KVQ_CHANNEL_WISE) {
          sb = ((const float2*)(lds + M::KB))[gi * 4 + smhh];
          const float nb = sb.y - m_run;
#pragma unroll
          for (int j = 0; j < 4; ++j) S[j] = fmaf(acc[j], sb.x, nb);
        } else {
          const float4* kt = (const float4*)(lds + M::KB);  // (s', z'') per token, two per float4
          p0 = kt[(rel + tk0) / 2];
          p1 = kt[(rel + tk0 + C::D2) / 2];
          S[0] = fmaf(acc[0], p0.x, fmaf(p0.y, Qh, -m_run));  // token tk0
          S[1] = fmaf(acc[1], p1.x, fmaf(p1.y, Qh, -m_run));  // tk0 + D2
          S[2] = fmaf(acc[2], p0.z, fmaf(p0.w, Qh, -m_run));  // tk0 + 1
          S[3] = fmaf(acc[3], p1.z, fmaf(p1.w, Qh, -m_run));  // tk0 + D2 + 1
        }
      }
      auto score = [&](int j) {
        if (KAX == KVQ_CHANNEL_WISE) return fmaf(acc[j], sb.x, sb.y);
        const float4 p = (j & 1) ? p1 : p0;
        return (j & 2) ? fmaf(acc[j], p.z, p.w * Qh) : fmaf(acc[j], p.x, p.y * Qh);
      };
      if (t0 + C::TIT > te) {  // the split's partial last iteration only
        // (an instruction with side effects keeps this a branch: speculated,
        // the masks would cost 8 vector instructions in every iteration)
        asm volatile("");
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (t0 + tk0 + (j >> 1) + C::D2 * (j & 1) >= te) S[j] = -INFINITY;
      }
      // m_run is the same in all lanes of a head, so a lane's own maximum
      // past m_run + kThr is the same test as its head's: the cross-lane
      // reduction is needed only when the running maximum moves (and at a
      // wave's first scores, which stand at +inf against m_run = -inf)
      const float lmx = fmaxf(fmaxf(S[0], S[1]), fmaxf(S[2], S[3]));
      if (__any(lmx > (float)kThr)) {
        float Sr[4];  // the scores themselves (masked tokens stay -inf)
#pragma unroll
        for (int j = 0; j < 4; ++j) Sr[j] = S[j] == -INFINITY ? -INFINITY : score(j);
        const float lm = fmaxf(fmaxf(Sr[0], Sr[1]), fmaxf(Sr[2], Sr[3]));
        const float mn = fmaxf(m_run, SQK ? row_max(lm) : head_max(lm));
#pragma unroll
        for (int j = 0; j < 4; ++j) S[j] = Sr[j] - mn;
        const float sc = exp2_fast(m_run - mn);
        if (SEED) {
          // the first scores of this wave (sc = 0) plant the seed
          const float k0 = m_run == -INFINITY ? kSeedV : 0.f;
          // sparse P.V: lane (g, n)'s tiles hold head g, whose scale score lane g has
          const int hsrc = SQK ? 16 * mg : mg;  // the score lane of head mg
          const float so = SPV ? __shfl(sc, hsrc) : sc, ko = SPV ? __shfl(k0, hsrc) : k0;
#pragma unroll
          for (int c = 0; c < 8; ++c)
#pragma unroll
            for (int j = 0; j < 4; ++j) O[c][j] = fmaf(O[c][j], so, ko);
          kseed = fmaf(kseed, sc, k0);
        } else if (SPVC) {
          const float so = __shfl(sc, SQK ? 16 * mg : mg);  // head mg's factor
#pragma unroll
          for (int c = 0; c < 8; ++c) Oc[c] *= so;
          lsum *= so;
        } else {
#pragma unroll
          for (int c = 0; c < 8; ++c) O[c] *= sc;
        }
        X *= sc;
        if (!SPVC) lsum *= sc;
        m_run = mn;
      }
      float P[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) P[j] = exp2_fast(S[j]);

      if (PV8) {
        // P'' = P * coef as an E4M3 pair hi + lo / 16 in bytes [jj0, jj1, jj2, jj3]
        // (tokens tk0, tk0 + D2, tk0 + 1, tk0 + D2 + 1)
        float x0, x1, x2, x3;
        if (VAX == KVQ_TOKEN_WISE) {
          const unsigned char* cf = lds + M::VA;
          const float2 c0 = *(const float2*)(cf + 4 * rel + cfo0);
          const float2 c1 = *(const float2*)(cf + 4 * rel + cfo1);
          x0 = P[0] * c0.x, x1 = P[1] * c1.x, x2 = P[2] * c0.y, x3 = P[3] * c1.y;
        } else {  // P'' = P 2^-F / w8 (tk0 is even: INT2 tokens tk0 + 1, tk0 + D2 + 1 weigh 4)
          x0 = P[0] * cw8[0], x1 = P[1] * cw8[0], x2 = P[2] * cw8[1], x3 = P[3] * cw8[1];
        }
        lsum += (P[0] + P[1]) + (P[2] + P[3]);
        const uint32_t hw = cvt_fp8x2<true>(x2, x3, cvt_fp8x2<false>(x0, x1, any_u32()));
        const f2 h01 = fp8x2_val<false>(hw), h23 = fp8x2_val<true>(hw);
        const uint32_t lw = cvt_fp8x2<true>((x2 - h23.x) * 16.f, (x3 - h23.y) * 16.f,
                                            cvt_fp8x2<false>((x0 - h01.x) * 16.f, (x1 - h01.y) * 16.f, any_u32()));
        if (VAX == KVQ_TOKEN_WISE) {
          // offset sum from the same rounded P'' (consistent offsets)
          const f2 l01 = fp8x2_val<false>(lw), l23 = fp8x2_val<true>(lw);
          const unsigned char* rb = lds + M::VR;
          const float2 r0 = *(const float2*)(rb + 4 * rel + cfo0);
          const float2 r1 = *(const float2*)(rb + 4 * rel + cfo1);
          float ox = X[0];
          ox = fmaf(fmaf(l01.x, 0.0625f, h01.x), r0.x, ox);
          ox = fmaf(fmaf(l01.y, 0.0625f, h01.y), r1.x, ox);
          ox = fmaf(fmaf(l23.x, 0.0625f, h23.x), r0.y, ox);
          ox = fmaf(fmaf(l23.y, 0.0625f, h23.y), r1.y, ox);
          X[0] = ox;
        }
        // gather the A row: two source dwords per A dword, byte-interleaved
        uint32_t G[4];
#pragma unroll
        for (int qd = 0; qd < 4; ++qd) {
          const uint32_t gh = (uint32_t)__builtin_amdgcn_ds_bpermute(asrc[qd], (int)hw);
          const uint32_t gl = (uint32_t)__builtin_amdgcn_ds_bpermute(asrc[qd], (int)lw);
          G[qd] = arow_lo ? gl : gh;
        }
        int hv[8];
#pragma unroll
        for (int dw = 0; dw < 8; ++dw)
          hv[dw] = (int)__builtin_amdgcn_perm(G[2 * ((dw >> 1) & 1) + 1], G[2 * ((dw >> 1) & 1)],
                                              asel[dw >> 2][dw & 1]);
        const v8i av = v8i{hv[0], hv[1], hv[2], hv[3], hv[4], hv[5], hv[6], hv[7]};
        if (VAX == KVQ_TOKEN_WISE) {
#pragma unroll
          for (int c = 0; c < 4; ++c) O[c] = mfma8pv(av, unpack_v8<BITS>(cur.v, c), O[c], ascale);
        } else {
          // channel-wise V, acc-fold per group: this iteration's products in
          // fresh accumulators, and a fifth product against code 1 in every
          // k position (weight 1 or 4 like the codes) that gives each row's
          // sum of the same rounded P''; then O_d += sigma_d (G_d + rho_d sum P'')
          // for this lane's channels 8 n + 2 c + (g & 1) (C row 4 g + x: head x,
          // channel half g & 1, hi or lo part g >> 1)
          f4 Gc[4];
#pragma unroll
          for (int c = 0; c < 4; ++c)
            Gc[c] = mfma8pv(av, unpack_v8<BITS>(cur.v, c), f4{0.f, 0.f, 0.f, 0.f}, ascale);
          const f4 ps = mfma8pv(av, ones8<BITS>(), f4{0.f, 0.f, 0.f, 0.f}, ascale);
          const unsigned char* vgb = lds + M::VA + vg_off<KAX, VAX>(gi, 8 * mn_ + (mg & 1));
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const float2 sr = *(const float2*)(vgb + 16 * c);  // (sigma, rho) of channel 8 n + 2 c + (g & 1)
#pragma unroll
            for (int x = 0; x < 4; ++x) O[c][x] = fmaf(sr.x, fmaf(sr.y, ps[x], Gc[c][x]), O[c][x]);
          }
        }
      } else {
        // P'' into packed pairs: pk[a] = (token tk0 + a, token tk0 + a + D2)
        uint32_t pk[2];
        if (VAX == KVQ_TOKEN_WISE) {
          const unsigned char* cf = lds + M::VA;
          const float2 c0 = *(const float2*)(cf + 4 * rel + cfo0);
          const float2 c1 = *(const float2*)(cf + 4 * rel + cfo1);
          pk[0] = pack_f16x2(P[0] * c0.x, P[1] * c1.x);
          pk[1] = pack_f16x2(P[2] * c0.y, P[3] * c1.y);
          lsum += (P[0] + P[1]) + (P[2] + P[3]);
          // offset sum over the same rounded P'' (consistent offsets): the
          // lane's four tokens times their fp32 w * rho, addressed like coef.
          // Four VALU operations in place of an extra matrix tile (two
          // products per iteration, which the vector unit waits out).
          const unsigned char* rb = lds + M::VR;
          const float2 r0 = *(const float2*)(rb + 4 * rel + cfo0);
          const float2 r1 = *(const float2*)(rb + 4 * rel + cfo1);
          float ox = X[0];
          ox = fmaf(f16lo(pk[0]), r0.x, ox);  // token tk0
          ox = fmaf(f16hi(pk[0]), r1.x, ox);  // tk0 + D2
          ox = fmaf(f16lo(pk[1]), r0.y, ox);  // tk0 + 1
          ox = fmaf(f16hi(pk[1]), r1.y, ox);  // tk0 + D2 + 1
          X[0] = ox;
        } else {
          pk[0] = pack_f16x2(P[0] * cw[0], P[1] * cw[0]);
          pk[1] = pack_f16x2(P[2] * cw[1], P[3] * cw[1]);
        }
        // B columns 0-3 carry the four heads; the other twelve only repeated
        // them and nothing reads their results: zeros there cost 8 selects
        // per iteration and take switching power off the matrix unit, whose
        // clock this loop follows (measured 2 % faster, results unchanged)
        u4 bp[2];
        u4 ap;  // sparse P.V A operand: 4 permutes
        if (SPV || SPVC) {
#pragma unroll
          for (int p = 0; p < 4; ++p) ap[p] = (uint32_t)__builtin_amdgcn_ds_bpermute(sadr[p], (int)pk[p & 1]);
        } else {
#pragma unroll
          for (int k = 0; k < 2; ++k)
#pragma unroll
            for (int m = 0; m < 4; ++m) {
              const uint32_t v = (uint32_t)__builtin_amdgcn_ds_bpermute(src[k][m >> 1], (int)pk[m & 1]);
              bp[k][m] = mn_ < 4 ? v : 0u;
            }
        }

        if (SPV) {
          // PV: 8 sparse products of 64 tokens; B group m = (VGPR m of unpack
          // half 0, VGPR m ^ 2 of half 1) of the lane's word
#pragma unroll
          for (int c = 0; c < 8; ++c) {
            const uint32_t w = cur.v[c >> 2][c & 3];
            const u4 h0 = BITS == 4 ? unpack4v(w) : unpack2v(w, 0);
            const u4 h1 = BITS == 4 ? unpack4v(cur.v[2 + (c >> 2)][c & 3]) : unpack2v(w, 1);
            O[c] = smfmac(ap, u8v{h0[0], h1[2], h0[1], h1[3], h0[2], h1[0], h0[3], h1[1]}, O[c], sidx);
          }
        } else if (SPVC) {
          // sums of P'' per replica row from one product against +-w 2^-14:
          // column 0 every slot (minus on the mirrored ones), column 1 the
          // mirrored slots only (minus); the two VGPRs of a B group (m, m ^ 2)
          // share the slot's parity but not its weight 4^m
          u8v ob;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int m = (e & 1) ? ((e >> 1) ^ 2) : (e >> 1);
            const uint32_t hb = (uint32_t)(2 * m + 1) << 10;  // w 2^-14
            const uint32_t h = mn_ < 2 ? ((m & 1) ? (hb | 0x8000u) : (mn_ == 0 ? hb : 0u)) : 0u;
            ob[e] = h | (h << 16);
          }
          const f4 xs = smfmac(ap, ob, f4{0.f, 0.f, 0.f, 0.f}, sidx);
          // lane (x, 0): this iteration's sum P'' of head x; lane (x, 1): its mirrored part
          const float xr = xs[0] + xs[1];
          const float psum = __shfl(xr, 16 * mg) * 0x1p-10f;
          const float pneg = __shfl(xr, 16 * mg + 1) * 0x1p-10f;
          // the start value qmax sum_N P'' + kKappa sum P'' (taken back out
          // through rho - kKappa): the group's first iteration seeds the two
          // replica rows with half of its own each; the second adds its own
          // in the fold
          const float c0 = fmaf((float)((1 << BITS) - 1), pneg, kKappa * psum);
          const unsigned char* vgb = lds + M::VA + vg_off<KAX, VAX>(gi, 8 * mn_);
          // fresh products per iteration, 4 tiles at a time; each replica row
          // starts from half of the start value; O_d += sigma_d (G_d + rho_d sum P'')
#pragma unroll
          for (int hf = 0; hf < 2; ++hf) {
            float ch = 0.5f * c0;
            asm volatile("" : "+v"(ch));
            f4 G4[4];
#pragma unroll
            for (int c4 = 0; c4 < 4; ++c4) {
              const int c = 4 * hf + c4;
              const uint32_t w = cur.v[c >> 2][c & 3];
              const u4 h0 = unpack2v(w, 0), h1 = unpack2v(w, 1);
              G4[c4] = smfmac(ap, u8v{h0[0], h1[2], h0[1], h1[3], h0[2], h1[0], h0[3], h1[1]},
                              f4{ch, ch, 0.f, 0.f}, sidx);
            }
#pragma unroll
            for (int c4 = 0; c4 < 4; c4 += 2) {
              const int c = 4 * hf + c4;
              const float4 sr = *(const float4*)(vgb + 8 * c);  // (sigma, rho) of channels 8 n + c, + 1
              Oc[c] = fmaf(sr.x, fmaf(sr.y, psum, G4[c4][0] + G4[c4][1]), Oc[c]);
              Oc[c + 1] = fmaf(sr.z, fmaf(sr.w, psum, G4[c4 + 1][0] + G4[c4 + 1][1]), Oc[c + 1]);
            }
          }
          lsum += psum;
        } else if (VAX == KVQ_TOKEN_WISE) {
          // PV: 8 channel tiles, 2 k-steps of 32 tokens
#pragma unroll
          for (int k = 0; k < 2; ++k) {
#pragma unroll
            for (int c = 0; c < 8; ++c) {
              const uint32_t w = BITS == 4 ? cur.v[2 * k + (c >> 2)][c & 3] : cur.v[c >> 2][c & 3];
              const u4 av = BITS == 4 ? unpack4v(w) : unpack2v(w, k);
              O[c] = mfma(av, bp[k], O[c]);
            }
          }
        } else {
          // offset weights from the extra tile: row 0 holds +-w 2^-14 (minus
          // on the mirrored slots, whose P'' are negative) and gives sum P'';
          // row 1 holds -w 2^-14 on the mirrored slots only and gives their
          // sum. Normal binary16 rows: these sums keep the window's 24 bits.
          f4 Xg = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int k = 0; k < 2; ++k) {
            u4 ones = u4{0u, 0u, 0u, 0u};
            if (mn_ < 2) {
#pragma unroll
              for (int m = 0; m < 4; ++m) {
                const uint32_t hb = (uint32_t)(BITS * (m % C::SLOTS) + 1) << 10;  // w 2^-14
                const bool odd = (m % C::SLOTS) & 1;
                const uint32_t h = odd ? (hb | 0x8000u) : (mn_ == 0 ? hb : 0u);
                ones[m] = h | (h << 16);
              }
            }
            Xg = mfma(ones, bp[k], Xg);
          }
          // rows 0 and 1 live in lane group 0; back to the code products' units
          const float psum = __shfl(Xg[0], mn_) * 0x1p-10f;
          const float pneg = __shfl(Xg[1], mn_) * 0x1p-10f;
          // the group's products start from qmax sum_N P'' (the mirrored
          // tokens' offset) + kKappa sum P'' (taken back out through rho - kKappa)
          const float c0 = fmaf((float)((1 << BITS) - 1), pneg, kKappa * psum);
          const float4* vg = (const float4*)(lds + M::VA + vg_off<KAX, VAX>(gi, 32 * mg));
          // the group's partials in two halves of 4 channel tiles (16 accumulator
          // registers live instead of 32), each folded as soon as it is complete:
          // O_d += sigma_d (G_d + rho_d * sum P)
#pragma unroll
          for (int hf = 0; hf < 2; ++hf) {
            // the start value is rebuilt per half from a copy the compiler
            // must treat as new: four registers live only until the first
            // products of the half have issued
            float c0h = c0;
            asm volatile("" : "+v"(c0h));
            const f4 seed = f4{c0h, c0h, c0h, c0h};
            f4 G4[4];
#pragma unroll
            for (int k = 0; k < 2; ++k) {
#pragma unroll
              for (int c4 = 0; c4 < 4; ++c4) {
                const int c = 4 * hf + c4;
                const uint32_t w = BITS == 4 ? cur.v[2 * k + (c >> 2)][c & 3] : cur.v[c >> 2][c & 3];
                const u4 av = BITS == 4 ? unpack4v(w) : unpack2v(w, k);
                G4[c4] = mfma(av, bp[k], k == 0 ? seed : G4[c4]);
              }
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
#pragma unroll
              for (int c4 = 0; c4 < 4; c4 += 2) {
                // channels 32g + 8j + c and +1: (sigma, rho, sigma, rho)
                const int c = 4 * hf + c4;
                const float4 sr = vg[(8 * j + c) / 2];
                O[c][j] = fmaf(sr.x, fmaf(sr.y, psum, G4[c4][j]), O[c][j]);
                O[c + 1][j] = fmaf(sr.z, fmaf(sr.w, psum, G4[c4 + 1][j]), O[c + 1][j]);
              }
            }
          }
          lsum += psum;
        }
      }
      cur = nxt;
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  }

  // ---- per-wave result: numerator N and normaliser l (same scale) --------
  float lw;
  if (PV8) {
    // C rows 4 g + x of the four products: head x, channel half g & 1, part
    // g >> 1 (lo rows already scaled by 2^-4): add the lo rows (lane + 32),
    // then O[c][x] = (sum + offset of head x) * 2^F for channel 8 n + 2 c + (g & 1)
    lsum = head_sum(lsum);
    const float offh = head_sum(X[0]);
    const float sF = ldexpf(1.f, F);
    float offx[4];
#pragma unroll
    for (int x = 0; x < 4; ++x) offx[x] = __shfl(offh, x);
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int x = 0; x < 4; ++x) O[c][x] = (O[c][x] + __shfl_xor(O[c][x], 32) + offx[x]) * sF;
    lw = lsum;
  } else if (VAX == KVQ_TOKEN_WISE) {
    lsum = SQK ? row_sum(lsum) : head_sum(lsum);
    const float off = SQK ? row_sum(X[0]) : head_sum(X[0]);  // the lane's head's offset sum (every lane of the head)
    const float s24 = ldexpf(1.f, F + 24), sF = ldexpf(1.f, F);
    // (O - kseed) 2^(F + 24) + off 2^F
    if (SPV) {
      // head g's two replica rows, each started from the seed
      const float offk = __shfl(fmaf(-2.f * kseed, s24, off * sF), SQK ? 16 * g : g);
#pragma unroll
      for (int c = 0; c < 8; ++c) O[c][0] = fmaf(O[c][0] + O[c][1], s24, offk);
    } else {
      const float offk = fmaf(-kseed, s24, off * sF);
#pragma unroll
      for (int c = 0; c < 8; ++c)
#pragma unroll
        for (int j = 0; j < 4; ++j) O[c][j] = fmaf(O[c][j], s24, offk);
    }
    lw = lsum;
  } else if (SPVC) {
    const float s24 = ldexpf(1.f, F + 24);
#pragma unroll
    for (int c = 0; c < 8; ++c) Oc[c] *= s24;
    lw = __shfl(lsum, 16 * sn) * s24;  // score lanes (0, sn < 4): head sn
  } else {
    const float s24 = ldexpf(1.f, F + 24);
#pragma unroll
    for (int c = 0; c < 8; ++c) O[c] *= s24;
    lw = lsum * s24;
  }

  // ---- merge the four waves --------------------------------------------
  __syncthreads();  // main-loop LDS no longer needed
  float* mo = (float*)(lds + M::MO);
  float* ml = (float*)(lds + M::ML);
  if (sn < 4 && sg == 0) {
    ml[(wv * 4 + sn) * 2] = m_run;
  }
  __syncthreads();
  float mall = -INFINITY;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) mall = fmaxf(mall, ml[(w * 4 + shh) * 2]);
  const float f = (m_run == -INFINITY) ? 0.f : exp2_fast(m_run - mall);
  __syncthreads();
  if (PV8) {
    float fx[4];
#pragma unroll
    for (int x = 0; x < 4; ++x) fx[x] = __shfl(f, x);  // lane x holds head x
    if (g < 2) {
#pragma unroll
      for (int x = 0; x < 4; ++x)
#pragma unroll
        for (int c = 0; c < 4; ++c) mo[(wv * 4 + x) * kHeadDim + 8 * n + 2 * c + g] = O[c][x] * fx[x];
    }
    if (n < 4 && g == 0) ml[(wv * 4 + n) * 2 + 1] = lw * f;
  } else if (SPV || SPVC) {
    const float fo = __shfl(f, SQK ? 16 * g : g);  // head g's factor
    float* dst = mo + (wv * 4 + g) * kHeadDim + 8 * n;
#pragma unroll
    for (int c = 0; c < 8; ++c) dst[c] = (SPVC ? Oc[c] : O[c][0]) * fo;
    if (sn < 4 && sg == 0) ml[(wv * 4 + sn) * 2 + 1] = lw * f;
  } else if (n < 4) {
    float* dst = mo + (wv * 4 + n) * kHeadDim + 32 * g;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int c = 0; c < 8; ++c) dst[8 * j + c] = O[c][j] * f;
    if (g == 0) ml[(wv * 4 + n) * 2 + 1] = lw * f;
  }
  if (sn < 4 && sg == 0) ml[(wv * 4 + sn) * 2] = mall;
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
        // m in log2 units, l in units of 2^(S - m)
        a.part_ml[pr * 2] = ml[(0 * 4 + qh) * 2];
        a.part_ml[pr * 2 + 1] = lt;
      }
    }
  }
}

// LSE merge of n split partials: O = sum_i 2^(m_i - M) l_i O_i / sum_i 2^(m_i - M) l_i
// over the partials slot(0 .. n-1) (empty ones carry m = -inf and are skipped).
template <class Slot>
__device__ inline float merge_parts(const float* part_o, const float* part_ml, int n, int d, Slot slot) {
  float M = -INFINITY;
  for (int i = 0; i < n; ++i) M = fmaxf(M, part_ml[2 * slot(i)]);
  float num = 0.f, den = 0.f;
  if (M != -INFINITY) {
    for (int i = 0; i < n; ++i) {
      const long p = slot(i);
      const float m = part_ml[2 * p];
      if (m == -INFINITY) continue;
      const float w = exp2_fast(m - M) * part_ml[2 * p + 1];
      num = fmaf(w, part_o[p * kHeadDim + d], num);
      den += w;
    }
  }
  return den > 0.f ? num / den : 0.f;
}

__device__ inline void store_row(void* out, int out_bf16, long row, int d, float o) {
  if (out_bf16) ((__bf16*)out)[row * kHeadDim + d] = (__bf16)o;
  else ((float*)out)[row * kHeadDim + d] = o;
}

// LSE combine of a host plan's partials, [row][num_splits] slots per row.
__global__ void __launch_bounds__(128) combine_kernel(const float* part_o, const float* part_ml,
                                                      int num_splits, void* out, int out_bf16) {
  const long row = __builtin_amdgcn_workgroup_id_x();
  const int d = __builtin_amdgcn_workitem_id_x();
  const float o = merge_parts(part_o, part_ml, num_splits, d,
                              [&](int i) { return row * num_splits + i; });
  store_row(out, out_bf16, row, d, o);
}

// Combine of a device-planned call. Plan mode 0 (about equal lengths): the
// max_len plan's partials, [row][ns]. Mode 1 (ragged): row (sequence b, query
// head hq) has n = ceil(L / S) splits, the work-items row_first .. row_first
// + n - 1 of its KV head (partial slot item * 4 + hq mod 4); a row with one
// split was written by the decode, an empty row gets zeros.
__global__ void __launch_bounds__(128) combine_plan_kernel(DecodeArgs a) {
  const long row = __builtin_amdgcn_workgroup_id_x();
  const int d = __builtin_amdgcn_workitem_id_x();
  const int S = a.plan_hdr[0], mode = a.plan_hdr[1];
  if (mode == 0) {
    const int ns = a.num_splits;
    if (ns == 1) return;
    const float o = merge_parts(a.part_o, a.part_ml, ns, d, [&](int i) { return row * ns + i; });
    store_row(a.out, a.out_bf16, row, d, o);
    return;
  }
  const int Hq = a.num_kv_heads * kGqa;
  const int b = (int)(row / Hq), hq = (int)(row % Hq);
  int L = min(max(a.seq_lens[b], 0), a.max_len);
  if (a.len_mode == 1) L -= L % kGroup;
  const int n = L > 0 ? (L + S - 1) / S : 0;
  if (n == 1) return;
  float o = 0.f;
  if (n > 1) {
    const long first = a.row_first[(long)b * a.num_kv_heads + hq / kGqa];
    o = merge_parts(a.part_o, a.part_ml, n, d,
                    [&](int i) { return (first + i) * kGqa + hq % kGqa; });
  }
  store_row(a.out, a.out_bf16, row, d, o);
}

template <int BITS, int KAX, int VAX, bool PAGED>
hipError_t launch_t(const DecodeArgs& a, hipStream_t s) {
  dim3 grid((unsigned)(a.dev_plan ? a.plan_items : decode_grid_blocks((long)a.batch * a.num_kv_heads, a.num_splits)));
  if (a.fp8_qk) decode_kernel<BITS, KAX, VAX, PAGED, true><<<grid, kThreads, 0, s>>>(a);
  else decode_kernel<BITS, KAX, VAX, PAGED, false><<<grid, kThreads, 0, s>>>(a);
  return hipGetLastError();
}

template <int BITS, int KAX, int VAX>
hipError_t launch_p(const DecodeArgs& a, bool paged, hipStream_t s) {
  return paged ? launch_t<BITS, KAX, VAX, true>(a, s) : launch_t<BITS, KAX, VAX, false>(a, s);
}

template <int BITS>
hipError_t launch_b(const kvq_format& f, const DecodeArgs& a, hipStream_t s) {
  const bool paged = f.page_size != 0;
  if (f.k_axis == KVQ_CHANNEL_WISE) {
    if (f.v_axis == KVQ_TOKEN_WISE) return launch_p<BITS, KVQ_CHANNEL_WISE, KVQ_TOKEN_WISE>(a, paged, s);
    return launch_p<BITS, KVQ_CHANNEL_WISE, KVQ_CHANNEL_WISE>(a, paged, s);
  }
  if (f.v_axis == KVQ_TOKEN_WISE) return launch_p<BITS, KVQ_TOKEN_WISE, KVQ_TOKEN_WISE>(a, paged, s);
  return launch_p<BITS, KVQ_TOKEN_WISE, KVQ_CHANNEL_WISE>(a, paged, s);
}

}  // namespace

hipError_t launch_decode_quant(const kvq_format& f, const DecodeArgs& a, hipStream_t s) {
  if (f.group != kGroup) return launch_decode_quant_tg(f, a, s);
  return f.bits == 4 ? launch_b<4>(f, a, s) : launch_b<2>(f, a, s);
}

hipError_t launch_combine_plan(const DecodeArgs& a, hipStream_t s) {
  combine_plan_kernel<<<(unsigned)((long)a.batch * a.num_kv_heads * kGqa), kHeadDim, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_combine(const float* part_o, const float* part_ml, int rows, int num_splits,
                          void* out, int out_bf16, hipStream_t s) {
  combine_kernel<<<rows, kHeadDim, 0, s>>>(part_o, part_ml, num_splits, out, out_bf16);
  return hipGetLastError();
}

}  // namespace kvq
