/*
 * oracle.c -- plain, slow, fp64 CPU reference for single-token decode
 * attention over INT2/INT4 asymmetrically quantised KV caches.
 *
 * TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the CPU
 * baseline leg of the benchmark may load this library. It shares no code,
 * header, table or helper with the GPU library.
 *
 * What it computes (FOSCAR pages, see the citations at each function):
 *   - group-wise asymmetric quantisation x ~ s*c + z with one (s, z) per
 *     group, groups taken token-wise or channel-wise, independently for K
 *     and V (pages: grafy.ai "What is FOSCAR and how does it work?";
 *     rag-lover.com "conditions of use");
 *   - the plain definition of decode attention over the fully dequantised
 *     cache, in fp64: softmax(scale * q.K^T) . V with GQA (consecutive
 *     query heads share a KV head);
 *   - the same output through the four affine folds (token-wise K acc-fold,
 *     channel-wise K operand-fold, token-wise V operand-fold, channel-wise V
 *     acc-fold, rag-lover.com explainer; the arXiv abstract states they are
 *     exact in exact arithmetic), used only as an internal cross-check.
 *
 * Readings where the pages are silent (scale/offset derivation, fp16
 * storage, tie-breaking, the bit layout) follow the library's documented
 * format: s = fp16((max - min) / (2^b - 1)) with an fp32 division, z =
 * fp16(min), c = clamp(rint((x - z) / s), 0, 2^b - 1) in fp32 using the
 * stored fp16 s and z, c = 0 when s == 0; min and max order -0 below +0
 * (finite values).
 *
 * Packed layout, version 2 (little-endian; Lp = max_len rounded up to 128;
 * paged caches use 64-token pages and a page table). Codes live in 64-token
 * blocks (a page, or tokens 64k..64k+63 of a contiguous sequence):
 *   K codes  contiguous [B][Hkv][Lp/64][64*D*b/8] bytes, paged [P][Hkv][64*D*b/8];
 *            channel d of a token at bit b*d of its row; the row's 16-byte
 *            pieces sit 1024 bytes apart, in the token's slot (k_slot).
 *   V codes  contiguous [B][Hkv][Lp/64][(64/tpw)*D] uint32, paged
 *            [P][Hkv][(64/tpw)*D], tpw = 32/b tokens per word; token j of a
 *            word at bit b*j; word (row r, channel d) placed by v_word_idx.
 *   (s, z)   fp16 pairs, s first.
 *            token-wise:   contiguous [B][Hkv][Lp][D/G][2], paged [P][Hkv][64][D/G][2]
 *            channel-wise: contiguous [B][Hkv][Lp/G][D][2], paged [P][Hkv][D][2]
 *                          (paged: G = 128, a group's pair sits in the page
 *                          holding its first token; the other page's slot is unused;
 *                          token-wise pairs of any G sit with their token).
 *
 * parity unpinned: none of the pages prints a worked numeric example, so the
 * end-to-end output is pinned only by the tests' closed forms, brute force
 * and library cross-checks, not against numbers from the authors.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_TOKEN_WISE 0
#define ORC_CHANNEL_WISE 1

typedef struct {
  int32_t bits;         /* 2 or 4 */
  int32_t k_axis;       /* ORC_TOKEN_WISE / ORC_CHANNEL_WISE */
  int32_t v_axis;
  int32_t group;        /* G */
  int32_t head_dim;     /* D */
  int32_t num_kv_heads; /* Hkv */
  int32_t num_q_heads;  /* Hq, a multiple of Hkv */
  int32_t page_size;    /* 0 = contiguous, else 64 */
} orc_format;

/* ------------------------------------------------------------------ */
/* IEEE binary16 / bfloat16 conversions, written from the format        */
/* definitions (1 sign, 5 exponent bits with bias 15, 10 fraction bits;  */
/* bfloat16 = the top 16 bits of binary32).                              */
/* ------------------------------------------------------------------ */

/* float32 -> binary16, round to nearest, ties to even. */
uint16_t orc_f32_to_f16(float x) {
  uint32_t f;
  memcpy(&f, &x, 4);
  uint16_t sign = (uint16_t)((f >> 16) & 0x8000u);
  int32_t e = (int32_t)((f >> 23) & 0xFFu);
  uint32_t m = f & 0x7FFFFFu;
  if (e == 0xFF) return (uint16_t)(sign | (m ? 0x7E00u : 0x7C00u));
  if (e == 0 && m == 0) return sign;
  /* value = sig * 2^(exp2) with sig an integer of up to 24 bits */
  uint32_t sig = (e == 0) ? m : (m | 0x800000u);
  int32_t exp2 = (e == 0) ? -149 : e - 150;
  /* binary16 normal numbers: 11-bit significand, weight 2^(E-25) for
   * biased exponent E in 1..30; subnormals: 10-bit, weight 2^-24.
   * Find the target weight w (power of two) for this magnitude. */
  int32_t top = 31 - __builtin_clz(sig) + exp2; /* floor(log2(|x|)) */
  int32_t wexp = top - 10;                       /* unit in last place for 11-bit sig */
  if (wexp < -24) wexp = -24;                    /* subnormal range */
  /* q = sig * 2^(exp2 - wexp), rounded to nearest even */
  int32_t sh = wexp - exp2;
  uint32_t q;
  if (sh <= 0) {
    q = sig << (-sh);
  } else if (sh >= 32) {
    q = 0;
  } else {
    uint32_t keep = sig >> sh;
    uint32_t rem = sig & ((1u << sh) - 1u);
    uint32_t half = 1u << (sh - 1);
    if (rem > half || (rem == half && (keep & 1u))) keep += 1u;
    q = keep;
  }
  /* q may have grown to 2^11 after rounding: renormalise */
  if (q >= 2048u) { q >>= 1; wexp += 1; }
  if (q == 0) return sign;
  if (q < 1024u) return (uint16_t)(sign | q); /* subnormal (wexp == -24) */
  int32_t E = wexp + 25;
  if (E >= 31) return (uint16_t)(sign | 0x7C00u);
  return (uint16_t)(sign | ((uint32_t)E << 10) | (q - 1024u));
}

double orc_f16_to_f64(uint16_t h) {
  int32_t e = (h >> 10) & 0x1F;
  int32_t m = h & 0x3FF;
  double v;
  if (e == 0) v = ldexp((double)m, -24);
  else if (e == 31) v = m ? NAN : INFINITY;
  else v = ldexp((double)(m + 1024), e - 25);
  return (h & 0x8000) ? -v : v;
}

double orc_bf16_to_f64(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* ------------------------------------------------------------------ */
/* Group quantisation (pages: grafy.ai "What is FOSCAR", rag-lover.com  */
/* "conditions of use": each group shares a scale s and an offset z).   */
/* ------------------------------------------------------------------ */

/* Quantise n values x[i*stride] into codes[i*cstride]; writes s, z (fp16 bits). */
void orc_quantize_group(const float* x, long stride, int n, int bits, uint16_t* s_out,
                        uint16_t* z_out, uint8_t* codes, long cstride) {
  const int qmax = (1 << bits) - 1;
  /* min and max as a total order on the (finite) values with -0 below +0,
   * so that the stored z of a group holding both zeros does not depend on
   * the order the group is scanned in */
  float mn = x[0], mx = x[0];
  for (int i = 1; i < n; ++i) {
    float v = x[(long)i * stride];
    if (v < mn || (v == mn && signbit(v))) mn = v;
    if (v > mx || (v == mx && !signbit(v))) mx = v;
  }
  volatile float range = mx - mn;          /* fp32 subtraction */
  volatile float s32 = range / (float)qmax; /* fp32 IEEE division */
  uint16_t s16 = orc_f32_to_f16(s32);
  uint16_t z16 = orc_f32_to_f16(mn);
  float S = (float)orc_f16_to_f64(s16);
  float Z = (float)orc_f16_to_f64(z16);
  for (int i = 0; i < n; ++i) {
    int c = 0;
    if (S != 0.0f) {
      volatile float d = x[(long)i * stride] - Z; /* fp32 */
      volatile float t = d / S;                   /* fp32 IEEE division */
      float r = rintf(t);                         /* nearest, ties to even */
      if (r < 0.0f) r = 0.0f;
      if (r > (float)qmax) r = (float)qmax;
      c = (int)r;
    }
    codes[(long)i * cstride] = (uint8_t)c;
  }
  *s_out = s16;
  *z_out = z16;
}

/* ------------------------------------------------------------------ */
/* Layout: where a unit's token rows, words and (s, z) pairs live.       */
/* ------------------------------------------------------------------ */

typedef struct {
  const orc_format* f;
  const int32_t* page_table;
  int max_pages;
  int Lp; /* contiguous padded length */
} orc_layout;

static long kv_row_bytes(const orc_format* f) { return (long)f->head_dim * f->bits / 8; }
static int tpw(const orc_format* f) { return 32 / f->bits; }

/* Page/unit base for token t of (b, h): returns the index of the 64-token
 * chunk "slot" and the token offset within it. For contiguous caches the
 * unit (b, h) is treated as Lp/64 consecutive chunks. */
static long chunk_index(const orc_layout* lo, int b, int h, int t, int* tt) {
  const orc_format* f = lo->f;
  if (f->page_size == 0) {
    *tt = t % 64;
    return ((long)b * f->num_kv_heads + h) * (lo->Lp / 64) + t / 64;
  }
  int phys = lo->page_table[(long)b * lo->max_pages + t / 64];
  *tt = t % 64;
  return (long)phys * f->num_kv_heads + h;
}

/* Position of token u (0..63 within its 64-token block) among the block's
 * 16-byte K slots, layout version 2: 16*floor(u/16) + rho(u mod 16), rho
 * written out as the table the documented formula gives. */
static int k_slot(int bits, int u) {
  static const int rho4[16] = {0, 2, 4, 6, 1, 3, 5, 7, 8, 10, 12, 14, 9, 11, 13, 15};
  static const int rho2[16] = {0, 2, 4, 6, 8, 10, 12, 14, 1, 3, 5, 7, 9, 11, 13, 15};
  return 16 * (u / 16) + (bits == 4 ? rho4[u % 16] : rho2[u % 16]);
}

/* byte offset of byte o of token t's K row: the row's 16-byte pieces sit
 * 1024 bytes apart in the token's 64-token block, in the token's slot */
static long k_byte_off(const orc_layout* lo, int b, int h, int t, int o) {
  int tt;
  long c = chunk_index(lo, b, h, t, &tt);
  return c * 64 * kv_row_bytes(lo->f) + 1024L * (o / 16) + 16L * k_slot(lo->f->bits, tt) + o % 16;
}

/* uint32 word index of the V word holding token t of channel d: word-row
 * r = (t mod 64) / tpw of the block, placed at
 * 512*(r/4) + 256*((d/4) mod 2) + 64*(r mod 4) + 4*(d/8) + d mod 4 */
static long v_word_idx(const orc_layout* lo, int b, int h, int t, int d) {
  int tt;
  long c = chunk_index(lo, b, h, t, &tt);
  const int r = tt / tpw(lo->f);
  const long pos = 512L * (r / 4) + 256L * ((d / 4) % 2) + 64L * (r % 4) + 4L * (d / 8) + d % 4;
  return c * (64 / tpw(lo->f)) * lo->f->head_dim + pos;
}

/* uint16 index of the (s, z) pair (s at idx, z at idx + 1) for element (t, d) */
static long sz_idx(const orc_layout* lo, int axis, int b, int h, int t, int d) {
  const orc_format* f = lo->f;
  const int G = f->group, D = f->head_dim;
  if (axis == ORC_TOKEN_WISE) {
    int tt;
    long c = chunk_index(lo, b, h, t, &tt);
    return ((c * 64 + tt) * (D / G) + d / G) * 2;
  }
  if (f->page_size == 0) {
    long unit = (long)b * f->num_kv_heads + h;
    return ((unit * (lo->Lp / G) + t / G) * D + d) * 2;
  }
  /* paged channel-wise: pair stored in the page of the group's first token */
  int t0 = (t / G) * G;
  int tt;
  long c = chunk_index(lo, b, h, t0, &tt);
  return (c * D + d) * 2;
}

/* ------------------------------------------------------------------ */
/* Pack                                                                 */
/* ------------------------------------------------------------------ */

typedef struct {
  const orc_format* f;
  orc_layout lo;
  const float* k;
  const float* v;
  const int32_t* seq_lens;
  int max_len;
  uint8_t* k_codes;
  uint32_t* v_words;
  uint16_t* k_sz;
  uint16_t* v_sz;
  int batch;
  int next_unit;
  pthread_mutex_t mu;
} pack_job;

static void put_k_code(pack_job* J, int b, int h, int t, int d, int c) {
  const orc_format* f = J->f;
  long bit = (long)d * f->bits;
  J->k_codes[k_byte_off(&J->lo, b, h, t, (int)(bit / 8))] |= (uint8_t)(c << (bit % 8));
}

static void put_v_code(pack_job* J, int b, int h, int t, int d, int c) {
  const orc_format* f = J->f;
  long w = v_word_idx(&J->lo, b, h, t, d);
  J->v_words[w] |= (uint32_t)c << (f->bits * (t % tpw(f)));
}

/* Quantise one tensor of one unit: x is [max_len][D] fp32. */
static void pack_tensor(pack_job* J, int is_k, int b, int h, const float* x, int L) {
  const orc_format* f = J->f;
  const int D = f->head_dim, G = f->group;
  const int axis = is_k ? f->k_axis : f->v_axis;
  uint16_t* sz = is_k ? J->k_sz : J->v_sz;
  /* padded extent written by the pack: whole 128-token groups (contiguous)
   * or whole 64-token pages (paged); codes beyond L are 0. */
  int Lw = (f->page_size == 0) ? J->lo.Lp : ((L + 63) / 64) * 64;
  /* clear the codes and pairs of the written extent */
  for (int t = 0; t < Lw; ++t) {
    if (is_k) {
      for (int o = 0; o < kv_row_bytes(f); ++o) J->k_codes[k_byte_off(&J->lo, b, h, t, o)] = 0;
    } else {
      for (int d = 0; d < D; ++d) {
        long w = v_word_idx(&J->lo, b, h, t, d);
        J->v_words[w] &= ~(((1u << f->bits) - 1u) << (f->bits * (t % tpw(f))));
      }
    }
    if (axis == ORC_TOKEN_WISE) {
      for (int j = 0; j < D / G; ++j) {
        long si = sz_idx(&J->lo, axis, b, h, t, j * G);
        sz[si] = 0;
        sz[si + 1] = 0;
      }
    } else if (t % G == 0) {
      for (int d = 0; d < D; ++d) {
        long si = sz_idx(&J->lo, axis, b, h, t, d);
        sz[si] = 0;
        sz[si + 1] = 0;
      }
    }
  }
  uint8_t* codes = (uint8_t*)malloc((size_t)(L > 0 ? L : 1) * D);
  if (axis == ORC_TOKEN_WISE) {
    for (int t = 0; t < L; ++t)
      for (int j = 0; j < D / G; ++j) {
        long si = sz_idx(&J->lo, axis, b, h, t, j * G);
        orc_quantize_group(x + (long)t * D + j * G, 1, G, f->bits, &sz[si], &sz[si + 1],
                           codes + (long)t * D + j * G, 1);
      }
  } else {
    for (int t0 = 0; t0 < L; t0 += G) {
      int n = (L - t0 < G) ? (L - t0) : G;
      for (int d = 0; d < D; ++d) {
        long si = sz_idx(&J->lo, axis, b, h, t0, d);
        orc_quantize_group(x + (long)t0 * D + d, D, n, f->bits, &sz[si], &sz[si + 1],
                           codes + (long)t0 * D + d, D);
      }
    }
  }
  for (int t = 0; t < L; ++t)
    for (int d = 0; d < D; ++d) {
      int c = codes[(long)t * D + d];
      if (is_k) put_k_code(J, b, h, t, d, c);
      else put_v_code(J, b, h, t, d, c);
    }
  free(codes);
}

static void* pack_worker(void* arg) {
  pack_job* J = (pack_job*)arg;
  const orc_format* f = J->f;
  const int units = J->batch * f->num_kv_heads;
  for (;;) {
    pthread_mutex_lock(&J->mu);
    int u = J->next_unit++;
    pthread_mutex_unlock(&J->mu);
    if (u >= units) break;
    int b = u / f->num_kv_heads, h = u % f->num_kv_heads;
    int L = J->seq_lens[b];
    long base = ((long)b * f->num_kv_heads + h) * J->max_len * f->head_dim;
    pack_tensor(J, 1, b, h, J->k + base, L);
    pack_tensor(J, 0, b, h, J->v + base, L);
  }
  return NULL;
}

static int run_pool(void* (*fn)(void*), void* job, int nthreads) {
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  pthread_t th[256];
  int started = 0;
  for (int i = 1; i < nthreads; ++i)
    if (pthread_create(&th[started], NULL, fn, job) == 0) ++started;
  fn(job);
  for (int i = 0; i < started; ++i) pthread_join(th[i], NULL);
  return 0;
}

static int check_format(const orc_format* f) {
  if (f->bits != 2 && f->bits != 4) return -1;
  if (f->head_dim <= 0 || f->group <= 0 || f->num_kv_heads <= 0 || f->num_q_heads <= 0) return -1;
  if (f->num_q_heads % f->num_kv_heads) return -1;
  if (f->head_dim != 128) return -1; /* the block order of the codes is defined for D = 128 */
  if (f->k_axis == ORC_TOKEN_WISE || f->v_axis == ORC_TOKEN_WISE)
    if (f->head_dim % f->group) return -1;
  if (f->k_axis == ORC_CHANNEL_WISE || f->v_axis == ORC_CHANNEL_WISE)
    if (128 % f->group) return -1;
  /* paged: 64-token pages; a channel-wise group (G tokens) spans a page pair,
   * so G = 128 there, while token-wise pairs live with their token */
  if (f->page_size != 0) {
    if (f->page_size != 64) return -1;
    if ((f->k_axis == ORC_CHANNEL_WISE || f->v_axis == ORC_CHANNEL_WISE) && f->group != 128) return -1;
  }
  return 0;
}

/* Quantise and pack K and V ([B][Hkv][max_len][D] fp32) of every unit. */
int orc_quantize_pack(const orc_format* f, const float* k, const float* v, const int32_t* seq_lens,
                      const int32_t* page_table, int max_pages, int batch, int max_len,
                      uint8_t* k_codes, uint32_t* v_words, uint16_t* k_sz, uint16_t* v_sz,
                      int nthreads) {
  if (check_format(f)) return -1;
  pack_job J;
  memset(&J, 0, sizeof J);
  J.f = f;
  J.lo.f = f;
  J.lo.page_table = page_table;
  J.lo.max_pages = max_pages;
  J.lo.Lp = ((max_len + 127) / 128) * 128;
  J.k = k;
  J.v = v;
  J.seq_lens = seq_lens;
  J.max_len = max_len;
  J.k_codes = k_codes;
  J.v_words = v_words;
  J.k_sz = k_sz;
  J.v_sz = v_sz;
  J.batch = batch;
  pthread_mutex_init(&J.mu, NULL);
  run_pool(pack_worker, &J, nthreads);
  pthread_mutex_destroy(&J.mu);
  return 0;
}

/* ------------------------------------------------------------------ */
/* Dequantise (x^ = s*c + z, exact in fp64)                             */
/* ------------------------------------------------------------------ */

static int get_k_code(const orc_layout* lo, const uint8_t* kc, int b, int h, int t, int d) {
  long bit = (long)d * lo->f->bits;
  return (kc[k_byte_off(lo, b, h, t, (int)(bit / 8))] >> (bit % 8)) & ((1 << lo->f->bits) - 1);
}

static int get_v_code(const orc_layout* lo, const uint32_t* vw, int b, int h, int t, int d) {
  long w = v_word_idx(lo, b, h, t, d);
  return (int)((vw[w] >> (lo->f->bits * (t % tpw(lo->f)))) & ((1u << lo->f->bits) - 1u));
}

/* Fill codes [L][D], s [L][D], z [L][D] (per element, fp64) of one unit. */
static void unit_codes(const orc_layout* lo, int is_k, const void* codes, const uint16_t* sz,
                       int b, int h, int L, int* c_out, double* s_out, double* z_out) {
  const orc_format* f = lo->f;
  const int D = f->head_dim;
  const int axis = is_k ? f->k_axis : f->v_axis;
  for (int t = 0; t < L; ++t)
    for (int d = 0; d < D; ++d) {
      long i = (long)t * D + d;
      c_out[i] = is_k ? get_k_code(lo, (const uint8_t*)codes, b, h, t, d)
                      : get_v_code(lo, (const uint32_t*)codes, b, h, t, d);
      long si = sz_idx(lo, axis, b, h, t, d);
      s_out[i] = orc_f16_to_f64(sz[si]);
      z_out[i] = orc_f16_to_f64(sz[si + 1]);
    }
}

int orc_dequantize_unit(const orc_format* f, int is_k, const void* codes, const uint16_t* sz,
                        const int32_t* page_table, int max_pages, int max_len, int b, int h,
                        int L, double* out) {
  if (check_format(f)) return -1;
  orc_layout lo = {f, page_table, max_pages, ((max_len + 127) / 128) * 128};
  const int D = f->head_dim;
  int* c = (int*)malloc(sizeof(int) * (size_t)(L > 0 ? L : 1) * D);
  double* s = (double*)malloc(sizeof(double) * (size_t)(L > 0 ? L : 1) * D);
  double* z = (double*)malloc(sizeof(double) * (size_t)(L > 0 ? L : 1) * D);
  unit_codes(&lo, is_k, codes, sz, b, h, L, c, s, z);
  for (long i = 0; i < (long)L * D; ++i) out[i] = s[i] * (double)c[i] + z[i];
  free(c);
  free(s);
  free(z);
  return 0;
}

/* ------------------------------------------------------------------ */
/* Attention, plain definition, fp64                                    */
/* ------------------------------------------------------------------ */

/* q [R][D], K^ and V^ [L][D]: out[r][d] = sum_t softmax_t(scale*q_r.K^_t) V^_t[d].
 * L == 0 gives zeros. */
void orc_attention_f64(const double* q, const double* kh, const double* vh, int L, int D, int R,
                       double scale, double* out) {
  double* w = (double*)malloc(sizeof(double) * (size_t)(L > 0 ? L : 1));
  for (int r = 0; r < R; ++r) {
    double* o = out + (long)r * D;
    for (int d = 0; d < D; ++d) o[d] = 0.0;
    if (L == 0) continue;
    double m = -INFINITY;
    for (int t = 0; t < L; ++t) {
      double acc = 0.0;
      for (int d = 0; d < D; ++d) acc += q[(long)r * D + d] * kh[(long)t * D + d];
      w[t] = scale * acc;
      if (w[t] > m) m = w[t];
    }
    double l = 0.0;
    for (int t = 0; t < L; ++t) {
      w[t] = exp(w[t] - m);
      l += w[t];
    }
    for (int t = 0; t < L; ++t)
      for (int d = 0; d < D; ++d) o[d] += w[t] * vh[(long)t * D + d];
    for (int d = 0; d < D; ++d) o[d] /= l;
  }
  free(w);
}

/* ------------------------------------------------------------------ */
/* Folded attention, fp64 (oracle-internal cross-check of the algebra)  */
/* rag-lover.com explainer: QK^T contracts over channels, so token-wise */
/* K folds onto the partial product (acc-fold: scale it, add z times    */
/* the query sum) and channel-wise K folds into the query (operand-     */
/* fold); PV contracts over tokens, so token-wise V folds into P and    */
/* channel-wise V onto the partial product, applied per group (the     */
/* limits section: partial products cannot be accumulated across        */
/* quantisation-group boundaries).                                      */
/* ------------------------------------------------------------------ */

/* bug != 0 plants the mistake the pages warn about: acc-fold partials are
 * accumulated across group boundaries and scaled once (by the last group's
 * parameters). Used only to show the tests can see it. */
static void attention_folded_unit(const orc_format* f, const double* q, const int* kc,
                                  const double* ks, const double* kz, const int* vc,
                                  const double* vs, const double* vz, int L, double scale,
                                  int bug, double* out) {
  const int D = f->head_dim, G = f->group, R = f->num_q_heads / f->num_kv_heads;
  double* w = (double*)malloc(sizeof(double) * (size_t)(L > 0 ? L : 1));
  for (int r = 0; r < R; ++r) {
    const double* qr = q + (long)r * D;
    double* o = out + (long)r * D;
    for (int d = 0; d < D; ++d) o[d] = 0.0;
    if (L == 0) continue;
    double m = -INFINITY;
    for (int t = 0; t < L; ++t) {
      double S = 0.0;
      if (f->k_axis == ORC_TOKEN_WISE) {
        /* acc-fold: per channel group j, s_j * sum_{d in j} q_d c_d + z_j * sum_{d in j} q_d */
        double part = 0.0, qsum = 0.0;
        for (int d = 0; d < D; ++d) {
          long i = (long)t * D + d;
          part += qr[d] * kc[i];
          qsum += qr[d];
          if ((d + 1) % G == 0) {
            if (!bug || d + 1 == D) {
              S += ks[i] * part + kz[i] * qsum;
              part = 0.0;
              qsum = 0.0;
            }
          }
        }
      } else {
        /* operand-fold: q'_d = q_d * s_{i,d}; bias_i = sum_d q_d z_{i,d} */
        double dot = 0.0, bias = 0.0;
        for (int d = 0; d < D; ++d) {
          long i = (long)t * D + d;
          dot += (qr[d] * ks[i]) * kc[i];
          bias += qr[d] * kz[i];
        }
        S = dot + bias;
      }
      w[t] = scale * S;
      if (w[t] > m) m = w[t];
    }
    double l = 0.0;
    for (int t = 0; t < L; ++t) {
      w[t] = exp(w[t] - m);
      l += w[t];
    }
    if (f->v_axis == ORC_TOKEN_WISE) {
      /* operand-fold: P'_t = w_t * s_{t,j(d)}; offset sum_t w_t z_{t,j(d)} */
      for (int d = 0; d < D; ++d) {
        double acc = 0.0, off = 0.0;
        for (int t = 0; t < L; ++t) {
          long i = (long)t * D + d;
          acc += (w[t] * vs[i]) * vc[i];
          off += w[t] * vz[i];
        }
        o[d] = (acc + off) / l;
      }
    } else {
      /* acc-fold per token group: s_{i,d} * sum_{t in i} w_t c_{t,d} + z_{i,d} * sum_{t in i} w_t */
      for (int d = 0; d < D; ++d) {
        double acc = 0.0, part = 0.0, wsum = 0.0;
        for (int t = 0; t < L; ++t) {
          long i = (long)t * D + d;
          part += w[t] * vc[i];
          wsum += w[t];
          if ((t + 1) % G == 0 || t + 1 == L) {
            if (!bug || t + 1 == L) {
              acc += vs[i] * part + vz[i] * wsum;
              part = 0.0;
              wsum = 0.0;
            }
          }
        }
        o[d] = acc / l;
      }
    }
  }
  free(w);
}

/* ------------------------------------------------------------------ */
/* Decode attention over a packed cache (all units or a list of units)  */
/* ------------------------------------------------------------------ */

typedef struct {
  const orc_format* f;
  orc_layout lo;
  const uint16_t* q; /* bf16 bits [B][Hq][D] */
  const void* kc;
  const void* vc;
  const uint16_t* ksz;
  const uint16_t* vsz;
  const int32_t* seq_lens;
  const int32_t* units; /* (b, h) pairs or NULL */
  int n_units;
  double scale;
  double* out; /* [B][Hq][D] */
  int folded;
  int bug;
  int next;
  pthread_mutex_t mu;
} attn_job;

static void* attn_worker(void* arg) {
  attn_job* J = (attn_job*)arg;
  const orc_format* f = J->f;
  const int D = f->head_dim, R = f->num_q_heads / f->num_kv_heads;
  for (;;) {
    pthread_mutex_lock(&J->mu);
    int u = J->next++;
    pthread_mutex_unlock(&J->mu);
    if (u >= J->n_units) break;
    int b, h;
    if (J->units) {
      b = J->units[2 * u];
      h = J->units[2 * u + 1];
    } else {
      b = u / f->num_kv_heads;
      h = u % f->num_kv_heads;
    }
    int L = J->seq_lens[b];
    size_t n = (size_t)(L > 0 ? L : 1) * D;
    double* q = (double*)malloc(sizeof(double) * (size_t)R * D);
    for (int r = 0; r < R; ++r)
      for (int d = 0; d < D; ++d)
        q[(long)r * D + d] =
            orc_bf16_to_f64(J->q[((long)b * f->num_q_heads + (long)h * R + r) * D + d]);
    double* o = J->out + ((long)b * f->num_q_heads + (long)h * R) * D;
    int *kc = (int*)malloc(sizeof(int) * n), *vc = (int*)malloc(sizeof(int) * n);
    double *ks = (double*)malloc(sizeof(double) * n), *kz = (double*)malloc(sizeof(double) * n);
    double *vs = (double*)malloc(sizeof(double) * n), *vz = (double*)malloc(sizeof(double) * n);
    unit_codes(&J->lo, 1, J->kc, J->ksz, b, h, L, kc, ks, kz);
    unit_codes(&J->lo, 0, J->vc, J->vsz, b, h, L, vc, vs, vz);
    if (J->folded) {
      attention_folded_unit(f, q, kc, ks, kz, vc, vs, vz, L, J->scale, J->bug, o);
    } else {
      /* dequantise every element, then the plain definition */
      for (size_t i = 0; i < (size_t)L * D; ++i) {
        ks[i] = ks[i] * (double)kc[i] + kz[i];
        vs[i] = vs[i] * (double)vc[i] + vz[i];
      }
      orc_attention_f64(q, ks, vs, L, D, R, J->scale, o);
    }
    free(q);
    free(kc);
    free(vc);
    free(ks);
    free(kz);
    free(vs);
    free(vz);
  }
  return NULL;
}

static int run_attention(const orc_format* f, const uint16_t* q, const void* kc, const void* vc,
                         const uint16_t* ksz, const uint16_t* vsz, const int32_t* seq_lens,
                         const int32_t* page_table, int max_pages, int batch, int max_len,
                         double scale, const int32_t* units, int n_units, double* out,
                         int folded, int bug, int nthreads) {
  if (check_format(f)) return -1;
  attn_job J;
  memset(&J, 0, sizeof J);
  J.f = f;
  J.lo.f = f;
  J.lo.page_table = page_table;
  J.lo.max_pages = max_pages;
  J.lo.Lp = ((max_len + 127) / 128) * 128;
  J.q = q;
  J.kc = kc;
  J.vc = vc;
  J.ksz = ksz;
  J.vsz = vsz;
  J.seq_lens = seq_lens;
  J.units = units;
  J.n_units = units ? n_units : batch * f->num_kv_heads;
  J.scale = scale;
  J.out = out;
  J.folded = folded;
  J.bug = bug;
  pthread_mutex_init(&J.mu, NULL);
  run_pool(attn_worker, &J, nthreads);
  pthread_mutex_destroy(&J.mu);
  return 0;
}

/* Plain definition: dequantise, then softmax attention in fp64.
 * units: NULL for every (b, h), else n_units (b, h) pairs; only their
 * query heads of out are written. */
int orc_decode_attention(const orc_format* f, const uint16_t* q, const uint8_t* k_codes,
                         const uint32_t* v_words, const uint16_t* k_sz, const uint16_t* v_sz,
                         const int32_t* seq_lens, const int32_t* page_table, int max_pages,
                         int batch, int max_len, double scale, const int32_t* units, int n_units,
                         double* out, int nthreads) {
  return run_attention(f, q, k_codes, v_words, k_sz, v_sz, seq_lens, page_table, max_pages, batch,
                       max_len, scale, units, n_units, out, 0, 0, nthreads);
}

/* The same output through the four folds (fp64). */
int orc_decode_attention_folded(const orc_format* f, const uint16_t* q, const uint8_t* k_codes,
                                const uint32_t* v_words, const uint16_t* k_sz,
                                const uint16_t* v_sz, const int32_t* seq_lens,
                                const int32_t* page_table, int max_pages, int batch, int max_len,
                                double scale, int bug, double* out, int nthreads) {
  return run_attention(f, q, k_codes, v_words, k_sz, v_sz, seq_lens, page_table, max_pages, batch,
                       max_len, scale, NULL, 0, out, 1, bug, nthreads);
}

/* ------------------------------------------------------------------ */
/* Attention over an unquantised bf16 cache (for the bf16 decode path)  */
/* K, V bf16 bits: contiguous [B][Hkv][max_len][D], paged [P][Hkv][64][D]. */
/* ------------------------------------------------------------------ */

typedef struct {
  int Hkv, Hq, D, page_size, max_pages, max_len;
  const uint16_t *q, *k, *v;
  const int32_t *seq_lens, *page_table, *units;
  int n_units;
  double scale;
  double* out;
  int next;
  pthread_mutex_t mu;
} bf16_job;

static void* bf16_worker(void* arg) {
  bf16_job* J = (bf16_job*)arg;
  const int D = J->D, R = J->Hq / J->Hkv;
  for (;;) {
    pthread_mutex_lock(&J->mu);
    int u = J->next++;
    pthread_mutex_unlock(&J->mu);
    if (u >= J->n_units) break;
    int b, h;
    if (J->units) {
      b = J->units[2 * u];
      h = J->units[2 * u + 1];
    } else {
      b = u / J->Hkv;
      h = u % J->Hkv;
    }
    int L = J->seq_lens[b];
    size_t n = (size_t)(L > 0 ? L : 1) * D;
    double *kh = (double*)malloc(sizeof(double) * n), *vh = (double*)malloc(sizeof(double) * n);
    double* q = (double*)malloc(sizeof(double) * (size_t)R * D);
    for (int t = 0; t < L; ++t) {
      long row;
      if (J->page_size == 0) row = ((long)b * J->Hkv + h) * J->max_len + t;
      else row = ((long)J->page_table[(long)b * J->max_pages + t / 64] * J->Hkv + h) * 64 + t % 64;
      for (int d = 0; d < D; ++d) {
        kh[(long)t * D + d] = orc_bf16_to_f64(J->k[row * D + d]);
        vh[(long)t * D + d] = orc_bf16_to_f64(J->v[row * D + d]);
      }
    }
    for (int r = 0; r < R; ++r)
      for (int d = 0; d < D; ++d)
        q[(long)r * D + d] = orc_bf16_to_f64(J->q[((long)b * J->Hq + (long)h * R + r) * D + d]);
    orc_attention_f64(q, kh, vh, L, D, R, J->scale, J->out + ((long)b * J->Hq + (long)h * R) * D);
    free(kh);
    free(vh);
    free(q);
  }
  return NULL;
}

int orc_decode_attention_bf16(int Hkv, int Hq, int D, int page_size, const uint16_t* q,
                              const uint16_t* k, const uint16_t* v, const int32_t* seq_lens,
                              const int32_t* page_table, int max_pages, int batch, int max_len,
                              double scale, const int32_t* units, int n_units, double* out,
                              int nthreads) {
  if (Hkv <= 0 || Hq % Hkv || D <= 0) return -1;
  bf16_job J;
  memset(&J, 0, sizeof J);
  J.Hkv = Hkv;
  J.Hq = Hq;
  J.D = D;
  J.page_size = page_size;
  J.max_pages = max_pages;
  J.max_len = max_len;
  J.q = q;
  J.k = k;
  J.v = v;
  J.seq_lens = seq_lens;
  J.page_table = page_table;
  J.units = units;
  J.n_units = units ? n_units : batch * Hkv;
  J.scale = scale;
  J.out = out;
  pthread_mutex_init(&J.mu, NULL);
  run_pool(bf16_worker, &J, nthreads);
  pthread_mutex_destroy(&J.mu);
  return 0;
}
