/*
 * kvq_oracle.c - TEST INFRASTRUCTURE. A plain, slow CPU reference of the Q4 KV-cache codec and of
 * single-token decode attention over the decoded cache. It exists only to check the GPU library:
 * tests, the smoke check and the benchmark's CPU-baseline leg may load it; nothing on the product
 * path may. It shares no code, header or constant table with the GPU library; the two agree only on
 * the storage layout and arithmetic the pages define, which this file states for itself below.
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fno-fast-math -fopenmp -shared -fPIC
 *        (no FMA contraction; x86-64 SSE arithmetic, so every float operation rounds once, to nearest
 *        even).
 *
 * Pages followed (by title and section):
 *   [AMB] "Agent Memory Below the Prompt: Persistent Q4 KV Cache for Multi-Agent LLM Inference on Edge
 *         Devices", technical summary 2.1: 256-token blocks per agent; codes packed into uint32 words
 *         with one 16-bit scale and one 16-bit bias per group; the quantised cache is read directly by
 *         attention; many agents batched; an existing cache is extended rather than re-prefilled.
 *         2.2: GQA.
 *   [UQ]  UltraQuant article, technology section: Walsh-Hadamard rotation before 4-bit compression,
 *         K and V quantised with different parameters.
 *   [IKV] IntentKV article, section on invalidating instead of compacting: dropped slots point at one
 *         sentinel whose key is -1e4, so their softmax weight collapses to zero.
 *   [QKV] QKVShare explainer, methodology: bit width chosen per token.
 *
 * Readings where the pages are silent (each is listed in the design notes):
 *   affine min/max groups, bias = group minimum; parameters stored as IEEE fp16 (the pages say bf16);
 *   codes computed from the stored fp16 parameters; one correctly rounded reciprocal per group;
 *   round-half-to-even then clamp; a constant group gets scale 0 and codes 0; a zero extreme is +0;
 *   low nibble first; natural-order Hadamard, butterflies in fp32 with strides 1, 2, ..., d/2, then one
 *   multiply by fp32(1/sqrt(d)); a sentinel slot has logit -1e4 and value 0; query head j reads KV
 *   head j / G; 8-bit rows use the same formula with L = 255.
 *
 * Parity status of each entry point is stated beside it ("pinned by" = the tests that fix it against
 * something other than this file).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_OK 0
#define ORC_ERR_ARG -1
#define ORC_ERR_UNSUPPORTED -2
#define ORC_ROWS 256

/* Same field order as the library's layout struct; the oracle reads it through its own definition. */
typedef struct orc_layout {
  int32_t head_dim;
  int32_t num_kv_heads;
  int32_t block_tokens;
  int32_t k_group;
  int32_t v_group;
  int32_t rotate;
  int32_t mixed;
  int32_t format; /* 0: group-wise integer codes; 1: FP8 E4M3 per element */
  int32_t v_head_dim; /* V's head dim when it differs from K's (MLA); 0 = head_dim */
} orc_layout;

/* ---------------------------------------------------------------- fp16 <-> fp32 (IEEE binary16) */

/* fp32 -> fp16, round to nearest, ties to even, with subnormals, overflow to infinity and NaN kept.
 * Pinned by: tests/test_oracle_codec.py::test_f16_conversion_matches_numpy. */
uint16_t orc_f32_to_f16(float f) {
  uint32_t x;
  memcpy(&x, &f, 4);
  uint16_t sign = (uint16_t)((x >> 16) & 0x8000u);
  int32_t bexp = (int32_t)((x >> 23) & 0xffu);
  uint32_t man = x & 0x7fffffu;
  if (bexp == 0xff) return (uint16_t)(sign | (man ? 0x7e00u : 0x7c00u));
  if (bexp == 0) return sign; /* fp32 zero or subnormal: far below half the smallest fp16 subnormal */
  int32_t e = bexp - 127;     /* value = m * 2^(e - 23), m has 24 significant bits */
  if (e > 15) return (uint16_t)(sign | 0x7c00u);
  uint32_t m = man | 0x800000u;
  int shift = (e >= -14) ? 13 : 13 + (-14 - e); /* fp16 normal: 11-bit significand; subnormal: unit 2^-24 */
  if (shift > 25) return sign;                  /* below 2^-25: rounds to zero */
  uint32_t q = m >> shift;
  uint32_t rem = m & ((1u << shift) - 1u);
  uint32_t halfway = 1u << (shift - 1);
  if (rem > halfway || (rem == halfway && (q & 1u))) q++;
  if (e >= -14) {
    uint32_t he = (uint32_t)(e + 15);
    if (q == 0x800u) { q = 0x400u; he++; }
    if (he >= 31) return (uint16_t)(sign | 0x7c00u);
    return (uint16_t)(sign | (he << 10) | (q & 0x3ffu));
  }
  return (uint16_t)(sign | q); /* subnormal; q == 0x400 is exactly the smallest normal */
}

/* fp16 -> fp32, exact. */
float orc_f16_to_f32(uint16_t h) {
  uint32_t sign = (uint32_t)(h & 0x8000u) << 16;
  uint32_t he = (h >> 10) & 0x1fu;
  uint32_t hm = h & 0x3ffu;
  float mag;
  if (he == 0) {
    mag = ldexpf((float)hm, -24);
  } else if (he == 31) {
    uint32_t bits = 0x7f800000u | (hm << 13);
    memcpy(&mag, &bits, 4);
  } else {
    mag = ldexpf((float)(hm | 0x400u), (int)he - 25);
  }
  uint32_t b;
  memcpy(&b, &mag, 4);
  b |= sign;
  float out;
  memcpy(&out, &b, 4);
  return out;
}

/* ---------------------------------------------------------------- Walsh-Hadamard ([UQ]) */

/* Unnormalised fast Walsh-Hadamard transform in fp32, in place: for stride h = 1, 2, 4, ..., n/2 every
 * pair (x[i], x[i+h]) with (i & h) == 0 becomes (x[i] + x[i+h], x[i] - x[i+h]). Equals H x with
 * H[i][j] = (-1)^popcount(i & j). Pinned by: test_oracle_fwht.py (H H^T = n I, columns, involution,
 * explicit fp64 matrix product). */
void orc_fwht_f32(float* x, int32_t n) {
  for (int32_t h = 1; h < n; h *= 2) {
    for (int32_t i = 0; i < n; i += 2 * h) {
      for (int32_t j = i; j < i + h; ++j) {
        float a = x[j], b = x[j + h];
        x[j] = a + b;
        x[j + h] = a - b;
      }
    }
  }
}

/* The same transform in fp64 (used to undo the rotation when decoding). */
static void fwht_f64(double* x, int32_t n) {
  for (int32_t h = 1; h < n; h *= 2) {
    for (int32_t i = 0; i < n; i += 2 * h) {
      for (int32_t j = i; j < i + h; ++j) {
        double a = x[j], b = x[j + h];
        x[j] = a + b;
        x[j + h] = a - b;
      }
    }
  }
}

/* Rotation scale c = fp32(1/sqrt(n)), so that c * H is orthogonal up to the rounding of c. */
float orc_rot_scale(int32_t n) { return (float)(1.0 / sqrt((double)n)); }

/* Rotate one row: y = c * (H x), fp32. */
static void rotate_row(float* x, int32_t n) {
  float c = orc_rot_scale(n);
  orc_fwht_f32(x, n);
  for (int32_t i = 0; i < n; ++i) x[i] = x[i] * c;
}

/* ---------------------------------------------------------------- FP8 E4M3 */

/* OCP FP8 E4M3 ("fn": no infinities): sign, 4 exponent bits (bias 7), 3 mantissa bits; exponent field 0
 * holds subnormals m * 2^-9; S.1111.111 is NaN, so the largest finite magnitude is 1.75 * 2^8 = 448.
 * fp32 -> E4M3: round to nearest, ties to even, magnitudes of 448 and more saturate to 448, NaN -> 0x7F.
 * Pinned by: test_oracle_fp8.py (every code's value from the format definition, code -> value -> code,
 * ties between neighbours, saturation, torch's own E4M3 conversion inside the range). */
uint8_t orc_f32_to_e4m3(float f) {
  const uint8_t sign = signbit(f) ? 0x80u : 0u;
  double a = fabs((double)f);
  if (isnan(a)) return 0x7Fu;
  if (a >= 448.0) return (uint8_t)(sign | 0x7Eu);
  if (a < ldexp(1.0, -6)) { /* subnormal: quantum 2^-9 (a result of 8 is the smallest normal) */
    const double q = nearbyint(ldexp(a, 9));
    return (uint8_t)(sign | (uint8_t)q);
  }
  int e;
  frexp(a, &e);
  int E = e - 1; /* a in [2^E, 2^(E+1)), E in -6 .. 8 */
  double q = nearbyint(ldexp(a, 3 - E)); /* in [8, 16] */
  if (q >= 16.0) {
    q = 8.0;
    E += 1;
  }
  if (E > 8 || (E == 8 && q > 14.0)) return (uint8_t)(sign | 0x7Eu);
  return (uint8_t)(sign | (uint8_t)((E + 7) << 3) | (uint8_t)(q - 8.0));
}

/* E4M3 -> fp32, exact. */
float orc_e4m3_to_f32(uint8_t b) {
  const int e = (b >> 3) & 15, m = b & 7;
  double v;
  if (e == 15 && m == 7) return NAN;
  if (e == 0) v = ldexp((double)m, -9);
  else v = ldexp(8.0 + m, e - 10);
  return (float)((b & 0x80u) ? -v : v);
}

/* ---------------------------------------------------------------- one quantisation group */

/* Quantise the n values x[i * stride] with L = 2^bits - 1 levels ([AMB] 2.1 item 2, affine form):
 *   mn = min, mx = max (a zero extreme is taken as +0), scale = fp16(rne((mx - mn) / L)),
 *   zero = fp16(rne(mn)); s, z = the stored values; s == 0 -> all codes 0; else r = 1 / s and
 *   code = clamp(rint_even((x - z) * r), 0, L), each operation one fp32 rounding.
 * Pinned by: test_oracle_codec.py (worked tie example, grid-exact groups, constant group, error bound
 * from the stored parameters, code range). */
void orc_quantize_group(const float* x, int32_t n, int32_t stride, int32_t bits, uint8_t* codes,
                        uint16_t* scale_h, uint16_t* zero_h) {
  const int32_t L = (1 << bits) - 1;
  float mn = x[0], mx = x[0];
  for (int32_t i = 1; i < n; ++i) {
    float v = x[(size_t)i * stride];
    if (v < mn) mn = v;
    if (v > mx) mx = v;
  }
  mn = mn + 0.0f; /* a -0 extreme becomes +0 (so zero and scale are never -0); other values unchanged */
  mx = mx + 0.0f;
  float s32 = (mx - mn) / (float)L;
  *scale_h = orc_f32_to_f16(s32);
  *zero_h = orc_f32_to_f16(mn);
  float s = orc_f16_to_f32(*scale_h);
  float z = orc_f16_to_f32(*zero_h);
  if (s == 0.0f) {
    for (int32_t i = 0; i < n; ++i) codes[i] = 0;
    return;
  }
  float r = 1.0f / s;
  for (int32_t i = 0; i < n; ++i) {
    float t = x[(size_t)i * stride] - z;
    float u = t * r;
    float qv = rintf(u); /* default rounding mode: nearest, ties to even */
    if (qv < 0.0f) qv = 0.0f;
    if (qv > (float)L) qv = (float)L;
    codes[i] = (uint8_t)qv;
  }
}

/* ---------------------------------------------------------------- layout arithmetic */

static int is_pow2(int32_t v) { return v > 0 && (v & (v - 1)) == 0; }

/* V's head dim: head_dim unless the layout gives another (MLA, [AMB] 2.2: K and V dims differ). */
static int32_t vdim(const orc_layout* L) { return L->v_head_dim > 0 ? L->v_head_dim : L->head_dim; }

/* Which layouts the oracle can express: K and V head dims that are multiples of 8 (powers of two when
 * rotated), groups that are multiples of 8 dividing their tensor's head dim, 256-row blocks. */
int orc_check_layout(const orc_layout* L) {
  if (!L) return ORC_ERR_ARG;
  int32_t d = L->head_dim, dv = vdim(L);
  if (d <= 0 || d % 8 != 0 || d > 4096) return ORC_ERR_ARG;
  if (L->v_head_dim < 0 || dv % 8 != 0 || dv > 4096) return ORC_ERR_ARG;
  if (L->num_kv_heads <= 0 || L->block_tokens != ORC_ROWS) return ORC_ERR_ARG;
  if (L->format == 1) { /* FP8: one byte per element, no groups, no per-token widths */
    if (L->k_group != 0 || L->v_group != 0 || L->mixed != 0) return ORC_ERR_ARG;
    if (L->rotate != 0 && L->rotate != 1) return ORC_ERR_ARG;
    if (L->rotate && !(is_pow2(d) && is_pow2(dv))) return ORC_ERR_UNSUPPORTED;
    return ORC_OK;
  }
  if (L->format != 0) return ORC_ERR_ARG;
  if (!(L->k_group == -1 || (L->k_group > 0 && L->k_group % 8 == 0 && d % L->k_group == 0)))
    return ORC_ERR_ARG;
  if (!(L->v_group > 0 && L->v_group % 8 == 0 && dv % L->v_group == 0)) return ORC_ERR_ARG;
  if (L->rotate != 0 && L->rotate != 1) return ORC_ERR_ARG;
  if (L->mixed < 0 || L->mixed > 2) return ORC_ERR_ARG;
  if (L->rotate && !(is_pow2(d) && is_pow2(dv))) return ORC_ERR_UNSUPPORTED;
  if (L->mixed && L->k_group < 0) return ORC_ERR_UNSUPPORTED;
  return ORC_OK;
}

/* Tile layout (one block of 256 rows, one KV head; d = K's head dim, dv = V's):
 *   row records       256 x rec bytes (rec = (d + dv) * w / 8, w the widest width the pool allows):
 *                     record t holds the row's K codes (d * b / 8 bytes, b its width) immediately followed
 *                     by its V codes (dv * b / 8 bytes); the rest of a narrower row's record is zero;
 *   per-channel K     K grouped per channel: d x {fp16 scale, fp16 zero};
 *   parameter records 256 x prow bytes: record t holds K params [group] {scale, zero} (per-token K
 *                     groups only) then V params [group] {scale, zero};
 *   header            mixed pools: 8 uint32 words, bit t % 32 of word t / 32 set = row t is 8-bit;
 *   zero padding to a multiple of 256 bytes.
 * The pages fix only the content (codes and a 16-bit scale and bias per group); this arrangement keeps a
 * row's K and V codes in one record so a row is one contiguous read. */
/* Bytes of one row record: K and V at the widest width the pool allows (FP16 in pools with widths
 * {2, 4, 8, FP16}, 8 bits in 4/8-bit pools and FP8 pools, else 4 bits). */
static size_t row_rec_bytes(const orc_layout* L) {
  const int32_t wmax = L->mixed == 2 ? 16 : ((L->mixed || L->format == 1) ? 8 : 4);
  return (size_t)(L->head_dim + vdim(L)) * wmax / 8;
}
/* Header bytes: mixed 1 = one width bit per row; mixed 2 = a 2-bit width code per row. */
static size_t header_bytes(const orc_layout* L) { return L->mixed == 2 ? 64 : (L->mixed ? 32 : 0); }
static size_t kcodes_off(const orc_layout* L, int32_t t) { return (size_t)t * row_rec_bytes(L); }
static size_t vcodes_off(const orc_layout* L, int32_t t, int32_t bits) {
  return kcodes_off(L, t) + (size_t)L->head_dim * bits / 8;
}
static size_t off_params(const orc_layout* L) { return (size_t)ORC_ROWS * row_rec_bytes(L); }
static size_t kparams_per_row(const orc_layout* L) { return L->k_group > 0 ? (size_t)(L->head_dim / L->k_group) : 0; }
static size_t prow_bytes(const orc_layout* L) {
  if (L->format == 1) return 0;
  return (kparams_per_row(L) + (size_t)(vdim(L) / L->v_group)) * 4;
}
static size_t off_prows(const orc_layout* L) {
  return off_params(L) + ((L->k_group > 0 || L->format == 1) ? 0 : (size_t)L->head_dim * 4);
}
static size_t kparams_off(const orc_layout* L, int32_t t) { return off_prows(L) + (size_t)t * prow_bytes(L); }
static size_t vparams_off(const orc_layout* L, int32_t t) { return kparams_off(L, t) + kparams_per_row(L) * 4; }
static size_t kchan_off(const orc_layout* L, int32_t c) { return off_params(L) + (size_t)c * 4; }
static size_t off_header(const orc_layout* L) { return off_prows(L) + (size_t)ORC_ROWS * prow_bytes(L); }

size_t orc_tile_bytes(const orc_layout* L) {
  if (orc_check_layout(L) != ORC_OK) return 0;
  size_t end = off_header(L) + header_bytes(L);
  return (end + 255) / 256 * 256;
}

static uint8_t* tile_ptr(const orc_layout* L, uint8_t* pool, int64_t block, int32_t head) {
  return pool + ((size_t)block * L->num_kv_heads + head) * orc_tile_bytes(L);
}

static void put_u16(uint8_t* p, uint16_t v) { p[0] = (uint8_t)(v & 0xff); p[1] = (uint8_t)(v >> 8); }
static uint16_t get_u16(const uint8_t* p) { return (uint16_t)(p[0] | (p[1] << 8)); }

/* Pack one row's codes (d * bits / 8 bytes): 4-bit rows two per byte, low nibble first; 8-bit rows one
 * per byte; 2-bit rows four per byte, lowest bits first. */
static void pack_row(const uint8_t* codes, int32_t d, int32_t bits, uint8_t* dst) {
  memset(dst, 0, (size_t)d * bits / 8);
  if (bits == 8) {
    for (int32_t j = 0; j < d; ++j) dst[j] = codes[j];
  } else if (bits == 4) {
    for (int32_t j = 0; j < d; ++j) dst[j / 2] |= (uint8_t)((codes[j] & 0xf) << (4 * (j % 2)));
  } else {
    for (int32_t j = 0; j < d; ++j) dst[j / 4] |= (uint8_t)((codes[j] & 0x3) << (2 * (j % 4)));
  }
}

static uint8_t unpack_code(const uint8_t* row, int32_t j, int32_t bits) {
  if (bits == 8) return row[j];
  if (bits == 2) return (uint8_t)((row[j / 4] >> (2 * (j % 4))) & 0x3);
  return (uint8_t)((row[j / 2] >> (4 * (j % 2))) & 0xf);
}

/* Quantise one token row (already fp32 and, if requested, rotated) with per-token groups of g. */
static void quantize_row_groups(const float* x, int32_t d, int32_t g, int32_t bits, uint8_t* code_dst,
                                uint8_t* param_dst) {
  uint8_t codes[4096];
  for (int32_t k = 0; k < d / g; ++k) {
    uint16_t sh, zh;
    orc_quantize_group(x + (size_t)k * g, g, 1, bits, codes + (size_t)k * g, &sh, &zh);
    put_u16(param_dst + 4 * k, sh);
    put_u16(param_dst + 4 * k + 2, zh);
  }
  pack_row(codes, d, bits, code_dst);
}

/* Width of row t from the caller's width words: mixed 1 = bit t % 32 of word t / 32 (set = 8-bit, else
 * 4-bit); mixed 2 = the 2-bit code at bits 2 (t % 16) of word t / 16 (0, 1, 2, 3 = 2, 4, 8, 16 bits; 4 bits
 * without words). */
static int row_bits(const orc_layout* L, const uint32_t* bitmap, int32_t t) {
  if (L->mixed == 2) {
    const uint32_t c = bitmap ? (bitmap[t / 16] >> (2 * (t % 16))) & 3u : 1u;
    return 2 << c;
  }
  return (bitmap && ((bitmap[t / 32] >> (t % 32)) & 1u)) ? 8 : 4;
}
/* A row stored at FP16 width: the (rotated) fp32 values rounded to fp16, no parameters. */
static void store_f16_row(const float* x, int32_t d, uint8_t* dst) {
  for (int32_t c = 0; c < d; ++c) put_u16(dst + 2 * c, orc_f32_to_f16(x[c]));
}

/* Quantise one tile from its 256 fp16 rows: row t of K at k_rows + t * k_stride (d values), of V at
 * v_rows + t * v_stride (dv values). */
static void quantize_tile(const orc_layout* L, uint8_t* tile, const uint16_t* k_rows, size_t k_stride,
                          const uint16_t* v_rows, size_t v_stride, const uint32_t* bitmap) {
  const int32_t d = L->head_dim, dv = vdim(L);
  memset(tile, 0, orc_tile_bytes(L));
  float* xk = (float*)malloc(sizeof(float) * ORC_ROWS * d);
  float* xv = (float*)malloc(sizeof(float) * ORC_ROWS * dv);
  for (int32_t t = 0; t < ORC_ROWS; ++t) {
    for (int32_t c = 0; c < d; ++c) xk[(size_t)t * d + c] = orc_f16_to_f32(k_rows[(size_t)t * k_stride + c]);
    for (int32_t c = 0; c < dv; ++c) xv[(size_t)t * dv + c] = orc_f16_to_f32(v_rows[(size_t)t * v_stride + c]);
    if (L->rotate) {
      rotate_row(xk + (size_t)t * d, d);
      rotate_row(xv + (size_t)t * dv, dv);
    }
  }
  if (L->format == 1) { /* FP8: K bytes then V bytes of each row record */
    for (int32_t t = 0; t < ORC_ROWS; ++t) {
      uint8_t* rec = tile + kcodes_off(L, t);
      for (int32_t c = 0; c < d; ++c) rec[c] = orc_f32_to_e4m3(xk[(size_t)t * d + c]);
      for (int32_t c = 0; c < dv; ++c) rec[d + c] = orc_f32_to_e4m3(xv[(size_t)t * dv + c]);
    }
    free(xk);
    free(xv);
    return;
  }
  /* K */
  if (L->k_group > 0) {
    for (int32_t t = 0; t < ORC_ROWS; ++t) {
      const int32_t b = row_bits(L, bitmap, t);
      if (b == 16)
        store_f16_row(xk + (size_t)t * d, d, tile + kcodes_off(L, t));
      else
        quantize_row_groups(xk + (size_t)t * d, d, L->k_group, b, tile + kcodes_off(L, t), tile + kparams_off(L, t));
    }
  } else {
    /* one group per channel over the 256 rows of the block; always 4-bit (mixed is rejected) */
    uint8_t* codes = (uint8_t*)malloc((size_t)ORC_ROWS * d);
    uint8_t col[ORC_ROWS];
    for (int32_t c = 0; c < d; ++c) {
      uint16_t sh, zh;
      orc_quantize_group(xk + c, ORC_ROWS, d, 4, col, &sh, &zh);
      for (int32_t t = 0; t < ORC_ROWS; ++t) codes[(size_t)t * d + c] = col[t];
      put_u16(tile + kchan_off(L, c), sh);
      put_u16(tile + kchan_off(L, c) + 2, zh);
    }
    for (int32_t t = 0; t < ORC_ROWS; ++t) pack_row(codes + (size_t)t * d, d, 4, tile + kcodes_off(L, t));
    free(codes);
  }
  /* V */
  for (int32_t t = 0; t < ORC_ROWS; ++t) {
    const int32_t b = row_bits(L, bitmap, t);
    if (b == 16)
      store_f16_row(xv + (size_t)t * dv, dv, tile + vcodes_off(L, t, b));
    else
      quantize_row_groups(xv + (size_t)t * dv, dv, L->v_group, b, tile + vcodes_off(L, t, b), tile + vparams_off(L, t));
  }
  if (L->mixed) {
    uint8_t* hdr = tile + off_header(L);
    for (int32_t w = 0; w < (int32_t)header_bytes(L) / 4; ++w) {
      /* without width words every row is 4-bit: code 1 in each 2-bit field of a mixed-2 header */
      uint32_t word = bitmap ? bitmap[w] : (L->mixed == 2 ? 0x55555555u : 0u);
      for (int32_t b = 0; b < 4; ++b) hdr[4 * w + b] = (uint8_t)((word >> (8 * b)) & 0xff);
    }
  }
  free(xk);
  free(xv);
}

/* Host-memory counterpart of kvq_quantize_blocks: same argument meaning, every pointer on the host.
 * Pinned by: the group pins above plus test_oracle_codec.py layout tests (byte positions of codes,
 * params and header checked against hand-built tiles). */
int orc_quantize_blocks(const orc_layout* L, uint8_t* pool, const int32_t* block_ids, int32_t n_blocks,
                        const uint16_t* k, const uint16_t* v, const uint32_t* prec_bits) {
  int st = orc_check_layout(L);
  if (st != ORC_OK) return st;
  if (n_blocks < 0) return ORC_ERR_ARG;
  if (prec_bits && !L->mixed) return ORC_ERR_ARG;
  const int32_t H = L->num_kv_heads, d = L->head_dim, dv = vdim(L);
  /* tiles are independent (block ids are distinct): one (block, head) tile per iteration, in any order */
#pragma omp parallel for collapse(2) schedule(dynamic, 4)
  for (int32_t i = 0; i < n_blocks; ++i) {
    for (int32_t h = 0; h < H; ++h) {
      const size_t row0 = (size_t)i * ORC_ROWS * H + h;
      quantize_tile(L, tile_ptr(L, pool, block_ids[i], h), k + row0 * d, (size_t)H * d, v + row0 * dv, (size_t)H * dv,
                    prec_bits ? prec_bits + (size_t)i * (header_bytes(L) / 4) : NULL);
    }
  }
  return ORC_OK;
}

/* Host-memory counterpart of kvq_append_tokens. prec[s] is the row's width: 8 in a mixed pool, 2, 8 or 16
 * in a mixed-2 pool; any other value (or no prec) stores a 4-bit row. Pinned by: test_oracle_codec.py and
 * test_oracle_widths.py (an appended row equals the same row inside a whole quantised block). */
int orc_append_tokens(const orc_layout* L, uint8_t* pool, int32_t n_seqs, const uint16_t* k,
                      const uint16_t* v, const int32_t* block_table, int32_t max_blocks_per_seq,
                      const int32_t* positions, const uint8_t* prec) {
  int st = orc_check_layout(L);
  if (st != ORC_OK) return st;
  if (L->k_group < 0) return ORC_ERR_UNSUPPORTED;
  if (n_seqs < 0 || max_blocks_per_seq <= 0) return ORC_ERR_ARG;
  if (prec && !L->mixed) return ORC_ERR_ARG;
  const int32_t H = L->num_kv_heads, d = L->head_dim, dv = vdim(L);
  const size_t rec_bytes = row_rec_bytes(L);
  float x[4096];
  for (int32_t s = 0; s < n_seqs; ++s) {
    int32_t p = positions[s];
    int32_t blk = block_table[(size_t)s * max_blocks_per_seq + p / ORC_ROWS];
    int32_t row = p % ORC_ROWS;
    int32_t bits = (prec && prec[s] == 8) ? 8 : 4;
    if (L->mixed == 2 && prec && (prec[s] == 2 || prec[s] == 16)) bits = prec[s]; /* any other value: 4 */
    for (int32_t h = 0; h < H; ++h) {
      uint8_t* tile = tile_ptr(L, pool, blk, h);
      memset(tile + kcodes_off(L, row), 0, rec_bytes); /* the whole record: a wider row may have been here */
      for (int32_t which = 0; which < 2; ++which) {
        const int32_t n = which == 0 ? d : dv;
        const uint16_t* src = which == 0 ? k + ((size_t)s * H + h) * d : v + ((size_t)s * H + h) * dv;
        for (int32_t c = 0; c < n; ++c) x[c] = orc_f16_to_f32(src[c]);
        if (L->rotate) rotate_row(x, n);
        if (L->format == 1) {
          uint8_t* rec = tile + kcodes_off(L, row) + (size_t)which * d;
          for (int32_t c = 0; c < n; ++c) rec[c] = orc_f32_to_e4m3(x[c]);
          continue;
        }
        int32_t g = which == 0 ? L->k_group : L->v_group;
        size_t code_off = which == 0 ? kcodes_off(L, row) : vcodes_off(L, row, bits);
        size_t par_off = which == 0 ? kparams_off(L, row) : vparams_off(L, row);
        if (bits == 16) {
          store_f16_row(x, n, tile + code_off);
          memset(tile + par_off, 0, (size_t)(n / g) * 4); /* an FP16 row has no parameters */
        } else {
          quantize_row_groups(x, n, g, bits, tile + code_off, tile + par_off);
        }
      }
      if (L->mixed == 1) {
        uint8_t* byte = tile + off_header(L) + row / 8;
        if (bits == 8) *byte |= (uint8_t)(1u << (row % 8));
        else *byte &= (uint8_t)~(1u << (row % 8));
      } else if (L->mixed == 2) {
        uint8_t* byte = tile + off_header(L) + row / 4;
        const uint32_t code = bits == 2 ? 0u : bits == 4 ? 1u : bits == 8 ? 2u : 3u;
        *byte = (uint8_t)((*byte & ~(3u << (2 * (row % 4)))) | (code << (2 * (row % 4))));
      }
    }
  }
  return ORC_OK;
}

/* ---------------------------------------------------------------- decoding */

/* Dequantise row t of one tile into fp64 (rotated domain, no inverse rotation): k_out[d], v_out[dv]:
 * value = code * scale + zero, exact in fp64. Returns the row's bit width. */
int32_t orc_dequant_row(const orc_layout* L, const uint8_t* tile, int32_t t, double* k_out, double* v_out) {
  const int32_t d = L->head_dim, dv = vdim(L);
  if (L->format == 1) {
    const uint8_t* rec = tile + kcodes_off(L, t);
    for (int32_t c = 0; c < d; ++c) k_out[c] = (double)orc_e4m3_to_f32(rec[c]);
    for (int32_t c = 0; c < dv; ++c) v_out[c] = (double)orc_e4m3_to_f32(rec[d + c]);
    return 8;
  }
  int32_t bits = 4;
  if (L->mixed == 1) bits = ((tile[off_header(L) + t / 8] >> (t % 8)) & 1u) ? 8 : 4;
  if (L->mixed == 2) bits = 2 << ((tile[off_header(L) + t / 4] >> (2 * (t % 4))) & 3u);
  const uint8_t* kr = tile + kcodes_off(L, t);
  const uint8_t* vr = tile + vcodes_off(L, t, bits);
  if (bits == 16) {
    for (int32_t c = 0; c < d; ++c) k_out[c] = (double)orc_f16_to_f32(get_u16(kr + 2 * c));
    for (int32_t c = 0; c < dv; ++c) v_out[c] = (double)orc_f16_to_f32(get_u16(vr + 2 * c));
    return bits;
  }
  for (int32_t c = 0; c < d; ++c) {
    const uint8_t* kp = L->k_group > 0 ? tile + kparams_off(L, t) + (size_t)(c / L->k_group) * 4
                                       : tile + kchan_off(L, c);
    k_out[c] = (double)unpack_code(kr, c, bits) * (double)orc_f16_to_f32(get_u16(kp)) +
               (double)orc_f16_to_f32(get_u16(kp + 2));
  }
  for (int32_t c = 0; c < dv; ++c) {
    const uint8_t* vp = tile + vparams_off(L, t) + (size_t)(c / L->v_group) * 4;
    v_out[c] = (double)unpack_code(vr, c, bits) * (double)orc_f16_to_f32(get_u16(vp)) +
               (double)orc_f16_to_f32(get_u16(vp + 2));
  }
  return bits;
}

/* fp64 -> IEEE binary16 bits, one rounding to nearest, ties to even (overflow to infinity). */
static uint16_t f64_to_f16(double x) {
  const uint16_t sign = signbit(x) ? 0x8000u : 0u;
  double a = fabs(x);
  if (isnan(a)) return 0x7e00u;
  if (a >= 65520.0) return (uint16_t)(sign | 0x7c00u); /* at or above max + half an ulp */
  if (a < ldexp(1.0, -14)) {                            /* subnormal range: quantum 2^-24 */
    const double q = nearbyint(ldexp(a, 24));          /* may reach 1024, the smallest normal */
    return (uint16_t)(sign | (uint16_t)q);
  }
  int e;
  frexp(a, &e); /* a in [2^(e-1), 2^e) */
  int E = e - 1;
  double q = nearbyint(ldexp(a, 10 - E)); /* in [1024, 2048] */
  if (q >= 2048.0) {
    q = 1024.0;
    E += 1;
  }
  if (E > 15) return (uint16_t)(sign | 0x7c00u);
  return (uint16_t)(sign | (uint16_t)((E + 15) << 10) | (uint16_t)(q - 1024.0));
}

/* The cache restored as fp16 rows ([QKV] methodology section, injection path: the quantised cache
 * rebuilt as fp16 key/value tensors before the forward pass). For every listed block b = block_ids[i],
 * KV head h and row t: the row's K and V are dequantised exactly (orc_dequant_row), un-rotated for a
 * rotated pool by (1 / (n c)) H in fp64 (the exact inverse of the rotation c H at length n = d or dv), and
 * rounded once to fp16. Output layout is the input layout of orc_quantize_blocks: k_out [n_blocks * 256][H][d],
 * v_out [n_blocks * 256][H][dv].
 * Pinned by: test_oracle_dequant.py (grid-exact blocks restored bit for bit, the per-element error bound
 * of the stored scales carried through the rotation, an explicit Hadamard matrix for the inverse). */
int orc_dequantize_blocks(const orc_layout* L, const uint8_t* pool, const int32_t* block_ids, int32_t n_blocks,
                          uint16_t* k_out, uint16_t* v_out) {
  int st = orc_check_layout(L);
  if (st != ORC_OK) return st;
  if (n_blocks < 0) return ORC_ERR_ARG;
  const int32_t H = L->num_kv_heads, d = L->head_dim, dv = vdim(L);
  const double unrot_k = 1.0 / ((double)d * (double)orc_rot_scale(d));
  const double unrot_v = 1.0 / ((double)dv * (double)orc_rot_scale(dv));
  double* k = (double*)malloc(sizeof(double) * ((size_t)d + (size_t)dv));
  if (!k) return ORC_ERR_ARG;
  double* v = k + d;
  for (int32_t i = 0; i < n_blocks; ++i) {
    for (int32_t h = 0; h < H; ++h) {
      const uint8_t* tile = tile_ptr(L, (uint8_t*)pool, block_ids[i], h);
      for (int32_t t = 0; t < ORC_ROWS; ++t) {
        orc_dequant_row(L, tile, t, k, v);
        if (L->rotate) {
          fwht_f64(k, d);
          fwht_f64(v, dv);
          for (int32_t c = 0; c < d; ++c) k[c] *= unrot_k;
          for (int32_t c = 0; c < dv; ++c) v[c] *= unrot_v;
        }
        const size_t row = ((size_t)i * ORC_ROWS + t) * H + h;
        for (int32_t c = 0; c < d; ++c) k_out[row * d + c] = f64_to_f16(k[c]);
        for (int32_t c = 0; c < dv; ++c) v_out[row * dv + c] = f64_to_f16(v[c]);
      }
    }
  }
  free(k);
  return ORC_OK;
}

/* Host-memory counterpart of kvq_decode_attention, in fp64, by the plain definition:
 *   for sequence s and query head j (KV head h = j / G): for every slot t < seq_lens[s], a sentinel
 *   slot has logit -1e4 and value 0; any other slot's K and V rows are dequantised exactly (and, for a
 *   rotated pool, un-rotated by (1 / (n c)) H, the exact inverse of c H at length n = d or dv),
 *   logit = scale * (q . k); out = sum_t softmax(logits)_t * v_t. A sequence with no slot gives 0.
 *   q is [n_seqs][num_q_heads][d], out [n_seqs][num_q_heads][dv].
 * weights (optional, may be NULL): fp64 [n_seqs][num_q_heads][max_seq_len] softmax weights.
 * n_threads > 0 sets the OpenMP thread count (one (s, h) pair per iteration).
 * Pinned by: test_oracle_attention.py (numpy dense brute force with an explicit Hadamard matrix,
 * seq_len 1, equal keys, G = 1, all-sentinel, sentinel weight). */
int orc_decode_attention(const orc_layout* L, const uint8_t* pool, const uint16_t* q, int32_t n_seqs,
                         int32_t num_q_heads, const int32_t* block_table, int32_t max_blocks_per_seq,
                         const int32_t* seq_lens, const uint32_t* sentinel_mask,
                         int32_t mask_words_per_seq, float softmax_scale, double* out, double* weights,
                         int32_t max_seq_len, int32_t n_threads) {
  int st = orc_check_layout(L);
  if (st != ORC_OK) return st;
  const int32_t H = L->num_kv_heads, d = L->head_dim, dv = vdim(L);
  if (n_seqs < 0 || num_q_heads <= 0 || num_q_heads % H != 0) return ORC_ERR_ARG;
  const int32_t G = num_q_heads / H;
  const double unrot_k = 1.0 / ((double)d * (double)orc_rot_scale(d));
  const double unrot_v = 1.0 / ((double)dv * (double)orc_rot_scale(dv));
#ifdef _OPENMP
  if (n_threads > 0) omp_set_num_threads(n_threads);
#pragma omp parallel for schedule(dynamic, 1)
#endif
  for (int64_t sh = 0; sh < (int64_t)n_seqs * H; ++sh) {
    const int32_t s = (int32_t)(sh / H), h = (int32_t)(sh % H);
    const int32_t n = seq_lens[s];
    if (n <= 0) {
      for (int32_t jj = 0; jj < G; ++jj)
        for (int32_t c = 0; c < dv; ++c) out[((size_t)s * num_q_heads + h * G + jj) * dv + c] = 0.0;
      continue;
    }
    double* kt = (double*)malloc(sizeof(double) * (size_t)n * d);
    double* vt = (double*)malloc(sizeof(double) * (size_t)n * dv);
    char* sent = (char*)malloc((size_t)n);
    for (int32_t t = 0; t < n; ++t) {
      sent[t] = sentinel_mask && ((sentinel_mask[(size_t)s * mask_words_per_seq + t / 32] >> (t % 32)) & 1u);
      if (sent[t]) {
        for (int32_t c = 0; c < d; ++c) kt[(size_t)t * d + c] = 0.0;
        for (int32_t c = 0; c < dv; ++c) vt[(size_t)t * dv + c] = 0.0;
        continue;
      }
      int32_t blk = block_table[(size_t)s * max_blocks_per_seq + t / ORC_ROWS];
      const uint8_t* tile = pool + ((size_t)blk * H + h) * orc_tile_bytes(L);
      orc_dequant_row(L, tile, t % ORC_ROWS, kt + (size_t)t * d, vt + (size_t)t * dv);
      if (L->rotate) {
        fwht_f64(kt + (size_t)t * d, d);
        fwht_f64(vt + (size_t)t * dv, dv);
        for (int32_t c = 0; c < d; ++c) kt[(size_t)t * d + c] *= unrot_k;
        for (int32_t c = 0; c < dv; ++c) vt[(size_t)t * dv + c] *= unrot_v;
      }
    }
    double* logit = (double*)malloc(sizeof(double) * (size_t)n);
    for (int32_t jj = 0; jj < G; ++jj) {
      const int32_t j = h * G + jj;
      const uint16_t* qj = q + ((size_t)s * num_q_heads + j) * d;
      double m = -INFINITY;
      for (int32_t t = 0; t < n; ++t) {
        if (sent[t]) {
          logit[t] = -1e4;
        } else {
          double dot = 0.0;
          for (int32_t c = 0; c < d; ++c) dot += (double)orc_f16_to_f32(qj[c]) * kt[(size_t)t * d + c];
          logit[t] = (double)softmax_scale * dot;
        }
        if (logit[t] > m) m = logit[t];
      }
      double denom = 0.0;
      for (int32_t t = 0; t < n; ++t) denom += exp(logit[t] - m);
      double* o = out + ((size_t)s * num_q_heads + j) * dv;
      for (int32_t c = 0; c < dv; ++c) o[c] = 0.0;
      for (int32_t t = 0; t < n; ++t) {
        double w = exp(logit[t] - m) / denom;
        if (weights) weights[((size_t)s * num_q_heads + j) * max_seq_len + t] = w;
        for (int32_t c = 0; c < dv; ++c) o[c] += w * vt[(size_t)t * dv + c];
      }
    }
    free(logit);
    free(kt);
    free(vt);
    free(sent);
  }
  return ORC_OK;
}

/* Threads of the parallel loops that take no thread count (quantisation); 0 keeps OpenMP's default. */
void orc_set_threads(int32_t n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

/* Threads the OpenMP runtime will use for a parallel region (1 without OpenMP). */
int32_t orc_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
