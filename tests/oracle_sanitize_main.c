/* Host driver for the sanitizer build of the CPU oracle (tests/test_oracle_sanitizers.py): every oracle entry
 * point on small pools of several layouts - per-token and per-channel K groups, rotation, 4/8-bit and
 * {2, 4, 8, FP16} widths, FP8, unequal K/V head dims - with ragged lengths (0, 1, a partial block, several
 * blocks), sentinel masks and appends at block boundaries. Built with AddressSanitizer and
 * UndefinedBehaviorSanitizer; any out-of-bounds access, leak or undefined operation ends the run with an
 * error. The values are arbitrary (an LCG); nothing here is compared with anything. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

typedef struct orc_layout {
  int32_t head_dim, num_kv_heads, block_tokens, k_group, v_group, rotate, mixed, format, v_head_dim;
} orc_layout;

uint16_t orc_f32_to_f16(float f);
size_t orc_tile_bytes(const orc_layout* L);
int orc_check_layout(const orc_layout* L);
int orc_quantize_blocks(const orc_layout* L, uint8_t* pool, const int32_t* block_ids, int32_t n_blocks,
                        const uint16_t* k, const uint16_t* v, const uint32_t* prec_bits);
int orc_append_tokens(const orc_layout* L, uint8_t* pool, int32_t n_seqs, const uint16_t* k, const uint16_t* v,
                      const int32_t* block_table, int32_t max_blocks_per_seq, const int32_t* positions,
                      const uint8_t* prec);
int32_t orc_dequant_row(const orc_layout* L, const uint8_t* tile, int32_t t, double* k_out, double* v_out);
int orc_dequantize_blocks(const orc_layout* L, const uint8_t* pool, const int32_t* block_ids, int32_t n_blocks,
                          uint16_t* k_out, uint16_t* v_out);
int orc_decode_attention(const orc_layout* L, const uint8_t* pool, const uint16_t* q, int32_t n_seqs,
                         int32_t num_q_heads, const int32_t* block_table, int32_t max_blocks_per_seq,
                         const int32_t* seq_lens, const uint32_t* sentinel_mask, int32_t mask_words_per_seq,
                         float softmax_scale, double* out, double* weights, int32_t max_seq_len, int32_t n_threads);

static uint32_t lcg_state = 12345u;
static uint32_t lcg(void) {
  lcg_state = lcg_state * 1664525u + 1013904223u;
  return lcg_state >> 8;
}
static float uniform(float lo, float hi) { return lo + (hi - lo) * (float)(lcg() & 0xFFFF) / 65535.0f; }

static void fill_f16(uint16_t* x, size_t n, float scale) {
  for (size_t i = 0; i < n; ++i) x[i] = orc_f32_to_f16(uniform(-scale, scale));
}

#define CHECK(cond)                                                   \
  do {                                                                \
    if (!(cond)) {                                                    \
      fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
      exit(2);                                                        \
    }                                                                 \
  } while (0)

static void run_layout(orc_layout L, int G) {
  const int H = L.num_kv_heads, d = L.head_dim, dv = L.v_head_dim ? L.v_head_dim : L.head_dim;
  CHECK(orc_check_layout(&L) == 0);
  const size_t tb = orc_tile_bytes(&L);
  const int n_blocks = 5, n_seqs = 4, maxb = 3;
  uint8_t* pool = (uint8_t*)calloc((size_t)n_blocks * H * tb, 1);
  uint16_t* k = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)4 * 256 * H * d);
  uint16_t* v = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)4 * 256 * H * dv);
  fill_f16(k, (size_t)4 * 256 * H * d, 6.0f);
  fill_f16(v, (size_t)4 * 256 * H * dv, 2.0f);
  const int32_t ids[4] = {3, 0, 4, 1};
  uint32_t* bits = NULL;
  if (L.mixed) {
    const int W = L.mixed == 2 ? 16 : 8;
    bits = (uint32_t*)malloc(sizeof(uint32_t) * 4 * W);
    for (int i = 0; i < 4 * W; ++i) bits[i] = lcg() ^ (lcg() << 16);
  }
  CHECK(orc_quantize_blocks(&L, pool, ids, 4, k, v, bits) == 0);
  /* sequences: lengths 0, 1, 300, 700 after one appended token each (positions at and past block ends) */
  const int32_t table[4 * 3] = {2, 0, 0, 2, 0, 0, 3, 2, 0, 0, 1, 2};
  const int32_t pos[4] = {0, 0, 299, 699};
  const int32_t lens[4] = {0, 1, 300, 700};
  uint8_t prec[4] = {2, 8, 16, 4};
  uint16_t* ak = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)n_seqs * H * d);
  uint16_t* av = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)n_seqs * H * dv);
  fill_f16(ak, (size_t)n_seqs * H * d, 6.0f);
  fill_f16(av, (size_t)n_seqs * H * dv, 2.0f);
  if (L.k_group > 0) {
    /* sequence 0 appends nothing (its length stays 0): append the other three */
    CHECK(orc_append_tokens(&L, pool, 3, ak + (size_t)H * d, av + (size_t)H * dv, table + maxb, maxb, pos + 1,
                            L.mixed ? prec + 1 : NULL) == 0);
  }
  double kr[512], vr[512];
  for (int t = 0; t < 256; t += 37) {
    const int32_t b = orc_dequant_row(&L, pool + ((size_t)3 * H + 1 % H) * tb, t, kr, vr);
    CHECK(b > 0);
    for (int c = 0; c < d; ++c) CHECK(isfinite(kr[c]));
  }
  uint16_t* kd = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)4 * 256 * H * d);
  uint16_t* vd = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)4 * 256 * H * dv);
  CHECK(orc_dequantize_blocks(&L, pool, ids, 4, kd, vd) == 0);
  const int words = (700 + 31) / 32;
  uint32_t* mask = (uint32_t*)malloc(sizeof(uint32_t) * (size_t)n_seqs * words);
  for (int i = 0; i < n_seqs * words; ++i) mask[i] = lcg() & lcg();
  for (int i = 0; i < words; ++i) mask[(size_t)2 * words + i] = 0xFFFFFFFFu; /* one sequence all sentinel */
  uint16_t* q = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)n_seqs * H * G * d);
  fill_f16(q, (size_t)n_seqs * H * G * d, 1.0f);
  double* out = (double*)malloc(sizeof(double) * (size_t)n_seqs * H * G * dv);
  double* w = (double*)malloc(sizeof(double) * (size_t)n_seqs * H * G * 700);
  for (int with_mask = 0; with_mask < 2; ++with_mask) {
    CHECK(orc_decode_attention(&L, pool, q, n_seqs, H * G, table, maxb, lens, with_mask ? mask : NULL,
                               with_mask ? words : 0, 1.0f / sqrtf((float)d), out, w, 700, 1) == 0);
    for (size_t i = 0; i < (size_t)n_seqs * H * G * dv; ++i) CHECK(isfinite(out[i]));
  }
  free(pool); free(k); free(v); free(bits); free(ak); free(av); free(kd); free(vd); free(mask); free(q);
  free(out); free(w);
}

int main(void) {
  /* head_dim, H_kv, block, k_group, v_group, rotate, mixed, format, v_head_dim ; G */
  const struct { orc_layout L; int G; } cases[] = {
      {{128, 2, 256, 64, 64, 0, 0, 0, 0}, 4},  {{128, 2, 256, -1, 32, 1, 0, 0, 0}, 5},
      {{64, 1, 256, 32, 16, 1, 1, 0, 0}, 2},   {{128, 2, 256, 64, 32, 1, 2, 0, 0}, 2},
      {{128, 2, 256, 0, 0, 1, 0, 1, 0}, 3},    {{192, 2, 256, 64, 64, 0, 2, 0, 128}, 1},
      {{256, 1, 256, 8, 128, 1, 0, 0, 128}, 2}, {{256, 1, 256, 64, 64, 0, 1, 0, 0}, 1},
  };
  for (size_t i = 0; i < sizeof(cases) / sizeof(cases[0]); ++i) {
    run_layout(cases[i].L, cases[i].G);
    printf("layout %zu ok\n", i);
  }
  printf("sanitized oracle run ok\n");
  return 0;
}
