// kvq_decode_precise.hpp - fp64 logits for the waves of the matrix-core decode kernels whose logit terms are
// too large for the fp32 combination those kernels use.
//
// The matrix-core kernels form a logit per group as scale * (q . codes) + zero * sum(q), from fp16 hi/lo query
// operands, and add the groups in fp32. For attention's usual logits that is accurate to a few 1e-4 of a logit.
// When the terms reach thousands (queries or keys scaled far beyond the usual range; the case that matters is
// live logits next to the sentinel's -1e4 of the IntentKV article's invalidation section, where the sentinel
// term enters the normaliser with an exactly known logit), fp32 roundings of terms that cancel grow with them.
// A wave that meets a logit whose terms exceed kPreciseAbove therefore recomputes its rows here, after its
// main loop: one token per lane, the K row dequantised exactly (code * scale + zero is exact in fp64) and
// dotted with the query in fp64 - the plain definition of the logit - then an online softmax over the wave's
// tokens, and the dequantised V rows weighted in fp32 with one output channel per lane. The pass writes the
// wave's (m, l, acc) per query head where the kernel's own wave merge would have; nothing else changes.
#pragma once

#include "kvq_decode_common.hpp"

namespace kvq {
namespace dec {

// Logit terms (base-2 units) above which a wave takes the fp64 pass.
constexpr float kPreciseAbove = 1024.0f;

// Channel c of a row's K or V codes (`codes` = the row's codes of that tensor, `bits` = the row's width) as its
// rotated-domain value: code * s + z, exact in fp64 (an 8-bit code times an fp16 scale has 19 significant bits);
// FP16 rows hold the value itself, FP8 pools the E4M3 value.
__device__ inline double code_value(const TileGeom& g, const uint8_t* codes, int bits, int c, float s, float z) {
  if (g.fp8) return (double)__builtin_amdgcn_cvt_f32_fp8((int)codes[c], 0);
  uint32_t code;
  if (bits == 4) {
    code = (codes[c >> 1] >> (4 * (c & 1))) & 15u;
  } else if (bits == 8) {
    code = codes[c];
  } else if (bits == 2) {
    code = (codes[c >> 2] >> (2 * (c & 3))) & 3u;
  } else {
    return (double)h2f(reinterpret_cast<const uint16_t*>(codes)[c]);
  }
  return (double)code * (double)s + (double)z;
}

// {scale, zero} of channel c of row `row`'s K (per-token groups or per-channel) or V.
__device__ inline void k_params(const TileGeom& g, const uint8_t* tile, int row, int c, float& s, float& z) {
  if (g.fp8) {
    s = 1.0f;
    z = 0.0f;
    return;
  }
  const uint32_t p = g.kg > 0 ? reinterpret_cast<const uint32_t*>(tile + g.kpar(row))[c / g.kg]
                              : reinterpret_cast<const uint32_t*>(tile + g.off_kch)[c];
  s = h2f(p & 0xffffu);
  z = h2f(p >> 16);
}
__device__ inline void v_params(const TileGeom& g, const uint8_t* tile, int row, int c, float& s, float& z) {
  if (g.fp8) {
    s = 1.0f;
    z = 0.0f;
    return;
  }
  const uint32_t p = reinterpret_cast<const uint32_t*>(tile + g.vpar(row))[c / g.vg];
  s = h2f(p & 0xffffu);
  z = h2f(p >> 16);
}

// The fp64 pass of one wave over n_pass passes of up to 64 tokens. tok(p, i, tile, row) sets token i of pass p
// (tile base and row) and returns whether it is live; it must be callable with any i in 0..63 by every lane.
// qv(j, c) is query head j's channel c (rotated domain) in fp64, scaled so that a logit in base-2 units is
// sum_c qv(j, c) * k_c. s_pw: 64 * G floats of this wave's LDS. Writes m_out[j], l_out[j] and acc_out[j * DV +
// c] (the weighted sum of dequantised V rows, zero points included) for j < G. All 64 lanes must call it.
template <int D, int DV, int G, class Tok, class QV>
__device__ void precise_wave_pass(const TileGeom& g, int n_pass, Tok tok, QV qv, float* s_pw, float* m_out,
                                  float* l_out, float* acc_out) {
  constexpr int NCH = (DV + 63) / 64;  // output channels per lane
  const int lane = threadIdx.x & 63;
  float m[G], l[G], acc[G][NCH];
#pragma unroll
  for (int j = 0; j < G; ++j) {
    m[j] = kNegInf;
    l[j] = 0.0f;
#pragma unroll
    for (int cc = 0; cc < NCH; ++cc) acc[j][cc] = 0.0f;
  }
  for (int p = 0; p < n_pass; ++p) {
    // logits: token `lane` of the pass
    const uint8_t* tile;
    int row;
    const bool live = tok(p, lane, tile, row);
    float sc[G];
#pragma unroll
    for (int j = 0; j < G; ++j) sc[j] = kNegInf;
    if (live) {
      const int bits = g.fp8 ? 8 : g.row_bits(tile, row);
      const uint8_t* kc = tile + g.kcode(row);
      double dot[G];
#pragma unroll
      for (int j = 0; j < G; ++j) dot[j] = 0.0;
      for (int c = 0; c < D; ++c) {
        float s, z;
        k_params(g, tile, row, c, s, z);
        const double kv = code_value(g, kc, bits, c, s, z);
#pragma unroll
        for (int j = 0; j < G; ++j) dot[j] += qv(j, c) * kv;
      }
#pragma unroll
      for (int j = 0; j < G; ++j) sc[j] = (float)dot[j];
    }
    // online softmax over the wave's tokens
    float alpha[G];
#pragma unroll
    for (int j = 0; j < G; ++j) {
      const float mnew = fmaxf(m[j], wave_max(sc[j]));
      alpha[j] = mnew == kNegInf ? 1.0f : exp2f(m[j] - mnew);  // exp2(-inf) = 0 for the first live token
      const float pj = (live && mnew != kNegInf) ? exp2f(sc[j] - mnew) : 0.0f;
      l[j] = l[j] * alpha[j] + wave_sum(pj);
      m[j] = mnew;
      s_pw[j * 64 + lane] = pj;
#pragma unroll
      for (int cc = 0; cc < NCH; ++cc) acc[j][cc] *= alpha[j];
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // values: one output channel per lane, the pass's live tokens in order
    for (int t = 0; t < 64; ++t) {
      const uint8_t* tt;
      int rr;
      if (!tok(p, t, tt, rr)) continue;  // the same for every lane
      const int bits = g.fp8 ? 8 : g.row_bits(tt, rr);
      const uint8_t* vc = tt + g.vcode(rr, bits);
#pragma unroll
      for (int cc = 0; cc < NCH; ++cc) {
        const int c = lane + 64 * cc;
        if (c < DV) {
          float s, z;
          v_params(g, tt, rr, c, s, z);
          const float v = (float)code_value(g, vc, bits, c, s, z);
#pragma unroll
          for (int j = 0; j < G; ++j) acc[j][cc] += s_pw[j * 64 + t] * v;
        }
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
#pragma unroll
  for (int j = 0; j < G; ++j) {
    if (lane == 0) {
      m_out[j] = m[j];
      l_out[j] = l[j];
    }
#pragma unroll
    for (int cc = 0; cc < NCH; ++cc) {
      const int c = lane + 64 * cc;
      if (c < DV) acc_out[j * DV + c] = acc[j][cc];
    }
  }
}

}  // namespace dec
}  // namespace kvq
