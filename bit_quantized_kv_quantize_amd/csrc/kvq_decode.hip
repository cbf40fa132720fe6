// kvq_decode.hip - single-token decode attention that reads packed Q4/Q8 tiles and dequantises in
// registers, with split-K over blocks, online softmax and a final reduction.
//
// Follows "Agent Memory Below the Prompt" (technical summary 2.1: the quantised cache goes straight into
// attention, many agents in one batch; 2.2: GQA), the IntentKV article (invalidation section: a slot
// remapped to the sentinel has key -1e4 and contributes no weight) and the UltraQuant article
// (technology section: rotated 4-bit cache, AMD decode kernel). Logits are kept in base-2 units
// (q is pre-scaled by softmax_scale * log2 e) so the softmax uses exp2.
//
// Sentinel slots are never loaded. Their exact contribution to the softmax, n_sentinel terms with logit
// -1e4 and value 0, is added in the reduction: it changes the normaliser only when no live logit is far
// above -1e4, and makes an all-sentinel sequence return zeros, as the definition does.
//
// Every split writes its partials (m, l, acc[d]) per query head; decode_reduce_k merges them in split
// order in a second kernel (the kernel boundary makes the partials visible across the chip's XCDs).
#include <stdlib.h>
#include <string.h>

#include "kvq_decode_common.hpp"
#include "kvq_decode_precise.hpp"

namespace kvq {
namespace {

using namespace dec;

// Codes of 8 consecutive channels starting at channel c0 of a row (4-bit or 8-bit).
__device__ __forceinline__ void codes8(const uint8_t* row, int c0, int bits, float (&c)[8]) {
  if (bits == 8) {
    uint2 w = *reinterpret_cast<const uint2*>(row + c0);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      c[e] = (float)((w.x >> (8 * e)) & 0xffu);
      c[4 + e] = (float)((w.y >> (8 * e)) & 0xffu);
    }
  } else if (bits == 4) {
    uint32_t w = *reinterpret_cast<const uint32_t*>(row + c0 / 2);
#pragma unroll
    for (int e = 0; e < 8; ++e) c[e] = (float)((w >> (4 * e)) & 0xfu);
  } else if (bits == 2) {
    uint32_t w = *reinterpret_cast<const uint16_t*>(row + c0 / 4);
#pragma unroll
    for (int e = 0; e < 8; ++e) c[e] = (float)((w >> (2 * e)) & 0x3u);
  } else {  // 16: the values themselves, fp16
    const uint4 w = *reinterpret_cast<const uint4*>(row + 2 * c0);
    const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      c[2 * e] = h2f(ww[e] & 0xffffu);
      c[2 * e + 1] = h2f(ww[e] >> 16);
    }
  }
}

// Scale and zero of a group from its stored word; a 16-bit row carries its values as they are.
__device__ __forceinline__ void group_params(uint32_t p, int bits, float& sc, float& zc) {
  sc = bits == 16 ? 1.0f : h2f(p & 0xffffu);
  zc = bits == 16 ? 0.0f : h2f(p >> 16);
}

// Values of 8 consecutive channels starting at channel c0 of an FP8 E4M3 row (exact in fp32).
__device__ __forceinline__ void fp8x8(const uint8_t* row, int c0, float (&c)[8]) {
  const uint2 w = *reinterpret_cast<const uint2*>(row + c0);
  c[0] = __builtin_amdgcn_cvt_f32_fp8((int)w.x, 0);
  c[1] = __builtin_amdgcn_cvt_f32_fp8((int)w.x, 1);
  c[2] = __builtin_amdgcn_cvt_f32_fp8((int)w.x, 2);
  c[3] = __builtin_amdgcn_cvt_f32_fp8((int)w.x, 3);
  c[4] = __builtin_amdgcn_cvt_f32_fp8((int)w.y, 0);
  c[5] = __builtin_amdgcn_cvt_f32_fp8((int)w.y, 1);
  c[6] = __builtin_amdgcn_cvt_f32_fp8((int)w.y, 2);
  c[7] = __builtin_amdgcn_cvt_f32_fp8((int)w.y, 3);
}

// Grid (n_splits, H_kv, n_seqs), 256 threads. Thread t scores token t of each block against the G query
// heads of its KV head; for the value pass thread (cl, tg) owns channels cl*8 .. cl*8+7 and the tokens
// t = tg (mod TG). Writes (m, l, acc[dv]) per query head and split. D = K's head dim (and the query's),
// DV = V's.
template <int D, int DV, int GMAX>
__global__ __launch_bounds__(256) void decode_attn_k(TileGeom g, DecodeArgs a) {
  constexpr int NT = 256;
  constexpr int CL = DV / 8;  // lanes per row in the value pass
  constexpr int TG = NT / CL; // token groups in the value pass
  __shared__ float s_q[GMAX][D];
  __shared__ float s_qk[GMAX][D];   // q * scale per channel (per-channel K groups only)
  __shared__ float s_qsum[GMAX][32];
  __shared__ float s_kconst[GMAX];
  __shared__ float s_p[GMAX][NT];
  __shared__ float s_red[GMAX][NT / 64];
  __shared__ float s_acc[TG][DV];

  const int split = blockIdx.x, h = blockIdx.y, seq = blockIdx.z;
  const int tid = threadIdx.x;
  const int G = a.G;
  const int len = a.seq_lens[seq];
  const int nblk = (len + kRows - 1) / kRows;
  int b0, b1;
  split_range(split, a.plan.n_splits, nblk, b0, b1);
  const uint32_t* mask_row = a.mask ? a.mask + (size_t)seq * a.mask_words : nullptr;
  const size_t part0 = ((size_t)seq * a.num_q_heads + (size_t)h * G) * a.plan.n_splits + split;

  if (b0 >= b1) {
    if (tid < G) {
      const size_t pi = part0 + (size_t)tid * a.plan.n_splits;
      a.ws_ml[2 * pi] = kNegInf;
      a.ws_ml[2 * pi + 1] = 0.0f;
    }
    return;
  }

  // q rows of this KV head's query heads, scaled to base-2 logits and rotated like the cache.
  for (int i = tid; i < GMAX * D; i += NT) {
    const int j = i / D, c = i % D;
    s_q[j][c] = j < G ? h2f(a.q[((size_t)seq * a.num_q_heads + h * G + j) * D + c]) * a.q_scale : 0.0f;
  }
  __syncthreads();
  if (g.rotate) {
    for (int hs = 1; hs < D; hs *= 2) {
      for (int i = tid; i < GMAX * D / 2; i += NT) {
        const int j = i / (D / 2), pidx = i % (D / 2);
        const int lo = (pidx / hs) * 2 * hs + (pidx % hs);
        float x = s_q[j][lo], y = s_q[j][lo + hs];
        s_q[j][lo] = x + y;
        s_q[j][lo + hs] = x - y;
      }
      __syncthreads();
    }
    for (int i = tid; i < GMAX * D; i += NT) s_q[i / D][i % D] *= a.unrot_c;
    __syncthreads();
  }
  if (g.kg > 0) {
    const int ng = D / g.kg;
    for (int i = tid; i < GMAX * ng; i += NT) {
      const int j = i / ng, gi = i % ng;
      float sum = 0.0f;
      for (int c = 0; c < g.kg; ++c) sum += s_q[j][gi * g.kg + c];
      s_qsum[j][gi] = sum;
    }
  }
  __syncthreads();

  float m_run[GMAX], l_run[GMAX], acc[GMAX][8], zacc[GMAX];
#pragma unroll
  for (int j = 0; j < GMAX; ++j) {
    m_run[j] = kNegInf;
    l_run[j] = 0.0f;
    zacc[j] = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[j][e] = 0.0f;
  }
  const int cl = tid % CL, tg = tid / CL;
  const int lane = tid & 63, wave = tid >> 6;

  for (int lb = b0; lb < b1; ++lb) {
    const int phys = a.block_table[(size_t)seq * a.max_blocks_per_seq + lb];
    const uint8_t* tile = a.pool + ((size_t)phys * g.H + h) * g.tile_bytes;

    if (g.kg < 0) {
      // per-channel K: fold scale into q and the zero into a per-head constant for this block
      for (int i = tid; i < GMAX * D; i += NT) {
        const int j = i / D, c = i % D;
        const uint32_t p = reinterpret_cast<const uint32_t*>(tile + g.off_kch)[c];
        s_qk[j][c] = s_q[j][c] * h2f(p & 0xffffu);
      }
      if (tid < GMAX) {
        float cst = 0.0f;
        for (int c = 0; c < D; ++c)
          cst += s_q[tid][c] * h2f(reinterpret_cast<const uint32_t*>(tile + g.off_kch)[c] >> 16);
        s_kconst[tid] = cst;
      }
      __syncthreads();
    }

    // scores of token tid
    const int pos = lb * kRows + tid;
    const bool live = pos < len && !is_sentinel(mask_row, pos);
    const int bits = g.row_bits(tile, tid);
    float score[GMAX];
#pragma unroll
    for (int j = 0; j < GMAX; ++j) score[j] = 0.0f;
    float terms = 0.0f;  // largest sum of term magnitudes of this token's logits (per-token K groups)
    if (live) {
      const uint8_t* krow = tile + g.kcode(tid);
      if (g.fp8) {
        for (int c0 = 0; c0 < D; c0 += 8) {
          float c[8];
          fp8x8(krow, c0, c);
#pragma unroll
          for (int j = 0; j < GMAX; ++j) {
#pragma unroll
            for (int e = 0; e < 8; ++e) score[j] += c[e] * s_q[j][c0 + e];
          }
        }
      } else if (g.kg > 0) {
        const uint32_t* kpar = reinterpret_cast<const uint32_t*>(tile + g.kpar(tid));
        float part[GMAX];
#pragma unroll
        for (int j = 0; j < GMAX; ++j) part[j] = 0.0f;
        for (int c0 = 0; c0 < D; c0 += 8) {
          float c[8];
          codes8(krow, c0, bits, c);
#pragma unroll
          for (int j = 0; j < GMAX; ++j) {
            float d8 = 0.0f;
#pragma unroll
            for (int e = 0; e < 8; ++e) d8 += c[e] * s_q[j][c0 + e];
            part[j] += d8;
          }
          if (((c0 + 8) % g.kg) == 0) {
            const int gi = c0 / g.kg;
            float sc, zc;
            group_params(kpar[gi], bits, sc, zc);
#pragma unroll
            for (int j = 0; j < GMAX; ++j) {
              score[j] += sc * part[j] + zc * s_qsum[j][gi];
              terms = fmaxf(terms, fabsf(sc * part[j]) + fabsf(zc * s_qsum[j][gi]));
              part[j] = 0.0f;
            }
          }
        }
      } else {
        for (int c0 = 0; c0 < D; c0 += 8) {
          float c[8];
          codes8(krow, c0, 4, c);
#pragma unroll
          for (int j = 0; j < GMAX; ++j) {
#pragma unroll
            for (int e = 0; e < 8; ++e) score[j] += c[e] * s_qk[j][c0 + e];
          }
        }
#pragma unroll
        for (int j = 0; j < GMAX; ++j) {
          terms = fmaxf(terms, fabsf(score[j]) + fabsf(s_kconst[j]));
          score[j] += s_kconst[j];
        }
      }
      // Logits with terms beyond kPreciseAbove (base-2 units): this token's logits again in fp64, from the
      // exactly dequantised K row (the plain definition; rare, so a per-thread branch).
      bool big = terms > kPreciseAbove;
#pragma unroll
      for (int j = 0; j < GMAX; ++j) big |= j < G && fabsf(score[j]) > kPreciseAbove;
      if (big) {
        const int kbits = g.fp8 ? 8 : bits;
        double dot[GMAX];
#pragma unroll
        for (int j = 0; j < GMAX; ++j) dot[j] = 0.0;
        for (int c = 0; c < D; ++c) {
          float ks, kz;
          k_params(g, tile, tid, c, ks, kz);
          const double kv = code_value(g, krow, kbits, c, ks, kz);
#pragma unroll
          for (int j = 0; j < GMAX; ++j) {
            const double qc = g.rotate || j >= G
                                  ? (double)s_q[j][c]
                                  : (double)h2f(a.q[((size_t)seq * a.num_q_heads + h * G + j) * D + c]) * a.q_scale64;
            dot[j] += qc * kv;
          }
        }
#pragma unroll
        for (int j = 0; j < GMAX; ++j) score[j] = (float)dot[j];
      }
    }
    // block max per head
#pragma unroll
    for (int j = 0; j < GMAX; ++j) {
      float v = wave_max(live ? score[j] : kNegInf);
      if (lane == 0) s_red[j][wave] = v;
    }
    __syncthreads();
    float alpha[GMAX], m_new[GMAX];
#pragma unroll
    for (int j = 0; j < GMAX; ++j) {
      float bm = s_red[j][0];
      for (int w = 1; w < NT / 64; ++w) bm = fmaxf(bm, s_red[j][w]);
      m_new[j] = fmaxf(m_run[j], bm);
      alpha[j] = m_new[j] == kNegInf ? 1.0f : exp2f(m_run[j] - m_new[j]);
      s_p[j][tid] = live ? exp2f(score[j] - m_new[j]) : 0.0f;
    }
    __syncthreads();
    // block sum per head
#pragma unroll
    for (int j = 0; j < GMAX; ++j) {
      float v = wave_sum(s_p[j][tid]);
      if (lane == 0) s_red[j][wave] = v;
    }
    // value pass
#pragma unroll
    for (int j = 0; j < GMAX; ++j) {
      zacc[j] *= alpha[j];
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[j][e] *= alpha[j];
    }
    const int vgi = g.fp8 ? 0 : (cl * 8) / g.vg;
    for (int t = tg; t < kRows; t += TG) {
      bool any = false;
#pragma unroll
      for (int j = 0; j < GMAX; ++j) any |= s_p[j][t] != 0.0f;
      if (!any) continue;
      if (g.fp8) {
        float c[8];
        fp8x8(tile + g.vcode(t, 8), cl * 8, c);
#pragma unroll
        for (int j = 0; j < GMAX; ++j) {
          const float pj = s_p[j][t];
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[j][e] += pj * c[e];
        }
        continue;
      }
      const int vbits = g.row_bits(tile, t);
      float c[8];
      codes8(tile + g.vcode(t, vbits), cl * 8, vbits, c);
      float sc, zc;
      group_params(reinterpret_cast<const uint32_t*>(tile + g.vpar(t))[vgi], vbits, sc, zc);
#pragma unroll
      for (int j = 0; j < GMAX; ++j) {
        const float pj = s_p[j][t];
        const float ps = pj * sc;
        zacc[j] += pj * zc;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[j][e] += ps * c[e];
      }
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < GMAX; ++j) {
      float bs = 0.0f;
      for (int w = 0; w < NT / 64; ++w) bs += s_red[j][w];
      l_run[j] = l_run[j] * alpha[j] + bs;
      m_run[j] = m_new[j];
    }
    __syncthreads();
  }

  // reduce the value accumulators over the token groups, one query head at a time
  for (int j = 0; j < G; ++j) {
#pragma unroll
    for (int e = 0; e < 8; ++e) s_acc[tg][cl * 8 + e] = acc[j][e] + zacc[j];
    __syncthreads();
    const size_t pi = part0 + (size_t)j * a.plan.n_splits;
    for (int c = tid; c < DV; c += NT) {
      float sum = 0.0f;
      for (int r = 0; r < TG; ++r) sum += s_acc[r][c];
      a.ws_acc[pi * DV + c] = sum;
    }
    if (tid == 0) {
      a.ws_ml[2 * pi] = m_run[j];
      a.ws_ml[2 * pi + 1] = l_run[j];
    }
    __syncthreads();
  }
}
template <int D, int DV, int GMAX>
hipError_t launch_t(const TileGeom& g, const DecodeArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL((decode_attn_k<D, DV, GMAX>), dim3(a.plan.n_splits, g.H, a.n_seqs), dim3(256), 0, stream,
                     g, a);
  hipLaunchKernelGGL(decode_reduce_k<DV>, dim3(a.num_q_heads, a.n_seqs), dim3(DV), 0, stream, g, a);
  return hipGetLastError();
}

template <int D, int DV>
hipError_t launch_d(const TileGeom& g, const DecodeArgs& a, hipStream_t stream) {
  // the head loops run over GMAX heads: the smallest instance that holds G
  if (a.G == 1) return launch_t<D, DV, 1>(g, a, stream);
  if (a.G == 2) return launch_t<D, DV, 2>(g, a, stream);
  if (a.G <= 4) return launch_t<D, DV, 4>(g, a, stream);
  if (a.G <= 8) return launch_t<D, DV, 8>(g, a, stream);
  return launch_t<D, DV, 16>(g, a, stream);
}

}  // namespace

hipError_t launch_decode(const TileGeom& g, const DecodeArgs& a, hipStream_t stream) {
#ifdef KVQ_DEBUG
  // test hook of the debug build only: KVQ_DECODE_KERNEL=generic|mfma|nocascade (read on every call)
  const char* force = getenv("KVQ_DECODE_KERNEL");
#else
  const char* force = nullptr;
#endif
  const bool generic = force && !strcmp(force, "generic");
  const bool mfma = force && !strcmp(force, "mfma");
  if (!generic && !mfma && decode_rows_supported(g, a.G, a.mask != nullptr)) return launch_decode_rows(g, a, stream);
  if (!generic && !mfma && decode_kchan_supported(g, a.G)) {
    // Blocks shared by two or more sequences go through the cascade kernel first (not for pools with sentinel
    // slots).
    const bool nocasc = force && !strcmp(force, "nocascade");
    if (!nocasc && a.plan.casc > 0 && !a.mask && a.n_seqs >= 2 && decode_cascade_supported(g, a.G)) {
      DecodeArgs b = a;
      b.casc = a.plan.casc;
      const hipError_t e = launch_decode_cascade(g, b, stream);
      if (e != hipSuccess) return e;
      return launch_decode_kchan(g, b, stream);
    }
    return launch_decode_kchan(g, a, stream);
  }
  if (!generic && decode_mfma_supported(g, a.G)) return launch_decode_mfma(g, a, stream);
  if (!generic && !a.mask && decode_fp8_supported(g, a.G)) return launch_decode_fp8(g, a, stream);
  return launch_decode_generic(g, a, stream);
}

hipError_t launch_decode_generic(const TileGeom& g, const DecodeArgs& a, hipStream_t stream) {
  if (g.dv == g.d) {
    switch (g.d) {
      case 64: return launch_d<64, 64>(g, a, stream);
      case 128: return launch_d<128, 128>(g, a, stream);
      case 256: return launch_d<256, 256>(g, a, stream);
    }
  }
  if (g.d == 192 && g.dv == 128) return launch_d<192, 128>(g, a, stream);
  if (g.d == 256 && g.dv == 128) return launch_d<256, 128>(g, a, stream);
  return hipErrorInvalidValue;
}

}  // namespace kvq
