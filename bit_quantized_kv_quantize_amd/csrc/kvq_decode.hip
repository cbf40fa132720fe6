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
// One kernel per call: every split writes its partials, then bumps a per-(sequence, KV head) counter;
// the split that arrives last merges all partials in split order (so the result does not depend on
// which split that is), writes the output and resets the counter to zero for the next call.
#include "kvq_internal.hpp"

namespace kvq {
namespace {

constexpr float kSentinelLog2 = -14426.950408889634f;  // -1e4 * log2(e)
constexpr float kNegInf = -__builtin_huge_valf();

__device__ __forceinline__ float h2f(uint32_t bits16) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
}

__device__ __forceinline__ float wave_max(float v) {
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m);
  return v;
}

__device__ __forceinline__ bool is_sentinel(const uint32_t* mask_row, int pos) {
  return mask_row && ((mask_row[pos >> 5] >> (pos & 31)) & 1u);
}

// Codes of 8 consecutive channels starting at channel c0 of a row (4-bit or 8-bit).
__device__ __forceinline__ void codes8(const uint8_t* row, int c0, int bits, float (&c)[8]) {
  if (bits == 8) {
    uint2 w = *reinterpret_cast<const uint2*>(row + c0);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      c[e] = (float)((w.x >> (8 * e)) & 0xffu);
      c[4 + e] = (float)((w.y >> (8 * e)) & 0xffu);
    }
  } else {
    uint32_t w = *reinterpret_cast<const uint32_t*>(row + c0 / 2);
#pragma unroll
    for (int e = 0; e < 8; ++e) c[e] = (float)((w >> (4 * e)) & 0xfu);
  }
}

// Called by every split of (seq, h) after its partials are written. The last split to arrive merges the
// n_splits partials of the G query heads in split order, adds the sentinel term, undoes the rotation and
// writes the output; it then resets the counter. scratch: at least 2 * D floats of LDS.
template <int D>
__device__ void finish_unit(const TileGeom& g, const DecodeArgs& a, int seq, int h, int tid, float* scratch) {
  constexpr int NT = 256;
  __shared__ int s_last;
  __shared__ int s_cnt[NT / 64];
  __threadfence();  // this thread's partial writes are visible device-wide before the counter moves
  __syncthreads();
  if (tid == 0) {
    unsigned* ctr = a.ws_ctr + (size_t)seq * g.H + h;
    const unsigned prev = atomicAdd(ctr, 1u);
    s_last = prev == (unsigned)(a.plan.n_splits - 1);
    if (s_last) atomicExch(ctr, 0u);
  }
  __syncthreads();
  if (!s_last) return;
  __threadfence();  // observe every other split's partials

  const int len = a.seq_lens[seq];
  // sentinel slots among 0 .. len-1
  int cnt = 0;
  if (a.mask && len > 0) {
    const uint32_t* mrow = a.mask + (size_t)seq * a.mask_words;
    const int words = (len + 31) / 32;
    for (int w = tid; w < words; w += NT) {
      uint32_t bits = mrow[w];
      const int valid = len - w * 32;
      if (valid < 32) bits &= (1u << valid) - 1u;
      cnt += __popc(bits);
    }
  }
  for (int m = 32; m >= 1; m >>= 1) cnt += __shfl_xor(cnt, m);
  if ((tid & 63) == 0) s_cnt[tid >> 6] = cnt;
  __syncthreads();
  int n_sent = 0;
  for (int w = 0; w < NT / 64; ++w) n_sent += s_cnt[w];

  float* s_o = scratch;
  for (int jj = 0; jj < a.G; ++jj) {
    const int j = h * a.G + jj;
    const size_t p0 = ((size_t)seq * a.num_q_heads + j) * a.plan.n_splits;
    float M = n_sent > 0 ? kSentinelLog2 : kNegInf;
    for (int i = 0; i < a.plan.n_splits; ++i)
      if (a.ws_ml[2 * (p0 + i) + 1] > 0.0f)
        M = fmaxf(M, a.ws_ml[2 * (p0 + i)]);
    float L = n_sent > 0 ? (float)n_sent * exp2f(kSentinelLog2 - M) : 0.0f;
    float o = 0.0f;
    for (int i = 0; i < a.plan.n_splits; ++i) {
      const float li = a.ws_ml[2 * (p0 + i) + 1];
      if (li > 0.0f) {
        const float w = exp2f(a.ws_ml[2 * (p0 + i)] - M);
        L += li * w;
        if (tid < D) o += a.ws_acc[(p0 + i) * D + tid] * w;
      }
    }
    o = (len > 0 && L > 0.0f) ? o / L : 0.0f;
    if (g.rotate) {
      if (tid < D) s_o[tid] = o;
      __syncthreads();
      for (int hs = 1; hs < D; hs *= 2) {
        float r = 0.0f;
        if (tid < D) {
          const float x = s_o[tid], y = s_o[tid ^ hs];
          r = (tid & hs) ? (y - x) : (x + y);
        }
        __syncthreads();
        if (tid < D) s_o[tid] = r;
        __syncthreads();
      }
      if (tid < D) o = s_o[tid] * a.unrot_c;
      __syncthreads();
    }
    if (tid < D) a.out[((size_t)seq * a.num_q_heads + j) * D + tid] = o;
  }
}

// Grid (n_splits, H_kv, n_seqs), 256 threads. Thread t scores token t of each block against the G query
// heads of its KV head; for the value pass thread (cl, tg) owns channels cl*8 .. cl*8+7 and the tokens
// t = tg (mod TG). Writes (m, l, acc[d]) per query head and split.
template <int D, int GMAX>
__global__ __launch_bounds__(256) void decode_attn_k(TileGeom g, DecodeArgs a) {
  constexpr int NT = 256;
  constexpr int CL = D / 8;   // lanes per row in the value pass
  constexpr int TG = NT / CL; // token groups in the value pass
  __shared__ float s_q[GMAX][D];
  __shared__ float s_qk[GMAX][D];   // q * scale per channel (per-channel K groups only)
  __shared__ float s_qsum[GMAX][32];
  __shared__ float s_kconst[GMAX];
  __shared__ float s_p[GMAX][NT];
  __shared__ float s_red[GMAX][NT / 64];
  __shared__ float s_acc[TG][D];

  const int split = blockIdx.x, h = blockIdx.y, seq = blockIdx.z;
  const int tid = threadIdx.x;
  const int G = a.G;
  const int len = a.seq_lens[seq];
  const int nblk = (len + kRows - 1) / kRows;
  const int b0 = split * a.plan.blocks_per_split;
  const int b1 = min(b0 + a.plan.blocks_per_split, nblk);
  const uint32_t* mask_row = a.mask ? a.mask + (size_t)seq * a.mask_words : nullptr;
  const size_t part0 = ((size_t)seq * a.num_q_heads + (size_t)h * G) * a.plan.n_splits + split;

  if (b0 >= b1) {
    if (tid < G) {
      const size_t pi = part0 + (size_t)tid * a.plan.n_splits;
      a.ws_ml[2 * pi] = kNegInf;
      a.ws_ml[2 * pi + 1] = 0.0f;
    }
    finish_unit<D>(g, a, seq, h, tid, &s_acc[0][0]);
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
    const uint32_t* hdr = reinterpret_cast<const uint32_t*>(tile + g.off_hdr);

    if (g.kg < 0) {
      // per-channel K: fold scale into q and the zero into a per-head constant for this block
      for (int i = tid; i < GMAX * D; i += NT) {
        const int j = i / D, c = i % D;
        const uint32_t p = reinterpret_cast<const uint32_t*>(tile + g.off_kp)[c];
        s_qk[j][c] = s_q[j][c] * h2f(p & 0xffffu);
      }
      if (tid < GMAX) {
        float cst = 0.0f;
        for (int c = 0; c < D; ++c)
          cst += s_q[tid][c] * h2f(reinterpret_cast<const uint32_t*>(tile + g.off_kp)[c] >> 16);
        s_kconst[tid] = cst;
      }
      __syncthreads();
    }

    // scores of token tid
    const int pos = lb * kRows + tid;
    const bool live = pos < len && !is_sentinel(mask_row, pos);
    const int bits = (g.mixed && ((hdr[tid >> 5] >> (tid & 31)) & 1u)) ? 8 : 4;
    float score[GMAX];
#pragma unroll
    for (int j = 0; j < GMAX; ++j) score[j] = 0.0f;
    if (live) {
      const uint8_t* krow = tile + (size_t)tid * g.slot;
      if (g.kg > 0) {
        const uint32_t* kpar = reinterpret_cast<const uint32_t*>(tile + g.off_kp) + (size_t)tid * g.kpr;
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
            const uint32_t p = kpar[gi];
            const float sc = h2f(p & 0xffffu), zc = h2f(p >> 16);
#pragma unroll
            for (int j = 0; j < GMAX; ++j) {
              score[j] += sc * part[j] + zc * s_qsum[j][gi];
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
        for (int j = 0; j < GMAX; ++j) score[j] += s_kconst[j];
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
    const int vgi = (cl * 8) / g.vg;
    for (int t = tg; t < kRows; t += TG) {
      bool any = false;
#pragma unroll
      for (int j = 0; j < GMAX; ++j) any |= s_p[j][t] != 0.0f;
      if (!any) continue;
      const int vbits = (g.mixed && ((hdr[t >> 5] >> (t & 31)) & 1u)) ? 8 : 4;
      float c[8];
      codes8(tile + g.off_vc + (size_t)t * g.slot, cl * 8, vbits, c);
      const uint32_t p = reinterpret_cast<const uint32_t*>(tile + g.off_vp)[(size_t)t * g.vpr + vgi];
      const float sc = h2f(p & 0xffffu), zc = h2f(p >> 16);
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
    for (int c = tid; c < D; c += NT) {
      float sum = 0.0f;
      for (int r = 0; r < TG; ++r) sum += s_acc[r][c];
      a.ws_acc[pi * D + c] = sum;
    }
    if (tid == 0) {
      a.ws_ml[2 * pi] = m_run[j];
      a.ws_ml[2 * pi + 1] = l_run[j];
    }
    __syncthreads();
  }
  finish_unit<D>(g, a, seq, h, tid, &s_acc[0][0]);
}
template <int D, int GMAX>
hipError_t launch_t(const TileGeom& g, const DecodeArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL((decode_attn_k<D, GMAX>), dim3(a.plan.n_splits, g.H, a.n_seqs), dim3(256), 0, stream,
                     g, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const TileGeom& g, const DecodeArgs& a, hipStream_t stream) {
  if (a.G <= 4) return launch_t<D, 4>(g, a, stream);
  if (a.G <= 8) return launch_t<D, 8>(g, a, stream);
  return launch_t<D, 16>(g, a, stream);
}

}  // namespace

hipError_t launch_decode(const TileGeom& g, const DecodeArgs& a, hipStream_t stream) {
  switch (g.d) {
    case 64: return launch_d<64>(g, a, stream);
    case 128: return launch_d<128>(g, a, stream);
    case 256: return launch_d<256>(g, a, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace kvq
