// kvq_decode_common.hpp - pieces shared by the decode-attention kernels: base-2 logit constants, the
// sentinel count, the final per-head normalisation (with the sentinel term and the inverse rotation) and
// the split-K reduction kernel.
#pragma once

#include "kvq_internal.hpp"

namespace kvq {
namespace dec {


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

// Number of sentinel slots among 0 .. len-1 of sequence seq (block-wide reduction over NT threads).
template <int NT>
__device__ int count_sentinels(const DecodeArgs& a, int seq, int len, int tid, int* s_cnt) {
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
  __syncthreads();
  if ((tid & 63) == 0) s_cnt[tid >> 6] = cnt;
  __syncthreads();
  int n = 0;
  for (int w = 0; w < NT / 64; ++w) n += s_cnt[w];
  return n;
}

// Final output row of query head j: live slots contribute (M, L, o) (base-2 max, sum of exp2(logit - M),
// sum of exp2(logit - M) * v; M = -inf and L = 0 when there are none), each of the n_sent sentinel slots
// contributes logit -1e4 and value 0. Thread c < D holds o for channel c (D = V's head dim). For a rotated
// pool the row is multiplied by (1 / (D c)) H, the inverse of the quantiser's rotation of V rows. All NT
// threads must call this.
template <int D, int NT>
__device__ void finalize_head(const TileGeom& g, const DecodeArgs& a, int seq, int j, int len, int n_sent,
                              float M, float L, float o, int tid, float* s_o) {
  const float Mt = n_sent > 0 ? fmaxf(M, kSentinelLog2) : M;
  float Lt = 0.0f;
  if (L > 0.0f) {
    const float w = exp2f(M - Mt);
    Lt = L * w;
    o *= w;
  } else {
    o = 0.0f;
  }
  if (n_sent > 0) Lt += (float)n_sent * exp2f(kSentinelLog2 - Mt);
  o = (len > 0 && Lt > 0.0f) ? o / Lt : 0.0f;
  if (g.rotate) {
    // butterflies of channel strides 1 .. 32 between the lanes of a wave (channel c in lane c mod 64), the
    // wider strides through LDS
    for (int hs = 1; hs < D && hs < 64; hs *= 2) {
      const float y = __shfl_xor(o, hs);
      o = (tid & hs) ? (y - o) : (o + y);
    }
    for (int hs = 64; hs < D; hs *= 2) {
      __syncthreads();
      if (tid < D) s_o[tid] = o;
      __syncthreads();
      const float y = tid < D ? s_o[tid ^ hs] : 0.0f;
      o = (tid & hs) ? (y - o) : (o + y);
    }
    o *= a.unrot_cv;
  }
  if (tid < D) a.out[((size_t)seq * a.num_q_heads + j) * D + tid] = o;
}

// Split-K reduction: grid (H_q, n_seqs), D threads. Merges the n_splits partials of one query head in
// split order and finalises the head. Split maxima and sums are staged in LDS by parallel loads, and the
// accumulator loads of different splits are independent, so the kernel is one or two memory latencies.
template <int D>
__global__ __launch_bounds__(D) void decode_reduce_k(TileGeom g, DecodeArgs a) {
  constexpr int kMaxStage = 512;
  __shared__ float s_m[kMaxStage], s_w[kMaxStage];
  __shared__ float s_o[D];
  __shared__ int s_cnt[D / 64];
  __shared__ float s_ML[2];
  const int j = blockIdx.x, seq = blockIdx.y, tid = threadIdx.x;
  const int ns = a.plan.n_splits;
  const int len = a.seq_lens[seq];
  const size_t p0 = ((size_t)seq * a.num_q_heads + j) * ns;
  const int n_sent = count_sentinels<D>(a, seq, len, tid, s_cnt);
  float M = kNegInf, L = 0.0f, o = 0.0f;
  for (int base = 0; base < ns; base += kMaxStage) {
    const int cnt = min(kMaxStage, ns - base);
    for (int i = tid; i < cnt; i += D) {
      const float li = a.ws_ml[2 * (p0 + base + i) + 1];
      s_m[i] = li > 0.0f ? a.ws_ml[2 * (p0 + base + i)] : kNegInf;
      s_w[i] = li;
    }
    __syncthreads();
    if (tid == 0) {
      float m = M;
      for (int i = 0; i < cnt; ++i) m = fmaxf(m, s_m[i]);
      float l = m == kNegInf ? 0.0f : L * exp2f(M - m);
      for (int i = 0; i < cnt; ++i) {
        const float w = s_m[i] == kNegInf ? 0.0f : exp2f(s_m[i] - m);
        l += s_w[i] * w;
        s_w[i] = w;
      }
      s_ML[0] = m;
      s_ML[1] = l;
    }
    __syncthreads();
    const float m_new = s_ML[0];
    if (m_new != kNegInf) {
      o = M == kNegInf ? 0.0f : o * exp2f(M - m_new);
      float acc = 0.0f;
#pragma unroll 8
      for (int i = 0; i < cnt; ++i) {
        // empty splits leave their accumulators unwritten: select, never multiply, them away
        const float x = a.ws_acc[(p0 + base + i) * D + tid];
        acc += s_w[i] != 0.0f ? x * s_w[i] : 0.0f;
      }
      o += acc;
    }
    M = m_new;
    L = s_ML[1];
    __syncthreads();
  }
  finalize_head<D, D>(g, a, seq, j, len, n_sent, M, L, o, tid, s_o);
}

}  // namespace dec
}  // namespace kvq
