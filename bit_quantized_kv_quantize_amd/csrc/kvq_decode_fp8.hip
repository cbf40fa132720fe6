// kvq_decode_fp8.hip - decode attention on the matrix cores over FP8 E4M3 pools (head_dim 128, GQA ratios up to
// 8, no sentinel mask): the FP8 cache the UltraQuant article's technology section compares the 4-bit cache
// against, run through the same kind of kernel as the 4-bit pools (split-K over blocks, each wave taking 64
// rows of every block, online softmax, the in-kernel split merge of splitk_arrive).
//
// Every E4M3 value is exact in fp16, so both operands come from the cache without rounding:
// * QK (v_mfma_f32_16x16x32_f16): A = the query as fp16 hi/lo rows (row 2h + part, heads h < 8), built once;
//   B = the K bytes of 16 tokens (lane = token) converted pairwise to fp16 (v_cvt_scalef32_pk_f16_fp8,
//   scale 1).
// * PV: A = p as fp16 hi/lo rows (the same row layout), written position-major and read with the 16-bit LDS
//   transpose load; B = the V bytes staged in LDS as loaded and read with the 8-bit transpose load (one
//   output channel and eight tokens per lane), converted to fp16. V is not offset by a group zero, so the
//   fp32 accumulation runs directly in the output tiles.
#include "kvq_decode_mfma_common.hpp"

namespace kvq {
namespace {

using namespace dec;

typedef int v2i __attribute__((ext_vector_type(2)));
typedef short v4s __attribute__((ext_vector_type(4)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) v2i lds_v2i;
typedef __attribute__((address_space(3))) v4s lds_v4s;

__device__ __forceinline__ v2i lds_tr8(const void* p) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i*)const_cast<void*>(p));
}
__device__ __forceinline__ v2i lds_tr16(const void* p) {
  return __builtin_bit_cast(v2i, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)const_cast<void*>(p)));
}
// fp16 pair of E4M3 bytes 2 SEL, 2 SEL + 1 of w (exact)
template <bool SEL>
__device__ __forceinline__ uint32_t e4m3_pair(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)w, 1.0f, SEL));
}

constexpr int kD = 128;
constexpr int kVP8 = 144;  // LDS row pitch (bytes) of staged V rows (128 bytes + pad)
constexpr int kPP = 20;    // halves per position of the position-major p tile (16 rows + pad)

// A chunk's 64 rows as loaded: K (V) slab j = the K (V) halves of rows 8j .. 8j+7, lane l holding bytes
// 16 (l % 8) .. +15 of row 8j + l / 8, so every 8 consecutive lanes read one whole 128-byte line. (Each lane
// reading its own token's channels instead - 16 lines per load, 64 bytes of each - was 8 % slower on the
// 4-bit pools' read pattern, 14 % against non-temporal slab loads.)
struct RawF {
  u32x4 k[8];
  u32x4 v[8];
  uint32_t live;  // bit c: token 16c + lj is below seq_len
};

// Grid (n_splits, H_kv, n_seqs), 256 threads = 4 waves; wave w owns rows 64w .. 64w+63 of each block.
template <int G>
__global__ __launch_bounds__(256, 2) void decode_fp8_k(TileGeom g, DecodeArgs a) {
  static_assert(G >= 1 && G <= 8, "GQA ratio 1..8 (two heads per 16-lane row group)");
  constexpr int D = kD;
  __shared__ float s_q[G][D];
  __shared__ __attribute__((aligned(16))) uint32_t s_qa[4][64][4];  // QK A operand [k-step][lane]
  __shared__ __attribute__((aligned(16))) uint8_t s_v[4][64 * kVP8];
  __shared__ __attribute__((aligned(16))) _Float16 s_p[4][64 * kPP];
  __shared__ float s_wm[4][G], s_wl[4][G];
  __shared__ int s_tbl[kMaxSplitBlocks];
  static_assert(sizeof(float) * 4 * G * D <= sizeof(s_v), "s_wacc fits in s_v");
  float (*s_wacc)[G][D] = reinterpret_cast<float (*)[G][D]>(&s_v[0][0]);  // used after the token loop

  const int split = blockIdx.x, h = blockIdx.y, seq = blockIdx.z;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, la = l >> 4, lj = l & 15;
  const int ns = a.plan.n_splits;
  const int len = a.seq_lens[seq];
  const int nblk = (len + kRows - 1) / kRows;
  int b0, b1;
  split_range(split, ns, nblk, b0, b1);
  const int nchunk = max(b1 - b0, 0);
  const uint8_t* pool_h = a.pool + (size_t)h * g.tile_bytes;
  const size_t tstride = (size_t)g.H * g.tile_bytes;

  if (nchunk == 0) {
    if (ns == 1) {
      for (int jj = 0; jj < G; ++jj)
        finalize_head<D, 256>(g, a, seq, h * G + jj, len, 0, kNegInf, 0.0f, 0.0f, tid, &s_q[0][0]);
    } else {
      if (tid < G) {
        s_wm[0][tid] = kNegInf;
        s_wl[0][tid] = 0.0f;
      }
      for (int i = tid; i < G * D; i += 256) s_wacc[1][i / D][i % D] = 0.0f;
      __syncthreads();
      splitk_arrive<D, G>(g, a, seq, h, split, ns, len, tid, &s_wm[0][0], &s_wl[0][0], &s_wacc[1][0][0],
                          &s_wacc[0][0][0]);
    }
    return;
  }

  for (int i = tid; i < nchunk; i += 256) s_tbl[i] = a.block_table[(size_t)seq * a.max_blocks_per_seq + b0 + i];
  __syncthreads();

  // on: false for a chunk past the split's end, whose loads the loop still issues (it has no exit between
  // chunks): they go through a zero-byte buffer resource, return zeros at once and fetch nothing.
  auto load = [&](RawF& r, int i, bool on = true) __attribute__((always_inline)) {
    const int phys = __builtin_amdgcn_readfirstlane(s_tbl[i]);
    const uint8_t* tile = pool_h + (size_t)phys * tstride;
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(tile), (short)0, on ? (int)g.tile_bytes : 0, kBufWord3);
    uint32_t live = 0;
#pragma unroll
    for (int c = 0; c < 4; ++c) live |= ((b0 + i) * kRows + 64 * w + 16 * c + lj < len) ? (1u << c) : 0u;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t off = (uint32_t)(64 * w + 8 * j + 2 * la + (lj >> 3)) * (uint32_t)g.rec + (lj & 7) * 16;
      r.k[j] = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, kBufNT);
      r.v[j] = __builtin_amdgcn_raw_buffer_load_b128(rs, off + D, 0, kBufNT);
    }
    r.live = live;
  };

  RawF ra, rb;
  load(ra, 0);

  // ------------------------------------------------------------ query: scale, rotation, A operand
  for (int i = tid; i < G * D; i += 256)
    s_q[i / D][i % D] = h2f(a.q[((size_t)seq * a.num_q_heads + h * G + i / D) * D + i % D]) * a.q_scale;
  for (int i = tid; i < 4 * 64 * kPP; i += 256) (&s_p[0][0])[i] = (_Float16)0.0f;
  __syncthreads();
  if (g.rotate) {
    for (int hs = 1; hs < D; hs *= 2) {
      for (int i = tid; i < G * D / 2; i += 256) {
        const int j = i / (D / 2), pi = i % (D / 2);
        const int lo = (pi / hs) * 2 * hs + (pi % hs);
        const float x = s_q[j][lo], y = s_q[j][lo + hs];
        s_q[j][lo] = x + y;
        s_q[j][lo + hs] = x - y;
      }
      __syncthreads();
    }
    for (int i = tid; i < G * D; i += 256) s_q[i / D][i % D] *= a.unrot_c;
    __syncthreads();
  }
  {
    // lane (la', lj') of k-step s: A[row lj'][k = 8 la' + e] = part(lj') of q[lj' / 2][32 la' + 8 s + e]
    const int s = tid >> 6, ln = tid & 63, lap = ln >> 4, ljp = ln & 15;
    const int hq = ljp >> 1, part = ljp & 1;
    uint32_t wv[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      _Float16 x[2];
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const float v = hq < G ? s_q[hq][32 * lap + 8 * s + 2 * p + k] : 0.0f;
        const _Float16 hi = (_Float16)v;
        x[k] = part ? (_Float16)(v - (float)hi) : hi;
      }
      wv[p] = pack_h2(x[0], x[1]);
    }
    *reinterpret_cast<u32x4*>(&s_qa[s][ln][0]) = u32x4{wv[0], wv[1], wv[2], wv[3]};
  }
  __syncthreads();
  u32x4 qa[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) qa[s] = *reinterpret_cast<const u32x4*>(&s_qa[s][l][0]);

  // lane (la, lj): heads 2 la + u (u = 0, 1) in MFMA rows 4 la + 2u + part
  const int h0 = 2 * la;
  const bool ok0 = h0 < G, ok1 = h0 + 1 < G;
  float m_run[2] = {kNegInf, kNegInf}, l_run[2] = {0.0f, 0.0f};
  floatx4 o[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) o[t] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
  uint8_t* sv = s_v[w];
  _Float16* sp = s_p[w];

  auto process = [&](const RawF& r) __attribute__((always_inline)) {
    // K halves through the row slots of the V staging area into the lane-per-token layout (tokens 16c + lj,
    // channels 32 la .. 32 la + 31), then the V halves into the same slots (the wave's LDS operations run in
    // order: the K reads are done before the V writes land)
    const int srow = 2 * la + (lj >> 3), spc = (lj & 7) * 16;
#pragma unroll
    for (int j = 0; j < 8; ++j) *reinterpret_cast<u32x4*>(sv + (8 * j + srow) * kVP8 + spc) = r.k[j];
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    u32x4 kt[4][2];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      kt[c][0] = *reinterpret_cast<const u32x4*>(sv + (16 * c + lj) * kVP8 + la * 32);
      kt[c][1] = *reinterpret_cast<const u32x4*>(sv + (16 * c + lj) * kVP8 + la * 32 + 16);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int j = 0; j < 8; ++j) *reinterpret_cast<u32x4*>(sv + (8 * j + srow) * kVP8 + spc) = r.v[j];
    // ---------------------------------------------------------- logits
    floatx4 acc[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[c] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const u32x4& kw = kt[c][s >> 1];
        const uint32_t w0 = kw[2 * (s & 1)], w1 = kw[2 * (s & 1) + 1];
        const u32x4 b = {e4m3_pair<false>(w0), e4m3_pair<true>(w0), e4m3_pair<false>(w1), e4m3_pair<true>(w1)};
        acc[c] = mfma16(qa[s], b, acc[c]);
      }
    }
    float sc[2][4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const bool live = (r.live >> c) & 1u;
      sc[0][c] = (live && ok0) ? acc[c][0] + acc[c][1] : kNegInf;
      sc[1][c] = (live && ok1) ? acc[c][2] + acc[c][3] : kNegInf;
    }
    // ---------------------------------------------------------- online softmax, two heads per lane
    float p[2][4];
    bool moved = false;
    float alpha[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      float mx = fmaxf(fmaxf(sc[u][0], sc[u][1]), fmaxf(sc[u][2], sc[u][3]));
      mx = row_max16(mx);
      const float mnew = fmaxf(m_run[u], mx);
      alpha[u] = mnew == m_run[u] ? 1.0f : __builtin_amdgcn_exp2f(m_run[u] - mnew);
      moved |= alpha[u] != 1.0f;
      float ps = 0.0f;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        p[u][c] = __builtin_amdgcn_exp2f(sc[u][c] - mnew);
        p[u][c] = mnew == kNegInf ? 0.0f : p[u][c];
        ps += p[u][c];
      }
      l_run[u] = l_run[u] * alpha[u] + ps;
      m_run[u] = mnew;
    }
    if (__builtin_amdgcn_ballot_w64(moved)) {
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        o[t][0] *= alpha[0];
        o[t][1] *= alpha[0];
        o[t][2] *= alpha[1];
        o[t][3] *= alpha[1];
      }
    }
    // ---------------------------------------------------------- p (hi, lo) to LDS, position = token
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const _Float16 a0 = (_Float16)p[0][c], a1 = (_Float16)p[1][c];
      uint2 wv;
      wv.x = pack_h2(a0, (_Float16)(p[0][c] - (float)a0));
      wv.y = pack_h2(a1, (_Float16)(p[1][c] - (float)a1));
      if (ok0) *reinterpret_cast<uint2*>(&sp[(16 * c + lj) * kPP + la * 4]) = wv;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // ---------------------------------------------------------- PV
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int base = 32 * kb + 8 * la + (lj >> 2);
      const v2i x0 = lds_tr16(&sp[base * kPP + (lj & 3) * 4]);
      const v2i x1 = lds_tr16(&sp[(base + 4) * kPP + (lj & 3) * 4]);
      const u32x4 pa = {(uint32_t)x0.x, (uint32_t)x0.y, (uint32_t)x1.x, (uint32_t)x1.y};
      const int tok = 32 * kb + 8 * la + (lj >> 1);
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        // channel 16 t + lj of tokens 32 kb + 8 la .. +7, in token order
        const v2i x = lds_tr8(sv + tok * kVP8 + 16 * t + 8 * (lj & 1));
        const u32x4 b = {e4m3_pair<false>((uint32_t)x.x), e4m3_pair<true>((uint32_t)x.x),
                         e4m3_pair<false>((uint32_t)x.y), e4m3_pair<true>((uint32_t)x.y)};
        o[t] = mfma16(pa, b, o[t]);
      }
    }
    __builtin_amdgcn_wave_barrier();
  };

  // Whole pairs with no exit in between (an exit there gives the compiler a path into the loop head on which
  // it waits for every load in flight before issuing the next chunk's); past the end the loads read nothing.
  int i = 0;
  for (; i + 1 < nchunk; i += 2) {
    load(rb, i + 1);
    __builtin_amdgcn_sched_barrier(0);
    process(ra);
    load(ra, min(i + 2, nchunk - 1), i + 2 < nchunk);
    __builtin_amdgcn_sched_barrier(0);
    process(rb);
  }
  if (i < nchunk) process(ra);
  lds_barrier();  // the waves' LDS work is done (nothing else is exchanged through memory here)

  // ---------------------------------------------------------------- merge the four waves
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int hq = h0 + u;
    const float lt = row_sum16(l_run[u]);
    if (hq < G) {
      if (lj == 0) {
        s_wm[w][hq] = m_run[u];
        s_wl[w][hq] = lt;
      }
#pragma unroll
      for (int t = 0; t < 8; ++t) s_wacc[w][hq][16 * t + lj] = o[t][2 * u] + o[t][2 * u + 1];
    }
  }
  __syncthreads();
  if (ns == 1) {
    __shared__ float s_o[D];
    for (int jj = 0; jj < G; ++jj) {
      float M = kNegInf;
#pragma unroll
      for (int ww = 0; ww < 4; ++ww) M = fmaxf(M, s_wm[ww][jj]);
      float acc = 0.0f, L = 0.0f;
      if (M != kNegInf) {
#pragma unroll
        for (int ww = 0; ww < 4; ++ww) {
          const float sc_w = exp2f(s_wm[ww][jj] - M);
          if (tid < D) acc += s_wacc[ww][jj][tid] * sc_w;
          L += s_wl[ww][jj] * sc_w;
        }
      }
      finalize_head<D, 256>(g, a, seq, h * G + jj, len, 0, M, L, acc, tid, s_o);
    }
    return;
  }
  __shared__ float s_pm[G], s_pl[G];
  __shared__ float s_pacc[G][D];
  for (int i = tid; i < G * D; i += 256) {
    const int jj = i / D, c = i % D;
    float M = kNegInf;
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) M = fmaxf(M, s_wm[ww][jj]);
    float acc = 0.0f, L = 0.0f;
    if (M != kNegInf) {
#pragma unroll
      for (int ww = 0; ww < 4; ++ww) {
        const float sc_w = exp2f(s_wm[ww][jj] - M);
        acc += s_wacc[ww][jj][c] * sc_w;
        L += s_wl[ww][jj] * sc_w;
      }
    }
    s_pacc[jj][c] = acc;
    if (c == 0) {
      s_pm[jj] = M;
      s_pl[jj] = L;
    }
  }
  __syncthreads();
  splitk_arrive<D, G>(g, a, seq, h, split, ns, len, tid, s_pm, s_pl, &s_pacc[0][0], &s_wacc[0][0][0]);
}

}  // namespace

// FP8 pools with head_dim 128 and G = 1..8, without a sentinel mask (masked FP8 calls take the generic kernel).
bool decode_fp8_supported(const TileGeom& g, int G) {
  return g.fp8 && g.d == 128 && g.dv == 128 && G >= 1 && G <= 8;
}

hipError_t launch_decode_fp8(const TileGeom& g, const DecodeArgs& a, hipStream_t stream) {
  const dim3 grid(a.plan.n_splits, g.H, a.n_seqs);
  switch (a.G) {
#define KVQ_FP8_CASE(GG) \
  case GG: hipLaunchKernelGGL((decode_fp8_k<GG>), grid, dim3(256), 0, stream, g, a); break;
    KVQ_FP8_CASE(1)
    KVQ_FP8_CASE(2)
    KVQ_FP8_CASE(3)
    KVQ_FP8_CASE(4)
    KVQ_FP8_CASE(5)
    KVQ_FP8_CASE(6)
    KVQ_FP8_CASE(7)
    KVQ_FP8_CASE(8)
#undef KVQ_FP8_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace kvq
