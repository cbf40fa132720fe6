// kvq_decode_mfma_common.hpp - matrix-core helpers shared by the decode kernels: MFMA and DPP wrappers,
// and the in-kernel split-K merge (the split that arrives last merges every split's partials).
#pragma once

#include "kvq_decode_common.hpp"

namespace kvq {
namespace dec {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Buffer resources for raw (untyped) loads on gfx950: the descriptor's fourth word with a 32-bit data format
// (a zero format would make every load return zeros), and the cache-policy operand of a non-temporal load.
// A raw load at an offset at or past the resource's size returns zeros without a memory access.
constexpr int kBufWord3 = 0x00020000;
constexpr int kBufNT = 2;

__device__ __forceinline__ floatx4 mfma16(const u32x4& a, const u32x4& b, const floatx4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, a), __builtin_bit_cast(half8, b), c,
                                                0, 0, 0);
}

__device__ __forceinline__ uint32_t pack_h2(_Float16 lo, _Float16 hi) {
  return (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
}

// Row (16-lane) reductions via DPP row rotations: every lane of the row ends with the result.
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xf, 0xf, false));
}
__device__ __forceinline__ float row_max16(float v) {
  v = fmaxf(v, dpp<0x128>(v));
  v = fmaxf(v, dpp<0x124>(v));
  v = fmaxf(v, dpp<0x122>(v));
  v = fmaxf(v, dpp<0x121>(v));
  return v;
}
__device__ __forceinline__ float row_sum16(float v) {
  v += dpp<0x128>(v);
  v += dpp<0x124>(v);
  v += dpp<0x122>(v);
  v += dpp<0x121>(v);
  return v;
}

constexpr float kTwo24 = 16777216.0f;

// Workgroup barrier for LDS traffic only: the fences are limited to the local address space, so the
// barrier waits for this wave's LDS operations but not for its outstanding global loads (__syncthreads
// waits for those too, which would drain every prefetch in flight). Not for code with DMA into LDS
// pending (the local fence then waits for the DMA).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Sum and maximum over the four lanes l, l ^ 16, l ^ 32, l ^ 48 (one query row) with the gfx950 row and
// half-wave swaps; every lane ends with the same value.
__device__ __forceinline__ float rows4_max(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float rows4_sum(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Wave-uniform power-of-two scale for the fp16 p * v_scale operands of one chunk, from the chunk's largest
// V scale vmax (this lane's value; reduced over the wave here): with p <= 1 every p * v_scale * scale is
// below 2^15, and the weights that matter stay far above the fp16 subnormal range instead of flushing to
// zero (a flushed product would drop the token's code term but keep its zero-point term). Returns the
// scale and sets inv to its inverse; both are exact powers of two.
__device__ __forceinline__ float chunk_pv_scale(float vmax, float& inv) {
  vmax = fmaxf(vmax, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(vmax), 0x128, 0xf, 0xf, false)));
  vmax = fmaxf(vmax, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(vmax), 0x124, 0xf, 0xf, false)));
  vmax = fmaxf(vmax, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(vmax), 0x122, 0xf, 0xf, false)));
  vmax = fmaxf(vmax, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(vmax), 0x121, 0xf, 0xf, false)));
  vmax = rows4_max(vmax);  // across the four rows: lane swaps, no LDS round trip
  const int ex = vmax > 0.0f ? ((__float_as_int(vmax) >> 23) & 0xff) - 126 : 0;  // vmax < 2^ex
  inv = __builtin_amdgcn_ldexpf(1.0f, ex - 15);
  return __builtin_amdgcn_ldexpf(1.0f, 15 - ex);
}
constexpr int kMaxSplitBlocks = 512;  // blocks one workgroup may own (its table slice is staged in LDS)
constexpr int kMaxSplits = 64;        // splits per (sequence, KV head)
constexpr float kTwo20 = 1048576.0f;

// Stages into s_tbl, in order, the block-table entries phys(i) of the columns 0 <= i < n for which keep(i)
// holds, and into s_idx their column indices (both evaluated by thread i mod 64 NW, all 64 NW threads of
// the workgroup taking part); returns their number. s_cnt: NW ints of scratch.
template <int NW = 4, class Idx, class Keep, class Phys>
__device__ int stage_columns(int n, int tid, int* s_tbl, Idx* s_idx, int* s_cnt, Keep keep, Phys phys) {
  const int w = tid >> 6, lane = tid & 63;
  int total = 0;
  for (int base = 0; base < n; base += 64 * NW) {
    const int i = base + tid;
    const bool k = i < n && keep(i);
    const int e = k ? phys(i) : 0;
    const uint64_t m = __builtin_amdgcn_ballot_w64(k);
    if (lane == 0) s_cnt[w] = __builtin_popcountll(m);
    __syncthreads();
    int off = total;
    for (int ww = 0; ww < w; ++ww) off += s_cnt[ww];
    if (k) {
      const int o = off + __builtin_popcountll(m & ((1ull << lane) - 1ull));
      s_tbl[o] = e;
      s_idx[o] = (Idx)i;
    }
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) total += s_cnt[ww];
    __syncthreads();
  }
  return total;
}

// Split-K arrival for split `split` of the `ns` splits of (seq, h) once its partials (m, l, acc[d]) per query head are
// ready: thread jj * D + c (and ml for c == 0) holds them in part_m / part_l / part_acc. The partials are
// written with relaxed agent-scope atomic stores, which compile to cache-coherent (sc1) stores, so no
// L2 write-back is needed; every thread waits for its stores to complete before the barrier, then one
// thread bumps the unit's arrival counter. The split that arrives last reads all partials back with
// agent-scope atomic loads (sc1, coherent across XCDs), merges them in split order - so the result does
// not depend on which split that is - finalises the output and resets the counter to zero. The merge also
// takes the n_pre partials that the cascade kernel left in the last n_pre slots of each row (earlier in
// stream order, so plain loads see them); those carry no arrival.
// An agent-scope release on the counter increment would make the hand-over an ordering of the memory model
// rather than of the stores' coherence, but on gfx950 it compiles to an L2 write-back (buffer_wbl2) in every
// workgroup, which made the 12 x 8K call 36 % slower (33 -> 45 us). The partials are agent-scope atomic
// stores, coherent across the XCDs by themselves, and each is acknowledged before the increment.
template <int D, int G>
__device__ inline void splitk_arrive(const TileGeom& g, const DecodeArgs& a, int seq, int h, int split, int ns, int len,
                              int tid, const float* part_m, const float* part_l, const float* part_acc, float* s_o,
                              int n_pre = 0) {
  __shared__ int s_last;
  __shared__ int s_cnt[4];
  const int st = a.plan.stride;
  // A unit with one split merges its own partials (still in LDS) with the n_pre earlier ones directly: no
  // store, arrival or reload.
  const bool local = ns == 1;
  if (!local) {
  for (int i = tid; i < G * D; i += 256) {
    const int jj = i / D, c = i % D;
    const size_t pi = ((size_t)seq * a.num_q_heads + h * G + jj) * st + split;
    __hip_atomic_store(&a.ws_acc[pi * D + c], part_acc[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (c == 0) {
      __hip_atomic_store(&a.ws_ml[2 * pi], part_m[jj], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&a.ws_ml[2 * pi + 1], part_l[jj], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  __builtin_amdgcn_s_waitcnt(0);  // this thread's partial stores have completed
  __syncthreads();
  if (tid == 0) {
    unsigned* ctr = a.ws_ctr + (size_t)seq * g.H + h;
    const unsigned prev = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = prev == (unsigned)(ns - 1);
    if (s_last) __hip_atomic_store(ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  if (!s_last) return;
  }
  // Merge: thread (head jj, channel c) for each of its NI items (jj, c) reads (m, l) and the accumulator of
  // up to KB splits at a time - the loads of all its items in one round - and folds them into a running
  // (M, L, o); the merged rows go through LDS to the finalisation, which wants channel c of one head in
  // thread c.
  __shared__ float s_hM[G], s_hL[G];
  float* s_merged = const_cast<float*>(part_acc);  // this split's own partials are no longer needed
  constexpr int NI = (G * D + 255) / 256;
  constexpr int KB = 8;
  float M[NI], L[NI], o[NI];
  size_t p0[NI];
  int cc[NI];
#pragma unroll
  for (int j = 0; j < NI; ++j) {
    const int i = min(tid + 256 * j, G * D - 1);
    const int jj = i / D;
    cc[j] = i % D;
    p0[j] = ((size_t)seq * a.num_q_heads + h * G + jj) * st;
    M[j] = kNegInf;
    L[j] = 0.0f;
    o[j] = 0.0f;
    if (local && part_l[jj] > 0.0f) {
      M[j] = part_m[jj];
      L[j] = part_l[jj];
      o[j] = part_acc[i];
    }
  }
  // merged index k: split k (k < ns), then the earlier partials in slots k + pre0; with a local split
  // only the earlier partials, in slots st - n_pre + k
  const int nt = local ? n_pre : ns + n_pre, pre0 = st - n_pre - ns;
  for (int base = 0; base < nt; base += KB) {
    float mi[NI][KB], li[NI][KB], xi[NI][KB];
#pragma unroll
    for (int k = 0; k < KB; ++k) {
      const int kk = min(base + k, nt - 1);
      const int sp = local ? st - n_pre + kk : kk < ns ? kk : kk + pre0;
#pragma unroll
      for (int j = 0; j < NI; ++j) {
        li[j][k] = __hip_atomic_load(&a.ws_ml[2 * (p0[j] + sp) + 1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        mi[j][k] = __hip_atomic_load(&a.ws_ml[2 * (p0[j] + sp)], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        xi[j][k] = __hip_atomic_load(&a.ws_acc[(p0[j] + sp) * D + cc[j]], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      float mb = M[j];
#pragma unroll
      for (int k = 0; k < KB; ++k)
        if (base + k < nt && li[j][k] > 0.0f) mb = fmaxf(mb, mi[j][k]);
      if (mb == kNegInf) continue;
      const float r = M[j] == kNegInf ? 0.0f : exp2f(M[j] - mb);
      L[j] *= r;
      o[j] *= r;
#pragma unroll
      for (int k = 0; k < KB; ++k) {
        if (base + k < nt && li[j][k] > 0.0f) {  // splits without live rows left their accumulators unwritten
          const float wgt = exp2f(mi[j][k] - mb);
          L[j] += li[j][k] * wgt;
          o[j] += xi[j][k] * wgt;
        }
      }
      M[j] = mb;
    }
  }
#pragma unroll
  for (int j = 0; j < NI; ++j) {
    const int i = tid + 256 * j;
    if (i < G * D) {
      s_merged[i] = o[j];
      if (cc[j] == 0) {
        s_hM[i / D] = M[j];
        s_hL[i / D] = L[j];
      }
    }
  }
  __syncthreads();
  const int n_sent = count_sentinels<256>(a, seq, len, tid, s_cnt);
  for (int jj = 0; jj < G; ++jj)
    finalize_head<D, 256>(g, a, seq, h * G + jj, len, n_sent, s_hM[jj], s_hL[jj], tid < D ? s_merged[jj * D + tid] : 0.0f,
                          tid, s_o);
}

}  // namespace dec
}  // namespace kvq
