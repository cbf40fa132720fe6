// kvq_quantize.hip - group-wise Q4 (and per-token Q8) quantisation of K/V rows into 256-token tiles.
//
// Follows "Agent Memory Below the Prompt" (technical summary 2.1: 256-token blocks, codes packed in
// uint32 words, one 16-bit scale and bias per group; 2.1 item 4: extending a cache row by row), the
// UltraQuant article (technology section: Walsh-Hadamard rotation first, K and V grouped differently)
// and QKVShare (methodology: width chosen per token). Every arithmetic step is a single IEEE fp32
// operation in a fixed order, so codes and fp16 parameters are reproducible bit for bit:
//   rotation: butterflies (a + b, a - b) with strides 1, 2, 4 inside a lane, then 8, 16, ... across lanes
//             (lane xor 1, 2, ...), then one multiply by c = fp32(1/sqrt(d));
//   group:    mn, mx (zero extremes canonicalised to +0), scale = fp16((mx - mn) / L), zero = fp16(mn),
//             r = 1 / fp32(scale), code = clamp(rint((x - fp32(zero)) * r), 0, L).
// FMA contraction is disabled for this file (contraction would change the rounding of those steps).
#pragma clang fp contract(off)

#include <type_traits>

#include "kvq_internal.hpp"

namespace kvq {
namespace {

__device__ __forceinline__ float h2f(uint32_t bits16) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
}
// fp32 -> fp16 bits, rounded from the fp32 value. The empty asm makes f an opaque fp32 register: otherwise the
// compiler may fuse the conversion into the fma that produced f (v_fma_mixlo_f16 rounds once, straight to
// fp16), which differs from rounding the fp32 result.
__device__ __forceinline__ uint32_t f2h(float f) {
  __asm__("" : "+v"(f));
  return __builtin_bit_cast(uint16_t, (_Float16)f);
}

// Eight consecutive fp16 values (one 16-byte load) -> fp32.
__device__ __forceinline__ void load8(const uint16_t* p, float (&x)[8]) {
  uint4 raw = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = h2f(w[i] & 0xffffu);
    x[2 * i + 1] = h2f(w[i] >> 16);
  }
}

// v of lane (this lane ^ m), m a power of two below 64: DPP moves inside a 16-lane row for m = 1, 2, 4, 8
// (m = 4 as the quad reversal followed by the half-row mirror, (i ^ 3) ^ 7 = i ^ 4 within eight lanes),
// so the rotations' and group reductions' exchanges stay on the VALU; a lane shuffle for m >= 16. The
// lanes exchanging values must be active (every caller runs these with its whole row group active).
__device__ __forceinline__ float lane_xor(float v, int m) {
  const int x = __float_as_int(v);
  switch (m) {
    case 1: return __int_as_float(__builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, false));  // quad_perm 1,0,3,2
    case 2: return __int_as_float(__builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, false));  // quad_perm 2,3,0,1
    case 4:
      return __int_as_float(__builtin_amdgcn_mov_dpp(__builtin_amdgcn_mov_dpp(x, 0x1B, 0xF, 0xF, false), 0x141,
                                                     0xF, 0xF, false));  // quad_perm 3,2,1,0; row_half_mirror
    case 8: return __int_as_float(__builtin_amdgcn_mov_dpp(x, 0x128, 0xF, 0xF, false));  // row_ror 8
    default: return __shfl_xor(v, m);
  }
}

// Min and max over the gl lanes of a group (gl a power of two, at most MAXL): every exchange width up to
// MAXL is issued with its width known to the compiler and applied where it lies below gl, so the DPP
// exchanges need no branch on the runtime group width (widths of 16 lanes and more take a lane shuffle
// behind a uniform branch).
template <int MAXL>
__device__ __forceinline__ void group_minmax(float& mn, float& mx, int gl) {
#pragma unroll
  for (int m = 1; m < MAXL; m *= 2) {
    if (m >= 16) {
      if (m < gl) {
        mn = fminf(mn, __shfl_xor(mn, m));
        mx = fmaxf(mx, __shfl_xor(mx, m));
      }
    } else {
      const float a = lane_xor(mn, m), b = lane_xor(mx, m);
      mn = m < gl ? fminf(mn, a) : mn;
      mx = m < gl ? fmaxf(mx, b) : mx;
    }
  }
}

// The scale before rounding, (mx - mn) / L for L = 3, 15 or 255 levels: the product with c = fp32(1/L) and one
// remainder correction. For these three divisors this equals the IEEE quotient for every non-negative finite
// fp32 dividend (an exhaustive comparison with the division over all 2^31 such values), in three
// instructions where the division takes about ten.
__device__ __forceinline__ float div_levels(float x, int bits) {
  const float L = bits == 8 ? 255.0f : bits == 2 ? 3.0f : 15.0f;
  const float c = bits == 8 ? 0x1.010102p-8f : bits == 2 ? 0x1.555556p-2f : 0x1.111112p-4f;
  const float q0 = x * c;
  const float r = __builtin_fmaf(-q0, L, x);
  return __builtin_fmaf(r, c, q0);
}

// 1 / s for a stored fp16 scale s > 0: the hardware reciprocal (within one ulp of 1 / s) and one Newton
// correction. For every positive fp16 value and any start within two ulps of 1 / s the result is the IEEE
// quotient (an exhaustive comparison over the 31743 values and five starts each).
__device__ __forceinline__ float rcp_scale(float s) {
  const float r0 = __builtin_amdgcn_rcpf(s);
  const float e = __builtin_fmaf(-s, r0, 1.0f);
  return __builtin_fmaf(e, r0, r0);
}

// y = c * H * x for one row spread over LPR lanes, lane li holding elements li*8 .. li*8+7.
template <int LPR>
__device__ __forceinline__ void rotate_row(float (&x)[8], int li, float c) {
#pragma unroll
  for (int h = 1; h < 8; h *= 2) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if ((i & h) == 0) {
        float a = x[i], b = x[i + h];
        x[i] = a + b;
        x[i + h] = a - b;
      }
    }
  }
#pragma unroll
  for (int m = 1; m < LPR; m *= 2) {
    const bool upper = (li & m) != 0;  // this lane holds the second element of each pair
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float p = lane_xor(x[i], m);
      x[i] = upper ? (p - x[i]) : (x[i] + p);
    }
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) x[i] = x[i] * c;
}

// Quantise this lane's 8 values as part of a group spanning gl lanes (gl a power of two dividing the
// row's lanes). Returns the 8 codes; every lane of the group gets the same packed {scale, zero}.
template <int MAXL>
__device__ __forceinline__ void quantize8(const float (&x)[8], int gl, int bits, uint32_t (&code)[8],
                                          uint32_t& param) {
  float mn = x[0], mx = x[0];
#pragma unroll
  for (int i = 1; i < 8; ++i) {
    mn = fminf(mn, x[i]);
    mx = fmaxf(mx, x[i]);
  }
  group_minmax<MAXL>(mn, mx, gl);
  mn = mn + 0.0f;  // a -0 extreme becomes +0
  mx = mx + 0.0f;
  const float L = bits == 8 ? 255.0f : bits == 2 ? 3.0f : 15.0f;
  const float s32 = div_levels(mx - mn, bits);
  const uint32_t sh = f2h(s32), zh = f2h(mn);
  param = sh | (zh << 16);
  const float s = h2f(sh), z = h2f(zh);
  if (s == 0.0f) {
#pragma unroll
    for (int i = 0; i < 8; ++i) code[i] = 0;
    return;
  }
  const float r = rcp_scale(s);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float t = x[i] - z;
    float u = t * r;
    float qv = __builtin_rintf(u);
    qv = fminf(fmaxf(qv, 0.0f), L);
    code[i] = (uint32_t)qv;
  }
}

// Store one lane's share of a code row (8 codes): 2-bit codes as one uint16 (lowest bits first), 4-bit codes
// as one uint32 (low nibble first), 8-bit codes as two. With tail > 0 (the V row of a row narrower than the
// pool's widest) the row's lanes also zero the tail bytes of the record after the row.
__device__ __forceinline__ void store_codes(uint8_t* row, int li, int lpr, int bits, int tail,
                                            const uint32_t (&code)[8]) {
  if (bits == 8) {
    uint2 w;
    w.x = code[0] | (code[1] << 8) | (code[2] << 16) | (code[3] << 24);
    w.y = code[4] | (code[5] << 8) | (code[6] << 16) | (code[7] << 24);
    *reinterpret_cast<uint2*>(row + li * 8) = w;
  } else if (bits == 4) {
    uint32_t w = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) w |= code[i] << (4 * i);
    *reinterpret_cast<uint32_t*>(row + li * 4) = w;
  } else {
    uint32_t w = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) w |= code[i] << (2 * i);
    *reinterpret_cast<uint16_t*>(row + li * 2) = (uint16_t)w;
  }
  if (tail > 0) {
    // the record's rest starts 4-byte aligned ((d + dv) * bits / 8 bytes in) and holds tail / 4 words: the
    // row's lanes zero them in turn
    uint32_t* z = reinterpret_cast<uint32_t*>(row + lpr * bits);
    for (int q = li; q < tail / 4; q += lpr) z[q] = 0u;
  }
}

// FP8 E4M3 bytes of a lane's 8 values (the FP8 pool format): the hardware conversion rounds to nearest
// even; clamping to +-448 first makes larger magnitudes saturate to the largest finite value.
__device__ __forceinline__ uint2 to_e4m3x8(const float (&x)[8]) {
  float c[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) c[i] = fminf(fmaxf(x[i], -448.0f), 448.0f);
  int lo = __builtin_amdgcn_cvt_pk_fp8_f32(c[0], c[1], 0, false);
  lo = __builtin_amdgcn_cvt_pk_fp8_f32(c[2], c[3], lo, true);
  int hi = __builtin_amdgcn_cvt_pk_fp8_f32(c[4], c[5], 0, false);
  hi = __builtin_amdgcn_cvt_pk_fp8_f32(c[6], c[7], hi, true);
  return uint2{(uint32_t)lo, (uint32_t)hi};
}

// One FP8 row of one tensor: optional rotation, then one byte per channel.
template <int LPR>
__device__ __forceinline__ void fp8_token_row(const TileGeom& g, float (&x)[8], int li, uint8_t* row, float rot_c) {
  if (g.rotate) rotate_row<LPR>(x, li, rot_c);
  *reinterpret_cast<uint2*>(row + li * 8) = to_e4m3x8(x);
}

// One row of one tensor (K or V) with per-token groups of grp channels, at width bits (2, 4, 8 or 16; a
// 16-bit row is the fp16 rounding of its values, with zero parameters); tail as for store_codes.
template <int LPR>
__device__ __forceinline__ void quantize_token_row(const TileGeom& g, float (&x)[8], int li, int grp, int bits,
                                                   int tail, uint8_t* code_row, uint8_t* param_row,
                                                   float rot_c) {
  if (g.rotate) rotate_row<LPR>(x, li, rot_c);
  const int gl = grp / 8;
  if (bits == 16) {
    uint4 o;
    o.x = f2h(x[0]) | (f2h(x[1]) << 16);
    o.y = f2h(x[2]) | (f2h(x[3]) << 16);
    o.z = f2h(x[4]) | (f2h(x[5]) << 16);
    o.w = f2h(x[6]) | (f2h(x[7]) << 16);
    *reinterpret_cast<uint4*>(code_row + li * 16) = o;
    if ((li & (gl - 1)) == 0) reinterpret_cast<uint32_t*>(param_row)[li / gl] = 0u;
    return;
  }
  uint32_t code[8];
  uint32_t param;
  quantize8<LPR>(x, gl, bits, code, param);
  store_codes(code_row, li, LPR, bits, tail, code);
  if ((li & (gl - 1)) == 0) reinterpret_cast<uint32_t*>(param_row)[li / gl] = param;
}

// Grid (n_blocks, H, n_tensors): one workgroup writes the 256 rows of tensor (blockIdx.z + kv_base) of
// tile (block_ids[blockIdx.x], blockIdx.y); LPR = d / 8 lanes per row, 256 / LPR rows per pass.
template <int LPR>
__global__ __launch_bounds__(256) void quantize_rows_k(TileGeom g, uint8_t* __restrict__ pool,
                                                       const int32_t* __restrict__ block_ids,
                                                       const uint16_t* __restrict__ k,
                                                       const uint16_t* __restrict__ v,
                                                       const uint32_t* __restrict__ prec_bits, float rot_c,
                                                       int kv_base) {
  constexpr int D = LPR * 8;
  constexpr int kRowsPerPass = 256 / LPR;
  const int i = blockIdx.x, h = blockIdx.y, kv = blockIdx.z + kv_base;
  const int li = threadIdx.x % LPR, r0 = threadIdx.x / LPR;
  uint8_t* tile = pool + ((size_t)block_ids[i] * g.H + h) * g.tile_bytes;
  const uint16_t* src = (kv ? v : k) + ((size_t)i * kRows * g.H + h) * D + li * 8;
  const int grp = kv ? g.vg : g.kg;
  const uint32_t* bitmap = prec_bits ? prec_bits + (size_t)i * (g.header_bytes() / 4) : nullptr;
  // (with d = 192, 24 lanes per row, the last 16 threads hold no row)
  for (int t = r0 < kRowsPerPass ? r0 : kRows; t < kRows; t += kRowsPerPass) {
    float x[8];
    load8(src + (size_t)t * g.H * D, x);
    if (g.fp8) {
      fp8_token_row<LPR>(g, x, li, tile + (kv ? g.vcode(t, 8) : g.kcode(t)), rot_c);
      continue;
    }
    const int bits = g.mixed == 2 ? (2 << (bitmap ? (bitmap[t >> 4] >> (2 * (t & 15))) & 3u : 1u))
                                  : (bitmap && ((bitmap[t >> 5] >> (t & 31)) & 1u)) ? 8 : 4;
    quantize_token_row<LPR>(g, x, li, grp, bits, kv && g.mixed ? g.rec - (g.d + g.dv) * bits / 8 : 0,
                            tile + (kv ? g.vcode(t, bits) : g.kcode(t)), tile + (kv ? g.vpar(t) : g.kpar(t)),
                            rot_c);
  }
  if (kv == 1) {
    // zero the tail padding (and write the width bitmap of mixed pools)
    const uint32_t end = g.off_hdr + g.header_bytes();
    for (uint32_t o = end + 4u * threadIdx.x; o < g.tile_bytes; o += 4u * blockDim.x)
      *reinterpret_cast<uint32_t*>(tile + o) = 0u;
    // width words (without them a mixed-2 pool's rows are 4-bit: code 1 in every field)
    if (g.mixed && threadIdx.x < g.header_bytes() / 4)
      reinterpret_cast<uint32_t*>(tile + g.off_hdr)[threadIdx.x] =
          bitmap ? bitmap[threadIdx.x] : (g.mixed == 2 ? 0x55555555u : 0u);
  }
}

// K grouped per channel over the block's 256 rows (always 4-bit), kKchanThreads threads per tile. Two passes
// over the rows: the first finds every column's min/max of the (rotated) values, the second encodes the same
// values against the column's parameters. A thread's rows (one lane of kRows / RPP rows) are all loaded at
// once. Where they fit (8 rows of 8 values: head dims up to 128) the rotated fp32 values stay in registers
// between the passes, so each row is converted and rotated once; otherwise the raw fp16 words stay and the
// second pass converts and rotates them again (the identical operations, so the identical values).
constexpr int kKchanThreads = 512;
template <int LPR>
__global__ __launch_bounds__(kKchanThreads) void quantize_kchan_k(TileGeom g, uint8_t* __restrict__ pool,
                                                                  const int32_t* __restrict__ block_ids,
                                                                  const uint16_t* __restrict__ k, float rot_c) {
  constexpr int D = LPR * 8;
  constexpr int RPP = kKchanThreads / LPR;  // rows per pass of the workgroup
  constexpr int NR = kRows / RPP;           // rows of one thread
  constexpr bool kHold = NR <= 8;           // rotated values held between the passes
  static_assert(RPP * LPR == kKchanThreads && NR * RPP == kRows, "a row's lanes divide the workgroup");
  __shared__ float s_min[RPP][D];
  __shared__ float s_max[RPP][D];
  __shared__ float s_z[D], s_r[D];
  __shared__ int s_zero_scale[D];
  const int i = blockIdx.x, h = blockIdx.y;
  const int li = threadIdx.x % LPR, r0 = threadIdx.x / LPR;
  uint8_t* tile = pool + ((size_t)block_ids[i] * g.H + h) * g.tile_bytes;
  const uint16_t* src = k + ((size_t)i * kRows * g.H + h) * D + li * 8;

  uint4 raw[NR];
#pragma unroll
  for (int j = 0; j < NR; ++j) raw[j] = *reinterpret_cast<const uint4*>(src + (size_t)(r0 + j * RPP) * g.H * D);
  auto row = [&](int j, float (&x)[8]) __attribute__((always_inline)) {
    const uint32_t w[4] = {raw[j].x, raw[j].y, raw[j].z, raw[j].w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[2 * e] = h2f(w[e] & 0xffffu);
      x[2 * e + 1] = h2f(w[e] >> 16);
    }
    if (g.rotate) rotate_row<LPR>(x, li, rot_c);
  };
  float held[kHold ? NR : 1][8];
  float cmin[8], cmax[8];
#pragma unroll
  for (int j = 0; j < NR; ++j) {
    float x[8];
    row(j, x);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      cmin[e] = j == 0 ? x[e] : fminf(cmin[e], x[e]);
      cmax[e] = j == 0 ? x[e] : fmaxf(cmax[e], x[e]);
      if constexpr (kHold) held[j][e] = x[e];
    }
    if constexpr (!kHold) __builtin_amdgcn_sched_barrier(0);  // one row's values live at a time
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    s_min[r0][li * 8 + e] = cmin[e];
    s_max[r0][li * 8 + e] = cmax[e];
  }
  __syncthreads();
  for (int c = threadIdx.x; c < D; c += blockDim.x) {
    float mn = s_min[0][c], mx = s_max[0][c];
    for (int r = 1; r < RPP; ++r) {
      mn = fminf(mn, s_min[r][c]);
      mx = fmaxf(mx, s_max[r][c]);
    }
    mn = mn + 0.0f;
    mx = mx + 0.0f;
    const float s32 = (mx - mn) / 15.0f;
    const uint32_t sh = f2h(s32), zh = f2h(mn);
    reinterpret_cast<uint32_t*>(tile + g.off_kch)[c] = sh | (zh << 16);
    const float s = h2f(sh);
    s_z[c] = h2f(zh);
    s_zero_scale[c] = s == 0.0f;
    s_r[c] = s == 0.0f ? 0.0f : 1.0f / s;
  }
  __syncthreads();
  if constexpr (!kHold) {
    // The second pass converts and rotates the raw words again; hiding their values from the compiler keeps
    // it from holding the first pass's converted rows live across the reduction instead (NR x 8 more
    // registers).
#pragma unroll
    for (int j = 0; j < NR; ++j) asm volatile("" : "+v"(raw[j].x), "+v"(raw[j].y), "+v"(raw[j].z), "+v"(raw[j].w));
  }
  float zc[8], rc[8];
  bool zs[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    zc[e] = s_z[li * 8 + e];
    rc[e] = s_r[li * 8 + e];
    zs[e] = s_zero_scale[li * 8 + e] != 0;
  }
#pragma unroll
  for (int j = 0; j < NR; ++j) {
    float x[8];
    if constexpr (kHold) {
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = held[j][e];
    } else {
      row(j, x);
    }
    uint32_t w = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      uint32_t code = 0;
      if (!zs[e]) {
        const float tt = x[e] - zc[e];
        const float u = tt * rc[e];
        float qv = __builtin_rintf(u);
        qv = fminf(fmaxf(qv, 0.0f), 15.0f);
        code = (uint32_t)qv;
      }
      w |= code << (4 * e);
    }
    reinterpret_cast<uint32_t*>(tile + g.kcode(r0 + j * RPP))[li] = w;
    if constexpr (!kHold) __builtin_amdgcn_sched_barrier(0);
  }
}

// Grid (n_seqs, H, tensors), LPR threads: row positions[s] % 256 of block block_table[s][positions[s] / 256];
// tensor kv_base + blockIdx.z (0 = K, 1 = V) of head dim D = 8 LPR.
template <int LPR>
__device__ __forceinline__ void append_row(const TileGeom& g, uint8_t* __restrict__ pool,
                                           const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
                                           const int32_t* __restrict__ block_table, int max_blocks_per_seq,
                                           const int32_t* __restrict__ positions, const uint8_t* __restrict__ prec,
                                           float rot_c, int kv, int li) {
  constexpr int D = LPR * 8;
  const int s = blockIdx.x, h = blockIdx.y;
  const int p = positions[s];
  const int row = p % kRows;
  const int blk = block_table[(size_t)s * max_blocks_per_seq + p / kRows];
  uint8_t* tile = pool + ((size_t)blk * g.H + h) * g.tile_bytes;
  const int pb = prec ? (int)prec[s] : 4;  // widths the pool does not hold are stored as 4-bit rows
  const int bits = (pb == 8 && g.mixed) || (g.mixed == 2 && (pb == 2 || pb == 16)) ? pb : 4;
  const int grp = kv ? g.vg : g.kg;
  float x[8];
  load8((kv ? v : k) + ((size_t)s * g.H + h) * D + li * 8, x);
  if (g.fp8) {
    fp8_token_row<LPR>(g, x, li, tile + (kv ? g.vcode(row, 8) : g.kcode(row)), rot_c);
    return;
  }
  quantize_token_row<LPR>(g, x, li, grp, bits, kv && g.mixed ? g.rec - (g.d + g.dv) * bits / 8 : 0,
                          tile + (kv ? g.vcode(row, bits) : g.kcode(row)), tile + (kv ? g.vpar(row) : g.kpar(row)),
                          rot_c);
  if (g.mixed == 1 && kv == 0 && li == 0) {
    uint32_t* word = reinterpret_cast<uint32_t*>(tile + g.off_hdr) + (row >> 5);
    const uint32_t bit = 1u << (row & 31);
    if (bits == 8) atomicOr(word, bit);
    else atomicAnd(word, ~bit);
  }
  if (g.mixed == 2 && kv == 0 && li == 0) {  // this row's 2-bit width code
    uint32_t* word = reinterpret_cast<uint32_t*>(tile + g.off_hdr) + (row >> 4);
    const int sh = 2 * (row & 15);
    const uint32_t code = bits == 2 ? 0u : bits == 4 ? 1u : bits == 8 ? 2u : 3u;
    atomicAnd(word, ~(3u << sh));
    atomicOr(word, code << sh);
  }
}

template <int LPR>
__global__ __launch_bounds__(LPR) void append_k(TileGeom g, uint8_t* __restrict__ pool,
                                                const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
                                                const int32_t* __restrict__ block_table, int max_blocks_per_seq,
                                                const int32_t* __restrict__ positions,
                                                const uint8_t* __restrict__ prec, float rot_c, int kv_base) {
  append_row<LPR>(g, pool, k, v, block_table, max_blocks_per_seq, positions, prec, rot_c, blockIdx.z + kv_base,
                  threadIdx.x);
}

// K and V rows of unequal head dims in one wave: K on lanes 0 .. LK - 1, V on lanes 32 .. 32 + LV - 1 (each
// row's lane exchanges stay inside its own lanes, which are the only active ones in its branch); one launch
// instead of one per tensor.
template <int LK, int LV>
__global__ __launch_bounds__(64) void append_pair_k(TileGeom g, uint8_t* __restrict__ pool,
                                                    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
                                                    const int32_t* __restrict__ block_table, int max_blocks_per_seq,
                                                    const int32_t* __restrict__ positions,
                                                    const uint8_t* __restrict__ prec, float rot_c, float rot_cv) {
  static_assert(LK <= 32 && LV <= 32, "each tensor's row within half a wave");
  const int l = threadIdx.x;
  if (l < LK)
    append_row<LK>(g, pool, k, v, block_table, max_blocks_per_seq, positions, prec, rot_c, 0, l);
  else if (l >= 32 && l < 32 + LV)
    append_row<LV>(g, pool, k, v, block_table, max_blocks_per_seq, positions, prec, rot_cv, 1, l - 32);
}

// y = c * H * x for one row spread over L16 lanes, lane li holding elements 16 li .. 16 li + 15: the butterflies
// of rotate_row in the same order (strides 1, 2, 4, 8 inside the lane, then 16, 32, ... across lanes), so the
// rotated values are the same bits. The exchanges are LDS lane shuffles here: with 16 values per lane they
// overlap the butterflies' VALU work better than DPP moves did (48 against 55 us per 256 blocks).
template <int L16>
__device__ __forceinline__ void rotate_row16(float (&x)[16], int li, float c) {
#pragma unroll
  for (int h = 1; h < 16; h *= 2) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if ((i & h) == 0) {
        const float a = x[i], b = x[i + h];
        x[i] = a + b;
        x[i + h] = a - b;
      }
    }
  }
#pragma unroll
  for (int m = 1; m < L16; m *= 2) {
    const bool upper = (li & m) != 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float p = __shfl_xor(x[i], m);
      x[i] = upper ? (p - x[i]) : (x[i] + p);
    }
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) x[i] = x[i] * c;
}

// Quantise this lane's 16 values at `bits` (2, 4 or 8) as part of a group spanning gl lanes: the same fp32
// operations per value as quantize8 (the clamp as one fmed3, which equals max then min for the non-NaN
// values here), so the same codes and parameters. Codes are packed into w low bits first (8-bit: four words,
// 4-bit: two, 2-bit: one): the codes of a byte are first combined exactly in fp32 (q0 + 16 q1, or q0 + 4 q1 +
// 16 q2 + 64 q3, integers below 256) and the byte placed with v_cvt_pk_u8_f32 (exact for such integers).
// The lane's extremes of 16 values, from the fp32 values, or (for values that are the stored fp16 inputs
// themselves) from the packed fp16 words two at a time: min and max are exact in either precision.
__device__ __forceinline__ void lane_extremes(const float (&x)[16], float& mn, float& mx) {
  mn = x[0];
  mx = x[0];
#pragma unroll
  for (int i = 1; i < 16; ++i) {
    mn = fminf(mn, x[i]);
    mx = fmaxf(mx, x[i]);
  }
}
__device__ __forceinline__ void lane_extremes_h(const uint32_t (&ww)[8], float& mn, float& mx) {
  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
  h2 lo = __builtin_bit_cast(h2, ww[0]), hi = lo;
#pragma unroll
  for (int e = 1; e < 8; ++e) {
    const h2 y = __builtin_bit_cast(h2, ww[e]);
    lo = __builtin_elementwise_min(lo, y);
    hi = __builtin_elementwise_max(hi, y);
  }
  mn = fminf((float)lo.x, (float)lo.y);
  mx = fmaxf((float)hi.x, (float)hi.y);
}

template <int MAXL>
__device__ __forceinline__ void quantize16(const float (&x)[16], float mn, float mx, int gl, int bits,
                                           uint32_t (&w)[4], uint32_t& param) {
  group_minmax<MAXL>(mn, mx, gl);
  mn = mn + 0.0f;  // a -0 extreme becomes +0
  mx = mx + 0.0f;
  const float L = bits == 8 ? 255.0f : bits == 2 ? 3.0f : 15.0f;
  const float s32 = div_levels(mx - mn, bits);
  const uint32_t sh = f2h(s32), zh = f2h(mn);
  param = sh | (zh << 16);
  const float s = h2f(sh), z = h2f(zh);
#pragma unroll
  for (int k = 0; k < 4; ++k) w[k] = 0u;
  if (s == 0.0f) return;
  const float r = rcp_scale(s);
  float q[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const float t = x[i] - z;
    const float u = t * r;
    q[i] = __builtin_amdgcn_fmed3f(__builtin_rintf(u), 0.0f, L);
  }
  if (bits == 8) {
#pragma unroll
    for (int i = 0; i < 16; ++i) w[i >> 2] = __builtin_amdgcn_cvt_pk_u8_f32(q[i], i & 3, w[i >> 2]);
  } else if (bits == 4) {
#pragma unroll
    for (int j = 0; j < 8; ++j)
      w[j >> 2] = __builtin_amdgcn_cvt_pk_u8_f32(__builtin_fmaf(q[2 * j + 1], 16.0f, q[2 * j]), j & 3, w[j >> 2]);
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float b = __builtin_fmaf(__builtin_fmaf(__builtin_fmaf(q[4 * j + 3], 4.0f, q[4 * j + 2]), 4.0f,
                                                    q[4 * j + 1]), 4.0f, q[4 * j]);
      w[0] = __builtin_amdgcn_cvt_pk_u8_f32(b, j, w[0]);
    }
  }
}

// quantize_rows_k with 16 values per lane (L16 = d / 16 lanes per row, 256 / L16 rows per pass) for pools with
// groups of 16 channels or more: rotation (ROT, rotate_row16) and per-token widths (MIX = the layout's mixed:
// {4, 8} or {2, 4, 8, FP16}) as compile-time variants, with the same codes, parameters, headers and zero
// padding. The per-row work (group extremes, the two divisions, addressing) is shared by twice as many values
// as with 8 per lane, and PF passes' rows are loaded while a pass is quantised. NT = 1: grid and output as
// quantize_rows_k (one tensor per workgroup). NT = 2: grid (n_blocks, H, 1), the workgroup quantises K and V of
// its tile, so each row record and parameter record is written whole by one wave (measured on the 12 x 8K
// pool: 133 -> 115 us per layer, the mixed workload 902 -> 705 us per 2048 blocks). Without rotation the
// lane's extremes come from the packed fp16 inputs (exact in fp16).
// The work of one 256-thread group (thread tid of nthr = 256) on tile (blockIdx.x, blockIdx.y): tensor kv0 (NT = 1)
// or both (NT = 2). No workgroup barrier, so two groups of one workgroup may run different instances.
template <int L16, bool ROT, int MIX, int NT, int PF>
__device__ __forceinline__ void rows16_tile(const TileGeom& g, uint8_t* __restrict__ pool,
                                            const int32_t* __restrict__ block_ids, const uint16_t* __restrict__ k,
                                            const uint16_t* __restrict__ v, const uint32_t* __restrict__ prec_bits,
                                            float rot_c, int kv0, int tid, int nthr) {
  constexpr int D = L16 * 16;
  constexpr int RPP = 256 / L16;                  // rows per pass (21 at L16 = 12: threads 252..255 idle)
  constexpr int NPASS = (kRows + RPP - 1) / RPP;  // passes (the last one partial at L16 = 12)
  static_assert(!ROT || (L16 & (L16 - 1)) == 0, "rotation needs a power-of-two head dim");
  static_assert(NT == 1 || NT == 2, "one tensor, or K and V of the tile");
  const int i = blockIdx.x, h = blockIdx.y;
  const int li = tid % L16, r0 = tid / L16;
  uint8_t* tile = pool + ((size_t)block_ids[i] * g.H + h) * g.tile_bytes;
  const uint32_t* bitmap = MIX && prec_bits ? prec_bits + (size_t)i * (g.header_bytes() / 4) : nullptr;
  // Rows past the block (the idle threads and the partial last pass when L16 does not divide 256) load the
  // block's last row instead, so every load is unconditional, and skip the work.
  auto row_ptr = [&](int kv, int t) {
    return (kv ? v : k) + ((size_t)i * kRows * g.H + h) * D + li * 16 + (size_t)min(t, kRows - 1) * g.H * D;
  };
  // PF passes' rows are in flight while one pass is quantised (a ring of PF + 1 register sets; the pass loop
  // is unrolled, so the ring indices are constants)
  uint4 buf[PF + 1][NT][2];
  auto issue = [&](uint4 (&b)[NT][2], int p) __attribute__((always_inline)) {
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      const uint16_t* rp = row_ptr(kv0 + n, r0 + p * RPP);
      b[n][0] = *reinterpret_cast<const uint4*>(rp);
      b[n][1] = *reinterpret_cast<const uint4*>(rp + 8);
    }
  };
  auto work = [&](const uint4 (&b)[NT][2], int p) __attribute__((always_inline)) {
    const int t = r0 + p * RPP;
    if (t >= kRows) return;
    int bits = 4;
    if constexpr (MIX == 2) bits = 2 << (bitmap ? (bitmap[t >> 4] >> (2 * (t & 15))) & 3u : 1u);
    if constexpr (MIX == 1) bits = (bitmap && ((bitmap[t >> 5] >> (t & 31)) & 1u)) ? 8 : 4;
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      const int kv = kv0 + n;
      const int gl = (kv ? g.vg : g.kg) / 16;
      float x[16];
      const uint32_t ww[8] = {b[n][0].x, b[n][0].y, b[n][0].z, b[n][0].w, b[n][1].x, b[n][1].y, b[n][1].z, b[n][1].w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        x[2 * e] = h2f(ww[e] & 0xffffu);
        x[2 * e + 1] = h2f(ww[e] >> 16);
      }
      if constexpr (ROT) rotate_row16<L16>(x, li, rot_c);
      uint8_t* row = tile + (kv ? g.vcode(t, bits) : g.kcode(t));
      uint32_t* prow = reinterpret_cast<uint32_t*>(tile + (kv ? g.vpar(t) : g.kpar(t)));
      if (MIX == 2 && bits == 16) {
        uint4 o0, o1;
        o0.x = f2h(x[0]) | (f2h(x[1]) << 16);
        o0.y = f2h(x[2]) | (f2h(x[3]) << 16);
        o0.z = f2h(x[4]) | (f2h(x[5]) << 16);
        o0.w = f2h(x[6]) | (f2h(x[7]) << 16);
        o1.x = f2h(x[8]) | (f2h(x[9]) << 16);
        o1.y = f2h(x[10]) | (f2h(x[11]) << 16);
        o1.z = f2h(x[12]) | (f2h(x[13]) << 16);
        o1.w = f2h(x[14]) | (f2h(x[15]) << 16);
        *reinterpret_cast<uint4*>(row + li * 32) = o0;
        *reinterpret_cast<uint4*>(row + li * 32 + 16) = o1;
        if ((li & (gl - 1)) == 0) prow[li / gl] = 0u;
        continue;
      }
      uint32_t w[4], param;
      float mn, mx;
      if constexpr (ROT) lane_extremes(x, mn, mx);
      else lane_extremes_h(ww, mn, mx);
      quantize16<L16>(x, mn, mx, gl, bits, w, param);
      if (MIX && bits == 8) {
        *reinterpret_cast<uint4*>(row + li * 16) = uint4{w[0], w[1], w[2], w[3]};
      } else if (MIX == 2 && bits == 2) {
        *reinterpret_cast<uint32_t*>(row + li * 4) = w[0];
      } else {
        *reinterpret_cast<uint2*>(row + li * 8) = uint2{w[0], w[1]};
      }
      if (MIX && kv) {  // the rest of a narrower row's record is zero (4-byte aligned, as in store_codes)
        uint32_t* z = reinterpret_cast<uint32_t*>(row + L16 * 2 * bits);
        const int nw = (g.rec - (g.d + g.dv) * bits / 8) / 4;
        for (int q = li; q < nw; q += L16) z[q] = 0u;
      }
      if ((li & (gl - 1)) == 0) prow[li / gl] = param;
    }
  };
#pragma unroll
  for (int p = 0; p < PF; ++p)
    if (p < NPASS) issue(buf[p], p);
#pragma unroll
  for (int p = 0; p < NPASS; ++p) {
    if (p + PF < NPASS) issue(buf[(p + PF) % (PF + 1)], p + PF);
    __builtin_amdgcn_sched_barrier(0);
    work(buf[p % (PF + 1)], p);
  }
  if (kv0 + NT - 1 == 1) {
    // zero the tail padding (and write the width words of pools with per-token widths)
    const uint32_t end = g.off_hdr + g.header_bytes();
    for (uint32_t o = end + 4u * (uint32_t)tid; o < g.tile_bytes; o += 4u * (uint32_t)nthr)
      *reinterpret_cast<uint32_t*>(tile + o) = 0u;
    if (MIX && tid < (int)(g.header_bytes() / 4))
      reinterpret_cast<uint32_t*>(tile + g.off_hdr)[tid] = bitmap ? bitmap[tid] : (MIX == 2 ? 0x55555555u : 0u);
  }
}

template <int L16, bool ROT, int MIX, int NT, int PF>
__global__ __launch_bounds__(256) void quantize_rows16_k(TileGeom g, uint8_t* __restrict__ pool,
                                                         const int32_t* __restrict__ block_ids,
                                                         const uint16_t* __restrict__ k,
                                                         const uint16_t* __restrict__ v,
                                                         const uint32_t* __restrict__ prec_bits, float rot_c,
                                                         int kv_base) {
  rows16_tile<L16, ROT, MIX, NT, PF>(g, pool, block_ids, k, v, prec_bits, rot_c, NT == 2 ? 0 : blockIdx.z + kv_base,
                                     threadIdx.x, blockDim.x);
}

// K and V of a tile whose head dims differ (no rotation): waves 0-3 quantise K with LK lanes per row, waves 4-7
// V with LV lanes per row. Both halves of each row record (K codes, then V codes, 160 bytes at K 192 / V 128)
// are written at about the same time, so L2 merges them into whole lines; with a launch per tensor each half
// reached HBM as partial lines of two 128-byte lines (the V-only launch ran at 2.6 TB/s).
template <int LK, int LV, int MIX>
__global__ __launch_bounds__(512) void quantize_rows16_pair_k(TileGeom g, uint8_t* __restrict__ pool,
                                                              const int32_t* __restrict__ block_ids,
                                                              const uint16_t* __restrict__ k,
                                                              const uint16_t* __restrict__ v,
                                                              const uint32_t* __restrict__ prec_bits) {
  if (threadIdx.x < 256)
    rows16_tile<LK, false, MIX, 1, 2>(g, pool, block_ids, k, v, prec_bits, 1.0f, 0, threadIdx.x, 256);
  else
    rows16_tile<LV, false, MIX, 1, 2>(g, pool, block_ids, k, v, prec_bits, 1.0f, 1, threadIdx.x - 256, 256);
}

template <int LPR>
hipError_t launch_quantize_t(const TileGeom& g, uint8_t* pool, const int32_t* block_ids, int n_blocks,
                             const uint16_t* k, const uint16_t* v, const uint32_t* prec_bits, float rot_c,
                             int kv_base, int n_tensors, hipStream_t stream) {
  if (kv_base == 0 && !(g.kg > 0 || g.fp8)) {  // per-channel K first, then the V rows
    // (head dims whose lanes divide the workgroup: the layout check admits per-channel K at 64, 128, 256)
    if constexpr (kKchanThreads % LPR == 0)
      hipLaunchKernelGGL(quantize_kchan_k<LPR>, dim3(n_blocks, g.H, 1), dim3(kKchanThreads), 0, stream, g, pool,
                         block_ids, k, rot_c);
    else
      return hipErrorInvalidValue;
    kv_base = 1;
    n_tensors -= 1;
  }
  if (n_tensors > 0) {
    // 16 values per lane where the tensors' groups span whole 16-channel lanes and a row's lanes divide a
    // wave (head dims 64, 128, 256)
    const bool k_lanes = kv_base > 0 || g.kg % 16 == 0;
    const bool v_lanes = kv_base + n_tensors < 2 || g.vg % 16 == 0;
    if (!g.fp8 && k_lanes && v_lanes) {
      constexpr int L16 = LPR / 2;
      // K and V of a tile in one workgroup (whole row records and parameter records written by one wave, two
      // passes in flight) once there are enough tiles to fill the chip with them (4 per CU); small calls keep
      // one workgroup per tensor.
      const bool both = n_tensors == 2 && (long)n_blocks * g.H >= 1024;
      const dim3 grid(n_blocks, g.H, both ? 1 : n_tensors);
      auto go = [&](auto kern1, auto kern2) {
        if (both)
          hipLaunchKernelGGL(kern2, grid, dim3(256), 0, stream, g, pool, block_ids, k, v, prec_bits, rot_c, kv_base);
        else
          hipLaunchKernelGGL(kern1, grid, dim3(256), 0, stream, g, pool, block_ids, k, v, prec_bits, rot_c, kv_base);
      };
      if constexpr ((L16 & (L16 - 1)) == 0) {
        if (g.rotate) {
          if (g.mixed == 2) go(quantize_rows16_k<L16, true, 2, 1, 1>, quantize_rows16_k<L16, true, 2, 2, 2>);
          else if (g.mixed) go(quantize_rows16_k<L16, true, 1, 1, 1>, quantize_rows16_k<L16, true, 1, 2, 2>);
          else go(quantize_rows16_k<L16, true, 0, 1, 1>, quantize_rows16_k<L16, true, 0, 2, 2>);
          return hipGetLastError();
        }
      }
      {
        if (g.mixed == 2) go(quantize_rows16_k<L16, false, 2, 1, 1>, quantize_rows16_k<L16, false, 2, 2, 2>);
        else if (g.mixed) go(quantize_rows16_k<L16, false, 1, 1, 1>, quantize_rows16_k<L16, false, 1, 2, 2>);
        else go(quantize_rows16_k<L16, false, 0, 1, 1>, quantize_rows16_k<L16, false, 0, 2, 2>);
      }
    } else
      hipLaunchKernelGGL(quantize_rows_k<LPR>, dim3(n_blocks, g.H, n_tensors), dim3(256), 0, stream, g, pool,
                         block_ids, k, v, prec_bits, rot_c, kv_base);
  }
  return hipGetLastError();
}

// The cache restored as fp16 rows (QKVShare methodology, injection path): grid (n_blocks, H, 2), one
// workgroup writes the 256 rows of tensor blockIdx.z (0 = K, 1 = V) of tile (block_ids[blockIdx.x],
// blockIdx.y) as fp16 [n_blocks * 256][H][d], the input layout of quantize_rows_k. LPR = d / 8 lanes per row,
// 8 channels each: value = fp32(code) * scale + zero (the product is exact), then for a rotated pool the
// same butterflies as the rotation with the inverse scale 1 / (d c), then one rounding to fp16. Up to the
// fp32 roundings of the sum and the butterflies this is the exact value rounded once.
template <int LPR>
__global__ __launch_bounds__(256) void dequantize_k(TileGeom g, const uint8_t* __restrict__ pool,
                                                   const int32_t* __restrict__ block_ids, uint16_t* __restrict__ k_out,
                                                   uint16_t* __restrict__ v_out, float unrot_c, int which_base) {
  constexpr int RPP = 256 / LPR;  // rows per pass
  const int h = blockIdx.y, which = blockIdx.z + which_base;
  const uint8_t* tile = pool + ((size_t)block_ids[blockIdx.x] * g.H + h) * g.tile_bytes;
  const int li = threadIdx.x % LPR, r0 = threadIdx.x / LPR;
  uint16_t* out = which ? v_out : k_out;
  const bool kchan = which == 0 && g.kg < 0;
  const int grp = which ? g.vg : g.kg;
  float cs[8], cz[8];  // per-channel K parameters of this lane's channels
  if (kchan) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t pr = *reinterpret_cast<const uint32_t*>(tile + g.off_kch + 4 * (8 * li + i));
      cs[i] = h2f(pr & 0xffffu);
      cz[i] = h2f(pr >> 16);
    }
  }
  for (int t = r0 < RPP ? r0 : kRows; t < kRows; t += RPP) {  // (24 lanes per row at d = 192: 16 idle threads)
    float x[8];
    if (g.fp8) {  // E4M3 -> fp32 is exact
      const uint2 w = *reinterpret_cast<const uint2*>(tile + (which ? g.vcode(t, 8) : g.kcode(t)) + li * 8);
      x[0] = __builtin_amdgcn_cvt_f32_fp8((int)w.x, 0);
      x[1] = __builtin_amdgcn_cvt_f32_fp8((int)w.x, 1);
      x[2] = __builtin_amdgcn_cvt_f32_fp8((int)w.x, 2);
      x[3] = __builtin_amdgcn_cvt_f32_fp8((int)w.x, 3);
      x[4] = __builtin_amdgcn_cvt_f32_fp8((int)w.y, 0);
      x[5] = __builtin_amdgcn_cvt_f32_fp8((int)w.y, 1);
      x[6] = __builtin_amdgcn_cvt_f32_fp8((int)w.y, 2);
      x[7] = __builtin_amdgcn_cvt_f32_fp8((int)w.y, 3);
    } else {
      const int bits = g.row_bits(tile, t);
      const uint8_t* row = tile + (which ? g.vcode(t, bits) : g.kcode(t));
      uint32_t code[8];
      if (bits == 16) {  // stored fp16: exact in fp32
        const uint4 w = *reinterpret_cast<const uint4*>(row + li * 16);
        const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          code[2 * i] = ww[i] & 0xffffu;
          code[2 * i + 1] = ww[i] >> 16;
        }
      } else if (bits == 8) {
        const uint2 w = *reinterpret_cast<const uint2*>(row + li * 8);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          code[i] = (w.x >> (8 * i)) & 255u;
          code[4 + i] = (w.y >> (8 * i)) & 255u;
        }
      } else if (bits == 4) {
        const uint32_t w = *reinterpret_cast<const uint32_t*>(row + li * 4);
#pragma unroll
        for (int i = 0; i < 8; ++i) code[i] = (w >> (4 * i)) & 15u;
      } else {
        const uint32_t w = *reinterpret_cast<const uint16_t*>(row + li * 2);
#pragma unroll
        for (int i = 0; i < 8; ++i) code[i] = (w >> (2 * i)) & 3u;
      }
      if (bits == 16) {
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = h2f(code[i]);
      } else if (kchan) {
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = (float)code[i] * cs[i] + cz[i];
      } else {
        // the lane's 8 channels lie in one group (groups are multiples of 8)
        const uint32_t pr = *reinterpret_cast<const uint32_t*>(tile + (which ? g.vpar(t) : g.kpar(t)) +
                                                               4 * ((8 * li) / grp));
        const float s = h2f(pr & 0xffffu), z = h2f(pr >> 16);
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = (float)code[i] * s + z;
      }
    }
    if (g.rotate) rotate_row<LPR>(x, li, unrot_c);
    uint4 o;
    o.x = f2h(x[0]) | (f2h(x[1]) << 16);
    o.y = f2h(x[2]) | (f2h(x[3]) << 16);
    o.z = f2h(x[4]) | (f2h(x[5]) << 16);
    o.w = f2h(x[6]) | (f2h(x[7]) << 16);
    *reinterpret_cast<uint4*>(out + (((size_t)blockIdx.x * kRows + t) * g.H + h) * (8 * LPR) + 8 * li) = o;
  }
}

}  // namespace

// One launch per tensor when K and V head dims differ (D = 8 LPR is the tensor's own), one for both otherwise.
template <class F>
static hipError_t per_tensor(const TileGeom& g, F&& launch) {
  auto one = [&](int dim, int kv_base, int n_tensors) -> hipError_t {
    switch (dim) {
      case 64: return launch(std::integral_constant<int, 8>{}, kv_base, n_tensors);
      case 128: return launch(std::integral_constant<int, 16>{}, kv_base, n_tensors);
      case 192: return launch(std::integral_constant<int, 24>{}, kv_base, n_tensors);
      case 256: return launch(std::integral_constant<int, 32>{}, kv_base, n_tensors);
    }
    return hipErrorInvalidValue;
  };
  if (g.dv == g.d) return one(g.d, 0, 2);
  const hipError_t e = one(g.d, 0, 1);
  return e != hipSuccess ? e : one(g.dv, 1, 1);
}

hipError_t launch_quantize_blocks(const TileGeom& g, uint8_t* pool, const int32_t* block_ids, int n_blocks,
                                  const uint16_t* k, const uint16_t* v, const uint32_t* prec_bits,
                                  float rot_c, float rot_cv, hipStream_t stream) {
  // Unequal head dims with per-token groups spanning whole 16-channel lanes and no rotation (the MLA pools): K
  // and V of each tile in one workgroup once there are enough tiles to fill the chip (4 per CU).
  if (g.dv != g.d && !g.fp8 && !g.rotate && g.kg > 0 && g.kg % 16 == 0 && g.vg % 16 == 0 && g.dv == 128 &&
      (g.d == 192 || g.d == 256) && (long)n_blocks * g.H >= 1024) {
    const dim3 grid(n_blocks, g.H, 1);
    auto go = [&](auto kern) {
      hipLaunchKernelGGL(kern, grid, dim3(512), 0, stream, g, pool, block_ids, k, v, prec_bits);
      return hipGetLastError();
    };
    if (g.d == 192) {
      if (g.mixed == 2) return go(quantize_rows16_pair_k<12, 8, 2>);
      if (g.mixed == 1) return go(quantize_rows16_pair_k<12, 8, 1>);
      return go(quantize_rows16_pair_k<12, 8, 0>);
    }
    if (g.mixed == 2) return go(quantize_rows16_pair_k<16, 8, 2>);
    if (g.mixed == 1) return go(quantize_rows16_pair_k<16, 8, 1>);
    return go(quantize_rows16_pair_k<16, 8, 0>);
  }
  return per_tensor(g, [&](auto lpr, int kv_base, int n_tensors) {
    return launch_quantize_t<decltype(lpr)::value>(g, pool, block_ids, n_blocks, k, v, prec_bits,
                                                   kv_base ? rot_cv : rot_c, kv_base, n_tensors, stream);
  });
}

hipError_t launch_append_tokens(const TileGeom& g, uint8_t* pool, int n_seqs, const uint16_t* k,
                                const uint16_t* v, const int32_t* block_table, int max_blocks_per_seq,
                                const int32_t* positions, const uint8_t* prec, float rot_c, float rot_cv,
                                hipStream_t stream) {
  if (g.dv != g.d && g.dv == 128 && (g.d == 192 || g.d == 256)) {  // unequal head dims: one launch
    if (g.d == 192)
      hipLaunchKernelGGL((append_pair_k<24, 16>), dim3(n_seqs, g.H, 1), dim3(64), 0, stream, g, pool, k, v,
                         block_table, max_blocks_per_seq, positions, prec, rot_c, rot_cv);
    else
      hipLaunchKernelGGL((append_pair_k<32, 16>), dim3(n_seqs, g.H, 1), dim3(64), 0, stream, g, pool, k, v,
                         block_table, max_blocks_per_seq, positions, prec, rot_c, rot_cv);
    return hipGetLastError();
  }
  return per_tensor(g, [&](auto lpr, int kv_base, int n_tensors) {
    constexpr int LPR = decltype(lpr)::value;
    hipLaunchKernelGGL(append_k<LPR>, dim3(n_seqs, g.H, n_tensors), dim3(LPR), 0, stream, g, pool, k, v,
                       block_table, max_blocks_per_seq, positions, prec, kv_base ? rot_cv : rot_c, kv_base);
    return hipGetLastError();
  });
}

hipError_t launch_dequantize_blocks(const TileGeom& g, const uint8_t* pool, const int32_t* block_ids, int n_blocks,
                                    uint16_t* k_out, uint16_t* v_out, float unrot_c, float unrot_cv,
                                    hipStream_t stream) {
  return per_tensor(g, [&](auto lpr, int kv_base, int n_tensors) {
    constexpr int LPR = decltype(lpr)::value;
    hipLaunchKernelGGL(dequantize_k<LPR>, dim3(n_blocks, g.H, n_tensors), dim3(256), 0, stream, g, pool, block_ids,
                       k_out, v_out, kv_base ? unrot_cv : unrot_c, kv_base);
    return hipGetLastError();
  });
}

}  // namespace kvq
