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
__device__ __forceinline__ uint32_t f2h(float f) { return __builtin_bit_cast(uint16_t, (_Float16)f); }

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
      float p = __shfl_xor(x[i], m);
      x[i] = upper ? (p - x[i]) : (x[i] + p);
    }
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) x[i] = x[i] * c;
}

// Quantise this lane's 8 values as part of a group spanning gl lanes (gl a power of two dividing the
// row's lanes). Returns the 8 codes; every lane of the group gets the same packed {scale, zero}.
__device__ __forceinline__ void quantize8(const float (&x)[8], int gl, int bits, uint32_t (&code)[8],
                                          uint32_t& param) {
  float mn = x[0], mx = x[0];
#pragma unroll
  for (int i = 1; i < 8; ++i) {
    mn = fminf(mn, x[i]);
    mx = fmaxf(mx, x[i]);
  }
  for (int m = 1; m < gl; m *= 2) {
    mn = fminf(mn, __shfl_xor(mn, m));
    mx = fmaxf(mx, __shfl_xor(mx, m));
  }
  mn = mn + 0.0f;  // a -0 extreme becomes +0
  mx = mx + 0.0f;
  const float L = bits == 8 ? 255.0f : bits == 2 ? 3.0f : 15.0f;
  const float s32 = (mx - mn) / L;
  const uint32_t sh = f2h(s32), zh = f2h(mn);
  param = sh | (zh << 16);
  const float s = h2f(sh), z = h2f(zh);
  if (s == 0.0f) {
#pragma unroll
    for (int i = 0; i < 8; ++i) code[i] = 0;
    return;
  }
  const float r = 1.0f / s;
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
// pool's widest) the lane also zeroes its share (tail / lpr bytes) of the record after the row.
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
    const int share = tail / lpr;  // a multiple of 4 bytes
    uint32_t* z = reinterpret_cast<uint32_t*>(row + lpr * bits + li * share);
    for (int k = 0; k < share / 4; ++k) z[k] = 0u;
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
  quantize8(x, gl, bits, code, param);
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

// K grouped per channel over the block's 256 rows (always 4-bit). Two passes over the rows: the first
// finds every column's min/max of the (rotated) values, the second recomputes the identical rotated
// values and encodes them against the column's parameters.
template <int LPR>
__global__ __launch_bounds__(256) void quantize_kchan_k(TileGeom g, uint8_t* __restrict__ pool,
                                                        const int32_t* __restrict__ block_ids,
                                                        const uint16_t* __restrict__ k, float rot_c) {
  constexpr int D = LPR * 8;
  constexpr int kRowsPerPass = 256 / LPR;
  __shared__ float s_min[kRowsPerPass][D];
  __shared__ float s_max[kRowsPerPass][D];
  __shared__ float s_z[D], s_r[D];
  __shared__ int s_zero_scale[D];
  const int i = blockIdx.x, h = blockIdx.y;
  const int li = threadIdx.x % LPR, r0 = threadIdx.x / LPR;
  uint8_t* tile = pool + ((size_t)block_ids[i] * g.H + h) * g.tile_bytes;
  const uint16_t* src = k + ((size_t)i * kRows * g.H + h) * D + li * 8;

  float cmin[8], cmax[8];
  for (int t = r0; t < kRows; t += kRowsPerPass) {
    float x[8];
    load8(src + (size_t)t * g.H * D, x);
    if (g.rotate) rotate_row<LPR>(x, li, rot_c);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      cmin[e] = t == r0 ? x[e] : fminf(cmin[e], x[e]);
      cmax[e] = t == r0 ? x[e] : fmaxf(cmax[e], x[e]);
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    s_min[r0][li * 8 + e] = cmin[e];
    s_max[r0][li * 8 + e] = cmax[e];
  }
  __syncthreads();
  for (int c = threadIdx.x; c < D; c += blockDim.x) {
    float mn = s_min[0][c], mx = s_max[0][c];
    for (int r = 1; r < kRowsPerPass; ++r) {
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
  for (int t = r0; t < kRows; t += kRowsPerPass) {
    float x[8];
    load8(src + (size_t)t * g.H * D, x);
    if (g.rotate) rotate_row<LPR>(x, li, rot_c);
    uint32_t w = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int c = li * 8 + e;
      uint32_t code = 0;
      if (!s_zero_scale[c]) {
        float tt = x[e] - s_z[c];
        float u = tt * s_r[c];
        float qv = __builtin_rintf(u);
        qv = fminf(fmaxf(qv, 0.0f), 15.0f);
        code = (uint32_t)qv;
      }
      w |= code << (4 * e);
    }
    reinterpret_cast<uint32_t*>(tile + g.kcode(t))[li] = w;
  }
}

// Grid (n_seqs, H, tensors), LPR threads: row positions[s] % 256 of block block_table[s][positions[s] / 256];
// tensor kv_base + blockIdx.z (0 = K, 1 = V) of head dim D = 8 LPR.
template <int LPR>
__global__ __launch_bounds__(LPR) void append_k(TileGeom g, uint8_t* __restrict__ pool,
                                                const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
                                                const int32_t* __restrict__ block_table, int max_blocks_per_seq,
                                                const int32_t* __restrict__ positions,
                                                const uint8_t* __restrict__ prec, float rot_c, int kv_base) {
  constexpr int D = LPR * 8;
  const int s = blockIdx.x, h = blockIdx.y, kv = blockIdx.z + kv_base;
  const int li = threadIdx.x;
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

// Quantise this lane's 16 values at 4 bits as part of a group spanning gl lanes: the same fp32 operations
// per value as quantize8, so the same codes and parameters. Codes are packed low nibble first.
__device__ __forceinline__ void quantize16_q4(const float (&x)[16], int gl, uint2& codes, uint32_t& param) {
  float mn = x[0], mx = x[0];
#pragma unroll
  for (int i = 1; i < 16; ++i) {
    mn = fminf(mn, x[i]);
    mx = fmaxf(mx, x[i]);
  }
  for (int m = 1; m < gl; m *= 2) {
    mn = fminf(mn, __shfl_xor(mn, m));
    mx = fmaxf(mx, __shfl_xor(mx, m));
  }
  mn = mn + 0.0f;  // a -0 extreme becomes +0
  mx = mx + 0.0f;
  const float s32 = (mx - mn) / 15.0f;
  const uint32_t sh = f2h(s32), zh = f2h(mn);
  param = sh | (zh << 16);
  const float s = h2f(sh), z = h2f(zh);
  uint32_t w[2] = {0u, 0u};
  if (s != 0.0f) {
    const float r = 1.0f / s;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float qv = __builtin_rintf((x[i] - z) * r);
      qv = fminf(fmaxf(qv, 0.0f), 15.0f);
      w[i >> 3] |= (uint32_t)qv << (4 * (i & 7));
    }
  }
  codes = uint2{w[0], w[1]};
}

// quantize_rows_k for 4-bit pools without rotation whose groups span whole 16-channel lanes: LPR = d / 16
// lanes per row with 16 values each, so the per-row work (group extremes, the two divisions, addressing)
// is shared by twice as many values. Grid and output as quantize_rows_k.
template <int LPR>
__global__ __launch_bounds__(256) void quantize_rows16_k(TileGeom g, uint8_t* __restrict__ pool,
                                                         const int32_t* __restrict__ block_ids,
                                                         const uint16_t* __restrict__ k,
                                                         const uint16_t* __restrict__ v, int kv_base) {
  constexpr int D = LPR * 16;
  constexpr int kRowsPerPass = 256 / LPR;
  const int i = blockIdx.x, h = blockIdx.y, kv = blockIdx.z + kv_base;
  const int li = threadIdx.x % LPR, r0 = threadIdx.x / LPR;
  uint8_t* tile = pool + ((size_t)block_ids[i] * g.H + h) * g.tile_bytes;
  const uint16_t* src = (kv ? v : k) + ((size_t)i * kRows * g.H + h) * D + li * 16;
  const int gl = (kv ? g.vg : g.kg) / 16;
  for (int t = r0; t < kRows; t += kRowsPerPass) {
    float a[8], b[8], x[16];
    load8(src + (size_t)t * g.H * D, a);
    load8(src + (size_t)t * g.H * D + 8, b);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      x[e] = a[e];
      x[8 + e] = b[e];
    }
    uint2 codes;
    uint32_t param;
    quantize16_q4(x, gl, codes, param);
    *reinterpret_cast<uint2*>(tile + (kv ? g.vcode(t, 4) : g.kcode(t)) + li * 8) = codes;
    if ((li & (gl - 1)) == 0) reinterpret_cast<uint32_t*>(tile + (kv ? g.vpar(t) : g.kpar(t)))[li / gl] = param;
  }
  if (kv == 1) {  // zero the tail padding
    for (uint32_t o = g.off_hdr + 4u * threadIdx.x; o < g.tile_bytes; o += 4u * blockDim.x)
      *reinterpret_cast<uint32_t*>(tile + o) = 0u;
  }
}

template <int LPR>
hipError_t launch_quantize_t(const TileGeom& g, uint8_t* pool, const int32_t* block_ids, int n_blocks,
                             const uint16_t* k, const uint16_t* v, const uint32_t* prec_bits, float rot_c,
                             int kv_base, int n_tensors, hipStream_t stream) {
  if (kv_base == 0 && !(g.kg > 0 || g.fp8)) {  // per-channel K first, then the V rows
    hipLaunchKernelGGL(quantize_kchan_k<LPR>, dim3(n_blocks, g.H, 1), dim3(256), 0, stream, g, pool,
                       block_ids, k, rot_c);
    kv_base = 1;
    n_tensors -= 1;
  }
  if (n_tensors > 0) {
    const bool k_lanes = kv_base > 0 || g.kg % 16 == 0;  // the K rows' groups span whole 16-channel lanes
    if (LPR == 16 && !g.fp8 && !g.mixed && !g.rotate && g.dv == g.d && k_lanes && g.vg % 16 == 0)
      hipLaunchKernelGGL(quantize_rows16_k<8>, dim3(n_blocks, g.H, n_tensors), dim3(256), 0, stream, g, pool,
                         block_ids, k, v, kv_base);
    else
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
  return per_tensor(g, [&](auto lpr, int kv_base, int n_tensors) {
    return launch_quantize_t<decltype(lpr)::value>(g, pool, block_ids, n_blocks, k, v, prec_bits,
                                                   kv_base ? rot_cv : rot_c, kv_base, n_tensors, stream);
  });
}

hipError_t launch_append_tokens(const TileGeom& g, uint8_t* pool, int n_seqs, const uint16_t* k,
                                const uint16_t* v, const int32_t* block_table, int max_blocks_per_seq,
                                const int32_t* positions, const uint8_t* prec, float rot_c, float rot_cv,
                                hipStream_t stream) {
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
