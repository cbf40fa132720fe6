// kvq_decode_cascade.hip - decode attention over the blocks that every sequence of a batch shares, for head_dim
// 128 pools whose K is grouped per channel over each 256-token block (the long shared-prefix serving workload
// of the UltraQuant article's technology section, with the prefix reuse of "Agent Memory Below the Prompt",
// technical summary 2.1-2.2, and its packed-block decode).
//
// A logical block that all sequences map to the same physical block (a shared prompt prefix) is read once for
// all of them. The work unit is (range of logical blocks, KV head, kCascRows query rows), a query row being one
// (sequence, query head) pair of that KV head. The unit's partial softmax state per row goes to the split-K
// workspace; the per-sequence kernel (decode_kchan_k) then skips those blocks and merges these partials with
// its own. Every unit finds the shared blocks of its range itself (same physical block in every sequence's
// table, and full in the shortest sequence), and the units of KV head 0 and row group 0 publish them.
//
// Per block, with the block's K channel scales folded into the query (q . k_t = sum_c (q_c s_c) code_tc +
// sum_c q_c z_c):
// * QK on the matrix cores (v_mfma_f32_16x16x32_f16): A = q_c s_c as fp16 hi/lo rows (eight query rows per
//   16-row tile), built once per block by the whole workgroup; B = the K codes as exact fp16 subnormals.
// * PV: A = p in fp16 (sixteen query rows per tile), written position-major and read with the 16-bit LDS
//   transpose load; B = V dequantised to fp16 (v_scale * code + v_zero, one rounding) from the 4-bit LDS
//   transpose load. The values are centred on zero, so neither PV operand needs a hi/lo split.
// Wave w takes tokens 64w .. 64w+63 of every block for all the unit's rows; the waves' softmax states merge at
// the end.
#include "kvq_decode_mfma_common.hpp"

namespace kvq {
namespace {

using namespace dec;

typedef int v2i __attribute__((ext_vector_type(2)));
typedef short v4s __attribute__((ext_vector_type(4)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) v2i lds_v2i;
typedef __attribute__((address_space(3))) v4s lds_v4s;

__device__ __forceinline__ v2i lds_tr4(const void* p) {
  return __builtin_amdgcn_ds_read_tr4_b64_v2i32((lds_v2i*)const_cast<void*>(p));
}
__device__ __forceinline__ v2i lds_tr16(const void* p) {
  return __builtin_bit_cast(v2i, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)const_cast<void*>(p)));
}

constexpr uint32_t kLo4 = 0x000F000Fu, kHi4 = 0x00F000F0u;
constexpr int kD = 128;
constexpr int kVP = 80;  // LDS row pitch (bytes) of staged V rows
constexpr int kPP = 20;  // halves per position of a position-major p tile (16 rows + pad)
constexpr int kNT = kCascRows / 16;  // 16-row PV tiles per workgroup

// (x & m) | c in one VALU operation
__device__ __forceinline__ uint32_t and_or(uint32_t x, uint32_t m, uint32_t c) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(x), "v"(m), "v"(c));
  return r;
}

struct RawS {
  u32x4 k[4];   // K codes of tokens 16c + lj, channels 32 la .. 32 la + 31
  u32x4 v[4];   // V codes of the same tokens and channels
  u32x4 vp[4];  // V parameter records of tokens 16c + lj (first NGV entries used)
  u32x4 kp[2];  // K channel parameters 8 cb .. 8 cb + 7 (cb = tid mod 16), for the A operand build
};

// One-dimensional grid: workgroup wg -> unit u = (wg >> 3) / casc_rg * 8 + (wg & 7), row group
// (wg >> 3) mod casc_rg, so every workgroup of KV head h (u mod H = h) and one block range shares an XCD.
template <int VG>
__global__ __launch_bounds__(256, 2) void cascade_k(TileGeom g, DecodeArgs a) {
  constexpr int D = kD, NT = kNT, NR = kCascRows, NQT = 2 * NT, NGV = D / VG;
  static_assert(NGV == 2 || NGV == 4, "V groups of 64 or 32");
  // The loop's QK A operands [buf][tile][k-step][lane] and staged V rows [wave], and after the loop the
  // waves' accumulators, share one buffer.
  constexpr int kQaBytes = 2 * NQT * 4 * 64 * 4 * 4, kVBytes = 4 * 64 * kVP, kWaccBytes = 4 * 16 * D * 4;
  __shared__ __attribute__((aligned(16))) uint8_t s_buf[kQaBytes + kVBytes > kWaccBytes ? kQaBytes + kVBytes
                                                                                       : kWaccBytes];
  auto s_qa = reinterpret_cast<uint32_t (*)[NQT][4][64][4]>(&s_buf[0]);
  auto s_v = reinterpret_cast<uint8_t (*)[64 * kVP]>(&s_buf[kQaBytes]);
  __shared__ float s_zq[2][NR];                                           // sum_c q_c z_c per row and block
  __shared__ __attribute__((aligned(16))) _Float16 s_p[4][NT][64 * kPP];
  // V parameters of each wave's 8-token groups as fp16 pairs of tokens (r, r + 4): [wave][k-block][group of
  // 8][V group][2 r + {scale, zero}]
  __shared__ __attribute__((aligned(16))) uint32_t s_vp[4][2][4][NGV][8];
  __shared__ int s_tbl[kMaxSplitBlocks], s_col[kMaxSplitBlocks];
  __shared__ int s_bad[kMaxSplitBlocks];
  __shared__ int s_ccnt[4], s_minlen;
  __shared__ float s_wm[4][16], s_wl[4][16];
  static_assert(sizeof(float) * NR * D <= sizeof(s_p), "query set-up fits in s_p");
  float (*s_wacc)[16][D] = reinterpret_cast<float (*)[16][D]>(&s_buf[0]);  // after the block loop
  float (*s_q)[D] = reinterpret_cast<float (*)[D]>(&s_p[0][0][0]);                    // during the set-up

  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, la = l >> 4, lj = l & 15;
  const int H = g.H, S = a.plan.casc, RG = a.plan.casc_rg;
  const int wg = blockIdx.x, rest = wg >> 3;
  const int rg = rest % RG, u = (rest / RG) * 8 + (wg & 7);
  if (u >= S * H) return;
  const int h = u % H, split = u / H;
  const int n_rows = a.n_seqs * a.G;
  int c0, c1;
  split_range(split, S, a.plan.max_blocks, c0, c1);
  const uint8_t* pool_h = a.pool + (size_t)h * g.tile_bytes;
  const size_t tstride = (size_t)H * g.tile_bytes;
  const size_t mbs = (size_t)a.max_blocks_per_seq;

  // ------------------------------------------------------------ shared blocks of [c0, c1)
  if (tid == 0) s_minlen = 0x7fffffff;
  for (int i = tid; i < c1 - c0; i += 256) s_bad[i] = 0;
  __syncthreads();
  for (int s = tid; s < a.n_seqs; s += 256) atomicMin(&s_minlen, a.seq_lens[s]);
  {
    // every (sequence, column) pair once, four independent loads per thread per round
    const int ncol = c1 - c0, total = ncol * a.n_seqs;
    for (int base = 0; base < total; base += 1024) {
      int x[4], y[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int idx = min(base + tid + 256 * k, total - 1);
        const int s = idx / ncol, i = idx - s * ncol;
        x[k] = a.block_table[(size_t)s * mbs + c0 + i];
        y[k] = a.block_table[c0 + i];
      }
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int idx = base + tid + 256 * k;
        if (idx < total && x[k] != y[k]) s_bad[idx % ncol] = 1;
      }
    }
  }
  __syncthreads();
  const int nfull = s_minlen / kRows;  // blocks that are full in every sequence
  const int nc = stage_columns(
      c1 - c0, tid, s_tbl, s_col, s_ccnt, [&](int i) { return c0 + i < nfull && s_bad[i] == 0; },
      [&](int i) { return a.block_table[c0 + i]; });
  if (h == 0 && rg == 0)
    for (int i = tid; i < c1 - c0; i += 256) a.ws_cflag[c0 + i] = (c0 + i < nfull && s_bad[i] == 0) ? 1 : 0;

  const size_t pslot = (size_t)(a.plan.stride - S + split);  // this unit's partial slot in each row
  if (nc == 0) {
    for (int q = tid; q < NR; q += 256) {
      const int gr = rg * NR + q;
      if (gr < n_rows) {
        const int seq = gr / a.G, jj = gr - seq * a.G;
        const size_t pi = ((size_t)seq * a.num_q_heads + h * a.G + jj) * a.plan.stride + pslot;
        a.ws_ml[2 * pi] = kNegInf;
        a.ws_ml[2 * pi + 1] = 0.0f;
      }
    }
    return;
  }

  auto load = [&](RawS& r, int i) __attribute__((always_inline)) {
    const int phys = __builtin_amdgcn_readfirstlane(s_tbl[i]);
    const uint8_t* tile = pool_h + (size_t)phys * tstride;
    // the channel parameters first: the A operand build waits only for them
    const u32x4* kc = reinterpret_cast<const u32x4*>(tile + g.off_kch + 32 * (tid & 15));
    r.kp[0] = kc[0];
    r.kp[1] = kc[1];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint32_t row = 64 * w + 16 * c + lj;
      const uint8_t* rp = tile + (row * (uint32_t)g.rec + la * 16);
      r.k[c] = *reinterpret_cast<const u32x4*>(rp);
      r.v[c] = *reinterpret_cast<const u32x4*>(rp + D / 2);
      const uint8_t* pp = tile + (g.off_prow + row * (uint32_t)g.prow);
      if (NGV == 4) {
        r.vp[c] = *reinterpret_cast<const u32x4*>(pp);
      } else {
        const uint2 x = *reinterpret_cast<const uint2*>(pp);
        r.vp[c] = u32x4{x.x, x.y, 0u, 0u};
      }
    }
  };

  RawS ra, rb;
  load(ra, 0);

  // ------------------------------------------------------------ query rows: scale and rotation
  for (int i = tid; i < NR * D; i += 256) {
    const int q = i / D, c = i % D, gr = rg * NR + q;
    float v = 0.0f;
    if (gr < n_rows) {
      const int seq = gr / a.G, jj = gr - seq * a.G;
      v = h2f(a.q[((size_t)seq * a.num_q_heads + h * a.G + jj) * D + c]) * a.q_scale;
    }
    s_q[q][c] = v;
  }
  __syncthreads();
  if (g.rotate) {
    for (int hs = 1; hs < D; hs *= 2) {
      for (int i = tid; i < NR * D / 2; i += 256) {
        const int j = i / (D / 2), pi = i % (D / 2);
        const int lo = (pi / hs) * 2 * hs + (pi % hs);
        const float x = s_q[j][lo], y = s_q[j][lo + hs];
        s_q[j][lo] = x + y;
        s_q[j][lo + hs] = x - y;
      }
      __syncthreads();
    }
    for (int i = tid; i < NR * D; i += 256) s_q[i / D][i % D] *= a.unrot_c;
    __syncthreads();
  }
  // This thread builds the A operand entries of rows (tid >> 4) + 16 k, channels 8 cb + nib(e) (cb = tid mod
  // 16, nib = 0,4,1,5,2,6,3,7): it keeps those query values in registers.
  const int cb = tid & 15;
  float qv[NT][8];
#pragma unroll
  for (int k = 0; k < NT; ++k)
#pragma unroll
    for (int e = 0; e < 8; ++e) qv[k][e] = s_q[(tid >> 4) + 16 * k][8 * cb + (e >> 1) + 4 * (e & 1)];
  __syncthreads();  // s_q's space is s_p from here on

  // QK A operand of one block into buffer buf. Query row q (0..63) sits in PV tile q >> 4, as row q16 = q & 15,
  // which lane group q16 >> 2 holds in the QK and PV results; in QK tile 2 (q >> 4) + (q16 & 3) / 2 it is
  // MFMA row pair j = 2 (q16 >> 2) + (q16 & 1) (rows 2j = hi, 2j + 1 = lo). Lane group cb >> 2 of k-step cb & 3
  // covers channels 8 cb + nib(e); the high nibbles enter the MFMA multiplied by 16, so their entries are /16.
  auto build = [&](const RawS& r, int buf) __attribute__((always_inline)) {
    const uint32_t kw[8] = {r.kp[0][0], r.kp[0][1], r.kp[0][2], r.kp[0][3],
                            r.kp[1][0], r.kp[1][1], r.kp[1][2], r.kp[1][3]};
#pragma unroll
    for (int k = 0; k < NT; ++k) {
      const int q = (tid >> 4) + 16 * k, q16 = q & 15;
      const int qt = 2 * (q >> 4) + ((q16 & 3) >> 1), j = 2 * (q16 >> 2) + (q16 & 1);
      uint32_t hi4[4], lo4[4];
      float zs = 0.0f;
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        _Float16 hx[2], lx[2];
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          const int e = 2 * p + kk, m = (e >> 1) + 4 * (e & 1);
          const float f = (e & 2) ? 0.0625f : 1.0f;
          const float x = qv[k][e] * h2f(kw[m] & 0xffffu) * f;
          hx[kk] = (_Float16)x;
          lx[kk] = (_Float16)(x - (float)hx[kk]);
          zs += qv[k][e] * h2f(kw[m] >> 16);
        }
        hi4[p] = pack_h2(hx[0], hx[1]);
        lo4[p] = pack_h2(lx[0], lx[1]);
      }
      uint32_t* dst = &s_qa[buf][qt][cb & 3][(cb >> 2) * 16 + 2 * j][0];
      *reinterpret_cast<u32x4*>(dst) = u32x4{hi4[0], hi4[1], hi4[2], hi4[3]};
      *reinterpret_cast<u32x4*>(dst + 4) = u32x4{lo4[0], lo4[1], lo4[2], lo4[3]};
      zs = row_sum16(zs);  // the 16 threads of row q hold its 16 channel groups
      if (cb == 0) s_zq[buf][q] = zs;
    }
  };
  build(ra, 0);
  lds_barrier();

  // lane (la, lj): rows 16 pt + 4 la + i of each PV tile pt
  float m_run[NT][4], l_run[NT][4];
  floatx4 o[NT][8];
#pragma unroll
  for (int pt = 0; pt < NT; ++pt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      m_run[pt][i] = kNegInf;
      l_run[pt][i] = 0.0f;
    }
#pragma unroll
    for (int t = 0; t < 8; ++t) o[pt][t] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
  }
  uint8_t* sv = s_v[w];
  const h2 k1024 = {(_Float16)1024.0f, (_Float16)1024.0f};

  auto process = [&](const RawS& r, int buf) __attribute__((always_inline)) {
    // ---------------------------------------------------------- stage V codes and V parameters
#pragma unroll
    for (int c = 0; c < 4; ++c) *reinterpret_cast<u32x4*>(sv + (16 * c + lj) * kVP + la * 16) = r.v[c];
    if (la < NGV) {
      uint16_t* vp16 = reinterpret_cast<uint16_t*>(&s_vp[w][0][0][0][0]);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int tt = 16 * c + lj, kb = tt >> 5, grp = (tt >> 3) & 3, u8 = tt & 7, rr = u8 & 3, hf = u8 >> 2;
        const uint32_t pr = r.vp[c][la];
        uint16_t* d = vp16 + (((kb * 4 + grp) * NGV + la) * 8) * 2;
        d[(2 * rr) * 2 + hf] = (uint16_t)(pr & 0xffffu);
        d[(2 * rr + 1) * 2 + hf] = (uint16_t)(pr >> 16);
      }
    }
    // ---------------------------------------------------------- logits
    floatx4 acc[NQT][4];
#pragma unroll
    for (int qt = 0; qt < NQT; ++qt)
#pragma unroll
      for (int c = 0; c < 4; ++c) acc[qt][c] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      u32x4 qa[NQT];
#pragma unroll
      for (int qt = 0; qt < NQT; ++qt) qa[qt] = *reinterpret_cast<const u32x4*>(&s_qa[buf][qt][s][l][0]);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const uint32_t wd = r.k[c][s], w8 = wd >> 8;
        const u32x4 b = {wd & kLo4, wd & kHi4, w8 & kLo4, w8 & kHi4};
#pragma unroll
        for (int qt = 0; qt < NQT; ++qt) acc[qt][c] = mfma16(qa[qt], b, acc[qt][c]);
      }
    }
    // ---------------------------------------------------------- online softmax, p to LDS (fp16)
#pragma unroll
    for (int pt = 0; pt < NT; ++pt) {
      float sc[4][4];  // [token tile c][row i]
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float zq = s_zq[buf][16 * pt + 4 * la + i];
        const int qt = 2 * pt + (i >> 1), hp = 2 * (i & 1);
#pragma unroll
        for (int c = 0; c < 4; ++c) sc[c][i] = (acc[qt][c][hp] + acc[qt][c][hp + 1]) * kTwo24 + zq;
      }
      float alpha[4];
      bool moved = false;
      float p[4][4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float mx = fmaxf(fmaxf(sc[0][i], sc[1][i]), fmaxf(sc[2][i], sc[3][i]));
        mx = row_max16(mx);
        const float mnew = fmaxf(m_run[pt][i], mx);
        alpha[i] = mnew == m_run[pt][i] ? 1.0f : __builtin_amdgcn_exp2f(m_run[pt][i] - mnew);
        moved |= alpha[i] != 1.0f;
        float ps = 0.0f;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          p[c][i] = __builtin_amdgcn_exp2f(sc[c][i] - mnew);
          ps += p[c][i];
        }
        l_run[pt][i] = l_run[pt][i] * alpha[i] + ps;
        m_run[pt][i] = mnew;
      }
      if (__builtin_amdgcn_ballot_w64(moved)) {
#pragma unroll
        for (int t = 0; t < 8; ++t)
#pragma unroll
          for (int i = 0; i < 4; ++i) o[pt][t][i] *= alpha[i];
      }
      // position of token t: (t & ~7) | sinv(t & 7), sinv(u) = 2 (u & 3) + (u >> 2), the inverse of the token
      // order 0,4,1,5,2,6,3,7 in which the transposed V operand delivers each lane's eight tokens
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int t = 16 * c + lj, u8 = lj & 7;
        const int pos = (t & ~7) | (((u8 & 3) << 1) | (u8 >> 2));
        uint2 wv;
        wv.x = pack_h2((_Float16)p[c][0], (_Float16)p[c][1]);
        wv.y = pack_h2((_Float16)p[c][2], (_Float16)p[c][3]);
        *reinterpret_cast<uint2*>(&s_p[w][pt][pos * kPP + la * 4]) = wv;
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // ---------------------------------------------------------- PV
    u32x4 pa[NT][2];
#pragma unroll
    for (int pt = 0; pt < NT; ++pt)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int base = 32 * kb + 8 * la + (lj >> 2);
        const v2i x0 = lds_tr16(&s_p[w][pt][base * kPP + (lj & 3) * 4]);
        const v2i x1 = lds_tr16(&s_p[w][pt][(base + 4) * kPP + (lj & 3) * 4]);
        pa[pt][kb] = u32x4{(uint32_t)x0.x, (uint32_t)x0.y, (uint32_t)x1.x, (uint32_t)x1.y};
      }
    const int tok = lj < 8 ? 8 * la + lj : 32 + 8 * la + (lj - 8);
#pragma unroll
    for (int gm = 0; gm < NGV; ++gm) {
      u32x4 vz[2][2];  // [k-block][half]: words 2 r = scale pair, 2 r + 1 = zero pair of tokens (r, r + 4)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const u32x4* src = reinterpret_cast<const u32x4*>(&s_vp[w][kb][la][gm][0]);
        vz[kb][0] = src[0];
        vz[kb][1] = src[1];
      }
#pragma unroll
      for (int tt = 0; tt < 8 / NGV; ++tt) {
        const int t = gm * (8 / NGV) + tt;  // output tile (16 channels) inside V group gm
        const v2i x = lds_tr4(sv + tok * kVP + 8 * t);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const uint32_t wd = (uint32_t)(kb ? x.y : x.x);
          u32x4 b;
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) {
            // nibbles rr and rr + 4 (tokens rr, rr + 4) as 1024 + code, exact in fp16
            const uint32_t xx = and_or(rr ? wd >> (4 * rr) : wd, 0x000F000Fu, 0x64006400u);
            const h2 code = __builtin_bit_cast(h2, xx) - k1024;
            const uint32_t sw = vz[kb][rr >> 1][2 * (rr & 1)], zw = vz[kb][rr >> 1][2 * (rr & 1) + 1];
            const h2 v = __builtin_elementwise_fma(code, __builtin_bit_cast(h2, sw), __builtin_bit_cast(h2, zw));
            b[rr] = __builtin_bit_cast(uint32_t, v);
          }
#pragma unroll
          for (int pt = 0; pt < NT; ++pt) o[pt][t] = mfma16(pa[pt][kb], b, o[pt][t]);
        }
      }
    }
    __builtin_amdgcn_wave_barrier();
  };

  // Step i: the loads of block i + 1 are issued, block i is computed, and the A operand of block i + 1 is
  // built into the other LDS buffer and published by the barrier that ends the step. An index past the last
  // block repeats it (loaded and built again, never computed).
  auto step = [&](const RawS& cur, RawS& nxt, int i) __attribute__((always_inline)) {
    load(nxt, min(i + 1, nc - 1));
    __builtin_amdgcn_sched_barrier(0);
    process(cur, i & 1);
    build(nxt, (i + 1) & 1);
    lds_barrier();
  };
  int i = 0;
  for (; i + 1 < nc; i += 2) {
    step(ra, rb, i);
    step(rb, ra, i + 1);
  }
  if (i < nc) step(ra, rb, i);
  __syncthreads();

  // ---------------------------------------------------------------- merge the four waves, one PV tile at a time
#pragma unroll
  for (int pt = 0; pt < NT; ++pt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float lt = row_sum16(l_run[pt][i]);
      if (lj == 0) {
        s_wm[w][4 * la + i] = m_run[pt][i];
        s_wl[w][4 * la + i] = lt;
      }
#pragma unroll
      for (int t = 0; t < 8; ++t) s_wacc[w][4 * la + i][16 * t + lj] = o[pt][t][i];
    }
    __syncthreads();
    for (int idx = tid; idx < 16 * D; idx += 256) {
      const int q16 = idx / D, c = idx % D, gr = rg * NR + 16 * pt + q16;
      if (gr >= n_rows) continue;
      float M = kNegInf;
#pragma unroll
      for (int ww = 0; ww < 4; ++ww) M = fmaxf(M, s_wm[ww][q16]);
      float acc = 0.0f, L = 0.0f;
#pragma unroll
      for (int ww = 0; ww < 4; ++ww) {
        const float sc_w = exp2f(s_wm[ww][q16] - M);
        acc += s_wacc[ww][q16][c] * sc_w;
        L += s_wl[ww][q16] * sc_w;
      }
      const int seq = gr / a.G, jj = gr - seq * a.G;
      const size_t pi = ((size_t)seq * a.num_q_heads + h * a.G + jj) * a.plan.stride + pslot;
      a.ws_acc[pi * D + c] = acc;
      if (c == 0) {
        a.ws_ml[2 * pi] = M;
        a.ws_ml[2 * pi + 1] = L;
      }
    }
    __syncthreads();
  }
}

}  // namespace

// Layouts of the per-channel-K kernel with V groups of 32 or 64.
bool decode_cascade_supported(const TileGeom& g, int G) {
  return g.d == 128 && g.dv == 128 && g.kg < 0 && !g.mixed && (g.vg == 32 || g.vg == 64) && G >= 1 && G <= 8;
}

hipError_t launch_decode_cascade(const TileGeom& g, const DecodeArgs& a, hipStream_t stream) {
  const int units = a.plan.casc * g.H;
  const dim3 grid(8 * a.plan.casc_rg * ((units + 7) / 8));
  if (g.vg == 32)
    hipLaunchKernelGGL(cascade_k<32>, grid, dim3(256), 0, stream, g, a);
  else
    hipLaunchKernelGGL(cascade_k<64>, grid, dim3(256), 0, stream, g, a);
  return hipGetLastError();
}

}  // namespace kvq
