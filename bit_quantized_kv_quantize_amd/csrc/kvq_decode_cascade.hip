// kvq_decode_cascade.hip - decode attention over the blocks that every sequence of a batch shares, for head_dim
// 128 pools whose K is grouped per channel over each 256-token block (the long shared-prefix serving workload
// of the UltraQuant article's technology section, with the prefix reuse of "Agent Memory Below the Prompt",
// technical summary 2.1-2.2, and its packed-block decode).
//
// A logical block that all sequences map to the same physical block (a shared prompt prefix) is read once for
// all of them. The work unit is (range of logical blocks, KV head, row group), a row being one (sequence,
// query head) pair of that KV head and a row group up to eight 16-row tiles, one per wave. The unit's partial
// softmax state per row goes to the split-K workspace; the per-sequence kernel (decode_kchan_k) then skips
// those blocks and merges these partials with its own. Every unit finds the shared blocks of its range itself
// (same physical block in every sequence's table, and full in the shortest sequence), and the units of KV
// head 0 and row group 0 publish them.
//
// The blocks are walked in 64-token chunks. All 512 threads stage a chunk once for the eight waves: its K codes
// as stored, its V rows dequantised to fp16 (v_scale * code + v_zero, one rounding) and, with a block's first
// chunk, the block's K channel parameters. Each wave then takes its 16 rows against the chunk:
// * QK token-major on the matrix cores (v_mfma_f32_16x16x32_f16): A = the K codes of 16 tokens as exact fp16
//   subnormals (lane = token), B = q_c s_c of the wave's 16 rows as fp16 hi and lo (two MFMAs into one
//   accumulator), rebuilt from the fp32 query in registers at every block; the channel zeros enter as the
//   per-row constant sum_c q_c z_c (q . k_t = sum_c (q_c s_c) code_tc + sum_c q_c z_c).
// * The logits of a row sit in one column of the result: the row maximum is four lanes' worth of in-lane
//   maxima, and p (fp16) is already laid out as the B operand of PV.
// * PV channel-major: A = the staged fp16 V rows through the 16-bit LDS transpose load (lane = channel),
//   B = p. The values are centred on zero, so neither operand needs a hi/lo split.
// The result of a wave is its rows' partial state over the unit's blocks; no merge inside the workgroup.
#include "kvq_decode_mfma_common.hpp"

namespace kvq {
namespace {

using namespace dec;

typedef int v2i __attribute__((ext_vector_type(2)));
typedef short v4s __attribute__((ext_vector_type(4)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef float f2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) v4s lds_v4s;

__device__ __forceinline__ v2i lds_tr16(const void* p) {
  return __builtin_bit_cast(v2i, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)const_cast<void*>(p)));
}

constexpr uint32_t kLo4 = 0x000F000Fu, kHi4 = 0x00F000F0u;
constexpr int kD = 128;
constexpr int kCW = kCascRows / 16;  // waves per workgroup, one 16-row tile each
constexpr int kKP = 80;              // LDS pitch (bytes) of staged K code rows (64 B of codes)
constexpr int kVP = 288;             // LDS pitch (bytes) of staged fp16 V rows (256 B of values)

// (x & m) | c in one VALU operation
__device__ __forceinline__ uint32_t and_or(uint32_t x, uint32_t m, uint32_t c) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(x), "v"(m), "v"(c));
  return r;
}

// The chunk share of one thread: token tid / 8 of the chunk, byte quarter-pair tid % 8 of its K and V codes
// (16 channels), the V parameters of their group, and for a block's first chunk one K channel parameter.
struct Raw {
  uint2 k, v;
  uint32_t vp, kc;
};

// Channel order of the staged V rows inside each group of 8: the pairs (c, c + 4) that one and-or extracts.
__device__ __forceinline__ constexpr int nib(int e) { return (e >> 1) + 4 * (e & 1); }

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

// One-dimensional grid: workgroup wg -> unit u = (wg >> 3) / casc_rg * 8 + (wg & 7), row group
// (wg >> 3) mod casc_rg, so every workgroup of KV head h (u mod H = h) and one block range shares an XCD.
template <int VG>
__global__ __launch_bounds__(64 * kCW, 1) void cascade_k(TileGeom g, DecodeArgs a) {
  constexpr int D = kD, NW = kCW;
  static_assert(VG == 32 || VG == 64, "V groups of 32 or 64");
  constexpr int kKBytes = 64 * kKP, kBuf = kKBytes + 64 * kVP;  // one staged chunk: K rows, then V rows
  __shared__ __attribute__((aligned(16))) uint8_t s_ring[3][kBuf];
  __shared__ __attribute__((aligned(16))) float2 s_kc[2][D];  // (scale / 16 on odd channels, zero) per channel
  __shared__ int s_tbl[kMaxSplitBlocks], s_col[kMaxSplitBlocks];
  __shared__ int s_bad[kMaxSplitBlocks];
  __shared__ int s_ccnt[NW], s_minlen;
  // the scaled (and rotated) query of each lane: 32 channels at a pitch of 36 floats (conflict-free reads)
  __shared__ __attribute__((aligned(16))) float s_qv[NW][64][36];

  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, la = l >> 4, lj = l & 15;
  const int H = g.H, S = a.plan.casc, RG = a.plan.casc_rg, NT = a.plan.casc_nt;
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
  for (int i = tid; i < c1 - c0; i += 64 * NW) s_bad[i] = 0;
  __syncthreads();
  for (int s = tid; s < a.n_seqs; s += 64 * NW) atomicMin(&s_minlen, a.seq_lens[s]);
  {
    // every (sequence, column) pair once, four independent loads per thread per round
    const int ncol = c1 - c0, total = ncol * a.n_seqs;
    for (int base = 0; base < total; base += 4 * 64 * NW) {
      int x[4], y[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int idx = min(base + tid + 64 * NW * k, total - 1);
        const int s = idx / ncol, i = idx - s * ncol;
        x[k] = a.block_table[(size_t)s * mbs + c0 + i];
        y[k] = a.block_table[c0 + i];
      }
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int idx = base + tid + 64 * NW * k;
        if (idx < total && x[k] != y[k]) s_bad[idx % ncol] = 1;
      }
    }
  }
  __syncthreads();
  const int nfull = s_minlen / kRows;  // blocks that are full in every sequence
  const int nc = stage_columns<NW>(
      c1 - c0, tid, s_tbl, s_col, s_ccnt, [&](int i) { return c0 + i < nfull && s_bad[i] == 0; },
      [&](int i) { return a.block_table[c0 + i]; });
  if (h == 0 && rg == 0)
    for (int i = tid; i < c1 - c0; i += 64 * NW) a.ws_cflag[c0 + i] = (c0 + i < nfull && s_bad[i] == 0) ? 1 : 0;

  // this wave's rows: row0 + lj, lane (la, lj) holding channels 32 la .. 32 la + 31 of row lj in the query
  const int row0 = (rg * NT + w) * 16, row = row0 + lj;
  const bool wave_rows = w < NT && row0 < n_rows;
  const bool row_ok = w < NT && row < n_rows;
  const int seq = row_ok ? row / a.G : 0, jj = row_ok ? row - seq * a.G : 0;
  const size_t pslot = (size_t)(a.plan.stride - S + split);  // this unit's partial slot in each row
  const size_t pi = ((size_t)seq * a.num_q_heads + h * a.G + jj) * a.plan.stride + pslot;
  if (nc == 0) {
    if (row_ok && la == 0) {
      a.ws_ml[2 * pi] = kNegInf;
      a.ws_ml[2 * pi + 1] = 0.0f;
    }
    return;
  }

  // ------------------------------------------------------------ chunk loads and staging
  const int tt = tid >> 3, part = tid & 7;  // staging: token tt of the chunk, codes of channels 16 part ..
  const int n_chunks = 4 * nc;
  const uint32_t code_off = (uint32_t)tt * (uint32_t)g.rec + 8u * (uint32_t)part;
  const uint32_t vpar_off = g.off_prow + (uint32_t)tt * (uint32_t)g.prow + 4u * (uint32_t)((16 * part) / VG);
  const uint32_t kch_off = g.off_kch + 4u * (uint32_t)(tid & (D - 1));
  auto load = [&](Raw& r, int j) __attribute__((always_inline)) {
    j = min(j, n_chunks - 1);
    const int phys = __builtin_amdgcn_readfirstlane(s_tbl[j >> 2]);
    const uint8_t* tile = pool_h + (size_t)phys * tstride;
    const uint32_t t0 = 64u * (uint32_t)(j & 3);  // first token of the chunk
    const uint8_t* rp = tile + t0 * (uint32_t)g.rec + code_off;
    r.k = *reinterpret_cast<const uint2*>(rp);
    r.v = *reinterpret_cast<const uint2*>(rp + D / 2);
    r.vp = *reinterpret_cast<const uint32_t*>(tile + t0 * (uint32_t)g.prow + vpar_off);
    r.kc = *reinterpret_cast<const uint32_t*>(tile + kch_off);
  };
  const h2 k1024 = {(_Float16)1024.0f, (_Float16)1024.0f};
  auto stage = [&](const Raw& r, int j, uint8_t* sb) __attribute__((always_inline)) {
    *reinterpret_cast<uint2*>(sb + tt * kKP + 8 * part) = r.k;
    const h2 sc = __builtin_bit_cast(h2, __builtin_amdgcn_perm(r.vp, r.vp, 0x01000100u));
    const h2 zr = __builtin_bit_cast(h2, __builtin_amdgcn_perm(r.vp, r.vp, 0x03020302u));
    uint32_t o[8];
#pragma unroll
    for (int hw = 0; hw < 2; ++hw) {
      const uint32_t wd = hw ? r.v.y : r.v.x;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        // nibbles k and k + 4 (channels k, k + 4 of these 8) as 1024 + code, exact in fp16
        const uint32_t xx = and_or(k ? wd >> (4 * k) : wd, 0x000F000Fu, 0x64006400u);
        const h2 code = __builtin_bit_cast(h2, xx) - k1024;
        o[4 * hw + k] = __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(code, sc, zr));
      }
    }
    uint8_t* dv = sb + kKBytes + tt * kVP + 32 * part;
    *reinterpret_cast<u32x4*>(dv) = u32x4{o[0], o[1], o[2], o[3]};
    *reinterpret_cast<u32x4*>(dv + 16) = u32x4{o[4], o[5], o[6], o[7]};
    if ((j & 3) == 0 && tid < D) {
      const float f = (tid & 1) ? 0.0625f : 1.0f;  // odd channels enter the QK MFMA multiplied by 16
      s_kc[(j >> 2) & 1][tid] = make_float2(h2f(r.kc & 0xffffu) * f, h2f(r.kc >> 16));
    }
  };

  Raw ra, rb;
  load(ra, 0);
  load(rb, 1);

  // ------------------------------------------------------------ query: scale and rotation, in registers
  float qv[32];
  {
    const u32x4* qp = reinterpret_cast<const u32x4*>(
        a.q + ((size_t)seq * a.num_q_heads + h * a.G + jj) * D + 32 * la);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const u32x4 x = row_ok ? qp[k] : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        qv[8 * k + 2 * e] = h2f(x[e] & 0xffffu) * a.q_scale;
        qv[8 * k + 2 * e + 1] = h2f(x[e] >> 16) * a.q_scale;
      }
    }
    if (g.rotate) {
#pragma unroll
      for (int hs = 1; hs < 32; hs *= 2)
#pragma unroll
        for (int i = 0; i < 32; ++i)
          if ((i & hs) == 0) {
            const float x = qv[i], y = qv[i + hs];
            qv[i] = x + y;
            qv[i + hs] = x - y;
          }
#pragma unroll
      for (int m = 16; m <= 32; m *= 2) {  // channel strides 32 and 64: lanes la ^ 1 and la ^ 2
        const bool upper = (l & m) != 0;
#pragma unroll
        for (int i = 0; i < 32; ++i) {
          const float p = __shfl_xor(qv[i], m);
          qv[i] = upper ? (p - qv[i]) : (qv[i] + p);
        }
      }
#pragma unroll
      for (int i = 0; i < 32; ++i) qv[i] *= a.unrot_c;
    }
#pragma unroll
    for (int k = 0; k < 8; ++k)
      *reinterpret_cast<float4*>(&s_qv[w][l][4 * k]) = make_float4(qv[4 * k], qv[4 * k + 1], qv[4 * k + 2], qv[4 * k + 3]);
  }

  stage(ra, 0, &s_ring[0][0]);
  load(ra, 2);
  stage(rb, 1, &s_ring[1][0]);
  load(rb, 3);
  lds_barrier();

  float m_run = kNegInf, l_run = 0.0f;
  floatx4 o[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) o[t] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
  u32x4 qh[4], ql[4];

  // B operand of QK for block b: row lj, k-step s, entry e = channel 32 la + 8 s + nib(e) (the order in
  // which the and-masks deliver a K code word's nibbles), value q_c s_c (odd channels / 16) as fp16 hi + lo;
  // returns the row's constant sum_c q_c z_c over all 128 channels.
  auto build = [&](int b) __attribute__((always_inline)) -> float {
    const float2* kc = &s_kc[b & 1][32 * la];
    float zs = 0.0f;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      float2 pr[8];
      float qs[8];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float4 x = *reinterpret_cast<const float4*>(&kc[8 * s + 2 * k]);
        pr[2 * k] = make_float2(x.x, x.y);
        pr[2 * k + 1] = make_float2(x.z, x.w);
      }
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const float4 x = *reinterpret_cast<const float4*>(&s_qv[w][l][8 * s + 4 * k]);
        qs[4 * k] = x.x;
        qs[4 * k + 1] = x.y;
        qs[4 * k + 2] = x.z;
        qs[4 * k + 3] = x.w;
      }
      uint32_t hw[4], lw[4];
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        float xs[2], rs[2];
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          const int c = nib(2 * p + kk);
          const float qc = qs[c];
          xs[kk] = qc * pr[c].x;
          zs = __builtin_fmaf(qc, pr[c].y, zs);
        }
        const h2 hx = __builtin_convertvector(f2{xs[0], xs[1]}, h2);
        rs[0] = xs[0] - (float)hx[0];
        rs[1] = xs[1] - (float)hx[1];
        hw[p] = __builtin_bit_cast(uint32_t, hx);
        lw[p] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f2{rs[0], rs[1]}, h2));
      }
      qh[s] = u32x4{hw[0], hw[1], hw[2], hw[3]};
      ql[s] = u32x4{lw[0], lw[1], lw[2], lw[3]};
    }
    return rows4_sum(zs);
  };

  // logits of one staged chunk against the current B operands: token-major, lane (la, lj)
  // holds tokens 16 c + 4 la + i of row lj in acc[c][i] (before the 2^24 scale and the row constant)
  auto qk = [&](const uint8_t* sk, floatx4 (&acc)[4]) __attribute__((always_inline)) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const u32x4 kw = *reinterpret_cast<const u32x4*>(sk + (16 * c + lj) * kKP + 16 * la);
      acc[c] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const uint32_t wd = kw[s], w8 = wd >> 8;
        const u32x4 ka = {wd & kLo4, wd & kHi4, w8 & kLo4, w8 & kHi4};
        acc[c] = mfma16(ka, qh[s], acc[c]);
        acc[c] = mfma16(ka, ql[s], acc[c]);
      }
    }
  };

  // Online softmax (base 2) of one chunk's logits: p (fp16, already in the place of PV's B operand) and the
  // rescale factor of the running state. The running maximum moves only when a logit exceeds it by more than
  // kSlack (or on the first chunk), so p <= 2^kSlack and the rescale is rare.
  constexpr float kSlack = 8.0f;
  auto softmax = [&](const floatx4 (&acc)[4], float zq, u32x4 (&pb)[2]) __attribute__((always_inline)) -> float {
    float m4[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) m4[c] = fmaxf(fmaxf(acc[c][0], acc[c][1]), fmaxf(acc[c][2], acc[c][3]));
    const float mx = __builtin_fmaf(rows4_max(fmaxf(fmaxf(m4[0], m4[1]), fmaxf(m4[2], m4[3]))), kTwo24, zq);
    const float mnew = mx > m_run + kSlack ? mx : m_run;
    const float alpha = mnew == m_run ? 1.0f : __builtin_amdgcn_exp2f(m_run - mnew);
    const float off = zq - mnew;
    float p[4][4];
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int i = 0; i < 4; ++i) p[c][i] = __builtin_amdgcn_exp2f(__builtin_fmaf(acc[c][i], kTwo24, off));
    float s4[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) s4[c] = (p[c][0] + p[c][1]) + (p[c][2] + p[c][3]);
    l_run = l_run * alpha + ((s4[0] + s4[1]) + (s4[2] + s4[3]));  // this lane's share of the row sum
    m_run = mnew;
    // k-block kb holds tokens 32 kb + 4 la + e (e < 4) and 32 kb + 16 + 4 la + e - 4: p of S tiles 2 kb and
    // 2 kb + 1
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      uint32_t x[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int c = 2 * kb + (q >> 1), i = 2 * (q & 1);
        x[q] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f2{p[c][i], p[c][i + 1]}, h2));
      }
      pb[kb] = u32x4{x[0], x[1], x[2], x[3]};
    }
    return alpha;
  };
  // PV of one chunk with its V rows (channel-major A operand through the 16-bit transpose load)
  auto pv = [&](const uint8_t* sb, const u32x4 (&pb)[2]) __attribute__((always_inline)) {
    const uint8_t* sv = sb + kKBytes;
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int r0 = 32 * kb + 4 * la + (lj >> 2), col = 2 * (16 * t + 4 * (lj & 3));
        const v2i x0 = lds_tr16(sv + r0 * kVP + col);
        const v2i x1 = lds_tr16(sv + (r0 + 16) * kVP + col);
        o[t] = mfma16(u32x4{(uint32_t)x0.x, (uint32_t)x0.y, (uint32_t)x1.x, (uint32_t)x1.y}, pb[kb], o[t]);
      }
  };

  // Step j (four per block, k = j mod 4): the logits of chunk j + 1 (staged one step earlier) go to the matrix
  // cores while the softmax of chunk j runs; then chunk j's PV while chunk j + 2 (in registers since step
  // j - 2) is staged into the third ring buffer and the loads of chunk j + 4 are issued. Every step runs in
  // full: past the last chunk the logits are computed and dropped, and the loads repeat the last chunk, whose
  // staging lands in a buffer no longer read.
  uint8_t* b_cur = &s_ring[0][0];
  uint8_t* b_nxt = &s_ring[1][0];
  uint8_t* b_stg = &s_ring[2][0];
  auto rotate = [&]() __attribute__((always_inline)) {
    uint8_t* t = b_cur;
    b_cur = b_nxt;
    b_nxt = b_stg;
    b_stg = t;
  };
  if (wave_rows) {
    floatx4 sc[4];
    float zc = build(0);
    qk(b_cur, sc);
    auto step = [&](Raw& nxt, int j, auto kc) __attribute__((always_inline)) {
      constexpr int k = decltype(kc)::value;
      floatx4 sn[4];
      const float zn = k == 3 ? build((j + 1) >> 2) : zc;
      qk(b_nxt, sn);
      u32x4 pb[2];
      const float alpha = softmax(sc, zc, pb);
      if (__builtin_amdgcn_ballot_w64(alpha != 1.0f)) {
#pragma unroll
        for (int t = 0; t < 8; ++t) o[t] *= alpha;
      }
      pv(b_cur, pb);
      stage(nxt, j + 2, b_stg);
      load(nxt, j + 4);
#pragma unroll
      for (int c = 0; c < 4; ++c) sc[c] = sn[c];
      zc = zn;
      rotate();
      lds_barrier();
    };
    for (int j = 0; j < n_chunks; j += 4) {
      step(ra, j, std::integral_constant<int, 0>{});
      step(rb, j + 1, std::integral_constant<int, 1>{});
      step(ra, j + 2, std::integral_constant<int, 2>{});
      step(rb, j + 3, std::integral_constant<int, 3>{});
    }
  } else {
    // waves without rows stage their share of every chunk
    for (int j = 0; j < n_chunks; j += 2) {
      stage(ra, j + 2, b_stg);
      load(ra, j + 4);
      rotate();
      lds_barrier();
      stage(rb, j + 3, b_stg);
      load(rb, j + 5);
      rotate();
      lds_barrier();
    }
  }

  // ------------------------------------------------------------ this wave's rows: partial state
  if (!row_ok) return;
  const float lsum = rows4_sum(l_run);
  // o[t][i]: staged column 16 t + 4 la + i, channel 8 (2 t + (la >> 1)) + nib(4 (la & 1) + i)
  float* acc = a.ws_acc + pi * D;
#pragma unroll
  for (int t = 0; t < 8; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[8 * (2 * t + (la >> 1)) + nib(4 * (la & 1) + i)] = o[t][i];
  if (la == 0) {
    a.ws_ml[2 * pi] = m_run;
    a.ws_ml[2 * pi + 1] = lsum;
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
    hipLaunchKernelGGL(cascade_k<32>, grid, dim3(64 * kCW), 0, stream, g, a);
  else
    hipLaunchKernelGGL(cascade_k<64>, grid, dim3(64 * kCW), 0, stream, g, a);
  return hipGetLastError();
}

}  // namespace kvq
