// kvq_decode_kchan.hip - decode attention on the matrix cores for head_dim 128 pools whose K is grouped per
// channel over each 256-token block (the asymmetric K/V treatment of the UltraQuant article's technology
// section: K per channel, V per token), V groups of 32 or 64, GQA ratios up to 8, optional Walsh-Hadamard
// rotation (single-token decode attention over the packed cache of "Agent Memory Below the Prompt",
// technical summary 2.1-2.2, with the sentinel slots of the IntentKV article).
//
// Per block, the K channel scales fold into the query: q . k_t = sum_c (q_c s_c) code_tc + sum_c q_c z_c,
// so the workgroup builds one QK A operand per block (rows = (query head, fp16 hi/lo part) of q_c s_c) and
// one additive constant per head, shared by its four waves through LDS. Each wave takes 64 rows of every
// block of its split:
// * QK: B = the wave's K codes (lane = token), nibbles unpacked by masking into exact fp16 subnormals.
// * PV: one A operand per V group (rows = (head, part) of p * v_scale of that group), written
//   position-major and read with the 16-bit LDS transpose load; B = V codes staged in LDS and read with the
//   4-bit transpose load, one output channel per lane; each 16-channel output tile uses its group's A.
// Sentinel slots are skipped (their exact term is added when the output is finalised), and the split-K
// merge runs in the split that arrives last (splitk_arrive). After the cascade kernel (a.casc > 0) the blocks
// it took for the sequence (shared with other sequences) are skipped, and its partials join the merge.
#include "kvq_decode_mfma_common.hpp"
#include "kvq_decode_precise.hpp"

namespace kvq {
namespace {

using namespace dec;

typedef int v2i __attribute__((ext_vector_type(2)));
typedef short v4s __attribute__((ext_vector_type(4)));
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
constexpr int kPP = 20;  // halves per position of a position-major p * v_scale tile (16 rows + pad)

struct RawC {
  u32x4 k[4];     // K codes of tokens 16c + lj, channels 32 la .. 32 la + 31
  u32x4 v[4];     // V codes of the same tokens and channels
  uint32_t live;  // bit c: token 16c + lj is below seq_len and not a sentinel slot
  uint32_t kc;    // K channel record (fp16 scale, fp16 zero) of channel tid mod 128
};

// Grid (n_splits, H_kv, n_seqs), 256 threads = 4 waves; wave w owns rows 64w .. 64w+63 of each block.
template <int G, int VG>
__global__ __launch_bounds__(256, 2) void decode_kchan_k(TileGeom g, DecodeArgs a) {
  static_assert(G >= 1 && G <= 8, "GQA ratio 1..8 (two heads per 16-lane row group)");
  constexpr int D = kD;
  constexpr int NGV = D / VG;  // V groups per row (2 or 4)
  static_assert(NGV == 2 || NGV == 4, "V groups of 64 or 32");
  __shared__ float s_q[G][D];
  __shared__ __attribute__((aligned(16))) uint32_t s_qa[2][4][64][4];  // QK A operand per block [buf][s][lane]
  __shared__ float s_zq[2][8];                                        // per-head constant per block
  __shared__ __attribute__((aligned(16))) uint8_t s_v[4][64 * kVP];
  __shared__ __attribute__((aligned(16))) _Float16 s_p[4][NGV][64 * kPP];
  __shared__ float s_wm[4][G], s_wl[4][G];
  __shared__ int s_tbl[kMaxSplitBlocks];
  __shared__ uint16_t s_col[kMaxSplitBlocks];
  static_assert(sizeof(float) * 4 * G * D <= sizeof(_Float16) * 4 * NGV * 64 * kPP, "s_wacc fits in s_p");
  float (*s_wacc)[G][D] = reinterpret_cast<float (*)[G][D]>(&s_p[0][0][0]);  // used after the token loop
  uint32_t* s_kch = reinterpret_cast<uint32_t*>(&s_p[0][0][0]);  // K channel records of one block (in build_block)

  const int split = blockIdx.x, h = blockIdx.y, seq = blockIdx.z;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, la = l >> 4, lj = l & 15;
  const int ns = a.plan.n_splits;
  const int len = a.seq_lens[seq];
  const int nblk = (len + kRows - 1) / kRows;
  int b0, b1;
  split_range(split, a.plan.n_splits, nblk, b0, b1);
  // Blocks the cascade kernel took for this sequence are skipped here; its partials join the merge.
  const int n_pre = a.casc;
  const int* cflag = a.ws_cflag + (size_t)seq * a.plan.max_blocks;
  const int nchunk = stage_columns(
      max(b1 - b0, 0), tid, s_tbl, s_col, reinterpret_cast<int*>(&s_wm[0][0]),
      [&](int i) { return n_pre == 0 || cflag[b0 + i] == 0; },
      [&](int i) { return a.block_table[(size_t)seq * a.max_blocks_per_seq + b0 + i]; });
  const uint32_t* mask_row = a.mask ? a.mask + (size_t)seq * a.mask_words : nullptr;
  const uint8_t* pool_h = a.pool + (size_t)h * g.tile_bytes;
  const size_t tstride = (size_t)g.H * g.tile_bytes;

  if (nchunk == 0) {
    if (ns == 1 && n_pre == 0) {
      __shared__ int s_cnt0[4];
      const int n_sent = count_sentinels<256>(a, seq, len, tid, s_cnt0);
      for (int jj = 0; jj < G; ++jj)
        finalize_head<D, 256>(g, a, seq, h * G + jj, len, n_sent, kNegInf, 0.0f, 0.0f, tid, &s_q[0][0]);
    } else {
      if (tid < G) {
        s_wm[0][tid] = kNegInf;
        s_wl[0][tid] = 0.0f;
      }
      for (int i = tid; i < G * D; i += 256) s_wacc[1][i / D][i % D] = 0.0f;
      __syncthreads();
      splitk_arrive<D, G>(g, a, seq, h, split, ns, len, tid, &s_wm[0][0], &s_wl[0][0], &s_wacc[1][0][0],
                          &s_wacc[0][0][0], n_pre);
    }
    return;
  }

  // Addresses are a wave-uniform part (tile, row 64 w + 16 c) plus one lane offset each, so that few
  // per-lane values stay live across the token loop.
  const int wu = __builtin_amdgcn_readfirstlane(w);
  const uint32_t code_lane = (uint32_t)lj * (uint32_t)g.rec + 16u * (uint32_t)la;
  const uint32_t prow_lane = (uint32_t)lj * (uint32_t)g.prow;
  auto load = [&](RawC& r, int i) __attribute__((always_inline)) {
    const int phys = __builtin_amdgcn_readfirstlane(s_tbl[i]);
    const uint8_t* tile = pool_h + (size_t)phys * tstride;
    const int pos0 = (b0 + s_col[i]) * kRows + 64 * wu;  // position of row 64 w of the block
    uint32_t live = 0;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint8_t* tc = tile + (uint32_t)(64 * wu + 16 * c) * (uint32_t)g.rec;
      r.k[c] = *reinterpret_cast<const u32x4*>(tc + code_lane);
      r.v[c] = *reinterpret_cast<const u32x4*>(tc + code_lane + D / 2);
      const int pos = pos0 + 16 * c + lj;
      // the 16 rows 64 w + 16 c .. + 15 share one mask word
      const uint32_t mw = (mask_row && pos0 + 16 * c < len) ? mask_row[(pos0 + 16 * c) >> 5] : 0u;
      live |= (pos < len && !((mw >> (pos & 31)) & 1u)) ? (1u << c) : 0u;
    }
    r.live = live;
    r.kc = *reinterpret_cast<const uint32_t*>(tile + g.off_kch + 4u * (uint32_t)(threadIdx.x & (D - 1)));
  };
  // V parameter records of tokens 16c + lj of block i (first NGV entries used). One set only: the next
  // block's records are loaded once this block's have been used, and arrive during its PV.
  u32x4 vp[4];
  auto load_vp = [&](int i) __attribute__((always_inline)) {
    const int phys = __builtin_amdgcn_readfirstlane(s_tbl[i]);
    const uint8_t* tile = pool_h + (size_t)phys * tstride;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint8_t* pp = tile + (g.off_prow + (uint32_t)(64 * wu + 16 * c) * (uint32_t)g.prow) + prow_lane;
      if (NGV == 4) {
        vp[c] = *reinterpret_cast<const u32x4*>(pp);
      } else {
        const uint2 x = *reinterpret_cast<const uint2*>(pp);
        vp[c] = u32x4{x.x, x.y, 0u, 0u};
      }
    }
  };

  // QK A operand and head constants of block i into buffer buf from its K channel records kc (loaded with the
  // block's codes, staged in s_kch here; all 256 threads; caller synchronises).
  // Lane (la', lj') of k-step s holds A[row lj'][k = 8 la' + e] = part(lj') of q[hq][c] * s_c * f(e),
  // hq = lj' / 2, c = 32 la' + 8 s + nib(e), nib = 0,4,1,5,2,6,3,7, f = 1/16 on the high nibbles.
  auto build_block = [&](uint32_t kc, int buf) __attribute__((always_inline)) {
    lds_barrier();  // every wave is done with the p tiles, which s_kch aliases
    if (tid < D) s_kch[tid] = kc;
    lds_barrier();
    const uint32_t* kch = s_kch;
    // the thread index passes through an opaque copy, so that the addresses below are recomputed here
    // rather than hoisted out of the token loop, where they would be live (and spilled) throughout
    int t = tid;
    asm volatile("" : "+v"(t));
    {
      const int s = t >> 6, ln = t & 63, lap = ln >> 4, ljp = ln & 15;
      const int hq = ljp >> 1, part = ljp & 1;
      uint32_t wv[4];
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        _Float16 x[2];
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          const int e = 2 * p + k;
          const int c = 32 * lap + 8 * s + (e >> 1) + 4 * (e & 1);
          const float f = (e & 2) ? 0.0625f : 1.0f;
          const float v = hq < G ? s_q[hq][c] * h2f(kch[c] & 0xffffu) * f : 0.0f;
          const _Float16 hi = (_Float16)v;
          x[k] = part ? (_Float16)(v - (float)hi) : hi;
        }
        wv[p] = pack_h2(x[0], x[1]);
      }
      *reinterpret_cast<u32x4*>(&s_qa[buf][s][ln][0]) = u32x4{wv[0], wv[1], wv[2], wv[3]};
    }
    {
      // head constants: 8 heads x 32 threads, each thread 4 channels of the 128-channel dot product
      const int hq = t >> 5, part = t & 31;
      float zs = 0.0f;
      if (hq < G)
#pragma unroll
        for (int k = 0; k < 4; ++k) zs += s_q[hq][part * 4 + k] * h2f(kch[part * 4 + k] >> 16);
      for (int m = 16; m >= 1; m >>= 1) zs += __shfl_xor(zs, m);
      if (part == 0) s_zq[buf][hq] = zs;
    }
  };

  RawC ra, rb;
  load(ra, 0);
  load_vp(0);

  // ------------------------------------------------------------ query: scale and rotation
  for (int i = tid; i < G * D; i += 256)
    s_q[i / D][i % D] = h2f(a.q[((size_t)seq * a.num_q_heads + h * G + i / D) * D + i % D]) * a.q_scale;
  for (int i = tid; i < 4 * NGV * 64 * kPP; i += 256) (&s_p[0][0][0])[i] = (_Float16)0.0f;
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
  build_block(ra.kc, 0);
  __syncthreads();

  // lane (la, lj): heads 2 la + u (u = 0, 1) in MFMA rows 4 la + 2u + part
  const int h0 = 2 * la;
  const bool ok0 = h0 < G, ok1 = h0 + 1 < G;
  float m_run[2] = {kNegInf, kNegInf}, l_run[2] = {0.0f, 0.0f};
  float zacc[2][NGV];
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int gm = 0; gm < NGV; ++gm) zacc[u][gm] = 0.0f;
  floatx4 o[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) o[t] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
  uint8_t* sv = s_v[w];

  auto process = [&](const RawC& r, int i) __attribute__((always_inline)) {
    const int buf = i & 1;
#pragma unroll
    for (int c = 0; c < 4; ++c) *reinterpret_cast<u32x4*>(sv + (16 * c + lj) * kVP + la * 16) = r.v[c];
    // ---------------------------------------------------------- logits
    floatx4 acc[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[c] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const u32x4 qa = *reinterpret_cast<const u32x4*>(&s_qa[buf][s][l][0]);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const uint32_t wd = r.k[c][s], w8 = wd >> 8;
        const u32x4 b = {wd & kLo4, wd & kHi4, w8 & kLo4, w8 & kHi4};
        acc[c] = mfma16(qa, b, acc[c]);
      }
      __builtin_amdgcn_sched_barrier(0);  // one k-step's B operands live at a time
    }
    const float zq0 = s_zq[buf][min(h0, 7)], zq1 = s_zq[buf][min(h0 + 1, 7)];
    float sc[2][4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const bool live = (r.live >> c) & 1u;
      sc[0][c] = (live && ok0) ? (acc[c][0] + acc[c][1]) * kTwo24 + zq0 : kNegInf;
      sc[1][c] = (live && ok1) ? (acc[c][2] + acc[c][3]) * kTwo24 + zq1 : kNegInf;
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
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int gm = 0; gm < NGV; ++gm) zacc[u][gm] *= alpha[u];
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        o[t][0] *= alpha[0];
        o[t][1] *= alpha[0];
        o[t][2] *= alpha[1];
        o[t][3] *= alpha[1];
      }
    }
    // ---------------------------------------------------------- p * v_scale per V group to LDS
    // (with the chunk's wave-uniform operand scale, undone when the chunk is added to the output). Odd
    // tokens enter the MFMA as -p * v_scale times the complemented code (15 - code) and add
    // p * (v_zero + 15 v_scale) to the zero-point term, the same value: products of both signs keep the
    // matrix core's rounding of long all-positive sums from biasing the code term, which cancels against
    // the zero-point term down to the much smaller output.
    float vmax = 0.0f;
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int gm = 0; gm < NGV; ++gm) vmax = fmaxf(vmax, h2f(vp[c][gm] & 0xffffu));
    float pv_inv;
    const float pv_scale = chunk_pv_scale(vmax, pv_inv);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int t = 16 * c + lj, u8 = lj & 7;
      const int pos = (t & ~7) | (((u8 & 3) << 1) | (u8 >> 2));
      const bool odd = u8 & 1;
      const float f = odd ? -0.0625f * pv_scale : pv_scale;
      const float Lc = odd ? 15.0f : 0.0f;
      const bool on = p[0][c] != 0.0f || p[1][c] != 0.0f;
#pragma unroll
      for (int gm = 0; gm < NGV; ++gm) {
        const uint32_t pr = vp[c][gm];
        const float vs = on ? h2f(pr & 0xffffu) : 0.0f, vz = on ? h2f(pr >> 16) : 0.0f;
        zacc[0][gm] += p[0][c] * (vz + Lc * vs);
        zacc[1][gm] += p[1][c] * (vz + Lc * vs);
        const float pv0 = (p[0][c] * f) * vs, pv1 = (p[1][c] * f) * vs;
        const _Float16 a0 = (_Float16)pv0, a1 = (_Float16)pv1;
        uint2 wv;
        wv.x = pack_h2(a0, (_Float16)(pv0 - (float)a0));
        wv.y = pack_h2(a1, (_Float16)(pv1 - (float)a1));
        // (lanes of heads >= G store zeros: their p is 0)
        *reinterpret_cast<uint2*>(&s_p[w][gm][pos * kPP + la * 4]) = wv;
      }
    }
    load_vp(min(i + 1, nchunk - 1));
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // ---------------------------------------------------------- PV
    // The chunk accumulates into fresh MFMA tiles that are then added to the running output in fp32: the
    // code sum p * v_scale * code is much larger than the output it cancels down to (the group zeros'
    // term is added separately), and a long chain of MFMA accumulations would lose that difference.
    const int tok = lj < 8 ? 8 * la + lj : 32 + 8 * la + (lj - 8);
#pragma unroll
    for (int gm = 0; gm < NGV; ++gm) {
      floatx4 ob[8 / NGV];
#pragma unroll
      for (int tt = 0; tt < 8 / NGV; ++tt) ob[tt] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
      u32x4 pa[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int base = 32 * kb + 8 * la + (lj >> 2);
        const v2i x0 = lds_tr16(&s_p[w][gm][base * kPP + (lj & 3) * 4]);
        const v2i x1 = lds_tr16(&s_p[w][gm][(base + 4) * kPP + (lj & 3) * 4]);
        pa[kb] = u32x4{(uint32_t)x0.x, (uint32_t)x0.y, (uint32_t)x1.x, (uint32_t)x1.y};
      }
#pragma unroll
      for (int tt = 0; tt < 8 / NGV; ++tt) {
        const int t = gm * (8 / NGV) + tt;  // output tile (16 channels) inside V group gm
        const v2i x = lds_tr4(sv + tok * kVP + 8 * t);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          // high nibbles (odd tokens) complemented: 15 - code
          const uint32_t wd = (uint32_t)(kb ? x.y : x.x) ^ 0xF0F0F0F0u, w8 = wd >> 8;
          const u32x4 b = {wd & kLo4, wd & kHi4, w8 & kLo4, w8 & kHi4};
          ob[tt] = mfma16(pa[kb], b, ob[tt]);
        }
      }
#pragma unroll
      for (int tt = 0; tt < 8 / NGV; ++tt) o[gm * (8 / NGV) + tt] += ob[tt] * pv_inv;
    }
    __builtin_amdgcn_wave_barrier();
  };

  // The next block's codes are in flight while this block is computed; its A operand is built after this
  // block's logits (the two LDS buffers alternate) and published by the barrier that ends the step.
  for (int i = 0; i < nchunk; i += 2) {
    load(rb, min(i + 1, nchunk - 1));
    __builtin_amdgcn_sched_barrier(0);
    process(ra, i);
    __builtin_amdgcn_sched_barrier(0);
    if (i + 1 < nchunk) build_block(rb.kc, (i + 1) & 1);
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
    if (i + 1 >= nchunk) break;
    load(ra, min(i + 2, nchunk - 1));
    __builtin_amdgcn_sched_barrier(0);
    process(rb, i + 1);
    __builtin_amdgcn_sched_barrier(0);
    if (i + 2 < nchunk) build_block(ra.kc, (i + 2) & 1);
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
  }

  // ---------------------------------------------------------------- merge the four waves
  // A wave whose largest logit of some head lies beyond kPreciseAbove (base-2 units) redoes its rows with fp64
  // logits (checked once, after the loop, which has no register to spare), writing its merge slots itself.
  const bool big = (ok0 && m_run[0] != kNegInf && fabsf(m_run[0]) > kPreciseAbove) ||
                   (ok1 && m_run[1] != kNegInf && fabsf(m_run[1]) > kPreciseAbove);
  if (__builtin_amdgcn_ballot_w64(big) != 0) {
    auto qv = [&](int j, int c) __attribute__((always_inline)) -> double {
      return g.rotate ? (double)s_q[j][c]
                      : (double)h2f(a.q[((size_t)seq * a.num_q_heads + h * G + j) * D + c]) * a.q_scale64;
    };
    auto tok = [&](int p, int i, const uint8_t*& tile, int& row) __attribute__((always_inline)) -> bool {
      tile = pool_h + (size_t)s_tbl[p] * tstride;
      row = 64 * w + i;
      const int pos = (b0 + s_col[p]) * kRows + row;
      const uint32_t mw = (mask_row && pos < len) ? mask_row[pos >> 5] : 0u;
      return pos < len && !((mw >> (row & 31)) & 1u);
    };
    // scratch: this wave's V staging area (s_p is aliased by the merge slots of other waves)
    precise_wave_pass<D, D, G>(g, nchunk, tok, qv, reinterpret_cast<float*>(sv), &s_wm[w][0], &s_wl[w][0],
                               &s_wacc[w][0][0]);
  } else {
    const float lt0 = row_sum16(l_run[0]), lt1 = row_sum16(l_run[1]);
    float zt[2][NGV];
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int gm = 0; gm < NGV; ++gm) zt[u][gm] = row_sum16(zacc[u][gm]);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int hq = h0 + u;
      if (hq < G) {
        if (lj == 0) {
          s_wm[w][hq] = m_run[u];
          s_wl[w][hq] = u ? lt1 : lt0;
        }
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const int gm = t / (8 / NGV);
          float zz = 0.0f;
#pragma unroll
          for (int q = 0; q < NGV; ++q) zz = q == gm ? zt[u][q] : zz;
          s_wacc[w][hq][16 * t + lj] = (o[t][2 * u] + o[t][2 * u + 1]) * kTwo24 + zz;
        }
      }
    }
  }
  __syncthreads();
  if (ns == 1 && n_pre == 0) {
    __shared__ int s_cnt[4];
    __shared__ float s_o[D];
    const int n_sent = count_sentinels<256>(a, seq, len, tid, s_cnt);
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
      finalize_head<D, 256>(g, a, seq, h * G + jj, len, n_sent, M, L, acc, tid, s_o);
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
  splitk_arrive<D, G>(g, a, seq, h, split, ns, len, tid, s_pm, s_pl, &s_pacc[0][0], &s_wacc[0][0][0], n_pre);
}

template <int VG>
hipError_t launch_vg(const TileGeom& g, const DecodeArgs& a, hipStream_t stream) {
  const dim3 grid(a.plan.n_splits, g.H, a.n_seqs);
  switch (a.G) {
#define KVQ_KCHAN_CASE(GG) \
  case GG: hipLaunchKernelGGL((decode_kchan_k<GG, VG>), grid, dim3(256), 0, stream, g, a); break;
    KVQ_KCHAN_CASE(1)
    KVQ_KCHAN_CASE(2)
    KVQ_KCHAN_CASE(3)
    KVQ_KCHAN_CASE(4)
    KVQ_KCHAN_CASE(5)
    KVQ_KCHAN_CASE(6)
    KVQ_KCHAN_CASE(7)
    KVQ_KCHAN_CASE(8)
#undef KVQ_KCHAN_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

// Layouts with this kernel: head_dim 128, K grouped per channel, V groups of 32 or 64, G = 1..8.
bool decode_kchan_supported(const TileGeom& g, int G) {
  return g.d == 128 && g.dv == 128 && g.kg < 0 && (g.vg == 32 || g.vg == 64) && G >= 1 && G <= 8;
}

hipError_t launch_decode_kchan(const TileGeom& g, const DecodeArgs& a, hipStream_t stream) {
  return g.vg == 32 ? launch_vg<32>(g, a, stream) : launch_vg<64>(g, a, stream);
}

}  // namespace kvq
