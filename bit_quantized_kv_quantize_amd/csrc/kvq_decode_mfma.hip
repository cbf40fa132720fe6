// kvq_decode_mfma.hip - decode attention over 4-bit per-token-grouped tiles on the matrix cores.
//
// Same computation as the generic kernel (single-token decode attention reading the packed Q4 cache of
// "Agent Memory Below the Prompt", technical summary 2.1, with GQA from 2.2, sentinel slots of the
// IntentKV article and the rotated cache of the UltraQuant article), organised for gfx950:
//
// * Both contractions run as v_mfma_f32_16x16x32_f16. For QK the A operand holds the query rows, one
//   MFMA row per (query head, K group) so each group's partial dot product stays separate and its scale
//   and zero apply afterwards; the B operand is the K codes of 16 tokens. For PV the A operand holds
//   p * v_scale, one row per (query head, V group); the B operand is the V codes of 32 tokens.
// * Codes become fp16 operands without arithmetic: masking a packed word with 0x000F000F leaves two
//   nibbles as fp16 subnormals n * 2^-24 (0x00F000F0 gives 16 n * 2^-24). Subnormal fp16 inputs are
//   exact in the MFMA, and the 2^24 / 16 factors fold into the scales. V codes are transposed to
//   token-major operands in registers with byte permutes of 8 rows.
// * The query and p * v_scale are each split into fp16 hi + lo parts (two MFMAs on the same codes): a
//   dequantised value is scale * code + zero, a difference of two larger terms, so a single fp16
//   rounding of the scaled operand would cost up to 2^-12 of scale * 15 per element.
// * Each wave owns 64 rows of every block and keeps its own online softmax (16-lane DPP reductions, no
//   block-wide barrier in the token loop); the four waves merge at the end of the split. With one split
//   per (sequence, KV head) the workgroup finalises the output itself; otherwise the split that arrives
//   last merges all splits' partials (splitk_arrive) - one kernel per call either way.
#include "kvq_decode_mfma_common.hpp"
#include "kvq_decode_precise.hpp"

namespace kvq {
namespace {

using namespace dec;

// Grid (n_splits, H_kv, n_seqs), 256 threads = 4 waves; wave w owns rows 64w .. 64w+63 of each block.
// D = K's head dim (and the query's), DV = V's (and the output's): 128/128, 256/256 or, for MLA pools,
// 192/128.
template <int D, int DV, int G, int KG, int VG>
__global__ __launch_bounds__(256, D >= 192 ? 1 : 2) void decode_mfma_k(TileGeom g, DecodeArgs a) {
  constexpr int NGK = D / KG;      // K groups per row
  constexpr int NGV = DV / VG;     // V groups per row
  constexpr int HPL = (G + 3) / 4; // query heads per 16-lane row group
  static_assert(HPL * NGK <= 4 && HPL * NGV <= 4, "MFMA rows: heads x groups per lane group <= 4");
  constexpr int KW = D / 32;       // K words per lane per row = QK k-steps
  constexpr int VW = DV / 128;     // V words per lane per row
  constexpr int NTILE = 8 * VW;    // PV output tiles of 16 channels
  constexpr int PSTR = 72;         // LDS row stride (halves) of the p * v_scale tiles
  static_assert((D == 128 || D == 192 || D == 256) && (DV == 128 || DV == 256), "head dims");

  __shared__ float s_q[G][D];
  __shared__ float s_qsum[G][NGK];
  __shared__ __attribute__((aligned(16))) _Float16 s_p[4][2][16][PSTR];  // [wave][hi, lo][row][token]
  __shared__ float s_wm[4][G], s_wl[4][G];
  __shared__ float s_wacc[4][G][DV];
  __shared__ int s_tbl[kMaxSplitBlocks];
  __shared__ uint32_t s_mask[kMaxSplitBlocks * (kRows / 32)];

  const int split = blockIdx.x, h = blockIdx.y, seq = blockIdx.z;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, la = l >> 4, lj = l & 15;
  const int ns = a.plan.n_splits;
  const int len = a.seq_lens[seq];
  const int nblk = (len + kRows - 1) / kRows;
  int b0, b1;
  split_range(split, a.plan.n_splits, nblk, b0, b1);
  const uint32_t* mask_row = a.mask ? a.mask + (size_t)seq * a.mask_words : nullptr;

  if (b0 >= b1) {
    if (ns == 1) {  // empty sequence: the output row still has to be written
      __shared__ int s_cnt0[4];
      const int n_sent = count_sentinels<256>(a, seq, len, tid, s_cnt0);
      for (int jj = 0; jj < G; ++jj)
        finalize_head<DV, 256>(g, a, seq, h * G + jj, len, n_sent, kNegInf, 0.0f, 0.0f, tid, &s_wacc[0][0][0]);
    } else {
      if (tid < G) {
        s_wm[0][tid] = kNegInf;
        s_wl[0][tid] = 0.0f;
      }
      for (int i = tid; i < G * DV; i += 256) s_wacc[1][i / DV][i % DV] = 0.0f;
      __syncthreads();
      splitk_arrive<DV, G>(g, a, seq, h, split, ns, len, tid, &s_wm[0][0], &s_wl[0][0], &s_wacc[1][0][0],
                           &s_wacc[0][0][0]);
    }
    return;
  }

  const int r0 = w * 64;
  // Raw codes and parameters of one block for this wave's 64 rows. Two sets alternate so the loads of
  // block lb + 1 are in flight while block lb is computed.
  struct Raw {
    uint32_t kraw[4][KW];
    uint32_t kpar[4][NGK], vpar[4][NGV];
    uint32_t vraw[2][8][VW];
  };
  // Every load of the loop is unconditional and only fetches codes and parameters (the block table and
  // sentinel words of the split sit in LDS): with straight-line loads the compiler waits only for the
  // block being computed.
  auto load = [&](Raw& r, int phys) __attribute__((always_inline)) {
    const uint8_t* tile = a.pool + ((size_t)phys * g.H + h) * g.tile_bytes;
    // ------------------------------------------------------------ loads for this wave's 64 rows
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int row = r0 + 16 * c + lj;
      if constexpr (KW % 4 == 0) {
        const uint4* kp = reinterpret_cast<const uint4*>(tile + g.kcode(row) + la * KW * 4);
#pragma unroll
        for (int q4 = 0; q4 < KW / 4; ++q4) {
          const uint4 v4 = kp[q4];
          r.kraw[c][4 * q4 + 0] = v4.x;
          r.kraw[c][4 * q4 + 1] = v4.y;
          r.kraw[c][4 * q4 + 2] = v4.z;
          r.kraw[c][4 * q4 + 3] = v4.w;
        }
      } else {  // 6 words (K head dim 192): three 8-byte loads
        const uint2* kp = reinterpret_cast<const uint2*>(tile + g.kcode(row) + la * KW * 4);
#pragma unroll
        for (int q2 = 0; q2 < KW / 2; ++q2) {
          const uint2 v2 = kp[q2];
          r.kraw[c][2 * q2 + 0] = v2.x;
          r.kraw[c][2 * q2 + 1] = v2.y;
        }
      }
      const uint32_t* kpp = reinterpret_cast<const uint32_t*>(tile + g.kpar(row));
      const uint32_t* vpp = reinterpret_cast<const uint32_t*>(tile + g.vpar(row));
#pragma unroll
      for (int gm = 0; gm < NGK; ++gm) r.kpar[c][gm] = kpp[gm];
#pragma unroll
      for (int gm = 0; gm < NGV; ++gm) r.vpar[c][gm] = vpp[gm];
    }
    // sentinel bits of this wave's 64 rows: two mask words (zero past the mask's end)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int row = r0 + 32 * kb + 8 * la + e;
        const uint32_t* vp = reinterpret_cast<const uint32_t*>(tile + g.vcode(row, 4));
#pragma unroll
        for (int vw = 0; vw < VW; ++vw) r.vraw[kb][e][vw] = vp[lj + 16 * vw];
      }

  };
  // The first block's codes are requested before the query set-up, so their latency overlaps it.
  Raw ra, rb;
  load(ra, a.block_table[(size_t)seq * a.max_blocks_per_seq + b0]);

  // ---------------------------------------------------------------- block table and query operands
  for (int i = tid; i < b1 - b0; i += 256) s_tbl[i] = a.block_table[(size_t)seq * a.max_blocks_per_seq + b0 + i];
  if (mask_row) {  // sentinel words of this split's slots (zero past the mask's end)
    const int wbase = b0 * (kRows / 32), nw = (b1 - b0) * (kRows / 32);
    for (int i = tid; i < nw; i += 256) s_mask[i] = wbase + i < a.mask_words ? mask_row[wbase + i] : 0u;
  }
  for (int i = tid; i < G * D; i += 256)
    s_q[i / D][i % D] = h2f(a.q[((size_t)seq * a.num_q_heads + h * G + i / D) * D + i % D]) * a.q_scale;
  for (int i = tid; i < 4 * 2 * 16 * PSTR; i += 256) (&s_p[0][0][0][0])[i] = (_Float16)0.0f;
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
  for (int i = tid; i < G * NGK; i += 256) {
    float sum = 0.0f;
    for (int c = 0; c < KG; ++c) sum += s_q[i / NGK][(i % NGK) * KG + c];
    s_qsum[i / NGK][i % NGK] = sum;
  }
  __syncthreads();

  // QK A operand: row lj = 4*ai + ri -> head ai*HPL + ri/NGK, K group ri%NGK; lane group la supplies words
  // la*KW .. la*KW+KW-1, k-step s uses word la*KW + s. Element e of an operand is nibble nib(e) of the
  // word, pre-divided by 16 for the high nibbles (e & 2) to match the unpacking.
  u32x4 qa_hi[KW], qa_lo[KW];
  {
    const int ai = lj >> 2, ri = lj & 3;
    const int jj = ai * HPL + ri / NGK, gam = ri % NGK;
    const bool valid = ri < HPL * NGK && jj < G;
#pragma unroll
    for (int s = 0; s < KW; ++s) {
      const int word = la * KW + s;
      const bool in_group = valid && (word * 8) / KG == gam;
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        _Float16 hi[2], lo[2];
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          const int e = 2 * p + k;
          const int nib = (e >> 1) + 4 * (e & 1);  // 0,4,1,5,2,6,3,7
          const float sc = (e & 2) ? 0.0625f : 1.0f;
          const float v = in_group ? s_q[jj][word * 8 + nib] * sc : 0.0f;
          hi[k] = (_Float16)v;
          lo[k] = (_Float16)(v - (float)hi[k]);
        }
        qa_hi[s][p] = pack_h2(hi[0], hi[1]);
        qa_lo[s][p] = pack_h2(lo[0], lo[1]);
      }
    }
  }
  float qsum[HPL][NGK];
#pragma unroll
  for (int u = 0; u < HPL; ++u)
#pragma unroll
    for (int gm = 0; gm < NGK; ++gm) qsum[u][gm] = (la * HPL + u) < G ? s_qsum[la * HPL + u][gm] : 0.0f;

  float m_run[HPL], l_run[HPL], zacc[HPL][NGV];
#pragma unroll
  for (int u = 0; u < HPL; ++u) {
    m_run[u] = kNegInf;
    l_run[u] = 0.0f;
#pragma unroll
    for (int gm = 0; gm < NGV; ++gm) zacc[u][gm] = 0.0f;
  }
  floatx4 o[NTILE];
#pragma unroll
  for (int t = 0; t < NTILE; ++t) o[t] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
  float alpha_u[HPL];

  const uint32_t sel_base = (0x0Cu << 8) | (0x0Cu << 24);

  auto process = [&](const Raw& r, int lb) __attribute__((always_inline)) {
    // ------------------------------------------------------------ logits: QK on the matrix cores
    // The four 16-token chunks accumulate side by side (independent MFMA chains).
    floatx4 acc[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[c] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int s = 0; s < KW; ++s)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const uint32_t wd = r.kraw[c][s], w8 = wd >> 8;
        const u32x4 b = {wd & 0x000F000Fu, wd & 0x00F000F0u, w8 & 0x000F000Fu, w8 & 0x00F000F0u};
        acc[c] = mfma16(qa_hi[s], b, acc[c]);
        acc[c] = mfma16(qa_lo[s], b, acc[c]);
      }
    float sc[HPL][4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int pos = lb * kRows + r0 + 16 * c + lj;
      const uint32_t mword = mask_row ? s_mask[(lb - b0) * (kRows / 32) + (r0 >> 5) + (c >> 1)] : 0u;
      const bool live = pos < len && !((mword >> ((16 * c + lj) & 31)) & 1u);
#pragma unroll
      for (int u = 0; u < HPL; ++u) {
        float dotq = 0.0f, zq = 0.0f;
#pragma unroll
        for (int gm = 0; gm < NGK; ++gm) {
          dotq += h2f(r.kpar[c][gm] & 0xffffu) * acc[c][u * NGK + gm];
          zq += h2f(r.kpar[c][gm] >> 16) * qsum[u][gm];
        }
        const bool head_ok = (G % 4 == 0) || (la * HPL + u < G);
        sc[u][c] = (live && head_ok) ? dotq * kTwo24 + zq : kNegInf;
      }
    }

    // ------------------------------------------------------------ online softmax of this wave's rows
    float p[HPL][4];
    bool rescale = false;
#pragma unroll
    for (int u = 0; u < HPL; ++u) {
      float mx = fmaxf(fmaxf(sc[u][0], sc[u][1]), fmaxf(sc[u][2], sc[u][3]));
      mx = row_max16(mx);
      const float mnew = fmaxf(m_run[u], mx);
      const float alpha = mnew == m_run[u] ? 1.0f : __builtin_amdgcn_exp2f(m_run[u] - mnew);
      rescale |= alpha != 1.0f;
      float ps = 0.0f;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        p[u][c] = __builtin_amdgcn_exp2f(sc[u][c] - mnew);  // -inf - finite -> 0; an all-dead row keeps 0
        p[u][c] = mnew == kNegInf ? 0.0f : p[u][c];
        ps += p[u][c];
      }
      l_run[u] = l_run[u] * alpha + ps;
      m_run[u] = mnew;
      alpha_u[u] = alpha;
    }
    if (__builtin_amdgcn_ballot_w64(rescale)) {  // wave-uniform: skip when no running max moved
#pragma unroll
      for (int u = 0; u < HPL; ++u) {
#pragma unroll
        for (int gm = 0; gm < NGV; ++gm) zacc[u][gm] *= alpha_u[u];
#pragma unroll
        for (int t = 0; t < NTILE; ++t)
#pragma unroll
          for (int gm = 0; gm < NGV; ++gm) o[t][u * NGV + gm] *= alpha_u[u];
      }
    }

    // p * v_scale to LDS (A operand of PV), p * v_zero into the per-lane zero term. Dead slots have p = 0
    // and their (possibly uninitialised) parameters are selected away, never multiplied.
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int u = 0; u < HPL; ++u) {
#pragma unroll
        for (int gm = 0; gm < NGV; ++gm) {
          const float pp = p[u][c];
          const bool on = pp != 0.0f;
          const float vs = on ? h2f(r.vpar[c][gm] & 0xffffu) : 0.0f;
          const float vz = on ? h2f(r.vpar[c][gm] >> 16) : 0.0f;
          const float pv = pp * vs;
          zacc[u][gm] += pp * vz;
          const _Float16 pv_hi = (_Float16)pv;
          const int row = la * 4 + u * NGV + gm;
          if ((G % 4 == 0) || (la * HPL + u < G)) {
            s_p[w][0][row][16 * c + lj] = pv_hi;
            s_p[w][1][row][16 * c + lj] = (_Float16)(pv - (float)pv_hi);
          }
        }
      }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // ------------------------------------------------------------ PV on the matrix cores
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const u32x4 pa_hi = *reinterpret_cast<const u32x4*>(&s_p[w][0][lj][32 * kb + 8 * la]);
      const u32x4 pa_lo = *reinterpret_cast<const u32x4*>(&s_p[w][1][lj][32 * kb + 8 * la]);
#pragma unroll
      for (int vw = 0; vw < VW; ++vw)
#pragma unroll
        for (int bb = 0; bb < 4; ++bb) {
          const uint32_t sel = sel_base | (uint32_t)bb | ((uint32_t)(4 + bb) << 16);
          u32x4 blo, bhi;
#pragma unroll
          for (int pq = 0; pq < 4; ++pq) {
            const uint32_t x = __builtin_amdgcn_perm(r.vraw[kb][2 * pq + 1][vw], r.vraw[kb][2 * pq][vw], sel);
            blo[pq] = x & 0x000F000Fu;
            bhi[pq] = x & 0x00F000F0u;
          }
          o[vw * 8 + 2 * bb] = mfma16(pa_hi, blo, o[vw * 8 + 2 * bb]);
          o[vw * 8 + 2 * bb] = mfma16(pa_lo, blo, o[vw * 8 + 2 * bb]);
          o[vw * 8 + 2 * bb + 1] = mfma16(pa_hi, bhi, o[vw * 8 + 2 * bb + 1]);
          o[vw * 8 + 2 * bb + 1] = mfma16(pa_lo, bhi, o[vw * 8 + 2 * bb + 1]);
        }
    }
    __builtin_amdgcn_wave_barrier();
  };
  const int blast = b1 - 1;
  for (int lb = b0; lb < b1; lb += 2) {
    // sched_barrier keeps the next block's loads ahead of this block's arithmetic, so they are in flight
    // while it runs (the scheduler would otherwise sink them below the first MFMAs)
    load(rb, s_tbl[min(lb + 1, blast) - b0]);  // past the end: reloads the last block (an L2 hit), unused
    __builtin_amdgcn_sched_barrier(0);
    process(ra, lb);
    if (lb + 1 >= b1) break;
    load(ra, s_tbl[min(lb + 2, blast) - b0]);
    __builtin_amdgcn_sched_barrier(0);
    process(rb, lb + 1);
  }

  // ---------------------------------------------------------------- merge the four waves
  // A wave whose largest logit of some head lies beyond kPreciseAbove (base-2 units) redoes its rows with fp64
  // logits. (This kernel checks the largest logit once, after its loop, rather than each logit's terms as the
  // row-list kernel does: its block loop has no register to spare. Terms beyond the bound that cancel to a
  // moderate logit are not caught here; the tokens that carry the weight have logits near the largest.)
  bool big = false;
#pragma unroll
  for (int u = 0; u < HPL; ++u) big |= m_run[u] != kNegInf && fabsf(m_run[u]) > kPreciseAbove;
  const bool wave_big = __builtin_amdgcn_ballot_w64(big) != 0;
  if (wave_big) {
    // this wave's rows again with fp64 logits; the pass writes the wave's merge slots itself
    auto qv = [&](int j, int c) __attribute__((always_inline)) -> double {
      return g.rotate ? (double)s_q[j][c]
                      : (double)h2f(a.q[((size_t)seq * a.num_q_heads + h * G + j) * D + c]) * a.q_scale64;
    };
    auto tok = [&](int p, int i, const uint8_t*& tile, int& row) __attribute__((always_inline)) -> bool {
      tile = a.pool + ((size_t)s_tbl[p] * g.H + h) * g.tile_bytes;
      row = r0 + i;
      const uint32_t mword = mask_row ? s_mask[p * (kRows / 32) + (row >> 5)] : 0u;
      return (b0 + p) * kRows + row < len && !((mword >> (row & 31)) & 1u);
    };
    precise_wave_pass<D, DV, G>(g, b1 - b0, tok, qv, reinterpret_cast<float*>(&s_p[w][0][0][0]), &s_wm[w][0],
                                &s_wl[w][0], &s_wacc[w][0][0]);
  } else {
#pragma unroll
  for (int u = 0; u < HPL; ++u) {
    const float lt = row_sum16(l_run[u]);
    float zt[NGV];
#pragma unroll
    for (int gm = 0; gm < NGV; ++gm) zt[gm] = row_sum16(zacc[u][gm]);
    const int jj = la * HPL + u;
    if (jj < G) {
      if (lj == 0) {
        s_wm[w][jj] = m_run[u];
        s_wl[w][jj] = lt;
      }
#pragma unroll
      for (int vw = 0; vw < VW; ++vw)
#pragma unroll
        for (int m = 0; m < 8; ++m) {
          const int c = vw * 128 + 8 * lj + m;
          const int gc = c / VG;
          float val = 0.0f;
#pragma unroll
          for (int gm = 0; gm < NGV; ++gm)
            if (gm == gc) val = o[vw * 8 + m][u * NGV + gm] * ((m & 1) ? kTwo20 : kTwo24) + zt[gm];
          s_wacc[w][jj][c] = val;
        }
    }
  }
  }
  __syncthreads();
  if (ns == 1) {
    // the whole sequence was this workgroup's: finalise the rows here
    __shared__ int s_cnt[4];
    __shared__ float s_o[DV];
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
          if (tid < DV) acc += s_wacc[ww][jj][tid] * sc_w;
          L += s_wl[ww][jj] * sc_w;
        }
      }
      finalize_head<DV, 256>(g, a, seq, h * G + jj, len, n_sent, M, L, acc, tid, s_o);
    }
    return;
  }
  // merge the four waves into this split's partials (staged in LDS), then arrive
  __shared__ float s_pm[G], s_pl[G];
  __shared__ float s_pacc[G][DV];
  for (int i = tid; i < G * DV; i += 256) {
    const int jj = i / DV, c = i % DV;
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
  splitk_arrive<DV, G>(g, a, seq, h, split, ns, len, tid, s_pm, s_pl, &s_pacc[0][0], &s_wacc[0][0][0]);
}

template <int D, int DV, int G, int KG, int VG>
hipError_t launch_one(const TileGeom& g, const DecodeArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL((decode_mfma_k<D, DV, G, KG, VG>), dim3(a.plan.n_splits, g.H, a.n_seqs), dim3(256), 0,
                     stream, g, a);
  return hipGetLastError();
}

}  // namespace

// Layouts with a compiled matrix-core kernel: 4-bit pools (not mixed) with per-token K and V groups of 64;
// head dims 128, 256, or K 192 with V 128 (MLA).
bool decode_mfma_supported(const TileGeom& g, int G) {
  if (g.mixed || g.kg != 64 || g.vg != 64) return false;
  if (g.d == 128 && g.dv == 128) return G == 1 || G == 2 || G == 4 || G == 8;
  if (g.d == 256 && g.dv == 256) return G == 1 || G == 2 || G == 4;
  if (g.d == 192 && g.dv == 128) return G == 1 || G == 2 || G == 4;
  return false;
}

hipError_t launch_decode_mfma(const TileGeom& g, const DecodeArgs& a, hipStream_t stream) {
  if (g.d == 128) {
    switch (a.G) {
      case 1: return launch_one<128, 128, 1, 64, 64>(g, a, stream);
      case 2: return launch_one<128, 128, 2, 64, 64>(g, a, stream);
      case 4: return launch_one<128, 128, 4, 64, 64>(g, a, stream);
      case 8: return launch_one<128, 128, 8, 64, 64>(g, a, stream);
    }
  } else if (g.d == 256) {
    switch (a.G) {
      case 1: return launch_one<256, 256, 1, 64, 64>(g, a, stream);
      case 2: return launch_one<256, 256, 2, 64, 64>(g, a, stream);
      case 4: return launch_one<256, 256, 4, 64, 64>(g, a, stream);
    }
  } else if (g.d == 192) {
    switch (a.G) {
      case 1: return launch_one<192, 128, 1, 64, 64>(g, a, stream);
      case 2: return launch_one<192, 128, 2, 64, 64>(g, a, stream);
      case 4: return launch_one<192, 128, 4, 64, 64>(g, a, stream);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace kvq
