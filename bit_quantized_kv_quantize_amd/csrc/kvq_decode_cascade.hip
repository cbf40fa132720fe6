// kvq_decode_cascade.hip - decode attention over the blocks that several sequences of a batch share, for
// head_dim 128 pools whose K is grouped per channel over each 256-token block (the long shared-prefix serving
// workload of the UltraQuant article's technology section, the prefix cache of the IntentKV article's section
// on the hidden cost of dropping old tokens, with the prefix reuse of "Agent Memory Below the Prompt",
// technical summary 2.1-2.2, and its packed-block decode).
//
// A block that several sequences map to (a shared prompt prefix, also one shared by a subset of the batch) is
// read once for all of them. The planning kernel groups the sequences of every block range by the physical
// block at the range's first logical block (an inverted index of the block tables) and flags, per sequence
// and logical block, the blocks the cascade takes; the work items are (block range, KV head, row group), a
// row being one (member sequence, query head) pair and a row group up to eight 16-row tiles, one per wave.
// An item's partial softmax state per row goes to the split-K workspace; the per-sequence kernel
// (decode_kchan_k) then skips the flagged blocks and merges these partials with its own.
//
// The blocks are walked in 64-token chunks. All 512 threads stage a chunk once for the eight waves: its K codes
// as stored, its V rows dequantised to fp16 (v_scale * code + v_zero, one rounding) and, with a block's first
// chunk, the block's K channel parameters. Each wave then takes its 16 rows against the chunk:
// * QK token-major on the matrix cores (v_mfma_f32_16x16x32_f16): A = the K codes of 16 tokens as exact fp16
//   subnormals (lane = token), B = q_c s_c of the wave's 16 rows as fp16 hi and lo (two MFMAs into one
//   accumulator), rebuilt from the fp32 query in LDS at every block; the channel zeros enter as the
//   per-row constant sum_c q_c z_c (q . k_t = sum_c (q_c s_c) code_tc + sum_c q_c z_c).
// * The logits of a row sit in one column of the result: the row maximum is four lanes' worth of in-lane
//   maxima, and p (fp16) is already laid out as the B operand of PV. A row whose sequence does not take the
//   block sees its logits as -inf.
// * PV channel-major: A = the staged fp16 V rows through the 16-bit LDS transpose load (lane = channel),
//   B = p. The values are centred on zero, so neither operand needs a hi/lo split.
// The result of a wave is its rows' partial state over the item's blocks; no merge inside the workgroup.
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

// Exclusive prefix sums of x[0 .. n) in place (n <= 2 * blockDim.x = 512) and their total, by all 256 threads;
// s_w: four ints of scratch.
__device__ int block_scan(int* x, int n, int tid, int* s_w) {
  const int i0 = 2 * tid, i1 = 2 * tid + 1;
  const int a0 = i0 < n ? x[i0] : 0, a1 = i1 < n ? x[i1] : 0;
  int v = a0 + a1, incl = v;
  const int lane = tid & 63, w = tid >> 6;
#pragma unroll
  for (int d = 1; d < 64; d *= 2) {
    const int y = __shfl_up(incl, d);
    if (lane >= d) incl += y;
  }
  if (lane == 63) s_w[w] = incl;
  __syncthreads();
  int base = 0;
  for (int k = 0; k < w; ++k) base += s_w[k];
  const int total = s_w[0] + s_w[1] + s_w[2] + s_w[3];
  const int excl = base + incl - v;
  if (i0 < n) x[i0] = excl;
  if (i1 < n) x[i1] = excl + a0;
  __syncthreads();
  return total;
}

// Groups of sequences per block range (an inverted index of the block tables at the range's first logical
// block), one workgroup of 256 threads per range:
// * a sequence's key is its physical block at the range's first column if that block is full in it; the
//   sequences of one key form a group, led by its lowest-numbered member, and groups of two or more take the
//   cascade;
// * the members of those groups go to the range's member list, group by group in leader order with the
//   leader first, and each group's (member, query head) rows are cut into row groups of at most kCascRows
//   rows (the work items);
// * a member takes column c of the range when its block there is the leader's and full in it: its flag is
//   set (the per-sequence kernel skips the block for it) and the column's bit in its mask (the group's item
//   reads the block for it);
// * every row's partial slot of the range starts empty (m = -inf, l = 0), for the rows no group covers.
__global__ __launch_bounds__(256) void cascade_plan_k(TileGeom g, DecodeArgs a) {
  __shared__ int s_len[kCascMaxSeqs], s_key[kCascMaxSeqs], s_lead[kCascMaxSeqs], s_cnt[kCascMaxSeqs];
  __shared__ int s_rank[kCascMaxSeqs], s_pos[kCascMaxSeqs], s_mstart[kCascMaxSeqs], s_rstart[kCascMaxSeqs];
  __shared__ uint32_t s_m[kCascMaxSeqs][2];
  __shared__ int s_w[4];
  constexpr int kHashBits = 10, kHashSlots = 1 << kHashBits;  // 2 * kCascMaxSeqs slots
  static_assert(kHashSlots >= 2 * kCascMaxSeqs, "hash table at most half full");
  __shared__ int s_hkey[kHashSlots], s_hlead[kHashSlots], s_hcnt[kHashSlots], s_slot[kCascMaxSeqs];
  const int split = blockIdx.x, tid = threadIdx.x, n = a.n_seqs, S = a.plan.casc, G = a.G;
  const int MB = a.plan.max_blocks;
  const size_t mbs = (size_t)a.max_blocks_per_seq;
  int c0, c1;
  split_range(split, S, MB, c0, c1);
  const int ncol = c1 - c0;  // at most kCascRangeCols
  const size_t pslot = (size_t)(a.plan.stride - S + split);
  // The range's slice of the block tables goes to LDS with one round of loads when it fits (n * ncol <=
  // kSlice), else the table is read from memory where needed.
  constexpr int kSlice = 8192;
  __shared__ int s_tab[kSlice];
  const bool in_lds = n * ncol <= kSlice;
  auto table = [&](int s, int c) {
    return in_lds ? s_tab[s * ncol + c - c0] : a.block_table[(size_t)s * mbs + c];
  };
  for (int r = tid; r < n * a.num_q_heads; r += 256) {
    a.ws_ml[2 * ((size_t)r * a.plan.stride + pslot)] = kNegInf;
    a.ws_ml[2 * ((size_t)r * a.plan.stride + pslot) + 1] = 0.0f;
  }
  if (in_lds) {
    for (int base = 0; base < n * ncol; base += 4 * 256) {
      int x[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int idx = min(base + tid + 256 * k, n * ncol - 1), sq = idx / ncol;
        x[k] = a.block_table[(size_t)sq * mbs + c0 + idx - sq * ncol];
      }
#pragma unroll
      for (int k = 0; k < 4; ++k)
        if (base + tid + 256 * k < n * ncol) s_tab[base + tid + 256 * k] = x[k];
    }
  }
  for (int s = tid; s < n; s += 256) {
    s_len[s] = a.seq_lens[s];
    s_cnt[s] = 0;
    s_m[s][0] = 0u;
    s_m[s][1] = 0u;
  }
  for (int i = tid; i < kHashSlots; i += 256) {
    s_hkey[i] = -1;
    s_hlead[i] = 0x7fffffff;
    s_hcnt[i] = 0;
  }
  __syncthreads();
  for (int s = tid; s < n; s += 256) s_key[s] = (ncol > 0 && (c0 + 1) * kRows <= s_len[s]) ? table(s, c0) : -1;
  __syncthreads();
  // Groups through an LDS hash table keyed by physical block: a sequence claims its key's slot (linear
  // probing; at most kCascMaxSeqs keys in twice as many slots), the slot keeps the lowest member (the
  // leader) and counts the members; a member's place in its group is the order in which it arrived (the
  // place decides only which item row holds the sequence, not what is computed for it).
  for (int s = tid; s < n; s += 256) {
    const int key = s_key[s];
    int hs = -1, rank = 0;
    if (key >= 0) {
      hs = (int)(((uint32_t)key * 2654435761u) >> (32 - kHashBits));
      for (int probe = 0; probe < kHashSlots; ++probe) {
        const int prev = atomicCAS(&s_hkey[hs], -1, key);
        if (prev == -1 || prev == key) break;
        hs = (hs + 1) & (kHashSlots - 1);
      }
      atomicMin(&s_hlead[hs], s);
      rank = atomicAdd(&s_hcnt[hs], 1);
    }
    s_slot[s] = hs;
    s_rank[s] = rank;
  }
  __syncthreads();
  for (int s = tid; s < n; s += 256) {
    const int hs = s_slot[s];
    const int lead = hs >= 0 ? s_hlead[hs] : s;
    s_lead[s] = lead;
    if (lead == s) s_cnt[s] = hs >= 0 ? s_hcnt[hs] : 1;
  }
  __syncthreads();
  // the leader first in its group, the others after it in arrival order
  for (int s = tid; s < n; s += 256) {
    const int lead = s_lead[s], r = s_rank[s], rl = s_rank[lead];
    s_pos[s] = s == lead ? 0 : (r < rl ? r + 1 : r);
  }
  for (int s = tid; s < n; s += 256) {
    const bool grp = s_lead[s] == s && s_cnt[s] >= 2;
    s_mstart[s] = grp ? s_cnt[s] : 0;
    s_rstart[s] = grp ? (s_cnt[s] * G + kCascRows - 1) / kCascRows : 0;
  }
  __syncthreads();
  block_scan(s_mstart, n, tid, s_w);
  const int n_rg = block_scan(s_rstart, n, tid, s_w);
  int* perm = a.ws_cperm + (size_t)split * n;
  int* desc = a.ws_cdesc + (size_t)split * a.plan.casc_slots * 4;
  for (int s = tid; s < n; s += 256) {
    const int lead = s_lead[s];
    if (s_cnt[lead] < 2) continue;
    perm[s_mstart[lead] + s_pos[s]] = s;
    if (lead == s) {
      const int nrg = (s_cnt[s] * G + kCascRows - 1) / kCascRows;
      for (int q = 0; q < nrg; ++q) {
        int* d = desc + 4 * (s_rstart[s] + q);
        d[0] = s_mstart[s];
        d[1] = s_cnt[s];
        d[2] = q * kCascRows;
        d[3] = 0;
      }
    }
  }
  if (tid == 0) a.ws_cnrg[split] = n_rg;
  // every (sequence, column) pair of the range at once, four independent pairs per thread per round
  const int total = n * ncol;
  for (int base = 0; base < total; base += 4 * 256) {
    int x[4], y[4], sq[4], c[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int idx = min(base + tid + 256 * k, total - 1);
      sq[k] = idx / ncol;
      c[k] = idx - sq[k] * ncol;
      x[k] = table(sq[k], c0 + c[k]);
      y[k] = table(s_lead[sq[k]], c0 + c[k]);
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      if (base + tid + 256 * k >= total) continue;
      const bool take = s_cnt[s_lead[sq[k]]] >= 2 && (c0 + c[k] + 1) * kRows <= s_len[sq[k]] && x[k] == y[k];
      a.ws_cflag[(size_t)sq[k] * MB + c0 + c[k]] = take ? 1 : 0;
      if (take) atomicOr(&s_m[sq[k]][c[k] >> 5], 1u << (c[k] & 31));
    }
  }
  __syncthreads();
  uint64_t* cmask = a.ws_cmask + (size_t)split * n;
  for (int s = tid; s < n; s += 256) {
    const int lead = s_lead[s];
    if (s_cnt[lead] >= 2) cmask[s_mstart[lead] + s_pos[s]] = ((uint64_t)s_m[s][1] << 32) | s_m[s][0];
  }
}

// Persistent grid of at most kCascGrid workgroups looping over the work items: item i is row group k of
// block range r for KV head i mod H (items ordered by range, row group, head), so with H = 8 every item of
// KV head h runs on XCD h and the row groups of one block range share that XCD's L2.
template <int VG>
__global__ __launch_bounds__(64 * kCW, 1) void cascade_k(TileGeom g, DecodeArgs a) {
  constexpr int D = kD, NW = kCW;
  static_assert(VG == 32 || VG == 64, "V groups of 32 or 64");
  constexpr int kKBytes = 64 * kKP, kBuf = kKBytes + 64 * kVP;  // one staged chunk: K rows, then V rows
  __shared__ __attribute__((aligned(16))) uint8_t s_ring[3][kBuf];
  __shared__ __attribute__((aligned(16))) float2 s_kc[2][D];  // (scale / 16 on odd channels, zero) per channel
  __shared__ int s_tbl[kCascRangeCols], s_col[kCascRangeCols];
  __shared__ uint32_t s_cm[2];
  __shared__ int s_first[kCascMaxRanges + 1];
  // the scaled (and rotated) query of each lane: 32 channels at a pitch of 36 floats (conflict-free reads)
  __shared__ __attribute__((aligned(16))) float s_qv[NW][64][36];

  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, la = l >> 4, lj = l & 15;
  const int H = g.H, S = a.plan.casc, G = a.G;
  const int MB = a.plan.max_blocks;
  const uint8_t* pool_base = a.pool;
  const size_t tstride = (size_t)H * g.tile_bytes;
  if (tid < S) s_first[tid + 1] = a.ws_cnrg[tid];
  __syncthreads();
  if (tid == 0) {
    s_first[0] = 0;
    for (int r = 1; r <= S; ++r) s_first[r] += s_first[r - 1];
  }
  __syncthreads();
  const int n_items = s_first[S] * H;

  for (int item = blockIdx.x; item < n_items; item += gridDim.x) {
  const int h = item % H, ri = item / H;
  int split = 0;
  while (s_first[split + 1] <= ri) ++split;
  const int* d = a.ws_cdesc + ((size_t)split * a.plan.casc_slots + (ri - s_first[split])) * 4;
  const int m0 = d[0], n_mem = d[1], row_base = d[2];
  const int* members = a.ws_cperm + (size_t)split * a.n_seqs + m0;
  const int n_rows = min(kCascRows, n_mem * G - row_base);  // rows of this item
  const int NT = (n_rows + 15) / 16;
  const int lead = members[0];
  int c0, c1;
  split_range(split, S, MB, c0, c1);
  const uint8_t* pool_h = pool_base + (size_t)h * g.tile_bytes;

  // ------------------------------------------------------------ the group's blocks of [c0, c1)
  __syncthreads();  // the previous item's LDS is free
  const uint64_t* cmask = a.ws_cmask + (size_t)split * a.n_seqs + m0;
  if (tid < 2) s_cm[tid] = 0u;
  __syncthreads();
  // the group's columns: those any member takes
  for (int m = tid; m < n_mem; m += 64 * NW) {
    const uint64_t x = cmask[m];
    if ((uint32_t)x) atomicOr(&s_cm[0], (uint32_t)x);
    if ((uint32_t)(x >> 32)) atomicOr(&s_cm[1], (uint32_t)(x >> 32));
  }
  __syncthreads();
  const uint64_t cols = ((uint64_t)s_cm[1] << 32) | s_cm[0];
  const int nc = __builtin_popcountll(cols);
  if (tid < kCascRangeCols && ((cols >> tid) & 1u)) {
    const int b = __builtin_popcountll(cols & ((1ull << tid) - 1ull));
    s_tbl[b] = a.block_table[(size_t)lead * a.max_blocks_per_seq + c0 + tid];
    s_col[b] = tid;
  }
  __syncthreads();

  // this wave's rows: 16 w + lj of the item, lane (la, lj) holding channels 32 la .. 32 la + 31 of row lj in
  // the query; item row r is (member (row_base + r) / G, query head (row_base + r) mod G)
  const int row = 16 * w + lj;
  const bool wave_rows = w < NT;
  const bool row_ok = row < n_rows;
  const int gr = row_base + (row_ok ? row : 0);
  const int seq = members[gr / G], jj = gr % G;
  const uint64_t row_cols = row_ok ? cmask[gr / G] : 0ull;  // the columns this row's sequence takes
  const size_t pslot = (size_t)(a.plan.stride - S + split);  // this range's partial slot in each row
  const size_t pi = ((size_t)seq * a.num_q_heads + h * G + jj) * a.plan.stride + pslot;
  if (nc == 0) continue;  // (the row's slot stays empty, as the planning kernel left it)

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
  // A row that does not take the chunk's block (tk false) sees its logits as -inf: p = 0, state unchanged.
  auto softmax = [&](const floatx4 (&acc)[4], float zq, bool tk, u32x4 (&pb)[2])
                     __attribute__((always_inline)) -> float {
    float m4[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) m4[c] = fmaxf(fmaxf(acc[c][0], acc[c][1]), fmaxf(acc[c][2], acc[c][3]));
    const float mr = rows4_max(fmaxf(fmaxf(m4[0], m4[1]), fmaxf(m4[2], m4[3])));
    const float mx = tk ? __builtin_fmaf(mr, kTwo24, zq) : kNegInf;
    const float mnew = mx > m_run + kSlack ? mx : m_run;
    const float alpha = mnew == m_run ? 1.0f : __builtin_amdgcn_exp2f(m_run - mnew);
    const float off = tk ? zq - mnew : kNegInf;
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
  // whether this lane's row takes staged block b
  auto takes = [&](int b) __attribute__((always_inline)) {
    return ((row_cols >> s_col[min(b, nc - 1)]) & 1u) != 0u;
  };
  if (wave_rows) {
    floatx4 sc[4];
    float zc = build(0);
    bool tc = takes(0);
    qk(b_cur, sc);
    auto step = [&](Raw& nxt, int j, auto kc) __attribute__((always_inline)) {
      constexpr int k = decltype(kc)::value;
      floatx4 sn[4];
      const float zn = k == 3 ? build((j + 1) >> 2) : zc;
      const bool tn = k == 3 ? takes((j + 1) >> 2) : tc;
      qk(b_nxt, sn);
      u32x4 pb[2];
      const float alpha = softmax(sc, zc, tc, pb);
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
      tc = tn;
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
  if (wave_rows) {
    const float lsum = rows4_sum(l_run);
    if (row_ok) {
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
  }
  }  // items
}

}  // namespace

// Layouts of the per-channel-K kernel with V groups of 32 or 64.
bool decode_cascade_supported(const TileGeom& g, int G) {
  return g.d == 128 && g.dv == 128 && g.kg < 0 && !g.mixed && (g.vg == 32 || g.vg == 64) && G >= 1 && G <= 8;
}

hipError_t launch_decode_cascade(const TileGeom& g, const DecodeArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(cascade_plan_k, dim3(a.plan.casc), dim3(256), 0, stream, g, a);
  const long items = (long)a.plan.casc * a.plan.casc_slots * g.H;  // bound on the work items
  const dim3 grid((unsigned)std::min<long>(kCascGrid, items));
  if (g.vg == 32)
    hipLaunchKernelGGL(cascade_k<32>, grid, dim3(64 * kCW), 0, stream, g, a);
  else
    hipLaunchKernelGGL(cascade_k<64>, grid, dim3(64 * kCW), 0, stream, g, a);
  return hipGetLastError();
}

}  // namespace kvq
