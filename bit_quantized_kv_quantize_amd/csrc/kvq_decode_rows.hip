// kvq_decode_rows.hip - decode attention on the matrix cores for head_dim 128 pools with per-token K and V
// groups of 64 and GQA ratios 1, 2 and 4 (single-token decode attention over the packed cache of "Agent
// Memory Below the Prompt", technical summary 2.1-2.2, with the sentinel slots of the IntentKV article and
// the per-token bit widths of QKVShare's methodology).
//
// Work unit: a chunk of live rows of one (sequence, KV head) - 64 rows of 4-bit codes, 32 rows of 8-bit
// codes, 64 rows of 2-bit codes or 16 FP16 rows (8 KB of K and V, 4 KB for 2-bit chunks). Pure 4-bit pools
// without sentinel slots are read block by block (each wave takes 64 rows of every block of its split).
// Pools with sentinel slots or per-token widths are read as compacted row lists built by compact_rows_k:
// per sequence, the live rows of each width in slot order, so every chunk is of one width and sentinel
// rows are never fetched.
//
// Matrix-core layout (v_mfma_f32_16x16x32_f16 throughout):
// * MFMA row r = 4 h + 2 gamma + part: query head h, K (or V) group gamma, part 0/1 = fp16 hi/lo of the
//   operand. The hi and lo halves of the query and of p * v_scale share one MFMA (rows, not passes), so each
//   16-token slice of K costs one MFMA per 32 channels.
// * QK: B = K codes of 16 tokens (lane = token), unpacked without arithmetic: masking a packed word with
//   0x000F000F leaves two nibbles as fp16 subnormals n * 2^-24 (0x00F000F0 gives 16 n * 2^-24); 8-bit codes
//   are paired with byte permutes (bytes are exact subnormals too); 2-bit codes are masked field by field
//   (4^p n * 2^-24 for field p); FP16 rows are the operand as stored. The 2^24 and 1/16 (1/4^p) factors
//   fold into the group scales and the query.
// * PV: V rows are staged in LDS as loaded (lane = token; 2-bit codes widened to nibbles) and read back
//   transposed with the gfx950 LDS transpose loads (16 nibbles, 8 bytes or 4 halves per lane, one output
//   channel per lane), so the B operand of 32 tokens x 16 channels needs no per-element shuffling. The A operand (p * v_scale as hi/lo, one row per
//   (head, V group, part)) is written position-major and read with the 16-bit transpose load.
// Online softmax per wave (16-lane DPP reductions), the four waves merge at the end, and the split-K merge
// runs in the split that arrives last (splitk_arrive).
#include <type_traits>

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
__device__ __forceinline__ v2i lds_tr8(const void* p) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i*)const_cast<void*>(p));
}
__device__ __forceinline__ v2i lds_tr16(const void* p) {
  return __builtin_bit_cast(v2i, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)const_cast<void*>(p)));
}

constexpr uint32_t kLo4 = 0x000F000Fu, kHi4 = 0x00F000F0u;
// byte permute selector: bytes m and m + 4 of {hi:lo} into the low bytes of the two fp16 halves
__device__ __forceinline__ uint32_t pair_sel(int m) {
  return (uint32_t)m | (0x0Cu << 8) | ((uint32_t)(4 + m) << 16) | (0x0Cu << 24);
}

constexpr int kD = 128;
constexpr int kVP = 80;     // LDS row pitch (bytes) of staged 4-bit V rows
constexpr int kRP = 144;    // LDS row pitch (bytes) of whole staged 4-bit row records (streaming, K 128)
constexpr int kVP8 = 144;   // LDS row pitch (bytes) of staged 8-bit V rows
constexpr int kVP16 = 288;  // LDS row pitch (bytes) of staged FP16 V rows
constexpr int kPP = 20;     // halves per position of the position-major p * v_scale tile (16 rows + pad)

// ------------------------------------------------------------------------------------- row compaction
// Per sequence and width, the live rows in slot order as (physical block << 8 | row), and their counts:
// NWD = 2 lists (4-bit, 8-bit) for 4-bit pools and pools of 4- and 8-bit rows, NWD = 4 lists (4-bit, 8-bit,
// 2-bit, FP16) for pools of four widths. A slot is live when it is below seq_len and its sentinel bit is
// clear; its width comes from the pool header (KV head 0's tile: every head of a block holds the same
// per-token widths). Grid (n_seqs), 1024 threads. A wave takes 8 logical blocks at a time, 8 lanes per
// block and 32 rows per lane (one word of the sentinel mask): the waves count every block's live rows per
// width, the counts are scanned in the workspace, and the waves write each block's entries at its offsets.
constexpr int kCompactThreads = 1024;

template <int NWD>
struct RowBits {
  int b, phys;        // logical block (or -1 past the end), physical block
  uint32_t m[NWD];    // rows 32k .. 32k + 31 of the block (k = lane & 7), live and in width list i
};

// Bit j of the result set where 2-bit field j of the 64-bit (h1:h0) equals c.
__device__ __forceinline__ uint32_t fields_equal(uint32_t h0, uint32_t h1, uint32_t c) {
  auto one = [c](uint32_t h) {
    const uint32_t x = h ^ (c * 0x55555555u);  // equal fields become 00
    uint32_t z = ~(x | (x >> 1)) & 0x55555555u;
    z = (z | (z >> 1)) & 0x33333333u;            // gather the even bits into the low 16
    z = (z | (z >> 2)) & 0x0F0F0F0Fu;
    z = (z | (z >> 4)) & 0x00FF00FFu;
    return (z | (z >> 8)) & 0x0000FFFFu;
  };
  return one(h0) | (one(h1) << 16);
}

template <int NWD>
__device__ __forceinline__ RowBits<NWD> row_bits(const TileGeom& g, const DecodeArgs& a, int seq, int bb, int nblk,
                                                 int len, int l) {
  RowBits<NWD> r;
  const int k = l & 7;
  r.b = bb + (l >> 3);
  if (r.b >= nblk) {
    r.b = -1;
    r.phys = 0;
#pragma unroll
    for (int i = 0; i < NWD; ++i) r.m[i] = 0u;
    return r;
  }
  r.phys = a.block_table[(size_t)seq * a.max_blocks_per_seq + r.b];
  const int t0 = r.b * kRows + 32 * k;
  const int nvalid = min(max(len - t0, 0), 32);
  uint32_t live = nvalid >= 32 ? 0xFFFFFFFFu : ((1u << nvalid) - 1u);
  if (a.mask) live &= ~a.mask[(size_t)seq * a.mask_words + (t0 >> 5)];
  const uint32_t* hdr = reinterpret_cast<const uint32_t*>(a.pool + (size_t)r.phys * g.H * g.tile_bytes + g.off_hdr);
  if constexpr (NWD == 2) {
    const uint32_t wide = g.mixed ? hdr[k] : 0u;
    r.m[0] = live & ~wide;
    r.m[1] = live & wide;
  } else {  // width codes 0, 1, 2, 3 = 2, 4, 8, 16 bits -> lists 2, 0, 1, 3
    const uint32_t h0 = hdr[2 * k], h1 = hdr[2 * k + 1];
    r.m[0] = live & fields_equal(h0, h1, 1u);
    r.m[1] = live & fields_equal(h0, h1, 2u);
    r.m[2] = live & fields_equal(h0, h1, 0u);
    r.m[3] = live & fields_equal(h0, h1, 3u);
  }
  return r;
}

template <int NWD>
__global__ __launch_bounds__(kCompactThreads) void compact_rows_k(TileGeom g, DecodeArgs a) {
  constexpr int NW = kCompactThreads / 64;
  __shared__ int s_tot[NW][NWD];
  __shared__ int s_carry[NWD];
  const int seq = blockIdx.x, tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int len = a.seq_lens[seq];
  const int nblk = (len + kRows - 1) / kRows;
  int* cnt = a.ws_bcnt + (size_t)seq * a.bcnt_blocks * NWD;
  // counts of each block (the 8 lanes of a block add theirs up)
  for (int bb = 8 * w; bb < nblk; bb += 8 * NW) {
    const RowBits<NWD> r = row_bits<NWD>(g, a, seq, bb, nblk, len, l);
#pragma unroll
    for (int i = 0; i < NWD; ++i) {
      int c = __popc(r.m[i]);
#pragma unroll
      for (int m = 1; m < 8; m <<= 1) c += __shfl_xor(c, m);
      if ((l & 7) == 0 && r.b >= 0) cnt[NWD * r.b + i] = c;
    }
  }
  __syncthreads();
  // exclusive scan of the counts, kCompactThreads blocks at a time (thread = block)
  if (tid < NWD) s_carry[tid] = 0;
  __syncthreads();
  for (int b0 = 0; b0 < nblk; b0 += kCompactThreads) {
    const int b = b0 + tid;
    int c[NWD], x[NWD];
#pragma unroll
    for (int i = 0; i < NWD; ++i) {
      c[i] = b < nblk ? cnt[NWD * b + i] : 0;
      x[i] = c[i];  // inclusive scan within the wave
    }
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) {
#pragma unroll
      for (int i = 0; i < NWD; ++i) {
        const int u = __shfl_up(x[i], m);
        if (l >= m) x[i] += u;
      }
    }
    if (l == 63) {
#pragma unroll
      for (int i = 0; i < NWD; ++i) s_tot[w][i] = x[i];
    }
    __syncthreads();
    int o[NWD];
#pragma unroll
    for (int i = 0; i < NWD; ++i) {
      o[i] = s_carry[i] + x[i] - c[i];
      for (int j = 0; j < w; ++j) o[i] += s_tot[j][i];
    }
    __syncthreads();
    if (b < nblk) {
#pragma unroll
      for (int i = 0; i < NWD; ++i) cnt[NWD * b + i] = o[i];
    }
    if (tid == kCompactThreads - 1) {
#pragma unroll
      for (int i = 0; i < NWD; ++i) s_carry[i] = o[i] + c[i];
    }
    __syncthreads();
  }
  if (tid < NWD) a.ws_cnt[NWD * seq + tid] = s_carry[tid];
  // entries of each block at its offsets: lane k of a block starts after the live rows of lanes 0 .. k-1
  uint32_t* lists = a.ws_list + (size_t)seq * NWD * a.list_cap;
  for (int bb = 8 * w; bb < nblk; bb += 8 * NW) {
    const RowBits<NWD> r = row_bits<NWD>(g, a, seq, bb, nblk, len, l);
    const uint32_t hi = ((uint32_t)r.phys << 8) | (uint32_t)(32 * (l & 7));
#pragma unroll
    for (int i = 0; i < NWD; ++i) {
      const int c = __popc(r.m[i]);
      int x = c;  // inclusive scan over the block's 8 lanes
#pragma unroll
      for (int m = 1; m < 8; m <<= 1) {
        const int u = __shfl_up(x, m);
        if ((l & 7) >= m) x += u;
      }
      if (r.b < 0) continue;
      int o = cnt[NWD * r.b + i] + x - c;
      uint32_t* li = lists + (size_t)i * a.list_cap;
      for (uint32_t m = r.m[i]; m; m &= m - 1u) li[o++] = hi | (uint32_t)(__ffs(m) - 1);
    }
  }
}

// ------------------------------------------------------------------------------------- decode
// Raw codes and parameters of one chunk for one lane (channels 32 la .. 32 la + 31 of K and of V). 4-bit
// chunks: tokens 16c + lj (c = 0..3), 16 bytes each of K and V. 8-bit chunks: tokens 16c + lj (c = 0, 1),
// 32 bytes each (k[2c], k[2c + 1]). 2-bit chunks: tokens 16c + lj (c = 0..3), 8 bytes each (k[c].x, .y).
// FP16 chunks: token lj, 64 bytes each (k[0..3]).
// X: a K head dim of 192 (MLA pools), whose channels 128 .. 191 (K group 2) come as `kx`: 4-bit chunks 8 bytes
// per token (words 2c, 2c + 1 of kx), 8-bit chunks 16 bytes (kx[c]), 2-bit chunks 4 bytes (word c of kx[0]),
// FP16 chunks 32 bytes (kx[0], kx[1]): channels 128 + 16 la .. 128 + 16 la + 15.
template <bool X>
struct RawT {
  u32x4 k[4];
  u32x4 v[4];
  uint32_t prm[X ? 5 : 4];  // the parameter record of token 16 la + lj (K groups {scale, zero}, then V groups)
  u32x4 kx[X ? 2 : 1];      // (vectors: whole-register values the compiler keeps out of scratch)
  uint32_t valid;           // bit c: token 16c + lj of the chunk exists
};

// Chunk kinds, in the order of the row lists: 4-bit chunks of 64 rows, 8-bit chunks of 32 rows, and in
// pools of four widths 2-bit chunks of 64 rows and FP16 chunks of 16 rows.
constexpr int kK4 = 0, kK8 = 1, kK2 = 2, kK16 = 3;
template <int K>
using Kind = std::integral_constant<int, K>;

// 16 two-bit codes (8 in each 16-bit half) -> the same codes as nibbles, in order (8 per word).
__device__ __forceinline__ uint32_t spread2(uint32_t w, uint32_t sel) {
  uint32_t x = __builtin_amdgcn_perm(0u, w, sel);  // the half's two bytes at bytes 0 and 2
  x = ((x << 4) | x) & 0x0F0F0F0Fu;
  return ((x << 2) | x) & 0x33333333u;
}

template <int G, bool GATHER, bool MIX2, int DK>
__global__ __launch_bounds__(256, 2) void decode_rows_k(TileGeom g, DecodeArgs a) {
  static_assert(G == 1 || G == 2 || G == 4, "GQA ratio 1, 2 or 4");
  static_assert(GATHER || !MIX2, "pools of four widths are read through the row lists");
  static_assert(DK == 128 || DK == 192, "K head dim 128, or 192 (MLA: 128 + 64 channels, V 128)");
  constexpr int D = kD;                  // V's head dim, and the first 128 channels of K
  constexpr bool X = DK == 192;          // K channels 128 .. 191 (K group 2)
  constexpr int NGK = DK / 64;           // K groups per row
  constexpr int NP = NGK + 2;            // parameter words per row
  constexpr int NWD = MIX2 ? 4 : 2;  // row lists per sequence
  using Raw = RawT<X>;
  // Streaming 4-bit chunks at K 128 are loaded as whole row records in address order and staged in LDS,
  // K codes included (kSlab below); the other kinds load each lane's own token row.
  constexpr bool kSlab = !GATHER && !X;
  __shared__ float s_q[G][DK];
  __shared__ float s_qsum[G][NGK];
  __shared__ __attribute__((aligned(16))) uint8_t s_v[4][64 * (kSlab ? kRP : kVP)];  // staged rows, per wave
  __shared__ __attribute__((aligned(16))) _Float16 s_p[4][64 * kPP];  // p * v_scale, position-major, per wave
  __shared__ uint32_t s_par[4][64 * NP];                              // the chunk's parameter records, per wave
  __shared__ float s_wm[4][G], s_wl[4][G];
  __shared__ float s_wacc[4][G][D];
  __shared__ int s_tbl[GATHER ? 1 : kMaxSplitBlocks];

  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, la = l >> 4, lj = l & 15;
  int pair, split, ns;  // ns: the split count of this workgroup's (sequence, KV head) pair
  rows_work(a.plan, a.n_seqs * g.H, blockIdx.x, pair, split, ns);
  const int seq = pair / g.H, h = pair - seq * g.H;
  const int len = a.seq_lens[seq];
  const uint32_t R = (uint32_t)g.rec;  // bytes of a row record
  const uint8_t* pool_h = a.pool + (size_t)h * g.tile_bytes;
  const size_t tstride = (size_t)g.H * g.tile_bytes;  // bytes between consecutive blocks of one KV head

  // ------------------------------------------------------------ this workgroup's chunks
  // Streaming: chunk i of wave w = rows 64w .. 64w+63 of logical block b0 + i. Gather: chunks c0 + w + 4i
  // of the sequence's chunk list (4-bit chunks of 64 rows first, then 8-bit chunks of 32 rows).
  // The query and (streaming) the block-table slice are loaded into registers first: neither depends on the
  // sequence length, so their loads overlap its load. Streaming splits cut the longest sequence's blocks;
  // a shorter sequence clips them.
  constexpr int kQPer = (G * DK + 255) / 256;
  uint16_t qraw[kQPer];
#pragma unroll
  for (int k = 0; k < kQPer; ++k) {
    const int i = min(tid + 256 * k, G * DK - 1);  // unconditional loads: no branch waits for them
    qraw[k] = a.q[((size_t)seq * a.num_q_heads + h * G + i / DK) * DK + i % DK];
  }
  // rows per chunk of each kind, and the kind of chunk ci (wave-uniform)
  auto chunk_rows = [](int kind) __attribute__((always_inline)) {
    return kind == kK8 ? 32 : kind == kK16 ? 16 : 64;
  };
  int b0 = 0, ntbl = 0, nchunk = 0, c0 = 0;
  int nrow[NWD] = {};     // gather: live rows per list
  int cend[NWD] = {};     // gather: end of each kind's chunks in the chunk order
  int tb0 = 0, tb1 = 0;
  if (!GATHER) {
    int b1;
    piece_range(split, ns, a.plan.max_blocks, b0, b1);
    ntbl = b1 - b0;  // 1 .. kMaxSplitBlocks
    const int32_t* bt = a.block_table + (size_t)seq * a.max_blocks_per_seq + b0;
    tb0 = bt[min(tid, ntbl - 1)];
    if (ntbl > 256) tb1 = bt[min(tid + 256, ntbl - 1)];
  }
  auto kind_of = [&](int ci) __attribute__((always_inline)) {
    if (!MIX2) return ci >= cend[0] ? kK8 : kK4;
    return ci < cend[0] ? kK4 : ci < cend[1] ? kK8 : ci < cend[2] ? kK2 : kK16;
  };
  bool wg_empty;
  const uint32_t* lists = nullptr;
  if (GATHER) {
    int nc = 0;
#pragma unroll
    for (int k = 0; k < NWD; ++k) {
      nrow[k] = a.ws_cnt[NWD * seq + k];
      nc += (nrow[k] + chunk_rows(k) - 1) / chunk_rows(k);
      cend[k] = nc;
    }
    c0 = (int)(((long)split * nc) / ns);
    const int c1 = (int)(((long)(split + 1) * nc) / ns);
    nchunk = c1 - c0 > w ? (c1 - c0 - w + 3) / 4 : 0;
    wg_empty = c1 <= c0;
    lists = a.ws_list + (size_t)seq * NWD * a.list_cap;
  } else {
    nchunk = min(b0 + ntbl, (len + kRows - 1) / kRows) - b0;
    wg_empty = nchunk <= 0;
  }

  if (wg_empty) {
    if (ns == 1) {  // nothing live in the sequence: the output row still has to be written
      __shared__ int s_cnt0[4];
      const int n_sent = count_sentinels<256>(a, seq, len, tid, s_cnt0);
      for (int jj = 0; jj < G; ++jj)
        finalize_head<D, 256>(g, a, seq, h * G + jj, len, n_sent, kNegInf, 0.0f, 0.0f, tid, &s_wacc[0][0][0]);
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
  // The chunks' loads are issued after the table slice is in LDS; the query set-up below waits only for
  // the query.
  if (!GATHER) {
    if (tid < nchunk) s_tbl[tid] = tb0;
    if (tid + 256 < nchunk) s_tbl[tid + 256] = tb1;
    __syncthreads();
  }

  // Rows of the wave's chunk i for this lane: tokens 16c + lj. In gather mode the list entries are fetched
  // one chunk ahead of the codes (fetch, then load), so the codes' addresses never wait on the list.
  struct Ent {
    uint32_t e[4];   // gather: list entries (physical block << 8 | row)
    uint32_t valid;  // bit c: token 16c + lj exists
    int lim;         // streaming 4-bit chunks at K 128: rows of the wave's chunk below the sequence's end
  };
  auto fetch = [&](Ent& en, int i) __attribute__((always_inline)) {
    if (GATHER) {
      const int ci = c0 + w + 4 * i;
      const int kind = kind_of(ci);
      const uint32_t* lst = lists + (size_t)kind * a.list_cap;
      const int rpc = chunk_rows(kind);
      // register selects rather than indexing the arrays with a run-time kind
      int start = 0, n = nrow[0];
#pragma unroll
      for (int k = 1; k < NWD; ++k) {
        start = kind == k ? cend[k - 1] : start;
        n = kind == k ? nrow[k] : n;
      }
      const int e0 = (ci - start) * rpc;
      uint32_t valid = 0;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        int idx = e0 + 16 * c + lj;
        const bool ok = idx < n && 16 * c < rpc;
        valid |= ok ? (1u << c) : 0u;
        en.e[c] = lst[ok ? idx : e0];  // the chunk's first row always exists
      }
      en.valid = valid;
    } else {
      uint32_t valid = 0;
#pragma unroll
      for (int c = 0; c < 4; ++c) valid |= ((b0 + i) * kRows + 64 * w + 16 * c + lj < len) ? (1u << c) : 0u;
      en.valid = valid;
      if constexpr (kSlab) en.lim = len - ((b0 + i) * kRows + 64 * w);
    }
  };
  // Issue the code and parameter loads of chunk i (rows from en) into r.
  // live: false for a streaming chunk past the split's end, whose loads the loop still issues so that it
  // has no exit between chunks; those loads go through an empty buffer range and read nothing.
  auto load = [&](Raw& r, const Ent& en, int i, bool live = true) __attribute__((always_inline)) {
    const uint8_t* tile[4];
    uint32_t row[4];
    int kind = kK4;
    if (GATHER) {
      kind = kind_of(c0 + w + 4 * i);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        tile[c] = pool_h + (size_t)(en.e[c] >> 8) * tstride;
        row[c] = en.e[c] & 255u;
      }
    } else {
      // the block's tile base is wave-uniform: scalar base, 32-bit per-lane offsets; a row past the
      // sequence's end reads row 0 instead (live, and fetched for wave 0 anyway, so an L2 hit)
      const int phys = __builtin_amdgcn_readfirstlane(s_tbl[i]);
      const uint8_t* t0 = pool_h + (size_t)phys * tstride;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        tile[c] = t0;
        row[c] = ((en.valid >> c) & 1u) ? (uint32_t)(64 * w + 16 * c + lj) : 0u;
      }
    }
    r.valid = en.valid;
    // Streaming 4-bit chunks at K 128 read through a buffer resource over the tile (wave-uniform: four
    // scalar registers). A chunk past the split's end gets a resource of zero bytes, so its loads return
    // zeros at once and fetch nothing, instead of re-reading the last chunk and holding the workgroup's
    // merge until they return.
    auto slab_rsrc = [&]() __attribute__((always_inline)) {
      return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(tile[0]), (short)0,
                                               live ? (int)g.tile_bytes : 0, kBufWord3);
    };
    if constexpr (kSlab) {
      const __amdgpu_buffer_rsrc_t rs = slab_rsrc();
      // The wave's 64 records (8 KB) as eight 1 KB slabs in address order: lane l takes the 16-byte piece
      // l % 8 of row 8 j + l / 8 of slab j, so every 8 consecutive lanes read one whole record. Slab 2c
      // holds rows 16c .. 16c+7 (in r.k[c]) and slab 2c + 1 rows 16c+8 .. 16c+15 (in r.v[c]); the chunk's
      // processing moves them to the lane-per-token layout through LDS. Measured on the 12 x 8K pool's
      // read pattern: 8 % faster than each lane reading its own token's K and V halves (16-lane groups
      // touching 16 records per load), 14 % with non-temporal loads (which slow that pattern down).
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int rw = 8 * j + 2 * la + (lj >> 3);  // lane l = 16 la + lj: row 8 j + l / 8, piece l % 8
        const uint32_t off = (rw < en.lim ? (uint32_t)(64 * w + rw) : 0u) * R + (lj & 7) * 16;
        const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, kBufNT);
        if (j & 1) r.v[j >> 1] = x;
        else r.k[j >> 1] = x;
      }
    } else if (kind == kK4) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const uint8_t* rp = tile[c] + row[c] * R;
        r.k[c] = *reinterpret_cast<const u32x4*>(rp + la * 16);
        r.v[c] = *reinterpret_cast<const u32x4*>(rp + DK / 2 + la * 16);  // V codes follow the 4-bit K codes
        if constexpr (X) {
          const uint2 xx = *reinterpret_cast<const uint2*>(rp + 64 + la * 8);
          r.kx[c >> 1][2 * (c & 1)] = xx.x;
          r.kx[c >> 1][2 * (c & 1) + 1] = xx.y;
        }
      }
    } else if (MIX2 && kind == kK2) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const uint8_t* rp = tile[c] + row[c] * R;
        const uint2 kk = *reinterpret_cast<const uint2*>(rp + la * 8);
        const uint2 vv = *reinterpret_cast<const uint2*>(rp + DK / 4 + la * 8);  // V codes follow the 2-bit K codes
        r.k[c] = u32x4{kk.x, kk.y, 0u, 0u};
        r.v[c] = u32x4{vv.x, vv.y, 0u, 0u};
        if constexpr (X) r.kx[0][c] = *reinterpret_cast<const uint32_t*>(rp + 32 + la * 4);
      }
    } else if (MIX2 && kind == kK16) {
      const uint8_t* rp = tile[0] + row[0] * R;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        r.k[c] = *reinterpret_cast<const u32x4*>(rp + la * 64 + 16 * c);
        r.v[c] = *reinterpret_cast<const u32x4*>(rp + 2 * DK + la * 64 + 16 * c);  // V values follow the K values
      }
      if constexpr (X) {
#pragma unroll
        for (int c = 0; c < 2; ++c) r.kx[c] = *reinterpret_cast<const u32x4*>(rp + 256 + la * 32 + 16 * c);
      }
    } else {
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const uint8_t* rp = tile[c] + row[c] * R;
        r.k[2 * c] = *reinterpret_cast<const u32x4*>(rp + la * 32);
        r.k[2 * c + 1] = *reinterpret_cast<const u32x4*>(rp + la * 32 + 16);
        r.v[2 * c] = *reinterpret_cast<const u32x4*>(rp + DK + la * 32);  // V codes follow the 8-bit K codes
        r.v[2 * c + 1] = *reinterpret_cast<const u32x4*>(rp + DK + la * 32 + 16);
        if constexpr (X) r.kx[c] = *reinterpret_cast<const u32x4*>(rp + 128 + la * 16);
      }
    }
    // One parameter record per lane: the record of token 16 la + lj (lane (c, lj) holds the record every
    // lane with token 16c + lj needs; they are exchanged through LDS when the chunk is processed). Loading
    // each token's record in all four lanes of its 16-lane group instead (four loads per lane, each reading
    // one 128-byte line in four) made a read of the 12 x 8K pool with this work split 33 % slower.
    {
      const uint8_t* tp = tile[0];
      uint32_t rp = row[0];
#pragma unroll
      for (int c = 1; c < 4; ++c) {
        tp = la == c ? tile[c] : tp;
        rp = la == c ? row[c] : rp;
      }
      if constexpr (X) {
        const uint32_t* pr = reinterpret_cast<const uint32_t*>(tp + (g.off_prow + rp * (4 * NP)));
#pragma unroll
        for (int e = 0; e < NP; ++e) r.prm[e] = pr[e];
      } else if constexpr (kSlab) {
        const u32x4 pr = __builtin_amdgcn_raw_buffer_load_b128(slab_rsrc(), g.off_prow + rp * 16, 0, 0);
#pragma unroll
        for (int e = 0; e < 4; ++e) r.prm[e] = pr[e];
      } else {
        const u32x4 pr = *reinterpret_cast<const u32x4*>(tp + (g.off_prow + rp * 16));
#pragma unroll
        for (int e = 0; e < 4; ++e) r.prm[e] = pr[e];
      }
    }
  };

  // The first chunks' loads are issued before the query set-up, so their latency overlaps it: one chunk
  // in gather mode, two in streaming mode (which keeps two chunks in flight).
  Raw ra, rb, rc;
  Ent en;
  if (nchunk > 0) {
    fetch(en, 0);
    load(ra, en, 0);
    fetch(en, min(1, nchunk - 1));
    if (!GATHER) {
      load(rb, en, min(1, nchunk - 1), nchunk > 1);
      fetch(en, min(2, nchunk - 1));
    }
  }

  // ------------------------------------------------------------ query: scale, rotation, group sums
  // (LDS-only barriers: the chunks' loads stay in flight)
#pragma unroll
  for (int k = 0; k < kQPer; ++k) {
    const int i = tid + 256 * k;
    if (i < G * DK) s_q[i / DK][i % DK] = h2f(qraw[k]) * a.q_scale;
  }
  for (int i = tid; i < 4 * 64 * kPP; i += 256) (&s_p[0][0])[i] = (_Float16)0.0f;
  lds_barrier();
  if (!X && g.rotate) {  // (rotated pools have power-of-two head dims)
    for (int hs = 1; hs < D; hs *= 2) {
      for (int i = tid; i < G * D / 2; i += 256) {
        const int j = i / (D / 2), pi = i % (D / 2);
        const int lo = (pi / hs) * 2 * hs + (pi % hs);
        const float x = s_q[j][lo], y = s_q[j][lo + hs];
        s_q[j][lo] = x + y;
        s_q[j][lo + hs] = x - y;
      }
      lds_barrier();
    }
    for (int i = tid; i < G * D; i += 256) s_q[i / D][i % D] *= a.unrot_c;
    lds_barrier();
  }
  for (int i = tid; i < G * NGK; i += 256) {
    float sum = 0.0f;
    for (int c = 0; c < 64; ++c) sum += s_q[i / NGK][(i % NGK) * 64 + c];
    s_qsum[i / NGK][i % NGK] = sum;
  }
  lds_barrier();

  // QK A operand for k-step s: row lj = 4 hq + 2 gam + part; lane group la supplies channels
  // 32 la + ch(s, e), e = 0..7 = 2 p + k, in the unpacking order of the chunk's width:
  // * 4- and 8-bit: ch = 8 s + p + 4 k (nibbles 0,4,1,5,2,6,3,7); 4-bit chunks see the odd-p nibbles
  //   multiplied by 16, so their query entries are divided by 16;
  // * 2-bit: ch = 16 (s >> 1) + 4 (s & 1) + p + 8 k, the code field p of each 16-bit half, seen multiplied
  //   by 4^p, so the query entry is divided by 4^p;
  // * FP16: ch = 8 s + e, the values as stored.
  u32x4 qa[4];
  auto build_qa = [&](int kind) __attribute__((always_inline)) {
    const int hq = lj >> 2, gam = (lj >> 1) & 1, part = lj & 1;
    const bool in_group = hq < G && (la >> 1) == gam;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        _Float16 x[2];
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          int ch = 8 * s + p + 4 * k;
          float f = (kind == kK4 && (p & 1)) ? 0.0625f : 1.0f;
          if (MIX2 && kind == kK2) {
            ch = 16 * (s >> 1) + 4 * (s & 1) + p + 8 * k;
            f = p == 0 ? 1.0f : p == 1 ? 0.25f : p == 2 ? 0.0625f : 0.015625f;
          } else if (MIX2 && kind == kK16) {
            ch = 8 * s + 2 * p + k;
          }
          const float v = in_group ? s_q[hq][32 * la + ch] * f : 0.0f;
          const _Float16 hi = (_Float16)v;
          x[k] = part ? (_Float16)(v - (float)hi) : hi;
        }
        qa[s][p] = pack_h2(x[0], x[1]);
      }
    }
  };
  // K channels 128 .. 191 (X): A operand for extra k-step s of row lj = 4 hq + part (only rows whose
  // (lj >> 1) & 1 is 0), lane group la supplying channels 128 + 16 la + ch(s, e) in the unpacking order of
  // the chunk's width: 4- and 8-bit ch = 8 s + p + 4 k, 2-bit ch = 4 s + p + 8 k, FP16 ch = 8 s + 2 p + k.
  // (in pools of four widths the operand is kept in LDS, one slot per wave and lane: their K 192 instances are
  // short of registers; the others keep it in registers)
  constexpr bool kQaxLds = X && MIX2;
  u32x4 qax[X && !kQaxLds ? 2 : 1];
  __shared__ __attribute__((aligned(16))) u32x4 s_qax[kQaxLds ? 4 : 1][2][64];
  auto build_qax = [&](int kind) __attribute__((always_inline)) {
    if constexpr (X) {
      const int hq = lj >> 2, part = lj & 1;
      const bool in_group = hq < G && ((lj >> 1) & 1) == 0;
#pragma unroll
      for (int s = 0; s < 2; ++s) {
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          _Float16 x[2];
#pragma unroll
          for (int k = 0; k < 2; ++k) {
            int ch = 8 * s + p + 4 * k;
            float f = (kind == kK4 && (p & 1)) ? 0.0625f : 1.0f;
            if (MIX2 && kind == kK2) {
              ch = 4 * s + p + 8 * k;
              f = p == 0 ? 1.0f : p == 1 ? 0.25f : p == 2 ? 0.0625f : 0.015625f;
            } else if (MIX2 && kind == kK16) {
              ch = 8 * s + 2 * p + k;
            }
            const float v = in_group ? s_q[hq][128 + 16 * la + ch] * f : 0.0f;
            const _Float16 hi = (_Float16)v;
            x[k] = part ? (_Float16)(v - (float)hi) : hi;
          }
          if constexpr (kQaxLds) s_qax[w][s][l][p] = pack_h2(x[0], x[1]);
          else qax[s][p] = pack_h2(x[0], x[1]);
        }
      }
    }
  };
  build_qa(kK4);
  build_qax(kK4);
  int cur_kind = kK4;
  const bool head_ok = la < G;
  const float qs0 = head_ok ? s_qsum[la][0] : 0.0f, qs1 = head_ok ? s_qsum[la][1] : 0.0f;
  const float qs2 = X && head_ok ? s_qsum[la][NGK - 1] : 0.0f;

  float m_run = kNegInf, l_run = 0.0f, zacc0 = 0.0f, zacc1 = 0.0f;
  floatx4 o[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) o[t] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};

  uint8_t* sv = s_v[w];
  _Float16* sp = s_p[w];
  uint32_t* spar = s_par[w];
  // Set when a chunk of this wave had logit terms above kPreciseAbove: the wave's rows then go through the fp64
  // pass (precise_wave_pass) after the main loop (wave-uniform).
  bool wave_big = false;

  auto process = [&](const Raw& r, auto kc) __attribute__((always_inline)) {
    constexpr int KIND = decltype(kc)::value;
    constexpr bool W8 = KIND == kK8, F16 = KIND == kK16;
    constexpr int NC = W8 ? 2 : F16 ? 1 : 4;  // 16-token slices
    // ---------------------------------------------------------- stage V rows (lane = token) in LDS
    // (2-bit codes widened to nibbles, so the value pass of 2-bit chunks is the 4-bit one)
    if constexpr (KIND == kK4 && kSlab) {
      // whole records, row pitch kRP (K codes at 0, V codes at 64)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int rw = 16 * c + 2 * la + (lj >> 3);
        *reinterpret_cast<u32x4*>(sv + rw * kRP + (lj & 7) * 16) = r.k[c];
        *reinterpret_cast<u32x4*>(sv + (rw + 8) * kRP + (lj & 7) * 16) = r.v[c];
      }
    } else if constexpr (KIND == kK4) {
#pragma unroll
      for (int c = 0; c < 4; ++c) *reinterpret_cast<u32x4*>(sv + (16 * c + lj) * kVP + la * 16) = r.v[c];
    } else if constexpr (KIND == kK2) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const u32x4 nib = {spread2(r.v[c][0], 0x0C010C00u), spread2(r.v[c][0], 0x0C030C02u),
                           spread2(r.v[c][1], 0x0C010C00u), spread2(r.v[c][1], 0x0C030C02u)};
        *reinterpret_cast<u32x4*>(sv + (16 * c + lj) * kVP + la * 16) = nib;
      }
    } else if constexpr (W8) {
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        *reinterpret_cast<u32x4*>(sv + (16 * c + lj) * kVP8 + la * 32) = r.v[2 * c];
        *reinterpret_cast<u32x4*>(sv + (16 * c + lj) * kVP8 + la * 32 + 16) = r.v[2 * c + 1];
      }
    } else {
#pragma unroll
      for (int c = 0; c < 4; ++c) *reinterpret_cast<u32x4*>(sv + lj * kVP16 + la * 64 + 16 * c) = r.v[c];
    }
    // ---------------------------------------------------------- parameter records of tokens 16c + lj
    uint32_t kp[NC][NGK], vp[NC][2];
    if constexpr (!F16) {
      if constexpr (X) {
#pragma unroll
        for (int e = 0; e < NP; ++e) spar[NP * (16 * la + lj) + e] = r.prm[e];
      } else {
        *reinterpret_cast<u32x4*>(spar + 4 * (16 * la + lj)) = u32x4{r.prm[0], r.prm[1], r.prm[2], r.prm[3]};
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        uint32_t x[NP];
        if constexpr (X) {
#pragma unroll
          for (int e = 0; e < NP; ++e) x[e] = spar[NP * (16 * c + lj) + e];
        } else {
          const u32x4 y = *reinterpret_cast<const u32x4*>(spar + 4 * (16 * c + lj));
#pragma unroll
          for (int e = 0; e < 4; ++e) x[e] = y[e];
        }
#pragma unroll
        for (int e = 0; e < NGK; ++e) kp[c][e] = x[e];
        vp[c][0] = x[NGK];
        vp[c][1] = x[NGK + 1];
      }
    }
    // staged K codes back in the lane-per-token layout (row 16c + lj, bytes 16 la; the pitch of 9 16-byte
    // units puts 8 consecutive lanes in distinct banks)
    u32x4 ks[kSlab && KIND == kK4 ? 4 : 1];
    if constexpr (kSlab && KIND == kK4) {
#pragma unroll
      for (int c = 0; c < 4; ++c) ks[c] = *reinterpret_cast<const u32x4*>(sv + (16 * c + lj) * kRP + la * 16);
    }
    // ---------------------------------------------------------- logits: QK on the matrix cores
    floatx4 acc[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) acc[c] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        u32x4 b;
        if constexpr (KIND == kK4) {
          const uint32_t wd = kSlab ? ks[c][s] : r.k[c][s], w8 = wd >> 8;
          b = u32x4{wd & kLo4, wd & kHi4, w8 & kLo4, w8 & kHi4};
        } else if constexpr (KIND == kK2) {
          // field p of each 16-bit half as an fp16 subnormal (code * 4^p) * 2^-24
          const uint32_t wd = r.k[c][s >> 1] >> (8 * (s & 1));
          b = u32x4{wd & 0x00030003u, wd & 0x000C000Cu, wd & 0x00300030u, wd & 0x00C000C0u};
        } else if constexpr (W8) {
          const uint32_t lo = r.k[2 * c + (s >> 1)][2 * (s & 1)], hi = r.k[2 * c + (s >> 1)][2 * (s & 1) + 1];
          b = u32x4{__builtin_amdgcn_perm(hi, lo, pair_sel(0)), __builtin_amdgcn_perm(hi, lo, pair_sel(1)),
                    __builtin_amdgcn_perm(hi, lo, pair_sel(2)), __builtin_amdgcn_perm(hi, lo, pair_sel(3))};
        } else {
          b = r.k[s];  // fp16 values as stored
        }
        acc[c] = mfma16(qa[s], b, acc[c]);
      }
    // K channels 128 .. 191: two more k-steps into their own tiles (rows 4 hq + part)
    floatx4 accx[X ? NC : 1];
    if constexpr (X) {
      u32x4 qx[2];
      if constexpr (kQaxLds) {
        qx[0] = s_qax[w][0][l];
        qx[1] = s_qax[w][1][l];
      }
#pragma unroll
      for (int c = 0; c < NC; ++c) accx[c] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          u32x4 b;
          if constexpr (KIND == kK4) {
            const uint32_t wd = r.kx[c >> 1][2 * (c & 1) + s], w8 = wd >> 8;
            b = u32x4{wd & kLo4, wd & kHi4, w8 & kLo4, w8 & kHi4};
          } else if constexpr (KIND == kK2) {
            const uint32_t wd = r.kx[0][c] >> (8 * s);
            b = u32x4{wd & 0x00030003u, wd & 0x000C000Cu, wd & 0x00300030u, wd & 0x00C000C0u};
          } else if constexpr (W8) {
            const uint32_t lo = r.kx[c][2 * s], hi = r.kx[c][2 * s + 1];
            b = u32x4{__builtin_amdgcn_perm(hi, lo, pair_sel(0)), __builtin_amdgcn_perm(hi, lo, pair_sel(1)),
                      __builtin_amdgcn_perm(hi, lo, pair_sel(2)), __builtin_amdgcn_perm(hi, lo, pair_sel(3))};
          } else {
            b = r.kx[s];
          }
          accx[c] = mfma16(kQaxLds ? qx[s] : qax[s], b, accx[c]);
        }
    }
    float sc[NC];
    bool big = false;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const bool live = head_ok && ((r.valid >> c) & 1u);
      if constexpr (F16) {
        float dk = (acc[c][0] + acc[c][1]) + (acc[c][2] + acc[c][3]);
        if constexpr (X) dk += accx[c][0] + accx[c][1];
        sc[c] = live ? dk : kNegInf;
        big |= live && fabsf(dk) > kPreciseAbove;
      } else {
        float dot = h2f(kp[c][0] & 0xffffu) * (acc[c][0] + acc[c][1]) +
                    h2f(kp[c][1] & 0xffffu) * (acc[c][2] + acc[c][3]);
        float zq = h2f(kp[c][0] >> 16) * qs0 + h2f(kp[c][1] >> 16) * qs1;
        if constexpr (X) {
          dot += h2f(kp[c][NGK - 1] & 0xffffu) * (accx[c][0] + accx[c][1]);
          zq += h2f(kp[c][NGK - 1] >> 16) * qs2;
        }
        const float dk = dot * kTwo24;
        sc[c] = live ? dk + zq : kNegInf;
        big |= live && fabsf(dk) + fabsf(zq) > kPreciseAbove;
      }
    }
    wave_big |= __builtin_amdgcn_ballot_w64(big) != 0;
    // ---------------------------------------------------------- online softmax (head la, 16-lane rows)
    float mx = sc[0];
#pragma unroll
    for (int c = 1; c < NC; ++c) mx = fmaxf(mx, sc[c]);
    mx = row_max16(mx);
    const float mnew = fmaxf(m_run, mx);
    const float alpha = mnew == m_run ? 1.0f : __builtin_amdgcn_exp2f(m_run - mnew);
    float p[NC], ps = 0.0f;
    const float mref = mnew == kNegInf ? 0.0f : mnew;  // no live logit yet: every p is exp2(-inf) = 0
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      p[c] = __builtin_amdgcn_exp2f(sc[c] - mref);  // -inf - finite -> 0
      ps += p[c];
    }
    l_run = l_run * alpha + ps;
    m_run = mnew;
    if (__builtin_amdgcn_ballot_w64(alpha != 1.0f)) {  // wave-uniform: skip when no running max moved
      zacc0 *= alpha;
      zacc1 *= alpha;
#pragma unroll
      for (int t = 0; t < 8; ++t) o[t] *= alpha;
    }
    // ---------------------------------------------------------- p * v_scale (hi, lo) to LDS
    // Position of token t: (t & ~7) | sinv(t & 7), sinv(u) = 2 (u & 3) + (u >> 2), the inverse of the
    // token order 0,4,1,5,2,6,3,7 of the V operand; odd tokens of 4-bit (and widened 2-bit) chunks are
    // divided by 16. The chunk's operands carry the wave-uniform scale of chunk_pv_scale (undone when the
    // chunk is added).
    // Odd tokens (u odd) enter the MFMA as -p * v_scale times the complemented code (L - code, L = 15 or
    // 255) and add p * (v_zero + L * v_scale) to the zero-point term, which is the same value: the
    // products then carry both signs, so the matrix core's rounding of long all-positive sums does not
    // bias the code term (which cancels against the zero-point term down to the much smaller output).
    // FP16 chunks: token t at position t, the weight p itself (scale 2^14) in the rows of both V groups.
    float pv_inv;
    if constexpr (F16) {
      pv_inv = 1.0f / (16384.0f * kTwo24);  // the values are not codes * 2^-24: undo that factor too
      const float pv = p[0] * 16384.0f;
      const _Float16 h0 = (_Float16)pv;
      const _Float16 e0 = (_Float16)(pv - (float)h0);
      if (head_ok) {
        const uint32_t x = pack_h2(h0, e0);
        *reinterpret_cast<uint2*>(sp + lj * kPP + la * 4) = uint2{x, x};
      }
    } else {
      // The chunk's largest V scale. At K 128 from each lane's own parameter record (one token per lane,
      // every token of the chunk once; the exchanged copies convert each token's scales in four lanes). At
      // K 192 from the exchanged copies: holding the own record that long makes those instances spill.
      float vmax = 0.0f;
      if constexpr (!X) {
        vmax = fmaxf(h2f(r.prm[NGK] & 0xffffu), h2f(r.prm[NGK + 1] & 0xffffu));
      } else {
#pragma unroll
        for (int c = 0; c < NC; ++c)
          vmax = fmaxf(vmax, fmaxf(h2f(vp[c][0] & 0xffffu), h2f(vp[c][1] & 0xffffu)));
      }
      const float pv_scale = chunk_pv_scale(vmax, pv_inv);
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const int t = 16 * c + lj, u = lj & 7;
        const int pos = (t & ~7) | (((u & 3) << 1) | (u >> 2));
        const float pp = p[c];
        const bool on = X ? pp != 0.0f : true;
        const bool odd = u & 1;
        const float f = odd ? (W8 ? -pv_scale : -0.0625f * pv_scale) : pv_scale;
        const float Lc = odd ? (W8 ? 255.0f : 15.0f) : 0.0f;
        // Every record read is one the quantiser wrote (a row past the end reads a live row's), so its scales
        // and zeros are finite and a token of weight 0 adds exact zeros without a select. (The K 192 instances
        // keep the selects: without them their register allocation spills more.)
        const float vs0 = on ? h2f(vp[c][0] & 0xffffu) : 0.0f, vz0 = on ? h2f(vp[c][0] >> 16) : 0.0f;
        const float vs1 = on ? h2f(vp[c][1] & 0xffffu) : 0.0f, vz1 = on ? h2f(vp[c][1] >> 16) : 0.0f;
        zacc0 += pp * (vz0 + Lc * vs0);
        zacc1 += pp * (vz1 + Lc * vs1);
        const float pv0 = (pp * f) * vs0, pv1 = (pp * f) * vs1;
        const _Float16 h0 = (_Float16)pv0, h1 = (_Float16)pv1;
        const _Float16 e0 = (_Float16)(pv0 - (float)h0), e1 = (_Float16)(pv1 - (float)h1);
        if (head_ok) {
          uint2 wv;
          wv.x = pack_h2(h0, e0);
          wv.y = pack_h2(h1, e1);
          *reinterpret_cast<uint2*>(sp + pos * kPP + la * 4) = wv;
        }
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // ---------------------------------------------------------- PV on the matrix cores
    // The chunk accumulates into fresh MFMA tiles that are then added to the running output in fp32: the
    // code sum p * v_scale * code is much larger than the output it cancels down to (the group zeros'
    // term is added separately), and a long chain of MFMA accumulations would lose that difference.
    floatx4 ob[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) ob[t] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
    constexpr int NKB = W8 || F16 ? 1 : 2;  // 32-token k-blocks
    u32x4 pa[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      const int base = 32 * kb + 8 * la + (lj >> 2);
      const v2i x0 = lds_tr16(sp + base * kPP + (lj & 3) * 4);
      const v2i x1 = lds_tr16(sp + (base + 4) * kPP + (lj & 3) * 4);
      pa[kb] = u32x4{(uint32_t)x0.x, (uint32_t)x0.y, (uint32_t)x1.x, (uint32_t)x1.y};
    }
    if constexpr (!W8 && !F16) {
      const int tok = lj < 8 ? 8 * la + lj : 32 + 8 * la + (lj - 8);
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const v2i x = lds_tr4(kSlab ? sv + tok * kRP + 64 + 8 * t : sv + tok * kVP + 8 * t);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          // high nibbles (odd tokens) complemented: 15 - code, i.e. the inverted bits under the mask
          const uint32_t wd = (uint32_t)(kb ? x.y : x.x), w8 = wd >> 8;
          const u32x4 b = {wd & kLo4, ~wd & kHi4, w8 & kLo4, ~w8 & kHi4};
          ob[t] = mfma16(pa[kb], b, ob[t]);
        }
      }
    } else if constexpr (W8) {
      const int tok = 8 * la + (lj >> 1);
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const v2i x = lds_tr8(sv + tok * kVP8 + 16 * t + 8 * (lj & 1));
        const uint32_t lo = (uint32_t)x.x, hi = (uint32_t)x.y;
        // tokens 1, 5 and 3, 7 (odd) complemented: 255 - code
        const u32x4 b = {__builtin_amdgcn_perm(hi, lo, pair_sel(0)),
                         __builtin_amdgcn_perm(hi, lo, pair_sel(1)) ^ 0x00FF00FFu,
                         __builtin_amdgcn_perm(hi, lo, pair_sel(2)),
                         __builtin_amdgcn_perm(hi, lo, pair_sel(3)) ^ 0x00FF00FFu};
        ob[t] = mfma16(pa[0], b, ob[t]);
      }
    } else {
      // B: V values of tokens 8 la + e at channel 16 t + lj (16-bit transpose read of the token-major rows).
      // The chunk has 16 tokens: lanes with la >= 2 (tokens 16..31) read rows of la - 2 and contribute zero.
      const bool hi_half = la >= 2;
      if (hi_half) pa[0] = u32x4{0u, 0u, 0u, 0u};
      const int row = 8 * (la & 1) + (lj >> 2);
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const v2i x0 = lds_tr16(sv + row * kVP16 + 2 * (16 * t + 4 * (lj & 3)));
        const v2i x1 = lds_tr16(sv + (row + 4) * kVP16 + 2 * (16 * t + 4 * (lj & 3)));
        u32x4 b = {(uint32_t)x0.x, (uint32_t)x0.y, (uint32_t)x1.x, (uint32_t)x1.y};
        if (hi_half) b = u32x4{0u, 0u, 0u, 0u};
        ob[t] = mfma16(pa[0], b, ob[t]);
      }
    }
#pragma unroll
    for (int t = 0; t < 8; ++t) o[t] += ob[t] * pv_inv;
    __builtin_amdgcn_wave_barrier();
  };
  auto run = [&](const Raw& r, int i) __attribute__((always_inline)) {
    if (GATHER) {
      const int kind = kind_of(c0 + w + 4 * i);
      if (kind != cur_kind) {
        build_qa(kind);
        build_qax(kind);
        cur_kind = kind;
      }
      if (kind == kK8) {
        process(r, Kind<kK8>{});
        return;
      }
      if constexpr (MIX2) {
        if (kind == kK2) {
          process(r, Kind<kK2>{});
          return;
        }
        if (kind == kK16) {
          process(r, Kind<kK16>{});
          return;
        }
      }
    }
    process(r, Kind<kK4>{});
  };

  // sched_barrier keeps a chunk's loads (and the list entries of the one after) ahead of the arithmetic
  // that follows, so they are in flight while it runs. Past the end the loads of streaming 4-bit chunks at
  // K 128 read nothing (a zero-byte buffer resource); the other kinds reload the last chunk (an L2 hit), and
  // the reload is not used.
  if constexpr (!GATHER) {
    // Streaming: three register sets, two chunks in flight while one is processed. The loop runs over
    // whole triples with no exit in between (an exit there gives the compiler a path into the loop head
    // on which it places over-strict waits); the last one or two chunks follow it.
    auto issue = [&](Raw& r, int j) __attribute__((always_inline)) {
      fetch(en, min(j, nchunk - 1));
      load(r, en, min(j, nchunk - 1), j < nchunk);
      __builtin_amdgcn_sched_barrier(0);
    };
    int i = 0;
    for (; i + 2 < nchunk; i += 3) {
      issue(rc, i + 2);
      run(ra, i);
      issue(ra, i + 3);
      run(rb, i + 1);
      issue(rb, i + 4);
      run(rc, i + 2);
    }
    if (i < nchunk) run(ra, i);
    if (i + 1 < nchunk) run(rb, i + 1);
  } else {
    for (int i = 0; i < nchunk; i += 2) {
      load(rb, en, min(i + 1, nchunk - 1));
      fetch(en, min(i + 2, nchunk - 1));
      __builtin_amdgcn_sched_barrier(0);
      run(ra, i);
      if (i + 1 >= nchunk) break;
      load(ra, en, min(i + 2, nchunk - 1));
      fetch(en, min(i + 3, nchunk - 1));
      __builtin_amdgcn_sched_barrier(0);
      run(rb, i + 1);
    }
  }

  // ---------------------------------------------------------------- merge the four waves
  if (wave_big) {
    // this wave's rows again with fp64 logits; the pass writes the wave's merge slots itself
    auto qv = [&](int j, int c) __attribute__((always_inline)) -> double {
      return g.rotate ? (double)s_q[j][c]
                      : (double)h2f(a.q[((size_t)seq * a.num_q_heads + h * G + j) * DK + c]) * a.q_scale64;
    };
    if constexpr (GATHER) {
      auto tok = [&](int p, int i, const uint8_t*& tile, int& row) __attribute__((always_inline)) -> bool {
        const int ci = c0 + w + 4 * p;
        const int kind = kind_of(ci);
        const int rpc = chunk_rows(kind);
        int start = 0, n = nrow[0];
#pragma unroll
        for (int k = 1; k < NWD; ++k) {
          start = kind == k ? cend[k - 1] : start;
          n = kind == k ? nrow[k] : n;
        }
        const int e0 = (ci - start) * rpc, idx = e0 + i;
        const bool ok = i < rpc && idx < n;
        const uint32_t e = lists[(size_t)kind * a.list_cap + (ok ? idx : e0)];
        tile = pool_h + (size_t)(e >> 8) * tstride;
        row = (int)(e & 255u);
        return ok;
      };
      precise_wave_pass<DK, D, G>(g, nchunk, tok, qv, reinterpret_cast<float*>(sp), &s_wm[w][0], &s_wl[w][0],
                                 &s_wacc[w][0][0]);
    } else {
      auto tok = [&](int p, int i, const uint8_t*& tile, int& row) __attribute__((always_inline)) -> bool {
        tile = pool_h + (size_t)s_tbl[p] * tstride;
        row = 64 * w + i;
        return (b0 + p) * kRows + row < len;
      };
      precise_wave_pass<DK, D, G>(g, nchunk, tok, qv, reinterpret_cast<float*>(sp), &s_wm[w][0], &s_wl[w][0],
                                 &s_wacc[w][0][0]);
    }
  } else {
    const float lt = row_sum16(l_run);
    const float zt0 = row_sum16(zacc0), zt1 = row_sum16(zacc1);
    if (head_ok) {
      if (lj == 0) {
        s_wm[w][la] = m_run;
        s_wl[w][la] = lt;
      }
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const int gam = t >> 2;  // channel 16t + lj lies in V group t / 4
        const float val = gam ? (o[t][2] + o[t][3]) * kTwo24 + zt1 : (o[t][0] + o[t][1]) * kTwo24 + zt0;
        s_wacc[w][la][16 * t + lj] = val;
      }
    }
  }
  // The waves' partials are exchanged through LDS only: a full barrier would also wait for loads still in
  // flight (the precise pass's, or a gather loop's last prefetch).
  lds_barrier();
  if (ns == 1) {
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
  lds_barrier();
  splitk_arrive<D, G>(g, a, seq, h, split, ns, len, tid, s_pm, s_pl, &s_pacc[0][0], &s_wacc[0][0][0]);
}

template <int G, int DK>
hipError_t launch_g(const TileGeom& g, const DecodeArgs& a, hipStream_t stream) {
  const dim3 grid(a.plan.wgs);
  if (g.mixed == 2) {
    hipLaunchKernelGGL(compact_rows_k<4>, dim3(a.n_seqs), dim3(kCompactThreads), 0, stream, g, a);
    hipLaunchKernelGGL((decode_rows_k<G, true, true, DK>), grid, dim3(256), 0, stream, g, a);
  } else if (a.mask || g.mixed) {
    hipLaunchKernelGGL(compact_rows_k<2>, dim3(a.n_seqs), dim3(kCompactThreads), 0, stream, g, a);
    hipLaunchKernelGGL((decode_rows_k<G, true, false, DK>), grid, dim3(256), 0, stream, g, a);
  } else {
    hipLaunchKernelGGL((decode_rows_k<G, false, false, DK>), grid, dim3(256), 0, stream, g, a);
  }
  return hipGetLastError();
}

}  // namespace

// Layouts with this kernel: per-token K and V groups of 64, 4-bit pools and pools of per-token widths, G = 1, 2,
// 4; head dim 128, or (MLA pools) K 192 and V 128 without rotation. (`masked`, whether the call has a sentinel
// mask, does not restrict it.)
bool decode_rows_supported(const TileGeom& g, int G, bool masked) {
  (void)masked;
  if (g.kg != 64 || g.vg != 64 || g.fp8 || !(G == 1 || G == 2 || G == 4)) return false;
  if (g.d == 128 && g.dv == 128) return true;
  return g.d == 192 && g.dv == 128 && !g.rotate;
}

hipError_t launch_decode_rows(const TileGeom& g, const DecodeArgs& a, hipStream_t stream) {
  if (g.d == 192) {
    switch (a.G) {
      case 1: return launch_g<1, 192>(g, a, stream);
      case 2: return launch_g<2, 192>(g, a, stream);
      case 4: return launch_g<4, 192>(g, a, stream);
    }
    return hipErrorInvalidValue;
  }
  switch (a.G) {
    case 1: return launch_g<1, 128>(g, a, stream);
    case 2: return launch_g<2, 128>(g, a, stream);
    case 4: return launch_g<4, 128>(g, a, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace kvq
