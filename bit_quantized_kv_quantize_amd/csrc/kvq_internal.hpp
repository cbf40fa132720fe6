// kvq_internal.hpp - geometry and launch interfaces shared by the HIP translation units of libkvq.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/kvq.h"

namespace kvq {

constexpr int kRows = 256;  // tokens per block (the block pool of "Agent Memory Below the Prompt", 2.1)

// Byte geometry of one tile, computed once on the host and passed to kernels by value. A tile holds 256
// row records (the K codes of one token, d * width / 8 bytes, immediately followed by its V codes,
// dv * width / 8 bytes; the rest of a narrower row's record is zero), the per-channel K parameters when K
// is grouped per channel, 256 parameter records (K groups then V groups of one token, each {fp16 scale,
// fp16 zero}), the width header of pools with per-token widths, and zero padding to a multiple of 256 bytes.
struct TileGeom {
  int d;            // K's head dim (and the query's)
  int dv;           // V's head dim (and the output's); d unless the layout gives another
  int H;            // KV heads
  int kg;           // K group (channels) or -1 for one group per channel over the block
  int vg;           // V group (channels)
  int rotate;       // Walsh-Hadamard rotation applied before quantisation
  int mixed;        // 1: per-token 4/8-bit rows, 32-byte bitmap at off_hdr; 2: per-token widths 2/4/8/16,
                    // a 2-bit width code per row in a 64-byte header at off_hdr
  int fp8;          // FP8 E4M3 per element: records of d K bytes then d V bytes, no parameters
  int rec;          // bytes of one row record: K and V at the pool's widest width, (d + dv) * w / 8
  int kpr;          // K param entries per row (d / kg), 0 for per-channel K
  int vpr;          // V param entries per row (dv / vg)
  int prow;         // bytes of one parameter record ((kpr + vpr) * 4)
  uint32_t off_kch; // per-channel K params, d entries (kg < 0 only)
  uint32_t off_prow;// parameter record of row 0
  uint32_t off_hdr; // end of the parameter records; the bitmap of mixed pools starts here
  uint32_t tile_bytes;
  __host__ __device__ uint32_t kcode(int t) const { return (uint32_t)t * (uint32_t)rec; }
  // a row's V codes follow its K codes: d/2 bytes in for a 4-bit row, d for an 8-bit row
  __host__ __device__ uint32_t vcode(int t, int bits) const { return kcode(t) + (uint32_t)(d * bits / 8); }
  __host__ __device__ uint32_t kpar(int t) const { return off_prow + (uint32_t)t * (uint32_t)prow; }
  __host__ __device__ uint32_t header_bytes() const { return mixed == 2 ? 64u : (mixed ? 32u : 0u); }
  // width in bits of row t of a tile (4 outside mixed pools; FP8 pools are handled apart)
  __device__ int row_bits(const uint8_t* tile, int t) const {
    if (mixed == 2) return 2 << ((tile[off_hdr + t / 4] >> (2 * (t % 4))) & 3);
    if (mixed) return ((tile[off_hdr + t / 8] >> (t % 8)) & 1) ? 8 : 4;
    return 4;
  }
  __host__ __device__ uint32_t vpar(int t) const { return off_prow + (uint32_t)t * (uint32_t)prow + (uint32_t)kpr * 4u; }
};

int check_layout(const kvq_layout* L);
TileGeom make_geom(const kvq_layout* L);

// Split-K plan of the decode kernels.
// The block kernels cut the logical blocks of every (sequence, KV head) pair into n_splits even ranges
// (split_range) on a (split, KV head, sequence) grid; no range is longer than blocks_per_split.
// The row-list kernel runs a one-dimensional grid of `wgs` workgroups: the first nA pairs get k splits and
// the others k + 1 (rows_work), which fills exactly two workgroups per CU when there are fewer pairs.
// The cascade kernel (blocks shared by two or more sequences, per-channel K layouts) cuts the logical block
// range into casc even ranges; in each range the sequences that share the range's first block form a
// group, whose (sequence, query head) rows are cut into row groups of at most kCascRows rows (at most
// casc_slots row groups per range); its partials take the last casc slots of each row's partial slots.
// `stride` is the number of partial slots per (sequence, query head) in the workspace: the largest split
// count of the per-sequence plans, plus casc.
struct SplitPlan {
  int n_splits;
  int blocks_per_split;
  int stride;
  int wgs;
  int k;
  int nA;
  int max_blocks;  // logical blocks of the longest sequence
  int casc;        // cascade block ranges (0: no cascade slots)
  int casc_slots;  // bound on the cascade row groups of one block range (over all groups of sequences)
};
// Blocks [b0, b1) of split `split` out of ns over a sequence of nblk blocks: even ranges, so the
// splits of a pair differ by at most one block.
__host__ __device__ inline void split_range(int split, int ns, int nblk, int& b0, int& b1) {
  b0 = (int)(((long)split * nblk) / ns);
  b1 = (int)(((long)(split + 1) * nblk) / ns);
}
// Even ranges with the longer ones first: split j of ns over nblk blocks.
__host__ __device__ inline void piece_range(int j, int ns, int nblk, int& b0, int& b1) {
  const int q = nblk / ns, rem = nblk % ns;
  b0 = j * q + (j < rem ? j : rem);
  b1 = b0 + q + (j < rem ? 1 : 0);
}
// Work of workgroup wg of the row-list kernel: the (sequence, KV head) pair, its split and that pair's split
// count. Slots are numbered split-major, first over the nA pairs with k splits, then over the pairs with
// k + 1, so with longer pieces first the slot sizes never grow along the numbering. The first half of the
// grid takes slots in order and the second half in reverse, so workgroups wg and wg + half pair the
// longest pieces with the shortest. (A full launch of 2 x 256 workgroups places those two on one CU.)
__host__ __device__ inline void rows_work(const SplitPlan& p, int n_pairs, int wg, int& pair, int& split, int& nsp) {
  const int half = (p.wgs + 1) / 2;
  const int s = wg < half ? wg : p.wgs - 1 - (wg - half);
  const int sa = p.k * p.nA;
  if (s < sa) {
    split = s / p.nA;
    pair = s - split * p.nA;
    nsp = p.k;
  } else {
    const int nB = n_pairs - p.nA, t = s - sa;
    split = t / nB;
    pair = p.nA + (t - split * nB);
    nsp = p.k + 1;
  }
}
SplitPlan plan_splits(const TileGeom& g, int n_seqs, int num_q_heads, int max_seq_len);
size_t decode_workspace_bytes(const TileGeom& g, int n_seqs, int num_q_heads, int max_seq_len);
// Byte offsets of the workspace regions (partial (m, l), partial accumulators, row counts, row lists,
// cascade flags) for a call of this size, all below `body`; the split-K arrival counters (ctr_bytes) take
// the end of the caller's workspace (ctr_offset). `total` is the size a call of this size needs.
struct WorkspaceLayout {
  size_t ml, acc, cnt, list, bcnt, cflag, cperm, cdesc, cnrg, cmask, body, ctr_bytes, total;
  size_t parts;  // partial slots the ml / acc regions hold
  int list_cap;
  int bcnt_blocks;  // blocks per sequence in the per-block live-row counts
};
WorkspaceLayout workspace_layout(const TileGeom& g, int n_seqs, int num_q_heads, int max_seq_len);
// Offset of the arrival counters in a workspace of workspace_bytes (>= w.total) bytes.
size_t ctr_offset(const WorkspaceLayout& w, size_t workspace_bytes);

// Launchers (defined next to their kernels). They return hipSuccess or the launch error.
// rot_c / unrot_c apply to K rows, rot_cv / unrot_cv to V rows (they differ when the head dims do).
hipError_t launch_quantize_blocks(const TileGeom& g, uint8_t* pool, const int32_t* block_ids, int n_blocks,
                                  const uint16_t* k, const uint16_t* v, const uint32_t* prec_bits,
                                  float rot_c, float rot_cv, hipStream_t stream);
hipError_t launch_dequantize_blocks(const TileGeom& g, const uint8_t* pool, const int32_t* block_ids, int n_blocks,
                                    uint16_t* k_out, uint16_t* v_out, float unrot_c, float unrot_cv,
                                    hipStream_t stream);
hipError_t launch_copy_blocks(const TileGeom& g, const uint8_t* src, const int32_t* src_ids, uint8_t* dst,
                              const int32_t* dst_ids, int n_blocks, hipStream_t stream);
hipError_t launch_append_tokens(const TileGeom& g, uint8_t* pool, int n_seqs, const uint16_t* k,
                                const uint16_t* v, const int32_t* block_table, int max_blocks_per_seq,
                                const int32_t* positions, const uint8_t* prec, float rot_c, float rot_cv,
                                hipStream_t stream);

struct DecodeArgs {
  const uint8_t* pool;
  const uint16_t* q;
  const int32_t* block_table;
  const int32_t* seq_lens;
  const uint32_t* mask;
  float* out;
  unsigned* ws_ctr; // [n_seqs][H_kv] split-K arrival counters (matrix-core kernels), at the workspace's end;
                    // zero between calls
  float* ws_ml;   // [n_seqs][H_q][plan.stride] x {m, l} (the generic kernel: [plan.n_splits])
  float* ws_acc;  // [n_seqs][H_q][plan.stride][d]
  int* ws_cnt;       // [n_seqs][W] live rows per width list (row-list kernel; W = 2: 4-bit, 8-bit; W = 4
                     // in pools of four widths: 4-bit, 8-bit, 2-bit, FP16)
  uint32_t* ws_list; // [n_seqs][W][list_cap] live rows as (physical block << 8 | row)
  int list_cap;
  int* ws_bcnt;      // [n_seqs][bcnt_blocks][W] live rows per width list of each logical block
  int bcnt_blocks;
  int* ws_cflag;     // [n_seqs][plan.max_blocks] 1 where the cascade kernel took the sequence's logical block
  int* ws_cperm;     // [kCascMaxRanges][n_seqs] per block range: the members of its groups, group by group
  int* ws_cdesc;     // [kCascMaxRanges][plan.casc_slots][4] per range: row groups {first member, members,
                     // first row, 0}
  int* ws_cnrg;      // [kCascMaxRanges] row groups of each range
  uint64_t* ws_cmask;  // [kCascMaxRanges][n_seqs] per range, at each member's place in the member list: the
                       // range's columns (bit i = column c0 + i) the member takes
  int casc;          // cascade partial slots merged by the per-sequence kernel in this call (0 or plan.casc)
  int n_seqs;
  int num_q_heads;
  int G;
  int max_blocks_per_seq;
  int mask_words;
  float q_scale;   // softmax_scale * log2(e): logits are kept in base-2 units
  double q_scale64;  // the same in fp64, for logits recomputed in fp64
  float unrot_c;   // 1 / (d * fp32(1/sqrt(d))): inverse of the quantiser's rotation scale of K rows
  float unrot_cv;  // the same for V rows (dv in place of d)
  SplitPlan plan;
};
// Decode dispatch: the row-list matrix-core kernel (per-token K groups) or the per-channel-K matrix-core
// kernel where their layouts are compiled, then the block matrix-core kernel, then the generic kernel.
// In the debug build (KVQ_DEBUG) only, the environment variable KVQ_DECODE_KERNEL (a test hook) may name
// "generic" or "mfma" to skip the kernels before it, or "nocascade" to keep shared blocks in the
// per-sequence kernel.
hipError_t launch_decode(const TileGeom& g, const DecodeArgs& a, hipStream_t stream);
bool decode_rows_supported(const TileGeom& g, int G, bool masked);  // masked: the call has a sentinel mask
bool decode_kchan_supported(const TileGeom& g, int G);
hipError_t launch_decode_kchan(const TileGeom& g, const DecodeArgs& a, hipStream_t stream);
hipError_t launch_decode_rows(const TileGeom& g, const DecodeArgs& a, hipStream_t stream);
hipError_t launch_decode_generic(const TileGeom& g, const DecodeArgs& a, hipStream_t stream);
bool decode_mfma_supported(const TileGeom& g, int G);
// FP8 pools (matrix-core kernel for head_dim 128, G <= 8, calls without a sentinel mask).
bool decode_fp8_supported(const TileGeom& g, int G);
hipError_t launch_decode_fp8(const TileGeom& g, const DecodeArgs& a, hipStream_t stream);
// Cascade kernel for blocks shared by all sequences: layouts of the per-channel-K kernel; the caller then
// runs that kernel with a.casc set.
bool decode_cascade_supported(const TileGeom& g, int G);
constexpr int kCascRows = 128;      // (sequence, query head) rows of one cascade workgroup at most
constexpr int kCascSlots = 32768;   // bound on (query rows of the call) x (cascade block ranges)
constexpr int kCascMaxSeqs = 512;   // sequences of a call that the cascade groups (more: no cascade)
constexpr int kCascMaxRanges = 64;  // cascade block ranges
constexpr int kCascRangeCols = 64;  // logical blocks of one cascade block range at most
constexpr int kCascGrid = 256;      // cascade workgroups (one per CU), each looping over the row groups
// Bound on the row groups of one block range: groups of two or more members (at most n_seqs / 2 of them),
// each cut into ceil(members * G / kCascRows) row groups.
inline int casc_slots(int n_seqs, int G) { return (n_seqs * G + kCascRows - 1) / kCascRows + n_seqs / 2; }
hipError_t launch_decode_cascade(const TileGeom& g, const DecodeArgs& a, hipStream_t stream);
hipError_t launch_decode_mfma(const TileGeom& g, const DecodeArgs& a, hipStream_t stream);

}  // namespace kvq
