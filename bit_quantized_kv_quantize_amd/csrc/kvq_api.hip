// kvq_api.hip - the C ABI of libkvq: argument validation, tile geometry, split planning and launches.
// Every entry point is declared and documented in include/kvq.h.
#include <math.h>
#include <stdlib.h>

#include <algorithm>
#include <mutex>
#ifdef KVQ_DEBUG
#include <stdio.h>

#include <vector>
#endif

#include "kvq_internal.hpp"

namespace kvq {

static bool is_group(int g, int d) {
  return (g == 8 || g == 16 || g == 32 || g == 64 || g == 128 || g == 256) && g <= d && d % g == 0;
}

static int v_dim(const kvq_layout* L) { return L->v_head_dim > 0 ? L->v_head_dim : L->head_dim; }

int check_layout(const kvq_layout* L) {
  if (!L) return KVQ_ERR_ARG;
  const int d = L->head_dim, dv = v_dim(L);
  if (!(d == 64 || d == 128 || d == 192 || d == 256) || L->v_head_dim < 0) return KVQ_ERR_ARG;
  if (!(dv == 64 || dv == 128 || dv == 192 || dv == 256)) return KVQ_ERR_ARG;
  if (L->num_kv_heads <= 0 || L->num_kv_heads > 4096) return KVQ_ERR_ARG;
  if (L->block_tokens != kRows) return KVQ_ERR_ARG;
  // unequal K and V head dims (MLA): K 192 or 256 with V 128, per-token K groups, integer codes
  const bool unequal = dv != d;
  if (unequal && !((d == 192 || d == 256) && dv == 128)) return KVQ_ERR_UNSUPPORTED;
  if (d == 192 && !unequal) return KVQ_ERR_UNSUPPORTED;  // (dv = 192 is covered by the pair check above)
  if (L->format == 1) {  // FP8 E4M3 per element
    if (L->k_group != 0 || L->v_group != 0 || L->mixed != 0) return KVQ_ERR_ARG;
    if (L->rotate != 0 && L->rotate != 1) return KVQ_ERR_ARG;
    return unequal ? KVQ_ERR_UNSUPPORTED : KVQ_OK;
  }
  if (L->format != 0) return KVQ_ERR_ARG;
  if (!(L->k_group == -1 || is_group(L->k_group, d))) return KVQ_ERR_ARG;
  if (!is_group(L->v_group, dv)) return KVQ_ERR_ARG;
  if ((L->rotate != 0 && L->rotate != 1) || L->mixed < 0 || L->mixed > 2) return KVQ_ERR_ARG;
  if (L->rotate && d == 192) return KVQ_ERR_UNSUPPORTED;  // the rotation needs power-of-two dims
  if (L->mixed && L->k_group < 0) return KVQ_ERR_UNSUPPORTED;
  if (unequal && L->k_group < 0) return KVQ_ERR_UNSUPPORTED;
  return KVQ_OK;
}

TileGeom make_geom(const kvq_layout* L) {
  TileGeom g{};
  g.d = L->head_dim;
  g.dv = v_dim(L);
  g.H = L->num_kv_heads;
  g.kg = L->k_group;
  g.vg = L->v_group;
  g.rotate = L->rotate;
  g.mixed = L->mixed;
  g.fp8 = L->format == 1;
  g.rec = (g.d + g.dv) * (g.mixed == 2 ? 16 : (g.mixed || g.fp8) ? 8 : 4) / 8;
  g.kpr = g.kg > 0 ? g.d / g.kg : 0;
  g.vpr = g.fp8 ? 0 : g.dv / g.vg;
  g.prow = (g.kpr + g.vpr) * 4;
  g.off_kch = (uint32_t)(kRows * g.rec);
  g.off_prow = g.off_kch + ((g.kg > 0 || g.fp8) ? 0u : (uint32_t)(g.d * 4));
  g.off_hdr = g.off_prow + (uint32_t)(kRows * g.prow);
  uint32_t end = g.off_hdr + g.header_bytes();
  g.tile_bytes = (end + 255u) / 256u * 256u;
  return g;
}

SplitPlan plan_splits(const TileGeom& g, int n_seqs, int num_q_heads, int max_seq_len) {
  // One round of resident workgroups on MI355X (256 CUs x 2 decode workgroups each): split each
  // (sequence, KV head) so the grid fills that round without exceeding it, never below one block per split.
  const long target_wgs = 256 * 2;
  int nb = (max_seq_len + kRows - 1) / kRows;
  if (nb < 1) nb = 1;
  long units = (long)(n_seqs > 0 ? n_seqs : 1) * g.H;
  long ns = target_wgs / units;
  if (ns < 1) ns = 1;
  if (ns > nb) ns = nb;
  if (ns > 64) ns = 64;                                // at most 64 splits per (sequence, KV head)
  if (ns < (nb + 511) / 512) ns = (nb + 511) / 512;  // a split owns at most 512 blocks
  SplitPlan p;
  p.n_splits = (int)ns;
  p.blocks_per_split = (int)((nb + ns - 1) / ns);
  // Row-list kernel: the same round of 512 workgroups, but as one-dimensional grid in which pairs may get
  // k or k + 1 splits, so that the grid is exactly full; at most 64 splits per pair and 512 blocks per
  // split, at least one block per workgroup and one workgroup per pair.
  long W = target_wgs;
  if (W > units * nb) W = units * nb;
  if (W > units * 64) W = units * 64;
  if (W < units * ((nb + 511) / 512)) W = units * ((nb + 511) / 512);
  if (W < units) W = units;
  p.wgs = (int)W;
  p.k = (int)(W / units);
  p.nA = (int)(units - (W - (long)p.k * units));
  p.max_blocks = nb;
  const int rows_max = p.nA < units ? p.k + 1 : p.k;
  // Cascade (per-channel K layouts, 2 .. kCascMaxSeqs sequences): row groups of at most kCascRows rows, one
  // workgroup per (block range, KV head, row group) and one workgroup per CU; block ranges of at most 512
  // blocks. The range count is chosen as if every sequence shared every block.
  const int G = g.H > 0 ? num_q_heads / g.H : 1;
  p.casc = 0;
  p.casc_slots = 0;
  if (n_seqs >= 2 && n_seqs <= kCascMaxSeqs && decode_cascade_supported(g, G) &&
      nb <= kCascMaxRanges * kCascRangeCols) {
    const long n_rows = (long)n_seqs * G;  // rows of one KV head
    const long rg = (n_rows + kCascRows - 1) / kCascRows;
    const long pairs = rg * g.H;
    // block ranges S: the count that minimises the work of the busiest CU, (units per CU) x (blocks per
    // unit), with at most kCascSlots / (rows of the call) ranges (the workspace bound), kCascMaxRanges
    // ranges and kCascRangeCols blocks per range
    long s_lo = std::max(1L, (long)(nb + kCascRangeCols - 1) / kCascRangeCols);
    long s_hi = std::min(std::min((long)kCascMaxRanges, (long)nb),
                         std::max(1L, (long)kCascSlots / (n_rows * g.H)));
    if (s_hi < s_lo) s_hi = s_lo;
    long S = s_lo, best = -1;
    for (long c = s_lo; c <= s_hi; ++c) {
      const long cost = ((c * pairs + 255) / 256) * ((nb + c - 1) / c);
      if (best < 0 || cost < best) {
        best = cost;
        S = c;
      }
    }
    p.casc = (int)S;
    p.casc_slots = casc_slots(n_seqs, G);
  }
  p.stride = (p.n_splits > rows_max ? p.n_splits : rows_max) + p.casc;
  return p;
}

WorkspaceLayout workspace_layout(const TileGeom& g, int n_seqs, int num_q_heads, int max_seq_len) {
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  SplitPlan p = plan_splits(g, n_seqs, num_q_heads, max_seq_len);
  size_t ns = (size_t)(n_seqs > 0 ? n_seqs : 0);
  // The partial slots actually used, ns * num_q_heads * p.stride, shrink or grow with the split plan; the
  // regions are sized by a bound that never decreases with n_seqs or max_seq_len, so that a workspace
  // sized for one call serves every smaller one. With G = num_q_heads / H, units = n_seqs * H and
  // c = ceil(blocks / 512): both per-sequence plans give at most G * max(512, units * c) + n_seqs *
  // num_q_heads slots, and the cascade at most kCascSlots + n_seqs * num_q_heads * c64 more (the plan takes
  // at most kCascSlots / (n_seqs * num_q_heads) ranges, or c64 = ceil(blocks / 64) when that is more).
  const size_t G = g.H > 0 ? (size_t)(num_q_heads / g.H) : 1;
  const size_t c512 = (size_t)(p.max_blocks + 511) / 512;
  const size_t rows = ns * (size_t)num_q_heads;
  // The cascade regions exist for every call of two or more sequences on a layout the cascade takes, also
  // where the plan leaves the cascade out (more than kCascMaxSeqs sequences), so that they never shrink.
  const bool casc = ns >= 2 && decode_cascade_supported(g, (int)G);
  size_t parts = G * std::max((size_t)512, ns * g.H * c512) + rows;
  const size_t c64 = (size_t)(p.max_blocks + kCascRangeCols - 1) / kCascRangeCols;
  if (casc) parts += (size_t)kCascSlots + rows * c64;
  WorkspaceLayout w{};
  w.parts = parts;
  w.ml = 0;
  w.acc = w.ml + up(parts * 2 * sizeof(float));  // accumulators of V's head dim
  // row lists only for layouts the row-list kernel reads: one list per width (4 and 8 bits, and 2 and 16
  // in pools of four widths)
  const size_t nwd = g.mixed == 2 ? 4 : 2;
  w.cnt = w.acc + up(parts * g.dv * sizeof(float));
  w.list = w.cnt + up(ns * nwd * sizeof(int));
  w.list_cap = decode_rows_supported(g, num_q_heads / g.H, true) ? (max_seq_len + 63) / 64 * 64 : 0;
  w.bcnt = w.list + up(ns * nwd * (size_t)w.list_cap * sizeof(uint32_t));
  // at least one block per sequence, so the count kernels always have a grid
  w.bcnt_blocks = decode_rows_supported(g, num_q_heads / g.H, true) ? max(1, (max_seq_len + kRows - 1) / kRows) : 0;
  w.cflag = w.bcnt + up(ns * nwd * (size_t)w.bcnt_blocks * sizeof(int));
  // cascade: a flag per (sequence, logical block), the member lists and row groups of every block range
  const size_t slots = casc ? (size_t)casc_slots((int)ns, (int)G) : 0;
  w.cperm = w.cflag + up(casc ? ns * (size_t)p.max_blocks * sizeof(int) : 0);
  w.cdesc = w.cperm + up(casc ? (size_t)kCascMaxRanges * ns * sizeof(int) : 0);
  w.cnrg = w.cdesc + up(slots * kCascMaxRanges * 4 * sizeof(int));
  w.cmask = w.cnrg + up(casc ? (size_t)kCascMaxRanges * sizeof(int) : 0);
  w.body = w.cmask + up(casc ? (size_t)kCascMaxRanges * ns * sizeof(uint64_t) : 0);
  // The split-K arrival counters sit at the end of the caller's workspace (ctr_offset), after every other
  // region: the other regions grow with n_seqs and max_seq_len, so no smaller call sharing the workspace
  // can write partials over a larger call's counters, and a smaller call's counters are a subset of the
  // larger call's (all zero between calls).
  w.ctr_bytes = ns * g.H * sizeof(unsigned);
  w.total = w.body + up(w.ctr_bytes);
  return w;
}

size_t ctr_offset(const WorkspaceLayout& w, size_t workspace_bytes) {
  // the last ctr_bytes below the 4-byte-aligned end; workspace_bytes >= w.total keeps this >= w.body
  return workspace_bytes / 4 * 4 - w.ctr_bytes;
}

size_t decode_workspace_bytes(const TileGeom& g, int n_seqs, int num_q_heads, int max_seq_len) {
  return workspace_layout(g, n_seqs, num_q_heads, max_seq_len).total;
}

static int hip_status(hipError_t e) { return e == hipSuccess ? KVQ_OK : KVQ_ERR_HIP; }

#ifdef KVQ_DEBUG
// Debug builds check the device-resident arguments on the host before any launch: the arrays are copied
// back (a stream synchronisation per array), every block id must address a whole block inside the pool's
// device allocation (hipMemGetAddressRange: the allocation that holds the pointer, so the bound is that
// allocation's end), and lengths and positions must lie in their stated ranges. A violation returns
// KVQ_ERR_ARG with a message on stderr and nothing is launched.
static bool fetch_i32(const int32_t* dev, size_t n, std::vector<int32_t>& host, hipStream_t stream) {
  host.resize(n);
  if (n == 0) return true;
  return hipMemcpyAsync(host.data(), dev, n * sizeof(int32_t), hipMemcpyDeviceToHost, stream) == hipSuccess &&
         hipStreamSynchronize(stream) == hipSuccess;
}
// Blocks of the pool that fit between `pool` and the end of its device allocation (-1 if unknown).
static long pool_blocks(const TileGeom& g, const void* pool) {
  hipDeviceptr_t base = nullptr;
  size_t size = 0;
  if (hipMemGetAddressRange(&base, &size, (hipDeviceptr_t)pool) != hipSuccess || !base) return -1;
  const size_t off = (size_t)((const uint8_t*)pool - (const uint8_t*)base);
  if (off > size) return 0;
  return (long)((size - off) / ((size_t)g.H * g.tile_bytes));
}
static int debug_fail(const char* fn, const char* what, long i, long v) {
  fprintf(stderr, "%s: %s (index %ld, value %ld)\n", fn, what, i, v);
  return KVQ_ERR_ARG;
}
static int check_ids(const char* fn, const TileGeom& g, const void* pool, const int32_t* ids, int n, bool distinct,
                     hipStream_t stream) {
  std::vector<int32_t> h;
  if (!fetch_i32(ids, (size_t)n, h, stream)) return KVQ_ERR_HIP;
  const long nb = pool_blocks(g, pool);
  for (int i = 0; i < n; ++i)
    if (h[i] < 0 || (nb >= 0 && h[i] >= nb)) return debug_fail(fn, "block id outside the pool", i, h[i]);
  if (distinct) {
    std::vector<int32_t> s(h);
    std::sort(s.begin(), s.end());
    for (size_t i = 1; i < s.size(); ++i)
      if (s[i] == s[i - 1]) return debug_fail(fn, "block id repeated", (long)i, s[i]);
  }
  return KVQ_OK;
}
// Table entries of the blocks that slots [0, len) (or the one slot pos) use, for each sequence.
static int check_table(const char* fn, const TileGeom& g, const void* pool, const int32_t* table, int n_seqs,
                       int max_blocks, const std::vector<int32_t>& first, const std::vector<int32_t>& last,
                       hipStream_t stream) {
  std::vector<int32_t> t;
  if (!fetch_i32(table, (size_t)n_seqs * max_blocks, t, stream)) return KVQ_ERR_HIP;
  const long nb = pool_blocks(g, pool);
  for (int s = 0; s < n_seqs; ++s)
    for (int b = first[s]; b < last[s]; ++b) {
      const int32_t id = t[(size_t)s * max_blocks + b];
      if (id < 0 || (nb >= 0 && id >= nb)) return debug_fail(fn, "block table entry outside the pool", s, id);
    }
  return KVQ_OK;
}
#endif

// The rotation of an n-channel row is c H with c = fp32(1 / sqrt(n)); its inverse is (1 / (n c)) H.
static float rot_scale(int n) { return (float)(1.0 / sqrt((double)n)); }
static float unrot_scale(int n) { return (float)(1.0 / ((double)n * (double)rot_scale(n))); }

}  // namespace kvq

using namespace kvq;

// ---------------------------------------------------------------------------------- static scratch
// kvq_decode_attention_static's workspace: one file-scope device array per GPU, held until the process ends.
// Its first kStaticBody bytes take the partials and row lists, the last kStaticCtrBytes the split-K arrival
// counters, which are cleared once per GPU (before the first call's kernels, on its stream) and left at zero
// by every completed call. Host code never uses the array's name as an address: the device address comes
// from hipGetSymbolAddress, once per GPU with that GPU current.
constexpr size_t kStaticBytes = (size_t)KVQ_STATIC_WORKSPACE_BYTES;
constexpr size_t kStaticCtrBytes = (size_t)1 << 20;
constexpr size_t kStaticBody = kStaticBytes - kStaticCtrBytes;
static __device__ __align__(256) uint8_t scratch[kStaticBytes];

namespace {
__global__ void clear_words_k(unsigned* p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) p[i] = 0u;
}
}  // namespace

constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static uint8_t* g_scratch[kMaxDevices];

// The current GPU's scratch address in *base (set up on the first call on that GPU).
static int static_scratch(hipStream_t stream, uint8_t** base) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return KVQ_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return KVQ_ERR_HIP;
    hipLaunchKernelGGL(clear_words_k, dim3(256), dim3(256), 0, stream, (unsigned*)((uint8_t*)ptr + kStaticBody),
                       kStaticCtrBytes / sizeof(unsigned));
    if (hipGetLastError() != hipSuccess) return KVQ_ERR_HIP;
    g_scratch[dev] = (uint8_t*)ptr;
  }
  *base = g_scratch[dev];
  return KVQ_OK;
}

// Both decode entry points. With ctr == nullptr the workspace is the caller's (workspace_bytes of it, split-K
// counters at its end); otherwise `workspace` holds the body regions (workspace_bytes of room for them) and
// `ctr` the counters (ctr_words of room).
static int decode_entry(const char* fn, const kvq_layout* L, const void* pool, const uint16_t* q, int32_t n_seqs,
                        int32_t num_q_heads, const int32_t* block_table, int32_t max_blocks_per_seq,
                        const int32_t* seq_lens, int32_t max_seq_len, const uint32_t* sentinel_mask,
                        int32_t mask_words_per_seq, float softmax_scale, float* out, void* workspace,
                        size_t workspace_bytes, unsigned* ctr, size_t ctr_words, void* stream) {
  int st = check_layout(L);
  if (st != KVQ_OK) return st;
  if (n_seqs < 0 || n_seqs > 65535 || num_q_heads <= 0 || max_blocks_per_seq <= 0 || max_seq_len < 0)
    return KVQ_ERR_ARG;
  if (num_q_heads % L->num_kv_heads != 0) return KVQ_ERR_ARG;
  if ((long)max_seq_len > (long)max_blocks_per_seq * kRows) return KVQ_ERR_ARG;
  if (sentinel_mask && (long)mask_words_per_seq * 32 < (long)max_seq_len) return KVQ_ERR_ARG;
  if (!(softmax_scale == softmax_scale) || isinf(softmax_scale)) return KVQ_ERR_ARG;
  if (n_seqs == 0) return KVQ_OK;
  if (!pool || !q || !block_table || !seq_lens || !out) return KVQ_ERR_ARG;
  TileGeom g = make_geom(L);
  const int G = num_q_heads / g.H;
  if (G > 16) return KVQ_ERR_UNSUPPORTED;
#ifdef KVQ_DEBUG
  {
    std::vector<int32_t> len, first(n_seqs, 0), last(n_seqs);
    if (!fetch_i32(seq_lens, (size_t)n_seqs, len, (hipStream_t)stream)) return KVQ_ERR_HIP;
    for (int s = 0; s < n_seqs; ++s) {
      if (len[s] < 0 || len[s] > max_seq_len)
        return debug_fail(fn, "sequence length outside [0, max_seq_len]", s, len[s]);
      last[s] = (len[s] + kRows - 1) / kRows;
    }
    if ((st = check_table(fn, g, pool, block_table, n_seqs, max_blocks_per_seq, first, last,
                          (hipStream_t)stream)) != KVQ_OK)
      return st;
  }
#endif
  const WorkspaceLayout wl = workspace_layout(g, n_seqs, num_q_heads, max_seq_len);
  const size_t need = ctr ? wl.body : wl.total;
  if (!workspace || workspace_bytes < need || ((uintptr_t)workspace & 255u)) return KVQ_ERR_WORKSPACE;
  if (ctr && wl.ctr_bytes > ctr_words * sizeof(unsigned)) return KVQ_ERR_WORKSPACE;
  DecodeArgs a{};
  a.pool = (const uint8_t*)pool;
  a.q = q;
  a.block_table = block_table;
  a.seq_lens = seq_lens;
  a.mask = sentinel_mask;
  a.out = out;
  a.plan = plan_splits(g, n_seqs, num_q_heads, max_seq_len);
  if ((size_t)n_seqs * num_q_heads * a.plan.stride > wl.parts) return KVQ_ERR_UNSUPPORTED;  // never, by the bound
  uint8_t* ws = (uint8_t*)workspace;
  a.ws_ctr = ctr ? ctr : (unsigned*)(ws + ctr_offset(wl, workspace_bytes));
  a.ws_ml = (float*)(ws + wl.ml);
  a.ws_acc = (float*)(ws + wl.acc);
  a.ws_cnt = (int*)(ws + wl.cnt);
  a.ws_list = (uint32_t*)(ws + wl.list);
  a.list_cap = wl.list_cap;
  a.ws_bcnt = (int*)(ws + wl.bcnt);
  a.bcnt_blocks = wl.bcnt_blocks;
  a.ws_cflag = (int*)(ws + wl.cflag);
  a.ws_cperm = (int*)(ws + wl.cperm);
  a.ws_cdesc = (int*)(ws + wl.cdesc);
  a.ws_cnrg = (int*)(ws + wl.cnrg);
  a.ws_cmask = (uint64_t*)(ws + wl.cmask);
  a.casc = 0;  // set by the dispatcher when the cascade kernel runs
  a.n_seqs = n_seqs;
  a.num_q_heads = num_q_heads;
  a.G = G;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.mask_words = sentinel_mask ? mask_words_per_seq : 0;
  a.q_scale64 = (double)softmax_scale * 1.4426950408889634;  // log2(e)
  a.q_scale = (float)a.q_scale64;
  a.unrot_c = unrot_scale(g.d);
  a.unrot_cv = unrot_scale(g.dv);
  return hip_status(launch_decode(g, a, (hipStream_t)stream));
}


extern "C" {

int kvq_check_layout(const kvq_layout* L) { return check_layout(L); }

size_t kvq_tile_bytes(const kvq_layout* L) {
  if (check_layout(L) != KVQ_OK) return 0;
  return make_geom(L).tile_bytes;
}

size_t kvq_pool_bytes(const kvq_layout* L, int32_t num_blocks) {
  if (check_layout(L) != KVQ_OK || num_blocks < 0) return 0;
  TileGeom g = make_geom(L);
  return (size_t)num_blocks * g.H * g.tile_bytes;
}

size_t kvq_decode_workspace_bytes(const kvq_layout* L, int32_t n_seqs, int32_t num_q_heads,
                                  int32_t max_seq_len) {
  if (check_layout(L) != KVQ_OK || n_seqs < 0 || num_q_heads <= 0 || max_seq_len < 0) return 0;
  TileGeom g = make_geom(L);
  if (num_q_heads % g.H != 0) return 0;
  return decode_workspace_bytes(g, n_seqs, num_q_heads, max_seq_len);
}

const char* kvq_status_string(int status) {
  switch (status) {
    case KVQ_OK: return "ok";
    case KVQ_ERR_ARG: return "invalid argument";
    case KVQ_ERR_UNSUPPORTED: return "unsupported layout or request";
    case KVQ_ERR_WORKSPACE: return "workspace missing or too small";
    case KVQ_ERR_HIP: return "HIP launch error";
    default: return "unknown status";
  }
}

int kvq_quantize_blocks(const kvq_layout* L, void* pool, const int32_t* block_ids, int32_t n_blocks,
                        const uint16_t* k, const uint16_t* v, const uint32_t* prec_bits, void* stream) {
  int st = check_layout(L);
  if (st != KVQ_OK) return st;
  if (n_blocks < 0) return KVQ_ERR_ARG;
  if (prec_bits && !L->mixed) return KVQ_ERR_ARG;
  if (n_blocks == 0) return KVQ_OK;
  if (!pool || !block_ids || !k || !v) return KVQ_ERR_ARG;
  TileGeom g = make_geom(L);
#ifdef KVQ_DEBUG
  if ((st = check_ids("kvq_quantize_blocks", g, pool, block_ids, n_blocks, true, (hipStream_t)stream)) != KVQ_OK)
    return st;
#endif
  return hip_status(launch_quantize_blocks(g, (uint8_t*)pool, block_ids, n_blocks, k, v, prec_bits, rot_scale(g.d),
                                           rot_scale(g.dv), (hipStream_t)stream));
}

int kvq_dequantize_blocks(const kvq_layout* L, const void* pool, const int32_t* block_ids, int32_t n_blocks,
                          uint16_t* k_out, uint16_t* v_out, void* stream) {
  int st = check_layout(L);
  if (st != KVQ_OK) return st;
  if (n_blocks < 0) return KVQ_ERR_ARG;
  if (n_blocks == 0) return KVQ_OK;
  if (!pool || !block_ids || !k_out || !v_out) return KVQ_ERR_ARG;
  TileGeom g = make_geom(L);
#ifdef KVQ_DEBUG
  if ((st = check_ids("kvq_dequantize_blocks", g, pool, block_ids, n_blocks, false, (hipStream_t)stream)) != KVQ_OK)
    return st;
#endif
  return hip_status(launch_dequantize_blocks(g, (const uint8_t*)pool, block_ids, n_blocks, k_out, v_out,
                                             unrot_scale(g.d), unrot_scale(g.dv), (hipStream_t)stream));
}

int kvq_copy_blocks(const kvq_layout* L, const void* src_pool, const int32_t* src_ids, void* dst_pool,
                    const int32_t* dst_ids, int32_t n_blocks, void* stream) {
  int st = check_layout(L);
  if (st != KVQ_OK) return st;
  if (n_blocks < 0) return KVQ_ERR_ARG;
  if (n_blocks == 0) return KVQ_OK;
  if (!src_pool || !src_ids || !dst_pool || !dst_ids) return KVQ_ERR_ARG;
  if (((uintptr_t)src_pool & 15u) || ((uintptr_t)dst_pool & 15u)) return KVQ_ERR_ARG;
  TileGeom g = make_geom(L);
#ifdef KVQ_DEBUG
  if ((st = check_ids("kvq_copy_blocks", g, src_pool, src_ids, n_blocks, false, (hipStream_t)stream)) != KVQ_OK ||
      (st = check_ids("kvq_copy_blocks", g, dst_pool, dst_ids, n_blocks, true, (hipStream_t)stream)) != KVQ_OK)
    return st;
#endif
  return hip_status(launch_copy_blocks(g, (const uint8_t*)src_pool, src_ids, (uint8_t*)dst_pool, dst_ids, n_blocks,
                                       (hipStream_t)stream));
}

int kvq_append_tokens(const kvq_layout* L, void* pool, int32_t n_seqs, const uint16_t* k, const uint16_t* v,
                      const int32_t* block_table, int32_t max_blocks_per_seq, const int32_t* positions,
                      const uint8_t* prec, void* stream) {
  int st = check_layout(L);
  if (st != KVQ_OK) return st;
  if (L->k_group < 0) return KVQ_ERR_UNSUPPORTED;
  if (n_seqs < 0 || max_blocks_per_seq <= 0) return KVQ_ERR_ARG;
  if (prec && !L->mixed) return KVQ_ERR_ARG;
  if (n_seqs == 0) return KVQ_OK;
  if (!pool || !k || !v || !block_table || !positions) return KVQ_ERR_ARG;
  TileGeom g = make_geom(L);
#ifdef KVQ_DEBUG
  {
    std::vector<int32_t> pos, first(n_seqs), last(n_seqs);
    if (!fetch_i32(positions, (size_t)n_seqs, pos, (hipStream_t)stream)) return KVQ_ERR_HIP;
    for (int s = 0; s < n_seqs; ++s) {
      if (pos[s] < 0 || (long)pos[s] >= (long)max_blocks_per_seq * kRows)
        return debug_fail("kvq_append_tokens", "position outside the block table", s, pos[s]);
      first[s] = pos[s] / kRows;
      last[s] = first[s] + 1;
    }
    if ((st = check_table("kvq_append_tokens", g, pool, block_table, n_seqs, max_blocks_per_seq, first, last,
                          (hipStream_t)stream)) != KVQ_OK)
      return st;
  }
#endif
  return hip_status(launch_append_tokens(g, (uint8_t*)pool, n_seqs, k, v, block_table, max_blocks_per_seq,
                                         positions, prec, rot_scale(g.d), rot_scale(g.dv), (hipStream_t)stream));
}

int kvq_decode_attention(const kvq_layout* L, const void* pool, const uint16_t* q, int32_t n_seqs,
                         int32_t num_q_heads, const int32_t* block_table, int32_t max_blocks_per_seq,
                         const int32_t* seq_lens, int32_t max_seq_len, const uint32_t* sentinel_mask,
                         int32_t mask_words_per_seq, float softmax_scale, float* out, void* workspace,
                         size_t workspace_bytes, void* stream) {
  return decode_entry("kvq_decode_attention", L, pool, q, n_seqs, num_q_heads, block_table, max_blocks_per_seq,
                      seq_lens, max_seq_len, sentinel_mask, mask_words_per_seq, softmax_scale, out, workspace,
                      workspace_bytes, nullptr, 0, stream);
}

int kvq_decode_attention_static(const kvq_layout* L, const void* pool, const uint16_t* q, int32_t n_seqs,
                                int32_t num_q_heads, const int32_t* block_table, int32_t max_blocks_per_seq,
                                const int32_t* seq_lens, int32_t max_seq_len, const uint32_t* sentinel_mask,
                                int32_t mask_words_per_seq, float softmax_scale, float* out, void* stream) {
  uint8_t* base = nullptr;
  const int st = static_scratch((hipStream_t)stream, &base);
  if (st != KVQ_OK) return st;
  return decode_entry("kvq_decode_attention_static", L, pool, q, n_seqs, num_q_heads, block_table,
                      max_blocks_per_seq, seq_lens, max_seq_len, sentinel_mask, mask_words_per_seq, softmax_scale,
                      out, base, kStaticBody, (unsigned*)(base + kStaticBody), kStaticCtrBytes / sizeof(unsigned),
                      stream);
}

}  // extern "C"
