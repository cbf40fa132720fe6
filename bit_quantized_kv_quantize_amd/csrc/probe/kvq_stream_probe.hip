// kvq_stream_probe.hip - the streaming-read ceiling the decode kernels are measured against (a measurement
// aid loaded only by the benchmark; it is not part of libkvq).
//
// kvq_probe_read_tiles reads the bytes the 4-bit streaming decode reads from a pool - for every (sequence, KV
// head) pair, every live block's tile, each row's 128 code bytes and 16 parameter bytes (rows past a sequence's
// end re-read row 0 of the wave's rows, as the decode does) - with the same work split (512 workgroups of 4
// waves, each wave 64 rows of every block of its range) and the same loads (whole records in address order
// with non-temporal 16-byte buffer loads, one parameter record per lane), and does no arithmetic beyond folding the loaded words
// into one value per workgroup (written out so nothing is optimised away). Its time is the floor of a kernel with that decode's
// load pattern. kvq_probe_read_linear streams a flat buffer with 16-byte loads from 2048 workgroups: the
// chip's plain read bandwidth. kvq_probe_stream_rw reads one flat buffer and writes a smaller one at a given
// ratio: the read-plus-write ceiling the prefill quantiser is measured against.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
// raw buffer resources on gfx950: the descriptor's fourth word (32-bit data format) and the cache-policy
// operand of a non-temporal load
constexpr int kBufWord3 = 0x00020000;
constexpr int kBufNT = 2;

// grid (wgs), 256 threads. The work split of the decode's one-dimensional plan: with P pairs and W workgroups,
// k = W / P, the first nA = P - (W - k P) pairs take k even pieces of their blocks and the others k + 1; the
// first half of the grid takes pieces in order and the second half in reverse. Each wave reads its 64 rows of
// four blocks at a time (36 16-byte loads per lane in flight), then folds them.
__global__ __launch_bounds__(256) void read_tiles_k(const uint8_t* pool, const int32_t* table, const int32_t* lens,
                                                    int n_seqs, int H, int max_blocks, uint32_t tile_bytes,
                                                    uint32_t rec, uint32_t off_prow, uint32_t prow, int wgs,
                                                    uint32_t* sink) {
  const int pairs = n_seqs * H;
  const int k = wgs / pairs, nA = pairs - (wgs - k * pairs);
  const int half = (wgs + 1) / 2;
  const int slot = (int)blockIdx.x < half ? (int)blockIdx.x : wgs - 1 - ((int)blockIdx.x - half);
  int pair, split, ns;
  if (slot < k * nA) {
    split = slot / nA;
    pair = slot - split * nA;
    ns = k;
  } else {
    const int nB = pairs - nA, t = slot - k * nA;
    split = t / nB;
    pair = nA + (t - split * nB);
    ns = k + 1;
  }
  const int seq = pair / H, h = pair % H;
  const int len = lens[seq];
  const int nblk = (len + 255) / 256;
  const int q = nblk / ns, rem = nblk % ns;
  const int b0 = split * q + (split < rem ? split : rem), b1 = b0 + q + (split < rem ? 1 : 0);
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, la = l >> 4, lj = l & 15;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (int b = b0; b < b1; b += 4) {
    u32x4 x[4][9];
    int phys[4];  // the four blocks' table entries first (the decode stages its table slice before its loads)
#pragma unroll
    for (int i = 0; i < 4; ++i) phys[i] = table[(size_t)seq * max_blocks + min(b + i, b1 - 1)];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int bb = min(b + i, b1 - 1);
      const uint8_t* tile = pool + ((size_t)phys[i] * H + h) * tile_bytes;
      // a block past the range's end reads nothing (a zero-byte buffer resource), as in the decode
      const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint8_t*>(tile), (short)0, b + i < b1 ? (int)tile_bytes : 0, kBufWord3);
      const int lim = len - (bb * 256 + 64 * w);  // rows of the wave's 64 below the sequence's end
      // the wave's 64 records as eight 1 KB slabs in address order, lane l reading piece l % 8 of row
      // 8 j + l / 8 of slab j (non-temporal), then one parameter record per lane (token 16 la + lj)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int rw = 8 * j + 2 * la + (lj >> 3);
        const uint32_t off = (rw < lim ? (uint32_t)(64 * w + rw) : 0u) * rec + (lj & 7) * 16;
        x[i][j] = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, kBufNT);
      }
      const int pr = 16 * la + lj;
      x[i][8] = __builtin_amdgcn_raw_buffer_load_b128(rs, off_prow + (uint32_t)(pr < lim ? 64 * w + pr : 0) * prow,
                                                      0, 0);
    }
    __builtin_amdgcn_sched_barrier(0);  // every load of the four blocks is issued before the first fold
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 9; ++j) acc ^= x[i][j];
  }
  const uint32_t v = acc.x ^ acc.y ^ acc.z ^ acc.w;
  if (v == 0x9E3779B9u) sink[blockIdx.x] = v;  // practically never true; keeps the loads live
}

__global__ __launch_bounds__(256) void read_linear_k(const u32x4* buf, size_t n16, uint32_t* sink) {
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += (size_t)gridDim.x * 256) acc ^= buf[i];
  const uint32_t x = acc.x ^ acc.y ^ acc.z ^ acc.w;
  if (x == 0x9E3779B9u) sink[blockIdx.x] = x;
}

// Streams n_in16 16-byte words in and n_out16 out (n_out16 <= n_in16) with 16-byte loads and stores from a
// grid-stride loop, the output interleaved with the input at their ratio: after input word i the words up to
// floor((i + 1) * n_out16 / n_in16) are written (each the running fold of the thread's input). The
// read-plus-write ceiling of a kernel that transforms one stream into a smaller one, as quantisation does.
__global__ __launch_bounds__(256) void stream_rw_k(const u32x4* in, size_t n_in16, u32x4* out, size_t n_out16) {
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n_in16; i += (size_t)gridDim.x * 256) {
    acc ^= in[i];
    const size_t o0 = i * n_out16 / n_in16, o1 = (i + 1) * n_out16 / n_in16;
    for (size_t o = o0; o < o1; ++o) out[o] = acc;
  }
}

}  // namespace

extern "C" {

// Returns 0, or -1 for bad sizes, -4 for a launch error. sink: device uint32 [wgs] (written only in the
// practically impossible case that a workgroup's fold equals a fixed constant).
__attribute__((visibility("default"))) int kvq_probe_read_tiles(const void* pool, const int32_t* table,
                                                                const int32_t* lens, int n_seqs, int H,
                                                                int max_blocks, uint32_t tile_bytes, uint32_t rec,
                                                                uint32_t off_prow, uint32_t prow, int wgs,
                                                                uint32_t* sink, void* stream) {
  if (n_seqs <= 0 || H <= 0 || wgs < n_seqs * H || max_blocks <= 0) return -1;
  hipLaunchKernelGGL(read_tiles_k, dim3(wgs), dim3(256), 0, (hipStream_t)stream, (const uint8_t*)pool, table, lens,
                     n_seqs, H, max_blocks, tile_bytes, rec, off_prow, prow, wgs, sink);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

__attribute__((visibility("default"))) int kvq_probe_read_linear(const void* buf, size_t bytes, int wgs,
                                                                 uint32_t* sink, void* stream) {
  if (bytes % 16 || wgs <= 0 || ((uintptr_t)buf & 15u)) return -1;
  hipLaunchKernelGGL(read_linear_k, dim3(wgs), dim3(256), 0, (hipStream_t)stream, (const u32x4*)buf, bytes / 16,
                     sink);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

// Returns 0, or -1 for bad sizes, -4 for a launch error. in, out: device buffers of in_bytes and out_bytes
// (16-byte multiples, out_bytes <= in_bytes, 16-byte aligned); out is overwritten.
__attribute__((visibility("default"))) int kvq_probe_stream_rw(const void* in, size_t in_bytes, void* out,
                                                               size_t out_bytes, int wgs, void* stream) {
  if (in_bytes % 16 || out_bytes % 16 || out_bytes > in_bytes || wgs <= 0 || ((uintptr_t)in & 15u) ||
      ((uintptr_t)out & 15u))
    return -1;
  hipLaunchKernelGGL(stream_rw_k, dim3(wgs), dim3(256), 0, (hipStream_t)stream, (const u32x4*)in, in_bytes / 16,
                     (u32x4*)out, out_bytes / 16);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

}  // extern "C"
