/*
 * kvq.h - C ABI of the Q4 KV-cache codec and of fused-dequant decode attention (MI355X, gfx950).
 *
 * Sources the operations follow (cited by page title and section; no page prints code):
 *   [AMB]  "Agent Memory Below the Prompt: Persistent Q4 KV Cache for Multi-Agent LLM Inference on
 *          Edge Devices" (gist.science explainer), technical summary, section 2.1 (block pool, Q4
 *          pipeline, BatchQuantizedKVCache, cross-phase injection) and section 2.2 (GQA).
 *   [IKV]  IntentKV article (qiita), section on invalidating instead of compacting (sentinel slot).
 *   [UQ]   UltraQuant news article (poko-everyday), technology section (Walsh-Hadamard rotation,
 *          asymmetric K/V treatment, decode-attention kernel tuned for AMD GPUs).
 *   [QKV]  QKVShare explainer (gist.science, French), methodology section (per-token bit widths,
 *          CacheCard) and claims section (a fused quantized attention kernel is the missing piece).
 *
 * Conventions shared by every entry point
 *   - Every pointer argument except the kvq_layout pointer is a DEVICE pointer to caller-owned memory.
 *     The library allocates nothing, frees nothing, keeps no pointer after returning, and keeps no
 *     mutable global state.
 *   - `stream` is a hipStream_t handle passed as void* (NULL = the null stream). Work is enqueued
 *     asynchronously; the caller keeps buffers alive until the stream has finished and synchronises
 *     itself. Calls that do not write the same pool rows may run concurrently.
 *   - Return value: KVQ_OK (0) or a negative kvq_status. Nothing throws or aborts across the ABI.
 *     Host-visible arguments (layout, sizes, null pointers, workspace size) are validated; device-resident
 *     data (block ids, seq_lens, positions) is trusted and must be in range.
 *   - fp16 values are passed as uint16_t bit patterns (IEEE binary16).
 *
 * Pool layout (the block pool of [AMB] 2.1 item 1 with the Q4 format of [AMB] 2.1 item 2)
 *   A pool holds num_blocks * H_kv tiles; tile (b, h) starts at byte (b * H_kv + h) * kvq_tile_bytes().
 *   A tile holds the 256 token rows of one KV head of one block, in this order (R = 256, d = head_dim,
 *   dv = V's head dim (v_head_dim, else d), w = the pool's widest width: 4; 8 in mixed = 1 and FP8 pools;
 *   16 in mixed = 2 pools):
 *     row records   R x S bytes, S = (d + dv) * w / 8: record t at t * S holds row t's K codes (d * b / 8
 *                   bytes, b = the row's width: 4; 4 or 8; 2, 4, 8 or 16) immediately followed by its V
 *                   codes (dv * b / 8 bytes); the rest of a narrower row's record is zero. A 16-bit row
 *                   holds the (rotated) values themselves as fp16, and its parameter record is zero
 *     K per channel when k_group == -1: d x 4 bytes, [c] {scale, zero}
 *     param records R x P bytes, P = 4 * (d / k_group + dv / v_group) (4 * dv / v_group when K is grouped
 *                   per channel): record t holds row t's K params [group] {scale, zero}, then its V params
 *     header        mixed = 1: 8 x uint32, bit (t % 32) of word (t / 32) set = row t holds 8-bit codes;
 *                   mixed = 2: 16 x uint32, bits 2 (t % 16) .. 2 (t % 16) + 1 of word t / 16 = row t's width
 *                   code (0, 1, 2, 3 = 2, 4, 8, 16 bits)
 *     padding       zero bytes up to the next multiple of 256
 *   A 4-bit row's K and V codes are one contiguous d-byte span, so a decode that gathers live rows reads
 *   each row's codes as one piece (one 128-byte line at d = 128).
 *   4-bit codes: element j of a row sits in bits 4*(j % 8) of little-endian uint32 word j / 8 (byte i holds
 *   elements 2i in its low nibble and 2i+1 in its high nibble). 8-bit codes: one byte per element. 2-bit
 *   codes: element j in bits 2 (j % 4) of byte j / 4.
 *   A parameter entry is {fp16 scale, fp16 zero} (scale at byte 0, zero at byte 2); the pages store a
 *   16-bit scale and bias per group, this library stores them as IEEE fp16.
 *
 * Codec (one group G of fp32 values x; L = 2^b - 1: 3, 15 or 255 for rows of b = 2, 4 or 8 bits)
 *   If layout.rotate: each fp16 row is first mapped to fp32 and rotated, y = c * H * x, H the natural
 *   (Sylvester) Hadamard matrix applied as butterflies with stage strides 1, 2, 4, ..., d/2, each pair
 *   (a, b) -> (a + b, a - b) in fp32, then one multiply by c = fp32(1/sqrt(d)) ([UQ] technology section).
 *   mn = min G, mx = max G (an extreme equal to zero is taken as +0), scale = fp16(rne((mx - mn) / L)),
 *   zero = fp16(rne(mn)); s, z = those fp16 values as fp32; if s == 0 every code is 0, else
 *   r = 1 / s and code = clamp(rint_even((x - z) * r), 0, L). Every step is one IEEE fp32 operation.
 *   Dequantisation is code * s + z (then the inverse rotation if the pool is rotated).
 */
#ifndef KVQ_H
#define KVQ_H

#include <stddef.h>
#include <stdint.h>

/* Every entry point is exported from the shared library; the library's internal symbols are hidden. */
#define KVQ_API __attribute__((visibility("default")))

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
enum kvq_status {
  KVQ_OK = 0,
  KVQ_ERR_ARG = -1,          /* null pointer, negative size, bad layout field, H_q not a multiple of H_kv */
  KVQ_ERR_UNSUPPORTED = -2,  /* valid request this build does not implement (e.g. append into per-channel K) */
  KVQ_ERR_WORKSPACE = -3,    /* workspace pointer null or smaller than kvq_decode_workspace_bytes() */
  KVQ_ERR_HIP = -4           /* the HIP runtime reported an error while launching */
};

/* Geometry and codec options of one pool (the per-architecture cache shape of [AMB] 2.2).
 * Passed by pointer; the library copies it on every call. */
typedef struct kvq_layout {
  int32_t head_dim;     /* d, K's (and the query's) head dim: 64, 128 or 256; 192 with v_head_dim 128 */
  int32_t num_kv_heads; /* H_kv >= 1 */
  int32_t block_tokens; /* rows per block; must be 256 ([AMB] 2.1 item 1) */
  int32_t k_group;      /* > 0: K groups are k_group consecutive channels of one token (8 .. 256, a power
                           of two dividing d); -1: one K group per channel spanning the block's 256 rows
                           (asymmetric K/V grouping, [UQ] technology section) */
  int32_t v_group;      /* > 0: V groups are v_group consecutive channels of one token (8 .. 256, a power
                           of two dividing dv) */
  int32_t rotate;       /* 0 or 1: Walsh-Hadamard rotation of every K and V row before quantisation */
  int32_t mixed;        /* 0: every row 4-bit; 1: each token row is 4-bit or 8-bit; 2: each token row is
                           2-, 4-, 8-bit or FP16 - the per-token widths of [QKV] methodology section.
                           Requires per-token K groups */
  int32_t format;       /* 0: the group-wise integer codes described above (the Q4 cache);
                           1: FP8 E4M3 per element, the FP8 cache the [UQ] technology section compares the
                           4-bit cache against. Requires k_group = v_group = 0 and mixed = 0; a tile is 256
                           records of d K bytes then d V bytes (no parameters), padded to 256 bytes; each
                           (optionally rotated) fp32 value becomes E4M3 ("fn": bias 7, no infinities) by
                           rounding to nearest even, magnitudes of 448 and more saturating to 448. */
  int32_t v_head_dim;   /* dv, V's (and the output's) head dim when it differs from K's, as in MLA models
                           ([AMB] 2.2: K and V head dims differ, e.g. DeepSeek-Coder-V2-Lite); 0 means
                           head_dim. Unequal dims: head_dim 192 or 256 with v_head_dim 128, per-token K
                           groups, format 0; rotation needs power-of-two dims (each tensor is rotated at
                           its own length). Other pairs return KVQ_ERR_UNSUPPORTED. */
} kvq_layout;

/* KVQ_OK if the layout is one this library can store and process, else the status explaining why. */
KVQ_API int kvq_check_layout(const kvq_layout* L);

/* Bytes of one tile (256 rows of one KV head), a multiple of 256; 0 if the layout is invalid. */
KVQ_API size_t kvq_tile_bytes(const kvq_layout* L);

/* Bytes of a pool of num_blocks blocks (num_blocks * H_kv tiles); 0 if invalid. */
KVQ_API size_t kvq_pool_bytes(const kvq_layout* L, int32_t num_blocks);

/* Bytes of device workspace kvq_decode_attention needs for these sizes; 0 if invalid. The value depends
 * only on the arguments and never decreases as n_seqs or max_seq_len grow, so a workspace sized here is
 * valid for every call with the same layout and num_q_heads and the same or smaller n_seqs and
 * max_seq_len. */
KVQ_API size_t kvq_decode_workspace_bytes(const kvq_layout* L, int32_t n_seqs, int32_t num_q_heads,
                                  int32_t max_seq_len);

/* Static, human-readable name of a status code. Never NULL. */
KVQ_API const char* kvq_status_string(int status);

/*
 * kvq_quantize_blocks - quantise whole 256-token blocks into the pool ([AMB] 2.1 items 1-2; rotation
 * and asymmetric K/V grouping from [UQ] technology section; per-token widths from [QKV] methodology).
 *
 *   pool       device, kvq_pool_bytes(L, num_blocks) bytes; every byte of tiles (block_ids[i], h) for
 *              all h is overwritten (codes, params, header, zero padding).
 *   block_ids  device int32 [n_blocks]: physical block receiving input block i. Ids must be distinct
 *              and < the pool's block count (trusted).
 *   n_blocks   >= 0 (0 is a no-op).
 *   k, v       device fp16 k [n_blocks * 256][H_kv][d] and v [n_blocks * 256][H_kv][dv], token-major: row t
 *              of input block i for head h starts at element ((i * 256 + t) * H_kv + h) * d (dv for v).
 *   prec_bits  device uint32 [n_blocks][W] or NULL, the widths of each block's rows (K and V, every head)
 *              in the header's own encoding: mixed = 1, W = 8, bit (t % 32) of word t / 32 set = token t
 *              of block i is 8-bit; mixed = 2, W = 16, bits 2 (t % 16) of word t / 16 = token t's width
 *              code (0, 1, 2, 3 = 2, 4, 8, 16 bits). Must be NULL unless L->mixed; NULL means every token
 *              is 4-bit.
 * Errors: KVQ_ERR_ARG (null pool/k/v/block_ids with n_blocks > 0, prec_bits for a non-mixed layout,
 * invalid layout), KVQ_ERR_UNSUPPORTED, KVQ_ERR_HIP.
 */
KVQ_API int kvq_quantize_blocks(const kvq_layout* L, void* pool, const int32_t* block_ids, int32_t n_blocks,
                        const uint16_t* k, const uint16_t* v, const uint32_t* prec_bits,
                        void* stream);

/*
 * kvq_append_tokens - quantise one new token per sequence into its slot, extending the cached prefix
 * instead of re-encoding it ([AMB] 2.1 item 4, cross-phase injection). Same arithmetic as
 * kvq_quantize_blocks on a single row.
 *
 *   n_seqs       >= 0.
 *   k, v         device fp16 k [n_seqs][H_kv][d], v [n_seqs][H_kv][dv].
 *   block_table  device int32 [n_seqs][max_blocks_per_seq]: logical block -> physical block.
 *   positions    device int32 [n_seqs]: slot of the new token (usually the old sequence length). The
 *                row written is positions[s] % 256 of block block_table[s][positions[s] / 256], which
 *                the caller must have allocated (trusted). Other rows are untouched.
 *   prec         device uint8 [n_seqs]: the row's width - 4 or 8 (mixed = 1), 2, 4, 8 or 16 (mixed =
 *                2); any other value stores a 4-bit row - or NULL (all 4-bit). Must be NULL unless
 *                L->mixed. The row's header field is rewritten and the whole record cleared first, so a
 *                slot may be rewritten at another width.
 * The caller advances its own seq_lens afterwards; this call does not touch them.
 * Errors: KVQ_ERR_ARG, KVQ_ERR_UNSUPPORTED (per-channel K groups: a partial block has no defined
 * channel statistics), KVQ_ERR_HIP.
 */
KVQ_API int kvq_append_tokens(const kvq_layout* L, void* pool, int32_t n_seqs, const uint16_t* k,
                      const uint16_t* v, const int32_t* block_table, int32_t max_blocks_per_seq,
                      const int32_t* positions, const uint8_t* prec, void* stream);

/*
 * kvq_dequantize_blocks - the cache restored as fp16 rows, the unfused path of [QKV] methodology section
 * (injection path: the quantised cache is rebuilt as fp16 key/value tensors before the forward pass),
 * for callers that need plain fp16 K/V; decode attention itself never materialises them.
 *   block_ids  device int32 [n_blocks]: physical blocks to restore, each < num_blocks.
 *   k_out      device fp16 [n_blocks * 256][H_kv][d]: row t of block_ids[i], KV head h, at
 *              ((i * 256 + t) * H_kv + h) * d - the layout kvq_quantize_blocks reads.
 *   v_out      the same for V, with dv channels.
 * Each value is code * scale + zero of its group (per-token or per-channel K groups, the row's own width
 * in mixed pools), un-rotated by (1 / (n c)) H for rotated pools (the inverse of the rotation c H at the
 * tensor's length n = d or dv), rounded
 * once to fp16 (round to nearest even). The arithmetic is fp32: a result may differ from the exact value
 * rounded to fp16 by one fp16 ulp.
 * Errors: KVQ_ERR_ARG, KVQ_ERR_HIP.
 */
KVQ_API int kvq_dequantize_blocks(const kvq_layout* L, const void* pool, const int32_t* block_ids, int32_t n_blocks,
                          uint16_t* k_out, uint16_t* v_out, void* stream);

/*
 * kvq_copy_blocks - copy whole blocks (all H_kv tiles of each) from one pool to another, or within one pool
 * when source and destination tiles do not overlap: the device side of persisting and restoring quantised
 * blocks ([AMB] 2.1: blocks saved and reloaded in their stored form; [QKV] methodology section, the
 * CacheCard passed between agents). A tile holds only its own rows, so a copy is valid at any block id.
 *   src_pool, dst_pool  device pools of the same layout, 16-byte aligned.
 *   src_ids, dst_ids    device int32 [n_blocks]; block src_ids[i] of src_pool goes to block dst_ids[i] of
 *                       dst_pool. Destination ids must be distinct.
 * Errors: KVQ_ERR_ARG, KVQ_ERR_HIP.
 */
KVQ_API int kvq_copy_blocks(const kvq_layout* L, const void* src_pool, const int32_t* src_ids, void* dst_pool,
                    const int32_t* dst_ids, int32_t n_blocks, void* stream);

/*
 * kvq_decode_attention - one decode query per sequence attending over its quantised cache, reading
 * the packed tiles directly and dequantising in registers ([AMB] 2.1 item 2, direct restore without a
 * dequantised copy; 2.1 item 3, many agents batched in one launch; 2.2, GQA; [UQ] technology section,
 * AMD decode-attention kernel; [QKV] claims section, fused quantized attention kernel).
 * Pools with K grouped per channel and no sentinel mask: a logical block that every sequence of the
 * call maps to the same physical block, full in every sequence (a shared prompt prefix, [UQ] technology
 * section), is read once for the whole batch and its partial results merged into each sequence's.
 *
 *   q              device fp16 [n_seqs][num_q_heads][d]; query head j reads KV head j / G,
 *                  G = num_q_heads / H_kv (contiguous GQA groups).
 *   block_table    device int32 [n_seqs][max_blocks_per_seq].
 *   seq_lens       device int32 [n_seqs]: slots 0 .. seq_lens[s]-1 are attended; each value must lie in
 *                  [0, max_seq_len] (trusted) and max_seq_len <= max_blocks_per_seq * 256.
 *   sentinel_mask  device uint32 [n_seqs][mask_words_per_seq] or NULL. Bit (t % 32) of word t / 32 set
 *                  = slot t was remapped to the sentinel slot ([IKV] invalidation section): its logit is
 *                  -1e4 and its value row is 0, so its softmax weight underflows to zero while the
 *                  surviving slots keep their positions. mask_words_per_seq >= ceil(max_seq_len / 32).
 *   softmax_scale  logit = softmax_scale * (q . k) for live slots (usually 1/sqrt(d)).
 *   out            device fp32 [n_seqs][num_q_heads][dv]: softmax-weighted sum of the dequantised (and,
 *                  for rotated pools, un-rotated) V rows. A sequence with seq_lens[s] == 0 gets zeros.
 *   workspace      device scratch of workspace_bytes >= kvq_decode_workspace_bytes(L, n_seqs,
 *                  num_q_heads, max_seq_len) bytes, 256-byte aligned: split-K partials and live-row lists
 *                  from its start, and per-(sequence, KV head) arrival counters (uint32) in its last
 *                  n_seqs * H_kv * 4 bytes below workspace_bytes rounded down to a multiple of 4. Zero-fill
 *                  it once before its first use; every completed call leaves the counters at zero again,
 *                  and no call writes anything else into the counter span of a call of the same or larger
 *                  size, so the same workspace serves later calls of the same or smaller size (same
 *                  layout and num_q_heads) without clearing, provided every call passes the same
 *                  workspace_bytes. Calls sharing one workspace must not overlap on the device.
 * Errors: KVQ_ERR_ARG (also n_seqs > 65535), KVQ_ERR_UNSUPPORTED (more than 16 query heads per
 * KV head), KVQ_ERR_WORKSPACE, KVQ_ERR_HIP.
 */
KVQ_API int kvq_decode_attention(const kvq_layout* L, const void* pool, const uint16_t* q, int32_t n_seqs,
                         int32_t num_q_heads, const int32_t* block_table, int32_t max_blocks_per_seq,
                         const int32_t* seq_lens, int32_t max_seq_len, const uint32_t* sentinel_mask,
                         int32_t mask_words_per_seq, float softmax_scale, float* out, void* workspace,
                         size_t workspace_bytes, void* stream);

/* Bytes of the per-GPU device array that kvq_decode_attention_static uses as its workspace: the last 1 MiB
 * holds the split-K arrival counters, the rest the partials and live-row lists. */
#define KVQ_STATIC_WORKSPACE_BYTES (64u << 20)

/*
 * kvq_decode_attention_static - kvq_decode_attention with no workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * The call allocates nothing (no hipMalloc, hipFree or allocating library routine); its scratch is a
 * file-scope device array of KVQ_STATIC_WORKSPACE_BYTES that each GPU the library runs on holds until the
 * process ends. The first call on a GPU looks up that GPU's copy (hipGetSymbolAddress) and clears its counter
 * span with a small kernel on `stream`, ahead of its own kernels; every completed call leaves the counters at
 * zero again. Arguments, results and errors are those of kvq_decode_attention, plus:
 *   - KVQ_ERR_WORKSPACE when the call needs more than KVQ_STATIC_WORKSPACE_BYTES - 1 MiB of partials and row
 *     lists (kvq_decode_workspace_bytes minus the counters) or more than 1 MiB of counters (n_seqs * H_kv >
 *     262144); nothing is launched;
 *   - KVQ_ERR_HIP when the current GPU's copy of the array cannot be found.
 * Every call on one GPU shares that GPU's array and it keeps the last call's contents: calls that may overlap
 * on one GPU (different streams without ordering between them, or different host threads) race and must be
 * serialised by the caller.
 */
KVQ_API int kvq_decode_attention_static(const kvq_layout* L, const void* pool, const uint16_t* q, int32_t n_seqs,
                                        int32_t num_q_heads, const int32_t* block_table,
                                        int32_t max_blocks_per_seq, const int32_t* seq_lens, int32_t max_seq_len,
                                        const uint32_t* sentinel_mask, int32_t mask_words_per_seq,
                                        float softmax_scale, float* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* KVQ_H */
