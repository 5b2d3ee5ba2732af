/*
 * libkvq2 — HQMQ KV-cache codec: quaternion chunks coded by a product
 * codebook of the binary tetrahedral group and random unit quaternions,
 * median-multiple fp16 outlier chunks, and fused split-K decode attention
 * over the paged codes, for AMD Instinct MI355X (gfx950).  Part of
 * libkvq2.so beside the INT2 path of kvq2.h (status codes, kvq_last_error).
 *
 * Method (web page, cited by title and section):
 *   "Technical summary: Hurwitz quaternion multiplicative quantization for
 *    KV cache compression" (gist.science 2605.27646):
 *      Method 1  each 4-element chunk of a K or V vector is a quaternion
 *                x = r u (r = |x|); u is coded by the word c of
 *                C = {q_p q_s} maximising <u, c>, with q_p in the 24 unit
 *                Hurwitz quaternions (the binary tetrahedral group 2T) and
 *                q_s in S random unit quaternions per (layer, head, role);
 *      Method 2  the secondary quaternions are drawn at random, without
 *                calibration;
 *      Method 3  Med3x: chunks with r > 3 r_med (r_med the median chunk norm
 *                of the current batch) are kept in fp16 with a one-bit flag;
 *      "Memory and latency"  the fused kernel decodes K and V inside the
 *                attention loop.
 *
 * Conventions (readings where the page is silent):
 *   - head_dim = 128; chunk j is channels 4j..4j+3 = (a, b, c, d) of
 *     a + b i + c j + d k; query head g uses KV head g / (Hq / Hkv).
 *   - 2T enumeration: word p < 8 is the unit along axis p / 2 (1, i, j, k)
 *     with sign (-1)^(p % 2); word 8 + m is (1/2)(+-1, +-1, +-1, +-1) with
 *     component t negative iff bit t of m is set.  Codeword 24 s + p is the
 *     Hamilton product q_p q_s, computed in fp64 (each component summed left
 *     to right: a1a2 - b1b2 - c1c2 - d1d2, a1b2 + b1a2 + c1d2 - d1c2,
 *     a1c2 - b1d2 + c1a2 + d1b2, a1d2 + b1c2 - c1b2 + d1a2) and rounded to
 *     fp32.  1 <= S <= 10, so an index fits one byte.
 *   - Encoding, all in fp32 with every operation rounded separately:
 *     r = sqrt(((x0^2 + x1^2) + x2^2) + x3^2); the threshold is
 *     3 * r_med with r_med the lower median (element (n - 1) / 2 in
 *     ascending order) of all n chunk norms of one role (K or V) over every
 *     token and KV head of one append call; chunks with r > threshold are
 *     kept in fp16, at most 3 per record (the largest radii; ties to the
 *     lower chunk index); the other chunks are coded: index = first argmax
 *     of ((u0 c0 + u1 c1) + u2 c2) + u3 c3 with u = x / r (r = 0 gives
 *     index 0), radius code = clamp(rint(r * (255 / r_max)), 0, 255) with
 *     r_max the fp16 (round-to-nearest-even) largest coded radius of the
 *     record (0 codes when r_max is 0).
 *   - Decoding: a coded chunk is (code * r_max / 255) c_index, a kept chunk
 *     its fp16 values.  There is no rotation and no bf16 window: every
 *     token is coded when it is appended.
 *
 * Memory layout (all device buffers are owned by the caller):
 *   codebook_K, codebook_V  fp32 [n_kv_heads][24 S][4]
 *   pool         uint8 [num_pages][n_kv_heads][page_size][2][96]: the K and
 *                V records of position pos of sequence b, KV head h, are at
 *                ((page * n_kv_heads + h) * page_size + pos % page_size)
 *                * 192 (+ 96 for V), page = block_table[b][pos / page_size].
 *                A 96-byte record:
 *                  [ 0, 32)  codeword index of chunk j at byte j
 *                  [32, 64)  radius code of chunk j at byte 32 + j
 *                  [64, 66)  r_max, fp16          [66, 68) zero
 *                  [68, 72)  flags, uint32: bit j = chunk j kept in fp16
 *                  [72, 96)  three slots of 4 fp16: the kept chunks in
 *                            ascending chunk order, unused slots zero
 *                (index and radius bytes of kept chunks are zero).
 *   block_table  int32 [batch][bt_stride]; every page a call touches must be
 *                in [0, num_pages) (others are skipped, memory-safe).
 *
 * Error behaviour as in kvq2.h: arguments are validated on the host before
 * any HIP call (negative kvq_status, no side effects); device faults
 * surface at the caller's next synchronisation; calls are asynchronous on
 * `stream` except kvq_hqmq_codebook.  All pointers 16-byte aligned.
 */
#ifndef KVQ2_HQMQ_H
#define KVQ2_HQMQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
  int32_t n_q_heads;
  int32_t n_kv_heads;
  int32_t head_dim;      /* must be 128 */
  int32_t page_size;     /* 16, 32 or 64 */
  int32_t n_secondary;   /* S in [1, 10] */
  float sm_scale;        /* <= 0: 1 / sqrt(head_dim) */
} kvq_hqmq_dims;

typedef struct {
  const float* codebook_K;   /* device fp32 [n_kv_heads][24 S][4] */
  const float* codebook_V;
} kvq_hqmq_layer;

typedef struct {
  uint8_t* pool;
  int64_t num_pages;
  const int32_t* block_table;
  int32_t bt_stride;
} kvq_hqmq_cache;

/* The codebook of one (layer, head, role): secondary host fp32 [S][4]
 * (unit quaternions, S in [1, 10]) -> codebook host fp32 [24 S][4], word
 * 24 s + p = fp32(q_p q_s) (Method 1).  Synchronous, host memory only.
 * KVQ_ERR_ARG for a null pointer or S out of range, KVQ_ERR_NUMERIC for a
 * non-finite input. */
int kvq_hqmq_codebook(int32_t n_secondary, const float* secondary, float* codebook);

/* Workspace of kvq_hqmq_append for total_new new tokens: the Med3x median
 * selection (histograms and thresholds).  The caller zeroes it once before
 * its first use; every call leaves its histograms zero again.  0 for bad
 * dims. */
size_t kvq_hqmq_append_workspace_bytes(const kvq_hqmq_dims* dims, int32_t total_new);

/* Code and store new tokens (Method 1 and 3): sequence b's new tokens are
 * rows cu_new[b] .. cu_new[b + 1] - 1 of k_new / v_new (bf16 bit patterns
 * [total_new][n_kv_heads][128]) and go to positions start_pos[b] ... The
 * Med3x median of each role runs over all chunks of the call.
 *   start_pos  device int32 [batch]; cu_new device int32 [batch + 1]
 *              (cu_new[0] = 0, non-decreasing, cu_new[batch] = total_new);
 *   max_new    host bound on the new tokens of any sequence;
 *   workspace  device, >= kvq_hqmq_append_workspace_bytes, zeroed once.
 * total_new == 0 returns KVQ_OK and does nothing. */
int kvq_hqmq_append(const kvq_hqmq_dims* dims, const kvq_hqmq_layer* layer,
                    const kvq_hqmq_cache* cache, int32_t batch, const int32_t* start_pos,
                    const int32_t* cu_new, int32_t total_new, int32_t max_new,
                    const uint16_t* k_new, const uint16_t* v_new, void* workspace,
                    size_t workspace_bytes, void* stream);

/* Workspace of kvq_hqmq_decode_attention (split-K partials); 0 for bad
 * arguments.  No zeroing needed. */
size_t kvq_hqmq_decode_workspace_bytes(const kvq_hqmq_dims* dims, int32_t batch,
                                       int32_t max_seq_len);

/* Decode attention of one query per sequence over positions
 * [0, seq_len[b]) of the coded cache ("Memory and latency": K and V are
 * decoded inside the attention loop): out = softmax(sm_scale q K^T) V per
 * query head, with K, V the decoded vectors.
 *   seq_len      device int32 [batch], 0 <= seq_len[b] <= max_seq_len
 *                (0 gives a zero output row);
 *   max_seq_len  host bound, sizes the split-K grid;
 *   q            device bf16 bit patterns [batch][n_q_heads][128];
 *   out          device fp32 [batch][n_q_heads][128];
 *   workspace    device, >= kvq_hqmq_decode_workspace_bytes. */
int kvq_hqmq_decode_attention(const kvq_hqmq_dims* dims, const kvq_hqmq_layer* layer,
                              const kvq_hqmq_cache* cache, int32_t batch, const int32_t* seq_len,
                              int32_t max_seq_len, const uint16_t* q, float* out,
                              void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* KVQ2_HQMQ_H */
