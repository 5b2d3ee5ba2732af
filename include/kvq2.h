/*
 * libkvq2 — OSCAR-style INT2 KV-cache quantize-append and fused split-K
 * decode attention for AMD Instinct MI355X (gfx950).
 *
 * Method (web pages, cited by title and section):
 *   "Technical summary: OSCAR - Offline Spectral Covariance-Aware Rotation
 *    for 2-bit KV cache quantization" (gist.science 2605.17757):
 *      sec. 2.2-A items 1-4  offline calibration: C_Q, C_S, eigenbasis,
 *                            R = U . H_Had . P_br, per-layer clip thresholds;
 *      sec. 2.2-B            online serving: bf16 sink + recent tokens, INT2
 *                            history after the fixed rotation and clipping, a
 *                            fused kernel that unpacks, dequantizes, undoes the
 *                            rotation and attends, over a paged cache.
 *   tilnote.io note on OSCAR (Together AI), "why it matters for serving":
 *      INT2 history with bf16 sink and recent tokens in a paged KV cache.
 *
 * Conventions (readings where the pages are silent):
 *   - head_dim = 128; query head g uses KV head g / (n_q_heads / n_kv_heads).
 *   - R is stored row-major fp32 [128][128] per KV head and applied as
 *     x' = R^T x (x'_i = sum_j R[j][i] x_j).  Keys are rotated by R_K, values
 *     by R_V; the query is rotated once by R_K^T and the output mapped back
 *     once with o = R_V o'.
 *   - Rotation of a new vector: fp64 accumulation over j = 0..127 in order,
 *     rounded to fp32 then to bf16 (round-to-nearest-even).
 *   - INT2 quantizer per (token, KV head, K|V) group of quant_group
 *     contiguous rotated channels (128: the whole vector; 32 or 64: 4 or 2
 *     groups, each with its own pair):
 *     x = clamp(r, -clip, clip) + 0; s = fp16((max x - min x) / 3);
 *     z = fp16(min x); code = clamp(rint((x - z) * (1 / s)), 0, 3) with each
 *     fp32 step rounded separately; s == 0 gives all-zero codes.
 *     Dequantized value: z + code * s.
 *   - Segments of a sequence of length L (positions 0..L-1):
 *       sink   [0, min(L, n_sink))                 bf16, rotated
 *       INT2   [n_sink, max(n_sink, L - n_recent))  paged INT2
 *       recent [max(n_sink, L - n_recent), L)      bf16 ring, rotated
 *
 * Memory layout (all device buffers are owned by the caller):
 *   pool         uint8 [num_pages][n_kv_heads][page_size/16][C]
 *                with C = 1024 + 128 ng bytes, ng = 128 / quant_group
 *                (1152 for one pair per vector, 1280 or 1536).
 *                One C-byte chunk holds 16 consecutive positions
 *                16c..16c+15 of one sequence and one KV head.  Position pos
 *                lives in physical page block_table[b][pos / page_size],
 *                chunk (pos % page_size) / 16, slot t = pos % 16.
 *                Chunk bytes (four channels 4g..4g+3 of one token share a
 *                byte; channel 4g+k occupies bits 2k..2k+1):
 *                  [   0,  512) K codes: byte 32*t + g
 *                  [ 512, 1024) V codes: byte 512 + 32*(g % 16) + 8*(t / 4)
 *                                              + 4*(g / 16) + (t % 4)
 *                  [1024, 1024 + 64 ng) K params: group k of slot t at
 *                        1024 + 4 (t ng + k): fp16 s, fp16 z
 *                  [1024 + 64 ng, C) V params: group k of slot t at
 *                        1024 + 64 ng + 4 (t ng + k)
 *                (fp16 little-endian; g = channel / 4 in 0..31; group k
 *                covers channels [k quant_group, (k + 1) quant_group).)
 *                Slots of sink positions and of positions still in the recent
 *                window are never written or read.
 *   sink         bf16 [batch][n_kv_heads][n_sink][2][128]   (K' then V')
 *   recent       bf16 [batch][n_kv_heads][n_recent][2][128] ring: position
 *                pos lives in slot (pos - n_sink) % n_recent
 *   block_table  int32 [batch][bt_stride]; entries for every page that holds
 *                an INT2 position of the sequence must be valid page numbers
 *                in [0, num_pages).  Several sequences may share pages (a
 *                shared read-only prefix).
 *
 * Error behaviour: every entry point validates its arguments on the host
 * before any HIP call and returns a negative kvq_status without side effects
 * on failure.  Device faults surface at the caller's next synchronisation.
 * Non-finite q/K/V values give unspecified (but memory-safe) results.
 * All pointers must be 16-byte aligned.  Calls are asynchronous on `stream`
 * (a hipStream_t; NULL means the default stream) except kvq_calibrate.
 */
#ifndef KVQ2_H
#define KVQ2_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum kvq_status {
  KVQ_OK = 0,
  KVQ_ERR_ARG = -1,          /* null/misaligned pointer, bad size or count */
  KVQ_ERR_UNSUPPORTED = -2,  /* head_dim != 128, page size, group size > 16 */
  KVQ_ERR_WORKSPACE = -3,    /* decode workspace smaller than required */
  KVQ_ERR_NUMERIC = -4,      /* calibrate: non-finite input, no convergence,
                                clip threshold outside (0, 16384] */
  KVQ_ERR_HIP = -5           /* a HIP launch or runtime call failed */
};

typedef struct kvq_dims {
  int32_t n_q_heads;   /* Hq  >= 1, a multiple of n_kv_heads               */
  int32_t n_kv_heads;  /* Hkv >= 1; Hq / Hkv <= 16                          */
  int32_t head_dim;    /* must be 128                                       */
  int32_t page_size;   /* tokens per page: 16, 32 or 64                     */
  int32_t n_sink;      /* >= 0 bf16 sink tokens                             */
  int32_t n_recent;    /* >= 1 bf16 recent-window tokens (ring size)        */
  float sm_scale;      /* softmax scale; <= 0 selects 1/sqrt(head_dim)      */
  int32_t quant_group; /* channels per INT2 (scale, zero) pair: 32, 64 or    */
                       /* 128 (0 selects 128, one pair per vector)           */
  int32_t hadamard_block; /* kvq_calibrate: size of the diagonal Hadamard   */
                       /* blocks, 32, 64 or 128 (0 selects 128, the full    */
                       /* transform); the online calls take R as given      */
} kvq_dims;

/* Per-layer calibration products (device pointers for the online calls). */
typedef struct kvq_layer {
  const float* R_K;    /* fp32 [Hkv][128][128], orthogonal, applied as R^T x */
  const float* R_V;    /* fp32 [Hkv][128][128]                              */
  float clip_K;        /* 0 < clip <= 16384                                 */
  float clip_V;
} kvq_layer;

typedef struct kvq_cache {
  uint8_t* pool;              /* see layout above                           */
  int64_t num_pages;          /* physical pages in `pool`                   */
  uint16_t* sink;             /* bf16; may be NULL when n_sink == 0         */
  uint16_t* recent;           /* bf16 ring                                  */
  const int32_t* block_table; /* int32 [batch][bt_stride]                   */
  int32_t bt_stride;          /* >= ceil(max length / page_size)            */
} kvq_cache;

/*
 * Offline calibration of one layer on the host (synchronous, host memory).
 * OSCAR summary sec. 2.2-A: C_Q = (1/N) sum q q^T pooled over the query heads
 * of each KV head; C_S = (1/N) V^T S^T S V = (1/N) O^T O with S the causal
 * softmax scores of the calibration tokens; eigenbases U_Q, U_S (descending
 * eigenvalues; each column's largest-magnitude entry positive); R = U H P
 * with H the 128x128 Sylvester Hadamard / sqrt(128) and P the 7-bit
 * bit-reversal permutation; clip = nearest-rank `clip_quantile` quantile of
 * |rotated calibration values| over all tokens, KV heads and channels.
 *   q   bf16 [n_tokens][Hq][128];  k, v  bf16 [n_tokens][Hkv][128]
 *   R_K, R_V  out fp32 [Hkv][128][128];  clip_K, clip_V  out (one float each)
 * 0 < clip_quantile <= 1.  n_tokens >= 1.  Uses up to 16 host threads.
 */
int kvq_calibrate(const kvq_dims* dims, int32_t n_tokens,
                  const uint16_t* q, const uint16_t* k, const uint16_t* v,
                  double clip_quantile,
                  float* R_K, float* R_V, float* clip_K, float* clip_V);

/*
 * Quantize-append (OSCAR summary sec. 2.2-B).  For every sequence b, the
 * tokens cu_new[b] .. cu_new[b+1]-1 of k_new/v_new are appended at positions
 * start_pos[b], start_pos[b]+1, ...  Each new K/V head-vector is rotated;
 * positions < n_sink go to the sink; positions older than the recent window
 * at the end of this append go straight to INT2 pages; the rest go to the
 * ring.  Ring tokens pushed out of the window are first quantized from their
 * stored bf16 values into INT2.  Byte-identical to appending one token at a
 * time.
 *   start_pos  device int32 [batch]      length of each sequence before the call
 *   cu_new     device int32 [batch + 1]  token offsets (cu_new[0] = 0)
 *   total_new  host: cu_new[batch];  max_new host: max per-sequence count
 *   k_new, v_new  device bf16 [total_new][Hkv][128]
 * Page entries of every INT2 position written must exist in block_table.
 */
int kvq_quantize_append(const kvq_dims* dims, const kvq_layer* layer,
                        const kvq_cache* cache, int32_t batch,
                        const int32_t* start_pos, const int32_t* cu_new,
                        int32_t total_new, int32_t max_new,
                        const uint16_t* k_new, const uint16_t* v_new,
                        void* stream);

/*
 * Bytes of device workspace kvq_decode_attention needs for this batch and
 * longest sequence: split-K partial results and one arrival counter per
 * (sequence, KV head).  The caller allocates it, zero-fills it once, and may
 * reuse it for every later call with the same or smaller sizes: each call
 * leaves the counters at zero again.  Concurrent calls must not share it.
 */
size_t kvq_decode_workspace_bytes(const kvq_dims* dims, int32_t batch,
                                  int32_t max_seq_len);

/*
 * Decode attention of one new query per sequence over its whole cache
 * (OSCAR summary sec. 2.2-B, fused INT2 attention).  q' = R_K^T q once per
 * query head; logits sm_scale * q' . k' over the sink, INT2 (dequantized in
 * registers) and recent segments; one softmax; o' = sum p v' in rotated
 * space; out = R_V o' once.
 *   seq_len      device int32 [batch]  length L of every sequence (>= 0)
 *   max_seq_len  host, >= every seq_len (sizes the split-K grid)
 *   q            device bf16 [batch][Hq][128]
 *   out          device fp32 [batch][Hq][128]  (an empty sequence gives 0)
 * Split-K boundaries, and so the last bits of `out`, can differ between
 * calls on identical inputs: for long contexts the matrix-core decode cuts
 * its ranges with weights it calibrates from the durations measured in
 * earlier calls on the same GPU (library-owned device state, shared by every
 * caller on that GPU; concurrent calls only perturb the weights within
 * their bounds).  The environment variable KVQ_ADAPT=0 keeps the launch
 * weights fixed.
 */
int kvq_decode_attention(const kvq_dims* dims, const kvq_layer* layer,
                         const kvq_cache* cache, int32_t batch,
                         const int32_t* seq_len, int32_t max_seq_len,
                         const uint16_t* q, float* out,
                         void* workspace, size_t workspace_bytes,
                         void* stream);

/*
 * Multi-query attention over the same cache (speculative verification,
 * chunked prefill; OSCAR summary sec. 2.2-B: one fused kernel serves the
 * mixed-precision cache).  Each sequence b has n_query = M queries at its
 * last M positions L - M .. L - 1, whose keys and values were appended
 * before this call (seq_len holds L, including them); query m attends
 * causally to positions 0 .. L - M + m.  Same rotation, segments, softmax
 * and output mapping as kvq_decode_attention, which is the case M = 1.
 *   n_query      1 <= M <= n_recent, else KVQ_ERR_ARG (every query then
 *                sees the whole INT2 history, so the causal mask touches
 *                the bf16 window only)
 *   q            device bf16 [batch][M][Hq][128]
 *   out          device fp32 [batch][M][Hq][128]; a query with no visible
 *                position (L < M) gives 0
 *   workspace    kvq_decode_multi_workspace_bytes(dims, batch, max_seq_len, M)
 *                bytes, zero-filled once, reusable as for kvq_decode_attention
 * The queries of a (sequence, KV head) share the passes over its pages: the
 * matrix-core decode takes up to 8 rows (queries x Hq / Hkv) per pass, the
 * VALU decode up to 16, so M queries cost ceil(M Hq / Hkv / 8) passes
 * instead of M decodes.
 */
size_t kvq_decode_multi_workspace_bytes(const kvq_dims* dims, int32_t batch,
                                        int32_t max_seq_len, int32_t n_query);
int kvq_decode_multi_attention(const kvq_dims* dims, const kvq_layer* layer,
                               const kvq_cache* cache, int32_t batch,
                               const int32_t* seq_len, int32_t max_seq_len,
                               int32_t n_query, const uint16_t* q, float* out,
                               void* workspace, size_t workspace_bytes,
                               void* stream);

/*
 * kvq_decode_attention without a caller workspace, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  Same arguments (minus the workspace),
 * validation and results as kvq_decode_attention; the call itself allocates
 * nothing.  Its workspace is a library-owned device scratch of 64 MiB per GPU
 * (a static device array, present on every GPU the library is loaded on until
 * the process ends); the decode's workspace (kvq_decode_workspace_bytes) must
 * fit in it, else KVQ_ERR_WORKSPACE (kvq_last_error says why) before any
 * launch.  The first call on a device resolves that device's scratch address.
 * All calls on one GPU share its scratch and each leaves its contents behind:
 * calls that may overlap in time on one GPU (different streams, or host
 * threads without ordering) race and must not be issued; calls in one
 * stream's order are safe.
 */
int kvq_decode_attention_noalloc(const kvq_dims* dims, const kvq_layer* layer,
                                 const kvq_cache* cache, int32_t batch,
                                 const int32_t* seq_len, int32_t max_seq_len,
                                 const uint16_t* q, float* out, void* stream);

/*
 * One decode step: kvq_quantize_append of the new tokens, then
 * kvq_decode_attention over the cache that includes them (OSCAR summary sec.
 * 2.2-B: quantize on eviction from the recent window, fused INT2 attention).
 * The arguments mean what they mean for those two calls, with the same
 * validation (every error is reported before any launch); the results are
 * identical to theirs, call for call.  Decode-size appends (total_new <=
 * 1024, at most 8 query heads per KV head) run the append inside the decode's
 * q-rotation pre-pass launch, which takes one launch and the pre-pass off
 * the step's critical path; other shapes run the two calls in stream order.
 * seq_len must hold the lengths after the append (start_pos + new tokens).
 */
int kvq_decode_step(const kvq_dims* dims, const kvq_layer* layer,
                    const kvq_cache* cache, int32_t batch,
                    const int32_t* start_pos, const int32_t* cu_new,
                    int32_t total_new, int32_t max_new,
                    const uint16_t* k_new, const uint16_t* v_new,
                    const int32_t* seq_len, int32_t max_seq_len,
                    const uint16_t* q, float* out,
                    void* workspace, size_t workspace_bytes,
                    void* stream);

/*
 * Shared-prefix groups of a batch (prefix caching; OSCAR summary sec. 2.2-B
 * and sec. 3: the fused kernel works with paged attention and prefix
 * caching).  Group j lists the member sequences
 * members[member_start[j] .. member_start[j + 1]) whose positions
 * [0, prefix_len[j]) lie on the same physical pages (equal block-table
 * entries, pages written once and read-only afterwards).  All arrays are
 * device int32:
 *   member_start [n_groups + 1], non-decreasing, member_start[0] = 0 and
 *                member_start[n_groups] = n_members
 *   members      [n_members] sequence indices in [0, batch); a sequence
 *                listed more than once counts as a member of its first
 *                listing only
 *   prefix_len   [n_groups] tokens, >= 0
 * n_groups (0 .. 256) and n_members (0 .. 1024) are host values.
 */
typedef struct kvq_prefix_groups {
  int32_t n_groups;
  int32_t n_members;
  const int32_t* member_start;
  const int32_t* members;
  const int32_t* prefix_len;
} kvq_prefix_groups;

/*
 * kvq_decode_attention with shared prefixes read once per group of four
 * member sequences instead of once per member.  Same arguments, validation
 * and results as kvq_decode_attention (up to the rounding of a different
 * split order), plus the groups.  The INT2 tiles of a member that lie
 * wholly inside its group's prefix are read by the group: each tile is
 * brought into LDS once and attended by up to four members' query rows (one
 * wave each); the rest of the member's cache is decoded as usual and the two
 * parts meet in the split-K combine.  A member whose whole INT2 tiles do not
 * cover the group's prefix (seq_len - n_recent too short) is decoded on its
 * own, as is every sequence when the matrix-core decode does not take the
 * shape (more than 8 query heads per KV head, or quantization groups
 * narrower than 128 channels).
 *   groups     host pointer; groups->n_groups = 0 is a plain decode
 *   workspace  kvq_decode_prefix_workspace_bytes(dims, batch, max_seq_len,
 *              groups) bytes, zero-filled once, reusable as for
 *              kvq_decode_attention (for groups of the same or smaller
 *              n_groups and n_members)
 * Returns KVQ_ERR_ARG for a null groups, n_groups outside 0..256,
 * n_members outside 0..1024, or null arrays when n_groups > 0, and
 * KVQ_ERR_UNSUPPORTED when the batch's and the groups' tiles together
 * exceed the decode's 32-bit tile counters.
 */
size_t kvq_decode_prefix_workspace_bytes(const kvq_dims* dims, int32_t batch,
                                         int32_t max_seq_len,
                                         const kvq_prefix_groups* groups);
int kvq_decode_prefix_attention(const kvq_dims* dims, const kvq_layer* layer,
                                const kvq_cache* cache, int32_t batch,
                                const int32_t* seq_len, int32_t max_seq_len,
                                const uint16_t* q, float* out,
                                const kvq_prefix_groups* groups,
                                void* workspace, size_t workspace_bytes,
                                void* stream);

/* Human-readable name of a kvq_status value (static storage). */
const char* kvq_status_string(int status);

/* Last error text recorded by this thread: the HIP error after KVQ_ERR_HIP,
 * or the reason of a KVQ_ERR_WORKSPACE of kvq_decode_attention_noalloc
 * ("" if none). */
const char* kvq_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* KVQ2_H */
