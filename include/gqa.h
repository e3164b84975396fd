/*
 * gqa.h - GroupQueryAttention over a shared-buffer KV cache, for gfx950.
 *
 * The operation (from the pages, by title and section):
 *  - "Clarification about GroupQueryAttention behavior" (onnxruntime
 *    discussion), question: past_key and present_key may be one tensor in
 *    BNSH layout [batch, kv_num_heads, max_sequence_length, head_size];
 *    answer: a runtime check that both point to the same address, and the
 *    operator fails when there is no room to append; sliding-window
 *    follow-up: the op keeps the min(total, capacity) most recent tokens,
 *    contiguously.
 *  - "[TorchOnnxToTorch] Add pad+scatter KV cache and mask to GQA"
 *    (torch-mlir pull request), paragraph 1: Q/K/V arrive as
 *    [batch, seq, heads*head_size]; rotary positions are past_len + arange;
 *    K is rotated with kv_num_heads; seqlens_k is 0 for an empty past; the
 *    output is [batch, seq, hidden]. Paragraph 2: new K/V are scattered at
 *    the seqlens_k positions of the buffer; causal visibility is
 *    k_pos <= past_len + q_pos; seqlens_k is int32.
 *  - "KV Cache" (rocMLIR discussion), worked example and notes: per head
 *    softmax(Q K^T) V where the key axis grows inside a max_seq_len buffer
 *    and the key-tile loop ends at the current length instead of masking
 *    the whole buffer.
 *
 * Notation: B batch, S new tokens per sequence, H num_heads, Hkv
 * kv_num_heads (H % Hkv == 0, G = H / Hkv, query head h reads KV head
 * h / G), D head_size, M max_seq_len (= buffer length = window capacity),
 * L_b = seqlens_k[b] = tokens already valid in sequence b's buffer rows.
 *
 * Layouts (all row-major, contiguous, element type = shape->dtype):
 *   q      [B, S, H*D]          k_new, v_new [B, S, Hkv*D]
 *   out    [B, S, H*D]          k_cache, v_cache [B, Hkv, M, D] (BNSH)
 *   cos_cache, sin_cache: fp32 [rotary_rows, D/2]
 *
 * Semantics of one attention call (prefill or decode):
 *   1. rotary (if cos/sin given) on Q (H heads) and K (Hkv heads) at
 *      positions offset_b + L_b + i (offset_b = position_offset[b], 0 when
 *      not given, L_b before any eviction); pairs (j, j + D/2), or (2j, 2j+1) when
 *      rotary_interleaved; each rotated value is the fp64 expression
 *      x1*c - x2*s (resp. x2*c + x1*s) rounded to fp32 then to dtype,
 *      both nearest-even (exact products, so the cache is reproducible
 *      bit for bit);
 *   2. window eviction (only when local_window_size > 0 and L_b + S > M):
 *      rows [d, L_b) move to [0, L_b - d) with d = L_b + S - M, or with
 *      greedy_eviction d = L_b - min(L_b, max(0, W - S)) (the sliding-window
 *      follow-up's "conditional and greedy" eviction);
 *   3. append: cache[b, g, L'_b + i, :] = K/V row (b, i, g); no other byte
 *      of either cache is written;
 *   4. attention: query i of head h at position p = L'_b + i sees key j iff
 *      j <= p and (window off or j >= p - W + 1); out = softmax(scale *
 *      q k^T + bias) v with fp32 accumulation; bytes of the cache past
 *      L'_b + S are never read. The optional bias (attention_bias, the
 *      sliding-window follow-up of the GroupQueryAttention clarification
 *      gives its shape) takes bias[b, h, i, j + d_b] for the key at row j
 *      after an eviction of d_b rows, i.e. its column is the key's position
 *      in past ++ new. With a bias the split-KV decode (S = 1, fp16/bf16,
 *      D = 128 or 64) and the MFMA prefill (fp16/bf16, D = 128 or 64, bias_total a
 *      multiple of 4, bias 8-byte aligned) keep their kernels; other calls
 *      use the plain kernel.
 *
 * Ownership and threading: every pointer except *_host arguments is device
 * memory owned by the caller. The library never allocates, frees or
 * synchronises; all work is enqueued on `stream` (a hipStream_t, NULL =
 * the null stream) and the call returns before it completes. The library
 * keeps no state between calls except the error-message buffer, which is
 * thread-local.
 *
 * Alignment: q, k_new, v_new, out and the caches (and a separate past) must
 * start at a multiple of 16 bytes (the kernels move 16-byte units; torch
 * allocations are 256-byte aligned); otherwise GQA_ERR_INVALID_ARG.
 *
 * Errors: every argument is validated before the first launch, so any
 * status other than GQA_OK and GQA_ERR_HIP guarantees that nothing was
 * enqueued and both caches are untouched. GQA_ERR_HIP means a launch
 * failed; cache contents are then undefined and the workspace must be
 * zero-filled again before reuse. gqa_last_error() returns a message for
 * the most recent failing call on this thread.
 *
 * seqlens_k_host and seqlens_k_dev must hold the same values (the host copy
 * validates and sizes the launch; kernels read the device copy). If they
 * differ the results are undefined, but every access stays inside the
 * buffers whose sizes the shape implies.
 */
#ifndef GQA_H
#define GQA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum gqa_status {
  GQA_OK = 0,
  GQA_ERR_NO_ROOM = 1,      /* some L_b + S > M with the window off */
  GQA_ERR_INVALID_ARG = 2,  /* bad shape, option, pointer or length */
  GQA_ERR_UNSUPPORTED = 3,  /* valid but not served: gqa_attention_decode_noalloc on a device
                               beyond the ones its static scratch covers */
  GQA_ERR_WORKSPACE = 4,    /* workspace missing or smaller than needed */
  GQA_ERR_HIP = 5           /* a HIP launch failed */
} gqa_status;

typedef enum gqa_dtype { GQA_FP32 = 0, GQA_FP16 = 1, GQA_BF16 = 2 } gqa_dtype;

typedef struct gqa_shape {
  int32_t batch;         /* B >= 0 (0: nothing to do) */
  int32_t new_tokens;    /* S >= 1 for attention, >= 0 for append */
  int32_t num_heads;     /* H >= 1 */
  int32_t kv_num_heads;  /* Hkv >= 1, H % Hkv == 0 */
  int32_t head_size;     /* 1 <= D <= 256 (even with rotary) */
  int32_t max_seq_len;   /* M >= 1: buffer rows per (b, kv head) */
  int32_t dtype;         /* gqa_dtype */
} gqa_shape;

typedef struct gqa_options {
  float scale;                 /* 0 -> 1/sqrt(D); otherwise finite */
  int32_t local_window_size;   /* -1: off; otherwise 1 <= W <= M */
  const float* cos_cache;      /* NULL: no rotary; else [rotary_rows, D/2] */
  const float* sin_cache;      /* given together with cos_cache */
  int32_t rotary_rows;         /* rows in the tables; need L_b + S <= rows */
  int32_t rotary_interleaved;  /* 0: rotate-half pairs; 1: adjacent pairs */
  int32_t greedy_eviction;     /* 0: on overflow keep the min(L_b + S, M) most
                                  recent tokens (every step of a full cache
                                  moves it); 1: needs a window W; on overflow
                                  keep only min(L_b, max(0, W - S)) past rows,
                                  so the buffer then holds the W most recent
                                  tokens and the next M - W steps append
                                  without moving anything */
  const void* attention_bias;  /* NULL: none; else device [bias_batch,
                                  bias_heads, S, bias_total] in the dtype,
                                  added to scale * q.k before the softmax */
  int32_t bias_batch;          /* B, or 1 to share one bias across sequences */
  int32_t bias_heads;          /* H, or 1 to share one bias across heads */
  int32_t bias_total;          /* T >= max_b (L_b + S): column j is the key at
                                  position j of past ++ new (before any
                                  eviction of this call) */
  const int32_t* position_offset_host;  /* NULL: 0 for every sequence; else
                                  [B] host: absolute position of sequence b's
                                  buffer row 0 (>= 0); rotary positions are
                                  offset_b + L_b + i, and offset_b + L_b + S
                                  <= rotary_rows. A caller keeping a rolling
                                  window adds each call's dropped count
                                  (L_b + S - new length) to offset_b */
  const int32_t* position_offset_dev;   /* the same values on the device;
                                  given together with the host copy */
} gqa_options;

/*
 * Bytes of workspace the attention and eviction entry points need for this
 * shape and options (opts may be NULL: no window), for any seqlens_k (an
 * upper bound over all lengths 0..M). With a window and S > 1 it includes
 * two staging frames of B * Hkv * (M + S) rows (see gqa_attention_prefill).
 * The workspace must be zero-filled before its first use; each successful
 * call leaves it reusable (its counters return to zero). 0 means none is
 * needed. A call whose local_window_size is -1 may use a workspace sized
 * with any window.
 */
size_t gqa_workspace_bytes(const gqa_shape* shape, const gqa_options* opts);

/*
 * Append half (steps 1 and 3 for K/V only): rotary on k_new when tables are
 * given, then the in-place scatter at L_b. No eviction: any L_b + S > M
 * returns GQA_ERR_NO_ROOM, window or not. opts->scale and the window are
 * ignored. Source: pad+scatter pull request, paragraph 2; shared-buffer
 * question and answer of the GroupQueryAttention clarification.
 */
gqa_status gqa_append_kv(const gqa_shape* shape, const gqa_options* opts,
                         const void* k_new, const void* v_new,
                         void* k_cache, void* v_cache,
                         const int32_t* seqlens_k_host, const int32_t* seqlens_k_dev,
                         void* stream);

/*
 * The whole op for S >= 1 new tokens per sequence (steps 1-4): fused
 * flash-style attention on MFMA for fp16/bf16 with D = 128 or 64, a plain
 * kernel otherwise. When the shape has too few 256-row blocks to fill the
 * GPU, each block's key range is split over several workgroups whose
 * partials (kept in the workspace) the last one merges by log-sum-exp.
 * With a window, S > 1 and an eviction needed by some sequence, queries
 * early in the chunk see keys the eviction drops: attention then runs over
 * each sequence before its eviction (past ++ new, positions L_b + i): the
 * new rows, and the past rows from the 64-key tile holding L_b on, go to
 * staging frames in the workspace, from which the MFMA kernel reads those
 * tiles while it reads earlier tiles from the cache (the plain kernel
 * reads every row the window reaches from the frames); the cache then
 * takes the eviction and the append. Source:
 * all three pages as summarised above; the key-tile loop ends at each
 * sequence's length ("KV Cache", notes and short-term plan); the window
 * keeps the most recent tokens contiguously (sliding-window follow-up of
 * the GroupQueryAttention clarification).
 */
gqa_status gqa_attention_prefill(const gqa_shape* shape, const gqa_options* opts,
                                 const void* q, const void* k_new, const void* v_new,
                                 void* k_cache, void* v_cache,
                                 const int32_t* seqlens_k_host, const int32_t* seqlens_k_dev,
                                 void* out, void* workspace, size_t workspace_bytes,
                                 void* stream);

/*
 * The whole op for exactly one new token per sequence (S must be 1):
 * split-KV attention (fp16/bf16, D = 128 or 64, one launch per 64 sequences; the
 * plain kernel otherwise). The valid 16-key blocks of all (sequence, kv head) units form
 * one list cut into equal slices, one per wave; each wave streams its slice
 * once, with the new token's append fused, and a unit cut between
 * workgroups is merged by log-sum-exp by the last of them to finish. With a
 * window and L_b = M it evicts instead of failing (one row, or with
 * greedy_eviction down to W - 1 rows). Source: as for prefill; decoding
 * phase of the "KV Cache" worked example.
 */
gqa_status gqa_attention_decode(const gqa_shape* shape, const gqa_options* opts,
                                const void* q, const void* k_new, const void* v_new,
                                void* k_cache, void* v_cache,
                                const int32_t* seqlens_k_host, const int32_t* seqlens_k_dev,
                                void* out, void* workspace, size_t workspace_bytes,
                                void* stream);

/*
 * The whole op with separate past and present buffers: past_key/past_value
 * [B, Hkv, past_rows, D] hold sequence b's first L_b rows (L_b <= past_rows)
 * and are only read; present_key/present_value [B, Hkv, M, D] (M =
 * shape->max_seq_len) receive past rows [0, L_b) at the same rows, then the
 * call proceeds exactly as gqa_attention_prefill on the present buffers
 * (any S >= 1; one token per sequence takes the split-KV decode). When the
 * split-KV decode reads every row [0, L_b) (S = 1, fp16/bf16, D = 128 or
 * 64, nothing evicted, the window off or reaching row 0) it moves the past
 * rows itself as it reads them, with no separate copy; the result is the
 * same. Present rows [L_b + S, M) are not written, past is never written;
 * afterwards the
 * present buffers can serve as a shared buffer for the next call.
 * Passing the same K and V buffers as past and present (with past_rows = M)
 * is the shared mode and copies nothing; any other overlap of past and
 * present is undefined. L_b + S > M fails with GQA_ERR_NO_ROOM (window off),
 * L_b > past_rows with GQA_ERR_INVALID_ARG, both before any launch.
 * Workspace: gqa_workspace_bytes of the present shape. Source: question of
 * the GroupQueryAttention clarification (past of length
 * past_sequence_length unless it is the present tensor) and its summary
 * (with different shapes, present is past + new in a different tensor).
 */
gqa_status gqa_attention_present(const gqa_shape* shape, const gqa_options* opts,
                                 const void* q, const void* k_new, const void* v_new,
                                 const void* past_key, const void* past_value, int32_t past_rows,
                                 void* present_key, void* present_value,
                                 const int32_t* seqlens_k_host, const int32_t* seqlens_k_dev,
                                 void* out, void* workspace, size_t workspace_bytes,
                                 void* stream);

/*
 * Eviction half (step 2 alone): make room for `incoming` tokens
 * (0 <= incoming <= M) in every sequence by dropping its oldest
 * d_b = max(0, L_b + incoming - M) rows and shifting the rest to row 0, in
 * place. Writes seqlens_after_host[b] = min(L_b, M - incoming) (host
 * memory, B entries) before returning; updating the device copy of the
 * lengths is the caller's job. Uses shape->batch, kv_num_heads, head_size,
 * max_seq_len and dtype only. Source: sliding-window follow-up of the
 * GroupQueryAttention clarification (keep the most recent tokens,
 * contiguously; each step's eviction costs a copy of the cache).
 */
gqa_status gqa_evict_window(const gqa_shape* shape, int32_t incoming,
                            void* k_cache, void* v_cache,
                            const int32_t* seqlens_k_host, const int32_t* seqlens_k_dev,
                            int32_t* seqlens_after_host,
                            void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of the static device scratch behind gqa_attention_decode_noalloc
 * (one copy per GPU the library runs on, held until the process ends). */
#define GQA_NOALLOC_SCRATCH_BYTES (64u << 20)

/*
 * gqa_attention_decode without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation). Same arguments, semantics, errors and
 * kernels as gqa_attention_decode; the workspace is a static device array of
 * GQA_NOALLOC_SCRATCH_BYTES on the current device, and nothing is allocated
 * or freed. A call whose workspace (gqa_workspace_bytes of the shape, plus
 * 64 KiB of merge counters) does not fit returns GQA_ERR_WORKSPACE before any
 * launch: the decode workloads of up to 64 sequences with 8 KV heads and
 * 4096-row fp16/bf16 buffers fit. Every call on one GPU shares that GPU's
 * array, which keeps the last call's contents: calls that overlap in time on
 * one GPU (two streams, two host threads) race and give undefined results.
 * The first call on a device, and the first after a GQA_ERR_HIP, zeroes the
 * array's counter area with a small kernel on `stream`. The split-KV
 * decode takes its work plan and past lengths from seqlens_k_host when the
 * call is made; under graph capture that is when it is captured, so a
 * replay is valid only for the captured lengths (with seqlens_k_dev holding
 * the same values).
 */
gqa_status gqa_attention_decode_noalloc(const gqa_shape* shape, const gqa_options* opts,
                                        const void* q, const void* k_new, const void* v_new,
                                        void* k_cache, void* v_cache,
                                        const int32_t* seqlens_k_host,
                                        const int32_t* seqlens_k_dev, void* out, void* stream);

/*
 * A plain streaming read of `bytes` bytes at `src` (device memory, 16-byte
 * aligned; bytes a positive multiple of 16), enqueued on `stream`. Not part
 * of the operation: the yardstick the memory-bound kernels are measured
 * against (the benchmark times it on buffers of the split-KV decode's byte
 * count that are not cache-resident). It reads the buffer once, with the
 * split-KV decode's launch shape (one workgroup of eight waves per CU, each
 * wave a contiguous slice, 16-byte loads, four in flight per lane), and
 * writes nothing the caller reads. Errors: GQA_ERR_INVALID_ARG before any
 * launch; GQA_ERR_HIP if the launch fails.
 */
gqa_status gqa_stream_read(const void* src, size_t bytes, void* stream);

/* Static description of a status code. */
const char* gqa_status_string(gqa_status status);

/* Message for the most recent failing call on this thread ("" if none). */
const char* gqa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* GQA_H */
