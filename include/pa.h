/*
 * pa.h -- paged attention over a block-table KV cache, for AMD Instinct
 * MI355X (gfx950).  C ABI of libpa.so.
 *
 * What is computed.  The pages this library follows name the pieces but not
 * the formulas: paged attention whose block table and sequence lengths stay
 * device tensors handed to the kernels (vllm-metal architecture article,
 * sections 三 and 四), prefix caching and chunked prefill (vllm-metis 0.1.0,
 * intro and "How the model maps onto vLLM"), GQA 4:1 (vllm-metis 0.1.0,
 * "Status") and FP8 with one scale of amax / 448 (same section).  Each call
 * below computes, for every query row, the plain definition
 *
 *     out = softmax(scale * q . K^T) V
 *
 * over the keys the row may see, with q-head j reading kv-head j / G
 * (G = num_q_heads / num_kv_heads, contiguous groups).
 *
 * Memory layouts (row-major, contiguous, all device memory):
 *   q, out (decode)    [num_seqs, num_q_heads, head_dim]
 *   q, out (prefill)   [total_q,  num_q_heads, head_dim]
 *   k_cache            [num_blocks, n, num_kv_heads, head_dim / X, 16, X], n = block_size
 *                      / 16, X the dims in 16 bytes (4 fp32, 8 bf16, 16 fp8): a block is
 *                      n consecutive 16-token sub-blocks, and each (sub-block, kv-head)
 *                      tile is a run of 16-byte chunks of consecutive dims, with the
 *                      token index inside each chunk.  Token slot s of a block is slot
 *                      s % 16 of sub-block s / 16; with 16-token blocks (n = 1) this is
 *                      [num_blocks, num_kv_heads, head_dim / X, 16, X].
 *   v_cache            [num_blocks, n, num_kv_heads, head_dim, 16]  (dim-major tiles)
 *                      The pages leave the cache layout to the platform (vllm-metal
 *                      architecture article, section 二).  These two differ from plain
 *                      token-major rows [num_blocks, num_kv_heads, block_size, head_dim]
 *                      on purpose: the score product contracts over dims, and with the
 *                      chunked K tile one load instruction of a wave reads 1 KiB in one
 *                      piece (16 half-lines with token-major rows; the bf16 Llama-3-8B
 *                      decode went from 58% to 67% of peak bandwidth with the change);
 *                      the output product contracts over tokens, which the dim-major V
 *                      tile serves with whole dim rows.  Splitting 32- and 64-token
 *                      blocks into 16-token sub-blocks keeps every V load a whole run of
 *                      16-token rows (with [.., head_dim, block_size] V tiles a load
 *                      covered 32-byte slices of 64- or 128-byte rows: 64-token blocks
 *                      measured 61% of peak bandwidth, 74% with sub-blocks).  The cache
 *                      of num_blocks blocks is byte for byte a cache of num_blocks * n
 *                      16-token blocks; slot numbers (block * block_size + offset) are
 *                      the same in both readings.
 *   block_table        int32 [num_seqs, max_blocks_per_seq]; logical token t of
 *                      sequence b lives in physical block block_table[b][t / block_size]
 *                      at slot t % block_size
 *   seq_lens           int32 [num_seqs]; tokens whose K/V are in the cache,
 *                      including the current decode token or the whole chunk
 *   k_scale, v_scale   fp32 [num_kv_heads] (fp8 KV only; NULL otherwise):
 *                      K value = e4m3fn(code) * k_scale[kv_head], likewise V
 *   partial_out        fp32 [num_seqs, num_q_heads, max_partitions, head_dim]
 *   partial_lse        fp32 [num_seqs, num_q_heads, max_partitions], natural log
 *
 * Supported: head_dim 64 or 128; block_size 16, 32 or 64 (vllm-mblt 0.8.0,
 * "Chunked Prefill Auto-Tuning": a 64-token block size as an override of the
 * default); num_q_heads a multiple of num_kv_heads with G <= 16; dtypes (q, kv) = (F32, F32), (BF16, BF16) or
 * (BF16, FP8_E4M3); out has q's dtype; q, out, k_cache, v_cache 16-byte
 * aligned.
 *
 * Ownership and execution.  The caller owns every buffer passed in.  Every
 * call only validates its scalar arguments and pointer alignment on the host
 * and enqueues kernels on `stream` (a hipStream_t; NULL = the default
 * stream).  It never reads device memory from the host, never synchronises
 * and never allocates, so calls can be captured in a HIP graph (the kernels
 * join the caller's step with no sync boundary, as the vllm-metal
 * architecture article, section 三, asks of its native kernels).  Host
 * state, kept per device for the life of the process: the number of
 * workgroups of the balanced decode mode the device holds at once (one
 * occupancy query on the first balanced call) and the address of
 * pa_decode_noalloc's fixed buffer (looked up on its first call).  Make
 * those first calls outside graph capture.  Results are reproducible: the
 * same arguments and device data give the same output bits on the same
 * device, call after call (every floating-point sum has a fixed order; the
 * only atomics are integer counts in LDS).  Table entries at or past
 * ceil(seq_len / block_size) and cache slots past seq_len are never read
 * (they may hold anything, NaN included).
 *
 * Errors.  A non-zero pa_status is returned before anything is enqueued when
 * the arguments are invalid.  A call with nothing to do (num_seqs == 0,
 * num_chunks == 0 or max_q_len == 0, num_tokens == 0) validates its sizes,
 * launches nothing and accepts NULL for its arrays.  PA_ERR_HIP reports a
 * failed launch (including a library built without a gfx950 code object).
 * There is no fallback path.
 * Block-table contents are not checked: an entry outside [0, num_blocks) or
 * a seq_len above max_blocks_per_seq * block_size is undefined behaviour.
 */
#ifndef PA_H
#define PA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    PA_F32 = 0,
    PA_BF16 = 1,
    PA_FP8_E4M3 = 2   /* OCP e4m3fn (largest finite 448), KV cache only */
} pa_dtype;

typedef enum {
    PA_OK = 0,
    PA_ERR_NULL = 1,         /* a required pointer is NULL */
    PA_ERR_SHAPE = 2,        /* a size is negative, inconsistent or too large */
    PA_ERR_DTYPE = 3,        /* unknown dtype or unsupported (q, kv) pair */
    PA_ERR_ALIGN = 4,        /* a tensor pointer is not 16-byte aligned */
    PA_ERR_UNSUPPORTED = 5,  /* head_dim, block_size, G or partition size not supported */
    PA_ERR_WORKSPACE = 6,    /* workspace missing or smaller than required */
    PA_ERR_HIP = 7           /* the HIP runtime rejected a launch */
} pa_status;

/* partition_size value selecting the balanced split-KV mode of pa_decode and
 * pa_decode_multi_query (see pa_decode). */
#define PA_PARTITION_BALANCED (-1)

/* Stages of pa_decode_stages. */
#define PA_STAGE_ATTENTION 1  /* the attention kernel (partials, or direct rows) */
#define PA_STAGE_MERGE 2      /* the log-sum-exp merge of the partials */
#define PA_STAGE_ALL 3

/* Human-readable name of a status code (static storage; never NULL). */
const char* pa_status_string(int status);

/* Library version as major*10000 + minor*100 + patch. */
int pa_version(void);

/*
 * Bytes of workspace pa_decode needs: 0 when partition_size == 0; for
 * partition_size > 0 room for fp32 partials [num_seqs, num_q_heads, P_max,
 * head_dim] and their lse [num_seqs, num_q_heads, P_max], P_max =
 * ceil(max_seq_len / partition_size); for PA_PARTITION_BALANCED room for
 * num_seqs piece records (2 int32) and the partials of up to
 * 1024 + num_seqs pieces of num_q_heads rows each.  Each region is 256-byte
 * aligned.  Returns 0 for invalid arguments and for sizes the decode calls
 * refuse (num_seqs * num_q_heads above 2^31 - 1, more than 65535 partitions).
 */
size_t pa_decode_workspace_size(int num_seqs, int num_q_heads, int head_dim,
                                int max_seq_len, int partition_size);

/*
 * Decode attention: one query per sequence (the newest token, already in the
 * cache) attends to keys 0 .. seq_lens[b]-1.  The pages name this step: the
 * native paged-attention kernel driven by block tables and sequence lengths
 * that stay device tensors (vllm-metal architecture article, sections 三
 * and 四), with GQA 4:1 and FP8 KV at scale amax / 448 (vllm-metis 0.1.0,
 * "Status"); the split of long contexts into partitions merged by their
 * log-sum-exp is this library's (the pages give no rule for it).
 *
 * partition_size == 0: one pass per (sequence, kv-head), out written
 * directly.  With at least 1024 (sequence, kv-head) pairs and at most 1024
 * sequences the workgroups take the sequences longest first (each
 * workgroup finds its sequence from seq_lens on the device), so the grid
 * does not end on a tail of long sequences; results are unchanged.
 *
 * partition_size > 0 (a multiple of 16 tokens): split-KV; each
 * partition p covers tokens [p*P, min((p+1)*P, L)) and writes its normalised
 * output and lse into `workspace`, then the log-sum-exp merge (the kernel of
 * pa_merge_partitions) writes out.  A sequence that fits in one partition
 * is written directly by the partition kernel (bit-identical to merging its
 * single partition).  When max_seq_len spans at least 16 partitions and a
 * partition is a multiple of 64 tokens (bf16 and fp8 KV), the partitions
 * are streamed: each workgroup takes a run of consecutive partitions, the
 * runs balanced over the batch and the device's resident workgroups, and
 * its loads run on across partition boundaries; every partition's result
 * is bit-identical to the one-workgroup-per-partition kernel's, so this
 * changes time, not results.  A workspace serves one call at a time.
 *
 * partition_size == PA_PARTITION_BALANCED: the blocks of all sequences, laid
 * end to end per kv-head, are cut into equal ranges, one per workgroup, with
 * as many workgroups as the device holds at once (measured once per device
 * with the runtime's occupancy query); a range covering parts of
 * several sequences yields one partial per part, and the merge combines each
 * sequence's parts.  Every workgroup then streams the same number of bytes
 * whatever the mix of lengths.  Results equal the other modes up to the
 * rounding of the merge.  The mode pays when lengths vary widely or there
 * are fewer (sequence, kv-head) pairs than resident workgroups; each
 * sequence a range covers costs it a table load and a first-block load in
 * series, so for large batches of short sequences (hundreds to thousands
 * of sequences of a few hundred tokens) the one-pass mode is faster.
 * Batch invariance: where a sequence's pieces begin depends on the whole
 * batch's blocks and on the device's occupancy, so in the balanced mode a
 * sequence's output bits can change with its batch-mates and with the GPU
 * model (within the merge's rounding: one bf16 step).  The one-pass mode and
 * fixed partitions are batch-invariant bit for bit: a sequence's result
 * depends only on its own inputs (the pages name batch-dependent outputs as
 * a limitation of per-batch FP8 scales: vllm-metis 0.1.0, "Limitations").
 * max_seq_len is the caller's host-side
 * bound on seq_lens; it sizes the grid.  A sequence of length 0 gets zeros.
 * scale is the softmax scale (1/sqrt(head_dim) for plain attention); it
 * must be finite and > 0 (PA_ERR_SHAPE otherwise), and so must every fp8
 * k_scale / v_scale entry (not checked: device data).
 */
int pa_decode(void* out, const void* q, int q_dtype,
              const void* k_cache, const void* v_cache, int kv_dtype,
              const int32_t* block_table, int max_blocks_per_seq,
              const int32_t* seq_lens, int num_seqs,
              int num_q_heads, int num_kv_heads, int head_dim, int block_size,
              int num_blocks, float scale, const float* k_scale, const float* v_scale,
              int partition_size, int max_seq_len,
              void* workspace, size_t workspace_bytes, void* stream);

/*
 * pa_decode for callers that cannot allocate device memory (code under HIP
 * graph capture, serving loops and harnesses that forbid hipMalloc): the
 * same arguments and results as pa_decode, without `workspace`, whose role a
 * fixed buffer inside the library takes: PA_STATIC_WORKSPACE_BYTES of device
 * memory per GPU, part of the library's code object, held by each GPU the
 * library runs on until the process ends.  The call allocates nothing.
 * Returns PA_ERR_WORKSPACE, before enqueuing anything, when
 * pa_decode_workspace_size(num_seqs, num_q_heads, head_dim, max_seq_len,
 * partition_size) exceeds the buffer (for 32 q-heads of 128 dims: the
 * balanced mode up to about 3000 sequences; 512-token partitions up to
 * 15 sequences of 128K tokens).  Every call on one GPU uses that GPU's one
 * buffer, which keeps the last call's contents (nothing in it needs to start
 * at zero): calls ordered on one stream are fine, calls that may overlap on
 * one GPU (other streams, other threads) race and give wrong results.  The
 * buffer's address is looked up on the first call with each device current
 * (make that call, like the balanced mode's first call, outside capture).
 */
#define PA_STATIC_WORKSPACE_BYTES ((size_t)64 << 20)

int pa_decode_noalloc(void* out, const void* q, int q_dtype,
                      const void* k_cache, const void* v_cache, int kv_dtype,
                      const int32_t* block_table, int max_blocks_per_seq,
                      const int32_t* seq_lens, int num_seqs,
                      int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                      int num_blocks, float scale, const float* k_scale, const float* v_scale,
                      int partition_size, int max_seq_len, void* stream);

/*
 * Multi-query decode: each sequence has q_len queries, the newest q_len
 * tokens already in its cache, as when drafted tokens are verified in one
 * step (speculative decoding: in vllm-mblt 0.8.0, "Serve an EAGLE-3 Model",
 * the base model verifies each round's drafted tokens).  Query i of
 * sequence b sits at position L - q_len + i
 * (L = seq_lens[b]) and attends to keys 0 .. L - q_len + i: the causal mask
 * of a prefill chunk whose context is L - q_len.
 *
 * q, out  [num_seqs, q_len, num_q_heads, head_dim] (out in q's dtype).
 * q_len = 1 is pa_decode.  With q_len * G <= 16 the (query, head) pairs share
 * one pass over each sequence's K/V (the decode kernel, split-KV and merge as
 * in pa_decode); the workspace is then
 * pa_decode_workspace_size(num_seqs, q_len * num_q_heads, head_dim,
 * max_seq_len, partition_size) bytes.  With q_len * G > 16 the prefill-chunk
 * kernel runs each sequence as one chunk (partition_size and workspace are
 * ignored).  A sequence with seq_len 0 gets zero rows; 0 < seq_len < q_len
 * breaks the contract (its rows are unspecified).
 */
int pa_decode_multi_query(void* out, const void* q, int q_dtype, int q_len,
                          const void* k_cache, const void* v_cache, int kv_dtype,
                          const int32_t* block_table, int max_blocks_per_seq,
                          const int32_t* seq_lens, int num_seqs,
                          int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                          int num_blocks, float scale, const float* k_scale,
                          const float* v_scale, int partition_size, int max_seq_len,
                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * pa_decode_multi_query (q_len = 1: pa_decode) split into its two stages:
 * `stages` is a mask of PA_STAGE_ATTENTION and PA_STAGE_MERGE.  Running the
 * attention stage, then (on the same stream, with the same arguments and
 * workspace) the merge stage equals one PA_STAGE_ALL call; other work, or
 * timing events, may go between the two.  Only the decode kernel's packings
 * (q_len * G <= 16) are accepted.  One-pass calls (partition_size 0) have no
 * merge: their merge stage does nothing.
 */
int pa_decode_stages(void* out, const void* q, int q_dtype, int q_len,
                     const void* k_cache, const void* v_cache, int kv_dtype,
                     const int32_t* block_table, int max_blocks_per_seq,
                     const int32_t* seq_lens, int num_seqs,
                     int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                     int num_blocks, float scale, const float* k_scale,
                     const float* v_scale, int partition_size, int max_seq_len,
                     void* workspace, size_t workspace_bytes, int stages, void* stream);

/*
 * Decode with a shared prefix (cascade): every sequence's cache is the same
 * prefix_len-token prefix (whole blocks, listed once in prefix_block_table)
 * followed by its own tokens (block_table / seq_lens describe only those:
 * seq_lens[b] tokens after the prefix, the current token(s) included).  The
 * result equals pa_decode_multi_query over the concatenated sequence (prefix
 * caching shares such blocks: vllm-metis 0.1.0, "How the model maps onto
 * vLLM"), but the prefix is read once for the whole batch instead of once per
 * sequence: (1) all queries against the prefix, split into key ranges, give
 * partial results; (2) each sequence's own tokens, split into partitions of
 * partition_size (> 0) tokens; (3) the log-sum-exp merge of both.
 * q, out [num_seqs, q_len, num_q_heads, head_dim] (q_len * G <= 16; q_len 1
 * is plain decode); workspace of at least
 * pa_decode_shared_prefix_workspace_size(...) bytes (0 for invalid arguments
 * and sizes the call refuses).  prefix_len 0 is pa_decode_multi_query in one
 * pass.
 */
size_t pa_decode_shared_prefix_workspace_size(int num_seqs, int q_len, int num_q_heads,
                                              int num_kv_heads, int head_dim, int prefix_len,
                                              int max_seq_len, int partition_size);

int pa_decode_shared_prefix(void* out, const void* q, int q_dtype, int q_len,
                            const void* k_cache, const void* v_cache, int kv_dtype,
                            const int32_t* prefix_block_table, int prefix_len,
                            const int32_t* block_table, int max_blocks_per_seq,
                            const int32_t* seq_lens, int num_seqs,
                            int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                            int num_blocks, float scale, const float* k_scale,
                            const float* v_scale, int partition_size, int max_seq_len,
                            void* workspace, size_t workspace_bytes, void* stream);

/*
 * Split-KV decode, partition kernel only: writes partial_out / partial_lse
 * for every partition of every sequence (partitions past ceil(L / P) are not
 * written and must not be read; pa_merge_partitions ignores them).
 * max_partitions is the P_max dimension of the partial arrays and must be at
 * least ceil(max_seq_len / partition_size).  partition_size > 0.
 */
int pa_decode_partitions(float* partial_out, float* partial_lse, int max_partitions,
                         const void* q, int q_dtype,
                         const void* k_cache, const void* v_cache, int kv_dtype,
                         const int32_t* block_table, int max_blocks_per_seq,
                         const int32_t* seq_lens, int num_seqs,
                         int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                         int num_blocks, float scale, const float* k_scale,
                         const float* v_scale, int partition_size, int max_seq_len,
                         void* stream);

/*
 * Log-sum-exp merge of split-KV partials (the standard combination of
 * softmax pieces over disjoint key sets; the pages give no merge rule, and
 * the exactness of the combination is what the oracle's split = unsplit pin
 * checks).  For sequence b only partitions
 * p < ceil(seq_lens[b] / partition_size) take part:
 *     M = max_p lse_p,  w_p = exp(lse_p - M),
 *     out = sum_p w_p o_p / sum_p w_p,  out_lse = M + ln sum_p w_p.
 * A sequence with no partition gets out = 0 and out_lse = -inf.
 * out_dtype is PA_F32 or PA_BF16 (round to nearest even); out_lse may be NULL.
 */
int pa_merge_partitions(void* out, int out_dtype, float* out_lse,
                        const float* partial_out, const float* partial_lse,
                        const int32_t* seq_lens, int partition_size, int max_partitions,
                        int num_seqs, int num_q_heads, int head_dim, void* stream);

/*
 * Causal chunked prefill over a paged context: chunked prefill and prefix
 * caching are how the pages' serving engine runs long prompts (vllm-metis
 * 0.1.0, "How the model maps onto vLLM"; its "Status" reports parity with
 * 64-token chunks and prefix-cache hits).  Chunk c owns query rows
 * cu_q_lens[c] .. cu_q_lens[c+1]-1 of `q`; its sequence has seq_lens[c]
 * tokens in the cache (the context followed by the chunk itself), so with
 * ctx = seq_lens[c] - q_len_c, query i of the chunk sits at position ctx + i
 * and attends to keys 0 .. ctx + i (the causal mask aligned to the
 * bottom-right of the score matrix).  Several block-table rows may reference
 * the same physical blocks (a shared prefix).  max_q_len is the host-side
 * bound on every chunk's length; it sizes the grid.  out_lse (fp32
 * [total_q, num_q_heads], natural log) may be NULL.  A chunk whose seq_len is
 * below its q_len has no context for its rows: they get zeros (lse -inf).
 */
int pa_prefill_chunk(void* out, float* out_lse, const void* q, int q_dtype,
                     const int32_t* cu_q_lens, int total_q, int max_q_len,
                     const void* k_cache, const void* v_cache, int kv_dtype,
                     const int32_t* block_table, int max_blocks_per_seq,
                     const int32_t* seq_lens, int num_chunks,
                     int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                     int num_blocks, float scale, const float* k_scale,
                     const float* v_scale, void* stream);

/*
 * One mixed serving step: decode rows and prefill chunks over one KV cache,
 * the way the pages' engine runs chunked prefill beside decoding sequences
 * (vllm-metis 0.1.0, "How the model maps onto vLLM").  The result is that of
 * pa_decode on the decode part (dec_*, num_seqs, max_seq_len,
 * partition_size, workspace: as there) followed by pa_prefill_chunk on the
 * chunk part (pre_*, cu_q_lens, total_q, max_q_len, num_chunks: as there),
 * bit for bit; the shared arguments (dtypes, caches, head counts, head_dim,
 * block size, pool size, scale, fp8 scales) describe both.  When the decode
 * rows need a split-KV merge, it runs inside the chunks' launch (the
 * workgroups of the first half of the chunks' row tiles merge their share of
 * the decode rows after their own rows) instead of as a launch of its own:
 * two launches per step instead of three (a merge over 32 or more fixed
 * partitions, which takes a workgroup per row, keeps its own launch).  Every argument of both parts is validated
 * before anything is enqueued; either part may be empty (num_seqs == 0, or
 * num_chunks == 0 / max_q_len == 0).  The workspace must not overlap any
 * output.
 */
int pa_mixed_step(void* dec_out, const void* dec_q, const int32_t* dec_block_table,
                  int dec_max_blocks_per_seq, const int32_t* dec_seq_lens, int num_seqs,
                  int max_seq_len, int partition_size, void* workspace, size_t workspace_bytes,
                  void* pre_out, float* pre_out_lse, const void* pre_q,
                  const int32_t* cu_q_lens, int total_q, int max_q_len,
                  const int32_t* pre_block_table, int pre_max_blocks_per_seq,
                  const int32_t* pre_seq_lens, int num_chunks,
                  int q_dtype, const void* k_cache, const void* v_cache, int kv_dtype,
                  int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                  int num_blocks, float scale, const float* k_scale, const float* v_scale,
                  void* stream);

/*
 * Cache write: store the K/V rows of num_tokens new tokens into their cache
 * slots, the step that precedes attention in every decode step and prefill
 * chunk (the cache is addressed by (block, offset) through block tables:
 * vllm-metal architecture article, section 四; FP8 with one scale of
 * amax / 448: vllm-metis 0.1.0, "Status").
 *
 * key, value       rows of token t at key + t * key_stride elements, laid out
 *                  [num_kv_heads, head_dim] (contiguous inside a row); a stride
 *                  above num_kv_heads * head_dim lets K and V be views into a
 *                  fused projection output.  in_dtype PA_F32 or PA_BF16;
 *                  16-byte aligned, and stride * element size a multiple of 16.
 * slot_mapping     int32 [num_tokens]: token t goes to physical block
 *                  slot / block_size, offset slot % block_size.  A negative
 *                  slot marks a padding token and is skipped; so is a slot at
 *                  or beyond num_blocks * block_size (no write lands outside
 *                  the caches).  Two tokens mapped to one slot race.
 * k_cache, v_cache the layouts above, kv_dtype equal to in_dtype (an exact
 *                  copy) or PA_FP8_E4M3.  An fp8 cache receives
 *                  e4m3fn(x / scale[kv_head]): the fp32 value of the input
 *                  divided by the fp32 scale (correctly rounded), clamped to
 *                  [-448, 448], rounded to the nearest code, ties to the even
 *                  code.  Inputs must be finite (a NaN gives an unspecified
 *                  code); k_scale and v_scale must be finite and > 0.
 * Slots not named by slot_mapping are left untouched.  With num_tokens == 0
 * nothing is launched, and key, value and slot_mapping may be NULL.
 * Cost: a whole 16-token group written into one block moves its rows at
 * copy speed; a single new token per sequence (a decode step) writes each
 * V element into its own dim row of the dim-major tile, so the memory
 * system writes whole 32-byte sectors for 2-byte elements (measured: about
 * 9x the row bytes for a 64-sequence bf16 decode step, 2.4 MB for 0.26 MB;
 * small beside the step's attention reads).
 */
int pa_write_kv(void* k_cache, void* v_cache, int kv_dtype,
                const void* key, const void* value, int in_dtype,
                int key_stride, int value_stride,
                const int32_t* slot_mapping, int num_tokens,
                int num_kv_heads, int head_dim, int block_size, int num_blocks,
                const float* k_scale, const float* v_scale, void* stream);

/*
 * A measurement aid, not a step of attention: reads the `bytes` bytes at buf
 * once, front to back, and XORs the buffer's 32-bit words (little-endian)
 * into the sink.  Timed over a buffer much larger than the device's caches it
 * gives the measured HBM read rate beside which the attention kernels'
 * live-K/V rates are reported.  nontemporal != 0 reads with the non-temporal
 * loads the attention kernels use for K and V, 0 with plain loads.
 * buf: device memory, 16-byte aligned, bytes a multiple of 16 (PA_ERR_ALIGN,
 * PA_ERR_SHAPE).  sink: PA_STREAM_READ_SINK_WORDS device uint32 words,
 * 4-byte aligned; each workgroup XORs its share into a word of its own, so
 * the XOR of all the words changes by the buffer's XOR (zero the sink first
 * to read the buffer's XOR off it).  Calls that overlap on one sink race.
 * bytes == 0 launches nothing and accepts NULL for buf.  Enqueued on stream;
 * the call does not wait.
 */
#define PA_STREAM_READ_SINK_WORDS 2048

int pa_stream_read(const void* buf, size_t bytes, int nontemporal, uint32_t* sink,
                   void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PA_H */
