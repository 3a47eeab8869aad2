// Internal interface between the C-ABI front end (api.cpp, host only) and the
// kernel translation units.  Arguments arrive here already validated.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace pa {

struct DecodeArgs {
    // outputs: exactly one of (out) or (part_out, part_lse) is used
    void* out;            // [B, Hq, D] in q's dtype (one-pass mode)
    float* part_out;      // [B, Hq, max_parts, D]     (split mode)
    float* part_lse;      // [B, Hq, max_parts]
    int single_direct;    // split mode: a sequence with one partition writes `out`
                          // directly instead of a partial (the merge then skips it)
    int part_offset;      // split mode: partition p goes to partial slot p + part_offset
    int max_parts;
    const void* q;
    const void* k_cache;
    const void* v_cache;
    const int32_t* block_table;
    const int32_t* seq_lens;
    const float* k_scale;
    const float* v_scale;
    int q_dtype;          // pa_dtype
    int kv_dtype;         // pa_dtype
    int num_seqs, num_q_heads, num_kv_heads, head_dim;
    int block_size;       // tokens per cache block: 16, 32 or 64
    int q_len;            // queries per sequence (the newest q_len cached tokens), q_len * G <= 16
    int max_blocks_per_seq;
    int partition_blocks; // blocks per partition; 0 = whole sequence in one pass
    int grid_parts;       // partitions in the grid (1 in one-pass mode); balanced: splits per kv-head
    int balanced;         // balanced split-KV: grid (splits, kv-heads), partials by piece slot
    void* piece_info;     // balanced: int2 [num_seqs] = (first piece slot, piece count)
    int lpt_order;        // one-pass: workgroups take sequences longest first (set at launch)
    float scale;
};

struct MergeArgs {
    void* out;
    int out_dtype;
    float* out_lse;       // nullable
    const float* part_out;
    const float* part_lse;
    const int32_t* seq_lens;
    int partition_size, max_parts;
    int num_seqs, num_q_heads, head_dim;
    int skip_single;      // leave sequences with exactly one partition untouched
    int lead_slots;       // partition mode: partials 0 .. lead_slots-1 precede the
                          // sequence's partitions (a shared prefix's key ranges)
    // balanced split-KV pieces (instead of partition_size / max_parts):
    // partial row of (kv-head h, slot, column) = (h * piece_slots + slot) * cols + column
    const void* piece_info;  // int2 [num_seqs] = (first slot, count); NULL: partition mode
    int piece_slots;      // splits per kv-head + num_seqs
    int q_len;            // queries per sequence; num_q_heads then counts its q_len * heads rows
    int num_kv_heads;
};

struct PrefillArgs {
    void* out;
    float* out_lse;       // nullable
    const void* q;
    const int32_t* cu_q_lens;
    int total_q, max_q_len;
    const void* k_cache;
    const void* v_cache;
    const int32_t* block_table;
    const int32_t* seq_lens;
    const float* k_scale;
    const float* v_scale;
    int q_dtype, kv_dtype;
    int num_chunks, num_q_heads, num_kv_heads, head_dim;
    int block_size;       // tokens per cache block: 16, 32 or 64
    int uniform_q_len;    // > 0: chunk c owns rows c*uniform_q_len .. (cu_q_lens unused)
    // key-range mode (kv_len > 0): every row of chunk c sees keys
    // [z * key_range, min((z + 1) * key_range, kv_len)) of its table row,
    // z = blockIdx.z, with no causal mask (seq_lens unused)
    int kv_len, key_range;
    // partial output (part_out non-NULL): fp32 normalised rows and lse at
    // partial index row * part_stride + (kv_len > 0 ? z : 0), instead of out
    float* part_out;
    float* part_lse;
    int part_stride;
    int max_blocks_per_seq;
    float scale;
    // merge_rows > 0: after its own rows, the kernel merges rows 0 ..
    // merge_rows - 1 of a decode step's split-KV partials described by merge
    // (same head_dim and output dtype), one wave per row (a mixed step)
    int merge_rows;
    MergeArgs merge;
};

struct WriteArgs {
    void* k_cache;
    void* v_cache;
    const void* key;          // [num_tokens, token stride] rows, (kv-head, dim) inside
    const void* value;
    const int32_t* slot_mapping;
    const float* k_scale;     // fp8 cache only
    const float* v_scale;
    long long key_stride, value_stride;   // elements between consecutive tokens
    int in_dtype, kv_dtype;   // pa_dtype
    int num_tokens, num_kv_heads, head_dim, num_blocks;
    int block_size;           // tokens per cache block: 16, 32 or 64
};

// Upper bound of the balanced split-KV splits per kv-head.
constexpr int kMaxBalancedSplits = 1024;

// Balanced splits per kv-head for these arguments on the current device
// (occupancy of the balanced kernel x compute units / kv-heads, clamped to
// [1, kMaxBalancedSplits]); -1 if the runtime cannot tell.
int balanced_splits(const DecodeArgs& a);

// Bytes of the library's fixed device workspace (pa_decode_noalloc).
constexpr size_t kStaticWorkspaceBytes = (size_t)64 << 20;

// The current device's copy of that workspace: its device address and size.
// The address is looked up once per device (the first call with that device
// current) and cached.  Returns 0, or the hipError_t of the lookup.
int static_workspace(void** ptr, size_t* bytes);

// Each returns 0 on success or the hipError_t of a failed launch.
int launch_decode(const DecodeArgs& a, void* stream);
// the same for a.q_len > 1 (called by launch_decode / balanced_splits)
int launch_decode_mq(const DecodeArgs& a, void* stream);
int balanced_splits_mq(const DecodeArgs& a);
int launch_merge(const MergeArgs& a, void* stream);
int launch_prefill(const PrefillArgs& a, void* stream);
// whether launch_merge would merge a's rows with one wave per row (the form
// a prefill launch can run after its own rows, bit for bit the same)
bool merge_fusable(const MergeArgs& a);
int launch_write_kv(const WriteArgs& a, void* stream);
// XOR of n16 16-byte words at buf (folded to 32 bits) into *sink
int launch_stream_read(const void* buf, size_t n16, int nontemporal, unsigned* sink, void* stream);

}  // namespace pa
