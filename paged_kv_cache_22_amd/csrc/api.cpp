// C-ABI front end of libpa.so: argument validation and dispatch.  Host code
// only; it never touches device memory, never synchronises and never
// allocates.  Every check runs before the first launch, so a rejected call
// enqueues nothing.  The contract is documented in include/pa.h.
#include "../../include/pa.h"

#include <cmath>
#include <cstdint>

#include "launch.h"

namespace {

constexpr int kUnit = 16;             // tokens per kernel unit; partitions are whole units

bool block_size_ok(int bs) { return bs == 16 || bs == 32 || bs == 64; }
constexpr int kMaxGroup = 16;          // q-heads per kv-head handled by one wave
constexpr int kMaxGridY = 65535;
constexpr size_t kRegionAlign = 256;


bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

int dtype_ok(int q_dtype, int kv_dtype) {
    if (q_dtype < PA_F32 || q_dtype > PA_BF16) return PA_ERR_DTYPE;
    if (kv_dtype < PA_F32 || kv_dtype > PA_FP8_E4M3) return PA_ERR_DTYPE;
    const bool ok = (q_dtype == PA_F32 && kv_dtype == PA_F32) ||
                    (q_dtype == PA_BF16 && (kv_dtype == PA_BF16 || kv_dtype == PA_FP8_E4M3));
    return ok ? PA_OK : PA_ERR_DTYPE;
}

// checks shared by decode and prefill; `empty` = the call launches nothing,
// so its arrays may be empty (NULL)
int common_checks(const void* q, const void* k_cache, const void* v_cache, int q_dtype, int kv_dtype,
                  const int32_t* block_table, int max_blocks_per_seq, const int32_t* seq_lens,
                  int num_q_heads, int num_kv_heads, int head_dim, int block_size, int num_blocks,
                  float scale, const float* k_scale, const float* v_scale, bool empty) {
    if (!empty && (!q || !k_cache || !v_cache || !block_table || !seq_lens)) return PA_ERR_NULL;
    int st = dtype_ok(q_dtype, kv_dtype);
    if (st != PA_OK) return st;
    if (!empty && kv_dtype == PA_FP8_E4M3 && (!k_scale || !v_scale)) return PA_ERR_NULL;
    if (num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 ||
        num_blocks < 0 || max_blocks_per_seq <= 0)
        return PA_ERR_SHAPE;
    if (num_q_heads % num_kv_heads != 0) return PA_ERR_SHAPE;
    if (num_q_heads / num_kv_heads > kMaxGroup) return PA_ERR_UNSUPPORTED;
    if (head_dim != 64 && head_dim != 128) return PA_ERR_UNSUPPORTED;
    if (!block_size_ok(block_size)) return PA_ERR_UNSUPPORTED;
    if (!std::isfinite(scale) || !(scale > 0.0f)) return PA_ERR_SHAPE;
    if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache)) return PA_ERR_ALIGN;
    if ((reinterpret_cast<uintptr_t>(block_table) & 3u) || (reinterpret_cast<uintptr_t>(seq_lens) & 3u))
        return PA_ERR_ALIGN;
    return PA_OK;
}

int decode_checks(const void* q, int q_dtype, const void* k_cache, const void* v_cache, int kv_dtype,
                  const int32_t* block_table, int max_blocks_per_seq, const int32_t* seq_lens,
                  int num_seqs, int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                  int num_blocks, float scale, const float* k_scale, const float* v_scale,
                  int partition_size, int max_seq_len) {
    int st = common_checks(q, k_cache, v_cache, q_dtype, kv_dtype, block_table, max_blocks_per_seq,
                           seq_lens, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                           scale, k_scale, v_scale, num_seqs == 0);
    if (st != PA_OK) return st;
    if (num_seqs < 0 || max_seq_len < 0) return PA_ERR_SHAPE;
    if ((long long)num_seqs * num_kv_heads > 0x7fffffffLL) return PA_ERR_SHAPE;
    if ((long long)max_seq_len > (long long)max_blocks_per_seq * block_size) return PA_ERR_SHAPE;
    if (partition_size < 0 && partition_size != PA_PARTITION_BALANCED) return PA_ERR_SHAPE;
    if (partition_size > 0 && partition_size % kUnit != 0) return PA_ERR_UNSUPPORTED;
    if (partition_size > 0) {
        const long long parts = ((long long)max_seq_len + partition_size - 1) / partition_size;
        if (parts > kMaxGridY) return PA_ERR_UNSUPPORTED;
    }
    return PA_OK;
}

pa::DecodeArgs make_decode_args(const void* q, int q_dtype, const void* k_cache, const void* v_cache,
                                int kv_dtype, const int32_t* block_table, int max_blocks_per_seq,
                                const int32_t* seq_lens, int num_seqs, int num_q_heads,
                                int num_kv_heads, int head_dim, int block_size, float scale,
                                const float* k_scale, const float* v_scale) {
    pa::DecodeArgs a{};
    a.block_size = block_size;
    a.q = q;
    a.q_dtype = q_dtype;
    a.k_cache = k_cache;
    a.v_cache = v_cache;
    a.kv_dtype = kv_dtype;
    a.block_table = block_table;
    a.max_blocks_per_seq = max_blocks_per_seq;
    a.seq_lens = seq_lens;
    a.num_seqs = num_seqs;
    a.num_q_heads = num_q_heads;
    a.num_kv_heads = num_kv_heads;
    a.head_dim = head_dim;
    a.scale = scale;
    a.q_len = 1;
    a.k_scale = kv_dtype == PA_FP8_E4M3 ? k_scale : nullptr;
    a.v_scale = kv_dtype == PA_FP8_E4M3 ? v_scale : nullptr;
    return a;
}

int hip_status(int e) { return e == 0 ? PA_OK : PA_ERR_HIP; }

// Key ranges of the shared-prefix pass: enough (row group, kv-head, range)
// workgroups to cover the chip (kPrefixWGs), each range at least 32 tokens
#ifndef PA_PREFIX_WGS
#define PA_PREFIX_WGS 256
#endif
constexpr int kPrefixWGs = PA_PREFIX_WGS;

// tokens per key range (a multiple of 32): about kPrefixWGs / (row groups x
// kv-heads) ranges over the prefix
long long prefix_key_range(int num_seqs, int q_len, int num_q_heads, int num_kv_heads,
                           int prefix_len) {
    const long long rows = (long long)num_seqs * q_len * (num_q_heads / num_kv_heads);
    const long long groups = (rows + 127) / 128 * num_kv_heads;   // 128 rows per workgroup
    long long want = groups > 0 ? (kPrefixWGs + groups - 1) / groups : 1;
    if (want < 1) want = 1;
    const long long per = ((long long)prefix_len + want - 1) / want;
    return (per + 31) / 32 * 32;
}

// the ranges that key range actually makes (every one holds keys)
int prefix_ranges(int num_seqs, int q_len, int num_q_heads, int num_kv_heads, int prefix_len) {
    if (prefix_len <= 0) return 0;
    const long long kr = prefix_key_range(num_seqs, q_len, num_q_heads, num_kv_heads, prefix_len);
    return (int)(((long long)prefix_len + kr - 1) / kr);
}

}  // namespace

extern "C" {

const char* pa_status_string(int status) {
    switch (status) {
        case PA_OK: return "PA_OK";
        case PA_ERR_NULL: return "PA_ERR_NULL: a required pointer is NULL";
        case PA_ERR_SHAPE: return "PA_ERR_SHAPE: a size is negative, inconsistent or too large";
        case PA_ERR_DTYPE: return "PA_ERR_DTYPE: unknown or unsupported dtype combination";
        case PA_ERR_ALIGN: return "PA_ERR_ALIGN: a tensor pointer is not 16-byte aligned";
        case PA_ERR_UNSUPPORTED:
            return "PA_ERR_UNSUPPORTED: head_dim, block_size, group size or partition size not supported";
        case PA_ERR_WORKSPACE: return "PA_ERR_WORKSPACE: workspace missing or too small";
        case PA_ERR_HIP: return "PA_ERR_HIP: the HIP runtime rejected a launch";
        default: return "PA_ERR_UNKNOWN";
    }
}

int pa_version(void) { return 100; }

size_t pa_decode_workspace_size(int num_seqs, int num_q_heads, int head_dim, int max_seq_len,
                                int partition_size) {
    if (num_seqs < 0 || num_q_heads <= 0 || head_dim <= 0 || max_seq_len < 0) return 0;
    // sizes the calls themselves refuse have no workspace size
    if ((long long)num_seqs * num_q_heads > 0x7fffffffLL) return 0;
    if (partition_size > 0 && ((long long)max_seq_len + partition_size - 1) / partition_size > kMaxGridY)
        return 0;
    if (partition_size == PA_PARTITION_BALANCED) {
        // piece records | partial outputs | partial lse, for up to
        // kMaxBalancedSplits splits per kv-head
        const size_t slots = (size_t)pa::kMaxBalancedSplits + num_seqs;
        return round_up((size_t)num_seqs * 2 * sizeof(int32_t), kRegionAlign) +
               round_up(slots * num_q_heads * head_dim * sizeof(float), kRegionAlign) +
               round_up(slots * num_q_heads * sizeof(float), kRegionAlign);
    }
    if (partition_size <= 0) return 0;
    const size_t parts = ((size_t)max_seq_len + partition_size - 1) / partition_size;
    const size_t rows = (size_t)num_seqs * num_q_heads * parts;
    return round_up(rows * head_dim * sizeof(float), kRegionAlign) +
           round_up(rows * sizeof(float), kRegionAlign);
}

int pa_decode_partitions(float* partial_out, float* partial_lse, int max_partitions, const void* q,
                         int q_dtype, const void* k_cache, const void* v_cache, int kv_dtype,
                         const int32_t* block_table, int max_blocks_per_seq, const int32_t* seq_lens,
                         int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                         int block_size, int num_blocks, float scale, const float* k_scale,
                         const float* v_scale, int partition_size, int max_seq_len, void* stream) {
    int st = decode_checks(q, q_dtype, k_cache, v_cache, kv_dtype, block_table, max_blocks_per_seq,
                           seq_lens, num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                           num_blocks, scale, k_scale, v_scale, partition_size, max_seq_len);
    if (st != PA_OK) return st;
    if (partition_size <= 0) return PA_ERR_UNSUPPORTED;
    if (num_seqs > 0 && (!partial_out || !partial_lse)) return PA_ERR_NULL;
    if (!aligned16(partial_out) || (reinterpret_cast<uintptr_t>(partial_lse) & 3u)) return PA_ERR_ALIGN;
    const int parts = (int)(((long long)max_seq_len + partition_size - 1) / partition_size);
    if (max_partitions < parts) return PA_ERR_SHAPE;
    if (num_seqs == 0 || parts == 0) return PA_OK;
    pa::DecodeArgs a = make_decode_args(q, q_dtype, k_cache, v_cache, kv_dtype, block_table,
                                        max_blocks_per_seq, seq_lens, num_seqs, num_q_heads,
                                        num_kv_heads, head_dim, block_size, scale, k_scale, v_scale);
    a.part_out = partial_out;
    a.part_lse = partial_lse;
    a.max_parts = max_partitions;
    a.partition_blocks = partition_size / kUnit;
    a.grid_parts = parts;
    return hip_status(pa::launch_decode(a, stream));
}

int pa_merge_partitions(void* out, int out_dtype, float* out_lse, const float* partial_out,
                        const float* partial_lse, const int32_t* seq_lens, int partition_size,
                        int max_partitions, int num_seqs, int num_q_heads, int head_dim, void* stream) {
    if (num_seqs != 0 && (!out || !partial_out || !partial_lse || !seq_lens)) return PA_ERR_NULL;
    if (out_dtype != PA_F32 && out_dtype != PA_BF16) return PA_ERR_DTYPE;
    if (num_seqs < 0 || num_q_heads <= 0 || max_partitions < 0 || partition_size <= 0)
        return PA_ERR_SHAPE;
    if ((long long)num_seqs * num_q_heads > 0x7fffffffLL) return PA_ERR_SHAPE;
    if (head_dim != 64 && head_dim != 128) return PA_ERR_UNSUPPORTED;
    if (!aligned16(out) || !aligned16(partial_out) || (reinterpret_cast<uintptr_t>(partial_lse) & 3u) ||
        (reinterpret_cast<uintptr_t>(seq_lens) & 3u) || (reinterpret_cast<uintptr_t>(out_lse) & 3u))
        return PA_ERR_ALIGN;
    if (num_seqs == 0) return PA_OK;
    pa::MergeArgs m{};
    m.out = out;
    m.out_dtype = out_dtype;
    m.out_lse = out_lse;
    m.part_out = partial_out;
    m.part_lse = partial_lse;
    m.seq_lens = seq_lens;
    m.partition_size = partition_size;
    m.max_parts = max_partitions;
    m.num_seqs = num_seqs;
    m.num_q_heads = num_q_heads;
    m.head_dim = head_dim;
    return hip_status(pa::launch_merge(m, stream));
}

}  // extern "C"

namespace {

// pa_decode and pa_decode_multi_query with q_len * G <= 16: the decode kernel
// (columns = (query, head) pairs), split-KV partials merged when P > 0
int decode_impl(void* out, const void* q, int q_dtype, int q_len, const void* k_cache,
                const void* v_cache, int kv_dtype, const int32_t* block_table,
                int max_blocks_per_seq, const int32_t* seq_lens, int num_seqs, int num_q_heads,
                int num_kv_heads, int head_dim, int block_size, float scale, const float* k_scale,
                const float* v_scale, int partition_size, int max_seq_len, void* workspace,
                size_t workspace_bytes, void* stream, int stages = PA_STAGE_ALL,
                pa::MergeArgs* deferred = nullptr) {
    // deferred: the merge is not launched but described there (its out left
    // NULL when none is due), for a later launch to run
    const bool run_attn = stages & PA_STAGE_ATTENTION, run_merge = stages & PA_STAGE_MERGE;
    const int rows_per_seq = q_len * num_q_heads;   // output rows of one sequence
    pa::DecodeArgs a = make_decode_args(q, q_dtype, k_cache, v_cache, kv_dtype, block_table,
                                        max_blocks_per_seq, seq_lens, num_seqs, num_q_heads,
                                        num_kv_heads, head_dim, block_size, scale, k_scale, v_scale);
    a.q_len = q_len;
    if (partition_size == 0) {
        if (num_seqs == 0) return PA_OK;
        a.out = out;
        a.partition_blocks = 0;
        a.grid_parts = 1;
        return run_attn ? hip_status(pa::launch_decode(a, stream)) : PA_OK;
    }
    const size_t need = pa_decode_workspace_size(num_seqs, rows_per_seq, head_dim, max_seq_len,
                                                 partition_size);
    if (num_seqs > 0 && need > 0 && (!workspace || workspace_bytes < need)) return PA_ERR_WORKSPACE;
    if (workspace && (reinterpret_cast<uintptr_t>(workspace) & (kRegionAlign - 1))) return PA_ERR_ALIGN;
    if (num_seqs == 0) return PA_OK;
    if (partition_size == PA_PARTITION_BALANCED) {
        // workspace: piece records | partial outputs | partial lse
        const int splits = pa::balanced_splits(a);
        if (splits < 1) return PA_ERR_HIP;
        const size_t slots = (size_t)splits + num_seqs;
        char* ws = reinterpret_cast<char*>(workspace);
        const size_t off_out = round_up((size_t)num_seqs * 2 * sizeof(int32_t), kRegionAlign);
        const size_t off_lse = off_out + round_up(slots * rows_per_seq * head_dim * sizeof(float), kRegionAlign);
        a.out = out;
        a.piece_info = ws;
        a.part_out = reinterpret_cast<float*>(ws + off_out);
        a.part_lse = reinterpret_cast<float*>(ws + off_lse);
        a.balanced = 1;
        a.grid_parts = splits;
        int st = run_attn ? hip_status(pa::launch_decode(a, stream)) : PA_OK;
        if (st != PA_OK || !run_merge) return st;
        pa::MergeArgs m{};
        m.out = out;
        m.out_dtype = q_dtype;
        m.part_out = a.part_out;
        m.part_lse = a.part_lse;
        m.seq_lens = seq_lens;
        m.partition_size = 1;
        m.num_seqs = num_seqs;
        m.num_q_heads = rows_per_seq;
        m.head_dim = head_dim;
        m.skip_single = 1;
        m.piece_info = ws;
        m.piece_slots = (int)slots;
        m.q_len = q_len;
        m.num_kv_heads = num_kv_heads;
        if (deferred) {
            *deferred = m;
            return PA_OK;
        }
        return hip_status(pa::launch_merge(m, stream));
    }
    const int parts = (int)(((long long)max_seq_len + partition_size - 1) / partition_size);
    if (parts == 0) {  // every sequence is empty: the one-pass kernel writes the zeros
        a.out = out;
        a.partition_blocks = 0;
        a.grid_parts = 1;
        return run_attn ? hip_status(pa::launch_decode(a, stream)) : PA_OK;
    }
    // workspace: partial outputs | partial lse
    const size_t rows = (size_t)num_seqs * rows_per_seq * parts;
    char* ws = reinterpret_cast<char*>(workspace);
    const size_t off_lse = round_up(rows * head_dim * sizeof(float), kRegionAlign);
    a.out = out;
    a.part_out = reinterpret_cast<float*>(ws);
    a.part_lse = reinterpret_cast<float*>(ws + off_lse);
    a.single_direct = 1;
    a.max_parts = parts;
    a.partition_blocks = partition_size / kUnit;
    a.grid_parts = parts;
    int st = run_attn ? hip_status(pa::launch_decode(a, stream)) : PA_OK;
    if (st != PA_OK || !run_merge) return st;
    pa::MergeArgs m{};
    m.out = out;
    m.out_dtype = q_dtype;
    m.out_lse = nullptr;
    m.part_out = a.part_out;
    m.part_lse = a.part_lse;
    m.seq_lens = seq_lens;
    m.partition_size = partition_size;
    m.max_parts = parts;
    m.num_seqs = num_seqs;
    m.num_q_heads = rows_per_seq;
    m.head_dim = head_dim;
    m.skip_single = 1;
    if (deferred) {
        *deferred = m;
        return PA_OK;
    }
    return hip_status(pa::launch_merge(m, stream));
}

// pa_prefill_chunk's checks and kernel arguments; *empty: nothing to launch
int prefill_prepare(void* out, float* out_lse, const void* q, int q_dtype, const int32_t* cu_q_lens,
                    int total_q, int max_q_len, const void* k_cache, const void* v_cache,
                    int kv_dtype, const int32_t* block_table, int max_blocks_per_seq,
                    const int32_t* seq_lens, int num_chunks, int num_q_heads, int num_kv_heads,
                    int head_dim, int block_size, int num_blocks, float scale,
                    const float* k_scale, const float* v_scale, pa::PrefillArgs& a, bool* empty) {
    *empty = num_chunks == 0 || max_q_len == 0;
    int st = common_checks(q, k_cache, v_cache, q_dtype, kv_dtype, block_table, max_blocks_per_seq,
                           seq_lens, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                           scale, k_scale, v_scale, *empty);
    if (st != PA_OK) return st;
    if (!*empty && (!out || !cu_q_lens)) return PA_ERR_NULL;
    if (!aligned16(out) || (reinterpret_cast<uintptr_t>(cu_q_lens) & 3u) ||
        (reinterpret_cast<uintptr_t>(out_lse) & 3u))
        return PA_ERR_ALIGN;
    if (num_chunks < 0 || total_q < 0 || max_q_len < 0) return PA_ERR_SHAPE;
    if ((long long)num_chunks * num_kv_heads > 0x7fffffffLL) return PA_ERR_SHAPE;
    const long long groups = ((long long)max_q_len * (num_q_heads / num_kv_heads) + 31) / 32;
    if (groups > kMaxGridY) return PA_ERR_UNSUPPORTED;
    a = pa::PrefillArgs{};
    a.out = out;
    a.out_lse = out_lse;
    a.q = q;
    a.cu_q_lens = cu_q_lens;
    a.total_q = total_q;
    a.max_q_len = max_q_len;
    a.k_cache = k_cache;
    a.v_cache = v_cache;
    a.block_table = block_table;
    a.seq_lens = seq_lens;
    a.k_scale = kv_dtype == PA_FP8_E4M3 ? k_scale : nullptr;
    a.v_scale = kv_dtype == PA_FP8_E4M3 ? v_scale : nullptr;
    a.q_dtype = q_dtype;
    a.kv_dtype = kv_dtype;
    a.num_chunks = num_chunks;
    a.num_q_heads = num_q_heads;
    a.num_kv_heads = num_kv_heads;
    a.head_dim = head_dim;
    a.block_size = block_size;
    a.max_blocks_per_seq = max_blocks_per_seq;
    a.scale = scale;
    return PA_OK;
}

}  // namespace

extern "C" {

int pa_decode(void* out, const void* q, int q_dtype, const void* k_cache, const void* v_cache,
              int kv_dtype, const int32_t* block_table, int max_blocks_per_seq,
              const int32_t* seq_lens, int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
              int block_size, int num_blocks, float scale, const float* k_scale,
              const float* v_scale, int partition_size, int max_seq_len, void* workspace,
              size_t workspace_bytes, void* stream) {
    int st = decode_checks(q, q_dtype, k_cache, v_cache, kv_dtype, block_table, max_blocks_per_seq,
                           seq_lens, num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                           num_blocks, scale, k_scale, v_scale, partition_size, max_seq_len);
    if (st != PA_OK) return st;
    if (num_seqs > 0 && !out) return PA_ERR_NULL;
    if (!aligned16(out)) return PA_ERR_ALIGN;
    return decode_impl(out, q, q_dtype, 1, k_cache, v_cache, kv_dtype, block_table,
                       max_blocks_per_seq, seq_lens, num_seqs, num_q_heads, num_kv_heads, head_dim,
                       block_size, scale, k_scale, v_scale, partition_size, max_seq_len, workspace,
                       workspace_bytes, stream);
}

static_assert(PA_STATIC_WORKSPACE_BYTES == pa::kStaticWorkspaceBytes,
              "pa.h and the library agree on the fixed workspace size");

int pa_decode_noalloc(void* out, const void* q, int q_dtype, const void* k_cache,
                      const void* v_cache, int kv_dtype, const int32_t* block_table,
                      int max_blocks_per_seq, const int32_t* seq_lens, int num_seqs,
                      int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                      int num_blocks, float scale, const float* k_scale, const float* v_scale,
                      int partition_size, int max_seq_len, void* stream) {
    int st = decode_checks(q, q_dtype, k_cache, v_cache, kv_dtype, block_table, max_blocks_per_seq,
                           seq_lens, num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                           num_blocks, scale, k_scale, v_scale, partition_size, max_seq_len);
    if (st != PA_OK) return st;
    if (num_seqs > 0 && !out) return PA_ERR_NULL;
    if (!aligned16(out)) return PA_ERR_ALIGN;
    const size_t need = pa_decode_workspace_size(num_seqs, num_q_heads, head_dim, max_seq_len,
                                                 partition_size);
    if (need > PA_STATIC_WORKSPACE_BYTES) return PA_ERR_WORKSPACE;
    void* ws = nullptr;
    size_t ws_bytes = 0;
    if (num_seqs > 0 && need > 0 && pa::static_workspace(&ws, &ws_bytes) != 0) return PA_ERR_HIP;
    return decode_impl(out, q, q_dtype, 1, k_cache, v_cache, kv_dtype, block_table,
                       max_blocks_per_seq, seq_lens, num_seqs, num_q_heads, num_kv_heads, head_dim,
                       block_size, scale, k_scale, v_scale, partition_size, max_seq_len, ws,
                       ws_bytes, stream);
}

int pa_decode_multi_query(void* out, const void* q, int q_dtype, int q_len, const void* k_cache,
                          const void* v_cache, int kv_dtype, const int32_t* block_table,
                          int max_blocks_per_seq, const int32_t* seq_lens, int num_seqs,
                          int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                          int num_blocks, float scale, const float* k_scale, const float* v_scale,
                          int partition_size, int max_seq_len, void* workspace,
                          size_t workspace_bytes, void* stream) {
    if (q_len <= 0) return PA_ERR_SHAPE;
    int st = decode_checks(q, q_dtype, k_cache, v_cache, kv_dtype, block_table, max_blocks_per_seq,
                           seq_lens, num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                           num_blocks, scale, k_scale, v_scale, partition_size, max_seq_len);
    if (st != PA_OK) return st;
    if (num_seqs > 0 && !out) return PA_ERR_NULL;
    if (!aligned16(out)) return PA_ERR_ALIGN;
    if ((long long)num_seqs * q_len * num_q_heads > 0x7fffffffLL) return PA_ERR_SHAPE;
    const int G = num_q_heads / num_kv_heads;
    if ((long long)q_len * G <= kMaxGroup)
        return decode_impl(out, q, q_dtype, q_len, k_cache, v_cache, kv_dtype, block_table,
                           max_blocks_per_seq, seq_lens, num_seqs, num_q_heads, num_kv_heads,
                           head_dim, block_size, scale, k_scale, v_scale, partition_size, max_seq_len,
                           workspace, workspace_bytes, stream);
    // more (query, head) pairs than MFMA columns: the prefill kernel, each
    // sequence a chunk of q_len rows (no partitions, no workspace)
    if (((long long)q_len * G + 127) / 128 > kMaxGridY) return PA_ERR_UNSUPPORTED;
    if (num_seqs == 0) return PA_OK;
    pa::PrefillArgs a{};
    a.out = out;
    a.out_lse = nullptr;
    a.q = q;
    a.cu_q_lens = nullptr;
    a.uniform_q_len = q_len;
    a.total_q = num_seqs * q_len;
    a.max_q_len = q_len;
    a.k_cache = k_cache;
    a.v_cache = v_cache;
    a.block_table = block_table;
    a.seq_lens = seq_lens;
    a.k_scale = kv_dtype == PA_FP8_E4M3 ? k_scale : nullptr;
    a.v_scale = kv_dtype == PA_FP8_E4M3 ? v_scale : nullptr;
    a.q_dtype = q_dtype;
    a.kv_dtype = kv_dtype;
    a.num_chunks = num_seqs;
    a.num_q_heads = num_q_heads;
    a.num_kv_heads = num_kv_heads;
    a.head_dim = head_dim;
    a.block_size = block_size;
    a.max_blocks_per_seq = max_blocks_per_seq;
    a.scale = scale;
    return hip_status(pa::launch_prefill(a, stream));
}

int pa_decode_stages(void* out, const void* q, int q_dtype, int q_len, const void* k_cache,
                     const void* v_cache, int kv_dtype, const int32_t* block_table,
                     int max_blocks_per_seq, const int32_t* seq_lens, int num_seqs, int num_q_heads,
                     int num_kv_heads, int head_dim, int block_size, int num_blocks, float scale,
                     const float* k_scale, const float* v_scale, int partition_size,
                     int max_seq_len, void* workspace, size_t workspace_bytes, int stages,
                     void* stream) {
    if (q_len <= 0) return PA_ERR_SHAPE;
    if (stages < 1 || stages > PA_STAGE_ALL) return PA_ERR_SHAPE;
    int st = decode_checks(q, q_dtype, k_cache, v_cache, kv_dtype, block_table, max_blocks_per_seq,
                           seq_lens, num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                           num_blocks, scale, k_scale, v_scale, partition_size, max_seq_len);
    if (st != PA_OK) return st;
    if (num_seqs > 0 && !out) return PA_ERR_NULL;
    if (!aligned16(out)) return PA_ERR_ALIGN;
    if ((long long)num_seqs * q_len * num_q_heads > 0x7fffffffLL) return PA_ERR_SHAPE;
    if ((long long)q_len * (num_q_heads / num_kv_heads) > kMaxGroup) return PA_ERR_UNSUPPORTED;
    return decode_impl(out, q, q_dtype, q_len, k_cache, v_cache, kv_dtype, block_table,
                       max_blocks_per_seq, seq_lens, num_seqs, num_q_heads, num_kv_heads, head_dim,
                       block_size, scale, k_scale, v_scale, partition_size, max_seq_len, workspace,
                       workspace_bytes, stream, stages);
}

size_t pa_decode_shared_prefix_workspace_size(int num_seqs, int q_len, int num_q_heads,
                                              int num_kv_heads, int head_dim, int prefix_len,
                                              int max_seq_len, int partition_size) {
    if (num_seqs < 0 || q_len <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
        prefix_len < 0 || max_seq_len < 0 || partition_size <= 0)
        return 0;
    // sizes the call itself refuses have no workspace size
    if (num_q_heads % num_kv_heads != 0) return 0;
    if ((long long)num_seqs * q_len > 0x7fffffffLL ||
        (long long)num_seqs * q_len * num_q_heads > 0x7fffffffLL)
        return 0;
    if (((long long)max_seq_len + partition_size - 1) / partition_size > kMaxGridY) return 0;
    const size_t slots = (size_t)prefix_ranges(num_seqs, q_len, num_q_heads, num_kv_heads, prefix_len) +
                         ((size_t)max_seq_len + partition_size - 1) / partition_size;
    const size_t rows = (size_t)num_seqs * q_len * num_q_heads * slots;
    return round_up(rows * head_dim * sizeof(float), kRegionAlign) +
           round_up(rows * sizeof(float), kRegionAlign);
}

int pa_decode_shared_prefix(void* out, const void* q, int q_dtype, int q_len, const void* k_cache,
                            const void* v_cache, int kv_dtype, const int32_t* prefix_block_table,
                            int prefix_len, const int32_t* block_table, int max_blocks_per_seq,
                            const int32_t* seq_lens, int num_seqs, int num_q_heads,
                            int num_kv_heads, int head_dim, int block_size, int num_blocks,
                            float scale, const float* k_scale, const float* v_scale,
                            int partition_size, int max_seq_len, void* workspace,
                            size_t workspace_bytes, void* stream) {
    if (q_len <= 0 || prefix_len < 0 || prefix_len > 0x7fffffff - 64) return PA_ERR_SHAPE;
    if (partition_size <= 0) return PA_ERR_UNSUPPORTED;
    int st = decode_checks(q, q_dtype, k_cache, v_cache, kv_dtype, block_table, max_blocks_per_seq,
                           seq_lens, num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                           num_blocks, scale, k_scale, v_scale, partition_size, max_seq_len);
    if (st != PA_OK) return st;
    if (prefix_len % block_size != 0) return PA_ERR_UNSUPPORTED;  // the prefix is whole blocks
    if (prefix_len > 0 && num_seqs > 0 && !prefix_block_table) return PA_ERR_NULL;
    if (reinterpret_cast<uintptr_t>(prefix_block_table) & 3u) return PA_ERR_ALIGN;
    if (num_seqs > 0 && !out) return PA_ERR_NULL;
    if (!aligned16(out)) return PA_ERR_ALIGN;
    const int G = num_q_heads / num_kv_heads;
    if ((long long)q_len * G > kMaxGroup) return PA_ERR_UNSUPPORTED;
    if ((long long)num_seqs * q_len * num_q_heads > 0x7fffffffLL) return PA_ERR_SHAPE;
    const size_t need = pa_decode_shared_prefix_workspace_size(
        num_seqs, q_len, num_q_heads, num_kv_heads, head_dim, prefix_len, max_seq_len, partition_size);
    if (num_seqs > 0 && (!workspace || workspace_bytes < need)) return PA_ERR_WORKSPACE;
    if (workspace && (reinterpret_cast<uintptr_t>(workspace) & (kRegionAlign - 1))) return PA_ERR_ALIGN;
    if (num_seqs == 0) return PA_OK;
    if (prefix_len == 0)
        return decode_impl(out, q, q_dtype, q_len, k_cache, v_cache, kv_dtype, block_table,
                           max_blocks_per_seq, seq_lens, num_seqs, num_q_heads, num_kv_heads,
                           head_dim, block_size, scale, k_scale, v_scale, 0, max_seq_len, nullptr, 0,
                           stream);

    const int ranges = prefix_ranges(num_seqs, q_len, num_q_heads, num_kv_heads, prefix_len);
    const int parts = (int)(((long long)max_seq_len + partition_size - 1) / partition_size);
    const int slots = ranges + parts;
    const size_t rows = (size_t)num_seqs * q_len * num_q_heads;
    char* ws = reinterpret_cast<char*>(workspace);
    float* part_out = reinterpret_cast<float*>(ws);
    float* part_lse = reinterpret_cast<float*>(ws + round_up(rows * slots * head_dim * sizeof(float), kRegionAlign));

    // 1. every query of the batch against the shared prefix, split into key ranges
    pa::PrefillArgs p{};
    p.q = q;
    p.q_dtype = q_dtype;
    p.uniform_q_len = num_seqs * q_len;     // one chunk: all queries, in (sequence, query) order
    p.total_q = num_seqs * q_len;
    p.max_q_len = num_seqs * q_len;
    p.num_chunks = 1;
    p.k_cache = k_cache;
    p.v_cache = v_cache;
    p.kv_dtype = kv_dtype;
    p.block_table = prefix_block_table;
    p.max_blocks_per_seq = prefix_len / block_size;
    p.k_scale = kv_dtype == PA_FP8_E4M3 ? k_scale : nullptr;
    p.v_scale = kv_dtype == PA_FP8_E4M3 ? v_scale : nullptr;
    p.num_q_heads = num_q_heads;
    p.num_kv_heads = num_kv_heads;
    p.head_dim = head_dim;
    p.block_size = block_size;
    p.scale = scale;
    p.kv_len = prefix_len;
    p.key_range = (int)prefix_key_range(num_seqs, q_len, num_q_heads, num_kv_heads, prefix_len);
    p.part_out = part_out;
    p.part_lse = part_lse;
    p.part_stride = slots;
    st = hip_status(pa::launch_prefill(p, stream));
    if (st != PA_OK) return st;

    // 2. each sequence's own tokens, split-KV partitions in the slots after the ranges
    pa::DecodeArgs a = make_decode_args(q, q_dtype, k_cache, v_cache, kv_dtype, block_table,
                                        max_blocks_per_seq, seq_lens, num_seqs, num_q_heads,
                                        num_kv_heads, head_dim, block_size, scale, k_scale, v_scale);
    a.q_len = q_len;
    if (parts > 0) {
        a.part_out = part_out;
        a.part_lse = part_lse;
        a.single_direct = 0;
        a.part_offset = ranges;
        a.max_parts = slots;
        a.partition_blocks = partition_size / kUnit;
        a.grid_parts = parts;
        st = hip_status(pa::launch_decode(a, stream));
        if (st != PA_OK) return st;
    }

    // 3. the log-sum-exp merge of prefix ranges and suffix partitions
    pa::MergeArgs m{};
    m.out = out;
    m.out_dtype = q_dtype;
    m.part_out = part_out;
    m.part_lse = part_lse;
    m.seq_lens = seq_lens;
    m.partition_size = partition_size;
    m.max_parts = slots;
    m.lead_slots = ranges;
    m.num_seqs = num_seqs;
    m.num_q_heads = q_len * num_q_heads;
    m.head_dim = head_dim;
    m.skip_single = 0;
    return hip_status(pa::launch_merge(m, stream));
}

int pa_prefill_chunk(void* out, float* out_lse, const void* q, int q_dtype, const int32_t* cu_q_lens,
                     int total_q, int max_q_len, const void* k_cache, const void* v_cache,
                     int kv_dtype, const int32_t* block_table, int max_blocks_per_seq,
                     const int32_t* seq_lens, int num_chunks, int num_q_heads, int num_kv_heads,
                     int head_dim, int block_size, int num_blocks, float scale, const float* k_scale,
                     const float* v_scale, void* stream) {
    pa::PrefillArgs a;
    bool empty;
    const int st = prefill_prepare(out, out_lse, q, q_dtype, cu_q_lens, total_q, max_q_len, k_cache,
                                   v_cache, kv_dtype, block_table, max_blocks_per_seq, seq_lens,
                                   num_chunks, num_q_heads, num_kv_heads, head_dim, block_size,
                                   num_blocks, scale, k_scale, v_scale, a, &empty);
    if (st != PA_OK || empty) return st;
    return hip_status(pa::launch_prefill(a, stream));
}

int pa_mixed_step(void* dec_out, const void* dec_q, const int32_t* dec_block_table,
                  int dec_max_blocks_per_seq, const int32_t* dec_seq_lens, int num_seqs,
                  int max_seq_len, int partition_size, void* workspace, size_t workspace_bytes,
                  void* pre_out, float* pre_out_lse, const void* pre_q, const int32_t* cu_q_lens,
                  int total_q, int max_q_len, const int32_t* pre_block_table,
                  int pre_max_blocks_per_seq, const int32_t* pre_seq_lens, int num_chunks,
                  int q_dtype, const void* k_cache, const void* v_cache, int kv_dtype,
                  int num_q_heads, int num_kv_heads, int head_dim, int block_size, int num_blocks,
                  float scale, const float* k_scale, const float* v_scale, void* stream) {
    // every argument of both parts is checked before anything is enqueued
    int st = decode_checks(dec_q, q_dtype, k_cache, v_cache, kv_dtype, dec_block_table,
                           dec_max_blocks_per_seq, dec_seq_lens, num_seqs, num_q_heads,
                           num_kv_heads, head_dim, block_size, num_blocks, scale, k_scale,
                           v_scale, partition_size, max_seq_len);
    if (st != PA_OK) return st;
    if (num_seqs > 0 && !dec_out) return PA_ERR_NULL;
    if (!aligned16(dec_out)) return PA_ERR_ALIGN;
    if ((long long)num_seqs * num_q_heads > 0x7fffffffLL) return PA_ERR_SHAPE;
    pa::PrefillArgs a;
    bool empty;
    st = prefill_prepare(pre_out, pre_out_lse, pre_q, q_dtype, cu_q_lens, total_q, max_q_len,
                         k_cache, v_cache, kv_dtype, pre_block_table, pre_max_blocks_per_seq,
                         pre_seq_lens, num_chunks, num_q_heads, num_kv_heads, head_dim, block_size,
                         num_blocks, scale, k_scale, v_scale, a, &empty);
    if (st != PA_OK) return st;
    // the decode rows' attention (the workspace is checked there, before any
    // launch); their merge, when one is due, goes into the chunks' launch
    // (or runs on its own when there are no chunks)
    pa::MergeArgs m{};
    st = decode_impl(dec_out, dec_q, q_dtype, 1, k_cache, v_cache, kv_dtype, dec_block_table,
                     dec_max_blocks_per_seq, dec_seq_lens, num_seqs, num_q_heads, num_kv_heads,
                     head_dim, block_size, scale, k_scale, v_scale, partition_size, max_seq_len,
                     workspace, workspace_bytes, stream, PA_STAGE_ALL, &m);
    if (st != PA_OK) return st;
    const bool merge_due = m.out != nullptr;
    if (merge_due && (empty || !pa::merge_fusable(m))) {
        // no chunks to carry it, or a merge of many partitions (a workgroup
        // per row): a launch of its own, as pa_decode makes it
        st = hip_status(pa::launch_merge(m, stream));
        if (st != PA_OK || empty) return st;
    } else if (merge_due) {
        a.merge = m;
        a.merge_rows = num_seqs * num_q_heads;
    }
    if (empty) return PA_OK;
    return hip_status(pa::launch_prefill(a, stream));
}

int pa_stream_read(const void* buf, size_t bytes, int nontemporal, uint32_t* sink,
                   void* stream) {
    if (!sink || (bytes > 0 && !buf)) return PA_ERR_NULL;
    if (bytes % 16) return PA_ERR_SHAPE;
    if (!aligned16(buf) || (reinterpret_cast<uintptr_t>(sink) & 3u)) return PA_ERR_ALIGN;
    if (bytes == 0) return PA_OK;
    return hip_status(pa::launch_stream_read(buf, bytes / 16, nontemporal ? 1 : 0, sink, stream));
}

int pa_write_kv(void* k_cache, void* v_cache, int kv_dtype, const void* key, const void* value,
                int in_dtype, int key_stride, int value_stride, const int32_t* slot_mapping,
                int num_tokens, int num_kv_heads, int head_dim, int block_size, int num_blocks,
                const float* k_scale, const float* v_scale, void* stream) {
    // with no tokens the per-token arrays may be empty (NULL)
    const bool none = num_tokens == 0;
    if (!k_cache || !v_cache || (!none && (!key || !value || !slot_mapping))) return PA_ERR_NULL;
    if (in_dtype != PA_F32 && in_dtype != PA_BF16) return PA_ERR_DTYPE;
    if (kv_dtype != PA_FP8_E4M3 && kv_dtype != in_dtype) return PA_ERR_DTYPE;
    if (kv_dtype == PA_FP8_E4M3 && (!k_scale || !v_scale)) return PA_ERR_NULL;
    if (num_tokens < 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 || num_blocks < 0)
        return PA_ERR_SHAPE;
    if (head_dim != 64 && head_dim != 128) return PA_ERR_UNSUPPORTED;
    if (!block_size_ok(block_size)) return PA_ERR_UNSUPPORTED;
    const long long row = (long long)num_kv_heads * head_dim;
    if (key_stride < row || value_stride < row) return PA_ERR_SHAPE;
    if ((long long)num_blocks * block_size > 0x7fffffffLL) return PA_ERR_SHAPE;
    const int in_bytes = in_dtype == PA_BF16 ? 2 : 4;
    if (((long long)key_stride * in_bytes) % 16 || ((long long)value_stride * in_bytes) % 16)
        return PA_ERR_ALIGN;
    if (!aligned16(k_cache) || !aligned16(v_cache) || !aligned16(key) || !aligned16(value) ||
        (reinterpret_cast<uintptr_t>(slot_mapping) & 3u))
        return PA_ERR_ALIGN;
    const int chunk = kv_dtype == PA_FP8_E4M3 ? 16 : kv_dtype == PA_BF16 ? 8 : 4;
    // one workgroup per (16 tokens, 16 chunk slots) at the least: the 1-D grid must fit
    if (((long long)num_tokens + 15) / 16 * (((long long)num_kv_heads * (head_dim / chunk) + 15) / 16) >
        0x7fffffffLL)
        return PA_ERR_SHAPE;
    if (num_tokens == 0) return PA_OK;
    pa::WriteArgs a{};
    a.k_cache = k_cache;
    a.v_cache = v_cache;
    a.key = key;
    a.value = value;
    a.slot_mapping = slot_mapping;
    a.k_scale = kv_dtype == PA_FP8_E4M3 ? k_scale : nullptr;
    a.v_scale = kv_dtype == PA_FP8_E4M3 ? v_scale : nullptr;
    a.key_stride = key_stride;
    a.value_stride = value_stride;
    a.in_dtype = in_dtype;
    a.kv_dtype = kv_dtype;
    a.num_tokens = num_tokens;
    a.num_kv_heads = num_kv_heads;
    a.head_dim = head_dim;
    a.num_blocks = num_blocks;
    a.block_size = block_size;
    return hip_status(pa::launch_write_kv(a, stream));
}

}  // extern "C"
