// Host-only driver of the C-ABI front end (csrc/api.cpp) for the sanitizer
// test: built with g++ under AddressSanitizer and UndefinedBehaviorSanitizer
// together with api.cpp only.  The kernel launchers are replaced by stubs
// that write every byte of the workspace regions the real kernels would
// write, computed from the arguments they are handed, so a region carved
// past the end of a caller's workspace is an AddressSanitizer error, and
// any overflow in the host-side size arithmetic a UBSan error.  No GPU and
// no HIP runtime are involved.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "../include/pa.h"
#include "../paged_kv_cache_22_amd/csrc/launch.h"

namespace {
int g_launches = 0;
int g_splits = 96;                 // what the balanced mode's occupancy query "returns"
std::vector<unsigned char> g_static;

void touch(const void* p, size_t bytes) {
    if (p && bytes) std::memset(const_cast<void*>(p), 0x5A, bytes);
}
}  // namespace

namespace pa {
int balanced_splits(const DecodeArgs&) { return g_splits; }

int static_workspace(void** ptr, size_t* bytes) {
    if (g_static.empty()) g_static.resize(kStaticWorkspaceBytes);
    *ptr = g_static.data();
    *bytes = g_static.size();
    return 0;
}

int launch_decode(const DecodeArgs& a, void*) {
    ++g_launches;
    const size_t rows = (size_t)a.q_len * a.num_q_heads;   // output rows of one sequence
    if (a.balanced) {
        const size_t slots = (size_t)a.grid_parts + a.num_seqs;
        touch(a.piece_info, (size_t)a.num_seqs * 2 * sizeof(int32_t));
        touch(a.part_out, slots * rows * a.head_dim * sizeof(float));
        touch(a.part_lse, slots * rows * sizeof(float));
    } else if (a.partition_blocks > 0) {
        // partial (b, row, slot) for slots part_offset .. part_offset + grid_parts - 1
        const size_t n = (size_t)a.num_seqs * rows * a.max_parts;
        if (a.part_offset + a.grid_parts > a.max_parts) return 1;
        touch(a.part_out, n * a.head_dim * sizeof(float));
        touch(a.part_lse, n * sizeof(float));
    }
    return 0;
}

int launch_merge(const MergeArgs& a, void*) {
    ++g_launches;
    return a.num_seqs > 0 && a.num_q_heads > 0 ? 0 : 1;
}

bool merge_fusable(const MergeArgs& a) { return a.piece_info || a.max_parts < 32; }

int launch_prefill(const PrefillArgs& a, void*) {
    ++g_launches;
    // a mixed step's merge rows: every decode row, of the prefill's head_dim
    if (a.merge_rows > 0 && ((long long)a.merge.num_seqs * a.merge.num_q_heads != a.merge_rows ||
                             a.merge.head_dim != a.head_dim))
        return 1;
    if (a.part_out) {
        const size_t n = (size_t)a.total_q * a.num_q_heads * a.part_stride;
        touch(a.part_out, n * a.head_dim * sizeof(float));
        touch(a.part_lse, n * sizeof(float));
    }
    return 0;
}

int launch_write_kv(const WriteArgs&, void*) {
    ++g_launches;
    return 0;
}

int launch_stream_read(const void* buf, size_t n16, int, unsigned* sink, void*) {
    ++g_launches;
    // read every byte the kernel would read and every sink word it may write
    const unsigned char* b = static_cast<const unsigned char*>(buf);
    unsigned x = 0;
    for (size_t i = 0; i < n16 * 16; ++i) x ^= (unsigned)b[i] << (8 * (i & 3));
    for (int g = 1; g < PA_STREAM_READ_SINK_WORDS; ++g) sink[g] ^= 0u;
    sink[0] ^= x;
    return 0;
}
}  // namespace pa

namespace {
int g_fail = 0;

void expect(bool ok, const char* what, int line) {
    if (!ok) {
        std::printf("FAIL line %d: %s\n", line, what);
        ++g_fail;
    }
}
#define EXPECT(x) expect((x), #x, __LINE__)

// a fake device address: never dereferenced by api.cpp, 256-byte aligned
void* fake(uintptr_t i) { return reinterpret_cast<void*>((uintptr_t)0x100000 + 0x1000 * i); }
const int32_t* ifake(uintptr_t i) { return static_cast<const int32_t*>(fake(i)); }
const float* ffake(uintptr_t i) { return static_cast<const float*>(fake(i)); }

// a workspace of exactly `bytes`, 256-byte aligned at its start
struct Workspace {
    void* raw = nullptr;
    void* p = nullptr;
    explicit Workspace(size_t bytes) {
        if (posix_memalign(&raw, 256, bytes ? bytes : 1) != 0) std::abort();
        p = raw;
    }
    ~Workspace() { std::free(raw); }
};

int decode(int B, int Hq, int Hkv, int d, int bs, int P, int max_len, void* ws, size_t ws_bytes,
           int kv = PA_BF16) {
    const int mb = (int)(((long long)max_len + bs - 1) / bs + 1);
    return pa_decode(fake(1), fake(2), kv == PA_F32 ? PA_F32 : PA_BF16, fake(3), fake(4), kv,
                     ifake(5), mb, ifake(6), B, Hq, Hkv, d, bs, 100000, 0.088f,
                     kv == PA_FP8_E4M3 ? ffake(7) : nullptr, kv == PA_FP8_E4M3 ? ffake(8) : nullptr,
                     P, max_len, ws, ws_bytes, nullptr);
}
}  // namespace

int main() {
    // decode in every mode with a workspace of exactly the size asked for
    const int shapes[][5] = {{64, 32, 8, 128, 16}, {8, 32, 8, 128, 16}, {256, 32, 8, 128, 64},
                             {3, 40, 10, 64, 32}, {1, 16, 1, 64, 16}, {700, 8, 8, 128, 16}};
    for (const auto& s : shapes) {
        for (int P : {0, 16, 512, 4096, PA_PARTITION_BALANCED}) {
            for (int max_len : {1, 100, 4096, 131072}) {
                for (int splits : {1, 96, 1024}) {
                    g_splits = splits;
                    const size_t need = pa_decode_workspace_size(s[0], s[1], s[3], max_len, P);
                    if (need > ((size_t)64 << 20)) continue;   // keep the run short
                    Workspace w(need);
                    const int st = decode(s[0], s[1], s[2], s[3], s[4], P, max_len, w.p, need);
                    const bool too_many = P > 0 && (max_len + P - 1) / P > 65535;
                    EXPECT(st == (too_many ? PA_ERR_UNSUPPORTED : PA_OK));
                    if (need > 0 && st == PA_OK)   // one byte short is refused
                        EXPECT(decode(s[0], s[1], s[2], s[3], s[4], P, max_len, w.p, need - 1) ==
                               PA_ERR_WORKSPACE);
                }
            }
        }
    }
    g_splits = 96;

    // multi-query decode and the staged form, q_len 1..4
    for (int q_len = 1; q_len <= 4; ++q_len) {
        for (int P : {0, 256, PA_PARTITION_BALANCED}) {
            const size_t need = pa_decode_workspace_size(64, q_len * 32, 128, 4096, P);
            Workspace w(need);
            EXPECT(pa_decode_multi_query(fake(1), fake(2), PA_BF16, q_len, fake(3), fake(4), PA_BF16,
                                         ifake(5), 256, ifake(6), 64, 32, 8, 128, 16, 10000,
                                         0.088f, nullptr, nullptr, P, 4096, w.p, need,
                                         nullptr) == PA_OK);
            for (int stages : {PA_STAGE_ATTENTION, PA_STAGE_MERGE, PA_STAGE_ALL})
                EXPECT(pa_decode_stages(fake(1), fake(2), PA_BF16, q_len, fake(3), fake(4), PA_BF16,
                                        ifake(5), 256, ifake(6), 64, 32, 8, 128, 16, 10000, 0.088f,
                                        nullptr, nullptr, P, 4096, w.p, need, stages,
                                        nullptr) == PA_OK);
        }
    }

    // shared-prefix cascade: prefix ranges + partitions in one workspace
    for (int q_len : {1, 2, 4}) {
        for (int prefix : {0, 16, 2048, 8192}) {
            const size_t need = pa_decode_shared_prefix_workspace_size(64, q_len, 32, 8, 128, prefix,
                                                                       4096, 1024);
            Workspace w(need);
            EXPECT(pa_decode_shared_prefix(fake(1), fake(2), PA_BF16, q_len, fake(3), fake(4), PA_BF16,
                                           ifake(9), prefix, ifake(5), 256, ifake(6), 64, 32, 8, 128,
                                           16, 10000, 0.088f, nullptr, nullptr, 1024, 4096, w.p,
                                           need, nullptr) == PA_OK);
        }
    }

    // the fixed-workspace decode: within the buffer, and refused beyond it
    EXPECT(pa_decode_noalloc(fake(1), fake(2), PA_BF16, fake(3), fake(4), PA_BF16, ifake(5), 256,
                             ifake(6), 64, 32, 8, 128, 16, 10000, 0.088f, nullptr, nullptr,
                             PA_PARTITION_BALANCED, 4096, nullptr) == PA_OK);
    EXPECT(pa_decode_noalloc(fake(1), fake(2), PA_BF16, fake(3), fake(4), PA_BF16, ifake(5), 8192,
                             ifake(6), 8, 32, 8, 128, 16, 100000, 0.088f, nullptr, nullptr, 512,
                             131072, nullptr) == PA_OK);
    EXPECT(pa_decode_noalloc(fake(1), fake(2), PA_BF16, fake(3), fake(4), PA_BF16, ifake(5), 4096,
                             ifake(6), 2, 32, 8, 128, 16, 100000, 0.088f, nullptr, nullptr, 16,
                             65536, nullptr) == PA_ERR_WORKSPACE);

    // prefill, merge, split partitions, cache writes
    EXPECT(pa_prefill_chunk(fake(1), nullptr, fake(2), PA_BF16, ifake(3), 2048, 512, fake(4), fake(5),
                            PA_BF16, ifake(6), 160, ifake(7), 4, 32, 8, 128, 16, 10000, 0.088f,
                            nullptr, nullptr, nullptr) == PA_OK);
    EXPECT(pa_merge_partitions(fake(1), PA_BF16, nullptr, ffake(2), ffake(3), ifake(4), 512, 8, 64, 32,
                               128, nullptr) == PA_OK);
    {
        Workspace po((size_t)64 * 32 * 8 * 128 * sizeof(float)), pl((size_t)64 * 32 * 8 * sizeof(float));
        EXPECT(pa_decode_partitions(static_cast<float*>(po.p), static_cast<float*>(pl.p), 8, fake(3),
                                    PA_BF16, fake(4), fake(5), PA_BF16, ifake(6), 256, ifake(7), 64,
                                    32, 8, 128, 16, 10000, 0.088f, nullptr, nullptr, 512, 4096,
                                    nullptr) == PA_OK);
    }
    EXPECT(pa_write_kv(fake(1), fake(2), PA_FP8_E4M3, fake(3), fake(4), PA_BF16, 2048, 2048,
                       ifake(5), 64, 8, 128, 16, 10000, ffake(6), ffake(7), nullptr) == PA_OK);

    // the mixed step: workspaces of exactly the queried size, both modes,
    // either part empty
    for (int P : {PA_PARTITION_BALANCED, 512, 0}) {
        const size_t need = pa_decode_workspace_size(16, 32, 128, 8192, P);
        Workspace ws(need);
        EXPECT(pa_mixed_step(fake(1), fake(2), ifake(3), 512, ifake(4), 16, 8192, P, ws.p, need,
                             fake(5), nullptr, fake(6), ifake(7), 2048, 512, ifake(8), 160,
                             ifake(9), 4, PA_BF16, fake(10), fake(11), PA_BF16, 32, 8, 128, 16,
                             100000, 0.088f, nullptr, nullptr, nullptr) == PA_OK);
        EXPECT(pa_mixed_step(fake(1), fake(2), ifake(3), 512, ifake(4), 16, 8192, P, ws.p, need,
                             nullptr, nullptr, nullptr, nullptr, 0, 0, nullptr, 160, nullptr, 0,
                             PA_BF16, fake(10), fake(11), PA_BF16, 32, 8, 128, 16, 100000, 0.088f,
                             nullptr, nullptr, nullptr) == PA_OK);
        EXPECT(pa_mixed_step(nullptr, nullptr, nullptr, 512, nullptr, 0, 0, P, nullptr, 0,
                             fake(5), nullptr, fake(6), ifake(7), 2048, 512, ifake(8), 160,
                             ifake(9), 4, PA_BF16, fake(10), fake(11), PA_BF16, 32, 8, 128, 16,
                             100000, 0.088f, nullptr, nullptr, nullptr) == PA_OK);
        if (need > 0)
            EXPECT(pa_mixed_step(fake(1), fake(2), ifake(3), 512, ifake(4), 16, 8192, P, ws.p,
                                 need - 1, fake(5), nullptr, fake(6), ifake(7), 2048, 512, ifake(8),
                                 160, ifake(9), 4, PA_BF16, fake(10), fake(11), PA_BF16, 32, 8, 128,
                                 16, 100000, 0.088f, nullptr, nullptr, nullptr) == PA_ERR_WORKSPACE);
    }

    // the read probe hands the kernel exactly the buffer's 16-byte words
    {
        const size_t bytes = 4096 + 16;
        Workspace buf(bytes), sink(PA_STREAM_READ_SINK_WORDS * sizeof(uint32_t));
        unsigned char* b = static_cast<unsigned char*>(buf.p);
        uint32_t want = 0;
        for (size_t i = 0; i < bytes; ++i) {
            b[i] = (unsigned char)(i * 131 + 7);
            want ^= (uint32_t)b[i] << (8 * (i & 3));
        }
        uint32_t* x = static_cast<uint32_t*>(sink.p);
        std::memset(x, 0, PA_STREAM_READ_SINK_WORDS * sizeof(uint32_t));
        EXPECT(pa_stream_read(buf.p, bytes, 1, x, nullptr) == PA_OK);
        uint32_t got = 0;
        for (int g = 0; g < PA_STREAM_READ_SINK_WORDS; ++g) got ^= x[g];
        EXPECT(got == want);
        EXPECT(pa_stream_read(buf.p, bytes - 8, 1, x, nullptr) == PA_ERR_SHAPE);
    }

    // extreme sizes are refused, not overflowed
    const int big = 0x7fffffff;
    EXPECT(decode(big, 32, 8, 128, 16, 512, 4096, nullptr, 0) != PA_OK);
    EXPECT(decode(64, 32, 8, 128, 16, 16, big - 15, nullptr, 0) != PA_OK);
    EXPECT(pa_decode_workspace_size(big, big, 128, big, 16) == 0);    // refused sizes
    EXPECT(pa_decode_workspace_size(1, 32, 128, big, 16) == 0);       // too many partitions
    EXPECT(pa_decode_multi_query(fake(1), fake(2), PA_BF16, big, fake(3), fake(4), PA_BF16, ifake(5),
                                 256, ifake(6), 64, 32, 8, 128, 16, 10000, 0.088f, nullptr, nullptr, 0,
                                 4096, nullptr, 0, nullptr) != PA_OK);
    EXPECT(pa_prefill_chunk(fake(1), nullptr, fake(2), PA_BF16, ifake(3), big, big, fake(4), fake(5),
                            PA_BF16, ifake(6), 160, ifake(7), big, 32, 8, 128, 16, 10000, 0.088f,
                            nullptr, nullptr, nullptr) != PA_OK);
    EXPECT(pa_write_kv(fake(1), fake(2), PA_BF16, fake(3), fake(4), PA_BF16, big, big, ifake(5), big,
                       big, 128, 16, big, nullptr, nullptr, nullptr) != PA_OK);
    EXPECT(pa_mixed_step(fake(1), fake(2), ifake(3), 512, ifake(4), big, 8192, PA_PARTITION_BALANCED,
                         nullptr, 0, fake(5), nullptr, fake(6), ifake(7), big, big, ifake(8), 160,
                         ifake(9), big, PA_BF16, fake(10), fake(11), PA_BF16, 32, 8, 128, 16,
                         100000, 0.088f, nullptr, nullptr, nullptr) != PA_OK);
    EXPECT(pa_decode_shared_prefix_workspace_size(big, big, big, 1, 128, big, big, 16) == 0);
    EXPECT(pa_decode_shared_prefix_workspace_size(64, 1, 32, 8, 128, big, 4096, 1024) > 0);

    std::printf("%s: %d launches, %d failures\n", g_fail ? "FAILED" : "ok", g_launches, g_fail);
    return g_fail ? 1 : 0;
}
