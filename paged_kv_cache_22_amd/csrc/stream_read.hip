// Streaming read of one device buffer: the measured HBM read rate that the
// attention kernels' live-K/V rates are reported beside (the 8 TB/s figure
// is the part's specification; this is what a plain linear read reaches on
// the device at hand).  Not a step of attention.
//
// Each workgroup reads one contiguous span of the buffer front to back,
// 32 KiB per iteration (eight 16-byte loads in flight per lane, each load
// instruction of a wave 1 KiB of consecutive bytes), so a workgroup stays on
// a few pages at a time (measured: contiguous spans read 6.75-6.9 TB/s on
// 1 GiB where a grid-stride order of the same loads reads 5.3-6.0).  Workgroup
// g XORs the words it read (folded to 32 bits) into sink word g, which keeps
// the loads live and gives the tests something exact to check; one atomic
// per workgroup on a single word instead serialises at the memory side and
// cost 20% of the time at 2048 workgroups.  KV loads in the library are
// non-temporal; `nontemporal` selects that load form or the plain one.
#include "../../include/pa.h"
#include "device.h"
#include "launch.h"

namespace pa {
namespace {

constexpr int kThreads = 256;
constexpr int kInFlight = 8;          // 16-byte loads per lane per iteration
constexpr unsigned kMaxGroups = PA_STREAM_READ_SINK_WORDS;  // 8 per compute unit

template <bool NT>
__device__ __forceinline__ u32x4 load16(const u32x4* p) {
    if constexpr (NT) return __builtin_nontemporal_load(p);
    else return *p;
}

// words [blockIdx.x * span, min((blockIdx.x + 1) * span, n)) of p
template <bool NT>
__global__ __launch_bounds__(kThreads) void stream_read_kernel(const u32x4* __restrict__ p,
                                                              size_t n, size_t span,
                                                              unsigned* sink) {
    const size_t begin = (size_t)blockIdx.x * span;
    const size_t end = begin + span < n ? begin + span : n;
    size_t i = begin + threadIdx.x;
    u32x4 acc = {0u, 0u, 0u, 0u};
    for (; i + (kInFlight - 1) * kThreads < end; i += kInFlight * kThreads) {
        u32x4 v[kInFlight];
#pragma unroll
        for (int u = 0; u < kInFlight; ++u) v[u] = load16<NT>(p + i + u * kThreads);
#pragma unroll
        for (int u = 0; u < kInFlight; ++u) acc ^= v[u];
    }
    for (; i < end; i += kThreads) acc ^= load16<NT>(p + i);
    unsigned x = acc.x ^ acc.y ^ acc.z ^ acc.w;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x ^= __shfl_xor(x, o, 64);
    __shared__ unsigned waves[kThreads / 64];
    if ((threadIdx.x & 63) == 0) waves[threadIdx.x >> 6] = x;
    __syncthreads();
    if (threadIdx.x == 0) {
        unsigned w = 0;
#pragma unroll
        for (int k = 0; k < kThreads / 64; ++k) w ^= waves[k];
        sink[blockIdx.x] ^= w;
    }
}

}  // namespace

int launch_stream_read(const void* buf, size_t n16, int nontemporal, unsigned* sink,
                       void* stream) {
    // spans of whole 32 KiB iterations, at most kMaxGroups of them
    const size_t step = (size_t)kThreads * kInFlight;
    const size_t steps = (n16 + step - 1) / step;
    const size_t per_group = (steps + kMaxGroups - 1) / kMaxGroups;
    const size_t span = per_group * step;
    const size_t groups = (n16 + span - 1) / span;
    const dim3 grid((unsigned)groups), block(kThreads);
    const auto* p = static_cast<const u32x4*>(buf);
    if (nontemporal)
        hipLaunchKernelGGL(stream_read_kernel<true>, grid, block, 0, (hipStream_t)stream, p, n16,
                           span, sink);
    else
        hipLaunchKernelGGL(stream_read_kernel<false>, grid, block, 0, (hipStream_t)stream, p, n16,
                           span, sink);
    return (int)hipGetLastError();
}

}  // namespace pa
