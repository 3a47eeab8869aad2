// Log-sum-exp merge of split-KV decode partials.  gfx950 / CDNA4.
// One wave per (sequence, q-head) row (merge_row.h states the combination
// and the partial layouts); long contexts in partition mode take a
// workgroup per row.
#include "merge_row.h"

namespace pa {
namespace {

template <int D, bool OUT_BF16>
__global__ __launch_bounds__(64) void merge_kernel(const MergeArgs a) {
    const int qh = blockIdx.x % a.num_q_heads;
    const int b = blockIdx.x / a.num_q_heads;
    merge_row<D, OUT_BF16>(a, b, qh, threadIdx.x);
}

// Partition mode with many partitions (long contexts): one workgroup of
// kWideWaves waves per row, wave w merging partitions w, w + kWideWaves, ...
// with all its loads in flight, then the waves' maxima, weight sums and
// weighted rows combined through LDS.  The same combination as above, in a
// different summation order.
constexpr int kWideWaves = 8;
constexpr int kWideMinParts = 32;   // max_parts from which the wide kernel is used

template <int D, bool OUT_BF16>
__global__ __launch_bounds__(64 * kWideWaves) void merge_wide_kernel(const MergeArgs a) {
    constexpr int V = D / 64;
    __shared__ float s_m[kWideWaves], s_den[kWideWaves], s_acc[kWideWaves][D];
    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
    const int Hq = a.num_q_heads;
    const int qh = blockIdx.x % Hq;
    const int b = blockIdx.x / Hq;
    const size_t row = (size_t)b * Hq + qh;
    const int L = a.seq_lens[b];
    const int np = a.lead_slots + min((L + a.partition_size - 1) / a.partition_size,
                                      a.max_parts - a.lead_slots);
    if (a.skip_single && np == 1) return;   // uniform over the workgroup
    const float* lse = a.part_lse + row * a.max_parts;
    const float* po = a.part_out + row * a.max_parts * D + lane * V;

    // this wave's maximum over its partitions (one lse per lane and round)
    float m = -INFINITY;
    for (int p = w + kWideWaves * lane; p < np; p += 64 * kWideWaves) m = fmaxf(m, lse[p]);
    m = wave_max(m);
    if (lane == 0) s_m[w] = m;
    __syncthreads();
    float M = s_m[0];
#pragma unroll
    for (int v = 1; v < kWideWaves; ++v) M = fmaxf(M, s_m[v]);

    float acc[V];
#pragma unroll
    for (int v = 0; v < V; ++v) acc[v] = 0.f;
    float den = 0.f;
    if (M != -INFINITY) {
#pragma unroll 8
        for (int p = w; p < np; p += kWideWaves) {
            const float wt = fast_exp2((lse[p] - M) * kLog2e);
            den += wt;
#pragma unroll
            for (int v = 0; v < V; ++v) acc[v] += wt * po[(size_t)p * D + v];
        }
    }
#pragma unroll
    for (int v = 0; v < V; ++v) s_acc[w][lane * V + v] = acc[v];
    if (lane == 0) s_den[w] = den;
    __syncthreads();
    if (w != 0) return;
    den = 0.f;
#pragma unroll
    for (int x = 0; x < kWideWaves; ++x) den += s_den[x];
#pragma unroll
    for (int v = 0; v < V; ++v) {
        float t = 0.f;
#pragma unroll
        for (int x = 0; x < kWideWaves; ++x) t += s_acc[x][lane * V + v];
        acc[v] = t;
    }
    const float inv = den > 0.f ? 1.0f / den : 0.f;
    if constexpr (OUT_BF16) {
        uint16_t* o = reinterpret_cast<uint16_t*>(a.out) + row * D + lane * V;
        if constexpr (V == 2) {
            *reinterpret_cast<unsigned*>(o) = pack_bf16x2(acc[0] * inv, acc[1] * inv);
        } else {
            __bf16 x = (__bf16)(acc[0] * inv);
            *o = bitcast<uint16_t>(x);
        }
    } else {
        float* o = reinterpret_cast<float*>(a.out) + row * D + lane * V;
#pragma unroll
        for (int v = 0; v < V; ++v) o[v] = acc[v] * inv;
    }
    if (a.out_lse && lane == 0)
        a.out_lse[row] = den > 0.f ? M + fast_log2(den) * kLn2 : -INFINITY;
}

template <int D>
hipError_t launch_d(const MergeArgs& a, hipStream_t s) {
    dim3 grid((unsigned)(a.num_seqs * a.num_q_heads));
    const bool wide = !a.piece_info && a.max_parts >= kWideMinParts;
    if (wide) {
        if (a.out_dtype == 1)
            hipLaunchKernelGGL((merge_wide_kernel<D, true>), grid, dim3(64 * kWideWaves), 0, s, a);
        else
            hipLaunchKernelGGL((merge_wide_kernel<D, false>), grid, dim3(64 * kWideWaves), 0, s, a);
        return hipGetLastError();
    }
    if (a.out_dtype == 1)
        hipLaunchKernelGGL((merge_kernel<D, true>), grid, dim3(64), 0, s, a);
    else
        hipLaunchKernelGGL((merge_kernel<D, false>), grid, dim3(64), 0, s, a);
    return hipGetLastError();
}

}  // namespace

bool merge_fusable(const MergeArgs& a) { return a.piece_info || a.max_parts < kWideMinParts; }

int launch_merge(const MergeArgs& a, void* stream) {
    if (a.num_seqs == 0) return 0;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    return (int)(a.head_dim == 64 ? launch_d<64>(a, s) : launch_d<128>(a, s));
}

}  // namespace pa
