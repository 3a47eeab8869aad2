// Log-sum-exp merge of split-KV decode partials.  gfx950 / CDNA4.
// Partials come either from fixed-size partitions ([row][partition]) or from
// the balanced split's pieces (a sequence's pieces at consecutive slots,
// (first slot, count) recorded by the decode kernel).
//
// Partition p of a sequence yields o_p (softmax-normalised over its tokens)
// and lse_p = ln sum exp(s) over the same tokens.  Attention over the union of
// the partitions is sum_p w_p o_p / sum_p w_p with w_p = exp(lse_p - M),
// M = max_p lse_p (the standard combination of softmax pieces; the pages give
// no merge rule of their own).  One wave per (sequence, q-head); every lane
// owns D / 64 consecutive output dims, so each partial row is read as one
// contiguous 256- or 512-byte run.
#include "device.h"
#include "launch.h"

namespace pa {
namespace {

__device__ __forceinline__ float wave_max(float x) { return group_max4(row_max16(x)); }

template <int D, bool OUT_BF16>
__global__ __launch_bounds__(64) void merge_kernel(const MergeArgs a) {
    constexpr int V = D / 64;  // dims per lane
    const int lane = threadIdx.x;
    const int Hq = a.num_q_heads;
    const int qh = blockIdx.x % Hq;
    const int b = blockIdx.x / Hq;
    const size_t row = (size_t)b * Hq + qh;
    const int L = a.seq_lens[b];
    // partials of this row: np of them at partial rows base + p * pstride
    int np;
    size_t base, pstride;
    if (a.piece_info) {
        // balanced pieces: row qh' = qi * H + qh of the sequence (H real heads)
        const int H = Hq / a.q_len, G = H / a.num_kv_heads;
        const int qi = qh / H, hq = qh - qi * H;
        const int h = hq / G, col = qi * G + (hq - h * G);
        const size_t cols = (size_t)a.q_len * G;
        // the record exists for every sequence slot (it is only written for
        // non-empty ones): read it alongside the length, use it only if L > 0
        const int2 rec = reinterpret_cast<const int2*>(a.piece_info)[b];
        const int2 info = L > 0 ? rec : make_int2(0, 0);
        np = info.y;
        base = ((size_t)h * a.piece_slots + info.x) * cols + col;
        pstride = cols;
    } else {
        np = a.lead_slots + min((L + a.partition_size - 1) / a.partition_size,
                                a.max_parts - a.lead_slots);
        base = row * a.max_parts;
        pstride = 1;
    }
    if (a.skip_single && np == 1) return;  // written by the partition kernel
    const float* lse = a.part_lse + base;
    const float* po = a.part_out + base * D + lane * V;

    // the first kAhead partials (lse and this lane's dims) are fetched
    // together with the lse values the maximum needs, so a row with few
    // partials costs one round trip after its record
    constexpr int kAhead = 4;   // (the max below is written out for 4)
    float l0[kAhead], o0[kAhead][V];
#pragma unroll
    for (int p = 0; p < kAhead; ++p) {
        l0[p] = p < np ? lse[(size_t)p * pstride] : -INFINITY;
#pragma unroll
        for (int v = 0; v < V; ++v) o0[p][v] = p < np ? po[(size_t)p * pstride * D + v] : 0.f;
    }
    float M = fmaxf(fmaxf(l0[0], l0[1]), fmaxf(l0[2], l0[3]));   // the same in every lane
    for (int p = kAhead + lane; p < np; p += 64) M = fmaxf(M, lse[(size_t)p * pstride]);
    M = wave_max(M);

    float acc[V];
#pragma unroll
    for (int v = 0; v < V; ++v) acc[v] = 0.f;
    float den = 0.f;
    if (M != -INFINITY) {
#pragma unroll
        for (int p = 0; p < kAhead; ++p) {
            if (p >= np) break;
            const float w = fast_exp2((l0[p] - M) * kLog2e);
            den += w;
#pragma unroll
            for (int v = 0; v < V; ++v) acc[v] += w * o0[p][v];
        }
#pragma unroll 4
        for (int p = kAhead; p < np; ++p) {
            // difference first: exactly 0 for the largest lse, whatever the
            // compiler fuses, so a lone partition passes through unchanged
            const float w = fast_exp2((lse[(size_t)p * pstride] - M) * kLog2e);
            den += w;
#pragma unroll
            for (int v = 0; v < V; ++v) acc[v] += w * po[(size_t)p * pstride * D + v];
        }
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

int launch_merge(const MergeArgs& a, void* stream) {
    if (a.num_seqs == 0) return 0;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    return (int)(a.head_dim == 64 ? launch_d<64>(a, s) : launch_d<128>(a, s));
}

}  // namespace pa
