// Log-sum-exp merge of one output row's split-KV partials, by one wave.
// gfx950 / CDNA4.  Shared by the merge kernel and by the prefill kernel,
// which can merge a decode step's rows before its own work (a mixed step).
//
// Partition p of a sequence yields o_p (softmax-normalised over its tokens)
// and lse_p = ln sum exp(s) over the same tokens.  Attention over the union of
// the partitions is sum_p w_p o_p / sum_p w_p with w_p = exp(lse_p - M),
// M = max_p lse_p (the standard combination of softmax pieces; the pages give
// no merge rule of their own).  Every lane owns D / 64 consecutive output
// dims, so each partial row is read as one contiguous 256- or 512-byte run.
// Partials come either from fixed-size partitions ([row][partition]) or from
// the balanced split's pieces (a sequence's pieces at consecutive slots,
// (first slot, count) recorded by the decode kernel).
#pragma once

#include "device.h"
#include "launch.h"

namespace pa {

__device__ __forceinline__ float wave_max(float x) { return group_max4(row_max16(x)); }

// merge output row qh of sequence b (rows of a sequence: a.num_q_heads)
template <int D, bool OUT_BF16>
__device__ __forceinline__ void merge_row(const MergeArgs& a, int b, int qh, int lane) {
    constexpr int V = D / 64;  // dims per lane
    const int Hq = a.num_q_heads;
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

}  // namespace pa
