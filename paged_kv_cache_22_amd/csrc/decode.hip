// Decode attention over a block-table KV cache, one wave per
// (sequence, kv-head, partition).  gfx950 / CDNA4.
//
// What is computed: for each query head j of sequence b, softmax(scale * q_j
// . K^T) V over the sequence's cached tokens, q-head j reading kv-head j / G.
// The pages name this operation (paged attention driven by device-side block
// tables and sequence lengths: vllm-metal architecture article, sections 三
// and 四; GQA 4:1: vllm-metis 0.1.0, "Status"); the formula is the plain
// definition of attention.
//
// How (one wave of 64 lanes handles one kv-head, i.e. G <= 16 query heads):
//   * per 16-token block, S^T[16 tokens x 16 heads] = K_blk . Q^T on MFMA
//     (K as the A operand exactly as it sits in the token-major tile, Q^T as
//     the B operand, heads >= G padded with zeros);
//   * online softmax in base 2: each lane owns one head (its column r) and
//     four tokens; block max / sum are reduced over the four lane groups with
//     row-swap permutes;
//   * O^T[d x 16 heads] += V^T_blk . P^T on MFMA; the dim-major V tile makes
//     V^T the A operand with each lane reading four consecutive tokens;
//   * K/V of the next STAGES-1 blocks are in flight while a block is
//     computed; block-table entries are fetched 64 at a time, one per lane,
//     and broadcast with readlane, so no load waits on a table lookup.
// Split-KV: partition p covers blocks [p*PB, (p+1)*PB); it writes its
// normalised output and lse (natural log) for the log-sum-exp merge.
#include "device.h"
#include "launch.h"
#include "tiles.h"

namespace pa {
namespace {

template <int D, int KIND, bool SPLIT, int STAGES>
__global__ __launch_bounds__(64) void decode_kernel(const DecodeArgs a) {
    using T = Tile<KIND, D>;
    using QT = typename QType<KIND>::T;
    constexpr int NT = T::NT;
    static_assert(64 % STAGES == 0, "STAGES must divide the 64-entry table window");

    const int lane = threadIdx.x;
    const int r = lane & 15, c = lane >> 4;
    const int Hkv = a.num_kv_heads, Hq = a.num_q_heads, G = Hq / Hkv;
    const int h = blockIdx.x % Hkv;
    const int b = blockIdx.x / Hkv;
    const int part = blockIdx.y;
    const int L = a.seq_lens[b];
    const int nblk = (L + kBS - 1) / kBS;
    const int pb = SPLIT ? a.partition_blocks : nblk;
    const int j0 = part * pb;
    const int qh = h * G + r;
    const bool col_ok = r < G;

    if (j0 >= nblk) {
        if (!SPLIT && col_ok) {  // empty sequence: zeros
            QT* o = reinterpret_cast<QT*>(a.out) + ((size_t)b * Hq + qh) * D;
#pragma unroll
            for (int n = 0; n < NT; ++n) store4(o + 16 * n + 4 * c, 0.f, 0.f, 0.f, 0.f);
        }
        return;
    }
    const int j1 = min(nblk, j0 + pb);

    typename T::QOp Q;
    T::load_q(Q, col_ok ? reinterpret_cast<const QT*>(a.q) + ((size_t)b * Hq + qh) * D : nullptr, c);
    const float kscale = KIND == KV_FP8 ? a.k_scale[h] : 1.0f;
    const float C = a.scale * kLog2e * kscale;  // raw score -> base-2 logit (C > 0)

    // block-table window: entries [tbase, tbase + 128), one per lane per half
    const int32_t* trow = a.block_table + (size_t)b * a.max_blocks_per_seq;
    int tbase = j0;
    int tcur = (j0 + lane < j1) ? trow[j0 + lane] : 0;
    int tnxt = (j0 + 64 + lane < j1) ? trow[j0 + 64 + lane] : 0;

    const char* kbase = reinterpret_cast<const char*>(a.k_cache) + (size_t)h * T::kTileBytes;
    const char* vbase = reinterpret_cast<const char*>(a.v_cache) + (size_t)h * T::kTileBytes;
    const size_t blk_stride = (size_t)Hkv * T::kTileBytes;

    auto issue = [&](typename T::Regs& R, int j) {
        const int idx = j - tbase;
        const int phys = idx < 64 ? __builtin_amdgcn_readlane(tcur, idx)
                                  : __builtin_amdgcn_readlane(tnxt, idx - 64);
        const size_t off = (size_t)phys * blk_stride;
        T::load(R, kbase + off, vbase + off, r, c);
    };

    float m = -INFINITY, l = 0.f;
    f32x4 acc[NT];
#pragma unroll
    for (int n = 0; n < NT; ++n) acc[n] = zero4();

    typename T::Regs buf[STAGES];
#pragma unroll
    for (int s = 0; s < STAGES - 1; ++s)
        if (j0 + s < j1) issue(buf[s], j0 + s);

    for (int j = j0; j < j1; j += STAGES) {
        if (j - tbase >= 64) {  // slide the table window (uniform, once per 64 blocks)
            tbase += 64;
            tcur = tnxt;
            tnxt = (tbase + 64 + lane < j1) ? trow[tbase + 64 + lane] : 0;
        }
#pragma unroll
        for (int s = 0; s < STAGES; ++s) {
            const int jj = j + s;
            if (jj < j1) {
                if (jj + STAGES - 1 < j1) issue(buf[(s + STAGES - 1) % STAGES], jj + STAGES - 1);
                typename T::Regs& R = buf[s];
                // raw scores; the softmax scale (times log2 e, times the fp8 K
                // scale) is applied to differences from the running max, so
                // the maximum's weight is exactly exp2(0) = 1
                const f32x4 sc = T::qk(R, Q);
                float t[4] = {sc[0], sc[1], sc[2], sc[3]};
                const int valid = L - jj * kBS;
                if (valid < kBS) {  // tail block: mask tokens past L (scores and V)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (4 * c + e >= valid) t[e] = -INFINITY;
                    T::mask_v(R, c, valid);
                }
                float bm = fmaxf(fmaxf(t[0], t[1]), fmaxf(t[2], t[3]));
                bm = group_max4(bm);
                const float mn = fmaxf(m, bm);
                const float alpha = fast_exp2((m - mn) * C);
                float p[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) p[e] = fast_exp2((t[e] - mn) * C);
                const float ps = group_sum4((p[0] + p[1]) + (p[2] + p[3]));
                l = l * alpha + ps;
                m = mn;
#pragma unroll
                for (int n = 0; n < NT; ++n) acc[n] *= alpha;
                T::pv(R, p, acc);
            }
        }
    }

    if (!col_ok) return;
    const float vscale = KIND == KV_FP8 ? a.v_scale[h] : 1.0f;
    const float inv = vscale / l;
    if constexpr (SPLIT) {
        const size_t row = (size_t)b * Hq + qh;
        float* po = a.part_out + (row * a.max_parts + part) * D;
#pragma unroll
        for (int n = 0; n < NT; ++n)
            store4(po + 16 * n + 4 * c, acc[n][0] * inv, acc[n][1] * inv, acc[n][2] * inv,
                   acc[n][3] * inv);
        if (c == 0) a.part_lse[row * a.max_parts + part] = (m * C + fast_log2(l)) * kLn2;
    } else {
        QT* o = reinterpret_cast<QT*>(a.out) + ((size_t)b * Hq + qh) * D;
#pragma unroll
        for (int n = 0; n < NT; ++n)
            store4(o + 16 * n + 4 * c, acc[n][0] * inv, acc[n][1] * inv, acc[n][2] * inv,
                   acc[n][3] * inv);
    }
}

template <int KIND> constexpr int stages_for() { return KIND == KV_FP8 ? 4 : 2; }

template <int D, int KIND, bool SPLIT>
hipError_t launch_t(const DecodeArgs& a, hipStream_t s) {
    dim3 grid((unsigned)(a.num_seqs * a.num_kv_heads), SPLIT ? (unsigned)a.grid_parts : 1u);
    hipLaunchKernelGGL((decode_kernel<D, KIND, SPLIT, stages_for<KIND>()>), grid, dim3(64), 0, s, a);
    return hipGetLastError();
}

template <int D, int KIND>
hipError_t launch_kind(const DecodeArgs& a, hipStream_t s) {
    return a.partition_blocks > 0 ? launch_t<D, KIND, true>(a, s) : launch_t<D, KIND, false>(a, s);
}

template <int D>
hipError_t launch_d(const DecodeArgs& a, hipStream_t s) {
    switch (a.kv_dtype) {
        case 0: return launch_kind<D, KV_F32>(a, s);
        case 1: return launch_kind<D, KV_BF16>(a, s);
        default: return launch_kind<D, KV_FP8>(a, s);
    }
}

}  // namespace

int launch_decode(const DecodeArgs& a, void* stream) {
    if (a.num_seqs == 0) return 0;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    hipError_t e = a.head_dim == 64 ? launch_d<64>(a, s) : launch_d<128>(a, s);
    return (int)e;
}

}  // namespace pa
