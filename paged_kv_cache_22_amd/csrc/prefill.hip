// Causal chunked prefill over a paged KV cache.  gfx950 / CDNA4.
//
// Chunked prefill and prefix caching are named on vllm-metis 0.1.0 (intro,
// "How the model maps onto vLLM", "Status": 64-token chunks and prefix-cache
// hits keep decode logprobs within 1e-5 of a reference).  The pages give no
// kernel; this one computes the plain definition: a chunk of n queries at
// the end of a sequence of L cached tokens has query i at position
// ctx + i (ctx = L - n), attending to keys 0 .. ctx + i.
//
// Layout of the work.  The chunk's (query, head-of-group) pairs are numbered
// rho = i * G + g and cut into 16-wide column tiles; one wave owns NC tiles
// of one (chunk, kv-head).  For each 16-token key block the wave computes
// S^T = K_blk . Q^T for each of its tiles on MFMA, runs the online softmax
// per column (base 2), and accumulates O^T += V^T_blk . P^T.  Every block is
// loaded once per wave and used by all NC tiles; blocks wholly below the
// diagonal skip the causal mask.  Blocks shared by several chunks (a common
// prefix) are simply read through each chunk's table.
#include "device.h"
#include "launch.h"
#include "tiles.h"

namespace pa {
namespace {

template <int D, int KIND, int NC>
__global__ __launch_bounds__(64) void prefill_kernel(const PrefillArgs a) {
    using T = Tile<KIND, D>;
    using QT = typename QType<KIND>::T;
    constexpr int NT = T::NT;

    const int lane = threadIdx.x;
    const int r = lane & 15, c = lane >> 4;
    const int Hkv = a.num_kv_heads, Hq = a.num_q_heads, G = Hq / Hkv;
    const int h = blockIdx.x % Hkv;
    const int ch = blockIdx.x / Hkv;
    const int qbeg = a.cu_q_lens[ch];
    const int qlen = a.cu_q_lens[ch + 1] - qbeg;
    const int L = a.seq_lens[ch];
    const int ctx = L - qlen;
    const int nrho = qlen * G;
    const int rho0 = blockIdx.y * (16 * NC);
    if (rho0 >= nrho || ctx < 0) return;  // ctx < 0 breaks the contract: read nothing

    const int last_rho = min(nrho, rho0 + 16 * NC) - 1;
    const int pos_max = ctx + last_rho / G;  // largest query position in this wave
    const int pos_min = ctx + rho0 / G;      // smallest
    const int nblk = pos_max / kBS + 1;      // key blocks anyone here sees
    const int full_end = (pos_min + 1) / kBS; // blocks below need no causal mask

    int pos[NC];
    bool ok[NC];
    int qrow_idx[NC];
    typename T::QOp Q[NC];
#pragma unroll
    for (int ct = 0; ct < NC; ++ct) {
        const int rho = rho0 + 16 * ct + r;
        ok[ct] = rho < nrho;
        const int i = rho / G, g = rho - (rho / G) * G;
        pos[ct] = ok[ct] ? ctx + i : pos_max;
        qrow_idx[ct] = (qbeg + i) * Hq + h * G + g;
        T::load_q(Q[ct], ok[ct] ? reinterpret_cast<const QT*>(a.q) + (size_t)qrow_idx[ct] * D : nullptr, c);
    }
    const float kscale = KIND == KV_FP8 ? a.k_scale[h] : 1.0f;
    const float C = a.scale * kLog2e * kscale;

    const int32_t* trow = a.block_table + (size_t)ch * a.max_blocks_per_seq;
    int tbase = 0;
    int tcur = (lane < nblk) ? trow[lane] : 0;
    int tnxt = (64 + lane < nblk) ? trow[64 + lane] : 0;
    const char* kbase = reinterpret_cast<const char*>(a.k_cache) + (size_t)h * T::kTileBytes;
    const char* vbase = reinterpret_cast<const char*>(a.v_cache) + (size_t)h * T::kTileBytes;
    const size_t blk_stride = (size_t)Hkv * T::kTileBytes;
    auto issue = [&](typename T::Regs& R, int jb) {
        const int idx = jb - tbase;
        const int phys = idx < 64 ? __builtin_amdgcn_readlane(tcur, idx)
                                  : __builtin_amdgcn_readlane(tnxt, idx - 64);
        const size_t off = (size_t)phys * blk_stride;
        T::load(R, kbase + off, vbase + off, r, c);
    };

    float m[NC], l[NC];
    f32x4 acc[NC][NT];
#pragma unroll
    for (int ct = 0; ct < NC; ++ct) {
        m[ct] = -INFINITY;
        l[ct] = 0.f;
#pragma unroll
        for (int n = 0; n < NT; ++n) acc[ct][n] = zero4();
    }

    // one key block against every column tile of the wave
    auto consume = [&](typename T::Regs& R, int jj) {
        const int valid = L - jj * kBS;
        if (valid < kBS) T::mask_v(R, c, valid);  // cache slots past L
        const bool diag = jj >= full_end;
#pragma unroll
        for (int ct = 0; ct < NC; ++ct) {
            const f32x4 sc = T::qk(R, Q[ct]);   // raw scores, as in decode
            float t[4] = {sc[0], sc[1], sc[2], sc[3]};
            if (diag) {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (jj * kBS + 4 * c + e > pos[ct]) t[e] = -INFINITY;
            }
            float bm = fmaxf(fmaxf(t[0], t[1]), fmaxf(t[2], t[3]));
            bm = group_max4(bm);
            const float mn = fmaxf(m[ct], bm);
            if (__ballot(mn > m[ct])) {
                const float alpha = fast_exp2((m[ct] - mn) * C);
                l[ct] *= alpha;
#pragma unroll
                for (int n = 0; n < NT; ++n) acc[ct][n] *= alpha;
                m[ct] = mn;
            }
            float p[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) p[e] = fast_exp2((t[e] - m[ct]) * C);
            l[ct] += group_sum4((p[0] + p[1]) + (p[2] + p[3]));
            T::pv(R, p, acc[ct]);
        }
    };

    // two-stage pipeline with a peeled tail, as in decode
    typename T::Regs b0, b1;
    issue(b0, 0);
    int j = 0;
    for (; j + 2 < nblk; j += 2) {
        if (j - tbase >= 64) {
            tbase += 64;
            tcur = tnxt;
            tnxt = (tbase + 64 + lane < nblk) ? trow[tbase + 64 + lane] : 0;
        }
        issue(b1, j + 1);
        consume(b0, j);
        issue(b0, j + 2);
        consume(b1, j + 1);
    }
    if (j - tbase >= 64) {
        tbase += 64;
        tcur = tnxt;
    }
    if (j + 1 < nblk) {
        issue(b1, j + 1);
        consume(b0, j);
        consume(b1, j + 1);
    } else {
        consume(b0, j);
    }

    const float vscale = KIND == KV_FP8 ? a.v_scale[h] : 1.0f;
#pragma unroll
    for (int ct = 0; ct < NC; ++ct) {
        if (!ok[ct]) continue;
        const float inv = vscale / l[ct];
        QT* o = reinterpret_cast<QT*>(a.out) + (size_t)qrow_idx[ct] * D;
#pragma unroll
        for (int n = 0; n < NT; ++n)
            store4(o + 16 * n + 4 * c, acc[ct][n][0] * inv, acc[ct][n][1] * inv,
                   acc[ct][n][2] * inv, acc[ct][n][3] * inv);
        if (a.out_lse && c == 0) a.out_lse[qrow_idx[ct]] = (m[ct] * C + fast_log2(l[ct])) * kLn2;
    }
}

constexpr int kNC = 2;

template <int D, int KIND>
hipError_t launch_t(const PrefillArgs& a, hipStream_t s) {
    const int G = a.num_q_heads / a.num_kv_heads;
    const long rows = (long)a.max_q_len * G;
    dim3 grid((unsigned)(a.num_chunks * a.num_kv_heads), (unsigned)((rows + 16 * kNC - 1) / (16 * kNC)));
    hipLaunchKernelGGL((prefill_kernel<D, KIND, kNC>), grid, dim3(64), 0, s, a);
    return hipGetLastError();
}

template <int D>
hipError_t launch_d(const PrefillArgs& a, hipStream_t s) {
    switch (a.kv_dtype) {
        case 0: return launch_t<D, KV_F32>(a, s);
        case 1: return launch_t<D, KV_BF16>(a, s);
        default: return launch_t<D, KV_FP8>(a, s);
    }
}

}  // namespace

int launch_prefill(const PrefillArgs& a, void* stream) {
    if (a.num_chunks == 0 || a.max_q_len == 0) return 0;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    return (int)(a.head_dim == 64 ? launch_d<64>(a, s) : launch_d<128>(a, s));
}

}  // namespace pa
