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
// rho = i * G + g and cut into 16-wide MFMA column tiles.  A workgroup of 4
// waves owns 4 * NC tiles of one (chunk, kv-head); each wave owns NC tiles.
// Key units go two at a time through a double-buffered LDS stage: the
// workgroup loads a step's K and V units once, every lane contiguous 16-byte
// pieces (plain loads, so blocks that several chunks share -- a common
// prefix -- can be served by L2), while the previous step is computed; one
// barrier per step.  Each of a wave's loads lies in one unit tile, so the
// block-table lookup and the tile's base address are scalar and only the
// lane's (loop-invariant) offset is a vector register.  K units keep their
// HBM layout in LDS; the two V units share one region whose rows interleave
// them by groups of 4 tokens, so a lane reads the whole K=32 operand of the
// output product in one piece.  Per step and column tile: S^T = K . Q^T on
// MFMA, online softmax per column (base 2), then O^T += V^T . P^T; the
// weights' column sums go through the MFMA too.  Steps wholly below a wave's
// diagonal skip the mask.
#include "device.h"
#include "launch.h"
#include "tiles.h"

namespace pa {
namespace {

constexpr int kWaves = 4;
constexpr int kStepBlocks = 2;  // key blocks per LDS stage (consumed as a pair)

template <int D, int KIND, int BS, int NC>
__global__ __launch_bounds__(64 * kWaves) void prefill_kernel(const PrefillArgs a) {
    using T = Tile<KIND, D, BS>;
    using QT = typename QType<KIND>::T;
    constexpr int NT = T::NT;
    constexpr int kSubShift = BS == 64 ? 2 : BS == 32 ? 1 : 0;   // log2(units per block)
    constexpr int TB = T::kUnitBytes;                       // one 16-token K (or V) unit
    constexpr int kUnitRun = kBS * 16;                       // one K chunk run of a unit
    constexpr int kTilePieces = TB / 16;                     // 16-byte pieces per unit
    static_assert(kTilePieces % 64 == 0, "a wave's load lies in one unit");
    constexpr int kPieces = kStepBlocks * 2 * kTilePieces;   // per step: 2 units of K and V
    constexpr int kPerThread = kPieces / (64 * kWaves);
    static_assert(kPieces % (64 * kWaves) == 0, "every thread loads whole pieces");
    constexpr int kOffV = kStepBlocks * TB;                  // the V pair region
    constexpr int kStage = (kOffV + D * T::kVPairRow + 15) / 16 * 16;
    __shared__ __attribute__((aligned(16))) char stage[2][kStage];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, known uniform
    const int r = lane & 15, c = lane >> 4;
    const int Hkv = a.num_kv_heads, Hq = a.num_q_heads, G = Hq / Hkv;
    const int h = blockIdx.x % Hkv;
    const int ch = blockIdx.x / Hkv;
    const int qbeg = a.uniform_q_len > 0 ? ch * a.uniform_q_len : a.cu_q_lens[ch];
    const int qlen = a.uniform_q_len > 0 ? a.uniform_q_len : a.cu_q_lens[ch + 1] - qbeg;
    // key-range mode: keys [ubeg * 16, kend) of a kv_len-token sequence, all
    // visible to every row; otherwise causal keys 0 .. ctx + i
    const bool ranged = a.kv_len > 0;
    const int L = ranged ? a.kv_len : a.seq_lens[ch];
    const int ctx = L - qlen;
    const int ubeg = ranged ? (int)blockIdx.z * (a.key_range / kBS) : 0;
    const int kend = ranged ? min(L, ((int)blockIdx.z + 1) * a.key_range) : L;
    const int nrho = qlen * G;
    const int rho_wg = blockIdx.y * (16 * NC * kWaves);
    if (rho_wg >= nrho) return;  // uniform
    if (!ranged && ctx < 0) {
        // fewer cached tokens than queries (an idle sequence has none): the
        // rows see no keys; they get zeros and lse -inf, and nothing is read
#pragma unroll
        for (int ct = 0; ct < NC; ++ct) {
            const int rho = rho_wg + w * 16 * NC + 16 * ct + r;
            if (rho >= nrho) continue;
            const int i = rho / G, g = rho - (rho / G) * G;
            const size_t qrow = (size_t)(qbeg + i) * Hq + h * G + g;
            QT* o = reinterpret_cast<QT*>(a.out) + qrow * D;
#pragma unroll
            for (int n = 0; n < T::NT; ++n) store4(o + 16 * n + 4 * c, 0.f, 0.f, 0.f, 0.f);
            if (a.out_lse && c == 0) a.out_lse[qrow] = -INFINITY;
        }
        return;
    }

    // the last key query i sees
    auto qpos = [&](int i) { return ranged ? kend - 1 : ctx + i; };
    // key units the workgroup needs (up to nblk), and this wave's share of the rows
    const int nblk = qpos((min(nrho, rho_wg + 16 * NC * kWaves) - 1) / G) / kBS + 1;
    const int rho0 = rho_wg + w * 16 * NC;
    const bool wave_rows = rho0 < nrho;
    const int w_last = min(nrho, rho0 + 16 * NC) - 1;
    const int w_nblk = wave_rows ? qpos(w_last / G) / kBS + 1 : 0;     // units this wave sees
    const int full_end = wave_rows ? (qpos(rho0 / G) + 1) / kBS : 0;   // no mask below this

    int pos[NC];
    bool ok[NC];
    int qrow_idx[NC];
    typename T::QOp Q[NC];
#pragma unroll
    for (int ct = 0; ct < NC; ++ct) {
        const int rho = rho0 + 16 * ct + r;
        ok[ct] = rho < nrho;
        const int i = rho / G, g = rho - (rho / G) * G;
        pos[ct] = ok[ct] ? qpos(i) : qpos(w_last / G);
        qrow_idx[ct] = (qbeg + i) * Hq + h * G + g;
        T::load_q(Q[ct], ok[ct] ? reinterpret_cast<const QT*>(a.q) + (size_t)qrow_idx[ct] * D : nullptr, c);
    }
    const float kscale = KIND == KV_FP8 ? a.k_scale[h] : 1.0f;
    const float C = a.scale * kLog2e * kscale;

    // block-table window (every wave holds the same 64 entries): lane i holds
    // the table entry of unit tbase + i, unit u lying in block u / (BS / 16)
    const int32_t* trow = a.block_table + (size_t)ch * a.max_blocks_per_seq;
    int tbase = ubeg;
    int tcur = (ubeg + lane < nblk) ? trow[(ubeg + lane) >> kSubShift] : 0;
    const char* kbase = reinterpret_cast<const char*>(a.k_cache) + (size_t)h * T::kTileBytes;
    const char* vbase = reinterpret_cast<const char*>(a.v_cache) + (size_t)h * T::kTileBytes;
    const size_t blk_stride = (size_t)Hkv * T::kTileBytes;

    // A step's pieces: wave w's load u covers pieces 64 * (w + 4u) + lane,
    // which lie in one unit tile (uniform over the wave): tile = 2 * unit of
    // the step + (0 for K, 1 for V).  off is the piece's byte in the unit's
    // own layout; voff its place in the cache block's tile (K chunk runs and
    // V rows are BS tokens long there), both fixed for the whole loop.
    auto piece_tile = [&](int u) { return (64 * (w + kWaves * u)) / kTilePieces; };
    auto piece_off = [&](int u) { return ((64 * (w + kWaves * u)) % kTilePieces + lane) * 16; };
    int voff[kPerThread];
#pragma unroll
    for (int u = 0; u < kPerThread; ++u) {
        const int off = piece_off(u);
        voff[u] = (piece_tile(u) & 1)
            ? (off / T::kVRow) * T::kVRow * (BS / kBS) + off % T::kVRow
            : (off / kUnitRun) * kUnitRun * (BS / kBS) + off % kUnitRun;
    }

    // global -> registers for the step starting at unit j0 (a missing second
    // unit re-reads the first, which the consumer masks)
    u32x4 held[kPerThread];
    auto fetch = [&](int j0) {
#pragma unroll
        for (int u = 0; u < kPerThread; ++u) {
            const int tile = piece_tile(u);
            const int jb = min(j0 + (tile >> 1), nblk - 1);
            const int phys = __builtin_amdgcn_readlane(tcur, __builtin_amdgcn_readfirstlane(jb - tbase));
            const int sub = jb & ((1 << kSubShift) - 1);    // unit within the block
            gchar* base = uniform_ptr((tile & 1)
                ? vbase + (size_t)phys * blk_stride + sub * T::kUnitV
                : kbase + (size_t)phys * blk_stride + sub * T::kUnitK);
            held[u] = ld16(base + (uint32_t)voff[u]);
        }
    };
    // registers -> LDS: K units verbatim; V pieces split into their groups of
    // 4 tokens, each to its place in the pair region
    auto stash = [&](int buf) {
#pragma unroll
        for (int u = 0; u < kPerThread; ++u) {
            const int tile = piece_tile(u), off = piece_off(u), unit = tile >> 1;
            if (!(tile & 1)) {
                *reinterpret_cast<u32x4*>(stage[buf] + unit * TB + off) = held[u];
                continue;
            }
            const int row = off / T::kVRow, g0 = (off % T::kVRow) / T::kVGrp;
            char* dst = stage[buf] + kOffV + row * T::kVPairRow + unit * T::kVGrp + g0 * 2 * T::kVGrp;
            if constexpr (T::kVGrp == 16) {
                *reinterpret_cast<u32x4*>(dst) = held[u];
            } else if constexpr (T::kVGrp == 8) {
                reinterpret_cast<u32x2*>(dst)[0] = u32x2{held[u].x, held[u].y};
                reinterpret_cast<u32x2*>(dst + 16)[0] = u32x2{held[u].z, held[u].w};
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) reinterpret_cast<unsigned*>(dst + 8 * e)[0] = held[u][e];
            }
        }
    };

    // m: running max (raw score units); accl: the weights' column sums,
    // accumulated by MFMA (every element of a lane's accl holds its column's sum)
    float m[NC];
    f32x4 accl[NC];
    f32x4 acc[NC][NT];
#pragma unroll
    for (int ct = 0; ct < NC; ++ct) {
        m[ct] = -INFINITY;
        accl[ct] = zero4();
#pragma unroll
        for (int n = 0; n < NT; ++n) acc[ct][n] = zero4();
    }

    // The two units of a step (jA, jA+1) against every column tile of this
    // wave: 8 scores per lane, one online-softmax round over 32 keys, one
    // K=32 MFMA per output tile.  A unit the wave does not need (past its
    // diagonal, or past the sequence) has all its scores masked to -inf and
    // its V zeroed, so it adds exactly nothing.
    auto consume2 = [&](int buf, int jA) {
        typename T::KRegs RA, RB;
        typename T::VPair VP;
        T::load_k_lds(RA, stage[buf], r, c);
        T::load_k_lds(RB, stage[buf] + TB, r, c);
        T::load_vpair(VP, stage[buf] + kOffV, r, c);
        const int jB = jA + 1;
        const bool needB = jB < w_nblk;
        const int validA = kend - jA * kBS;
        const int validB = needB ? kend - jB * kBS : 0;
        if (validA < kBS || validB < kBS) T::mask_vpair(VP, c, validA, validB);  // slots past L
        const bool diag = jB >= full_end || !needB;
#pragma unroll
        for (int ct = 0; ct < NC; ++ct) {
            const f32x4 sa = T::qk(RA, Q[ct]);   // raw scores, as in decode
            const f32x4 sb = T::qk(RB, Q[ct]);
            float t[8] = {sa[0], sa[1], sa[2], sa[3], sb[0], sb[1], sb[2], sb[3]};
            if (diag) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    if (jA * kBS + 4 * c + e > pos[ct]) t[e] = -INFINITY;
                    if (!needB || jB * kBS + 4 * c + e > pos[ct]) t[4 + e] = -INFINITY;
                }
            }
            float bm = fmaxf(fmaxf(fmaxf(t[0], t[1]), fmaxf(t[2], t[3])),
                             fmaxf(fmaxf(t[4], t[5]), fmaxf(t[6], t[7])));
            bm = group_max4(bm);
            const float mn = fmaxf(m[ct], bm);
            if (__ballot((mn - m[ct]) * C > kRescaleLog2)) {
                const float alpha = fast_exp2((m[ct] - mn) * C);
                accl[ct] *= alpha;
#pragma unroll
                for (int n = 0; n < NT; ++n) acc[ct][n] *= alpha;
                m[ct] = mn;
            }
            // exp2(t * C - m * C) as one FMA per weight: at the maximum it
            // leaves the rounding error of m * C, far below bf16's resolution,
            // so the packed weight is exactly 1 there and the normaliser (the
            // sum of the packed weights) matches it
            const float mc = m[ct] * C;
            float p[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) p[e] = fast_exp2(fmaf(t[e], C, -mc));
            const auto pk = T::pack_p2(p);
            T::pv2(VP, pk, acc[ct]);
            T::lsum2(pk, accl[ct]);
        }
    };

    const int nsteps = (nblk - ubeg + kStepBlocks - 1) / kStepBlocks;
    fetch(ubeg);
    stash(0);
    __syncthreads();
    for (int s = 0; s < nsteps; ++s) {
        const int j0 = ubeg + s * kStepBlocks;
        if (s + 1 < nsteps) {
            if (j0 + 2 * kStepBlocks - 1 - tbase >= 64) {  // next step leaves the table window
                tbase += 64 - kStepBlocks;                  // keep the 2 steps in one window
                tcur = (tbase + lane < nblk) ? trow[(tbase + lane) >> kSubShift] : 0;
            }
            fetch(j0 + kStepBlocks);  // in flight during this step's compute
        }
        if (j0 < w_nblk) consume2(s & 1, j0);
        if (s + 1 < nsteps) stash((s + 1) & 1);
        __syncthreads();
    }

    const float vscale = KIND == KV_FP8 ? a.v_scale[h] : 1.0f;
#pragma unroll
    for (int ct = 0; ct < NC; ++ct) {
        const float lsum = accl[ct][0];
        if (!ok[ct]) continue;
        const float inv = vscale / lsum;
        if (a.part_out) {
            const size_t pidx = (size_t)qrow_idx[ct] * a.part_stride + (ranged ? blockIdx.z : 0);
            float* po = a.part_out + pidx * D;
#pragma unroll
            for (int n = 0; n < NT; ++n)
                store4(po + 16 * n + 4 * c, acc[ct][n][0] * inv, acc[ct][n][1] * inv,
                       acc[ct][n][2] * inv, acc[ct][n][3] * inv);
            if (c == 0) a.part_lse[pidx] = (m[ct] * C + fast_log2(lsum)) * kLn2;
            continue;
        }
        QT* o = reinterpret_cast<QT*>(a.out) + (size_t)qrow_idx[ct] * D;
#pragma unroll
        for (int n = 0; n < NT; ++n)
            store4(o + 16 * n + 4 * c, acc[ct][n][0] * inv, acc[ct][n][1] * inv,
                   acc[ct][n][2] * inv, acc[ct][n][3] * inv);
        if (a.out_lse && c == 0) a.out_lse[qrow_idx[ct]] = (m[ct] * C + fast_log2(lsum)) * kLn2;
    }
}

#ifndef PA_PREFILL_NC
#define PA_PREFILL_NC 2
#endif
constexpr int kNC = PA_PREFILL_NC;

template <int D, int KIND, int BS>
hipError_t launch_t(const PrefillArgs& a, hipStream_t s) {
    const int G = a.num_q_heads / a.num_kv_heads;
    const long rows = (long)a.max_q_len * G;
    const long per_wg = 16L * kNC * kWaves;
    const unsigned ranges = a.kv_len > 0 ? (unsigned)((a.kv_len + a.key_range - 1) / a.key_range) : 1u;
    dim3 grid((unsigned)(a.num_chunks * a.num_kv_heads), (unsigned)((rows + per_wg - 1) / per_wg), ranges);
    hipLaunchKernelGGL((prefill_kernel<D, KIND, BS, kNC>), grid, dim3(64 * kWaves), 0, s, a);
    return hipGetLastError();
}

template <int D, int KIND>
hipError_t launch_kind(const PrefillArgs& a, hipStream_t s) {
    if (a.block_size == 64) return launch_t<D, KIND, 64>(a, s);
    if (a.block_size == 32) return launch_t<D, KIND, 32>(a, s);
    return launch_t<D, KIND, 16>(a, s);
}

template <int D>
hipError_t launch_d(const PrefillArgs& a, hipStream_t s) {
    switch (a.kv_dtype) {
        case 0: return launch_kind<D, KV_F32>(a, s);
        case 1: return launch_kind<D, KV_BF16>(a, s);
        default: return launch_kind<D, KV_FP8>(a, s);
    }
}

}  // namespace

int launch_prefill(const PrefillArgs& a, void* stream) {
    if (a.num_chunks == 0 || a.max_q_len == 0) return 0;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    return (int)(a.head_dim == 64 ? launch_d<64>(a, s) : launch_d<128>(a, s));
}

}  // namespace pa
