// Decode attention over a block-table KV cache, one wave per
// (sequence, kv-head, partition).  gfx950 / CDNA4.  The kernels and their
// launchers; decode.hip instantiates them for one query per sequence,
// decode_mq.hip for several (each translation unit with its own copies).
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
//     four tokens; the block max is reduced over the four lane groups with
//     row-swap permutes, the row sum only once at the end; the running max is
//     refreshed (and the accumulator rescaled) only when it jumps by more than
//     kRescaleLog2;
//   * O^T[d x 16 heads] += V^T_blk . P^T on MFMA; the dim-major V tile makes
//     V^T the A operand with each lane reading four consecutive tokens;
//   * a workgroup of 4 waves shares one (sequence, kv-head, partition): wave
//     w takes blocks w, w+4, ...; the waves' softmax states are combined
//     through LDS at the end;
//   * K/V of the next block are in flight while a block is computed;
//     block-table entries are fetched 64 at a time, one per lane, and
//     broadcast with readlane, so no load waits on a table lookup; KV loads
//     are non-temporal (each tile is read once).
// Split-KV: partition p covers blocks [p*PB, (p+1)*PB); it writes its
// normalised output and lse (natural log) for the log-sum-exp merge.
//
// Several queries per sequence (MQ): the q_len newest cached tokens are all
// queries, as when a batch of drafted tokens is verified in one step.  Query
// i sits at position L - q_len + i and sees keys 0 .. L - q_len + i.  With
// q_len * G <= 16 the (query, head) pairs fill the 16 MFMA columns, column
// r = i * G + g, so verifying q_len tokens reads the sequence's K/V once,
// like a single decode step; each column carries its own causal limit into
// the score mask of the last blocks.
#pragma once

#include "device.h"
#include "launch.h"
#include "tiles.h"

#include <type_traits>

namespace pa {
namespace {

// Where one (sequence, kv-head) range's result goes.  direct: the normalised
// output row; otherwise a partial (output and lse) at partial index
// prow_base + row * prow_stride (row = the column's output row) or, with
// prow_stride == 0, prow_base + r (r = the column).
struct RangeOut {
    bool direct;
    size_t prow_base;
    size_t prow_stride;
};

// The balanced kernel stages finished partials (of its pieces, or with
// PARTS below of its partitions) in LDS and writes them in bulk, at the end
// or when the slots are full: partial stores in the middle of the stream
// measured costly (on gfx950 a wave's stores share the load counter, and
// under full read traffic they hold back the loads issued after them).  A
// slot holds the normalised rows and lse of one (piece or partition,
// kv-head) and the index of its first partial row.
constexpr int kStageFloats = 18 * 256;   // 18 KiB of slots per workgroup
constexpr int kMaxStageSlots = 32;

struct Stage {
    float* data;        // slots of `size` floats: cols rows of D, then cols lse
    long long* base;    // [kMaxStageSlots]: partial index of a slot's row 0
    long long stride;   // partial indices between a slot's rows
    int cols, size;     // rows per slot, floats per slot (a multiple of 4)
    int slots;          // slots filled before a bulk store
    int n;              // slots filled (workgroup-uniform)
};

// Every wave of the workgroup writes a share of the n staged slots to the
// partials (row rr of slot j at partial index base[j] + rr * stride); the
// caller has passed a barrier since the slots were written.
template <int D, int WAVES>
__device__ __forceinline__ void store_staged(const DecodeArgs& a, Stage& st) {
    const int tid = threadIdx.x;
    const int per = st.cols * D / 4;   // float4s of one slot's rows
#pragma unroll 1
    for (int j = 0; j < st.n; ++j) {
        const float* slot = st.data + j * st.size;
        const long long base = st.base[j];
#pragma unroll 1
        for (int q = tid; q < per; q += 64 * WAVES) {
            const int rr = q / (D / 4), d4 = q % (D / 4);
            *reinterpret_cast<f32x4*>(a.part_out + (base + rr * st.stride) * D + 4 * d4) =
                *reinterpret_cast<const f32x4*>(slot + rr * D + 4 * d4);
        }
        if (tid < st.cols) a.part_lse[base + tid * st.stride] = slot[st.cols * D + tid];
    }
    st.n = 0;
}

// Attention of sequence b (L cached tokens), kv-head h, over its logical
// blocks [j0, j1) by the workgroup's WAVES waves (j0 < j1).  Wave w takes
// blocks j0 + w, j0 + w + WAVES, ...; wave 0 combines and writes.
//
// PARTS: [j0, j1) is a run of consecutive fixed partitions of upw * WAVES
// blocks each (j0 on a partition boundary; only the last may be short), and
// every partition gets its own result, exactly the one a workgroup given
// that partition alone computes (the same blocks per wave, the same
// combine).  The waves stream on across partition boundaries -- the next
// blocks' loads are in flight while a finished partition's states are
// combined.
//
// stage (balanced kernel): partials go to its slots instead of part_out.
template <int D, int KIND, int BS, bool MQ, int WAVES, bool PARTS = false>
__device__ __forceinline__ void attend_range(const DecodeArgs& a, int b, int h, int L, int j0, int j1,
                                             const RangeOut& dst, float* smem, int upw = 0,
                                             Stage* stage = nullptr) {
    using T = Tile<KIND, D>;
    constexpr int kSubShift = BS == 64 ? 2 : BS == 32 ? 1 : 0;   // log2(sub-blocks per block)
    using QT = typename QType<KIND>::T;
    constexpr int NT = T::NT;

    // The thread index goes through an empty asm so that what is derived
    // from it (load offsets, column indices) is recomputed for every range
    // instead of being hoisted out of the balanced kernel's piece loop and
    // held in registers across it.
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, known uniform
    const int r = lane & 15, c = lane >> 4;
    const int Hkv = a.num_kv_heads, Hq = a.num_q_heads, G = Hq / Hkv;
    // column r: query qi (0 without MQ), q-head qh; its output / q row
    const int qn = MQ ? a.q_len : 1;
    const int qi = MQ ? r / G : 0;
    const int qh = h * G + (MQ ? r - qi * G : r);
    const bool col_ok = r < qn * G;
    const size_t row = ((size_t)b * qn + qi) * Hq + qh;
    // keys this column sees: 0 .. lim-1 (L without MQ)
    const int lim = L - qn + 1 + qi;
    const int lim_min = L - qn + 1;  // the smallest limit of the sequence's columns
    // this wave takes blocks j0 + w, j0 + w + WAVES, ...: n_mine of them
    const int n_mine = max(0, (j1 - j0 - w + WAVES - 1) / WAVES);

    typename T::QOp Q;
    T::load_q(Q, col_ok ? reinterpret_cast<const QT*>(a.q) + row * D : nullptr, c);
    const float kscale = KIND == KV_FP8 ? a.k_scale[h] : 1.0f;
    const float C = a.scale * kLog2e * kscale;  // raw score -> base-2 logit (C > 0)

    // block-table window of this wave: lane i holds the table entry of its
    // unit number tbase + i (and tbase + 64 + i in tnxt); unit u of the
    // sequence is sub-block u mod (BS / 16) of block u / (BS / 16)
    const int32_t* trow = a.block_table + (size_t)b * a.max_blocks_per_seq;
    const int ubase = j0 + w;  // the wave's unit i is ubase + i * WAVES
    int tbase = 0;
    int tcur = (lane < n_mine) ? trow[(ubase + lane * WAVES) >> kSubShift] : 0;
    int tnxt = (64 + lane < n_mine) ? trow[(ubase + (64 + lane) * WAVES) >> kSubShift] : 0;

    const char* kbase = reinterpret_cast<const char*>(a.k_cache) + (size_t)h * T::kTileBytes;
    const char* vbase = reinterpret_cast<const char*>(a.v_cache) + (size_t)h * T::kTileBytes;
    const size_t sub_stride = (size_t)Hkv * T::kTileBytes;   // bytes of one 16-token sub-block

    auto issue = [&](typename T::Regs& R, int i) {
        const int idx = i - tbase;
        const int phys = idx < 64 ? __builtin_amdgcn_readlane(tcur, idx)
                                  : __builtin_amdgcn_readlane(tnxt, idx - 64);
        const int sub = (ubase + i * WAVES) & ((1 << kSubShift) - 1);  // sub-block within the block
        const size_t off = (((size_t)phys << kSubShift) + sub) * sub_stride;
        T::load(R, kbase + off, vbase + off, r, c);
    };

    float m = -INFINITY, l = 0.f;
    f32x4 acc[NT];
#pragma unroll
    for (int n = 0; n < NT; ++n) acc[n] = zero4();

    // one block: scores, online softmax, PV
    auto consume = [&](typename T::Regs& R, int ii) {
        const int jj = j0 + w + ii * WAVES;  // logical block
        // raw scores; the softmax scale (times log2 e, times the fp8 K scale)
        // is applied to differences from the running max, so the maximum's
        // weight is exactly exp2(0) = 1
        T::settle(R);
        const f32x4 sc = T::qk(R, Q);
        float t[4] = {sc[0], sc[1], sc[2], sc[3]};
        const int valid = L - jj * kBS;
        if constexpr (MQ) {
            // causal: column r sees tokens below lim; V rows past L are masked
            if (lim_min - jj * kBS < kBS) {
                const int vcol = lim - jj * kBS;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (4 * c + e >= vcol) t[e] = -INFINITY;
                if (valid < kBS) T::mask_v(R, c, valid);
            }
        } else if (valid < kBS) {  // tail block: mask tokens past L (scores and V)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (4 * c + e >= valid) t[e] = -INFINITY;
            T::mask_v(R, c, valid);
        }
        float bm = fmaxf(fmaxf(t[0], t[1]), fmaxf(t[2], t[3]));
        bm = group_max4(bm);
        const float mn = fmaxf(m, bm);
        if (__ballot((mn - m) * C > kRescaleLog2)) {  // some column's max jumped: rescale
            // (MQ) a column with no key yet keeps alpha = 1 (its m and mn are -inf)
            const float alpha = (MQ && mn == -INFINITY) ? 1.f : fast_exp2((m - mn) * C);
            l *= alpha;
#pragma unroll
            for (int n = 0; n < NT; ++n) acc[n] *= alpha;
            m = mn;
        }
        // with MQ a column may have seen no key yet (m = -inf, all its
        // scores -inf): its weights must be 0, not exp2(NaN)
        const float mref = (MQ && m == -INFINITY) ? 0.f : m;
        float p[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) p[e] = fast_exp2((t[e] - mref) * C);
        l += (p[0] + p[1]) + (p[2] + p[3]);  // this lane's tokens; reduced after the loop
        T::pv(R, p, acc);
    };

    // PARTS: the partitions of the range, and the wave's blocks in all but the last
    const int nparts = PARTS ? (j1 - j0 + upw * WAVES - 1) / (upw * WAVES) : 1;
    const int n_full = PARTS ? (nparts - 1) * upw : 0;
    // PARTS: combine and reset the states of partition kk of the range, into
    // a stage slot (or, for a sequence of one partition written directly,
    // into the output)
    auto flush = [&](int kk) {
        if constexpr (PARTS) {
            static_assert(!MQ, "partition streaming: one query per sequence");
            float* s_acc = smem;                         // [WAVES][NT][64 lanes][4]
            float* s_m = smem + WAVES * NT * 4 * 64;     // [WAVES][16]
            float* s_l = s_m + WAVES * 16;               // [WAVES][16]
            const float lsum = group_sum4(l);
            __syncthreads();   // the previous partition's combine has read the LDS
#pragma unroll
            for (int n = 0; n < NT; ++n)
                *reinterpret_cast<f32x4*>(s_acc + ((w * NT + n) * 64 + lane) * 4) = acc[n];
            if (c == 0) {
                s_m[w * 16 + r] = m;
                s_l[w * 16 + r] = lsum;
            }
            __syncthreads();
            // each wave finishes NT / WAVES of the output tiles, in the order
            // of the single-partition combine: wave 0's state scaled first,
            // then waves 1, 2, ... added
            constexpr int TW = NT / WAVES;
            static_assert(NT % WAVES == 0, "whole output tiles per wave");
            float M = s_m[r];
#pragma unroll
            for (int v = 1; v < WAVES; ++v) M = fmaxf(M, s_m[v * 16 + r]);
            float f = fast_exp2((s_m[r] - M) * C);
            float lt = s_l[r] * f;
            f32x4 o[TW];
#pragma unroll
            for (int t = 0; t < TW; ++t)
                o[t] = *reinterpret_cast<const f32x4*>(s_acc + ((w * TW + t) * 64 + lane) * 4) * f;
#pragma unroll
            for (int v = 1; v < WAVES; ++v) {
                f = fast_exp2((s_m[v * 16 + r] - M) * C);
                lt += f * s_l[v * 16 + r];
#pragma unroll
                for (int t = 0; t < TW; ++t) {
                    const f32x4 sv = *reinterpret_cast<const f32x4*>(
                        s_acc + ((v * NT + w * TW + t) * 64 + lane) * 4);
#pragma unroll
                    for (int e = 0; e < 4; ++e) o[t][e] += f * sv[e];
                }
            }
            if (col_ok) {
                const float vscale = KIND == KV_FP8 ? a.v_scale[h] : 1.0f;
                const float inv = vscale / lt;
                if (dst.direct) {
#pragma unroll
                    for (int t = 0; t < TW; ++t)
                        store4(reinterpret_cast<QT*>(a.out) + row * D + 16 * (w * TW + t) + 4 * c,
                               o[t][0] * inv, o[t][1] * inv, o[t][2] * inv, o[t][3] * inv);
                } else {
                    float* slot = stage->data + stage->n * stage->size;
#pragma unroll
                    for (int t = 0; t < TW; ++t)
                        store4(slot + r * D + 16 * (w * TW + t) + 4 * c, o[t][0] * inv,
                               o[t][1] * inv, o[t][2] * inv, o[t][3] * inv);
                    if (w == 0 && c == 0) slot[stage->cols * D + r] = (M * C + fast_log2(lt)) * kLn2;
                }
            }
            if (!dst.direct && threadIdx.x == 0)   // partial index of the slot's row 0
                stage->base[stage->n] =
                    (long long)(dst.prow_base + (size_t)kk + (row - r) * dst.prow_stride);
            if (!dst.direct && ++stage->n == stage->slots) {
                __syncthreads();   // the slots are written
                store_staged<D, WAVES>(a, *stage);
            }
            m = -INFINITY;
            l = 0.f;
#pragma unroll
            for (int n = 0; n < NT; ++n) acc[n] = zero4();
        }
    };
    // PARTS: after the wave's block u, a partition other than the last ends
    auto boundary = [&](int u) {
        if constexpr (PARTS) {
            if (u >= 0 && u < n_full && (u + 1) % upw == 0) flush(u / upw);
        }
    };

    // Two-stage software pipeline: block i+1 is in flight while block i is
    // computed.  The steady-state loop issues its loads unconditionally and
    // the tail is peeled, so the compiler's in-order load counting never
    // waits for a prefetch before using older data, and no block is loaded
    // twice.
    if (n_mine > 0) {
        typename T::Regs b0, b1;
        issue(b0, 0);
        int i = 0;
        for (; i + 2 < n_mine; i += 2) {
            if (i - tbase >= 64) {  // slide the table window (uniform, once per 64 blocks)
                tbase += 64;
                tcur = tnxt;
                tnxt = (tbase + 64 + lane < n_mine) ? trow[(ubase + (tbase + 64 + lane) * WAVES) >> kSubShift] : 0;
            }
            boundary(i - 1);
            issue(b1, i + 1);
            consume(b0, i);
            boundary(i);
            issue(b0, i + 2);
            consume(b1, i + 1);
        }
        if (i - tbase >= 64) {
            tbase += 64;
            tcur = tnxt;
        }
        if (i + 1 < n_mine) {
            boundary(i - 1);
            issue(b1, i + 1);
            consume(b0, i);
            boundary(i);
            consume(b1, i + 1);
        } else {
            boundary(i - 1);
            consume(b0, i);
        }
        // a wave with no block in the last partition ends the one before here
        boundary(n_mine - 1);
    }
    if constexpr (PARTS) {
        flush(nparts - 1);
        return;
    }

    l = group_sum4(l);

    // ---- combine the waves' softmax states through LDS (wave 0 holds the result)
    if constexpr (WAVES > 1) {
        float* s_acc = smem;                                  // [WAVES-1][NT*4][64]
        float* s_m = smem + (WAVES - 1) * NT * 4 * 64;       // [WAVES-1][16]
        float* s_l = s_m + (WAVES - 1) * 16;                 // [WAVES-1][16]
        if (w > 0) {
#pragma unroll
            for (int n = 0; n < NT; ++n)
#pragma unroll
                for (int e = 0; e < 4; ++e) s_acc[((w - 1) * NT * 4 + n * 4 + e) * 64 + lane] = acc[n][e];
            if (c == 0) {
                s_m[(w - 1) * 16 + r] = m;
                s_l[(w - 1) * 16 + r] = l;
            }
        }
        __syncthreads();
        if (w == 0) {
            float M = m;
#pragma unroll
            for (int v = 0; v < WAVES - 1; ++v) M = fmaxf(M, s_m[v * 16 + r]);
            // M is finite unless (MQ) the column saw no key in any wave
            const float f0 = (MQ && M == -INFINITY) ? 0.f : fast_exp2((m - M) * C);
            l *= f0;
#pragma unroll
            for (int n = 0; n < NT; ++n) acc[n] *= f0;
#pragma unroll
            for (int v = 0; v < WAVES - 1; ++v) {
                // 0 for a wave without blocks (or, with MQ, without keys of this column)
                const float f = (MQ && M == -INFINITY) ? 0.f : fast_exp2((s_m[v * 16 + r] - M) * C);
                l += f * s_l[v * 16 + r];
#pragma unroll
                for (int n = 0; n < NT; ++n)
#pragma unroll
                    for (int e = 0; e < 4; ++e) acc[n][e] += f * s_acc[(v * NT * 4 + n * 4 + e) * 64 + lane];
            }
            m = M;
        }
    }

    if (stage != nullptr && !dst.direct) {   // uniform: the balanced kernel's partials go to a stage slot
        if (w == 0 && col_ok) {
            const float vscale = KIND == KV_FP8 ? a.v_scale[h] : 1.0f;
            const float inv = (MQ && !(l > 0.f)) ? 0.f : vscale / l;
            float* slot = stage->data + stage->n * stage->size;
#pragma unroll
            for (int n = 0; n < NT; ++n)
                store4(slot + r * D + 16 * n + 4 * c, acc[n][0] * inv, acc[n][1] * inv,
                       acc[n][2] * inv, acc[n][3] * inv);
            if (c == 0) slot[stage->cols * D + r] = (m * C + fast_log2(l)) * kLn2;
        }
        if (threadIdx.x == 0) stage->base[stage->n] = (long long)dst.prow_base;
        if (++stage->n == stage->slots) {
            __syncthreads();   // the slots are written
            store_staged<D, WAVES>(a, *stage);
        }
        return;
    }
    if (w > 0 || !col_ok) return;
    const float vscale = KIND == KV_FP8 ? a.v_scale[h] : 1.0f;
    // l = 0 only for a column that saw no key (MQ): zeros, lse -inf
    const float inv = (MQ && !(l > 0.f)) ? 0.f : vscale / l;
    if (dst.direct) {
        QT* o = reinterpret_cast<QT*>(a.out) + row * D;
#pragma unroll
        for (int n = 0; n < NT; ++n)
            store4(o + 16 * n + 4 * c, acc[n][0] * inv, acc[n][1] * inv, acc[n][2] * inv,
                   acc[n][3] * inv);
        return;
    }
    const size_t pidx = dst.prow_base + (dst.prow_stride ? row * dst.prow_stride : (size_t)r);
    float* po = a.part_out + pidx * D;
#pragma unroll
    for (int n = 0; n < NT; ++n)
        store4(po + 16 * n + 4 * c, acc[n][0] * inv, acc[n][1] * inv, acc[n][2] * inv,
               acc[n][3] * inv);
    if (c == 0) a.part_lse[pidx] = (m * C + fast_log2(l)) * kLn2;
}


// LDS floats of the waves' softmax-state combine (PARTS: every wave's
// state, then the stage slots and their partial indices)
template <int D, int KIND, int WAVES, bool PARTS = false, bool STAGED = false>
constexpr int combine_floats() {
    constexpr int f = (PARTS ? WAVES : WAVES - 1) * (Tile<KIND, D>::NT * 4 * 64 + 32) +
                      (STAGED ? kStageFloats + 2 * kMaxStageSlots : 0);
    return f > 1 ? f : 1;
}

// zeros for every column row of an empty sequence
template <int D, int KIND, bool MQ>
__device__ __forceinline__ void zero_rows(const DecodeArgs& a, int b, int h) {
    using T = Tile<KIND, D>;
    using QT = typename QType<KIND>::T;
    const int lane = threadIdx.x & 63;
    const int r = lane & 15, c = lane >> 4;
    const int Hq = a.num_q_heads, G = Hq / a.num_kv_heads;
    const int qn = MQ ? a.q_len : 1;
    const int qi = MQ ? r / G : 0;
    const int qh = h * G + (MQ ? r - qi * G : r);
    if (r >= qn * G) return;
    QT* o = reinterpret_cast<QT*>(a.out) + (((size_t)b * qn + qi) * Hq + qh) * D;
#pragma unroll
    for (int n = 0; n < T::NT; ++n) store4(o + 16 * n + 4 * c, 0.f, 0.f, 0.f, 0.f);
}

// inclusive prefix sum over the wave's 64 lanes: DPP row shifts within each
// 16-lane row, then row broadcasts carry the row totals upward (no LDS)
__device__ __forceinline__ int wave_incl_scan_i(int x) {
    x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);  // row_shr:1
    x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);  // row_shr:2
    x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);  // row_shr:4
    x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);  // row_shr:8
    x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15 -> rows 1, 3
    x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31 -> rows 2, 3
    return x;
}

// Longest sequences first (one-pass mode).  Workgroups are dispatched in
// index order, so with many more (sequence, kv-head) pairs than the device
// holds at once, a long sequence reached late leaves a tail of one long
// workgroup per compute unit; taking sequences longest first fills that
// tail with short ones.  Workgroup x takes the sequence of rank x / Hkv in
// the order (16-token units descending, index ascending), found by a radix
// selection the workgroup runs on its own: a histogram of the units names
// the rank's length class, a count over the sequence indices its member.
// The order is a permutation of the batch, the same in every workgroup;
// results do not depend on it.  At most kLptMaxSeqs sequences (four per
// thread of a 256-thread workgroup).
constexpr int kLptMaxSeqs = 1024;
constexpr int kLptBins = 1024;

// inclusive prefix sum over the workgroup's 256 threads (one value each)
template <int WAVES>
__device__ __forceinline__ int block_incl_scan_i(int x, int* s_wave) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    x = wave_incl_scan_i(x);
    if (lane == 63) s_wave[w] = x;
    __syncthreads();
    int before = 0;
#pragma unroll
    for (int v = 0; v < WAVES - 1; ++v)
        if (v < w) before += s_wave[v];
    return x + before;
}

template <int WAVES>
__device__ __forceinline__ int lpt_sequence(const DecodeArgs& a, int rank, int* s_tmp, int* s_pick) {
    static_assert(WAVES * 64 * 4 == kLptMaxSeqs && kLptBins == kLptMaxSeqs, "four items per thread");
    const int tid = threadIdx.x;
    const int B = a.num_seqs;
    int* s_hist = s_tmp;                 // [kLptBins]
    int* s_wave = s_tmp + kLptBins;      // [WAVES] per scan
    // this thread's sequences 4 tid .. 4 tid + 3 and their classes
    // (0 = longest; an index past the batch has none)
    int cls[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int i = 4 * tid + k;
        const int u = i < B ? (a.seq_lens[i] + kBS - 1) / kBS : -1;
        cls[k] = u < 0 ? -1 : kLptBins - 1 - min(u, kLptBins - 1);
        s_hist[4 * tid + k] = 0;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 4; ++k)
        if (cls[k] >= 0) atomicAdd(&s_hist[cls[k]], 1);
    __syncthreads();
    // classes 4 tid .. 4 tid + 3: the first whose running count passes rank
    int c[4], sum = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        c[k] = s_hist[4 * tid + k];
        sum += c[k];
    }
    int run = block_incl_scan_i<WAVES>(sum, s_wave) - sum;   // sequences in classes before 4 tid
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        if (run <= rank && rank < run + c[k]) {
            s_pick[0] = 4 * tid + k;   // the class
            s_pick[1] = rank - run;    // the member's place in it
        }
        run += c[k];
    }
    __syncthreads();
    const int K = s_pick[0], m = s_pick[1];
    // the m-th sequence of class K in index order
    int f[4], fsum = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        f[k] = cls[k] == K;
        fsum += f[k];
    }
    int before = block_incl_scan_i<WAVES>(fsum, s_wave + WAVES) - fsum;
    __syncthreads();   // every thread has read s_pick
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        if (f[k] && before == m) s_pick[2] = 4 * tid + k;
        before += f[k];
    }
    __syncthreads();
    return s_pick[2];
}

// One workgroup per (sequence, kv-head, partition): the one-pass mode
// (SPLIT = false, one partition) and the fixed-size split-KV mode.
template <int D, int KIND, int BS, bool SPLIT, bool MQ, int WAVES>
__global__ __launch_bounds__(64 * WAVES) void decode_kernel(const DecodeArgs a) {
    __shared__ float smem[combine_floats<D, KIND, WAVES>()];
    const int Hkv = a.num_kv_heads;
    const int h = blockIdx.x % Hkv;
    int b = blockIdx.x / Hkv;
    if constexpr (!SPLIT) {
        if (a.lpt_order) {   // uniform
            static_assert(combine_floats<D, KIND, WAVES>() >= kLptBins + 2 * WAVES, "LDS for the selection");
            __shared__ int s_pick[3];
            b = lpt_sequence<WAVES>(a, b, reinterpret_cast<int*>(smem), s_pick);
        }
    }
    const int part = blockIdx.y;
    const int L = a.seq_lens[b];
    const int nblk = (L + kBS - 1) / kBS;
    const int pb = SPLIT ? a.partition_blocks : nblk;
    const int j0 = part * pb;
    if (j0 >= nblk) {  // uniform over the workgroup
        if (!SPLIT && (threadIdx.x >> 6) == 0) zero_rows<D, KIND, MQ>(a, b, h);  // empty sequence
        return;
    }
    const int j1 = min(nblk, j0 + pb);
    // the one-pass mode, and a split sequence with a single partition when
    // asked to, write the output directly
    const int np = (nblk + pb - 1) / pb;
    RangeOut dst;
    dst.direct = !SPLIT || (np == 1 && a.single_direct);
    dst.prow_base = (size_t)(part + a.part_offset);
    dst.prow_stride = (size_t)a.max_parts;
    attend_range<D, KIND, BS, MQ, WAVES>(a, b, h, L, j0, j1, dst, smem);
}

// ---------------------------------------------------------------------------
// Balanced split-KV.  For one kv-head, the sequences' blocks laid end to end
// form W = sum_b ceil(L_b / 16) units; split s of S owns units
// [s*W/S, (s+1)*W/S), so every workgroup streams the same number of blocks
// whatever the length mix, and S * Hkv matches the workgroups the chip holds
// at once.  A split's range may cover pieces of several sequences; each piece
// is one attend_range.  A sequence owned by one split only is written
// directly; otherwise its pieces go to partial slot s + b (strictly
// increasing along the pieces, so unique, and contiguous for one sequence)
// and the first piece's workgroup of kv-head 0 records (first slot, count)
// for the merge.  The partials are staged in LDS and stored at the end.
// ---------------------------------------------------------------------------
// the split that owns unit x: the largest s with floor(s * W / S) <= x
__device__ __forceinline__ int owner(long long x, long long W, int S) {
    return (int)(((x + 1) * S - 1) / W);
}

//
// PARTS: the same balance over the batch's fixed partitions instead of its
// units: split s of S owns partitions [s*I/S, (s+1)*I/S) of the I =
// sum_b ceil(units_b / PB) partitions laid end to end, and streams each
// sequence's run of them with one attend_range.  Every partition's result is
// the fixed-partition kernel's, bit for bit, at partial slot p + part_offset;
// the workgroup only saves that kernel's per-partition pipeline refill.
template <int D, int KIND, int BS, bool MQ, int WAVES, bool PARTS = false>
__global__ __launch_bounds__(64 * WAVES) __attribute__((amdgpu_waves_per_eu(KIND != KV_F32 && !MQ ? 3 : 1))) void decode_balanced_kernel(const DecodeArgs a) {
    // the pieces' partials are staged in LDS and stored in bulk (with
    // several queries too: measured 112.8 against 116.8 us for 64 x 4 bf16
    // verify queries, once those kernels hold their accumulators in AGPRs)
    __shared__ __align__(16) float smem[combine_floats<D, KIND, WAVES, PARTS, true>()];
    const int lane = threadIdx.x & 63;
    const int s = blockIdx.x;
    const int h = blockIdx.y;
    const int B = a.num_seqs;
    const int G = a.num_q_heads / a.num_kv_heads;
    const int cols = (MQ ? a.q_len : 1) * G;   // output rows of one (piece, kv-head)
    const int PB = a.partition_blocks;
    // what the split balances: a sequence's units, or (PARTS) its partitions,
    // at most the grid_parts the caller's max_seq_len allows (the partial
    // slots there are)
    auto items = [&](int len) {
        const int u = (len + kBS - 1) / kBS;
        return PARTS ? min((u + PB - 1) / PB, a.grid_parts) : u;
    };

    // W = sum of ceil(L / 16) over the batch.  Lane l owns the contiguous run
    // of sequences [l*C, min(B, (l+1)*C)), C = ceil(B / 64), and sums its run
    // with eight loads in flight at a time; one wave scan then gives W and
    // the units before every run (all bookkeeping below is wave-uniform)
    const int C = (B + 63) >> 6;
    const int rb0 = lane * C;
    int mine = 0, len0 = 0;
    for (int k0 = 0; k0 < C; k0 += 8) {
        int v[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const int bb = rb0 + k0 + k;
            v[k] = (k0 + k < C && bb < B) ? a.seq_lens[bb] : 0;
        }
        if (k0 == 0) len0 = v[0];
#pragma unroll
        for (int k = 0; k < 8; ++k) mine += items(v[k]);
    }
    const int incl = wave_incl_scan_i(mine);
    const int W = __builtin_amdgcn_readlane(incl, 63);
    // with fewer units than workgroups only the first W split (one unit
    // each): every split in use then owns at least one unit, so the splits
    // from a sequence's first to its last all hold a piece of it
    const int S = min((int)gridDim.x, W);
    if (s >= S) return;  // uniform
    const int start = (int)((long long)s * W / S), end = (int)((long long)(s + 1) * W / S);

    // the run holding unit `start` (the first lane whose inclusive sum
    // passes it), then the sequence inside the run and the units before it;
    // lw keeps the lengths of 64 consecutive sequences from lb (lane i holds
    // L[lb + i]) for the piece loop
    const int ln = __builtin_ctzll(__ballot(incl > start));
    int cum = __builtin_amdgcn_readlane(incl - mine, ln);
    const int rb = ln * C;
    int b = rb, lb = 0, lw = len0;   // C == 1: lane i holds L[i] and run ln is sequence ln
    if (C > 1) {
        for (int k0 = 0; k0 < C; k0 += 64) {
            const int i = k0 + lane;
            const int Li = rb + i < B ? a.seq_lens[rb + i] : 0;
            const int ni = items(Li);
            const int inc2 = wave_incl_scan_i(ni);
            const unsigned long long hit = __ballot(i < C && rb + i < B && cum + inc2 > start);
            if (hit) {
                const int k = __builtin_ctzll(hit);
                b = rb + k0 + k;
                cum += __builtin_amdgcn_readlane(inc2 - ni, k);
                lb = rb + k0;
                lw = Li;
                break;
            }
            cum += __builtin_amdgcn_readlane(inc2, 63);
        }
    }

    const size_t slots = (size_t)gridDim.x + B;  // the merge's piece_slots
    int2* info = reinterpret_cast<int2*>(a.piece_info);
    Stage stage;   // staged partials
    {
        constexpr int kComb = (PARTS ? WAVES : WAVES - 1) * (Tile<KIND, D>::NT * 4 * 64 + 32);
        stage.data = smem + kComb;
        stage.base = reinterpret_cast<long long*>(smem + kComb + kStageFloats);
        stage.stride = PARTS ? a.max_parts : 1;
        stage.cols = cols;
        stage.size = cols * D + ((cols + 3) & ~3);
        stage.slots = min(kMaxStageSlots, kStageFloats / stage.size);
        stage.n = 0;
    }
    for (int pos = start; pos < end && b < B; ++b) {
        if (b - lb >= 64) {  // uniform: the next 64 lengths
            lb = b;
            lw = b + lane < B ? a.seq_lens[b + lane] : 0;
        }
        const int L = __builtin_amdgcn_readlane(lw, b - lb);
        const int n = items(L);
        if (n == 0) continue;  // an empty sequence owns no unit (the merge writes its zeros)
        const int seg_end = min(end, cum + n);
        if constexpr (PARTS) {
            // partitions [pos - cum, seg_end - cum) of sequence b
            const int p0 = pos - cum, p1 = seg_end - cum;
            RangeOut dst;
            dst.direct = n == 1 && a.single_direct;
            dst.prow_base = (size_t)(p0 + a.part_offset);
            dst.prow_stride = (size_t)a.max_parts;
            attend_range<D, KIND, BS, false, WAVES, true>(
                a, b, h, L, p0 * PB, min(p1 * PB, (L + kBS - 1) / kBS), dst, smem, PB / WAVES,
                &stage);
            pos = seg_end;
            cum += n;
            continue;
        }
        const int s_first = owner(cum, W, S), s_last = owner(cum + n - 1, W, S);
        if (h == 0 && s == s_first && threadIdx.x == 0)
            info[b] = make_int2(s_first + b, s_last - s_first + 1);
        RangeOut dst;
        dst.direct = s_first == s_last;
        dst.prow_base = (((size_t)h * slots) + (size_t)(s + b)) * cols;
        dst.prow_stride = 0;
        attend_range<D, KIND, BS, MQ, WAVES>(a, b, h, L, pos - cum, seg_end - cum, dst, smem, 0,
                                             &stage);
        __syncthreads();  // the next piece reuses the combine LDS
        pos = seg_end;
        cum += n;
    }
    if (stage.n > 0) {   // uniform
        __syncthreads();   // the last slots are written
        store_staged<D, WAVES>(a, stage);
    }
}

#ifndef PA_DECODE_WAVES
#define PA_DECODE_WAVES 4
#endif
constexpr int kWaves = PA_DECODE_WAVES;

// one-pass mode: longest sequences first when the grid is several times
// what the device holds (below that the order hardly matters)
#ifndef PA_LPT_MIN_WORKGROUPS
#define PA_LPT_MIN_WORKGROUPS 1024
#endif

template <int D, int KIND, int BS, bool SPLIT, bool MQ>
hipError_t launch_t(const DecodeArgs& a, hipStream_t s) {
    dim3 grid((unsigned)(a.num_seqs * a.num_kv_heads), SPLIT ? (unsigned)a.grid_parts : 1u);
    DecodeArgs k = a;
    k.lpt_order = !SPLIT && kWaves == 4 && a.num_seqs <= kLptMaxSeqs &&
                  (long long)a.num_seqs * a.num_kv_heads >= PA_LPT_MIN_WORKGROUPS;
    hipLaunchKernelGGL((decode_kernel<D, KIND, BS, SPLIT, MQ, kWaves>), grid,
                       dim3(64 * kWaves), 0, s, k);
    return hipGetLastError();
}

template <int D, int KIND, int BS, bool MQ, bool PARTS = false>
int splits_t(int num_kv_heads);

// Fixed partitions are streamed (several consecutive partitions per
// workgroup, balanced over the batch) when sequences may hold at least this
// many of them and a partition is a whole number of blocks per wave; not for
// fp32 KV, whose streaming kernel would hold one wave per SIMD.  Below it
// (batches of sequences a few partitions long) the dispatcher's balancing of
// one workgroup per partition measured faster.
#ifndef PA_STREAM_MIN_PARTS
#define PA_STREAM_MIN_PARTS 16
#endif
constexpr int kStreamMinParts = PA_STREAM_MIN_PARTS;

template <int D, int KIND, int BS, bool MQ>
hipError_t launch_mq(const DecodeArgs& a, hipStream_t s) {
    if (a.balanced) {
        dim3 grid((unsigned)a.grid_parts, (unsigned)a.num_kv_heads);
        hipLaunchKernelGGL((decode_balanced_kernel<D, KIND, BS, MQ, kWaves>), grid, dim3(64 * kWaves),
                           0, s, a);
        return hipGetLastError();
    }
    if constexpr (!MQ && KIND != KV_F32) {
        if (a.partition_blocks > 0 && a.partition_blocks % kWaves == 0 &&
            a.grid_parts >= kStreamMinParts) {
            const int splits = splits_t<D, KIND, BS, false, true>(a.num_kv_heads);
            if (splits < 1) return hipErrorInvalidValue;
            dim3 grid((unsigned)splits, (unsigned)a.num_kv_heads);
            hipLaunchKernelGGL((decode_balanced_kernel<D, KIND, BS, false, kWaves, true>), grid,
                               dim3(64 * kWaves), 0, s, a);
            return hipGetLastError();
        }
    }
    return a.partition_blocks > 0 ? launch_t<D, KIND, BS, true, MQ>(a, s)
                                  : launch_t<D, KIND, BS, false, MQ>(a, s);
}

// Balanced splits per kv-head: the workgroups of the balanced kernel that
// the device holds at once (occupancy x compute units), shared by the
// kv-heads, at most kMaxBalancedSplits.  Cached per device and variant.
template <int D, int KIND, int BS, bool MQ, bool PARTS>
int splits_t(int num_kv_heads) {
    constexpr int kDevices = 64;
    static int resident[kDevices];  // 0 = not yet known; a racing first call stores the same value
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return -1;
    int total = dev < kDevices ? resident[dev] : 0;
    if (total == 0) {
        int cus = 0, per_cu = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            return -1;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
                &per_cu, decode_balanced_kernel<D, KIND, BS, MQ, kWaves, PARTS>, 64 * kWaves, 0) != hipSuccess)
            return -1;
#ifdef PA_BALANCED_PER_CU
        per_cu = PA_BALANCED_PER_CU;  // build-time override of the occupancy
#endif
        total = cus * (per_cu > 0 ? per_cu : 1);
        if (dev < kDevices) resident[dev] = total;
    }
    const int sp = total / num_kv_heads;
    return sp < 1 ? 1 : (sp > kMaxBalancedSplits ? kMaxBalancedSplits : sp);
}

// one dispatch over (head_dim, kv dtype, block size, multi-query): F is
// called with the matching template arguments
template <bool MQ, class F>
auto dispatch(const DecodeArgs& a, F&& f) {
    auto by_bs = [&](auto d, auto kind) {
        constexpr int D = decltype(d)::value, K = decltype(kind)::value;
        auto by_mq = [&](auto bs) {
            constexpr int BS = decltype(bs)::value;
            return f.template operator()<D, K, BS, MQ>();
        };
        if (a.block_size == 64) return by_mq(std::integral_constant<int, 64>{});
        if (a.block_size == 32) return by_mq(std::integral_constant<int, 32>{});
        return by_mq(std::integral_constant<int, 16>{});
    };
    auto by_kind = [&](auto d) {
        switch (a.kv_dtype) {
            case 0: return by_bs(d, std::integral_constant<int, KV_F32>{});
            case 1: return by_bs(d, std::integral_constant<int, KV_BF16>{});
            default: return by_bs(d, std::integral_constant<int, KV_FP8>{});
        }
    };
    return a.head_dim == 64 ? by_kind(std::integral_constant<int, 64>{})
                            : by_kind(std::integral_constant<int, 128>{});
}

struct LaunchF {
    const DecodeArgs& a;
    hipStream_t s;
    template <int D, int K, int BS, bool MQ>
    hipError_t operator()() const { return launch_mq<D, K, BS, MQ>(a, s); }
};

struct SplitsF {
    const DecodeArgs& a;
    template <int D, int K, int BS, bool MQ>
    int operator()() const { return splits_t<D, K, BS, MQ>(a.num_kv_heads); }
};

}  // namespace
}  // namespace pa
