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
// Key units go two at a time (a step) through a ring of kStages LDS stages,
// filled by direct global-to-LDS copies (global_load_lds_dwordx4: 16 bytes
// per lane, no registers, no LDS stores) issued ahead of use, so blocks that
// several chunks share -- a common prefix -- are served by L2 while earlier
// steps are computed.  Steps go in groups of one or two: wait for this
// wave's copies of the group, one barrier (then every wave's copies have
// landed, and every wave is done with the stages the next copies
// overwrite), issue the copies of a later group, compute.  Per step and column
// tile: S^T = K . Q^T on MFMA in two products X and Y whose rows give each
// lane 8 consecutive tokens of one unit, online softmax per column (base 2),
// then O^T += V^T . P^T with each lane's V operand one 16-byte piece; the
// weights' column sums go through the MFMA too.  Steps wholly below a wave's
// diagonal skip the mask.  The weights of one column tile are computed while
// the output products of the previous one run on the matrix cores.
#include "device.h"
#include "launch.h"
#include "merge_row.h"
#include "tiles.h"

namespace pa {
namespace {

constexpr int kWaves = 4;

// LDS address (offset in the workgroup's LDS) of a __shared__ object
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// One direct copy: every lane's 16 bytes at base + voff go to LDS address
// m0 + 16 * lane (base and m0 wave-uniform; the compiler loads m0 for the
// operand).  Written as asm so that the compiler neither reorders memory
// accesses across it nor inserts load-counter waits for it: the kernel waits
// for its copies itself (wait_copies), and any wait the compiler places for
// its own loads can only be stricter.
__device__ __forceinline__ void copy16_to_lds(const char* base, uint32_t voff, uint32_t m0) {
    // (readfirstlane returns a signed int: each half goes through uint32_t so
    // that widening never sign-extends the low word into the high one)
    const uint64_t b = reinterpret_cast<uint64_t>(base);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)b);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
    const uint64_t ub = ((uint64_t)hi << 32) | lo;
    asm volatile("global_load_lds_dwordx4 %0, %1"
                 :: "v"(voff), "s"(ub), "{m0}"(__builtin_amdgcn_readfirstlane(m0)) : "memory");
}
// wait until at most N of this wave's vector-memory loads are outstanding
// (they complete in issue order)
template <int N>
__device__ __forceinline__ void wait_copies() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory");
}
// workgroup barrier that also orders memory accesses for the compiler; LDS
// reads issued before it have returned
__device__ __forceinline__ void barrier_lds() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

template <int D, int KIND, int BS, int NC>
__device__ __forceinline__ void prefill_rows(const PrefillArgs& a) {
    using T = Tile<KIND, D>;
    using QT = typename QType<KIND>::T;
    constexpr int NT = T::NT;
    constexpr int kSubShift = BS == 64 ? 2 : BS == 32 ? 1 : 0;   // log2(sub-blocks per block)
    constexpr int UB = T::kTileBytes;                       // one 16-token K (or V) tile
    constexpr int kCopies = UB / 1024;                       // 1 KiB copies per unit
    static_assert(UB % 1024 == 0 && kCopies * 4 % kWaves == 0, "whole copies per wave");
    constexpr int kPerWave = kCopies * 4 / kWaves;           // copies per wave and step
    // a stage: K of unit A, K of unit B, V of unit A, V of unit B
    constexpr int kOffKB = UB, kOffVA = 2 * UB, kOffVB = 3 * UB;
    constexpr int kStage = 4 * UB;
    // Steps are consumed in groups of kGroup under one barrier: two when four
    // stages fit in 64 KiB of LDS (the next group's copies fly while a group
    // is computed), else one, with copies kStages - 1 steps ahead.
    constexpr int kGroup = kStage * 4 <= 64 * 1024 ? 2 : 1;
    constexpr int kStages = kGroup == 2 ? 4 : kStage * 3 <= 64 * 1024 ? 3 : 2;
    static_assert(kStage * kStages <= 64 * 1024, "LDS ring fits 64 KiB");
    static_assert(kStages - 2 * kGroup >= 0 && kStages - 2 * kGroup <= 1, "copies in flight past a group");
    __shared__ __attribute__((aligned(16))) char stage[kStages][kStage];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    // wave index: uniform, and known to be below kWaves (which folds the
    // copy bookkeeping below into constants where the wave does not matter)
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6) & (kWaves - 1);
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
    // Row tiles later in a causal chunk see more keys.  The second half of
    // the grid's row tiles runs in reverse order, so workgroups y and
    // y + ny/2 -- placed on one compute unit when the dispatcher fills the
    // units in order twice over -- hold a long and a short tile.
    const int ny = gridDim.y, yh = ny / 2;
    const int ytile = ((int)blockIdx.y < yh || (ny & 1)) ? (int)blockIdx.y
                                                         : ny - 1 - ((int)blockIdx.y - yh);
    const int rho_wg = ytile * (16 * NC * kWaves);
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
    // Q has arrived before the loop (a wait the compiler sees, so it places
    // none of its own inside the loop, where it would also wait for copies)
    __builtin_amdgcn_s_waitcnt(0);

    // the table row, read-only for the whole kernel: through the constant
    // address space its uniform entries are scalar loads, which wait on their
    // own counter rather than behind the copies in flight
    const __attribute__((address_space(4))) int32_t* trow =
        (const __attribute__((address_space(4))) int32_t*)(a.block_table) +
        (size_t)ch * a.max_blocks_per_seq;
    const char* kbase = reinterpret_cast<const char*>(a.k_cache) + (size_t)h * T::kTileBytes;
    const char* vbase = reinterpret_cast<const char*>(a.v_cache) + (size_t)h * T::kTileBytes;
    // bytes between consecutive 16-token sub-blocks (a 32-bit quantity: Hkv tiles)
    const uint32_t sub_stride = (uint32_t)Hkv * (uint32_t)T::kTileBytes;

    // Copy k of this wave in a step is copy q = w + kWaves * k of the step's
    // 4 * kCopies: region q / kCopies (K of A, K of B, V of A, V of B), its
    // KiB q % kCopies.  voff: the lane's byte in the block tile (unit 0), as
    // the region's layout in LDS asks (K by k_lds_hbm, V by v_slot_hbm);
    // fixed for the whole loop.
    uint32_t voff[kPerWave];
#pragma unroll
    for (int k = 0; k < kPerWave; ++k) {
        const int q = w + kWaves * k, reg = q / kCopies;
        const int b = (q % kCopies) * 1024 + lane * 16;   // byte of the unit's LDS copy
        voff[k] = reg < 2 ? (uint32_t)k_lds_hbm<T>(b) : (uint32_t)T::v_slot_hbm(b / 16);
    }
    const int nsteps = (nblk - ubeg + 1) / 2;
    // the physical blocks of step t's units (a missing second unit re-reads
    // the first, which the consumer masks); uniform, so scalar loads
    auto phys_of = [&](int t, int& pa, int& pb) {
        const int ja = ubeg + 2 * t, jb = min(ja + 1, nblk - 1);
        pa = trow[(unsigned)ja >> kSubShift];
        pb = trow[(unsigned)jb >> kSubShift];
    };
    auto copy_step = [&](int t, int pa, int pb) {
        const int ja = ubeg + 2 * t, jb = min(ja + 1, nblk - 1);
        char* st = stage[t % kStages];
        // sub-block index of each unit: block << kSubShift | unit within it
        // (block indices are >= 0)
        constexpr uint32_t kSubMask = (1u << kSubShift) - 1;
        const uint64_t oa = (uint64_t)(((uint32_t)pa << kSubShift) | ((uint32_t)ja & kSubMask)) * sub_stride;
        const uint64_t ob = (uint64_t)(((uint32_t)pb << kSubShift) | ((uint32_t)jb & kSubMask)) * sub_stride;
#pragma unroll
        for (int k = 0; k < kPerWave; ++k) {
            const int q = w + kWaves * k, reg = q / kCopies;
            const char* base = (reg < 2 ? kbase : vbase) + ((reg & 1) ? ob : oa);
            const int dst = (reg == 0 ? 0 : reg == 1 ? kOffKB : reg == 2 ? kOffVA : kOffVB) +
                            (q % kCopies) * 1024;
            copy16_to_lds(base, voff[k], lds_addr(st + dst));
        }
    };

    // m: running max (raw score units); accl: the weights' column sums,
    // accumulated by MFMA (every element of a lane's accl holds its column's sum);
    // thr = m + kRescaleLog2 / C, the score past which a rescale is due, and
    // mc = m * C, both updated only when m changes
    float m[NC], thr[NC], mcs[NC];
    const float dthr = kRescaleLog2 / C;
    f32x4 accl[NC];
    f32x4 acc[NC][NT];
#pragma unroll
    for (int ct = 0; ct < NC; ++ct) {
        m[ct] = -INFINITY;
        thr[ct] = -INFINITY;
        mcs[ct] = -INFINITY;
        accl[ct] = zero4();
#pragma unroll
        for (int n = 0; n < NT; ++n) acc[ct][n] = zero4();
    }

    // The two units of a step (jA, jA+1) against every column tile of this
    // wave: 8 scores per lane (tokens 8(c & 1) .. +7 of unit c >> 1), one
    // online-softmax round over 32 keys, one K=32 MFMA per output tile.  A
    // unit the wave does not need (past its diagonal, or past the sequence)
    // has all its scores masked to -inf and its V zeroed, so it adds exactly
    // nothing.
    auto consume = [&](int buf, int jA) {
        const char* st = stage[buf];
        typename T::KRegs X, Y;
        load_k_xy<T>(X, Y, st, st + kOffKB, r, c);
        typename T::VOp V;
        T::load_v_xy(V, st + ((c >> 1) ? kOffVB : kOffVA), r, c);
        const int jB = jA + 1;
        const bool needB = jB < w_nblk;
        const int validA = kend - jA * kBS;
        const int validB = needB ? kend - jB * kBS : 0;
        if (validA < kBS || validB < kBS) T::mask_v_xy(V, c, (c >> 1) ? validB : validA);  // slots past L
        const bool diag = jB >= full_end || !needB;
        const bool unit_ok = (c >> 1) == 0 || needB;
        const int kp0 = (jA + (c >> 1)) * kBS + 8 * (c & 1);   // key position of this lane's t[0]
        // the score products of every column tile first (independent MFMA
        // chains back to back), then the softmax and output products
        f32x4 sxa[NC], sya[NC];
#pragma unroll
        for (int ct = 0; ct < NC; ++ct) {
            sxa[ct] = T::qk(X, Q[ct]);   // raw scores, as in decode
            sya[ct] = T::qk(Y, Q[ct]);
        }
        // in three passes over the column tiles -- causal mask, running max
        // (with its rare rescale branch), then the weights and output products
        // -- so that the last pass is one branch-free block in which the
        // weights of one tile are computed while the products of the previous
        // tile run on the matrix cores
        float t[NC][8];
#pragma unroll
        for (int ct = 0; ct < NC; ++ct) {
            t[ct][0] = sxa[ct][0]; t[ct][1] = sxa[ct][1]; t[ct][2] = sxa[ct][2]; t[ct][3] = sxa[ct][3];
            t[ct][4] = sya[ct][0]; t[ct][5] = sya[ct][1]; t[ct][6] = sya[ct][2]; t[ct][7] = sya[ct][3];
        }
        if (diag) {
#pragma unroll
            for (int ct = 0; ct < NC; ++ct)
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    if (!unit_ok || kp0 + e > pos[ct]) t[ct][e] = -INFINITY;
        }
#pragma unroll
        for (int ct = 0; ct < NC; ++ct) {
            // each lane tests its own 8 scores against the column's running
            // max; only when one of them jumps by more than the threshold
            // (which is when the column max does) is the column max reduced
            // over the lane groups and the state rescaled
            const float* tc = t[ct];
            // (nested so that it compiles to three max3 and one max)
            const float bm = fmaxf(fmaxf(fmaxf(fmaxf(fmaxf(tc[0], tc[1]), tc[2]),
                                               fmaxf(fmaxf(tc[3], tc[4]), tc[5])), tc[6]), tc[7]);
            if (__ballot(bm > thr[ct])) {
                const float mn = fmaxf(m[ct], group_max4(bm));
                const float alpha = fast_exp2((m[ct] - mn) * C);
                accl[ct] *= alpha;
#pragma unroll
                for (int n = 0; n < NT; ++n) acc[ct][n] *= alpha;
                m[ct] = mn;
                thr[ct] = mn + dthr;
                mcs[ct] = mn * C;
            }
        }
        // Raised wave priority over that block: the compute unit's arbiter
        // then prefers this wave's output products and weights over the other
        // wave of the SIMD (another workgroup's), whose score products or
        // max pass fill the gaps; measured faster than no priority and than
        // raising it for the score products too.
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int ct = 0; ct < NC; ++ct) {
            // exp2(t * C - m * C) as one FMA per weight: at the maximum it
            // leaves the rounding error of m * C, far below bf16's resolution,
            // so the packed weight is exactly 1 there and the normaliser (the
            // sum of the packed weights) matches it
            const float mc = mcs[ct];
            float p[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) p[e] = fast_exp2(fmaf(t[ct][e], C, -mc));
            const auto pk = T::pack_p2(p);
            T::pv_xy(V, pk, acc[ct]);
            T::lsum2(pk, accl[ct]);
        }
        if constexpr (KIND == KV_BF16 && D == 128 && NC == 2) {
            // schedule of that block: the first tile's weights (about 22
            // VALU and transcendental ops), then each of its NT + 1 products
            // followed by 3 ops of the second tile's weights, then the second
            // tile's products
            constexpr int kValuTrans = 0x002 | 0x400, kMfma = 0x008;
            __builtin_amdgcn_sched_group_barrier(kValuTrans, 22, 0);
#pragma unroll
            for (int i = 0; i < NT + 1; ++i) {
                __builtin_amdgcn_sched_group_barrier(kMfma, 1, 0);
                __builtin_amdgcn_sched_group_barrier(kValuTrans, 3, 0);
            }
            __builtin_amdgcn_sched_group_barrier(kMfma, NT + 1, 0);
        }
        __builtin_amdgcn_s_setprio(0);
    };

    // prologue: steps 0 .. kStages-kGroup-1 in flight
    int pa = 0, pb = 0;
    phys_of(0, pa, pb);
#pragma unroll
    for (int t = 0; t < kStages - kGroup; ++t) {
        if (t < nsteps) {
            copy_step(t, pa, pb);
            if (t + 1 < nsteps) phys_of(t + 1, pa, pb);
        }
    }
    for (int s = 0; s < nsteps; s += kGroup) {
        // this wave's copies of the group's steps are done once at most the
        // copies of later steps issued so far (kStages - 2 * kGroup steps,
        // fewer at the end) are outstanding
        if (kStages - 2 * kGroup == 1 && s + kGroup < nsteps) wait_copies<kPerWave>();
        else wait_copies<0>();
        barrier_lds();
        // the next copies overwrite the stages the previous group used
#pragma unroll
        for (int i = 0; i < kGroup; ++i) {
            const int t = s + kStages - kGroup + i;
            if (t < nsteps) {
                copy_step(t, pa, pb);
                if (t + 1 < nsteps) phys_of(t + 1, pa, pb);
            }
        }
#pragma unroll
        for (int i = 0; i < kGroup; ++i) {
            const int j0 = ubeg + 2 * (s + i);
            if (s + i < nsteps && j0 < w_nblk) consume((s + i) % kStages, j0);
        }
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

// The workgroup's rows, then (a mixed step) its share of the decode rows'
// split-KV merge: the partials were written by the decode kernel launched
// before this one, and the merge needs no launch of its own.  The merge rows
// go to the workgroups of the first half of the grid's row tiles (all of
// them when there is one), the causal tiles that see the fewest keys; a
// wave merges its rows as soon as its own are done.  Row r: wave r / n of
// eligible workgroup r % n.
template <int D, int KIND, int BS, int NC>
__global__ __launch_bounds__(64 * kWaves) void prefill_kernel(const PrefillArgs a) {
    prefill_rows<D, KIND, BS, NC>(a);
    if (a.merge_rows > 0) {
        const unsigned yh = gridDim.y / 2;
        if (yh == 0 || blockIdx.y < yh) {
            const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
            const unsigned ny = yh ? yh : gridDim.y;
            const unsigned n = gridDim.x * ny * gridDim.z;
            const unsigned wg = blockIdx.x + gridDim.x * (blockIdx.y + ny * blockIdx.z);
            const int hq = a.merge.num_q_heads;
            for (long long r = wg + (long long)n * w; r < a.merge_rows; r += (long long)n * kWaves)
                merge_row<D, KIND != KV_F32>(a.merge, (int)(r / hq), (int)(r % hq), threadIdx.x & 63);
        }
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
