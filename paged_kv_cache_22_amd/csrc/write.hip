// KV-cache write: the K/V rows of new tokens scattered into their cache slots
// through a slot mapping (slot = physical block * block size + offset), with optional
// fp8-e4m3 quantisation by a per-kv-head scale (vllm-metis 0.1.0, "Status":
// FP8 with one scale of amax / 448; vllm-metal architecture article, section
// 四: the cache is addressed through block tables, so a new token's position
// is a (block, offset) pair).
//
// Lane map.  A lane handles one 16-byte K chunk (X dims) of one kv-head for
// TPL tokens (1, 2 or 4: about 128 input bytes per lane, so each wave keeps
// many loads in flight).  A wave is 16 tokens x 4 (kv-head, chunk) slots,
// the slots consecutive in a token's row: each load instruction reads
// 64-byte runs of 16 token rows.  The new tokens of a prefill chunk occupy
// consecutive offsets of a block, so the 16 tokens of a K store fill one
// 256-byte chunk run and each V store one 16-token V row.  A decode step
// writes one token per sequence into unrelated blocks: those stores scatter
// whatever the map, and the call is dominated by launch latency.
#include "device.h"
#include "launch.h"

namespace pa {
namespace {

constexpr int kWaves = 4;
constexpr int kUnit = 16;   // tokens of a whole-unit group (one wave's 16 token rows)

// cache elements per 16-byte K chunk
template <int KV>
constexpr int chunk_elems() { return KV == KV_FP8 ? 16 : KV == KV_BF16 ? 8 : 4; }

// one input row piece (X values in 16-byte pieces) -> fp32
template <int IN, int X>
__device__ __forceinline__ void unpack_row(const u32x4 (&w)[X * (IN == KV_BF16 ? 2 : 4) / 16],
                                           float (&x)[X]) {
    if constexpr (IN == KV_BF16) {
#pragma unroll
        for (int c = 0; c < X / 8; ++c)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                x[8 * c + 2 * i] = bf16_lo(w[c][i]);
                x[8 * c + 2 * i + 1] = bf16_hi(w[c][i]);
            }
    } else {
#pragma unroll
        for (int c = 0; c < X / 4; ++c)
#pragma unroll
            for (int i = 0; i < 4; ++i) x[4 * c + i] = __uint_as_float(w[c][i]);
    }
}

// x / scale (correctly rounded fp32 division), clamped to the e4m3fn range,
// then rounded to the nearest code, ties to even (hardware convert)
__device__ __forceinline__ float to_e4m3_range(float x, float scale) {
    const float y = x / scale;
    return fminf(fmaxf(y, -448.0f), 448.0f);
}

// The same quotient without the division sequence.  Markstein's theorem: with
// r = RN(1/s) and q within an ulp of x/s, RN(q + r * (x - s * q)) = RN(x/s),
// the residual x - s * q being exact by fma.  It stays exact while it is a
// normal number, which scales in [2^-60, 2^60] guarantee for every quotient
// of magnitude 2^-12 or more; smaller quotients encode to a signed zero
// whatever their last bits (copysign keeps the zero's sign, which the
// correction would lose for x = -0).  Quotients past 2^16 saturate to 448
// either way, so q is clamped there first, which also keeps an infinite x
// from turning the residual into NaN.  Checked on the device against the
// division for every bf16 input and 1.5e10 random fp32 inputs over 109
// scales (powers of two, their neighbours, amax / 448 values): the same fp32
// quotient wherever it is 2^-12 or more, the same code everywhere.
struct Quotient {
    float s, r;
    bool fast;   // s in [2^-60, 2^60]; else the division
};
__device__ __forceinline__ Quotient make_quotient(float s) {
    Quotient q;
    q.s = s;
    q.r = 1.0f / s;
    q.fast = s >= 0x1p-60f && s <= 0x1p60f;
    return q;
}
__device__ __forceinline__ float to_e4m3_range_fast(float x, const Quotient& d) {
    const float q = fminf(fmaxf(x * d.r, -65536.0f), 65536.0f);
    const float e = fmaf(-q, d.s, x);
    const float y = __builtin_copysignf(fmaf(e, d.r, q), x);
    return fminf(fmaxf(y, -448.0f), 448.0f);
}

__device__ __forceinline__ unsigned pack_fp8x4(float a, float b, float c, float d) {
    const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    return (unsigned)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true);
}

// most tokens per lane: about 128 input bytes (K and V) in flight per lane
template <int IN, int KV>
constexpr int max_tokens_per_lane() {
    return 64 / (chunk_elems<KV>() * (IN == KV_BF16 ? 2 : 4));
}

// The V rows of one wave's transposed region, read back from the staged
// chunks: lane L stores bytes [16L, 16L + 16) of the 1 KiB region that the
// wave's four chunks cover in a whole 16-token block (rows of 16 tokens,
// dim-major).  Staged entry c*16 + r holds chunk c (16 bytes) of token r.
template <int KV>
__device__ __forceinline__ u32x4 transposed_v(const uint8_t* st, int L) {
    const int c = L >> 4;
    u32x4 o;
    if constexpr (KV == KV_BF16) {          // row = 16 tokens x 2 B: lane -> half a row
        const int e = (L >> 1) & 7, t0 = 8 * (L & 1);
        const uint8_t* p = st + (c * 16 + t0) * 16 + 2 * e;
#pragma unroll
        for (int m = 0; m < 4; ++m)
            o[m] = (unsigned)*reinterpret_cast<const uint16_t*>(p + (2 * m) * 16) |
                   ((unsigned)*reinterpret_cast<const uint16_t*>(p + (2 * m + 1) * 16) << 16);
    } else if constexpr (KV == KV_FP8) {    // row = 16 tokens x 1 B: lane -> one row
        const int e = L & 15;
        const uint8_t* p = st + c * 16 * 16 + e;
#pragma unroll
        for (int m = 0; m < 4; ++m)
            o[m] = (unsigned)p[(4 * m) * 16] | ((unsigned)p[(4 * m + 1) * 16] << 8) |
                   ((unsigned)p[(4 * m + 2) * 16] << 16) | ((unsigned)p[(4 * m + 3) * 16] << 24);
    } else {                                // row = 16 tokens x 4 B: lane -> a quarter row
        const int e = (L >> 2) & 3, t0 = 4 * (L & 3);
        const uint8_t* p = st + (c * 16 + t0) * 16 + 4 * e;
#pragma unroll
        for (int m = 0; m < 4; ++m) o[m] = *reinterpret_cast<const unsigned*>(p + m * 16);
    }
    return o;
}

template <int IN, int KV, int TPL>
__global__ __launch_bounds__(64 * kWaves) void write_kv_kernel(const WriteArgs a) {
    constexpr int X = chunk_elems<KV>();
    constexpr int kInBytes = IN == KV_BF16 ? 2 : 4;
    constexpr int kCacheBytes = KV == KV_FP8 ? 1 : KV == KV_BF16 ? 2 : 4;
    constexpr int kPieces = X * kInBytes / 16;                 // 16-byte input loads per row
    __shared__ u32x4 stage[kWaves][64];
    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
    const int r = lane & 15;
    // 1-D grid, chunk-slot groups fastest: neighbouring workgroups take the
    // neighbouring (kv-head, chunk) slots of the same tokens, whose cache
    // tiles and input bytes are adjacent in memory
    const int slot_groups = (a.num_kv_heads * (a.head_dim / X) + 4 * kWaves - 1) / (4 * kWaves);
    const int tg = blockIdx.x / slot_groups;
    const int hc0 = (blockIdx.x - tg * slot_groups) * (4 * kWaves) + w * 4;   // the wave's first slot
    const int hc = hc0 + (lane >> 4);
    const int d = a.head_dim;
    const int nchunk = d / X;
    // rows and nchunk are multiples of 4, so a wave's four slots are all
    // valid or all past the end (the return is wave-uniform) and share a head
    if (hc >= a.num_kv_heads * nchunk) return;
    const int h = hc / nchunk;
    const int j = hc - h * nchunk;
    const int tbase = tg * (16 * TPL) + r;
    // a block of 16, 32 or 64 tokens is 1, 2 or 4 consecutive 16-token
    // sub-blocks, so slot s is offset s mod 16 of sub-block s / 16 whatever
    // the block size
    const int cap = a.num_blocks * a.block_size;

    // All loads first and unconditionally, so that they are all in flight
    // together: a token past the end reads the last token's row (always
    // valid memory) and is dropped at the store.
    int slot[TPL];
    u32x4 kraw[TPL][kPieces], vraw[TPL][kPieces];
#pragma unroll
    for (int i = 0; i < TPL; ++i) {
        const int t = min(tbase + 16 * i, a.num_tokens - 1);
        slot[i] = a.slot_mapping[t];
        if (tbase + 16 * i >= a.num_tokens) slot[i] = -1;
    }
#pragma unroll
    for (int i = 0; i < TPL; ++i) {
        const int t = min(tbase + 16 * i, a.num_tokens - 1);
        const char* ks = static_cast<const char*>(a.key) +
                         ((size_t)t * a.key_stride + (size_t)h * d + (size_t)j * X) * kInBytes;
        const char* vs = static_cast<const char*>(a.value) +
                         ((size_t)t * a.value_stride + (size_t)h * d + (size_t)j * X) * kInBytes;
#pragma unroll
        for (int p = 0; p < kPieces; ++p) {
            kraw[i][p] = ld16(ks + 16 * p);
            vraw[i][p] = ld16(vs + 16 * p);
        }
    }

#pragma unroll
    for (int i = 0; i < TPL; ++i) {
        const bool live = slot[i] >= 0 && slot[i] < cap;       // not padding, inside the pool
        // Wave-uniform: are the wave's 16 tokens one whole 16-token unit of a
        // block, in order?  (lane 0 holds token r = 0; every lane group holds
        // the same tokens)
        const int s0 = __builtin_amdgcn_readfirstlane(slot[i]);
        const bool whole = __all(live && slot[i] == s0 + r) && (s0 % kUnit) == 0;

        // this token's K chunk and V elements, in cache encoding
        u32x4 kw, vw;
        if constexpr (KV == KV_FP8) {
            float kx[X], vx[X];
            unpack_row<IN, X>(kraw[i], kx);
            unpack_row<IN, X>(vraw[i], vx);
            const float ksc = a.k_scale[h];
            const float vsc = a.v_scale[h];
            const Quotient kd = make_quotient(ksc), vd = make_quotient(vsc);
            if (kd.fast && vd.fast) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    kw[q] = pack_fp8x4(to_e4m3_range_fast(kx[4 * q], kd), to_e4m3_range_fast(kx[4 * q + 1], kd),
                                       to_e4m3_range_fast(kx[4 * q + 2], kd), to_e4m3_range_fast(kx[4 * q + 3], kd));
                    vw[q] = pack_fp8x4(to_e4m3_range_fast(vx[4 * q], vd), to_e4m3_range_fast(vx[4 * q + 1], vd),
                                       to_e4m3_range_fast(vx[4 * q + 2], vd), to_e4m3_range_fast(vx[4 * q + 3], vd));
                }
            } else {  // scales outside [2^-60, 2^60]: the division itself
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    kw[q] = pack_fp8x4(to_e4m3_range(kx[4 * q], ksc), to_e4m3_range(kx[4 * q + 1], ksc),
                                       to_e4m3_range(kx[4 * q + 2], ksc), to_e4m3_range(kx[4 * q + 3], ksc));
                    vw[q] = pack_fp8x4(to_e4m3_range(vx[4 * q], vsc), to_e4m3_range(vx[4 * q + 1], vsc),
                                       to_e4m3_range(vx[4 * q + 2], vsc), to_e4m3_range(vx[4 * q + 3], vsc));
                }
            }
        } else {
            // bf16 / fp32: the input bits themselves (no arithmetic)
            kw = kraw[i][0];
            vw = vraw[i][0];
        }
        const int blk = slot[i] >> 4;         // sub-block
        const int off = slot[i] & (kUnit - 1);
        const size_t tile = (size_t)blk * a.num_kv_heads + h;    // (sub-block, kv-head) tile
        // K: chunk j of the tile, 16 bytes at token offset `off`
        if (live)
            *reinterpret_cast<u32x4*>(static_cast<char*>(a.k_cache) +
                                      ((tile * nchunk + j) * kUnit + off) * 16) = kw;
        if (whole) {
            // V through LDS: the wave's four chunks of the 16 tokens cover the
            // unit's 16 * element bytes of 4X dim rows (hc0's first dim ..
            // +4X) of this block's tile, 1 KiB in all; lane L stores 16 bytes:
            // piece L % eb of row L / eb (eb = element bytes)
            stage[w][lane] = vw;
            __builtin_amdgcn_wave_barrier();
            const u32x4 o = transposed_v<KV>(reinterpret_cast<const uint8_t*>(stage[w]), lane);
            __builtin_amdgcn_wave_barrier();
            const int j0 = (hc0 - h * nchunk);
            const size_t vrow = tile * d + (size_t)j0 * X + lane / kCacheBytes;
            char* vdst = static_cast<char*>(a.v_cache) + vrow * kUnit * kCacheBytes +
                         16 * (lane % kCacheBytes);
            *reinterpret_cast<u32x4*>(vdst) = o;
        } else if (live) {
            // V: dims j*X .. j*X+X-1 of the tile, one element per dim row at `off`
            char* vdst = static_cast<char*>(a.v_cache) +
                         ((tile * d + (size_t)j * X) * kUnit + off) * kCacheBytes;
#pragma unroll
            for (int e = 0; e < X; ++e) {
                if constexpr (KV == KV_FP8)
                    reinterpret_cast<uint8_t*>(vdst)[e * kUnit] = (uint8_t)(vw[e >> 2] >> (8 * (e & 3)));
                else if constexpr (KV == KV_BF16)
                    reinterpret_cast<uint16_t*>(vdst)[e * kUnit] = (uint16_t)(vw[e >> 1] >> (16 * (e & 1)));
                else
                    reinterpret_cast<unsigned*>(vdst)[e * kUnit] = vw[e];
            }
        }
    }
}

template <int IN, int KV, int TPL>
hipError_t launch_tpl(const WriteArgs& a, hipStream_t s, long long slot_groups) {
    const long long groups = ((long long)a.num_tokens + 16 * TPL - 1) / (16 * TPL) * slot_groups;
    hipLaunchKernelGGL((write_kv_kernel<IN, KV, TPL>), dim3((unsigned)groups), dim3(64 * kWaves), 0, s, a);
    return hipGetLastError();
}

// Several tokens per lane keep more bytes in flight per wave, one token per
// lane gives more workgroups: take the most tokens per lane that still
// leaves at least kMinGroups workgroups (8 per CU).
constexpr long long kMinGroups = 2048;

template <int IN, int KV>
hipError_t launch_t(const WriteArgs& a, hipStream_t s) {
    constexpr int X = chunk_elems<KV>();
    constexpr int kMax = max_tokens_per_lane<IN, KV>();
    const long long rows = (long long)a.num_kv_heads * (a.head_dim / X);
    const long long slot_groups = (rows + 4 * kWaves - 1) / (4 * kWaves);
    const long long groups_max = ((long long)a.num_tokens + 16 * kMax - 1) / (16 * kMax) * slot_groups;
    if (kMax > 1 && groups_max >= kMinGroups) return launch_tpl<IN, KV, kMax>(a, s, slot_groups);
    return launch_tpl<IN, KV, 1>(a, s, slot_groups);
}

}  // namespace

int launch_write_kv(const WriteArgs& a, void* stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    // bf16 and fp32 inputs travel as their own bits: a bf16 cache takes bf16
    // input, an fp32 cache fp32 input, an fp8 cache either
    if (a.kv_dtype == KV_FP8)
        return a.in_dtype == KV_BF16 ? launch_t<KV_BF16, KV_FP8>(a, s) : launch_t<KV_F32, KV_FP8>(a, s);
    if (a.kv_dtype == KV_BF16) return launch_t<KV_BF16, KV_BF16>(a, s);
    return launch_t<KV_F32, KV_F32>(a, s);
}

}  // namespace pa
