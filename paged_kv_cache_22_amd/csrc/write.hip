// KV-cache write: the K/V rows of new tokens scattered into their cache slots
// through a slot mapping (slot = physical block * 16 + offset), with optional
// fp8-e4m3 quantisation by a per-kv-head scale (vllm-metis 0.1.0, "Status":
// FP8 with one scale of amax / 448; vllm-metal architecture article, section
// 四: the cache is addressed through block tables, so a new token's position
// is a (block, offset) pair).
//
// One lane per (token, kv-head, 16-byte K chunk).  Lanes of a wave take 64
// consecutive tokens of one (kv-head, chunk): the new tokens of a prefill
// chunk occupy consecutive offsets of a block, so 16 neighbouring lanes fill
// one 256-byte K chunk run and whole 16-token V rows, and the stores
// coalesce.  A decode step writes one token per sequence into unrelated
// blocks: those stores are scattered whatever the mapping, and the call is
// dominated by launch latency.
#include "device.h"
#include "launch.h"

namespace pa {
namespace {

constexpr int kTokensPerWave = 64;
constexpr int kWavesPerGroup = 4;
constexpr int kBlock = 16;

// cache elements per 16-byte K chunk
template <int KV>
constexpr int chunk_elems() { return KV == KV_FP8 ? 16 : KV == KV_BF16 ? 8 : 4; }

// X input values -> fp32
template <int IN, int X>
__device__ __forceinline__ void load_row(const char* p, float (&x)[X]) {
    if constexpr (IN == KV_BF16) {
#pragma unroll
        for (int c = 0; c < X / 8; ++c) {
            const u32x4 w = ld16(p + 16 * c);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                x[8 * c + 2 * i] = bf16_lo(w[i]);
                x[8 * c + 2 * i + 1] = bf16_hi(w[i]);
            }
        }
    } else {
#pragma unroll
        for (int c = 0; c < X / 4; ++c) {
            const u32x4 w = ld16(p + 16 * c);
#pragma unroll
            for (int i = 0; i < 4; ++i) x[4 * c + i] = __uint_as_float(w[i]);
        }
    }
}

// x / scale (correctly rounded fp32 division), clamped to the e4m3fn range,
// then rounded to the nearest code, ties to even (hardware convert)
__device__ __forceinline__ float to_e4m3_range(float x, float scale) {
    const float y = x / scale;
    return fminf(fmaxf(y, -448.0f), 448.0f);
}

__device__ __forceinline__ unsigned pack_fp8x4(float a, float b, float c, float d) {
    const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    return (unsigned)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true);
}

template <int IN, int KV>
__global__ __launch_bounds__(kTokensPerWave* kWavesPerGroup) void write_kv_kernel(const WriteArgs a) {
    constexpr int X = chunk_elems<KV>();
    constexpr int kInBytes = IN == KV_BF16 ? 2 : 4;
    constexpr int kCacheBytes = KV == KV_FP8 ? 1 : KV == KV_BF16 ? 2 : 4;
    const int t = blockIdx.x * kTokensPerWave + threadIdx.x;
    const int hc = blockIdx.y * kWavesPerGroup + threadIdx.y;
    const int d = a.head_dim;
    const int nchunk = d / X;
    if (t >= a.num_tokens || hc >= a.num_kv_heads * nchunk) return;
    const int slot = a.slot_mapping[t];
    if (slot < 0 || slot >= a.num_blocks * kBlock) return;   // padding / outside the pool
    const int h = hc / nchunk;
    const int j = hc - h * nchunk;
    const int blk = slot / kBlock;
    const int off = slot - blk * kBlock;
    const size_t tile = (size_t)blk * a.num_kv_heads + h;   // (block, kv-head) tile

    const char* ksrc = static_cast<const char*>(a.key) +
                       ((size_t)t * a.key_stride + (size_t)h * d + (size_t)j * X) * kInBytes;
    const char* vsrc = static_cast<const char*>(a.value) +
                       ((size_t)t * a.value_stride + (size_t)h * d + (size_t)j * X) * kInBytes;
    float kx[X], vx[X];
    load_row<IN, X>(ksrc, kx);
    load_row<IN, X>(vsrc, vx);

    // K: chunk j of the tile, 16 bytes at token offset `off`
    char* kdst = static_cast<char*>(a.k_cache) + ((tile * nchunk + j) * kBlock + off) * 16;
    // V: dims j*X .. j*X+X-1 of the tile, one element per dim row at `off`
    char* vdst = static_cast<char*>(a.v_cache) + ((tile * d + (size_t)j * X) * kBlock + off) * kCacheBytes;

    if constexpr (KV == KV_FP8) {
        const float ks = a.k_scale[h];
        const float vs = a.v_scale[h];
        u32x4 kw;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            kw[i] = pack_fp8x4(to_e4m3_range(kx[4 * i], ks), to_e4m3_range(kx[4 * i + 1], ks),
                               to_e4m3_range(kx[4 * i + 2], ks), to_e4m3_range(kx[4 * i + 3], ks));
        *reinterpret_cast<u32x4*>(kdst) = kw;
#pragma unroll
        for (int i = 0; i < X / 4; ++i) {
            const unsigned w = pack_fp8x4(to_e4m3_range(vx[4 * i], vs), to_e4m3_range(vx[4 * i + 1], vs),
                                          to_e4m3_range(vx[4 * i + 2], vs), to_e4m3_range(vx[4 * i + 3], vs));
#pragma unroll
            for (int e = 0; e < 4; ++e)
                reinterpret_cast<uint8_t*>(vdst)[(4 * i + e) * kBlock] = (uint8_t)(w >> (8 * e));
        }
    } else if constexpr (KV == KV_BF16) {
        u32x4 kw;
#pragma unroll
        for (int i = 0; i < 4; ++i) kw[i] = (__float_as_uint(kx[2 * i]) >> 16) | (__float_as_uint(kx[2 * i + 1]) & 0xffff0000u);
        *reinterpret_cast<u32x4*>(kdst) = kw;
#pragma unroll
        for (int i = 0; i < X; ++i)
            reinterpret_cast<uint16_t*>(vdst)[i * kBlock] = (uint16_t)(__float_as_uint(vx[i]) >> 16);
    } else {
        u32x4 kw;
#pragma unroll
        for (int i = 0; i < 4; ++i) kw[i] = __float_as_uint(kx[i]);
        *reinterpret_cast<u32x4*>(kdst) = kw;
#pragma unroll
        for (int i = 0; i < X; ++i) reinterpret_cast<float*>(vdst)[i * kBlock] = vx[i];
    }
}

template <int IN, int KV>
hipError_t launch_t(const WriteArgs& a, hipStream_t s) {
    constexpr int X = chunk_elems<KV>();
    const int rows = a.num_kv_heads * (a.head_dim / X);
    dim3 grid((a.num_tokens + kTokensPerWave - 1) / kTokensPerWave,
              (rows + kWavesPerGroup - 1) / kWavesPerGroup);
    dim3 block(kTokensPerWave, kWavesPerGroup);
    hipLaunchKernelGGL((write_kv_kernel<IN, KV>), grid, block, 0, s, a);
    return hipGetLastError();
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
