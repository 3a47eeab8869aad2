// Per-KV-dtype access to one 16-token tile of the paged cache, in the MFMA
// operand layouts the attention kernels use.  gfx950 / CDNA4.
//
// The cache is made of 16-token sub-blocks: a cache block of BS tokens (16,
// 32 or 64) is BS / 16 consecutive sub-blocks, each holding the tiles of all
// kv-heads for its 16 tokens, so every (sub-block, kv-head) tile has the
// same shape whatever the block size.  A K tile is [D*eb/16 chunks][16
// tokens][16 bytes]: 16-byte chunks of consecutive dims with the token index
// inside each chunk.  A V tile is [D][16 tokens] (dim-major).  Both products
// of attention then read their MFMA operands as whole contiguous runs: for
// the score product S^T = K . Q^T (contraction over dims) lane (r, c) takes
// chunk 4i + c of token r, so one load instruction of the wave reads 1 KiB
// in one piece; for the output product O^T = V^T . P^T (contraction over
// tokens) lane (r, c) takes tokens 4c..4c+3 of dim 16n + r, so one
// instruction reads 16 whole dim rows.
#pragma once

#include "device.h"

namespace pa {

constexpr int kBS = 16;  // tokens per unit (MFMA tile height) = tokens of a sub-block

// ---------------------------------------------------------------------------
// Per-KV-dtype tile access.  For every kind:
//   Regs  the lane's share of one tile's K and V
//   QOp   the lane's share of Q^T, the B operand of the score MFMAs
//   load  issues the global loads of one 16-token tile (kt, vt: its start)
//   qk    S^T fragment: lane (r, c) gets scores of head r, tokens 4c..4c+3
//   pv    acc[n] += V^T[16n..16n+15, tokens] . P^T for this block
// and for prefill, which stages two 16-token units (A, B) of K and V in LDS
// and contracts over both in one K=32 product.  The score rows are ordered
// so that lane group c holds 8 consecutive tokens of one unit: row 4c + e of
// product X is token 8(c & 1) + e of unit c >> 1, and product Y the same
// tokens + 4.  A lane's 8 weights then pair with one contiguous 8-token
// piece of a V row, so the output product reads its operand in one piece:
//   KRegs / load_k_xy    the K operands of X and Y from the staged units: a
//                        unit's LDS copy holds the rows of X, then those of
//                        Y, each as [chunk][8 rows][16 bytes]; k_lds_hbm maps
//                        a byte of that copy to its place in the tile
//   v_slot_hbm           where the 16-byte piece of LDS slot s of a staged V
//                        unit comes from in the tile
// Both layouts are free of LDS bank conflicts for 16-byte reads, which gfx950
// serves 16 lanes at a time -- lanes 0-7 with 24-31 and 8-15 with 16-23, the
// same in the upper half-wave -- two lanes of one such pass conflicting when
// they hit the same 16-byte slot of a 256-byte bank row (measured with the
// SQ_LDS_BANK_CONFLICT counter on read patterns, then checked against the
// kernels' own counts).
//   VOp / load_v_xy      the lane's 8-token piece of dim rows 16n + r
//   mask_v_xy            zero the V of tokens at or past `valid`
//   pv_xy  acc[n] += V^T . P^T over the 32 tokens; lsum2 the weights' sums
// ---------------------------------------------------------------------------
template <int KIND, int D> struct Tile;

template <int D> struct Tile<KV_BF16, D> {
    static constexpr int kTileBytes = kBS * D * 2;    // one (sub-block, kv-head) tile
    static constexpr int KL = D / 32;  // 16-byte K loads per lane = score MFMAs
    static constexpr int NT = D / 16;  // 16-dim tiles of the output
    struct Regs { u32x4 k[KL]; u32x2 v[NT]; };
    struct QOp { u32x4 b[KL]; };

    // k-slot (c, e) of MFMA i stands for dim (4i + c) * 8 + e
    __device__ static void load_q(QOp& Q, const uint16_t* qrow, int c) {
#pragma unroll
        for (int i = 0; i < KL; ++i)
            Q.b[i] = qrow ? ld16(qrow + (4 * i + c) * 8) : u32x4{0u, 0u, 0u, 0u};
    }
    __device__ static void load(Regs& R, const char* kt, const char* vt, int r, int c) {
#pragma unroll
        for (int i = 0; i < KL; ++i) R.k[i] = ldkv16(kt + ((4 * i + c) * kBS + r) * 16);
#pragma unroll
        for (int n = 0; n < NT; ++n) R.v[n] = ldkv8(vt + (16 * n + r) * (kBS * 2) + c * 8);
    }
    __device__ static void settle(Regs&) {}   // loads land in MFMA layout
    struct KRegs { u32x4 k[KL]; };
    // V slot s = 2 * row + h holds tokens 8h..8h+7 of dim row
    __device__ static int v_slot_hbm(int slot) { return (slot >> 1) * (kBS * 2) + (slot & 1) * 16; }
    struct VOp { u32x4 v[NT]; };
    __device__ static void load_v_xy(VOp& V, const char* vu, int r, int c) {
#pragma unroll
        for (int n = 0; n < NT; ++n) V.v[n] = ld16(vu + (2 * (16 * n + r) + (c & 1)) * 16);
    }
    __device__ static void mask_v_xy(VOp& V, int c, int valid) {
        const int t0 = 8 * (c & 1);
        u32x4 mk;
#pragma unroll
        for (int k = 0; k < 4; ++k)
            mk[k] = (t0 + 2 * k < valid ? 0x0000ffffu : 0u) | (t0 + 2 * k + 1 < valid ? 0xffff0000u : 0u);
#pragma unroll
        for (int n = 0; n < NT; ++n) V.v[n] &= mk;
    }
    template <class KR>
    __device__ static f32x4 qk(const KR& R, const QOp& Q) {
        f32x4 s = zero4();
#pragma unroll
        for (int i = 0; i < KL; ++i) s = mfma_16x16x32_bf16(R.k[i], Q.b[i], s);
        return s;
    }
    __device__ static void mask_v(Regs& R, int c, int valid) {
        const int t0 = 4 * c;
        const unsigned mx = (t0 + 0 < valid ? 0x0000ffffu : 0u) | (t0 + 1 < valid ? 0xffff0000u : 0u);
        const unsigned my = (t0 + 2 < valid ? 0x0000ffffu : 0u) | (t0 + 3 < valid ? 0xffff0000u : 0u);
#pragma unroll
        for (int n = 0; n < NT; ++n) { R.v[n].x &= mx; R.v[n].y &= my; }
    }
    __device__ static void pv(const Regs& R, const float p[4], f32x4* acc) {
        u32x2 pb;
        pb.x = pack_bf16x2(p[0], p[1]);
        pb.y = pack_bf16x2(p[2], p[3]);
#pragma unroll
        for (int n = 0; n < NT; ++n) acc[n] = mfma_16x16x16_bf16(R.v[n], pb, acc[n]);
    }
    // the 8 weights of lane group c (tokens 8(c & 1) + e of unit c >> 1) as
    // the bf16 B operand of the K=32 output product
    using P2 = u32x4;
    __device__ static P2 pack_p2(const float p[8]) {
        return u32x4{pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]),
                     pack_bf16x2(p[4], p[5]), pack_bf16x2(p[6], p[7])};
    }
    __device__ static void pv_xy(const VOp& V, const P2& pb, f32x4* acc) {
#pragma unroll
        for (int n = 0; n < NT; ++n) acc[n] = mfma_16x16x32_bf16(V.v[n], pb, acc[n]);
    }
    // column sums of the (bf16) weights, the normaliser that matches pv_xy
    // exactly: an all-ones A operand, every D row holds the sum
    __device__ static void lsum2(const P2& pb, f32x4& accl) {
        constexpr unsigned kOnes = 0x3f803f80u;   // two bf16 1.0
        accl = mfma_16x16x32_bf16(u32x4{kOnes, kOnes, kOnes, kOnes}, pb, accl);
    }
};

template <int D> struct Tile<KV_FP8, D> {
    static constexpr int kTileBytes = kBS * D;
    static constexpr int KL = D / 64;  // 16-byte K loads per lane, 16 codes = two MFMAs each
    static constexpr int NT = D / 16;
    struct Regs { u32x4 k[KL]; unsigned v[NT]; };
    struct QOp { u32x4 b[2 * KL]; };

    // k-slot (c, e) of MFMA 2i + h stands for dim (4i + c) * 16 + 8h + e
    __device__ static void load_q(QOp& Q, const uint16_t* qrow, int c) {
#pragma unroll
        for (int i = 0; i < KL; ++i)
#pragma unroll
            for (int hh = 0; hh < 2; ++hh)
                Q.b[2 * i + hh] = qrow ? ld16(qrow + (4 * i + c) * 16 + 8 * hh)
                                       : u32x4{0u, 0u, 0u, 0u};
    }
    // V: lane (r, c) reads the unit's whole 16-token row of dim 16(4m + c) + r
    // as one 16-byte piece (word j = tokens 4j..4j+3); settle() then hands
    // word c of dim 16n + r to lane (r, c) as v[n], the layout pv() takes
    __device__ static void load(Regs& R, const char* kt, const char* vt, int r, int c) {
#pragma unroll
        for (int i = 0; i < KL; ++i) R.k[i] = ldkv16(kt + ((4 * i + c) * kBS + r) * 16);
#pragma unroll
        for (int m = 0; m < NT / 4; ++m) {
            const u32x4 w = ldkv16(vt + (16 * (4 * m + c) + r) * kBS);
            R.v[4 * m] = w.x;
            R.v[4 * m + 1] = w.y;
            R.v[4 * m + 2] = w.z;
            R.v[4 * m + 3] = w.w;
        }
    }
    __device__ static void settle(Regs& R) {
#pragma unroll
        for (int m = 0; m < NT / 4; ++m) group_transpose4(R.v + 4 * m);
    }
    struct KRegs { u32x4 k[KL]; };
    // V slot s is the unit's 16-token row of dim s (one 16-byte piece)
    __device__ static int v_slot_hbm(int slot) { return slot * kBS; }
    struct VOp { u32x2 v[NT]; };   // codes of tokens 8(c & 1) .. +7
    __device__ static void load_v_xy(VOp& V, const char* vu, int r, int c) {
#pragma unroll
        for (int n = 0; n < NT; ++n) V.v[n] = ld8(vu + (16 * n + r) * 16 + 8 * (c & 1));
    }
    __device__ static void mask_v_xy(VOp& V, int c, int valid) {
        const int t0 = 8 * (c & 1);
        unsigned lo = 0, hi = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            lo |= (t0 + e < valid ? 0xffu : 0u) << (8 * e);
            hi |= (t0 + 4 + e < valid ? 0xffu : 0u) << (8 * e);
        }
#pragma unroll
        for (int n = 0; n < NT; ++n) { V.v[n].x &= lo; V.v[n].y &= hi; }  // code 0x00 is +0
    }
    template <class KR>
    __device__ static f32x4 qk(const KR& R, const QOp& Q) {
        f32x4 s = zero4();
#pragma unroll
        for (int i = 0; i < KL; ++i) {
            const u32x2 a0 = fp8x4_to_bf16x4(R.k[i].x), a1 = fp8x4_to_bf16x4(R.k[i].y);
            const u32x2 a2 = fp8x4_to_bf16x4(R.k[i].z), a3 = fp8x4_to_bf16x4(R.k[i].w);
            s = mfma_16x16x32_bf16(u32x4{a0.x, a0.y, a1.x, a1.y}, Q.b[2 * i], s);
            s = mfma_16x16x32_bf16(u32x4{a2.x, a2.y, a3.x, a3.y}, Q.b[2 * i + 1], s);
        }
        return s;
    }
    __device__ static void mask_v(Regs& R, int c, int valid) {
        const int t0 = 4 * c;
        unsigned mk = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) mk |= (t0 + e < valid ? 0xffu : 0u) << (8 * e);
#pragma unroll
        for (int n = 0; n < NT; ++n) R.v[n] &= mk;  // code 0x00 is +0
    }
    __device__ static void pv(const Regs& R, const float p[4], f32x4* acc) {
        u32x2 pb;
        pb.x = pack_bf16x2(p[0], p[1]);
        pb.y = pack_bf16x2(p[2], p[3]);
#pragma unroll
        for (int n = 0; n < NT; ++n) acc[n] = mfma_16x16x16_bf16(fp8x4_to_bf16x4(R.v[n]), pb, acc[n]);
    }
    using P2 = u32x4;
    __device__ static P2 pack_p2(const float p[8]) {
        return u32x4{pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]),
                     pack_bf16x2(p[4], p[5]), pack_bf16x2(p[6], p[7])};
    }
    __device__ static void pv_xy(const VOp& V, const P2& pb, f32x4* acc) {
#pragma unroll
        for (int n = 0; n < NT; ++n) {
            const u32x2 a = fp8x4_to_bf16x4(V.v[n].x), b = fp8x4_to_bf16x4(V.v[n].y);
            acc[n] = mfma_16x16x32_bf16(u32x4{a.x, a.y, b.x, b.y}, pb, acc[n]);
        }
    }
    __device__ static void lsum2(const P2& pb, f32x4& accl) {
        constexpr unsigned kOnes = 0x3f803f80u;
        accl = mfma_16x16x32_bf16(u32x4{kOnes, kOnes, kOnes, kOnes}, pb, accl);
    }
};

template <int D> struct Tile<KV_F32, D> {
    static constexpr int kTileBytes = kBS * D * 4;
    static constexpr int KL = D / 16;  // 16-byte K loads per lane, four MFMAs each
    static constexpr int NT = D / 16;
    struct Regs { u32x4 k[KL]; u32x4 v[NT]; };
    struct QOp { u32x4 b[KL]; };

    // k-slot c of MFMA 4i + e stands for dim (4i + c) * 4 + e
    __device__ static void load_q(QOp& Q, const float* qrow, int c) {
#pragma unroll
        for (int i = 0; i < KL; ++i)
            Q.b[i] = qrow ? ld16(qrow + (4 * i + c) * 4) : u32x4{0u, 0u, 0u, 0u};
    }
    __device__ static void load(Regs& R, const char* kt, const char* vt, int r, int c) {
#pragma unroll
        for (int i = 0; i < KL; ++i) R.k[i] = ldkv16(kt + ((4 * i + c) * kBS + r) * 16);
#pragma unroll
        for (int n = 0; n < NT; ++n) R.v[n] = ldkv16(vt + (16 * n + r) * (kBS * 4) + c * 16);
    }
    __device__ static void settle(Regs&) {}
    struct KRegs { u32x4 k[KL]; };
    // V slot s = 4 * row + j holds tokens 4j..4j+3 of dim row
    __device__ static int v_slot_hbm(int slot) { return (slot >> 2) * (kBS * 4) + (slot & 3) * 16; }
    struct VOp { u32x4 a[NT], b[NT]; };   // tokens 8(c & 1) + 0..3 and + 4..7
    __device__ static void load_v_xy(VOp& V, const char* vu, int r, int c) {
#pragma unroll
        for (int n = 0; n < NT; ++n) {
            V.a[n] = ld16(vu + (4 * (16 * n + r) + 2 * (c & 1)) * 16);
            V.b[n] = ld16(vu + (4 * (16 * n + r) + 2 * (c & 1) + 1) * 16);
        }
    }
    __device__ static void mask_v_xy(VOp& V, int c, int valid) {
        const int t0 = 8 * (c & 1);
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
            for (int n = 0; n < NT; ++n) {
                if (t0 + e >= valid) V.a[n][e] = 0u;
                if (t0 + 4 + e >= valid) V.b[n][e] = 0u;
            }
    }
    template <class KR>
    __device__ static f32x4 qk(const KR& R, const QOp& Q) {
        f32x4 s = zero4();
#pragma unroll
        for (int i = 0; i < KL; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                s = mfma_16x16x4_f32(__uint_as_float(R.k[i][e]), __uint_as_float(Q.b[i][e]), s);
        return s;
    }
    __device__ static void mask_v(Regs& R, int c, int valid) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (4 * c + e >= valid)
#pragma unroll
                for (int n = 0; n < NT; ++n) R.v[n][e] = 0u;
    }
    // PV MFMA e: k-slot c stands for token 4c + e
    __device__ static void pv(const Regs& R, const float p[4], f32x4* acc) {
#pragma unroll
        for (int n = 0; n < NT; ++n)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                acc[n] = mfma_16x16x4_f32(__uint_as_float(R.v[n][e]), p[e], acc[n]);
    }
    struct P2 { float p[8]; };
    __device__ static P2 pack_p2(const float p[8]) {
        P2 r;
#pragma unroll
        for (int e = 0; e < 8; ++e) r.p[e] = p[e];
        return r;
    }
    // output MFMA e (e = 0..7): k-slot c stands for token 8(c & 1) + e of unit c >> 1
    __device__ static void pv_xy(const VOp& V, const P2& pk, f32x4* acc) {
#pragma unroll
        for (int n = 0; n < NT; ++n)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                acc[n] = mfma_16x16x4_f32(__uint_as_float(V.a[n][e]), pk.p[e], acc[n]);
                acc[n] = mfma_16x16x4_f32(__uint_as_float(V.b[n][e]), pk.p[4 + e], acc[n]);
            }
    }
    // column sums by MFMA with a ones operand, as for the other kinds
    __device__ static void lsum2(const P2& pk, f32x4& accl) {
#pragma unroll
        for (int e = 0; e < 8; ++e) accl = mfma_16x16x4_f32(1.0f, pk.p[e], accl);
    }
};

// K of one staged unit in LDS: the rows of X (tokens 0-3 and 8-11), then
// those of Y (tokens 4-7 and 12-15), each half [chunk][8 rows][16 bytes];
// row rr of a half is token 8 * ((rr >> 2) & 1) + (rr & 3), + 4 in Y.
// k_lds_hbm: the tile byte of LDS byte b of that copy.
template <class T>
__device__ __forceinline__ int k_lds_hbm(int b) {
    constexpr int HK = T::kTileBytes / 2;
    const int xy = b / HK, bb = b % HK;
    const int chunk = bb >> 7, rr = (bb >> 4) & 7;
    const int tok = 8 * ((rr >> 2) & 1) + (rr & 3) + 4 * xy;
    return chunk * (kBS * 16) + tok * 16;
}

// K operands of the score products X and Y from two staged units (kA, kB:
// their LDS copies).  Row 4c + e of X is token 8(c & 1) + e of unit c >> 1,
// row 4c + e of Y token 8(c & 1) + 4 + e: lane (r, c) reads chunk 4i + c of
// row r & 7 of the X (Y) half of unit r >> 3.
template <class T>
__device__ __forceinline__ void load_k_xy(typename T::KRegs& X, typename T::KRegs& Y,
                                          const char* kA, const char* kB, int r, int c) {
    constexpr int HK = T::kTileBytes / 2;
    const char* ku = (r >> 3) ? kB : kA;
#pragma unroll
    for (int i = 0; i < T::KL; ++i) {
        const int off = ((4 * i + c) * 8 + (r & 7)) * 16;
        X.k[i] = ld16(ku + off);
        Y.k[i] = ld16(ku + HK + off);
    }
}

template <int KIND> struct QType { using T = uint16_t; };   // bf16 bits
template <> struct QType<KV_F32> { using T = float; };

// store 4 consecutive output values of one row
__device__ __forceinline__ void store4(float* p, float a, float b, float c, float d) {
    *reinterpret_cast<f32x4*>(p) = f32x4{a, b, c, d};
}
__device__ __forceinline__ void store4(uint16_t* p, float a, float b, float c, float d) {
    u32x2 w;
    w.x = pack_bf16x2(a, b);
    w.y = pack_bf16x2(c, d);
    *reinterpret_cast<u32x2*>(p) = w;
}

}  // namespace pa
