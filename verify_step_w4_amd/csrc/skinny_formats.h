// skinny_formats.h — the plane decoders of the weight formats other than W4
// for the skinny GEMM template of skinny_gemm.h (internal to libvw4, not
// public).  gist.science, "BaseRT: …", section "メソドロジー": one GEMV per
// quantisation format, Q2 ... FP16.
//
//  * W8 splits the 8-bit code into a high and a low 4-bit plane (W4 layout);
//    W6 into a 2-bit high plane and a 4-bit low plane; W5 into a 1-bit high
//    plane and a 4-bit low plane; W3 into a 1-bit high plane and a 2-bit low
//    plane; W2 is one sign-magnitude 2-bit plane; 16-bit float weights (bf16,
//    fp16) are read as whole operands.
#pragma once

#include "skinny_gemm.h"

namespace vw4 {
namespace sg {

// 1-bit fields, quarter q of a dword: element j of the 8 at bit 4 q + j / 2
// (low half) or 16 + 4 q + j / 2 (high half), as bf16 pairs 128 + b.
__device__ __forceinline__ bf16x8 one8(uint32_t w, int q, uint32_t magic_v) {
    const uint32_t v = w >> (4 * q);
    u32x4 r;
    r.x = and_or(v, 0x00010001u, magic_v);
    r.y = and_or(v >> 1, 0x00010001u, magic_v);
    r.z = and_or(v >> 2, 0x00010001u, magic_v);
    r.w = and_or(v >> 3, 0x00010001u, magic_v);
    return __builtin_bit_cast(bf16x8, r);
}
// 8 two-bit fields (k half s of one row block of a 2-bit plane word: bits
// 8 s + 2 (j / 2) + 16 (j % 2) for element j) -> the 8 bf16 values 128 + hi.
__device__ __forceinline__ bf16x8 two8(uint32_t w, int s, uint32_t magic_v) {
    const uint32_t v = w >> (8 * s);
    u32x4 r;
    r.x = and_or(v, 0x00030003u, magic_v);
    r.y = and_or(v >> 2, 0x00030003u, magic_v);
    r.z = and_or(v >> 4, 0x00030003u, magic_v);
    r.w = and_or(v >> 6, 0x00030003u, magic_v);
    return __builtin_bit_cast(bf16x8, r);
}

// W2: c in [-1, 1], stored sign-magnitude in one 2-bit plane with the lane
// mapping of the W4 layout (one 16-byte word per lane and group, dword nb =
// row block nb, the field of element j of k half s at bits 8 s + 2 (j / 2) +
// 16 (j % 2); field bit 0 = (c != 0), bit 1 = (c < 0)).  Moved to bits 14-15
// of a bf16 (bit 14 alone is 2.0, bit 15 the sign), a field is the exact bf16
// value 2 c: no offset chain, so the fp32 sums stay on the scale of
// sum |x| rather than 129 sum |x|.  acc += (scale / 2) * sum x (2 c).
__device__ __forceinline__ bf16x8 sm8(uint32_t w, int s) {
    u32x4 r;
    r.x = (w << (14 - 8 * s)) & 0xC000C000u;
    r.y = (w << (12 - 8 * s)) & 0xC000C000u;
    r.z = (w << (10 - 8 * s)) & 0xC000C000u;
    r.w = (w << (8 - 8 * s)) & 0xC000C000u;
    return __builtin_bit_cast(bf16x8, r);
}
struct FmtW2 {
    static constexpr int NW = 1;
    __device__ static void base(const Planes& P, int64_t t, int G, int lane, const u32x4*& b0, const u32x4*& b1) {
        b0 = P.p0 + t * G * 64 + lane;
        b1 = b0;
    }
    __device__ static void load(u32x4 (&w)[NW], const u32x4* b0, const u32x4*, int64_t g) {
        w[0] = __builtin_nontemporal_load(b0 + g * 64);
    }
    __device__ static void group(const u32x4 (&w)[NW], bf16x8 a0, bf16x8 a1, uint2 sc, uint32_t, uint32_t,
                                 f32x4 (&acc)[4]) {
        const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
        f32x4 d[4];
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) d[nb] = mfma16(a1, sm8(w[0][nb], 1), mfma16(a0, sm8(w[0][nb], 0), zero));
        float f[4];
        scales4(sc, f);
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[nb][r] = fmaf(0.5f * f[nb], d[nb][r], acc[nb][r]);
    }
    __host__ __device__ static Planes expert(Planes P, int64_t e, int64_t w_estride) {
        P.p0 += e * (w_estride / 2);
        return P;
    }
};

// The two-chain form, for W8 (u = c + 128 up to 255: 128 + u is not exact in
// bf16): code u = 16 hi + lo over two 4-bit planes; with D_hi = sum x (128 +
// hi) and D_lo = sum x (128 + lo), 16 D_hi + D_lo = sum x (2304 + c), so
// sum x c = 16 (D_hi - 144 sum x) + D_lo: the high plane's chain starts from
// x . (-144) (NEG_PAIR).
template <class Derived>
struct TwoPlane {
    __device__ static void finish(const bf16x8 (&hb)[4][2], const bf16x8 (&lb)[4][2], bf16x8 a0, bf16x8 a1,
                                  uint2 sc, f32x4 (&acc)[4]) {
        const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
        const f32x4 off = mfma16(a1, pair8(Derived::NEG_PAIR), mfma16(a0, pair8(Derived::NEG_PAIR), zero));
        float f[4];
        scales4(sc, f);
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
            const f32x4 dh = mfma16(a1, hb[nb][1], mfma16(a0, hb[nb][0], off));
            const f32x4 dl = mfma16(a1, lb[nb][1], mfma16(a0, lb[nb][0], zero));
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[nb][r] = fmaf(f[nb], fmaf(Derived::R, dh[r], dl[r]), acc[nb][r]);
        }
    }
};

// W8: c in [-127, 127], u = c + 128 = 16 hi + lo; both planes in the W4 layout.
struct FmtW8 : TwoPlane<FmtW8> {
    static constexpr float R = 16.0f;
    static constexpr int NW = 4;
    static constexpr uint32_t NEG_PAIR = 0xC310C310u;   // two bf16 -144.0
    __device__ static void base(const Planes& P, int64_t t, int G, int lane, const u32x4*& b0, const u32x4*& b1) {
        b0 = P.p0 + t * G * 128 + lane;
        b1 = P.p1 + t * G * 128 + lane;
    }
    __device__ static void load(u32x4 (&w)[NW], const u32x4* b0, const u32x4* b1, int64_t g) {
        w[0] = __builtin_nontemporal_load(b0 + g * 128);
        w[1] = __builtin_nontemporal_load(b0 + g * 128 + 64);
        w[2] = __builtin_nontemporal_load(b1 + g * 128);
        w[3] = __builtin_nontemporal_load(b1 + g * 128 + 64);
    }
    __device__ static void group(const u32x4 (&w)[NW], bf16x8 a0, bf16x8 a1, uint2 sc, uint32_t kmask,
                                 uint32_t magic_v, f32x4 (&acc)[4]) {
        bf16x8 hb[4][2], lb[4][2];
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                hb[nb][s] = nib8(w[nb >> 1][2 * (nb & 1) + s], kmask, magic_v);
                lb[nb][s] = nib8(w[2 + (nb >> 1)][2 * (nb & 1) + s], kmask, magic_v);
            }
        finish(hb, lb, a0, a1, sc, acc);
    }
    __host__ __device__ static Planes expert(Planes P, int64_t e, int64_t w_estride) {
        P.p0 += e * w_estride;
        P.p1 += e * w_estride;
        return P;
    }
};

// Single-chain formats: a code u = c + bias < 128 split over a low plane of
// BL bits and a high plane.  Per bf16 pair both fields are moved into place
// (the low field to bits 0 .. BL-1 of each half, the high field just above),
// merged with a bit-field insert, and and-or'ed with the magic into the bf16
// pair 128 + u; one matrix-core chain per row block starts from
// x . (-(128 + bias)), and acc += scale * D as in W4.  Derived supplies
// merge8(w, nb, s, magic): the 8 operands of row block nb, k half s.
__device__ __forceinline__ uint32_t shr_signed(uint32_t v, int sh) {   // sh < 0: shift left
    return sh >= 0 ? v >> sh : v << -sh;
}
template <uint32_t LO_MASK, uint32_t U_MASK>
__device__ __forceinline__ uint32_t merge_pair(uint32_t lo_sh, uint32_t hi_sh, uint32_t magic_v) {
    const uint32_t t = (lo_sh & LO_MASK) | (hi_sh & ~LO_MASK);
    return and_or(t, U_MASK, magic_v);
}
template <class Derived>
struct SingleChain {
    template <int NWD>
    __device__ static void group(const u32x4 (&w)[NWD], bf16x8 a0, bf16x8 a1, uint2 sc, uint32_t, uint32_t magic_v,
                                 f32x4 (&acc)[4]) {
        const bf16x8 neg = pair8(Derived::NEG_PAIR);
        f32x4 off = {0.f, 0.f, 0.f, 0.f};
        off = mfma16(a0, neg, off);
        off = mfma16(a1, neg, off);
        f32x4 d[4];
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
            d[nb] = mfma16(a1, Derived::merge8(w, nb, 1, magic_v), mfma16(a0, Derived::merge8(w, nb, 0, magic_v), off));
        float f[4];
        scales4(sc, f);
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[nb][r] = fmaf(f[nb], d[nb][r], acc[nb][r]);
    }
};

// W6: c in [-31, 31], u = c + 32 = 16 hi + lo; lo in the W4 layout, hi in a
// 2-bit plane with the same lane mapping (one 16-byte word per lane and group,
// dword nb = row block nb, element j of k half s at bits 8 s + 2 (j / 2) +
// 16 (j % 2)).  Offset 160 = 128 + 32.
struct FmtW6 : SingleChain<FmtW6> {
    static constexpr int NW = 3;
    static constexpr uint32_t NEG_PAIR = 0xC320C320u;   // two bf16 -160.0
    __device__ static void base(const Planes& P, int64_t t, int G, int lane, const u32x4*& b0, const u32x4*& b1) {
        b0 = P.p0 + t * G * 64 + lane;
        b1 = P.p1 + t * G * 128 + lane;
    }
    __device__ static void load(u32x4 (&w)[NW], const u32x4* b0, const u32x4* b1, int64_t g) {
        w[0] = __builtin_nontemporal_load(b0 + g * 64);
        w[1] = __builtin_nontemporal_load(b1 + g * 128);
        w[2] = __builtin_nontemporal_load(b1 + g * 128 + 64);
    }
    __device__ static bf16x8 merge8(const u32x4 (&w)[NW], int nb, int s, uint32_t magic_v) {
        const uint32_t lo = w[1 + (nb >> 1)][2 * (nb & 1) + s], hi = w[0][nb];
        uint32_t r[4];
#pragma unroll
        for (int p = 0; p < 4; ++p)   // pair p: low nibbles at 4 p, high fields at 8 s + 2 p -> bits 4-5
            r[p] = merge_pair<0x000F000Fu, 0x003F003Fu>(lo >> (4 * p), shr_signed(hi, 8 * s + 2 * p - 4), magic_v);
        return __builtin_bit_cast(bf16x8, u32x4{r[0], r[1], r[2], r[3]});
    }
    __host__ __device__ static Planes expert(Planes P, int64_t e, int64_t w_estride) {
        P.p0 += e * (w_estride / 2);
        P.p1 += e * w_estride;
        return P;
    }
};

// W5: c in [-15, 15], u = c + 16 = 16 hi + lo with hi in {0, 1}; lo in the W4
// layout, hi in a 1-bit plane with the same lane mapping (8 bytes per lane and
// group: dword nb / 2 holds row blocks nb = 2 d and 2 d + 1, quarter
// q = 2 (nb & 1) + s of it the k half s, element j at bit 4 q + j / 2 +
// 16 (j % 2)).  Offset 144 = 128 + 16.
struct FmtW5 : SingleChain<FmtW5> {
    static constexpr int NW = 3;
    static constexpr uint32_t NEG_PAIR = 0xC310C310u;   // two bf16 -144.0
    __device__ static void base(const Planes& P, int64_t t, int G, int lane, const u32x4*& b0, const u32x4*& b1) {
        b0 = (const u32x4*)((const u32x2*)P.p0 + t * G * 64 + lane);   // the 1-bit plane in 8-byte units
        b1 = P.p1 + t * G * 128 + lane;
    }
    __device__ static void load(u32x4 (&w)[NW], const u32x4* b0, const u32x4* b1, int64_t g) {
        const u32x2 h = __builtin_nontemporal_load((const u32x2*)b0 + g * 64);
        w[0] = u32x4{h.x, h.y, 0u, 0u};
        w[1] = __builtin_nontemporal_load(b1 + g * 128);
        w[2] = __builtin_nontemporal_load(b1 + g * 128 + 64);
    }
    __device__ static bf16x8 merge8(const u32x4 (&w)[NW], int nb, int s, uint32_t magic_v) {
        const uint32_t lo = w[1 + (nb >> 1)][2 * (nb & 1) + s], hi = w[0][nb >> 1];
        const int q = 2 * (nb & 1) + s;
        uint32_t r[4];
#pragma unroll
        for (int p = 0; p < 4; ++p)   // pair p: low nibbles at 4 p, high bits at 4 q + p -> bit 4
            r[p] = merge_pair<0x000F000Fu, 0x001F001Fu>(lo >> (4 * p), shr_signed(hi, 4 * q + p - 4), magic_v);
        return __builtin_bit_cast(bf16x8, u32x4{r[0], r[1], r[2], r[3]});
    }
    __host__ __device__ static Planes expert(Planes P, int64_t e, int64_t w_estride) {
        P.p0 += e * (w_estride / 4);
        P.p1 += e * w_estride;
        return P;
    }
};

// W3: c in [-3, 3], u = c + 4 = 4 hi + lo with hi in {0, 1}; hi in the 1-bit
// plane of the W5 layout, lo in the 2-bit plane of the W2 layout.  Offset
// 132 = 128 + 4.
struct FmtW3 : SingleChain<FmtW3> {
    static constexpr int NW = 2;
    static constexpr uint32_t NEG_PAIR = 0xC304C304u;   // two bf16 -132.0
    __device__ static void base(const Planes& P, int64_t t, int G, int lane, const u32x4*& b0, const u32x4*& b1) {
        b0 = (const u32x4*)((const u32x2*)P.p0 + t * G * 64 + lane);   // the 1-bit plane in 8-byte units
        b1 = P.p1 + t * G * 64 + lane;
    }
    __device__ static void load(u32x4 (&w)[NW], const u32x4* b0, const u32x4* b1, int64_t g) {
        const u32x2 h = __builtin_nontemporal_load((const u32x2*)b0 + g * 64);
        w[0] = u32x4{h.x, h.y, 0u, 0u};
        w[1] = __builtin_nontemporal_load(b1 + g * 64);
    }
    __device__ static bf16x8 merge8(const u32x4 (&w)[NW], int nb, int s, uint32_t magic_v) {
        const uint32_t lo = w[1][nb], hi = w[0][nb >> 1];
        const int q = 2 * (nb & 1) + s;
        uint32_t r[4];
#pragma unroll
        for (int p = 0; p < 4; ++p)   // pair p: low fields at 8 s + 2 p -> bits 0-1, high bits at 4 q + p -> bit 2
            r[p] = merge_pair<0x00030003u, 0x00070007u>(lo >> (8 * s + 2 * p), shr_signed(hi, 4 * q + p - 2), magic_v);
        return __builtin_bit_cast(bf16x8, u32x4{r[0], r[1], r[2], r[3]});
    }
    __host__ __device__ static Planes expert(Planes P, int64_t e, int64_t w_estride) {
        P.p0 += e * (w_estride / 4);
        P.p1 += e * (w_estride / 2);
        return P;
    }
};

// 16-bit float weights, no scales.  Layout (vw4_w16_pack): per 64-row tile
// and K-group 8 KiB, eight 1 KiB words; word 2 nb + s of lane l = 16 kq + i
// holds the eight 16-bit weights of row 16 nb + i at k = 32 s + 8 kq + j,
// j = 0..7 -- exactly the B operand of one row block and k half.  Two groups
// in flight per lane (16 words, 64 registers).
//
// BF16: the words are the B operands as they stand; the products accumulate
// straight into acc (one matrix-core chain per row block).
struct FmtB16 {
    static constexpr int NW = 8;
    static constexpr int PF_GROUPS = 2;
    static constexpr bool NO_SCALES = true;
    __device__ static void base(const Planes& P, int64_t t, int G, int lane, const u32x4*& b0, const u32x4*& b1) {
        b0 = P.p0 + t * G * 512 + lane;
        b1 = b0;
    }
    __device__ static void load(u32x4 (&w)[NW], const u32x4* b0, const u32x4*, int64_t g) {
#pragma unroll
        for (int q = 0; q < NW; ++q) w[q] = __builtin_nontemporal_load(b0 + g * 512 + q * 64);
    }
    __device__ static void group(const u32x4 (&w)[NW], bf16x8 a0, bf16x8 a1, uint2, uint32_t, uint32_t,
                                 f32x4 (&acc)[4]) {
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
            acc[nb] = mfma16(a1, __builtin_bit_cast(bf16x8, w[2 * nb + 1]),
                             mfma16(a0, __builtin_bit_cast(bf16x8, w[2 * nb]), acc[nb]));
    }
    __host__ __device__ static Planes expert(Planes P, int64_t e, int64_t w_estride) {
        P.p0 += e * w_estride * 4;
        return P;
    }
};

// FP16: each weight w (11-bit significand) is split exactly into two bf16
// values, hi = w truncated to 8 significant bits and lo = w - hi (at most 3
// significant bits, so exact in bf16): hi is the top half of w's binary32
// form, lo the top half of the binary32 difference.  Both products with the
// bf16 activations are exact in fp32; the chain adds x . hi, then x . lo.
// (The word's dwords are copied to scalars first: a bit cast applied to a
// subscripted element of a vector value was compiled as a read of element 0.)
__device__ __forceinline__ void split_f16x8(u32x4 w, bf16x8& hi, bf16x8& lo) {
    const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
    uint32_t h[4], l[4];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        const float f0 = (float)__builtin_bit_cast(_Float16, (uint16_t)(wd[d] & 0xFFFFu));
        const float f1 = (float)__builtin_bit_cast(_Float16, (uint16_t)(wd[d] >> 16));
        const uint32_t u0 = __builtin_bit_cast(uint32_t, f0), u1 = __builtin_bit_cast(uint32_t, f1);
        const float r0 = f0 - __builtin_bit_cast(float, u0 & 0xFFFF0000u);
        const float r1 = f1 - __builtin_bit_cast(float, u1 & 0xFFFF0000u);
        h[d] = __builtin_amdgcn_perm(u1, u0, 0x07060302u);   // the high halves of f0 (low), f1 (high)
        l[d] = __builtin_amdgcn_perm(__builtin_bit_cast(uint32_t, r1), __builtin_bit_cast(uint32_t, r0), 0x07060302u);
    }
    hi = __builtin_bit_cast(bf16x8, u32x4{h[0], h[1], h[2], h[3]});
    lo = __builtin_bit_cast(bf16x8, u32x4{l[0], l[1], l[2], l[3]});
}
struct FmtF16 : FmtB16 {
    __device__ static void group(const u32x4 (&w)[NW], bf16x8 a0, bf16x8 a1, uint2, uint32_t, uint32_t,
                                 f32x4 (&acc)[4]) {
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
            bf16x8 h0, l0, h1, l1;
            split_f16x8(w[2 * nb], h0, l0);
            split_f16x8(w[2 * nb + 1], h1, l1);
            acc[nb] = mfma16(a1, l1, mfma16(a0, l0, mfma16(a1, h1, mfma16(a0, h0, acc[nb]))));
        }
    }
};

}  // namespace sg
}  // namespace vw4
