// Device-side building blocks shared by the libmoe kernels (gfx950 only).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "../../include/moe.h"

typedef int   i32x4  __attribute__((ext_vector_type(4)));
typedef int   i32x8  __attribute__((ext_vector_type(8)));
typedef float f32x4  __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

#define MOE_DEV __device__ __forceinline__

// Operand format selectors of V_MFMA_SCALE_F32_*_F8F6F4 (cbsz / blgp fields).
enum { MFMA_FMT_FP8 = 0, MFMA_FMT_FP4 = 4 };

// ---------------------------------------------------------------------------
// Scaled MFMA, 16x16x128. Measured operand layout on gfx950 (G = 4 lane groups):
//   lane l -> row (A) / column (B) l % 16, lane group g = l / 16.
//   FP4 operand: the lane's 16 bytes are K [32g, 32g+32), element 2i in the low nibble.
//   FP8 operand: bytes 0..15 are K [16g, 16g+16), bytes 16..31 are K [64+16g, 64+16g+16).
//   Scale: the lane's selected E8M0 byte scales K-block g (K [32g, 32g+32)) of its row.
//   Result: lane l holds D[4*(l/16) + v][l % 16], v = 0..3.
// ---------------------------------------------------------------------------
template <int FA, int FB, int SELA, int SELB>
MOE_DEV f32x4 mfma16x16x128(const i32x8& a, const i32x8& b, f32x4 c, int sa, int sb) {
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, FA, FB, SELA, sa, SELB, sb);
}

// ---------------------------------------------------------------------------
// Number conversions (OCP MX v1.0 element rules), all exact bit manipulation.
// ---------------------------------------------------------------------------

// fp32 (finite) -> E4M3 code, round to nearest even, saturating to +-448; the
// sign bit follows the input's sign bit.
MOE_DEV uint32_t f32_to_e4m3(float v) {
    uint32_t u = __float_as_uint(v);
    uint32_t s = (u >> 24) & 0x80u;
    uint32_t a = u & 0x7FFFFFFFu;
    uint32_t c;
    if (a < 0x3C800000u) {                         // |v| < 2^-6: subnormal grid, step 2^-9
        c = (uint32_t)__builtin_rintf(__uint_as_float(a) * 512.0f);
    } else {
        uint32_t r = a + 0x7FFFFu + ((a >> 20) & 1u);  // RNE to 3 mantissa bits
        c = (r >> 20) - (120u << 3);               // rebias exponent 127 -> 7
        c = c > 0x7Eu ? 0x7Eu : c;
    }
    return s | c;
}

// fp32 (finite) -> E2M1 code (0..15), round to nearest even, saturating to +-6.
MOE_DEV uint32_t f32_to_e2m1(float v) {
    uint32_t u = __float_as_uint(v);
    uint32_t s = (u >> 28) & 0x8u;
    uint32_t a = u & 0x7FFFFFFFu;
    uint32_t c;
    if (a < 0x3F800000u) {                         // |v| < 1: subnormal grid, step 0.5
        c = (uint32_t)__builtin_rintf(__uint_as_float(a) * 2.0f);
    } else {
        uint32_t r = a + 0x1FFFFFu + ((a >> 22) & 1u);  // RNE to 1 mantissa bit
        c = (r >> 22) - (126u << 1);               // rebias exponent 127 -> 1
        c = c > 0x7u ? 0x7u : c;
    }
    return s | c;
}

// E8M0 scale code of a block from its amax (>= 0, finite).
//  OCP rule:  E = floor(log2 amax) - emax_elem, clamped to [-127, 127]; code = E + 127.
//  ceil rule: E = ceil(log2(amax / max_finite)).
// A zero or fp32-subnormal amax gives code 0.
template <int EMAX, uint32_t MAXMANT>
MOE_DEV uint32_t mx_scale_code(float amax, bool ceil_rule) {
    // ceil rule: amax <= max_finite * 2^(e - emax) iff its mantissa is at most
    // the largest element's, max_finite = (1 + MAXMANT / 2^23) * 2^EMAX; so the
    // exponent goes up by one iff the mantissa exceeds MAXMANT, which is the
    // carry out of the mantissa field when 2^23 - 1 - MAXMANT is added to the
    // bits (at most one carry: both terms are below 2^23)
    const uint32_t u = __float_as_uint(amax) + (ceil_rule ? 0x7FFFFFu - MAXMANT : 0u);
    // biased exponent minus EMAX, i.e. (e32 - 127 - EMAX) + 127; a zero or
    // subnormal amax (e32 = 0, or 1 after a carry) gives a negative code,
    // clamped to 0
    const int code = (int)(u >> 23) - EMAX;
    return (uint32_t)(code < 0 ? 0 : (code > 254 ? 254 : code));
}
// E4M3: emax 8, max 448 = 1.75 * 2^8 (mantissa 0x600000); E2M1: emax 2, max 6 = 1.5 * 2^2.
MOE_DEV uint32_t e4m3_scale_code(float amax, bool ceil_rule) { return mx_scale_code<8, 0x600000u>(amax, ceil_rule); }
MOE_DEV uint32_t e2m1_scale_code(float amax, bool ceil_rule) { return mx_scale_code<2, 0x400000u>(amax, ceil_rule); }

// 2^(127 - code): multiplying by it divides by the block scale, exactly.
MOE_DEV float inv_scale(uint32_t code) { return __uint_as_float((254u - code) << 23); }

// fp32 -> bf16 bits, round to nearest even (finite inputs).
MOE_DEV uint32_t f32_to_bf16(float v) {
    uint32_t u = __float_as_uint(v);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}
MOE_DEV float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// fp64 -> bf16 bits with a single rounding (nearest even): round to fp32 with
// round-to-odd (sticky last bit), then to bf16 with nearest-even. fp32 keeps
// 24 >= 8 + 2 significant bits, so the result equals direct rounding.
MOE_DEV uint32_t f64_to_bf16(double d) {
    float f = (float)d;
    if ((double)f != d) {
        uint32_t u = __float_as_uint(f);
        if ((u & 1u) == 0u) {
            // f was rounded to an even neighbour: step one ulp towards d
            bool mag_up = fabs(d) > fabs((double)f);
            u = mag_up ? u + 1u : u - 1u;
            if ((__float_as_uint(f) & 0x7FFFFFFFu) == 0u) u = (d < 0 ? 0x80000001u : 1u);
        }
        f = __uint_as_float(u);
    }
    return f32_to_bf16(f);
}

MOE_DEV float silu(float g) { return g / (1.0f + __expf(-g)); }

// Hardware conversions for the epilogues. Each gives the same bits as the
// software conversions above for every finite input (checked on 2^21 random
// and tie-case pairs): v_cvt_pk_fp8_f32 rounds to nearest even into OCP E4M3,
// and the clamp to +-448 first makes it saturate; v_cvt_pk_bf16_f32 rounds to
// nearest even.
MOE_DEV float e4m3_clamp(float v) { return __builtin_amdgcn_fmed3f(v, -448.0f, 448.0f); }
// codes of a, b in bytes 0, 1
// (the converter writes one 16-bit half of its destination and keeps the
// other: the first conversion's other half is don't-care, so it is given a
// register that dies there instead of a zeroed one)
MOE_DEV uint32_t e4m3x2(float a, float b) {
    const float ca = e4m3_clamp(a);
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(ca, e4m3_clamp(b), __float_as_int(ca), false) & 0xFFFFu;
}
// codes of a, b, c, d in bytes 0..3
MOE_DEV uint32_t e4m3x4(float a, float b, float c, float d) {
    const float ca = e4m3_clamp(a);
    const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(ca, e4m3_clamp(b), __float_as_int(ca), false);
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(e4m3_clamp(c), e4m3_clamp(d), lo, true);
}
typedef __bf16 moe_bf16x2 __attribute__((ext_vector_type(2)));
typedef float moe_f32x2 __attribute__((ext_vector_type(2)));
// bf16 bits of a (low half) and b (high half)
MOE_DEV uint32_t bf16x2(float a, float b) {
    const moe_f32x2 v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, moe_bf16x2));
}
// SiLU with the hardware reciprocal (1 ulp) instead of a full division
MOE_DEV float silu_fast(float g) { return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)); }

// Gate activations of the W1 epilogue variants (MOE_ACT_*): Swish with slope
// beta, the exact GELU z * Phi(z), and the squared ReLU. act_and_grad also
// gives da/dz for the backward.
MOE_DEV float gelu_cdf(float z) { return 0.5f * (1.0f + erff(z * 0.70710678118654752f)); }
MOE_DEV float act_value(float z, int act, float beta) {
    if (act == MOE_ACT_GEGLU) return z * gelu_cdf(z);
    if (act == MOE_ACT_SRELU) { const float r = fmaxf(z, 0.0f); return r * r; }
    return z / (1.0f + __expf(-beta * z));
}
MOE_DEV void act_and_grad(float z, int act, float beta, float& a, float& da) {
    if (act == MOE_ACT_GEGLU) {
        const float cdf = gelu_cdf(z);
        a = z * cdf;
        da = cdf + z * (0.39894228040143268f * __expf(-0.5f * z * z));
    } else if (act == MOE_ACT_SRELU) {
        const float r = fmaxf(z, 0.0f);
        a = r * r;
        da = 2.0f * r;
    } else {
        // the sigmoid with the hardware reciprocal (1 ulp) instead of a full
        // division; exp overflowing to inf gives s = 0, as the division does
        const float s = __builtin_amdgcn_rcpf(1.0f + __expf(-beta * z));
        a = z * s;
        da = s + beta * z * s * (1.0f - s);
    }
}

// f(std::integral_constant<int, i>) for i = 0 .. N-1, each with a
// compile-time index (register arrays indexed by it stay in registers, where
// an unrolled loop whose body is too large to unroll would index them at
// run time and move them to scratch memory).
template <int N, typename F, int I = 0>
MOE_DEV void static_for(F&& f) {
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        static_for<N, F, I + 1>(static_cast<F&&>(f));
    }
}

// Wave-wide helpers (wave64).
MOE_DEV float wave_max_xor(float v, int mask) { return fmaxf(v, __shfl_xor(v, mask, 64)); }

MOE_DEV int ceil_div(int a, int b) { return (a + b - 1) / b; }

// ---------------------------------------------------------------------------
// Wave64 reductions with DPP (no LDS traffic). The result is returned to every
// lane; the combination order is fixed, so sums are deterministic.
// ---------------------------------------------------------------------------
#define MOE_DPP(v, ctrl, rmask) \
    __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, v), \
                                                         __builtin_bit_cast(int, v), ctrl, rmask, 0xF, false))
#define MOE_DPP_XOR1 0xB1        // quad_perm(1,0,3,2)
#define MOE_DPP_XOR2 0x4E        // quad_perm(2,3,0,1)
#define MOE_DPP_HALF_MIRROR 0x141
#define MOE_DPP_MIRROR 0x140
#define MOE_DPP_BCAST15 0x142
#define MOE_DPP_BCAST31 0x143

MOE_DEV float wave_max(float v) {
    v = fmaxf(v, MOE_DPP(v, MOE_DPP_XOR1, 0xF));
    v = fmaxf(v, MOE_DPP(v, MOE_DPP_XOR2, 0xF));
    v = fmaxf(v, MOE_DPP(v, MOE_DPP_HALF_MIRROR, 0xF));
    v = fmaxf(v, MOE_DPP(v, MOE_DPP_MIRROR, 0xF));
    v = fmaxf(v, MOE_DPP(v, MOE_DPP_BCAST15, 0xA));
    v = fmaxf(v, MOE_DPP(v, MOE_DPP_BCAST31, 0xC));
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

MOE_DEV float wave_sum(float v) {
    v += MOE_DPP(v, MOE_DPP_XOR1, 0xF);
    v += MOE_DPP(v, MOE_DPP_XOR2, 0xF);
    v += MOE_DPP(v, MOE_DPP_HALF_MIRROR, 0xF);
    v += MOE_DPP(v, MOE_DPP_MIRROR, 0xF);
    v += MOE_DPP(v, MOE_DPP_BCAST15, 0xA);
    v += MOE_DPP(v, MOE_DPP_BCAST31, 0xC);
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

// Reductions over the 16 lanes of a DPP row (lanes 16r .. 16r+15); every lane
// of the row receives the row's result.
MOE_DEV float row16_max(float v) {
    v = fmaxf(v, MOE_DPP(v, MOE_DPP_XOR1, 0xF));
    v = fmaxf(v, MOE_DPP(v, MOE_DPP_XOR2, 0xF));
    v = fmaxf(v, MOE_DPP(v, MOE_DPP_HALF_MIRROR, 0xF));
    v = fmaxf(v, MOE_DPP(v, MOE_DPP_MIRROR, 0xF));
    return v;
}

// max over the 16 lanes of a DPP row of non-negative floats given as their
// bit patterns (integer order = float order for them): one fused DPP max each
MOE_DEV uint32_t row16_umax(uint32_t v) {
    v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, MOE_DPP_XOR1, 0xF, 0xF, true));
    v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, MOE_DPP_XOR2, 0xF, 0xF, true));
    v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, MOE_DPP_HALF_MIRROR, 0xF, 0xF, true));
    v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, MOE_DPP_MIRROR, 0xF, 0xF, true));
    return v;
}

// Unsigned max over the four lanes l, l ^ 16, l ^ 32, l ^ 48 (the same lane
// of each row of the wave), returned to all four: row-pair swaps of the value
// with itself.
MOE_DEV uint32_t rows4_umax(uint32_t v) {
    const auto a = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    v = max(a[0], a[1]);
    const auto b = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return max(b[0], b[1]);
}

// Unsigned max over the 64 lanes of the wave, returned as a scalar: the
// integer max takes the DPP operand directly (no canonicalising step).
MOE_DEV uint32_t wave_umax(uint32_t v) {
    v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, MOE_DPP_XOR1, 0xF, 0xF, true));
    v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, MOE_DPP_XOR2, 0xF, 0xF, true));
    v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, MOE_DPP_HALF_MIRROR, 0xF, 0xF, true));
    v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, MOE_DPP_MIRROR, 0xF, 0xF, true));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, MOE_DPP_BCAST15, 0xA, 0xF, false));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, MOE_DPP_BCAST31, 0xC, 0xF, false));
    return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// Inclusive prefix sum over the 64 lanes with DPP row shifts and row
// broadcasts (lanes without a source add 0), no LDS round trips.
MOE_DEV int wave_incl_scan(int v) {
    v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, false);     // row_shr:1
    v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, false);     // row_shr:2
    v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, false);     // row_shr:4
    v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, false);     // row_shr:8
    v += __builtin_amdgcn_update_dpp(0, v, MOE_DPP_BCAST15, 0xA, 0xF, false);
    v += __builtin_amdgcn_update_dpp(0, v, MOE_DPP_BCAST31, 0xC, 0xF, false);
    return v;
}

MOE_DEV float row16_sum(float v) {
    v += MOE_DPP(v, MOE_DPP_XOR1, 0xF);
    v += MOE_DPP(v, MOE_DPP_XOR2, 0xF);
    v += MOE_DPP(v, MOE_DPP_HALF_MIRROR, 0xF);
    v += MOE_DPP(v, MOE_DPP_MIRROR, 0xF);
    return v;
}

// Reductions over a half wave (lanes 32h .. 32h+31); every lane of the half
// receives the result. The float forms take the other row through a lane
// exchange (both lanes of a pair add the same two values, and fp32 addition
// is commutative, so both get the same bits); the integer max, used in every
// selection round, through a row swap.
MOE_DEV float row32_max(float v) {
    v = row16_max(v);
    return fmaxf(v, __shfl_xor(v, 16, 64));
}
MOE_DEV float row32_sum(float v) {
    v = row16_sum(v);
    return v + __shfl_xor(v, 16, 64);
}
MOE_DEV uint32_t row32_umax(uint32_t v) {
    v = row16_umax(v);
    const auto a = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    return max(a[0], a[1]);
}

// ---------------------------------------------------------------------------
// Top-k softmax routing with LPT lanes per token (LPT = 64: one token per
// wave; 32: two tokens per wave; 16: one token per DPP row, four tokens per
// wave). Lane i of a
// token's lane group holds experts [i*VPL, i*VPL + VPL), so among lanes whose
// best remaining logit equals the group maximum, the lowest lane holds the
// lowest expert id: ties resolve to the lower id. Selection compares fp32
// logits; the weight of a selected expert is exp(l - max) / sum_e exp(l_e -
// max) in fp32. On return, lane j < k of the group holds the token's j-th
// selection in (sel_e, sel_w). E <= LPT*VPL, k <= LPT.
// ---------------------------------------------------------------------------
// Order-preserving unsigned key of a finite fp32 value: a larger value has a
// larger key, -0 and +0 share the key of +0, and every key is above 0.
MOE_DEV uint32_t f32_order_key(float f) {
    uint32_t u = __builtin_bit_cast(uint32_t, f);
    u = u == 0x80000000u ? 0u : u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
MOE_DEV float order_key_f32(uint32_t k) {
    return __builtin_bit_cast(float, (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

template <int LPT>
MOE_DEV float group_max(float v) { return LPT == 64 ? wave_max(v) : (LPT == 32 ? row32_max(v) : row16_max(v)); }
template <int LPT>
MOE_DEV float group_sum(float v) { return LPT == 64 ? wave_sum(v) : (LPT == 32 ? row32_sum(v) : row16_sum(v)); }
template <int LPT>
MOE_DEV uint32_t group_umax(uint32_t v) { return LPT == 64 ? wave_umax(v) : (LPT == 32 ? row32_umax(v) : row16_umax(v)); }

template <int LPT, int VPL>
MOE_DEV void route_values(const float (&v)[VPL], int E, int k, bool renorm, int lane,
                          int& sel_e, float& sel_w) {
    const int li = lane & (LPT - 1);
    const int base = li * VPL;
    float lm = -INFINITY;
    #pragma unroll
    for (int i = 0; i < VPL; ++i) lm = (base + i < E) ? fmaxf(lm, v[i]) : lm;
    const float m = group_max<LPT>(lm);
    float ls = 0.f;
    #pragma unroll
    for (int i = 0; i < VPL; ++i) ls += (base + i < E) ? __expf(v[i] - m) : 0.f;
    const float inv = 1.0f / group_sum<LPT>(ls);

    // Candidates as order-preserving unsigned keys of the fp32 logits (-0
    // folded onto +0, since the two compare equal); 0 marks a taken or
    // out-of-range entry (logits are finite, so every real key is above it).
    uint32_t c[VPL];
    #pragma unroll
    for (int i = 0; i < VPL; ++i) c[i] = (base + i < E) ? f32_order_key(v[i]) : 0u;
    const int gshift = lane & (64 - LPT);           // the group's first lane
    uint32_t my_key = 0;
    int my_e = -1;
    for (int j = 0; j < k; ++j) {
        // the lane's best key, then the group's
        uint32_t bk = c[0];
        #pragma unroll
        for (int i = 1; i < VPL; ++i) bk = max(bk, c[i]);
        const uint32_t mk = group_umax<LPT>(bk);
        // the lowest lane holding it has the lowest expert id (ties go to
        // the lower id), and within the lane its first slot
        const uint64_t hit = __ballot(bk == mk && mk != 0u);
        const uint64_t ghit = LPT == 64 ? hit : ((hit >> gshift) & ((1ull << LPT) - 1));
        const int win = gshift + (ghit ? __ffsll((unsigned long long)ghit) - 1 : 0);
        int fi = VPL - 1;
        #pragma unroll
        for (int i = VPL - 2; i >= 0; --i) fi = c[i] == mk ? i : fi;
        const int e = LPT == 64 ? __builtin_amdgcn_readlane(base + fi, win)
                                : __shfl(base + fi, win, 64);
        const bool pop = ghit && lane == win;
        #pragma unroll
        for (int i = 0; i < VPL; ++i) c[i] = (pop && i == fi) ? 0u : c[i];
        if (li == j) { my_e = e; my_key = mk; }
    }
    // weights of the selections, once (the same fp32 expressions as a
    // per-round computation; the renormalising sum in selection order)
    const float my_w = li < k ? __expf(order_key_f32(my_key) - m) * inv : 0.f;
    float wsum = 0.f;
    if (renorm)
        for (int j = 0; j < k; ++j) wsum += __shfl(my_w, gshift + j, 64);
    if (li < k) {
        sel_e = my_e;
        sel_w = renorm ? my_w / wsum : my_w;
    }
}

// This lane's VPL logits of a token row (E floats); -inf past E.
template <int LPT, int VPL>
MOE_DEV void load_logits(const float* __restrict__ row, int E, int lane, float (&v)[VPL]) {
    const int base = (lane & (LPT - 1)) * VPL;
    if (VPL % 4 == 0 && base + VPL <= E && (E % 4) == 0) {      // whole run in bounds: 16-byte loads
        #pragma unroll
        for (int i = 0; i < VPL; i += 4) {
            const float4 f = *(const float4*)(row + base + i);
            v[i] = f.x; v[i + 1] = f.y; v[i + 2] = f.z; v[i + 3] = f.w;
        }
    } else {
        #pragma unroll
        for (int i = 0; i < VPL; ++i) v[i] = (base + i < E) ? row[base + i] : -INFINITY;
    }
}
