// kvq_device.h -- device helpers of the HIP library: format conversions and
// wave-level primitives for gfx950 (wave64).
//
// Every conversion is written from its format definition:
//  - OCP FP8 E4M3 ("e4m3fn"): bias 7, 3 mantissa bits, largest finite 448,
//    S.1111.111 is NaN; the pages read that code back as 0 (colibri PR #399,
//    HIP portability rebase note);
//  - IEEE 754 binary16 and bfloat16 (the upper half of a binary32), both
//    rounded to nearest, ties to even.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define KVQ_WAVE 64

namespace kvq {

__device__ __forceinline__ uint32_t f2u(float f) { return __float_as_uint(f); }
__device__ __forceinline__ float u2f(uint32_t u) { return __uint_as_float(u); }

// Two fp32 -> two e4m3 codes (byte 0: a, byte 1: b): |v| saturated to 448,
// then the hardware conversion on the OCP e4m3 grid, round to nearest even
// (the conversion probe checks it against the format definition on every
// code, every midpoint between codes and their neighbouring floats).  NaN
// input is outside the contract.
__device__ __forceinline__ uint32_t e4m3x2_rne(float a, float b) {
    typedef short s16x2_t __attribute__((ext_vector_type(2)));
    a = __builtin_amdgcn_fmed3f(a, -448.0f, 448.0f);
    b = __builtin_amdgcn_fmed3f(b, -448.0f, 448.0f);
    const s16x2_t r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(s16x2_t{0, 0}, a, b, 1.0f, false);
    return (uint32_t)(uint16_t)r[0];
}

// e4m3 code -> fp32, exact.  S.1111.111 -> +0.
__device__ __forceinline__ float e4m3_to_f32(uint32_t c) {
    uint32_t e = (c >> 3) & 15u, m = c & 7u;
    float mag = (e == 0u) ? (float)m * 0.001953125f                      // M * 2^-9
                          : u2f(((c & 0x7Fu) << 20) + (120u << 23));      // (1 + M/8) 2^(E-7)
    if ((c & 0x7Fu) == 0x7Fu) return 0.0f;
    return (c & 0x80u) ? -mag : mag;
}

// fp32 -> bf16 bits, round to nearest even (finite inputs; overflow -> Inf).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
    uint32_t b = f2u(f);
    return (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
}

// e4m3 code -> bf16 bits, exact (3 mantissa bits fit in 7).
__device__ __forceinline__ uint32_t e4m3_to_bf16(uint32_t c) { return f2u(e4m3_to_f32(c)) >> 16; }

// fp32 -> binary16 bits, round to nearest even (overflow to inf, subnormal
// results kept), by v_cvt_f16_f32 (the conversion probe checks it against the
// format definition on every binary16 midpoint and its neighbours).  The value
// is made opaque first: otherwise the compiler fuses a product feeding it into
// v_fma_mix with a +0 addend, which turns a -0 product into +0.
__device__ __forceinline__ uint32_t f32_to_f16_rne(float f) {
    asm("" : "+v"(f));
    return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)f);
}

// binary16 bits -> fp32, exact.
__device__ __forceinline__ float f16_to_f32(uint32_t h) {
    uint32_t sign = (h & 0x8000u) << 16;
    uint32_t e = (h >> 10) & 31u, m = h & 1023u;
    float mag;
    if (e == 0u) mag = (float)m * 5.9604644775390625e-8f;           // M * 2^-24
    else if (e == 31u) mag = u2f(0x7F800000u | (m << 13));
    else mag = u2f(((e + 112u) << 23) | (m << 13));
    return u2f(f2u(mag) | sign);
}

// Correctly rounded fp32 square root of a finite x >= 0.  v_sqrt_f32 alone is
// not correctly rounded; its estimate is moved to the representable value
// whose rounding interval contains sqrt(x), decided exactly in double: the
// midpoints of neighbouring floats have at most 25 significant bits, so their
// squares are exact in double.
__device__ __forceinline__ float sqrt_rn(float x) {
    if (!(x > 0.0f) || x > 3.4e38f) return x == 0.0f ? x : __builtin_sqrtf(x);
    float y = __builtin_sqrtf(x);
    const double xd = (double)x;
#pragma unroll
    for (int it = 0; it < 2; it++) {
        const float up = u2f(f2u(y) + 1u);
        const double mid_hi = 0.5 * ((double)y + (double)up);
        if (mid_hi * mid_hi < xd) { y = up; continue; }
        const float dn = u2f(f2u(y) - 1u);
        const double mid_lo = 0.5 * ((double)y + (double)dn);
        if (mid_lo * mid_lo > xd) y = dn;
    }
    return y;
}

// ---- wave primitives -------------------------------------------------------

__device__ __forceinline__ float shfl_xor_f(float v, int m) { return __shfl_xor(v, m, KVQ_WAVE); }
__device__ __forceinline__ uint32_t shfl_xor_u(uint32_t v, int m) {
    return (uint32_t)__shfl_xor((int)v, m, KVQ_WAVE);
}

// max over the wave (defined below, after the lane-exchange helpers it uses)
__device__ __forceinline__ float wave_max(float v);

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += shfl_xor_f(v, m);
    return v;
}

// ---- the fp8 row encoder ---------------------------------------------------
// One row of dim (a multiple of 8, <= 512 ITER) fp32 values, one wave (colibri
// PR #399 "KV cache quantization: fp8 (KV8) + 4-bit TurboQuant (KV_TQ) ...",
// Summary and commit 1: e4m3 codes with one amax/448 scale per row, round to
// nearest even):
//   *scale = fl(amax / 448) (0 for an all-zero row),
//   code_i = e4m3(fl(x_i / scale)) (0 for an all-zero row).
// Lane l holds elements 4 l .. 4 l + 3 and 256 + 4 l .. + 3 of each 512-element
// span, so every load covers 1 KB of the row contiguously (the steps are
// element-wise; the maximum does not depend on the order).  Codes are stored as
// one 4-byte store per lane and span, the scale by lane 0.
typedef float f32x4v __attribute__((ext_vector_type(4)));  // a native vector (non-temporal loads)

template <int ITER>
__device__ __forceinline__ void encode_fp8_row(const float* __restrict__ xr, int dim, uint8_t* __restrict__ cr,
                                               float* __restrict__ scale, int lane) {
    float v[ITER][8];
    float amax = 0.0f;
#pragma unroll
    for (int it = 0; it < ITER; it++) {
#pragma unroll
        for (int hf = 0; hf < 2; hf++) {
            const int base = it * 512 + 256 * hf + lane * 4;  // dim is a multiple of 8: all four or none
            if (base < dim) {
                const f32x4v a = __builtin_nontemporal_load(reinterpret_cast<const f32x4v*>(xr + base));
                v[it][4 * hf + 0] = a[0]; v[it][4 * hf + 1] = a[1]; v[it][4 * hf + 2] = a[2]; v[it][4 * hf + 3] = a[3];
            } else {
#pragma unroll
                for (int j = 0; j < 4; j++) v[it][4 * hf + j] = 0.0f;
            }
        }
#pragma unroll
        for (int j = 0; j < 8; j++) amax = fmaxf(amax, fabsf(v[it][j]));
    }
    amax = wave_max(amax);
    const float s = (amax == 0.0f) ? 0.0f : amax / 448.0f;  // correctly rounded division
    // x / s, correctly rounded: for amax >= 2^-90 from the correctly rounded
    // reciprocal r = 1/s with one fma correction, q = q0 + (x - q0 s) r with
    // q0 = x r (Markstein's theorem; the residual x - q0 s is exact in an fma).
    // Smaller rows, where 1/s can overflow, divide.  Wave-uniform branch.
    const bool recip = amax >= 0x1p-90f;
    const float r = recip ? 1.0f / s : 0.0f;
#pragma unroll
    for (int it = 0; it < ITER; it++) {
#pragma unroll
        for (int hf = 0; hf < 2; hf++) {
            const int base = it * 512 + 256 * hf + lane * 4;
            if (base < dim) {
                float qv[4];
                if (recip) {
#pragma unroll
                    for (int j = 0; j < 4; j++) {
                        const float q0 = v[it][4 * hf + j] * r;
                        qv[j] = __builtin_fmaf(__builtin_fmaf(-q0, s, v[it][4 * hf + j]), r, q0);
                    }
                } else {
#pragma unroll
                    for (int j = 0; j < 4; j++) qv[j] = (s != 0.0f) ? v[it][4 * hf + j] / s : 0.0f;
                }
                const uint32_t w = e4m3x2_rne(qv[0], qv[1]) | (e4m3x2_rne(qv[2], qv[3]) << 16);
                __builtin_nontemporal_store(w, reinterpret_cast<uint32_t*>(cr + base));
            }
        }
    }
    if (lane == 0) *scale = s;
}

// Cross-lane FWHT stage with partner lane^m: the lower lane keeps a + b, the
// upper lane keeps a - b, where a is the lower lane's value and b the upper's.
__device__ __forceinline__ float fwht_xlane(float v, int lane, int m) {
    float o = shfl_xor_f(v, m);
    return (lane & m) ? (o - v) : (v + o);
}

// The value of lane ^ M, for a compile-time M, without the LDS crossbar:
// DPP quad permutations (M = 1, 2), two row shifts and a select (M = 4), a row
// rotation (M = 8), the gfx950 16- and 32-lane swaps (M = 16, 32).
template <int M>
__device__ __forceinline__ float xor_lane(float v, int lane) {
    const int x = __float_as_int(v);
    int r;
    if constexpr (M == 1) {
        r = __builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, false);  // quad_perm [1, 0, 3, 2]
    } else if constexpr (M == 2) {
        r = __builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, false);  // quad_perm [2, 3, 0, 1]
    } else if constexpr (M == 4) {
        const int up = __builtin_amdgcn_mov_dpp(x, 0x104, 0xF, 0xF, false);  // row_shl:4, lane i <- i + 4
        const int dn = __builtin_amdgcn_mov_dpp(x, 0x114, 0xF, 0xF, false);  // row_shr:4, lane i <- i - 4
        r = (lane & 4) ? dn : up;
    } else if constexpr (M == 8) {
        r = __builtin_amdgcn_mov_dpp(x, 0x128, 0xF, 0xF, false);  // row_ror:8
    } else if constexpr (M == 16) {
        const auto p = __builtin_amdgcn_permlane16_swap((unsigned)x, (unsigned)x, false, false);
        r = (int)((lane & 16) ? p[0] : p[1]);
    } else {
        static_assert(M == 32, "xor_lane: M must be 1, 2, 4, 8, 16 or 32");
        const auto p = __builtin_amdgcn_permlane32_swap((unsigned)x, (unsigned)x, false, false);
        r = (int)((lane & 32) ? p[0] : p[1]);
    }
    return __int_as_float(r);
}

// Max over the wave by lane swaps and DPP moves (no LDS crossbar round trips:
// six short dependent steps).  The max is exact, so the order does not matter.
__device__ __forceinline__ float wave_max(float v) {
    const int lane = (int)__lane_id();
    v = fmaxf(v, xor_lane<32>(v, lane));
    v = fmaxf(v, xor_lane<16>(v, lane));
    v = fmaxf(v, xor_lane<8>(v, lane));
    v = fmaxf(v, xor_lane<4>(v, lane));
    v = fmaxf(v, xor_lane<2>(v, lane));
    return fmaxf(v, xor_lane<1>(v, lane));
}

// FWHT stage with partner lane ^ M (as fwht_xlane, M a compile-time constant).
// The lower lane keeps a + b, the upper b' = a - b; both as one fma with the
// exact product (+-1) * v, so the sum is rounded once, as an add or subtract.
template <int M>
__device__ __forceinline__ float fwht_xlane_c(float v, int lane) {
    const float o = xor_lane<M>(v, lane);
    return __builtin_fmaf((lane & M) ? -1.0f : 1.0f, v, o);
}

// ---- DPP helpers (lane patterns inside a 16-lane row) -----------------------
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
    // every source lane of the patterns below exists, so bound_ctrl never applies; the form
    // with an old value of 0 lets the compiler fold the move into the add that uses it
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}
// y[i0 + e] += c * (y[i0 + e] of the partner lane), e = 0..7, as v_fmac_f32_dpp (the
// compiler does not fold a DPP move into an fma whose addend is tied to the result).
// A DPP read of a VGPR needs 2 wait states after a VALU write of it; the block
// provides them up front (inside it, no instruction reads what the one before wrote).
#define KVQ_FMAC_DPP_X8(PAT, y, i0, c)                                                     \
    asm("s_nop 1\n\t"                                                                     \
        "v_fmac_f32_dpp %0, %0, %8 " PAT " row_mask:0xf bank_mask:0xf\n\t"                \
        "v_fmac_f32_dpp %1, %1, %8 " PAT " row_mask:0xf bank_mask:0xf\n\t"                \
        "v_fmac_f32_dpp %2, %2, %8 " PAT " row_mask:0xf bank_mask:0xf\n\t"                \
        "v_fmac_f32_dpp %3, %3, %8 " PAT " row_mask:0xf bank_mask:0xf\n\t"                \
        "v_fmac_f32_dpp %4, %4, %8 " PAT " row_mask:0xf bank_mask:0xf\n\t"                \
        "v_fmac_f32_dpp %5, %5, %8 " PAT " row_mask:0xf bank_mask:0xf\n\t"                \
        "v_fmac_f32_dpp %6, %6, %8 " PAT " row_mask:0xf bank_mask:0xf\n\t"                \
        "v_fmac_f32_dpp %7, %7, %8 " PAT " row_mask:0xf bank_mask:0xf"                      \
        : "+v"(y[(i0) + 0]), "+v"(y[(i0) + 1]), "+v"(y[(i0) + 2]), "+v"(y[(i0) + 3]),       \
          "+v"(y[(i0) + 4]), "+v"(y[(i0) + 5]), "+v"(y[(i0) + 6]), "+v"(y[(i0) + 7])        \
        : "v"(c))
constexpr int DPP_XOR1 = 0xB1;   // quad_perm [1, 0, 3, 2]
constexpr int DPP_XOR2 = 0x4E;   // quad_perm [2, 3, 0, 1]
constexpr int DPP_XOR7 = 0x141;  // row_half_mirror: lane i <- 7 - i within 8
constexpr int DPP_XOR8 = 0x128;  // row_ror:8 within a 16-lane row

// Largest-value selection on the key (|x|, x) with +0 above -0: the key is
// order-preserving as an unsigned integer.
__device__ __forceinline__ uint32_t absval_key(float x) {
    uint32_t b = f2u(x);
    return ((b & 0x7FFFFFFFu) << 1) | ((b >> 31) ^ 1u);
}

}  // namespace kvq
