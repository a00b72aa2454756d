// kvq_encode.hip -- row encoders of the quantized KV cache (gfx950).
//
// fp8: colibri PR #399 "KV cache quantization: fp8 (KV8) + 4-bit TurboQuant
//      (KV_TQ) ...", Summary and commit 1: e4m3 codes with one amax/448 scale
//      per row, round to nearest even.
// TQ4: same page, "Why rotated-int4 for the 4-bit tier": random sign flips,
//      a Walsh-Hadamard rotation, one radius per row and indices into a fixed
//      16-level Lloyd-Max codebook scaled by radius / sqrt(n).
//
// Both kernels are bandwidth kernels: one wave per row (fp8) or dim/8 lanes per
// row (TQ4), 8 consecutive fp32 per lane loaded as two 16-byte loads, codes
// stored as one 8-byte (fp8) or 4-byte (TQ4) store per lane, so every wave
// instruction touches one contiguous span.
#include <cstring>
#include <type_traits>

#include "kvq_device.h"
#include "kvq_internal.h"
#include "kvq_codebook.inc"

namespace kvq {

namespace {

__constant__ uint32_t c_tq4_thresh[15] = KVQ_TQ4_THRESH_BITS;

constexpr int ENC_WAVES = 4;  // waves per workgroup

// ---- fp8 -------------------------------------------------------------------
// One wave per row; ITER chunks of 512 elements (8 per lane).
template <int ITER>
__global__ __launch_bounds__(ENC_WAVES * KVQ_WAVE) void k_encode_fp8(const float* __restrict__ x, int64_t n_rows,
                                                                     int dim, uint8_t* __restrict__ codes,
                                                                     float* __restrict__ scales) {
    const int lane = threadIdx.x & (KVQ_WAVE - 1);
    const int64_t row = (int64_t)blockIdx.x * ENC_WAVES + (threadIdx.x >> 6);
    if (row >= n_rows) return;  // whole wave exits together
    const float* xr = x + row * dim;
    float v[ITER][8];
    float amax = 0.0f;
#pragma unroll
    for (int it = 0; it < ITER; it++) {
        const int base = it * 512 + lane * 8;
        if (base < dim) {
            const float4 a = *reinterpret_cast<const float4*>(xr + base);
            const float4 b = *reinterpret_cast<const float4*>(xr + base + 4);
            v[it][0] = a.x; v[it][1] = a.y; v[it][2] = a.z; v[it][3] = a.w;
            v[it][4] = b.x; v[it][5] = b.y; v[it][6] = b.z; v[it][7] = b.w;
        } else {
#pragma unroll
            for (int j = 0; j < 8; j++) v[it][j] = 0.0f;
        }
#pragma unroll
        for (int j = 0; j < 8; j++) amax = fmaxf(amax, fabsf(v[it][j]));
    }
    amax = wave_max(amax);
    const float s = (amax == 0.0f) ? 0.0f : amax / 448.0f;  // correctly rounded division
    uint8_t* cr = codes + row * dim;
#pragma unroll
    for (int it = 0; it < ITER; it++) {
        const int base = it * 512 + lane * 8;
        if (base < dim) {
            uint32_t lo = 0, hi = 0;
            if (s != 0.0f) {
#pragma unroll
                for (int j = 0; j < 4; j++) lo |= e4m3_rne(v[it][j] / s) << (8 * j);
#pragma unroll
                for (int j = 0; j < 4; j++) hi |= e4m3_rne(v[it][4 + j] / s) << (8 * j);
            }
            *reinterpret_cast<uint2*>(cr + base) = make_uint2(lo, hi);
        }
    }
    if (lane == 0) scales[row] = s;
}

// ---- TQ4 -------------------------------------------------------------------
// L = dim/8 lanes per row (1..64), 64/L rows per wave, 8 consecutive elements
// per lane.  FWHT stages h = 1, 2, 4 in registers, h >= 8 across lanes
// (partner lane ^ h/8); the same (a+b, a-b) data flow as the definition, so the
// result is bit-identical to any other evaluation in that stage order.
__global__ __launch_bounds__(ENC_WAVES * KVQ_WAVE) void k_encode_tq4(const float* __restrict__ x, int64_t n_rows,
                                                                     int dim, const uint8_t* __restrict__ sign_mask,
                                                                     uint8_t* __restrict__ codes,
                                                                     float* __restrict__ radii) {
    const int L = dim >> 3;
    const int lane = threadIdx.x & (KVQ_WAVE - 1);
    const int j = lane & (L - 1);                      // lane within the row
    const int64_t rows_per_wave = KVQ_WAVE / L;
    // grid-stride over groups of rows_per_wave rows; the next group's inputs
    // are loaded while this one is encoded
    const int64_t stride = (int64_t)gridDim.x * ENC_WAVES * rows_per_wave;
    const int64_t first = ((int64_t)blockIdx.x * ENC_WAVES + (threadIdx.x >> 6)) * rows_per_wave;
    const uint32_t sm = sign_mask[j];  // byte j of the mask covers elements 8j .. 8j+7
    auto load = [&](int64_t row, float (&v)[8]) {
        if (row < n_rows) {
            const float* xr = x + row * dim + 8 * j;
            const float4 a = *reinterpret_cast<const float4*>(xr);
            const float4 b = *reinterpret_cast<const float4*>(xr + 4);
            v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
            v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
        } else {
#pragma unroll
            for (int i = 0; i < 8; i++) v[i] = 0.0f;
        }
    };
    float nv[8];
    load(first + lane / L, nv);
    for (int64_t base = first; base < n_rows; base += stride) {
        const int64_t row = base + lane / L;
        const bool valid = row < n_rows;
        float v[8], sq[8];
#pragma unroll
        for (int i = 0; i < 8; i++) v[i] = nv[i];
        load(base + stride + lane / L, nv);
        // radius^2: pairwise tree, leaves fl(x_i * x_i)
#pragma unroll
        for (int i = 0; i < 8; i++) sq[i] = v[i] * v[i];
#pragma unroll
        for (int i = 0; i < 4; i++) sq[i] = sq[2 * i] + sq[2 * i + 1];
#pragma unroll
        for (int i = 0; i < 2; i++) sq[i] = sq[2 * i] + sq[2 * i + 1];
        float r2 = sq[0] + sq[1];
        // a + b == b + a exactly, so every lane of the row ends with the same sum
        if (L > 1) r2 = r2 + xor_lane<1>(r2, lane);
        if (L > 2) r2 = r2 + xor_lane<2>(r2, lane);
        if (L > 4) r2 = r2 + xor_lane<4>(r2, lane);
        if (L > 8) r2 = r2 + xor_lane<8>(r2, lane);
        if (L > 16) r2 = r2 + xor_lane<16>(r2, lane);
        if (L > 32) r2 = r2 + xor_lane<32>(r2, lane);
        const float rad = sqrt_rn(r2);
        // random signs
#pragma unroll
        for (int i = 0; i < 8; i++)
            if ((sm >> i) & 1u) v[i] = -v[i];
        // FWHT, unnormalized
#pragma unroll
        for (int h = 1; h < 8; h <<= 1)
#pragma unroll
            for (int i = 0; i < 8; i++)
                if (!(i & h)) {
                    const float a = v[i], b = v[i + h];
                    v[i] = a + b;
                    v[i + h] = a - b;
                }
        auto stage = [&](auto mc) {
            constexpr int M = decltype(mc)::value;
#pragma unroll
            for (int i = 0; i < 8; i++) v[i] = fwht_xlane_c<M>(v[i], lane);
        };
        if (L == 64) {  // dim 512: all six lane stages, no per-stage branch
            stage(std::integral_constant<int, 1>{});
            stage(std::integral_constant<int, 2>{});
            stage(std::integral_constant<int, 4>{});
            stage(std::integral_constant<int, 8>{});
            stage(std::integral_constant<int, 16>{});
            stage(std::integral_constant<int, 32>{});
        } else {
            if (L > 1) stage(std::integral_constant<int, 1>{});
            if (L > 2) stage(std::integral_constant<int, 2>{});
            if (L > 4) stage(std::integral_constant<int, 4>{});
            if (L > 8) stage(std::integral_constant<int, 8>{});
            if (L > 16) stage(std::integral_constant<int, 16>{});
            if (L > 32) stage(std::integral_constant<int, 32>{});
        }
        // bucketize against fl(t_k * r): idx = #{k : w > T_k}
        float T[15];
#pragma unroll
        for (int k = 0; k < 15; k++) T[k] = u2f(c_tq4_thresh[k]) * rad;
        // T is ascending, so #{k : w > T_k} is found by a branch-free binary search:
        // four comparisons against T_7, then T_3 / T_11, then T_1 / T_5 / T_9 /
        // T_13, then the even-indexed threshold below the interval found so far.
        uint32_t packed = 0;
#pragma unroll
        for (int i = 0; i < 8; i++) {
            const float w = v[i];
            const bool b3 = w > T[7];
            const bool b2 = w > (b3 ? T[11] : T[3]);
            const float t1 = b3 ? (b2 ? T[13] : T[9]) : (b2 ? T[5] : T[1]);
            const bool b1 = w > t1;
            const float e3 = b1 ? T[14] : T[12], e2 = b1 ? T[10] : T[8];
            const float e1 = b1 ? T[6] : T[4], e0 = b1 ? T[2] : T[0];
            const float t0 = b3 ? (b2 ? e3 : e2) : (b2 ? e1 : e0);
            const uint32_t idx = (b3 ? 8u : 0u) + (b2 ? 4u : 0u) + (b1 ? 2u : 0u) + ((w > t0) ? 1u : 0u);
            packed |= idx << (4 * i);
        }
        if (valid) {
            *reinterpret_cast<uint32_t*>(codes + row * (dim >> 1) + 4 * j) = packed;
            if (j == 0) radii[row] = rad;
        }
    }
}

// ---- conversion probe ---------------------------------------------------------
__global__ void k_convert(int kind, const void* __restrict__ in, int64_t n, void* __restrict__ out) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
        switch (kind) {
            case KVQ_CVT_F32_TO_E4M3:
                ((uint8_t*)out)[i] = (uint8_t)e4m3_rne(((const float*)in)[i]);
                break;
            case KVQ_CVT_E4M3_TO_BF16:
                ((uint16_t*)out)[i] = (uint16_t)e4m3_to_bf16(((const uint8_t*)in)[i]);
                break;
            case KVQ_CVT_F32_TO_F16:
                ((uint16_t*)out)[i] = (uint16_t)f32_to_f16_rne(((const float*)in)[i]);
                break;
            case KVQ_CVT_E4M3_TO_F16: {
                typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
                const f16x2_t h = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(((const uint8_t*)in)[i], 1.0f, false);
                ((uint16_t*)out)[i] = __builtin_bit_cast(uint16_t, h[0]);
                break;
            }
            default:
                ((uint16_t*)out)[i] = (uint16_t)f32_to_bf16_rne(((const float*)in)[i]);
                break;
        }
    }
}

}  // namespace

void host_codebook(float* levels16, float* thresholds15) {
    static const uint32_t lv[16] = KVQ_TQ4_LEVEL_BITS;
    static const uint32_t th[15] = KVQ_TQ4_THRESH_BITS;
    if (levels16)
        for (int k = 0; k < 16; k++) std::memcpy(&levels16[k], &lv[k], 4);
    if (thresholds15)
        for (int k = 0; k < 15; k++) std::memcpy(&thresholds15[k], &th[k], 4);
}

hipError_t launch_encode_fp8(const float* x, int64_t n_rows, int dim, uint8_t* codes, float* scales,
                             hipStream_t st) {
    if (n_rows == 0) return hipSuccess;
    const dim3 grid((unsigned)((n_rows + ENC_WAVES - 1) / ENC_WAVES)), block(ENC_WAVES * KVQ_WAVE);
    const int iter = (dim + 511) / 512;
    switch (iter) {
        case 1: hipLaunchKernelGGL(k_encode_fp8<1>, grid, block, 0, st, x, n_rows, dim, codes, scales); break;
        case 2: hipLaunchKernelGGL(k_encode_fp8<2>, grid, block, 0, st, x, n_rows, dim, codes, scales); break;
        case 3: hipLaunchKernelGGL(k_encode_fp8<3>, grid, block, 0, st, x, n_rows, dim, codes, scales); break;
        default: hipLaunchKernelGGL(k_encode_fp8<4>, grid, block, 0, st, x, n_rows, dim, codes, scales); break;
    }
    return hipGetLastError();
}

hipError_t launch_encode_tq4(const float* x, int64_t n_rows, int dim, const uint8_t* sign_mask,
                             uint8_t* codes, float* radii, hipStream_t st) {
    if (n_rows == 0) return hipSuccess;
    const int64_t rows_per_wave = KVQ_WAVE / (dim / 8);
    const int64_t waves = (n_rows + rows_per_wave - 1) / rows_per_wave;
    int64_t wgs = (waves + ENC_WAVES - 1) / ENC_WAVES;
    if (wgs > 4096) wgs = 4096;  // 16 waves per CU; the kernel strides over the rest
    const dim3 grid((unsigned)wgs), block(ENC_WAVES * KVQ_WAVE);
    hipLaunchKernelGGL(k_encode_tq4, grid, block, 0, st, x, n_rows, dim, sign_mask, codes, radii);
    return hipGetLastError();
}

hipError_t launch_convert(int kind, const void* in, int64_t n, void* out, hipStream_t st) {
    if (n == 0) return hipSuccess;
    int64_t blocks = (n + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(k_convert, dim3((unsigned)blocks), dim3(256), 0, st, kind, in, n, out);
    return hipGetLastError();
}

}  // namespace kvq
