// kvq_encode.hip -- row encoders of the quantized KV cache (gfx950).
//
// fp8: colibri PR #399 "KV cache quantization: fp8 (KV8) + 4-bit TurboQuant
//      (KV_TQ) ...", Summary and commit 1: e4m3 codes with one amax/448 scale
//      per row, round to nearest even.
// TQ4: same page, "Why rotated-int4 for the 4-bit tier": random sign flips,
//      a Walsh-Hadamard rotation, one radius per row and indices into a fixed
//      16-level Lloyd-Max codebook scaled by radius / sqrt(n); the 3- and 6-bit
//      tiers (TQ3, TQ6: the .coli_kv reply and the teacher-forcing table) are the
//      same codec with the 8- and 64-level codebooks.
//
// fp8: one wave per row, 8 consecutive fp32 per lane loaded as two 16-byte
// loads, codes stored as one 8-byte store per lane, so every wave instruction
// touches one contiguous span.  TQ4: a general kernel (dim/8 lanes per row) and
// one for dim 512 with well under half the vector instructions per row, which
// streams its input at close to the rate of a plain copy.
#include <cstring>
#include <type_traits>

#include "kvq_device.h"
#include "kvq_internal.h"
#include "kvq_codebook.inc"

namespace kvq {

namespace {

__constant__ uint32_t c_tq4_thresh[15] = KVQ_TQ4_THRESH_BITS;
__constant__ uint32_t c_tq3_thresh[7] = KVQ_TQ3_THRESH_BITS;
__constant__ uint32_t c_tq6_thresh[63] = KVQ_TQ6_THRESH_BITS;
__constant__ uint8_t c_tq6_cell[KVQ_TQ6_CELLS] = KVQ_TQ6_CELL_TABLE;

constexpr int ENC_WAVES = 4;  // waves per workgroup

// ---- fp8 -------------------------------------------------------------------
// One wave per row (encode_fp8_row in kvq_device.h); ITER chunks of 512 elements.
template <int ITER>
__global__ __launch_bounds__(ENC_WAVES * KVQ_WAVE) void k_encode_fp8(const float* __restrict__ x, int64_t n_rows,
                                                                     int dim, uint8_t* __restrict__ codes,
                                                                     float* __restrict__ scales) {
    const int lane = threadIdx.x & (KVQ_WAVE - 1);
    const int64_t row = (int64_t)blockIdx.x * ENC_WAVES + (threadIdx.x >> 6);
    if (row >= n_rows) return;  // whole wave exits together
    encode_fp8_row<ITER>(x + row * dim, dim, codes + row * dim, scales + row, lane);
}

// ---- rotated codec, any width ------------------------------------------------------
// L = dim/8 lanes per row (1..64), 64/L rows per wave, 8 consecutive elements
// per lane.  FWHT stages h = 1, 2, 4 in registers, h >= 8 across lanes
// (partner lane ^ h/8); the same (a+b, a-b) data flow as the definition, so the
// result is bit-identical to any other evaluation in that stage order.
// BITS = 4: nibbles, one 4-byte store per lane.  BITS = 3, 6: the lane's 8
// indices are 3 or 6 bytes of the row's little-endian bit stream (index i in
// bits BITS*i ..).  Their index #{k : w > T_k}, T_k = fl(t_k * r), comes from a
// cell: v = clamp(A w / r + OFF, 0, N - 1/2) and cell floor(v), where every
// threshold lies inside a cell, at least 0.05 cell widths from its edges, and
// no cell holds two (the generator of the cell constants asserts both; 3 bits:
// 7 cells of width 1/1.9, one per threshold; 6 bits: 173 cells of width
// 1/23.75, narrower than the closest pair of thresholds).  A cell's table entry
// is c, the number of thresholds below its lower edge, and t_c, the next one
// up, so idx = c + [w > fl(t_c r)] exactly (the rounding in A w / r is below
// 1e-3 cell widths).  A zero radius needs no special case (as in the dim-512
// TQ4 kernel below); a row whose r^2 is inf or NaN takes a binary search over
// all thresholds instead: T_k is ascending in k (or, for a radius of inf or
// NaN, w > T_k still holds for a prefix of k), so it returns the count exactly.
template <int BITS>
__global__ __launch_bounds__(ENC_WAVES * KVQ_WAVE) void k_encode_tq(const float* __restrict__ x, int64_t n_rows,
                                                                    int dim, const uint8_t* __restrict__ sign_mask,
                                                                    uint8_t* __restrict__ codes,
                                                                    float* __restrict__ radii) {
    constexpr int NL = 1 << BITS;  // levels
    constexpr int NC = BITS == 3 ? KVQ_TQ3_CELLS : BITS == 6 ? KVQ_TQ6_CELLS : 1;  // cells
    constexpr float CELL_A = BITS == 3 ? KVQ_TQ3_CELL_A : BITS == 6 ? KVQ_TQ6_CELL_A : 0.0f;
    constexpr float CELL_OFF = BITS == 3 ? KVQ_TQ3_CELL_OFF : BITS == 6 ? KVQ_TQ6_CELL_OFF : 0.0f;
    static_assert(NC <= ENC_WAVES * KVQ_WAVE, "one cell entry per thread");
    __shared__ float th_s[NL];
    __shared__ uint2 cell_s[NC];  // (bits of t_c, c)
    if (BITS != 4) {
        const int t = threadIdx.x;
        if (t < NL - 1) th_s[t] = u2f(BITS == 3 ? c_tq3_thresh[t] : c_tq6_thresh[t]);
        if (t < NC) {
            const uint32_t c = BITS == 3 ? (uint32_t)t : (uint32_t)c_tq6_cell[t];
            cell_s[t] = make_uint2(BITS == 3 ? c_tq3_thresh[c] : c_tq6_thresh[c], c);
        }
        __syncthreads();
    }
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
        if constexpr (BITS != 4) {
            const bool redo = !(r2 <= 3.40282347e38f);
            const float inv_a = CELL_A * __builtin_amdgcn_rcpf(rad);  // +inf for a zero radius
            uint64_t packed = 0;
#pragma unroll
            for (int i = 0; i < 8; i++) {
                const float w = v[i];
                // v_med3 returns the smaller bound or NaN for a NaN input (w = 0 with a zero
                // radius); v_cvt_u32_f32, written out, turns NaN into cell 0
                const float cf = __builtin_amdgcn_fmed3f(__builtin_fmaf(w, inv_a, CELL_OFF), 0.0f, NC - 0.5f);
                uint32_t ci;
                asm("v_cvt_u32_f32 %0, %1" : "=v"(ci) : "v"(cf));
                const uint2 e = cell_s[ci];
                const uint32_t idx = e.y + ((w > u2f(e.x) * rad) ? 1u : 0u);
                packed |= (uint64_t)idx << (BITS * i);
            }
            if (__builtin_amdgcn_ballot_w64(redo) != 0 && redo) {
                asm volatile("" ::: "memory");  // not evaluated speculatively
                packed = 0;
#pragma unroll
                for (int i = 0; i < 8; i++) {
                    const float w = v[i];
                    uint32_t idx = 0;
#pragma unroll
                    for (int step = NL / 2; step >= 1; step >>= 1) idx += (w > th_s[idx + step - 1] * rad) ? step : 0;
                    packed |= (uint64_t)idx << (BITS * i);
                }
            }
            if (valid) {
                uint8_t* cr = codes + row * (int64_t)(dim * BITS / 8) + BITS * j;
                if (BITS == 3) {
                    cr[0] = (uint8_t)packed;
                    cr[1] = (uint8_t)(packed >> 8);
                    cr[2] = (uint8_t)(packed >> 16);
                } else {  // 6 bytes at an even offset
                    uint16_t* c2 = reinterpret_cast<uint16_t*>(cr);
                    c2[0] = (uint16_t)packed;
                    c2[1] = (uint16_t)(packed >> 16);
                    c2[2] = (uint16_t)(packed >> 32);
                }
                if (j == 0) radii[row] = rad;
            }
            continue;
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

// ---- rotated codec, dim 512 ------------------------------------------------------
// The same result as k_encode_tq<4> with fewer vector instructions per row
// (the general kernel spends about 500 per 512-wide row):
//  - 16 lanes per row, 4 rows per wave.  Lane u of a row has the lane-stage
//    index q = u ^ 3 bit2(u) and loads column group g = q ^ 15, i.e. the 32
//    elements p = j + 4 g + 64 k (j = 0..3, k = 0..7), as eight 16-byte loads
//    (load k covers 256 contiguous bytes per row).  FWHT stages in the
//    definition's order: h = 1, 2 in registers (bits of j), h = 4, 8, 16, 32
//    across lanes (bits of q: partner lane u ^ 1, u ^ 2, u ^ 7, u ^ 8, each a
//    single DPP pattern inside a 16-lane row), h = 64, 128, 256 in registers
//    (bits of k).
//  - Each cross-lane stage is one fma with the partner's value as the DPP
//    operand: y + c * y_partner with c = +1 in the lower lane and -1 in the
//    upper.  The upper lane then holds -(a - b) instead of a - b (rounded once
//    either way; rounding to nearest is symmetric), so the four stages compute
//    (-1)^popcount(q) times the 16-point transform of what the lanes hold.
//    That sign pattern is a Walsh character: multiplying the transform's output
//    by it equals transforming the input with its lane index xor-ed by 15.  The
//    lanes load group q ^ 15 for that reason, and lane q ends with the
//    transform's value for group q itself, sign included, from the same
//    pairwise sums.
//  - Bucketing: idx = #{k : w > T_k} with T_k = fl(t_k * r).  The cell
//    c = clamp(floor(a w / r + 7.5), 0, 14) with a = D512_CELL_SCALE puts its
//    lower edges (c - 7.5) / a strictly between consecutive thresholds,
//    (c - 7.5) / a in (t_{c-1}, t_c) for c = 1..14, at least 0.05 from both, so
//    the cell holds no threshold but t_c and idx = c + [w > T_c] exactly
//    (rounding in a w / r is below 1e-6 relative; the clamp covers any |w| / r).
//    T_c comes from lane c of the row, which holds T_u = fl(t_u * r) for its
//    own u, through ds_bpermute.  A zero radius needs no special case (see
//    the code); a row whose r^2 is inf or NaN takes the defining comparisons
//    against all 15 thresholds.
//  - Inputs are read once, codes written once: both with non-temporal hints.
constexpr int D512_ROWS = 4;                // rows per wave
constexpr float D512_CELL_SCALE = 3.35f;    // a above; any a in (3.18, 3.53) separates the thresholds
constexpr int64_t D512_MAX_WGS = 1 << 24;   // grid cap; the kernel strides over the rest

//  - BITS = 3 and 6 (k_encode_tq_d512<3/6>) share the load, radius, signs and
//    transform, so their values are the general kernel's bit for bit; the
//    bucketing is the general kernel's cell table, and the codes go through a
//    per-wave LDS row: lane q holds the indices of elements 4 q + 64 k + j, for
//    each k a 24-bit piece (6 bits: its own four, at byte 3 q + 48 k; 3 bits:
//    an even lane's four and its odd partner's, at byte 3 (q / 2) + 24 k),
//    written as a 16-bit and an 8-bit LDS store, then read back as 24 (12)
//    contiguous bytes per lane and stored with 8-byte (4-byte) stores.
template <int BITS>
__global__ __launch_bounds__(ENC_WAVES * KVQ_WAVE) void k_encode_tq_d512(const float* __restrict__ x,
                                                                         int64_t n_rows,
                                                                         const uint8_t* __restrict__ sign_mask,
                                                                         uint8_t* __restrict__ codes,
                                                                         float* __restrict__ radii) {
    constexpr int D = 512;
    constexpr int NL = 1 << BITS;  // levels
    constexpr int NC = BITS == 3 ? KVQ_TQ3_CELLS : BITS == 6 ? KVQ_TQ6_CELLS : 1;  // cells
    constexpr float CELL_A = BITS == 3 ? KVQ_TQ3_CELL_A : BITS == 6 ? KVQ_TQ6_CELL_A : 0.0f;
    constexpr float CELL_OFF = BITS == 3 ? KVQ_TQ3_CELL_OFF : BITS == 6 ? KVQ_TQ6_CELL_OFF : 0.0f;
    constexpr int RB = D * BITS / 8;  // code bytes per row
    static_assert(NC <= ENC_WAVES * KVQ_WAVE, "one cell entry per thread");
    __shared__ float th_s[NL];
    __shared__ uint2 cell_s[NC];                                       // (bits of t_c, c)
    __shared__ __align__(16) uint8_t row_s[ENC_WAVES][D512_ROWS][BITS == 4 ? 16 : RB];  // BITS 3, 6
    if constexpr (BITS != 4) {
        const int t = threadIdx.x;
        if (t < NL - 1) th_s[t] = u2f(BITS == 3 ? c_tq3_thresh[t] : c_tq6_thresh[t]);
        if (t < NC) {
            const uint32_t c = BITS == 3 ? (uint32_t)t : (uint32_t)c_tq6_cell[t];
            cell_s[t] = make_uint2(BITS == 3 ? c_tq3_thresh[c] : c_tq6_thresh[c], c);
        }
        __syncthreads();
    }
    typedef float f4v __attribute__((ext_vector_type(4)));
    const int lane = threadIdx.x & (KVQ_WAVE - 1);
    const int slot = lane >> 4, u = lane & 15;
    const int q = u ^ (((u >> 2) & 1) * 3);
    const int g = q ^ 15;  // column group this lane loads
    // sign flip of element (j, k): bit j + 4 (g & 1) of mask byte 8 k + g / 2, gathered
    // into bit 4 k + j of one word
    uint32_t sbits = 0;
#pragma unroll
    for (int k = 0; k < 8; k++)
        sbits |= (((uint32_t)sign_mask[8 * k + (g >> 1)] >> (4 * (g & 1))) & 15u) << (4 * k);
    const float c0 = (q & 1) ? -1.0f : 1.0f, c1 = (q & 2) ? -1.0f : 1.0f;
    const float c2 = (q & 4) ? -1.0f : 1.0f, c3 = (q & 8) ? -1.0f : 1.0f;
    const float t_own = u2f(c_tq4_thresh[min(u, 14)]);  // lane u of a row provides T_u (lane 15: unused)
    const int perm_row = 64 * slot;                       // ds_bpermute byte address of the row's lane 0
    const bool qodd = q & 1;
    const uint32_t sel_lo = qodd ? 0x01000504u : 0x05040100u;  // own 16 bits low (even q) or high (odd q)
    const uint32_t sel_hi = qodd ? 0x03020706u : 0x07060302u;

    const int64_t stride = (int64_t)gridDim.x * ENC_WAVES * D512_ROWS;
    const int64_t first = ((int64_t)blockIdx.x * ENC_WAVES + (threadIdx.x >> 6)) * D512_ROWS;
    // clamped rows: no load waits on a lane condition; a row slot past the end works on a
    // copy of the last row
    auto load = [&](int64_t base, float4 (&v)[8]) __attribute__((always_inline)) {
        const int64_t row = min(base + slot, n_rows - 1);
        const float* xr = x + row * D + 4 * g;
#pragma unroll
        for (int k = 0; k < 8; k++) {
            const f4v t = __builtin_nontemporal_load(reinterpret_cast<const f4v*>(xr + 64 * k));
            v[k] = make_float4(t.x, t.y, t.z, t.w);
        }
    };
    float4 nv[8];
    load(first, nv);
    for (int64_t base = first; base < n_rows; base += stride) {
        float v[32];
#pragma unroll
        for (int k = 0; k < 8; k++) {
            v[4 * k + 0] = nv[k].x; v[4 * k + 1] = nv[k].y; v[4 * k + 2] = nv[k].z; v[4 * k + 3] = nv[k].w;
        }
        const int64_t row = base + slot;  // rows past the end hold a copy of the last row
        // radius^2: the pairwise tree over p (bits 0, 1 here, 2..5 across lanes, 6..8 here)
        float s2[8];
#pragma unroll
        for (int k = 0; k < 8; k++) {
            const float a0 = v[4 * k] * v[4 * k], a1 = v[4 * k + 1] * v[4 * k + 1];
            const float a2 = v[4 * k + 2] * v[4 * k + 2], a3 = v[4 * k + 3] * v[4 * k + 3];
            s2[k] = (a0 + a1) + (a2 + a3);
        }
#pragma unroll
        for (int k = 0; k < 8; k++) s2[k] = s2[k] + dpp_f32<DPP_XOR1>(s2[k]);  // a + b == b + a: both lanes agree
#pragma unroll
        for (int k = 0; k < 8; k++) s2[k] = s2[k] + dpp_f32<DPP_XOR2>(s2[k]);
#pragma unroll
        for (int k = 0; k < 8; k++) s2[k] = s2[k] + dpp_f32<DPP_XOR7>(s2[k]);
#pragma unroll
        for (int k = 0; k < 8; k++) s2[k] = s2[k] + dpp_f32<DPP_XOR8>(s2[k]);
        const float r2 = ((s2[0] + s2[1]) + (s2[2] + s2[3])) + ((s2[4] + s2[5]) + (s2[6] + s2[7]));
        const float rad = sqrt_rn(r2);
        // random signs, then the transform
        uint32_t sb = sbits;
        asm("" : "+v"(sb));  // opaque per iteration: the 32 masks are not hoisted into 32 registers
#pragma unroll
        for (int i = 0; i < 32; i++)  // bit i rotated to bit 31, xor-ed into the sign
            v[i] = u2f(f2u(v[i]) ^ (__builtin_amdgcn_alignbit(sb, sb, (i + 1) & 31) & 0x80000000u));
#pragma unroll
        for (int h = 1; h < 4; h <<= 1)
#pragma unroll
            for (int i = 0; i < 32; i++)
                if (!(i & h)) {
                    const float a = v[i], b = v[i + h];
                    v[i] = a + b;
                    v[i + h] = a - b;
                }
#pragma unroll
        for (int i = 0; i < 32; i += 8) KVQ_FMAC_DPP_X8("quad_perm:[1,0,3,2]", v, i, c0);
#pragma unroll
        for (int i = 0; i < 32; i += 8) KVQ_FMAC_DPP_X8("quad_perm:[2,3,0,1]", v, i, c1);
#pragma unroll
        for (int i = 0; i < 32; i += 8) KVQ_FMAC_DPP_X8("row_half_mirror", v, i, c2);
#pragma unroll
        for (int i = 0; i < 32; i += 8) KVQ_FMAC_DPP_X8("row_ror:8", v, i, c3);
#pragma unroll
        for (int h = 4; h < 32; h <<= 1)
#pragma unroll
            for (int i = 0; i < 32; i++)
                if (!(i & h)) {
                    const float a = v[i], b = v[i + h];
                    v[i] = a + b;
                    v[i + h] = a - b;
                }
        if constexpr (BITS != 4) {
            // lane q holds elements p = j + 4 q + 64 k (v[4 k + j]); cells as in k_encode_tq
            const bool redo = !(r2 <= 3.40282347e38f);
            const float inv_a = CELL_A * __builtin_amdgcn_rcpf(rad);  // +inf for a zero radius
            uint32_t V[8];  // the indices of elements 4 q + 64 k + j, BITS j bits up, for each k
#pragma unroll
            for (int k = 0; k < 8; k++) {
                V[k] = 0u;
#pragma unroll
                for (int j = 0; j < 4; j++) {
                    const float w = v[4 * k + j];
                    // v_med3 returns the smaller bound or NaN for a NaN input; v_cvt_u32_f32,
                    // written out, turns NaN into cell 0
                    const float cf = __builtin_amdgcn_fmed3f(__builtin_fmaf(w, inv_a, CELL_OFF), 0.0f, NC - 0.5f);
                    uint32_t ci;
                    asm("v_cvt_u32_f32 %0, %1" : "=v"(ci) : "v"(cf));
                    const uint2 e = cell_s[ci];
                    V[k] |= (e.y + ((w > u2f(e.x) * rad) ? 1u : 0u)) << (BITS * j);
                }
            }
            if (__builtin_amdgcn_ballot_w64(redo) != 0 && redo) {
                asm volatile("" ::: "memory");  // not evaluated speculatively
#pragma unroll
                for (int k = 0; k < 8; k++) {
                    V[k] = 0u;
#pragma unroll
                    for (int j = 0; j < 4; j++) {
                        const float w = v[4 * k + j];
                        uint32_t idx = 0;
#pragma unroll
                        for (int st = NL / 2; st >= 1; st >>= 1) idx += (w > th_s[idx + st - 1] * rad) ? st : 0;
                        V[k] |= idx << (BITS * j);
                    }
                }
            }
            // the row's code bytes in LDS (this wave's own rows: its LDS operations run in order)
            uint8_t* rs = &row_s[threadIdx.x >> 6][slot][0];
            const bool writer = BITS == 6 || !qodd;
            uint32_t off = BITS == 6 ? 3u * (uint32_t)q : 3u * (uint32_t)(q >> 1);
#pragma unroll
            for (int k = 0; k < 8; k++) {
                uint32_t w24 = V[k];
                if constexpr (BITS == 3)  // the odd partner's 12 bits above the even lane's
                    w24 |= (uint32_t)__builtin_amdgcn_mov_dpp((int)V[k], DPP_XOR1, 0xF, 0xF, false) << 12;
                const uint32_t o = off + (uint32_t)(k * (RB / 8));
                if (writer) {
                    if (o & 1u) {
                        rs[o] = (uint8_t)w24;
                        *reinterpret_cast<uint16_t*>(rs + o + 1) = (uint16_t)(w24 >> 8);
                    } else {
                        *reinterpret_cast<uint16_t*>(rs + o) = (uint16_t)w24;
                        rs[o + 2] = (uint8_t)(w24 >> 16);
                    }
                }
            }
            __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
            const int64_t srow = min(row, n_rows - 1);  // a slot past the end rewrites the last row
            if constexpr (BITS == 6) {  // lane u: bytes 24 u .. 24 u + 23
                const uint2* src2 = reinterpret_cast<const uint2*>(rs + 24 * u);
                uint2* dst2 = reinterpret_cast<uint2*>(codes + srow * RB + 24 * u);
                const uint2 w0 = src2[0], w1 = src2[1], w2 = src2[2];
                __builtin_nontemporal_store(w0.x, &dst2[0].x);
                __builtin_nontemporal_store(w0.y, &dst2[0].y);
                __builtin_nontemporal_store(w1.x, &dst2[1].x);
                __builtin_nontemporal_store(w1.y, &dst2[1].y);
                __builtin_nontemporal_store(w2.x, &dst2[2].x);
                __builtin_nontemporal_store(w2.y, &dst2[2].y);
            } else {  // lane u: bytes 12 u .. 12 u + 11
                const uint32_t* src1 = reinterpret_cast<const uint32_t*>(rs + 12 * u);
                uint32_t* dst1 = reinterpret_cast<uint32_t*>(codes + srow * RB + 12 * u);
                const uint32_t w0 = src1[0], w1 = src1[1], w2 = src1[2];
                __builtin_nontemporal_store(w0, dst1);
                __builtin_nontemporal_store(w1, dst1 + 1);
                __builtin_nontemporal_store(w2, dst1 + 2);
            }
            __builtin_nontemporal_store(rad, radii + srow);
            // every lane has read the row before the next iteration writes it
            __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
            if (base + stride < n_rows) load(base + stride, nv);
            continue;
        }
        // bucketing; nibble of element (j, k) -> bit 4 j + 16 bit1(k) of word P[2 (k & 1) + k / 4]
        // a zero radius gives inv_a = +inf: cell 14 for w > 0, cell 0 for w < 0 and, through
        // NaN, for w = +-0, where T_0 = -0 and T_14 = +0 make idx 15 and 0 as the definition
        // does; a radius of inf or NaN leaves every cell in [0, 14] and the row is redone below
        const bool redo = !(r2 <= 3.40282347e38f);
        const float inv_a = D512_CELL_SCALE * __builtin_amdgcn_rcpf(rad);
        const int t_me = (int)f2u(t_own * rad);
        uint32_t P[4] = {0u, 0u, 0u, 0u};
        // 16 elements at a time: their cells, then their 16 lane reads in flight together,
        // then the comparisons
#pragma unroll
        for (int h = 0; h < 32; h += 16) {
            uint32_t c[16];
            float tc[16];
#pragma unroll
            for (int i = 0; i < 16; i++) {
                const float cf = __builtin_amdgcn_fmed3f(__builtin_fmaf(v[h + i], inv_a, 7.5f), 0.0f, 14.5f);
                // v_med3 returns the smaller bound or NaN for a NaN input; v_cvt_u32_f32,
                // written out, turns NaN into 0
                asm("v_cvt_u32_f32 %0, %1" : "=v"(c[i]) : "v"(cf));
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < 16; i++)
                tc[i] = u2f((uint32_t)__builtin_amdgcn_ds_bpermute(perm_row + 4 * (int)c[i], t_me));
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < 16; i++) {
                const int e = h + i, k = e >> 2, j = e & 3;
                const uint32_t idx = c[i] + ((v[e] > tc[i]) ? 1u : 0u);
                P[2 * (k & 1) + (k >> 2)] |= idx << (4 * j + 16 * ((k >> 1) & 1));
            }
        }
        if (__builtin_amdgcn_ballot_w64(redo) != 0 && redo) {
            // radius inf or NaN (wave-uniform test first: the common path has no select of it;
            // the empty volatile block keeps the compiler from evaluating this path speculatively)
            asm volatile("" ::: "memory");
            float T[15];
#pragma unroll
            for (int k = 0; k < 15; k++) T[k] = u2f(c_tq4_thresh[k]) * rad;
#pragma unroll
            for (int i = 0; i < 4; i++) P[i] = 0u;
#pragma unroll
            for (int k = 0; k < 8; k++)
#pragma unroll
                for (int j = 0; j < 4; j++) {
                    const float w = v[4 * k + j];
                    uint32_t idx = 0;
#pragma unroll
                    for (int t = 0; t < 15; t++) idx += (w > T[t]) ? 1u : 0u;
                    P[2 * (k & 1) + (k >> 2)] |= idx << (4 * j + 16 * ((k >> 1) & 1));
                }
        }
        // lanes q and q ^ 1 (lane u ^ 1) own the two halves of each 4-byte word at
        // byte 32 k + 2 (q & ~1): the even lane assembles even k, the odd lane odd k
        const uint32_t send0 = qodd ? P[0] : P[2], send1 = qodd ? P[1] : P[3];
        const uint32_t keep0 = qodd ? P[2] : P[0], keep1 = qodd ? P[3] : P[1];
        const uint32_t r0 = (uint32_t)__builtin_amdgcn_mov_dpp((int)send0, DPP_XOR1, 0xF, 0xF, false);
        const uint32_t r1 = (uint32_t)__builtin_amdgcn_mov_dpp((int)send1, DPP_XOR1, 0xF, 0xF, false);
        // Unconditional stores (no branch): a row slot past the end loaded the last row
        // and writes that row's bytes again (identical values), and all 16 lanes of a
        // row store its radius.
        const int64_t srow = min(row, n_rows - 1);
        uint32_t* cr = reinterpret_cast<uint32_t*>(codes + srow * (D / 2) + 2 * (q & 14) + 32 * (qodd ? 1 : 0));
        __builtin_nontemporal_store(__builtin_amdgcn_perm(r0, keep0, sel_lo), cr);       // k = 0 / 1
        __builtin_nontemporal_store(__builtin_amdgcn_perm(r0, keep0, sel_hi), cr + 16);  // k = 2 / 3
        __builtin_nontemporal_store(__builtin_amdgcn_perm(r1, keep1, sel_lo), cr + 32);  // k = 4 / 5
        __builtin_nontemporal_store(__builtin_amdgcn_perm(r1, keep1, sel_hi), cr + 48);  // k = 6 / 7
        __builtin_nontemporal_store(rad, radii + srow);
        // wave-uniform test: a wave's last iteration issues no load it would wait on at the end
        if (base + stride < n_rows) load(base + stride, nv);
    }
}

// ---- conversion probe ---------------------------------------------------------
__global__ void k_convert(int kind, const void* __restrict__ in, int64_t n, void* __restrict__ out) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
        switch (kind) {
            case KVQ_CVT_F32_TO_E4M3:
                ((uint8_t*)out)[i] = (uint8_t)(e4m3x2_rne(((const float*)in)[i], 0.0f) & 0xFFu);
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

int host_codebook(int bits, float* levels, float* thresholds) {
    static const uint32_t lv3[8] = KVQ_TQ3_LEVEL_BITS, th3[7] = KVQ_TQ3_THRESH_BITS;
    static const uint32_t lv4[16] = KVQ_TQ4_LEVEL_BITS, th4[15] = KVQ_TQ4_THRESH_BITS;
    static const uint32_t lv6[64] = KVQ_TQ6_LEVEL_BITS, th6[63] = KVQ_TQ6_THRESH_BITS;
    const uint32_t* lv = bits == 3 ? lv3 : bits == 4 ? lv4 : bits == 6 ? lv6 : nullptr;
    const uint32_t* th = bits == 3 ? th3 : bits == 4 ? th4 : bits == 6 ? th6 : nullptr;
    if (!lv) return -1;
    const int n = 1 << bits;
    if (levels)
        for (int k = 0; k < n; k++) std::memcpy(&levels[k], &lv[k], 4);
    if (thresholds)
        for (int k = 0; k < n - 1; k++) std::memcpy(&thresholds[k], &th[k], 4);
    return n;
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

hipError_t launch_encode_tq(int bits, const float* x, int64_t n_rows, int dim, const uint8_t* sign_mask,
                            uint8_t* codes, float* radii, hipStream_t st) {
    if (n_rows == 0) return hipSuccess;
    // the 512-wide kernel's stores need 8-byte (6 bits) or 4-byte (3, 4 bits) aligned rows
    const uintptr_t calign = bits == 6 ? 7u : 3u;
    if (dim == 512 && (bits == 3 || bits == 4 || bits == 6) && ((uintptr_t)codes & calign) == 0) {
        const int64_t waves = (n_rows + D512_ROWS - 1) / D512_ROWS;
        int64_t wgs = (waves + ENC_WAVES - 1) / ENC_WAVES;
        if (wgs > D512_MAX_WGS) wgs = D512_MAX_WGS;
        const dim3 grid((unsigned)wgs), block(ENC_WAVES * KVQ_WAVE);
        if (bits == 3) hipLaunchKernelGGL(k_encode_tq_d512<3>, grid, block, 0, st, x, n_rows, sign_mask, codes, radii);
        else if (bits == 6) hipLaunchKernelGGL(k_encode_tq_d512<6>, grid, block, 0, st, x, n_rows, sign_mask, codes, radii);
        else hipLaunchKernelGGL(k_encode_tq_d512<4>, grid, block, 0, st, x, n_rows, sign_mask, codes, radii);
        return hipGetLastError();
    }
    const int64_t rows_per_wave = KVQ_WAVE / (dim / 8);
    const int64_t waves = (n_rows + rows_per_wave - 1) / rows_per_wave;
    int64_t wgs = (waves + ENC_WAVES - 1) / ENC_WAVES;
    if (wgs > 4096) wgs = 4096;  // 16 waves per CU; the kernel strides over the rest
    const dim3 grid((unsigned)wgs), block(ENC_WAVES * KVQ_WAVE);
    if (bits == 3) hipLaunchKernelGGL(k_encode_tq<3>, grid, block, 0, st, x, n_rows, dim, sign_mask, codes, radii);
    else if (bits == 6) hipLaunchKernelGGL(k_encode_tq<6>, grid, block, 0, st, x, n_rows, dim, sign_mask, codes, radii);
    else hipLaunchKernelGGL(k_encode_tq<4>, grid, block, 0, st, x, n_rows, dim, sign_mask, codes, radii);
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
