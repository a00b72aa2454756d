// kvq_attn.hip -- absorbed-MLA decode attention over quantized latent rows
// (gfx950).
//
// What is computed (colibri PR #399 "KV cache quantization: fp8 (KV8) + 4-bit
// TurboQuant (KV_TQ) ...": commit 6, the fused decode with a 3-way qmode --
// score a_score8 and context a_clat8 over fp8 rows; commit 2, split-T kernels;
// "Ready for review", the native 4-bit consumer: rotate q once per head, dot the
// codes through the codebook, un-rotate the weighted sum):
//
//   s_t = sm * (rho_t <q, c_t> + <q_rope, k_rope_t>),  p = softmax(s),
//   o   = sum_t p_t rho_t c_t
//
// where c_t is the decoded code row (fp8: e4m3 values, rho_t = scale; TQ4: the
// codebook levels, rho_t = radius / sqrt(512), q replaced by R q, and o
// un-rotated by R^T after the merge).  The latent rows are never rebuilt.
//
// Pipeline (all on the caller's stream, no host synchronisation):
//   1. k_plan     -- per-sequence split counts -> prefix (ragged batches);
//   2. k_qrot     -- TQ4 only: q~ = H D q / sqrt(512) per (sequence, head);
//   3. k_attn_*   -- one workgroup per (T-split, head group): online softmax
//                    over the split's rows, partial (m, l, O) to the workspace;
//   4. k_merge    -- one wave per (sequence, head): combine the splits,
//                    TQ4 un-rotation, write out / lse.
//
// Matrix-core path: the tile's codes are converted exactly to fp16 in LDS (row
// major for the score, transposed for PV); per wave 16x16x32 MFMAs compute
// S^T = X q^T (16 rows x 16 heads, K = 512 latent + 64 rope) with the latent
// and rope parts in separate accumulators so rho_t is applied in fp32;
// the probabilities come out of the score accumulators in exactly the layout
// the PV step needs as its B operand (the PV contraction's K order is a
// permutation of the tile's rows), and O^T = X^T P'^T accumulates 512 x 16 in
// 32 accumulator blocks.
#include "kvq_device.h"
#include "kvq_internal.h"
#include "kvq_codebook.inc"

namespace kvq {

namespace {

__constant__ uint32_t c_tq4_level[16] = KVQ_TQ4_LEVEL_BITS;

constexpr int DL = 512;  // latent width
constexpr int DR = 64;   // rope width
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;
constexpr float INV_SQRT_DL = 0.044194173824159216f;  // 1 / sqrt(512)

struct Plan {
    int64_t* chunk_prefix;  // [n_seqs + 1]
    float* q_rot;           // [n_seqs][H][512] (TQ4) or nullptr
    float* part_m;          // [max_chunks][H]
    float* part_l;          // [max_chunks][H]
    float* part_o;          // [max_chunks][H][512]
    int64_t max_chunks;
    int split_rows;
    int heads_per_group;
    int n_groups;
};

// ---- workspace plan ------------------------------------------------------------

constexpr int F32_HEADS = 8;
constexpr int MF_WAVE_HEADS = 16;
constexpr int MF_TILE = 32;

int auto_split_rows(const kvq_attn_args& a) {
    if (a.precision == KVQ_PREC_FP32) return 512;
    // about one workgroup per compute unit across all sequences and head groups
    const int heads_per_group = MF_WAVE_HEADS * ((a.n_heads + MF_WAVE_HEADS - 1) / MF_WAVE_HEADS > 4
                                                     ? 4
                                                     : (a.n_heads + MF_WAVE_HEADS - 1) / MF_WAVE_HEADS);
    const int64_t groups = (a.n_heads + heads_per_group - 1) / heads_per_group;
    const int64_t target_chunks = 512 / groups;
    int64_t split = (a.total_rows + target_chunks - 1) / (target_chunks > 0 ? target_chunks : 1);
    split = (split + MF_TILE - 1) / MF_TILE * MF_TILE;
    if (split < 128) split = 128;
    if (split > (1 << 20)) split = 1 << 20;
    return (int)split;
}

Plan make_plan(const kvq_attn_args& a, void* ws) {
    Plan p{};
    p.split_rows = a.split_rows > 0 ? a.split_rows : auto_split_rows(a);
    if (a.precision == KVQ_PREC_FP32) {
        p.heads_per_group = F32_HEADS;
    } else {
        int nw = (a.n_heads + MF_WAVE_HEADS - 1) / MF_WAVE_HEADS;
        if (nw > 4) nw = 4;
        p.heads_per_group = nw * MF_WAVE_HEADS;
    }
    p.n_groups = (a.n_heads + p.heads_per_group - 1) / p.heads_per_group;
    p.max_chunks = (int64_t)a.n_seqs + a.total_rows / p.split_rows + 1;
    auto align = [](int64_t v) { return (v + 255) & ~(int64_t)255; };
    int64_t off = 0;
    char* base = (char*)ws;
    auto take = [&](int64_t bytes) {
        char* q = base ? base + off : nullptr;
        off = align(off + bytes);
        return q;
    };
    p.chunk_prefix = (int64_t*)take(sizeof(int64_t) * (a.n_seqs + 1));
    p.q_rot = a.qmode == KVQ_QMODE_TQ4 ? (float*)take(sizeof(float) * (int64_t)a.n_seqs * a.n_heads * DL) : nullptr;
    p.part_m = (float*)take(sizeof(float) * p.max_chunks * a.n_heads);
    p.part_l = (float*)take(sizeof(float) * p.max_chunks * a.n_heads);
    p.part_o = (float*)take(sizeof(float) * p.max_chunks * a.n_heads * DL);
    return p;
}

int64_t plan_bytes(const kvq_attn_args& a) {
    Plan p = make_plan(a, nullptr);
    int64_t total = 0;
    auto align = [](int64_t v) { return (v + 255) & ~(int64_t)255; };
    total += align(sizeof(int64_t) * (a.n_seqs + 1));
    if (a.qmode == KVQ_QMODE_TQ4) total += align(sizeof(float) * (int64_t)a.n_seqs * a.n_heads * DL);
    total += align(sizeof(float) * p.max_chunks * a.n_heads);
    total += align(sizeof(float) * p.max_chunks * a.n_heads);
    total += align(sizeof(float) * p.max_chunks * a.n_heads * DL);
    return total;
}

// ---- 1. plan -----------------------------------------------------------------------
// chunk_prefix[s] = sum_{s' < s} max(1, ceil(T_s' / split)); one workgroup.
__global__ __launch_bounds__(256) void k_plan(const int64_t* __restrict__ seq_offsets, int n_seqs, int split,
                                             int64_t total_rows, int64_t* __restrict__ chunk_prefix) {
    __shared__ int64_t part[256];
    const int tid = threadIdx.x;
    const int per = (n_seqs + 255) / 256;
    const int s0 = tid * per, s1 = min(n_seqs, s0 + per);
    int64_t local = 0;
    for (int s = s0; s < s1; s++) {
        const int64_t T = min(seq_offsets[s + 1], total_rows) - max(seq_offsets[s], (int64_t)0);
        local += T > 0 ? (T + split - 1) / split : 1;
    }
    part[tid] = local;
    __syncthreads();
    for (int o = 1; o < 256; o <<= 1) {  // inclusive scan
        const int64_t v = tid >= o ? part[tid - o] : 0;
        __syncthreads();
        part[tid] += v;
        __syncthreads();
    }
    int64_t run = tid > 0 ? part[tid - 1] : 0;
    for (int s = s0; s < s1; s++) {
        chunk_prefix[s] = run;
        const int64_t T = min(seq_offsets[s + 1], total_rows) - max(seq_offsets[s], (int64_t)0);
        run += T > 0 ? (T + split - 1) / split : 1;
    }
    if (tid == 255) chunk_prefix[n_seqs] = part[255];
}

__device__ __forceinline__ int find_chunk_seq(const int64_t* __restrict__ cp, int n_seqs, int64_t c) {
    int lo = 0, hi = n_seqs - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (cp[mid] <= c) lo = mid; else hi = mid - 1;
    }
    return lo;
}

// ---- 2. TQ4 query rotation ----------------------------------------------------------
// One wave per (sequence, head): q~ = H (D q) / sqrt(512), 8 consecutive per lane.
__global__ __launch_bounds__(256) void k_qrot(const float* __restrict__ q, const uint8_t* __restrict__ sign_mask,
                                             int64_t n_rows, float* __restrict__ q_rot) {
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= n_rows) return;
    const float* src = q + row * DL + lane * 8;
    float v[8];
    const uint32_t sm = sign_mask[lane];
#pragma unroll
    for (int i = 0; i < 8; i++) v[i] = ((sm >> i) & 1u) ? -src[i] : src[i];
#pragma unroll
    for (int h = 1; h < 8; h <<= 1)
#pragma unroll
        for (int i = 0; i < 8; i++)
            if (!(i & h)) {
                const float a = v[i], b = v[i + h];
                v[i] = a + b;
                v[i + h] = a - b;
            }
#pragma unroll
    for (int m = 1; m < 64; m <<= 1)
#pragma unroll
        for (int i = 0; i < 8; i++) v[i] = fwht_xlane(v[i], lane, m);
    float* dst = q_rot + row * DL + lane * 8;
#pragma unroll
    for (int i = 0; i < 8; i++) dst[i] = v[i] * INV_SQRT_DL;
}

// Decoded value of element i of a code row (fp8: e4m3 value, TQ4: codebook level).
template <int QMODE>
__device__ __forceinline__ float code_value(const uint8_t* __restrict__ row, int i) {
    if (QMODE == KVQ_QMODE_FP8) return e4m3_to_f32(row[i]);
    const uint32_t b = row[i >> 1];
    return u2f(c_tq4_level[(i & 1) ? (b >> 4) : (b & 15u)]);
}

// ---- 3a. fp32 check path ----------------------------------------------------------------
// Workgroup = (chunk, group of 8 heads), 256 threads.  Tiles of 256 rows: one
// row per thread for the scores, then thread (head = tid/32, 16 dims) for PV.
template <int QMODE>
__global__ __launch_bounds__(256) void k_attn_f32(kvq_attn_args a, Plan p, const float* __restrict__ qsrc) {
    constexpr int TILE = 256;
    __shared__ float q_s[F32_HEADS][DL];
    __shared__ float qr_s[F32_HEADS][DR];
    __shared__ float pr_s[F32_HEADS][TILE];  // scores, then p * rho
    __shared__ float red_s[F32_HEADS][2];
    const int tid = threadIdx.x;
    const int64_t c = blockIdx.x;
    if (c >= p.chunk_prefix[a.n_seqs]) return;
    const int s = find_chunk_seq(p.chunk_prefix, a.n_seqs, c);
    const int64_t seq_lo = max(a.seq_offsets[s], (int64_t)0), seq_hi = min(a.seq_offsets[s + 1], a.total_rows);
    const int64_t r0 = seq_lo + (c - p.chunk_prefix[s]) * p.split_rows;
    const int64_t r1 = min(seq_hi, r0 + (int64_t)p.split_rows);
    const int h0 = blockIdx.y * F32_HEADS;
    const int nh = min(F32_HEADS, a.n_heads - h0);
    for (int i = tid; i < F32_HEADS * DL; i += 256) {
        const int hh = i / DL, d = i % DL;
        q_s[hh][d] = hh < nh ? qsrc[((int64_t)s * a.n_heads + h0 + hh) * DL + d] : 0.0f;
    }
    for (int i = tid; i < F32_HEADS * DR; i += 256) {
        const int hh = i / DR, d = i % DR;
        qr_s[hh][d] = hh < nh ? a.q_rope[((int64_t)s * a.n_heads + h0 + hh) * DR + d] : 0.0f;
    }
    __syncthreads();
    const int cb = QMODE == KVQ_QMODE_FP8 ? DL : DL / 2;  // code bytes per row
    const int ph = tid >> 5, pd = (tid & 31) * 16;       // PV ownership
    float m_run[F32_HEADS], l_run[F32_HEADS];
#pragma unroll
    for (int hh = 0; hh < F32_HEADS; hh++) { m_run[hh] = -INFINITY; l_run[hh] = 0.0f; }
    float acc[16];
#pragma unroll
    for (int j = 0; j < 16; j++) acc[j] = 0.0f;
    for (int64_t t0 = r0; t0 < r1; t0 += TILE) {
        const int nt = (int)min((int64_t)TILE, r1 - t0);
        float sc[F32_HEADS];
        float rho = 0.0f;
        if (tid < nt) {
            const int64_t t = t0 + tid;
            rho = a.row_scale[t];
            if (QMODE == KVQ_QMODE_TQ4) rho *= INV_SQRT_DL;
            const uint8_t* row = a.codes + t * cb;
            float dot[F32_HEADS], dr[F32_HEADS];
#pragma unroll
            for (int hh = 0; hh < F32_HEADS; hh++) { dot[hh] = 0.0f; dr[hh] = 0.0f; }
            for (int d = 0; d < DL; d++) {
                const float x = code_value<QMODE>(row, d);
#pragma unroll
                for (int hh = 0; hh < F32_HEADS; hh++) dot[hh] = __builtin_fmaf(q_s[hh][d], x, dot[hh]);
            }
            const uint16_t* kr = a.k_rope + t * DR;
            for (int d = 0; d < DR; d++) {
                const float x = u2f((uint32_t)kr[d] << 16);
#pragma unroll
                for (int hh = 0; hh < F32_HEADS; hh++) dr[hh] = __builtin_fmaf(qr_s[hh][d], x, dr[hh]);
            }
#pragma unroll
            for (int hh = 0; hh < F32_HEADS; hh++) sc[hh] = a.sm_scale * (rho * dot[hh] + dr[hh]);
        } else {
#pragma unroll
            for (int hh = 0; hh < F32_HEADS; hh++) sc[hh] = -INFINITY;
        }
#pragma unroll
        for (int hh = 0; hh < F32_HEADS; hh++) pr_s[hh][tid] = sc[hh];
        __syncthreads();
        {  // tile max per head: 32 threads per head
            const int hh = tid >> 5, l32 = tid & 31;
            float mx = -INFINITY;
            for (int k = l32; k < TILE; k += 32) mx = fmaxf(mx, pr_s[hh][k]);
#pragma unroll
            for (int o = 16; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 32));
            if (l32 == 0) red_s[hh][0] = mx;
        }
        __syncthreads();
        float alpha[F32_HEADS], m_new[F32_HEADS];
#pragma unroll
        for (int hh = 0; hh < F32_HEADS; hh++) {
            m_new[hh] = fmaxf(m_run[hh], red_s[hh][0]);
            alpha[hh] = m_new[hh] == -INFINITY ? 1.0f : expf(m_run[hh] - m_new[hh]);
        }
        __syncthreads();
#pragma unroll
        for (int hh = 0; hh < F32_HEADS; hh++) {
            const float pv = tid < nt ? expf(sc[hh] - m_new[hh]) : 0.0f;
            pr_s[hh][tid] = pv;
        }
        __syncthreads();
        {  // tile sum of p per head
            const int hh = tid >> 5, l32 = tid & 31;
            float sm = 0.0f;
            for (int k = l32; k < TILE; k += 32) sm += pr_s[hh][k];
#pragma unroll
            for (int o = 16; o >= 1; o >>= 1) sm += __shfl_xor(sm, o, 32);
            if (l32 == 0) red_s[hh][1] = sm;
        }
        __syncthreads();
#pragma unroll
        for (int hh = 0; hh < F32_HEADS; hh++) {
            l_run[hh] = l_run[hh] * alpha[hh] + red_s[hh][1];
            m_run[hh] = m_new[hh];
        }
        // p * rho for PV
#pragma unroll
        for (int hh = 0; hh < F32_HEADS; hh++) pr_s[hh][tid] *= rho;
        __syncthreads();
        // PV: thread owns head ph, dims pd .. pd+15
        {
            float al = alpha[0];
#pragma unroll
            for (int hh = 1; hh < F32_HEADS; hh++) if (hh == ph) al = alpha[hh];
#pragma unroll
            for (int j = 0; j < 16; j++) acc[j] *= al;
            for (int k = 0; k < nt; k++) {
                const float w = pr_s[ph][k];
                const uint8_t* row = a.codes + (t0 + k) * cb;
#pragma unroll
                for (int j = 0; j < 16; j++) acc[j] = __builtin_fmaf(w, code_value<QMODE>(row, pd + j), acc[j]);
            }
        }
        __syncthreads();
    }
    if (ph < nh) {
        float* dst = p.part_o + (c * a.n_heads + h0 + ph) * DL + pd;
#pragma unroll
        for (int j = 0; j < 16; j++) dst[j] = acc[j];
    }
    if (tid < nh) {
        float mv = m_run[0], lv = l_run[0];
#pragma unroll
        for (int hh = 1; hh < F32_HEADS; hh++) if (hh == tid) { mv = m_run[hh]; lv = l_run[hh]; }
        p.part_m[c * a.n_heads + h0 + tid] = mv;  // natural-log units
        p.part_l[c * a.n_heads + h0 + tid] = lv;
    }
}

// ---- 3b. matrix-core path ---------------------------------------------------------------------
// Operand precision (chosen by measurement: bf16 query and probabilities cost
// 2e-3 .. 1.5e-2 of the output on these workloads, whose outputs are
// near-cancelling averages):
//  - latent codes: fp16, exact (every e4m3 value and every bf16 codebook level);
//  - latent query: per head scaled by a power of two (max |q| in [256, 512)),
//    then split q = hi + lo in fp16 (22-bit significand), two MFMA chains;
//  - rope: k_rope is bf16; the rope query is split hi + lo in bf16;
//  - probabilities p * rho_t: times a per-split power of two rs (max rho * rs in
//    [0.5, 1)), then fp16;
//  - accumulation fp32; the power-of-two scales are undone exactly in fp32.
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

constexpr int XS_STRIDE = DL + DR + 8;  // halfwords per row-major tile row (padded)
constexpr int XT_STRIDE = MF_TILE + 8;  // halfwords per transposed tile row (padded)

__device__ __forceinline__ f16x8_t as_f16x8(uint4 u) { return __builtin_bit_cast(f16x8_t, u); }
__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8_t, u); }

__device__ __forceinline__ uint32_t f16_bits(float f) {
    return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)f);  // round to nearest even
}
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) { return f16_bits(lo) | (f16_bits(hi) << 16); }
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return f32_to_bf16_rne(lo) | (f32_to_bf16_rne(hi) << 16);
}

// e4m3 byte pair (bits 0..15 of w when HI is false, 16..31 otherwise) -> two fp16, exact.
template <bool HI>
__device__ __forceinline__ uint32_t e4m3x2_to_f16x2(uint32_t w) {
    const f16x2_t h = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, HI);
    return __builtin_bit_cast(uint32_t, h);
}

// TQ4 nibble -> fp16 bits of the codebook level (exact).
__device__ __forceinline__ uint32_t tq4_f16(uint32_t idx) { return f16_bits(u2f(c_tq4_level[idx])); }

// Power of two 2^k with max_abs * 2^k in [lo_target, 2 lo_target); 1 if max_abs == 0.
__device__ __forceinline__ float pow2_scale_for(float max_abs, int log2_target) {
    if (!(max_abs > 0.0f)) return 1.0f;
    int e = (int)((f2u(max_abs) >> 23) & 255u) - 127;  // floor(log2) for normal values
    if (e < -126) e = -126;
    int k = log2_target - e;
    if (k > 127) k = 127;
    if (k < -126) k = -126;
    return u2f((uint32_t)(k + 127) << 23);
}

// Workgroup = (chunk, head group of 16 * nw heads), nw = blockDim.x / 64 waves,
// wave w owns heads h0 + 16 w .. +15.  Tiles of 32 rows.
template <int QMODE>
__global__ __launch_bounds__(256) void k_attn_mfma(kvq_attn_args a, Plan p, const float* __restrict__ qsrc) {
    __shared__ __align__(16) uint16_t xs[MF_TILE][XS_STRIDE];
    __shared__ __align__(16) uint16_t xt[DL][XT_STRIDE];
    __shared__ float rho_s[MF_TILE];
    __shared__ float red_s[4];
    const int tid = threadIdx.x;
    const int nthreads = blockDim.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int g = lane >> 4, n = lane & 15;
    const int64_t c = blockIdx.x;
    if (c >= p.chunk_prefix[a.n_seqs]) return;
    const int s = find_chunk_seq(p.chunk_prefix, a.n_seqs, c);
    const int64_t seq_lo = max(a.seq_offsets[s], (int64_t)0), seq_hi = min(a.seq_offsets[s + 1], a.total_rows);
    const int64_t r0 = seq_lo + (c - p.chunk_prefix[s]) * p.split_rows;
    const int64_t r1 = min(seq_hi, r0 + (int64_t)p.split_rows);
    const int h0 = blockIdx.y * p.heads_per_group + wave * MF_WAVE_HEADS;
    const int head = h0 + n;
    const bool head_ok = head < a.n_heads;
    const float rho_mul = QMODE == KVQ_QMODE_TQ4 ? INV_SQRT_DL : 1.0f;

    // ---- per-split probability scale rs from the largest row scale
    float rmax = 0.0f;
    for (int64_t t = r0 + tid; t < r1; t += nthreads) rmax = fmaxf(rmax, fabsf(a.row_scale[t]));
    rmax = wave_max(rmax);
    if (lane == 0) red_s[wave] = rmax;
    __syncthreads();
    rmax = red_s[0];
    for (int i = 1; i < nthreads / 64; i++) rmax = fmaxf(rmax, red_s[i]);
    const float rs = pow2_scale_for(rmax * rho_mul, -1);  // max rho * rs in [0.5, 1)

    // ---- query operands: lane (g, n) holds q[head][32 ks + 8 g .. + 7]
    const float* ql = qsrc + ((int64_t)s * a.n_heads + (head_ok ? head : 0)) * DL;
    const float* qr = a.q_rope + ((int64_t)s * a.n_heads + (head_ok ? head : 0)) * DR;
    float qmax = 0.0f;
#pragma unroll
    for (int ks = 0; ks < 16; ks++)
#pragma unroll
        for (int i = 0; i < 8; i++) qmax = fmaxf(qmax, head_ok ? fabsf(ql[32 * ks + 8 * g + i]) : 0.0f);
    qmax = fmaxf(qmax, __shfl_xor(qmax, 16, 64));
    qmax = fmaxf(qmax, __shfl_xor(qmax, 32, 64));
    const float qs = pow2_scale_for(qmax, 8);  // max |q| * qs in [256, 512)
    const float qinv = 1.0f / qs;              // exact
    uint4 qh[16], qlo[16], rh[2], rl[2];
#pragma unroll
    for (int ks = 0; ks < 16; ks++) {
        uint32_t hw[4], lw[4];
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const float f0 = head_ok ? ql[32 * ks + 8 * g + 2 * i] * qs : 0.0f;
            const float f1 = head_ok ? ql[32 * ks + 8 * g + 2 * i + 1] * qs : 0.0f;
            const float h0f = (float)(_Float16)f0, h1f = (float)(_Float16)f1;
            hw[i] = pack_f16x2(h0f, h1f);
            lw[i] = pack_f16x2(f0 - h0f, f1 - h1f);
        }
        qh[ks] = make_uint4(hw[0], hw[1], hw[2], hw[3]);
        qlo[ks] = make_uint4(lw[0], lw[1], lw[2], lw[3]);
    }
#pragma unroll
    for (int ks = 0; ks < 2; ks++) {
        uint32_t hw[4], lw[4];
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const float f0 = head_ok ? qr[32 * ks + 8 * g + 2 * i] : 0.0f;
            const float f1 = head_ok ? qr[32 * ks + 8 * g + 2 * i + 1] : 0.0f;
            const float b0 = u2f(f32_to_bf16_rne(f0) << 16), b1 = u2f(f32_to_bf16_rne(f1) << 16);
            hw[i] = pack_bf16x2(b0, b1);
            lw[i] = pack_bf16x2(f0 - b0, f1 - b1);
        }
        rh[ks] = make_uint4(hw[0], hw[1], hw[2], hw[3]);
        rl[ks] = make_uint4(lw[0], lw[1], lw[2], lw[3]);
    }
    const float c2 = a.sm_scale * LOG2E;  // scores in log2 units
    f32x4_t acc_o[32];
#pragma unroll
    for (int mb = 0; mb < 32; mb++) acc_o[mb] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    float m_run = -INFINITY, l_part = 0.0f;
    const int cb = QMODE == KVQ_QMODE_FP8 ? DL : DL / 2;

    for (int64_t t0 = r0; t0 < r1; t0 += MF_TILE) {
        const int nt = (int)min((int64_t)MF_TILE, r1 - t0);
        // ---- stage the tile: codes -> fp16 (row-major xs and transposed xt), rope, rho
        if (QMODE == KVQ_QMODE_FP8) {
            for (int u = tid; u < MF_TILE * 32; u += nthreads) {
                const int row = u >> 5, col = (u & 31) * 16;
                uint4 raw = make_uint4(0, 0, 0, 0);
                if (row < nt) raw = *reinterpret_cast<const uint4*>(a.codes + (t0 + row) * cb + col);
                const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
                uint32_t o[8];
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    o[2 * i] = e4m3x2_to_f16x2<false>(w[i]);
                    o[2 * i + 1] = e4m3x2_to_f16x2<true>(w[i]);
                }
                *reinterpret_cast<uint4*>(&xs[row][col]) = make_uint4(o[0], o[1], o[2], o[3]);
                *reinterpret_cast<uint4*>(&xs[row][col + 8]) = make_uint4(o[4], o[5], o[6], o[7]);
#pragma unroll
                for (int i = 0; i < 8; i++) {
                    xt[col + 2 * i][row] = (uint16_t)(o[i] & 0xFFFF);
                    xt[col + 2 * i + 1][row] = (uint16_t)(o[i] >> 16);
                }
            }
        } else {
            for (int u = tid; u < MF_TILE * 16; u += nthreads) {
                const int row = u >> 4, col = (u & 15) * 32;
                uint4 raw = make_uint4(0, 0, 0, 0);
                if (row < nt) raw = *reinterpret_cast<const uint4*>(a.codes + (t0 + row) * cb + col / 2);
                const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
                uint32_t o[16];
#pragma unroll
                for (int i = 0; i < 4; i++)
#pragma unroll
                    for (int k = 0; k < 4; k++) {
                        const uint32_t byte = (w[i] >> (8 * k)) & 0xFF;
                        o[4 * i + k] = tq4_f16(byte & 15u) | (tq4_f16(byte >> 4) << 16);
                    }
                if (row >= nt) {
#pragma unroll
                    for (int i = 0; i < 16; i++) o[i] = 0;
                }
#pragma unroll
                for (int q = 0; q < 4; q++)
                    *reinterpret_cast<uint4*>(&xs[row][col + 8 * q]) =
                        make_uint4(o[4 * q], o[4 * q + 1], o[4 * q + 2], o[4 * q + 3]);
#pragma unroll
                for (int i = 0; i < 16; i++) {
                    xt[col + 2 * i][row] = (uint16_t)(o[i] & 0xFFFF);
                    xt[col + 2 * i + 1][row] = (uint16_t)(o[i] >> 16);
                }
            }
        }
        for (int u = tid; u < MF_TILE * 8; u += nthreads) {  // rope (bf16), 8 units of 16 bytes per row
            const int row = u >> 3, col = (u & 7) * 8;
            uint4 raw = make_uint4(0, 0, 0, 0);
            if (row < nt) raw = *reinterpret_cast<const uint4*>(a.k_rope + (t0 + row) * DR + col);
            *reinterpret_cast<uint4*>(&xs[row][DL + col]) = raw;
        }
        for (int u = tid; u < MF_TILE; u += nthreads) rho_s[u] = u < nt ? a.row_scale[t0 + u] * rho_mul : 0.0f;
        __syncthreads();

        // ---- scores S^T (rows x heads), two 16-row blocks
        f32x4_t sl[2], sr[2];
#pragma unroll
        for (int rb = 0; rb < 2; rb++) {
            sl[rb] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
            sr[rb] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
            const uint16_t* xrow = &xs[16 * rb + n][8 * g];
#pragma unroll
            for (int ks = 0; ks < 16; ks++) {
                const f16x8_t av = as_f16x8(*reinterpret_cast<const uint4*>(xrow + 32 * ks));
                sl[rb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, as_f16x8(qh[ks]), sl[rb], 0, 0, 0);
                sl[rb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, as_f16x8(qlo[ks]), sl[rb], 0, 0, 0);
            }
#pragma unroll
            for (int ks = 0; ks < 2; ks++) {
                const bf16x8_t av = as_bf16x8(*reinterpret_cast<const uint4*>(xrow + DL + 32 * ks));
                sr[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, as_bf16x8(rh[ks]), sr[rb], 0, 0, 0);
                sr[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, as_bf16x8(rl[ks]), sr[rb], 0, 0, 0);
            }
        }
        // lane (g, n): rows 16 rb + 4 g + r of head n
        float sc[2][4], rr[2][4];
        float tmax = -INFINITY;
#pragma unroll
        for (int rb = 0; rb < 2; rb++)
#pragma unroll
            for (int r = 0; r < 4; r++) {
                const int t = 16 * rb + 4 * g + r;
                rr[rb][r] = rho_s[t];
                const float v = t < nt ? c2 * (rr[rb][r] * (sl[rb][r] * qinv) + sr[rb][r]) : -INFINITY;
                sc[rb][r] = v;
                tmax = fmaxf(tmax, v);
            }
        tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
        const float m_new = fmaxf(m_run, tmax);
        const float alpha = (m_new == -INFINITY) ? 1.0f : exp2f(m_run - m_new);
        float psum = 0.0f;
        uint32_t pb[4];
#pragma unroll
        for (int rb = 0; rb < 2; rb++) {
            float pw[4];
#pragma unroll
            for (int r = 0; r < 4; r++) {
                const float pv = (sc[rb][r] == -INFINITY) ? 0.0f : exp2f(sc[rb][r] - m_new);
                psum += pv;
                pw[r] = pv * (rr[rb][r] * rs);
            }
            pb[2 * rb] = pack_f16x2(pw[0], pw[1]);
            pb[2 * rb + 1] = pack_f16x2(pw[2], pw[3]);
        }
        l_part = l_part * alpha + psum;
        m_run = m_new;
        // PV B operand: k-slots 8 g + j <-> rows {4g..4g+3, 16+4g..16+4g+3}
        const f16x8_t bop = as_f16x8(make_uint4(pb[0], pb[1], pb[2], pb[3]));
#pragma unroll
        for (int mb = 0; mb < 32; mb++) {
            const uint16_t* col = &xt[16 * mb + n][0];
            const uint2 lo = *reinterpret_cast<const uint2*>(col + 4 * g);
            const uint2 hi = *reinterpret_cast<const uint2*>(col + 16 + 4 * g);
            const f16x8_t aop = as_f16x8(make_uint4(lo.x, lo.y, hi.x, hi.y));
            acc_o[mb] = acc_o[mb] * alpha;
            acc_o[mb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(aop, bop, acc_o[mb], 0, 0, 0);
        }
        __syncthreads();
    }
    // ---- partials: lane (g, n) holds O[head n][16 mb + 4 g + r] * rs
    l_part += __shfl_xor(l_part, 16, 64);
    l_part += __shfl_xor(l_part, 32, 64);
    const float rsinv = 1.0f / rs;  // exact
    if (head_ok) {
        float* dst = p.part_o + (c * a.n_heads + head) * DL + 4 * g;
#pragma unroll
        for (int mb = 0; mb < 32; mb++)
            *reinterpret_cast<float4*>(dst + 16 * mb) =
                make_float4(acc_o[mb][0] * rsinv, acc_o[mb][1] * rsinv, acc_o[mb][2] * rsinv, acc_o[mb][3] * rsinv);
        if (g == 0) {
            p.part_m[c * a.n_heads + head] = m_run;  // log2 units
            p.part_l[c * a.n_heads + head] = l_part;
        }
    }
}

// ---- 4. merge --------------------------------------------------------------------------------
// One wave per (sequence, head); lane holds dims 8 lane .. 8 lane + 7.
template <bool TQ4, bool LOG2>
__global__ __launch_bounds__(256) void k_merge(kvq_attn_args a, Plan p) {
    const int lane = threadIdx.x & 63;
    const int64_t item = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (item >= (int64_t)a.n_seqs * a.n_heads) return;
    const int s = (int)(item / a.n_heads), h = (int)(item % a.n_heads);
    const int64_t c0 = min(p.chunk_prefix[s], p.max_chunks), c1 = min(p.chunk_prefix[s + 1], p.max_chunks);
    float M = -INFINITY;
    for (int64_t c = c0 + lane; c < c1; c += 64) M = fmaxf(M, p.part_m[c * a.n_heads + h]);
    M = wave_max(M);
    float L = 0.0f;
    float o[8];
#pragma unroll
    for (int i = 0; i < 8; i++) o[i] = 0.0f;
    if (M != -INFINITY) {
        for (int64_t c = c0; c < c1; c++) {
            const float mc = p.part_m[c * a.n_heads + h];
            const float w = (mc == -INFINITY) ? 0.0f : (LOG2 ? exp2f(mc - M) : expf(mc - M));
            L += w * p.part_l[c * a.n_heads + h];
            const float4* src = reinterpret_cast<const float4*>(p.part_o + (c * a.n_heads + h) * DL + 8 * lane);
            const float4 u = src[0], v = src[1];
            o[0] += w * u.x; o[1] += w * u.y; o[2] += w * u.z; o[3] += w * u.w;
            o[4] += w * v.x; o[5] += w * v.y; o[6] += w * v.z; o[7] += w * v.w;
        }
    }
    const float inv = L > 0.0f ? 1.0f / L : 0.0f;
#pragma unroll
    for (int i = 0; i < 8; i++) o[i] *= inv;
    if (TQ4) {  // o = D H o~ / sqrt(512)
#pragma unroll
        for (int hh = 1; hh < 8; hh <<= 1)
#pragma unroll
            for (int i = 0; i < 8; i++)
                if (!(i & hh)) {
                    const float x = o[i], y = o[i + hh];
                    o[i] = x + y;
                    o[i + hh] = x - y;
                }
#pragma unroll
        for (int m = 1; m < 64; m <<= 1)
#pragma unroll
            for (int i = 0; i < 8; i++) o[i] = fwht_xlane(o[i], lane, m);
        const uint32_t sm = a.sign_mask[lane];
#pragma unroll
        for (int i = 0; i < 8; i++) {
            o[i] *= INV_SQRT_DL;
            if ((sm >> i) & 1u) o[i] = -o[i];
        }
    }
    float4* dst = reinterpret_cast<float4*>(a.out + item * DL + 8 * lane);
    dst[0] = make_float4(o[0], o[1], o[2], o[3]);
    dst[1] = make_float4(o[4], o[5], o[6], o[7]);
    if (a.lse && lane == 0) {
        float v;
        if (!(L > 0.0f)) v = -INFINITY;
        else v = LOG2 ? (M + log2f(L)) * LN2 : M + logf(L);
        a.lse[item] = v;
    }
}

}  // namespace

int64_t attn_workspace_bytes(const kvq_attn_args& a) { return plan_bytes(a); }

hipError_t launch_decode_attn_stage(const kvq_attn_args& a, int stage, void* ws, hipStream_t st) {
    Plan p = make_plan(a, ws);
    const float* qsrc = a.qmode == KVQ_QMODE_TQ4 ? p.q_rot : a.q_lat;
    switch (stage) {
        case KVQ_STAGE_PLAN:
            hipLaunchKernelGGL(k_plan, dim3(1), dim3(256), 0, st, a.seq_offsets, a.n_seqs, p.split_rows, a.total_rows,
                               p.chunk_prefix);
            break;
        case KVQ_STAGE_QROT:
            if (a.qmode == KVQ_QMODE_TQ4) {
                const int64_t rows = (int64_t)a.n_seqs * a.n_heads;
                hipLaunchKernelGGL(k_qrot, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, st, a.q_lat, a.sign_mask,
                                   rows, p.q_rot);
            }
            break;
        case KVQ_STAGE_SPLITS: {
            const dim3 grid((unsigned)p.max_chunks, (unsigned)p.n_groups);
            if (a.precision == KVQ_PREC_FP32) {
                if (a.qmode == KVQ_QMODE_FP8)
                    hipLaunchKernelGGL(k_attn_f32<KVQ_QMODE_FP8>, grid, dim3(256), 0, st, a, p, qsrc);
                else
                    hipLaunchKernelGGL(k_attn_f32<KVQ_QMODE_TQ4>, grid, dim3(256), 0, st, a, p, qsrc);
            } else {
                const dim3 block(p.heads_per_group / MF_WAVE_HEADS * 64);
                if (a.qmode == KVQ_QMODE_FP8)
                    hipLaunchKernelGGL(k_attn_mfma<KVQ_QMODE_FP8>, grid, block, 0, st, a, p, qsrc);
                else
                    hipLaunchKernelGGL(k_attn_mfma<KVQ_QMODE_TQ4>, grid, block, 0, st, a, p, qsrc);
            }
            break;
        }
        default: {
            const int64_t items = (int64_t)a.n_seqs * a.n_heads;
            const dim3 mgrid((unsigned)((items + 3) / 4));
            const bool log2dom = a.precision != KVQ_PREC_FP32;
            if (a.qmode == KVQ_QMODE_TQ4) {
                if (log2dom) hipLaunchKernelGGL((k_merge<true, true>), mgrid, dim3(256), 0, st, a, p);
                else hipLaunchKernelGGL((k_merge<true, false>), mgrid, dim3(256), 0, st, a, p);
            } else {
                if (log2dom) hipLaunchKernelGGL((k_merge<false, true>), mgrid, dim3(256), 0, st, a, p);
                else hipLaunchKernelGGL((k_merge<false, false>), mgrid, dim3(256), 0, st, a, p);
            }
            break;
        }
    }
    return hipGetLastError();
}

hipError_t launch_decode_attn(const kvq_attn_args& a, void* ws, int64_t ws_bytes, hipStream_t st) {
    (void)ws_bytes;
    for (int stage = KVQ_STAGE_PLAN; stage <= KVQ_STAGE_MERGE; stage++) {
        const hipError_t e = launch_decode_attn_stage(a, stage, ws, st);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace kvq
