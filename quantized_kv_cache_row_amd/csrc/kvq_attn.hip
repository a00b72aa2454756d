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
//   prep  -- fp32 check path: k_plan (per-sequence T-split counts -> prefix)
//            and, TQ4, k_qrot (R q in fp32); matrix-core path, TQ4:
//            k_qprep_tq4 (R q as fp16 operands).  The matrix-core split
//            kernels plan their chunk themselves, the fp8 one also prepares
//            its query;
//   split -- k_attn_*: online softmax over every T-split, partial (m, l, O);
//   merge -- k_merge: combine the splits, TQ4 un-rotation, write out / lse.
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

constexpr int F32_HEADS = 8;      // fp32 path: heads per workgroup
constexpr int MF_HEADS = 16;      // matrix-core path: heads per workgroup (one MFMA N block)
constexpr int MF_WAVES = 4;       // matrix-core path: waves per workgroup, splitting the rows
constexpr int MF_TILE = 32;       // rows per wave tile
constexpr int TQ4_HEADS = 64;    // TQ4 matrix-core path: heads per workgroup (4 waves x 16)
constexpr int QPACK_U4 = 80;      // TQ4: uint4 per prepared query (fp16 latent 64, rope hi 8, rope lo 8)
constexpr int QP_RH = 64, QP_RL = 72;
constexpr int N_XCD = 8;          // MI355X: workgroups are dealt round-robin to 8 XCDs
constexpr float LAZY_LOG2 = 8.0f; // running-max slack before the accumulators are rescaled

struct Plan {
    int64_t* chunk_prefix;  // [n_seqs + 1]
    float* q_rot;           // fp32 path, TQ4: [n_seqs][H][512]
    uint4* q_pack;          // matrix-core path, TQ4: [n_seqs][H padded to 64][QPACK_U4]
    float* q_inv;           // matrix-core path, TQ4: [n_seqs][H padded to 64]
    float* part_m;          // [max_chunks][H]
    float* part_l;          // [max_chunks][H]
    float* part_o;          // [max_chunks][H][512]
    int64_t max_chunks;
    int split_rows;
    int heads_per_group;
    int n_groups;
    int heads_padded;
    int64_t chunks_per_xcd; // matrix-core grid: chunk c runs on XCD c % 8, all its head groups together
};

// ---- workspace plan ------------------------------------------------------------

int auto_split_rows(const kvq_attn_args& a) {
    if (a.precision == KVQ_PREC_FP32) return 512;
    if (a.qmode == KVQ_QMODE_TQ4) {
        // one workgroup per compute unit over all splits and groups of 64 heads,
        // whole tiles, at least 8 tiles per split
        const int64_t groups = (a.n_heads + TQ4_HEADS - 1) / TQ4_HEADS;
        int64_t split = (a.total_rows * groups + 255) / 256;
        if (split < 8 * MF_TILE) split = 8 * MF_TILE;
        split = (split + MF_TILE - 1) / MF_TILE * MF_TILE;
        if (split > (1 << 24)) split = 1 << 24;
        return (int)split;
    }
    // Large splits keep the partial states small next to the KV bytes they
    // summarize (a partial is 128 heads x 2 KB per split); about two
    // workgroups per compute unit over all splits and head groups.
    const int64_t groups = (a.n_heads + MF_HEADS - 1) / MF_HEADS;
    int64_t split = (a.total_rows * groups + 511) / 512;
    if (split < 1024) split = 1024;
    split = (split + MF_WAVES * MF_TILE - 1) / (MF_WAVES * MF_TILE) * (MF_WAVES * MF_TILE);
    if (split > (1 << 24)) split = 1 << 24;
    return (int)split;
}

Plan make_plan(const kvq_attn_args& a, void* ws, int64_t* bytes_out) {
    Plan p{};
    p.split_rows = a.split_rows > 0 ? a.split_rows : auto_split_rows(a);
    const bool f32 = a.precision == KVQ_PREC_FP32;
    p.heads_per_group = f32 ? F32_HEADS : (a.qmode == KVQ_QMODE_TQ4 ? TQ4_HEADS : MF_HEADS);
    p.n_groups = (a.n_heads + p.heads_per_group - 1) / p.heads_per_group;
    p.heads_padded = p.n_groups * p.heads_per_group;
    // sum_s max(1, ceil(T_s / split)) over T_s summing to at most total_rows is at
    // most floor(total / split) + n_seqs, and at most ceil(total / split) + n_seqs - 1
    // unless every sequence is empty
    p.max_chunks = std::max<int64_t>(a.n_seqs, std::min<int64_t>(a.total_rows / p.split_rows + a.n_seqs,
                                                                  (a.total_rows + p.split_rows - 1) / p.split_rows +
                                                                      a.n_seqs - 1));
    p.chunks_per_xcd = (p.max_chunks + N_XCD - 1) / N_XCD;
    auto align = [](int64_t v) { return (v + 255) & ~(int64_t)255; };
    int64_t off = 0;
    char* base = (char*)ws;
    auto take = [&](int64_t bytes) {
        char* q = base ? base + off : nullptr;
        off = align(off + bytes);
        return q;
    };
    p.chunk_prefix = (int64_t*)take(sizeof(int64_t) * (a.n_seqs + 1));
    if (f32 && a.qmode == KVQ_QMODE_TQ4) p.q_rot = (float*)take(sizeof(float) * (int64_t)a.n_seqs * a.n_heads * DL);
    if (!f32 && a.qmode == KVQ_QMODE_TQ4) {
        const int64_t rows_q = (int64_t)a.n_seqs * p.heads_padded;
        p.q_pack = (uint4*)take(sizeof(uint4) * rows_q * QPACK_U4);
        p.q_inv = (float*)take(sizeof(float) * rows_q);
    }
    p.part_m = (float*)take(sizeof(float) * p.max_chunks * a.n_heads);
    p.part_l = (float*)take(sizeof(float) * p.max_chunks * a.n_heads);
    p.part_o = (float*)take(sizeof(float) * p.max_chunks * a.n_heads * DL);
    if (bytes_out) *bytes_out = off;
    return p;
}

int64_t plan_bytes(const kvq_attn_args& a) {
    int64_t n = 0;
    make_plan(a, nullptr, &n);
    return n;
}

// ---- 0. plan -----------------------------------------------------------------------
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

// ---- 1a. TQ4 query rotation (fp32 path) ----------------------------------------------------------
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

// ---- 2a. fp32 check path ----------------------------------------------------------------
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
    if (c >= p.max_chunks || c >= p.chunk_prefix[a.n_seqs]) return;
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

// ---- matrix-core path ------------------------------------------------------------------------
// Operand precision (chosen by measurement: bf16 query and probabilities cost
// 2e-3 .. 1.5e-2 of the output on these workloads, whose outputs are
// near-cancelling averages):
//  - latent codes: fp16, exact (every e4m3 value and every bf16 codebook level);
//  - latent query: per head scaled by a power of two (max |q| in [256, 512)),
//    then rounded to fp16 (fp8 rows; an emulation of this arithmetic against
//    the fp64 evaluation measures 3.4e-4, and 7.0e-4 with 50x sharper scores);
//    the TQ4 kernel also applies the fp16 remainder q - hi;
//  - rope: k_rope is bf16; the rope query is split hi + lo in bf16;
//  - probabilities p * rho_t: times a per-split power of two rs (max rho * rs in
//    [0.5, 1)), then fp16;
//  - accumulation fp32; the power-of-two scales are undone exactly in fp32.
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f16x8_t as_f16x8(uint4 u) { return __builtin_bit_cast(f16x8_t, u); }
__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8_t, u); }

__device__ __forceinline__ uint32_t f16_bits(float f) {
    return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)f);  // round to nearest even
}
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) { return f16_bits(lo) | (f16_bits(hi) << 16); }
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return f32_to_bf16_rne(lo) | (f32_to_bf16_rne(hi) << 16);
}

// Power of two 2^k with max_abs * 2^k in [2^log2_target, 2^(log2_target+1)); 1 if max_abs == 0.
__device__ __forceinline__ float pow2_scale_for(float max_abs, int log2_target) {
    if (!(max_abs > 0.0f)) return 1.0f;
    int e = (int)((f2u(max_abs) >> 23) & 255u) - 127;  // floor(log2) for normal values
    if (e < -126) e = -126;
    int k = log2_target - e;
    if (k > 127) k = 127;
    if (k < -126) k = -126;
    return u2f((uint32_t)(k + 127) << 23);
}

// Two e4m3 codes (byte pair HI of w) -> two fp16, exact (hardware conversion, scale 1).
template <bool HI>
__device__ __forceinline__ uint32_t e4m3x2_to_f16x2(uint32_t w) {
    const f16x2_t h = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, HI);
    return __builtin_bit_cast(uint32_t, h);
}

__device__ __forceinline__ uint4 e4m3x8_to_f16x8(uint32_t w0, uint32_t w1) {
    return make_uint4(e4m3x2_to_f16x2<false>(w0), e4m3x2_to_f16x2<true>(w0), e4m3x2_to_f16x2<false>(w1),
                      e4m3x2_to_f16x2<true>(w1));
}

// Byte tables of the fp16 bits of the 8 positive codebook levels (index 8 + m).
struct Tq4Lut {
    uint32_t lo03, lo47, hi03, hi47;
};

__device__ __forceinline__ Tq4Lut make_tq4_lut() {
    Tq4Lut t{0, 0, 0, 0};
#pragma unroll
    for (int m = 0; m < 8; m++) {
        const uint32_t h = f16_bits(u2f(c_tq4_level[8 + m]));  // exact: 8 significant bits
        const uint32_t lo = h & 0xFF, hi = h >> 8;
        if (m < 4) { t.lo03 |= lo << (8 * m); t.hi03 |= hi << (8 * m); }
        else { t.lo47 |= lo << (8 * (m - 4)); t.hi47 |= hi << (8 * (m - 4)); }
    }
    return t;
}

// 8 nibble indices (element k = nibble k of x) -> 8 fp16 codebook levels.  The
// codebook is symmetric: index i >= 8 is +level[i], index i < 8 is
// -level[15 - i]; the magnitude comes from a byte table lookup (v_perm).
__device__ __forceinline__ uint4 tq4x8_to_f16x8(uint32_t x, const Tq4Lut& t) {
    const uint32_t neg = ((x >> 3) & 0x11111111u) ^ 0x11111111u;  // 1 where index < 8
    const uint32_t m = (x & 0x77777777u) ^ (neg * 7u);                // magnitude index
    const uint32_t me = m & 0x0F0F0F0Fu, mo = (m >> 4) & 0x0F0F0F0Fu;  // elements 0,2,4,6 / 1,3,5,7
    const uint32_t lo_e = __builtin_amdgcn_perm(t.lo47, t.lo03, me);
    const uint32_t lo_o = __builtin_amdgcn_perm(t.lo47, t.lo03, mo);
    const uint32_t hi_e = __builtin_amdgcn_perm(t.hi47, t.hi03, me) | ((neg & 0x01010101u) << 7);
    const uint32_t hi_o = __builtin_amdgcn_perm(t.hi47, t.hi03, mo) | (((neg >> 4) & 0x01010101u) << 7);
    const uint32_t ae = __builtin_amdgcn_perm(hi_e, lo_e, 0x05010400u);  // e0 | e2 << 16
    const uint32_t ao = __builtin_amdgcn_perm(hi_o, lo_o, 0x05010400u);  // o0 | o2 << 16
    const uint32_t be = __builtin_amdgcn_perm(hi_e, lo_e, 0x07030602u);  // e4 | e6 << 16
    const uint32_t bo = __builtin_amdgcn_perm(hi_o, lo_o, 0x07030602u);  // o4 | o6 << 16
    return make_uint4(__builtin_amdgcn_perm(ao, ae, 0x05040100u), __builtin_amdgcn_perm(ao, ae, 0x07060302u),
                      __builtin_amdgcn_perm(bo, be, 0x05040100u), __builtin_amdgcn_perm(bo, be, 0x07060302u));
}


// fp8 split kernel (raw-tile variant).  Same work items and wave split as
// k_attn_mfma, but every wave streams its rows' raw e4m3 codes into a
// double-buffered LDS tile with global_load_lds (no register staging, the next
// tile's load overlaps this tile's math).
//
// Tile layout, row-major with one 16-byte pad per row: chunk c (16 codes) of
// tile row r sits in 16-byte slot 33 sigma(r) + c, where
// sigma(r) = r ^ (bit3(r) << 2) ^ (bit4(r) << 3) is a bijection of 0..31.
// The DMA fills 64 consecutive slots per instruction (17 per tile, rows stay
// contiguous in global memory); each lane's source offset for instruction i
// is computed once per wave.  Every LDS read below is then a per-lane base
// plus a compile-time offset, and the 33-slot stride with sigma puts the rows
// one read serves on distinct bank groups:
//   score: lane (g, n) of row block rb reads tile row 8 (n / 4) + 4 rb + n % 4,
//          chunks 4 j + g (16 codes -> two fp16 k-steps) at
//          16 (33 sigma(row) + g) + 64 j; the accumulator row order then
//          matches the transposed read;
//   PV:    ds_read_b64_tr_b8: source lane (g, q) points at row 8 g + q / 2,
//          byte 8 (q % 2) of chunk mb; lane (g, p) receives the 8 codes of
//          rows 8 g .. 8 g + 7 in column 16 mb + p, converted to fp16 in
//          registers -- k-slots (g, j) = row 8 g + j, as the probabilities.
// The rope keys do not go through LDS: each lane loads its score rows' keys.
typedef int i32x2_t __attribute__((ext_vector_type(2)));
constexpr int RAW_ROW = DL;                   // bytes per raw fp8 code row
constexpr int RAW_SLOTS = 33;                 // 16-byte slots per padded tile row
constexpr int RAW_DMA = 17;                   // DMA instructions per code tile (1056 slots, 64 per instruction)
constexpr int RAW_TILE = RAW_DMA * 64 * 16;   // 17408 bytes

__device__ __forceinline__ void vm_wait_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }  // vmcnt(0)

// Workgroup barrier after this wave's LDS accesses have completed.  Unlike
// __syncthreads it does not wait for outstanding global loads (loads of later
// tiles stay in flight); the assembly is a compiler memory barrier as well.
__device__ __forceinline__ void wg_barrier_lds() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// LDS DMA (global_load_lds: each lane's bytes land at the wave-uniform LDS
// base in M0 + lane * size) issued from inline assembly.  The compiler does not
// see these LDS writes, so it adds no wait of its own before the LDS reads that
// follow -- with the builtin it waits for every outstanding DMA, the next
// tile's included, before the first read of the current tile.  The kernel
// waits explicitly (vmcnt) before it reads what a DMA wrote, and finishes its
// reads of a buffer (lgkmcnt) before a DMA refills it.
__device__ __forceinline__ uint32_t lds_offset(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}
// Scalar base + per-lane 32-bit offset form.  The global address is
// sbase + voff; the LDS address is M0 + 16 (or 4) * lane.  The compiler's
// hazard recognizer does not look inside the assembly, so each block starts
// with 5 wait states: a VALU write of an SGPR (v_readlane / v_readfirstlane,
// e.g. an SGPR reloaded from a spill lane) needs 5 before a VMEM instruction
// reads that SGPR as its base, and an SALU write of M0 needs 1 before LDS DMA.
// With fewer, the load can use a stale base register and fault.
__device__ __forceinline__ void dma_lds_b128(const void* sbase, uint32_t voff, uint32_t lds_base) {
    asm volatile("s_nop 4\n\tglobal_load_lds_dwordx4 %0, %1"
                 :
                 : "v"(voff), "s"(sbase), "{m0}"(lds_base)
                 : "memory");
}
__device__ __forceinline__ void dma_lds_b32(const void* sbase, uint32_t voff, uint32_t lds_base) {
    asm volatile("s_nop 4\n\tglobal_load_lds_dword %0, %1"
                 :
                 : "v"(voff), "s"(sbase), "{m0}"(lds_base)
                 : "memory");
}
// max over the four lanes n, n ^ 16, n ^ 32, n ^ 48 (gfx950 lane-swap
// instructions: each pairs a lane with the one 16 or 32 lanes away).
__device__ __forceinline__ float max_xor16_xor32(float v) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ int tile_sigma(int r) { return r ^ (((r >> 3) & 1) << 2) ^ (((r >> 4) & 1) << 3); }
__device__ __forceinline__ int tile_sigma_inv(int q) {
    return q ^ (((q >> 4) & 1) << 3) ^ ((((q >> 3) ^ (q >> 4)) & 1) << 2);
}

// The split plan, in-kernel (matrix-core paths), run by one wave: it scans
// max(1, ceil(T_s / split)) over the sequences, 64 at a time, and finds the
// one holding chunk c: plan_s = {first row, end row, sequence}, sequence -1
// if there is no such chunk.  The workgroup with blockIdx 0 also stores the
// prefix (chunk_prefix) for the merge.
__device__ __forceinline__ void plan_chunk(const kvq_attn_args& a, const Plan& p, int64_t c, int64_t* plan_s,
                                           int lane) {
    const bool writer = blockIdx.x == 0;
    const int64_t split = p.split_rows;
    int64_t run = 0;
    if (lane == 0) plan_s[2] = -1;
    for (int base = 0; base < a.n_seqs; base += 64) {
        const int sq = base + lane;
        int64_t cnt = 0, lo = 0, hi = 0;
        if (sq < a.n_seqs) {
            lo = max(a.seq_offsets[sq], (int64_t)0);
            hi = min(a.seq_offsets[sq + 1], a.total_rows);
            cnt = hi > lo ? (hi - lo + split - 1) / split : 1;
        }
        int64_t incl = cnt;  // inclusive scan over the wave
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int64_t v = __shfl_up(incl, o, 64);
            if (lane >= o) incl += v;
        }
        const int64_t excl = run + incl - cnt;
        const bool mine = sq < a.n_seqs && c >= excl && c < excl + cnt;  // one lane over all passes
        if (sq < a.n_seqs && writer) p.chunk_prefix[sq] = excl;
        if (mine) {
            const int64_t r0c = lo + (c - excl) * split;
            plan_s[0] = r0c;
            plan_s[1] = min(hi, r0c + split);
            plan_s[2] = sq;
        }
        run += __shfl(incl, 63, 64);
        if (!writer && __any(mine)) break;
    }
    if (writer && lane == 0) p.chunk_prefix[a.n_seqs] = run;
}

// This workgroup's chunk c: rows [r0, r1) of sequence sq; false if there is
// no such chunk (workgroup-uniform).  One sequence holds rows 0 .. total_rows - 1
// (seq_offsets[0] = 0 and seq_offsets[1] = total_rows by the interface), so its
// chunks need no loads and no barrier; otherwise wave 0 scans the offsets.
__device__ __forceinline__ bool locate_chunk(const kvq_attn_args& a, const Plan& p, int64_t c, int64_t* plan_s,
                                             int wave, int lane, int64_t& r0, int64_t& r1, int& sq) {
    if (a.n_seqs == 1) {
        const int64_t split = p.split_rows;
        const int64_t nch = max((int64_t)1, (a.total_rows + split - 1) / split);
        if (c >= nch) return false;
        r0 = c * split;
        r1 = min(a.total_rows, r0 + split);
        sq = 0;
        if (blockIdx.x == 0 && threadIdx.x == 0) {
            p.chunk_prefix[0] = 0;
            p.chunk_prefix[1] = nch;
        }
        return true;
    }
    if (wave == 0) plan_chunk(a, p, c, plan_s, lane);
    __syncthreads();  // plan_s
    if (plan_s[2] < 0) return false;
    r0 = plan_s[0];
    r1 = plan_s[1];
    sq = (int)plan_s[2];
    return true;
}

__global__ __launch_bounds__(MF_WAVES * 64) void k_attn_mfma_fp8(kvq_attn_args a, Plan p) {
    __shared__ __align__(16) uint8_t raw[MF_WAVES][2][RAW_TILE];     // codes, double-buffered
    __shared__ __align__(16) float rho_s[MF_WAVES][2][64];             // row scales
    __shared__ float ml_s[MF_WAVES][3][MF_HEADS];
    __shared__ int64_t plan_s[3];  // this chunk's first row, end row, sequence (-1: none)
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int g = lane >> 4, n = lane & 15;
    // workgroups are dealt round-robin to the XCDs: chunk c goes to XCD c % 8 and
    // its head groups are consecutive there, so they share that XCD's L2
    const int64_t local = blockIdx.x / N_XCD;
    const int64_t c = (int64_t)(blockIdx.x % N_XCD) + N_XCD * (local / p.n_groups);
    const int hg = (int)(local % p.n_groups);
    if (c >= p.max_chunks) return;
    const int head = hg * MF_HEADS + n;
    int64_t r0, r1;
    int sq;
    if (!locate_chunk(a, p, c, plan_s, wave, lane, r0, r1, sq)) return;  // workgroup-uniform
    const int64_t quarter = ((r1 - r0 + MF_WAVES - 1) / MF_WAVES + MF_TILE - 1) / MF_TILE * MF_TILE;
    const int64_t w0 = min(r1, r0 + wave * quarter), w1 = min(r1, w0 + quarter);

    // DMA loaders (global -> LDS, no registers).  Lane l of instruction i fills
    // slot 64 i + l: row sigma^-1(slot / 33), chunk slot % 33 (the pad slot and
    // the slots past the tile re-read chunk 0 of that row, or of row 0).  The
    // offsets are fixed per lane.  Rows past the wave's end are loaded too (and
    // masked later) while they lie inside the arrays; past the arrays' end a
    // lane loads their last 16 bytes instead.  Instruction k of a tile
    // (0..17: codes, scales) is issued on its own, so the issue can be spread
    // over the score steps.  The rope keys go straight to registers (load_rope).
    uint32_t voff_c[RAW_DMA];
#pragma unroll
    for (int i = 0; i < RAW_DMA; i++) {
        const int q = 64 * i + lane;
        const int k = q / RAW_SLOTS, ch = q % RAW_SLOTS;
        const int r = k < MF_TILE ? tile_sigma_inv(k) : 0;
        voff_c[i] = (uint32_t)(r * RAW_ROW + 16 * (ch < 32 && k < MF_TILE ? ch : 0));
    }
    const uint32_t lds_codes = lds_offset(&raw[wave][0][0]);
    const uint32_t lds_rho = lds_offset(&rho_s[wave][0][0]);
    constexpr int NDMA = RAW_DMA + 1;
    auto dma_one = [&](int k, int64_t t0, int buf, int lim) __attribute__((always_inline)) {
        // lim: rows of the tile inside the arrays (offsets are clamped to them)
        if (k < RAW_DMA) {
            dma_lds_b128(a.codes + t0 * RAW_ROW, min(voff_c[k], (uint32_t)lim * RAW_ROW - 16u),
                         __builtin_amdgcn_readfirstlane(lds_codes + (uint32_t)buf * RAW_TILE + 1024u * k));
        } else {
            const uint32_t voff_s = (uint32_t)((lane & 31) < lim ? (lane & 31) : 0) * 4u;
            dma_lds_b32(a.row_scale + t0, voff_s, __builtin_amdgcn_readfirstlane(lds_rho + 256u * buf));
        }
    };
    auto load_tile = [&](int64_t t0, int buf) __attribute__((always_inline)) {
        const int lim = (int)min((int64_t)MF_TILE, a.total_rows - t0);
#pragma unroll
        for (int k = 0; k < NDMA; k++) dma_one(k, t0, buf, lim);
    };
    // The rope keys of a tile, straight into registers one tile ahead: lane (g, n)
    // takes the score rows 8 (n / 4) + 4 rb + n % 4 (rb = 0, 1), dims 32 k + 8 g
    // .. + 7 (16-byte aligned), clamped to the arrays; unconditional loads.
    uint4 krn[2][2];
    auto load_rope = [&](int64_t t0) __attribute__((always_inline)) {
#pragma unroll
        for (int rb = 0; rb < 2; rb++) {
            const int64_t row = min(t0 + 8 * (n >> 2) + 4 * rb + (n & 3), a.total_rows - 1);
#pragma unroll
            for (int k = 0; k < 2; k++)
                krn[rb][k] = *reinterpret_cast<const uint4*>(a.k_rope + row * DR + 32 * k + 8 * g);
        }
    };

    // ---- query operands, in-kernel: lane (g, n) holds head n's latent dims
    // 64 j + 16 g + 8 hh + e as k-step 2 j + hh (e = 0..7), scaled by a power of
    // two qs (max |q| * qs in [256, 512)) and rounded to fp16; the rope dims
    // 32 ks' + 8 g + e, times sm_scale * log2(e), as a bf16 hi + lo pair.
    uint4 qh[16], rh[2], rl[2];
    float qinv;
    // the largest |row scale| of this wave's rows sets the probabilities' power-of-two
    // scale rsc (loads clamped to the wave's range, issued with the query's)
    float rsc;
    {
        // The group's 16 query heads are loaded once per workgroup: wave w brings
        // heads 4 w .. 4 w + 3 (fp32) and the first 256 of its rows' scales by DMA
        // into its second code buffer, which is free until the first tile's
        // next-tile DMA (after the barrier at the end of this block).  Head k's
        // latent row sits at QS_ROW * (k % 4) + 64 * (k / 4) of raw[k / 4][1] (the
        // 16-byte row pads and the 64-byte skew put the 16 heads one read serves on
        // distinct bank groups), its rope row at QS_ROPE + QS_RROW * (k % 4) +
        // 64 * (k / 4), the scales at QS_RS.  The first tile's DMA goes out right
        // after, and the wait below covers only the staging DMAs, so the three
        // latencies overlap.
        constexpr int QS_ROW = DL * 4 + 16, QS_ROPE = 8448, QS_RROW = DR * 4, QS_RS = 9728;
        static_assert(QS_ROPE >= 3 * QS_ROW + 192 + DL * 4 && QS_ROPE % 256 == 0 &&
                          QS_RS >= QS_ROPE + 192 + 4 * QS_RROW && QS_RS + 1024 <= RAW_TILE,
                      "query staging fits a code buffer");
        const bool hv = head < a.n_heads;
        uint8_t* const qst = &raw[wave][1][0];
        const uint32_t lqs = __builtin_amdgcn_readfirstlane(lds_offset(qst));
        {
            const int hq = hg * MF_HEADS + 4 * wave;  // first head of this wave's quarter (clamped below)
            const float* qb = a.q_lat + (int64_t)sq * a.n_heads * DL;
#pragma unroll
            for (int i = 0; i < 8; i++) {
                const int hi = min(hq + (i >> 1), a.n_heads - 1);
                dma_lds_b128(qb + (int64_t)hi * DL, 1024u * (i & 1) + 16u * lane,
                             lqs + QS_ROW * (i >> 1) + 64 * wave + 1024 * (i & 1));
            }
            const int hr = min(hq + (lane >> 4), a.n_heads - 1);
            dma_lds_b128(a.q_rope + (int64_t)sq * a.n_heads * DR, (uint32_t)hr * (DR * 4) + 16u * (lane & 15),
                         lqs + QS_ROPE + 64 * wave);
            // the row scales: clamped to the wave's rows; with no rows the loads read
            // the query instead (always present) and are discarded
            const float* rsp = a.total_rows > 0 ? a.row_scale : a.q_lat;
            const int64_t rb = w0 < w1 ? w0 : 0;
            const int rl = w0 < w1 ? (int)min((int64_t)255, w1 - 1 - w0) : 0;
#pragma unroll
            for (int u = 0; u < 4; u++)
                dma_lds_b32(rsp + rb, 4u * (uint32_t)min(64 * u + lane, rl), lqs + QS_RS + 256 * u);
        }
        if (w0 < w1) {  // wave-uniform
            load_tile(w0, 0);
            load_rope(w0);
            __builtin_amdgcn_s_waitcnt(0x0F70 | 6 | (16 << 10));  // vmcnt(22): the staging DMAs have landed
        } else {
            vm_wait_all();
        }
        static_assert(NDMA == 18, "the wait above counts the first tile's 18 DMAs and 4 rope loads");
        wg_barrier_lds();  // every quarter is in LDS (the first tile's DMA stays in flight)
        float rmw = 0.0f;
        if (w0 < w1) {  // wave-uniform
#pragma unroll
            for (int u = 0; u < 4; u++)
                rmw = fmaxf(rmw, fabsf(*reinterpret_cast<const float*>(qst + QS_RS + 256 * u + 4 * lane)));
            // the rest of a quarter longer than 256 rows
            for (int64_t t = w0 + 256 + lane; t < w1; t += 64) rmw = fmaxf(rmw, fabsf(a.row_scale[t]));
        }
        rsc = pow2_scale_for(wave_max(rmw), -1);  // rho * rsc < 1 for every row; 1 if all are 0
        // lane (g, n): head n's dims 64 j + 16 g + 8 hh + e and rope dims 32 k + 8 g + e
        const uint8_t* const hrow = &raw[n >> 2][1][0] + QS_ROW * (n & 3) + 64 * (n >> 2);
        const uint8_t* const rrow = &raw[n >> 2][1][0] + QS_ROPE + QS_RROW * (n & 3) + 64 * (n >> 2);
        float4 v[32], w[4];
#pragma unroll
        for (int ks = 0; ks < 16; ks++) {
            const uint8_t* src = hrow + 4 * (64 * (ks >> 1) + 16 * g + 8 * (ks & 1));
            v[2 * ks] = *reinterpret_cast<const float4*>(src);
            v[2 * ks + 1] = *reinterpret_cast<const float4*>(src + 16);
        }
#pragma unroll
        for (int k = 0; k < 2; k++) {
            const uint8_t* src = rrow + 4 * (32 * k + 8 * g);
            w[2 * k] = *reinterpret_cast<const float4*>(src);
            w[2 * k + 1] = *reinterpret_cast<const float4*>(src + 16);
        }
        float qmax = 0.0f;
#pragma unroll
        for (int k = 0; k < 32; k++)
            qmax = fmaxf(qmax, fmaxf(fmaxf(fabsf(v[k].x), fabsf(v[k].y)), fmaxf(fabsf(v[k].z), fabsf(v[k].w))));
        qmax = fmaxf(qmax, __shfl_xor(qmax, 16, 64));
        qmax = fmaxf(qmax, __shfl_xor(qmax, 32, 64));
        const float qs = hv ? pow2_scale_for(qmax, 8) : 0.0f;  // absent heads: a zero query
        qinv = hv ? 1.0f / qs : 0.0f;                           // exact
#pragma unroll
        for (int ks = 0; ks < 16; ks++) {
            const float4 x = v[2 * ks], y = v[2 * ks + 1];
            qh[ks] = make_uint4(pack_f16x2(x.x * qs, x.y * qs), pack_f16x2(x.z * qs, x.w * qs),
                                pack_f16x2(y.x * qs, y.y * qs), pack_f16x2(y.z * qs, y.w * qs));
        }
#pragma unroll
        for (int k = 0; k < 2; k++) {
            const float c2r = hv ? a.sm_scale * LOG2E : 0.0f;  // rope scores come out in log2 units
            const float f[8] = {w[2 * k].x * c2r, w[2 * k].y * c2r, w[2 * k].z * c2r, w[2 * k].w * c2r,
                                w[2 * k + 1].x * c2r, w[2 * k + 1].y * c2r, w[2 * k + 1].z * c2r,
                                w[2 * k + 1].w * c2r};
            float b[8];
#pragma unroll
            for (int e = 0; e < 8; e++) b[e] = u2f(f32_to_bf16_rne(f[e]) << 16);
            rh[k] = make_uint4(pack_bf16x2(b[0], b[1]), pack_bf16x2(b[2], b[3]), pack_bf16x2(b[4], b[5]),
                               pack_bf16x2(b[6], b[7]));
            rl[k] = make_uint4(pack_bf16x2(f[0] - b[0], f[1] - b[1]), pack_bf16x2(f[2] - b[2], f[3] - b[3]),
                               pack_bf16x2(f[4] - b[4], f[5] - b[5]), pack_bf16x2(f[6] - b[6], f[7] - b[7]));
        }
        wg_barrier_lds();  // every wave has read the staged query before the second buffers refill
    }
    auto tile_row = [](int rb, int nn) { return 8 * (nn >> 2) + 4 * rb + (nn & 3); };
    // per-lane LDS read offsets (bytes within a tile)
    const uint32_t rd_a = 16u * (RAW_SLOTS * tile_sigma(tile_row(0, n)) + g);   // score, row block 0
    const uint32_t rd_b = 16u * (RAW_SLOTS * tile_sigma(tile_row(1, n)) + g);   // score, row block 1
    const uint32_t rd_t = 16u * RAW_SLOTS * tile_sigma(8 * g + (n >> 1)) + 8u * (n & 1);  // PV transposed reads

    const float k1 = a.sm_scale * LOG2E * qinv;  // latent score scale (log2 units)

    // Softmax with a fixed reference per wave and head: p = 2^(s - m_run), with
    // m_run the first tile's maximum, and probabilities enter the matrix cores
    // as fp16 p * rho * rsc (rho * rsc < 1 for all of the wave's rows).  A later
    // tile may exceed the reference by 2^8, so p * rho * rsc <= 2^8.  A tile
    // beyond that raises the reference and the wave starts its rows again: the
    // accumulators are never rescaled inside the loop (they stay in the matrix
    // cores' registers), and for all but adversarial score sequences the first
    // pass is the only one.
    f32x4_t acc_o[32];
    float m_run = -INFINITY, l_part = 0.0f;
    bool restarted = false;
    for (;;) {
#pragma unroll
    for (int mb = 0; mb < 32; mb++) acc_o[mb] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    l_part = 0.0f;
    int buf = 0;
    bool again = false;
    if (restarted && w0 < w1) {
        load_tile(w0, 0);
        load_rope(w0);
    }
    restarted = true;
    for (int64_t t0 = w0; t0 < w1; t0 += MF_TILE) {
        const int nt = (int)min((int64_t)MF_TILE, w1 - t0);
        vm_wait_all();  // this tile's codes and scales are in LDS, its rope keys in registers
        const bool more = t0 + MF_TILE < w1;
        uint4 kr[2][2];
#pragma unroll
        for (int rb = 0; rb < 2; rb++)
#pragma unroll
            for (int k = 0; k < 2; k++) kr[rb][k] = krn[rb][k];
        const float4 rho0 = *reinterpret_cast<const float4*>(&rho_s[wave][buf][8 * g]);
        const float4 rho1 = *reinterpret_cast<const float4*>(&rho_s[wave][buf][8 * g + 4]);
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): those reads are done before the buffers refill
        // the next tile's DMA, three instructions per score step (after the last
        // tile: this tile again, into the free buffer)
        const int64_t tn = more ? t0 + MF_TILE : t0;
        // after the last tile the reload only has to be harmless: one row, from the cache
        const int limn = more ? (int)min((int64_t)MF_TILE, a.total_rows - tn) : 1;
        load_rope(tn);  // the next tile's rope keys (after the last tile: this tile's again)
        const uint8_t* tb = raw[wave][buf];
        // ---- scores: both row blocks together, the reads one k-chunk ahead
        const uint8_t* pa = tb + rd_a;
        const uint8_t* pbp = tb + rd_b;
        auto chunk = [&](const uint8_t* base, int j) { return *reinterpret_cast<const uint4*>(base + 64 * j); };
        f32x4_t sl[2], sr[2];
        sl[0] = sl[1] = sr[0] = sr[1] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
        // the reads run two k-chunks ahead and the conversions one, so a step's
        // matrix-core work and the next step's conversions are independent
        uint4 ca = chunk(pa, 0), cbv = chunk(pbp, 0);
        uint4 na = chunk(pa, 1), nb = chunk(pbp, 1);
        uint4 a0 = e4m3x8_to_f16x8(ca.x, ca.y), a1 = e4m3x8_to_f16x8(ca.z, ca.w);
        uint4 b0 = e4m3x8_to_f16x8(cbv.x, cbv.y), b1 = e4m3x8_to_f16x8(cbv.z, cbv.w);
#pragma unroll
        for (int j = 0; j < 8; j++) {
            const uint4 ua0 = a0, ua1 = a1, ub0 = b0, ub1 = b1;
            if (j < 7) {
                ca = na;
                cbv = nb;
                if (j < 6) {
                    na = chunk(pa, j + 2);
                    nb = chunk(pbp, j + 2);
                }
            }
#pragma unroll
            for (int k = 3 * j; k < 3 * j + 3; k++)
                if (k < NDMA) dma_one(k, tn, buf ^ 1, limn);
            __builtin_amdgcn_sched_barrier(0);  // the look-ahead reads issue before this chunk's math
            if (j < 7) {
                a0 = e4m3x8_to_f16x8(ca.x, ca.y);
                a1 = e4m3x8_to_f16x8(ca.z, ca.w);
                b0 = e4m3x8_to_f16x8(cbv.x, cbv.y);
                b1 = e4m3x8_to_f16x8(cbv.z, cbv.w);
            }
            sl[0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_f16x8(ua0), as_f16x8(qh[2 * j]), sl[0], 0, 0, 0);
            sl[1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_f16x8(ub0), as_f16x8(qh[2 * j]), sl[1], 0, 0, 0);
            sl[0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_f16x8(ua1), as_f16x8(qh[2 * j + 1]), sl[0], 0, 0, 0);
            sl[1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_f16x8(ub1), as_f16x8(qh[2 * j + 1]), sl[1], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int rb = 0; rb < 2; rb++)
#pragma unroll
            for (int k = 0; k < 2; k++) {
                sr[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kr[rb][k]), as_bf16x8(rh[k]), sr[rb], 0, 0, 0);
                sr[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kr[rb][k]), as_bf16x8(rl[k]), sr[rb], 0, 0, 0);
            }
        // the first PV operands are read now: their latency hides behind the softmax
        const uint8_t* trbase = tb + rd_t;
        auto trd = [&](int mb) __attribute__((always_inline)) {
            return __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) i32x2_t*)(trbase + 16 * mb));
        };
        i32x2_t nv[8];
#pragma unroll
        for (int i = 0; i < 8; i++) nv[i] = trd(i);
        // lane (g, n): accumulator register r of block rb = tile row 8 g + 4 rb + r
        const bool full = nt == MF_TILE;  // wave-uniform
        float sc[2][4], rr[2][4];
#pragma unroll
        for (int rb = 0; rb < 2; rb++) {
            const float4 rq = rb ? rho1 : rho0;
            const float rv[4] = {rq.x, rq.y, rq.z, rq.w};
#pragma unroll
            for (int r = 0; r < 4; r++) {
                const bool ok = full || 8 * g + 4 * rb + r < nt;
                rr[rb][r] = ok ? rv[r] : 0.0f;
                sc[rb][r] = ok ? fmaf(rv[r] * k1, sl[rb][r], sr[rb][r]) : -INFINITY;
            }
        }
        float tmax = fmaxf(fmaxf(fmaxf(sc[0][0], sc[0][1]), fmaxf(sc[0][2], sc[0][3])),
                           fmaxf(fmaxf(sc[1][0], sc[1][1]), fmaxf(sc[1][2], sc[1][3])));
        tmax = max_xor16_xor32(tmax);
        // the first column group's PV operands are converted now (independent of
        // the softmax, so they fill its latency), and the second group's reads issued
        uint4 pv0[8];
#pragma unroll
        for (int i = 0; i < 8; i++) pv0[i] = e4m3x8_to_f16x8((uint32_t)nv[i][0], (uint32_t)nv[i][1]);
#pragma unroll
        for (int i = 0; i < 8; i++) nv[i] = trd(8 + i);
        if (m_run == -INFINITY) m_run = tmax;  // first tile: every row valid
        const bool over = tmax > m_run + LAZY_LOG2;
        if (__any(over)) {
            // raise the reference past this tile and start the rows again
            m_run = fmaxf(m_run, tmax);
            again = true;
            __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): no LDS read pending when the buffers refill
            break;
        }
        float psum = 0.0f;
        uint32_t pb[4];
#pragma unroll
        for (int rb = 0; rb < 2; rb++) {
            float pw[4];
#pragma unroll
            for (int r = 0; r < 4; r++) {
                // v_exp_f32: masked rows (score -inf) give 0; m_run is finite after the first tile
                const float pv = __builtin_amdgcn_exp2f(sc[rb][r] - m_run);
                psum += pv;
                pw[r] = pv * (rr[rb][r] * rsc);
            }
            pb[2 * rb] = pack_f16x2(pw[0], pw[1]);
            pb[2 * rb + 1] = pack_f16x2(pw[2], pw[3]);
        }
        l_part += psum;
        const f16x8_t bop = as_f16x8(make_uint4(pb[0], pb[1], pb[2], pb[3]));
        // ---- PV: groups of 8 column blocks, the next group's reads in flight
#pragma unroll
        for (int i = 0; i < 8; i++)
            acc_o[i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_f16x8(pv0[i]), bop, acc_o[i], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int grp = 1; grp < 4; grp++) {
            i32x2_t cv[8];
#pragma unroll
            for (int i = 0; i < 8; i++) cv[i] = nv[i];
            if (grp < 3) {
#pragma unroll
                for (int i = 0; i < 8; i++) nv[i] = trd(8 * grp + 8 + i);
            }
            __builtin_amdgcn_sched_barrier(0);  // the next group's reads issue before this group's math
#pragma unroll
            for (int i = 0; i < 8; i++) {
                const uint4 aop = e4m3x8_to_f16x8((uint32_t)cv[i][0], (uint32_t)cv[i][1]);
                acc_o[8 * grp + i] =
                    __builtin_amdgcn_mfma_f32_16x16x32_f16(as_f16x8(aop), bop, acc_o[8 * grp + i], 0, 0, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        buf ^= 1;
    }
    vm_wait_all();  // the next tile's DMA may still be landing: drain it (restart or epilogue)
    if (!again) break;
    }
    // ---- merge the waves' states in LDS (each wave reuses its own raw buffers)
    l_part += __shfl_xor(l_part, 16, 64);
    l_part += __shfl_xor(l_part, 32, 64);
    float* st = reinterpret_cast<float*>(&raw[wave][0][0]);  // [16][512] O
    __syncthreads();  // every wave is done with its tiles
    // float4 slot f of head row hh is stored at slot f ^ hh (spreads the 16 rows over the banks)
#pragma unroll
    for (int mb = 0; mb < 32; mb++)
        *reinterpret_cast<float4*>(st + n * DL + 4 * ((4 * mb + g) ^ n)) =
            make_float4(acc_o[mb][0], acc_o[mb][1], acc_o[mb][2], acc_o[mb][3]);
    if (g == 0) {
        ml_s[wave][0][n] = m_run;
        ml_s[wave][1][n] = l_part;
        ml_s[wave][2][n] = rsc;
    }
    __syncthreads();
    {
        const int hh = tid >> 4;             // head within the group
        const int f0 = tid & 15;             // float4 columns f0 + 16 q: each store covers 256 contiguous bytes
        float mw[MF_WAVES], M = -INFINITY;
#pragma unroll
        for (int w = 0; w < MF_WAVES; w++) {
            mw[w] = ml_s[w][0][hh];
            M = fmaxf(M, mw[w]);
        }
        float sw[MF_WAVES], so[MF_WAVES], L = 0.0f;
#pragma unroll
        for (int w = 0; w < MF_WAVES; w++) {
            sw[w] = (mw[w] == -INFINITY) ? 0.0f : exp2f(mw[w] - M);
            L += sw[w] * ml_s[w][1][hh];
            const float rw = ml_s[w][2][hh];
            so[w] = rw > 0.0f ? sw[w] / rw : 0.0f;  // 1 / rsc is exact
        }
        const int h = hg * MF_HEADS + hh;
        if (h < a.n_heads) {
            float* dst = p.part_o + (c * a.n_heads + h) * DL;
#pragma unroll
            for (int q = 0; q < 8; q++) {
                const int f = f0 + 16 * q;
                float4 o = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
#pragma unroll
                for (int w = 0; w < MF_WAVES; w++) {
                    const float4 v = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(&raw[w][0][0]) +
                                                                      hh * DL + 4 * (f ^ hh));
                    o.x += so[w] * v.x; o.y += so[w] * v.y; o.z += so[w] * v.z; o.w += so[w] * v.w;
                }
                *reinterpret_cast<float4*>(dst + 4 * f) = o;
            }
            if ((tid & 15) == 0) {
                p.part_m[c * a.n_heads + h] = M;  // log2 units
                p.part_l[c * a.n_heads + h] = L;
            }
        }
    }
}

// TQ4 query preparation: q~ = H D q / sqrt(512) for every (sequence, head),
// scaled by a power of two qs (max |q~| * qs in [256, 512)) and rounded to
// fp16, in the split kernel's operand layout: uint4 16 g + ks holds dims
// 32 ks + 8 g .. + 7; the rope query (times sm_scale * log2(e)) as bf16 hi
// (uint4 QP_RH + 2 g + k) and lo (QP_RL + 2 g + k) terms of dims 32 k + 8 g ..
// + 7; 1 / qs in q_inv.  One wave per (sequence, head); lane l rotates dims
// 8 l .. 8 l + 7 (three butterfly stages in registers, six across lanes).
__global__ __launch_bounds__(256) void k_qprep_tq4(kvq_attn_args a, Plan p) {
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);  // = s * heads_padded + h
    if (row >= (int64_t)a.n_seqs * p.heads_padded) return;
    const int s = (int)(row / p.heads_padded), h = (int)(row % p.heads_padded);
    const bool valid = h < a.n_heads;
    // unconditional loads (a clamped head; a guarded load would wait for every load in flight)
    const float* src = a.q_lat + ((int64_t)s * a.n_heads + min(h, a.n_heads - 1)) * DL + 8 * lane;
    const float4 x0 = *reinterpret_cast<const float4*>(src), x1 = *reinterpret_cast<const float4*>(src + 4);
    const float* r = a.q_rope + ((int64_t)s * a.n_heads + min(h, a.n_heads - 1)) * DR + 8 * (lane & 7);
    const float4 y0 = *reinterpret_cast<const float4*>(r), y1 = *reinterpret_cast<const float4*>(r + 4);
    float v[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
    for (int i = 0; i < 8; i++) v[i] = valid ? v[i] : 0.0f;
    const uint32_t sm = a.sign_mask[lane];
#pragma unroll
    for (int i = 0; i < 8; i++)
        if ((sm >> i) & 1u) v[i] = -v[i];
#pragma unroll
    for (int hh = 1; hh < 8; hh <<= 1)
#pragma unroll
        for (int i = 0; i < 8; i++)
            if (!(i & hh)) {
                const float x = v[i], y = v[i + hh];
                v[i] = x + y;
                v[i + hh] = x - y;
            }
    // across lanes: DPP and lane-swap butterflies
#pragma unroll
    for (int i = 0; i < 8; i++) {
        float x = v[i];
        x = fwht_xlane_c<1>(x, lane);
        x = fwht_xlane_c<2>(x, lane);
        x = fwht_xlane_c<4>(x, lane);
        x = fwht_xlane_c<8>(x, lane);
        x = fwht_xlane_c<16>(x, lane);
        v[i] = fwht_xlane_c<32>(x, lane);
    }
    float qmax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; i++) {
        v[i] *= INV_SQRT_DL;
        qmax = fmaxf(qmax, fabsf(v[i]));
    }
    qmax = wave_max(qmax);
    const float qs = pow2_scale_for(qmax, 8);
    uint4* dst = p.q_pack + row * QPACK_U4;
    dst[16 * (lane & 3) + (lane >> 2)] = make_uint4(pack_f16x2(v[0] * qs, v[1] * qs), pack_f16x2(v[2] * qs, v[3] * qs),
                                                    pack_f16x2(v[4] * qs, v[5] * qs), pack_f16x2(v[6] * qs, v[7] * qs));
    if (lane < 8) {  // rope dims 8 lane .. + 7: k-step lane / 4, lane group lane % 4
        const float c2r = valid ? a.sm_scale * LOG2E : 0.0f;
        const float rv[8] = {y0.x, y0.y, y0.z, y0.w, y1.x, y1.y, y1.z, y1.w};
        uint32_t rh[4], rl[4];
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const float f0 = rv[2 * i] * c2r, f1 = rv[2 * i + 1] * c2r;
            const float b0 = u2f(f32_to_bf16_rne(f0) << 16), b1 = u2f(f32_to_bf16_rne(f1) << 16);
            rh[i] = pack_bf16x2(b0, b1);
            rl[i] = pack_bf16x2(f0 - b0, f1 - b1);
        }
        dst[QP_RH + 2 * (lane & 3) + (lane >> 2)] = make_uint4(rh[0], rh[1], rh[2], rh[3]);
        dst[QP_RL + 2 * (lane & 3) + (lane >> 2)] = make_uint4(rl[0], rl[1], rl[2], rl[3]);
    }
    if (lane == 0) p.q_inv[row] = 1.0f / qs;  // exact
}

// TQ4 split kernel.  Work item = (T-chunk, group of 64 heads); the items are
// dealt to XCDs in contiguous runs so the head groups of a chunk share one
// L2.  All 4 waves of a workgroup step through the chunk's tiles (32 rows)
// together, wave w for heads 16 w .. 16 w + 15: the nibble codes of a tile
// are decoded once per workgroup -- each wave decodes 8 rows into a shared,
// double-buffered fp16 LDS tile (rope keys and row scales next to it) -- and
// every wave then reads the whole tile:
//   score:  S^T (16 rows x 16 heads) += X(rows, k) q~^T, X from the tile
//           (lane (g, n): row 16 rb + n, dims 32 ks + 8 g .. + 7);
//   PV:     O^T (16 dims x 16 heads) += X^T P'^T, X^T via ds_read_b64_tr_b16
//           (lane (g, p) gets rows 4 g .. 4 g + 3 and 16 + 4 g .. + 3 of column
//           p, the k order the score accumulators hold P in).
// One barrier per tile.  While a wave multiplies tile t it decodes tile t + 1
// (its codes were loaded one tile earlier).  Softmax: fixed per-wave
// reference (first tile's max) and probabilities times rho * rs with rs from
// the chunk's largest radius; a tile more than 2^8 above the reference raises
// it, and the workgroup (which shares the tiles) starts its rows again.  One
// partial per (chunk, head), written by the wave that owns the head.
constexpr int XT = DL + 8;                // halfwords per fp16 tile row (rows 4 banks apart)
constexpr int KT = DR + 8;                // halfwords per rope tile row
__global__ __launch_bounds__(MF_WAVES * 64) void k_attn_mfma_tq4(kvq_attn_args a, Plan p) {
    __shared__ __align__(16) uint16_t xt[2][MF_TILE][XT];  // decoded latent rows, fp16
    __shared__ __align__(16) uint16_t kt[2][MF_TILE][KT];  // rope keys, bf16
    __shared__ __align__(16) float rho_s[2][MF_TILE];      // radius / sqrt(512)
    __shared__ float red_s[MF_WAVES];
    __shared__ int flag_s[2][MF_WAVES];
    __shared__ int64_t plan_s[3];
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int g = lane >> 4, n = lane & 15;
    const int64_t local = blockIdx.x / N_XCD;
    const int64_t c = (int64_t)(blockIdx.x % N_XCD) + N_XCD * (local / p.n_groups);
    const int hg = (int)(local % p.n_groups);
    if (c >= p.max_chunks) return;
    const int head = hg * TQ4_HEADS + MF_HEADS * wave + n;  // may exceed n_heads (its query is zero)
    constexpr int CB = DL / 2;                                 // code bytes per row
    int64_t r0, r1;
    int sq;
    if (!locate_chunk(a, p, c, plan_s, wave, lane, r0, r1, sq)) return;  // workgroup-uniform
    const int ntiles = (int)((r1 - r0 + MF_TILE - 1) / MF_TILE);

    // decode share of this wave: tile row 8 wave + lane / 8, code bytes
    // 32 (lane % 8) .. + 31 (dims 64 (lane % 8) .. + 63), rope bytes 16 (lane % 8)
    const int drow = 8 * wave + (lane >> 3), dq = lane & 7;
    uint4 ca[2], cr;  // codes and rope of the tile to decode next
    float cs;         // its row radius (scaled by 1 / sqrt(512) when it is stored)
    auto load_share = [&](int t) __attribute__((always_inline)) {
        const int64_t t0 = r0 + (int64_t)MF_TILE * t;
        const int64_t row = t0 + min(drow, (int)(r1 - t0) - 1);  // rows past the chunk re-read its last row
        const uint8_t* cp = a.codes + row * CB + 32 * dq;
        ca[0] = *reinterpret_cast<const uint4*>(cp);
        ca[1] = *reinterpret_cast<const uint4*>(cp + 16);
        cr = *reinterpret_cast<const uint4*>(a.k_rope + row * DR + 8 * dq);
        cs = a.row_scale[row];
    };
    const Tq4Lut lut = make_tq4_lut();
    auto decode_share = [&](int buf) __attribute__((always_inline)) {
        const uint32_t w[8] = {ca[0].x, ca[0].y, ca[0].z, ca[0].w, ca[1].x, ca[1].y, ca[1].z, ca[1].w};
#pragma unroll
        for (int i = 0; i < 8; i++)
            *reinterpret_cast<uint4*>(&xt[buf][drow][64 * dq + 8 * i]) = tq4x8_to_f16x8(w[i], lut);
        *reinterpret_cast<uint4*>(&kt[buf][drow][8 * dq]) = cr;
        rho_s[buf][drow] = cs * INV_SQRT_DL;  // the 8 lanes of a row store the same value
    };
    // ---- query operands (prepared once per sequence and head), loaded first: the
    // row-scale loop below waits for its loads, and with them for these
    const uint4* qp = p.q_pack + ((int64_t)sq * p.heads_padded + head) * QPACK_U4;
    uint4 qh[16], rh[2], rl[2];
#pragma unroll
    for (int k = 0; k < 16; k++) qh[k] = qp[16 * g + k];
#pragma unroll
    for (int k = 0; k < 2; k++) {
        rh[k] = qp[QP_RH + 2 * g + k];
        rl[k] = qp[QP_RL + 2 * g + k];
    }
    const float k1 = a.sm_scale * LOG2E * p.q_inv[(int64_t)sq * p.heads_padded + head];

    if (ntiles > 0) load_share(0);

    // ---- the chunk's largest row scale (four loads in flight per thread)
    float rmax = 0.0f;
    for (int64_t t = r0 + tid; t < r1; t += 4 * MF_WAVES * 64) {
        float x[4];
#pragma unroll
        for (int u = 0; u < 4; u++) x[u] = a.row_scale[min(t + u * MF_WAVES * 64, r1 - 1)];
#pragma unroll
        for (int u = 0; u < 4; u++) rmax = fmaxf(rmax, fabsf(x[u]));
    }
    rmax = wave_max(rmax);
    if (lane == 0) red_s[wave] = rmax;
    __syncthreads();
    rmax = fmaxf(fmaxf(red_s[0], red_s[1]), fmaxf(red_s[2], red_s[3]));
    const float rs = pow2_scale_for(rmax * INV_SQRT_DL, -1);  // max rho * rs in [0.5, 1)

    // per-lane LDS addresses: score row 16 rb + n, dims 8 g + 32 ks; PV source
    // lane (g, n) at row 4 g + n / 4, column 4 (n % 4) (+ 16 mb, + 16 rows)
    const int trow = 4 * g + (n >> 2), tcol = 4 * (n & 3);
    f32x4_t acc_o[32];
    float m_run = -INFINITY, l_part = 0.0f;
    bool over = false;
    // one vote + barrier per tile: every wave reports whether its last tile was
    // out of range (any such vote restarts the workgroup); the barrier also
    // publishes the tile decoded since the last one
    auto vote = [&](int t) __attribute__((always_inline)) {
        flag_s[t & 1][wave] = over ? 1 : 0;  // every lane stores the same value
        wg_barrier_lds();
        const int4 f = *reinterpret_cast<const int4*>(&flag_s[t & 1][0]);
        return (f.x | f.y | f.z | f.w) != 0;  // workgroup-uniform
    };
    for (;;) {
#pragma unroll
    for (int mb = 0; mb < 32; mb++) acc_o[mb] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    l_part = 0.0f;
    if (ntiles > 0) {
        decode_share(0);  // its codes were loaded above (or at the restart)
        load_share(min(1, ntiles - 1));
    }
    bool again = vote(0);
    if (!again && ntiles > 0) {
    int t = 0;
    do {
        const int buf = t & 1;
        const int nt = (int)min((int64_t)MF_TILE, r1 - (r0 + (int64_t)MF_TILE * t));
        // ---- scores S^T (two row blocks) from the tile: four independent
        // accumulator chains (row block x even / odd k-step), reads one step ahead
        f32x4_t sl[2], sr[2], sx[2];
        sl[0] = sl[1] = sr[0] = sr[1] = sx[0] = sx[1] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
        {
            const uint16_t* xa = &xt[buf][n][8 * g];
            const uint16_t* xb = &xt[buf][16 + n][8 * g];
            f16x8_t na = *reinterpret_cast<const f16x8_t*>(xa), nb = *reinterpret_cast<const f16x8_t*>(xb);
#pragma unroll
            for (int ks = 0; ks < 16; ks++) {
                const f16x8_t ca2 = na, cb2 = nb;
                if (ks < 15) {
                    na = *reinterpret_cast<const f16x8_t*>(xa + 32 * (ks + 1));
                    nb = *reinterpret_cast<const f16x8_t*>(xb + 32 * (ks + 1));
                }
                f32x4_t& s0 = (ks & 1) ? sx[0] : sl[0];
                f32x4_t& s1 = (ks & 1) ? sx[1] : sl[1];
                s0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(ca2, as_f16x8(qh[ks]), s0, 0, 0, 0);
                s1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(cb2, as_f16x8(qh[ks]), s1, 0, 0, 0);
            }
#pragma unroll
            for (int rb = 0; rb < 2; rb++) {
                const uint16_t* kr = &kt[buf][16 * rb + n][8 * g];
#pragma unroll
                for (int k = 0; k < 2; k++) {
                    const bf16x8_t kv = *reinterpret_cast<const bf16x8_t*>(kr + 32 * k);
                    sr[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kv, as_bf16x8(rh[k]), sr[rb], 0, 0, 0);
                    sr[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kv, as_bf16x8(rl[k]), sr[rb], 0, 0, 0);
                }
                sl[rb] += sx[rb];
            }
        }
        // ---- softmax: lane (g, n) holds rows 16 rb + 4 g + r of head n (no branches)
        float sc[2][4], rr[2][4];
        float tmax = -INFINITY;
#pragma unroll
        for (int rb = 0; rb < 2; rb++) {
            const float4 rq = *reinterpret_cast<const float4*>(&rho_s[buf][16 * rb + 4 * g]);
            const float rv[4] = {rq.x, rq.y, rq.z, rq.w};
#pragma unroll
            for (int r = 0; r < 4; r++) {
                const bool ok = 16 * rb + 4 * g + r < nt;
                rr[rb][r] = ok ? rv[r] : 0.0f;
                sc[rb][r] = ok ? fmaf(rv[r] * k1, sl[rb][r], sr[rb][r]) : -INFINITY;
                tmax = fmaxf(tmax, sc[rb][r]);
            }
        }
        tmax = max_xor16_xor32(tmax);
        m_run = m_run == -INFINITY ? tmax : m_run;  // first tile: row 0 is valid
        // a tile more than 2^8 above the reference raises it; the workgroup
        // restarts at the next vote
        const bool ov = __any(tmax > m_run + LAZY_LOG2);
        m_run = ov ? fmaxf(m_run, tmax) : m_run;
        over = over || ov;
        float psum = 0.0f;
        uint32_t pb[4];
#pragma unroll
        for (int rb = 0; rb < 2; rb++) {
            float pw[4];
#pragma unroll
            for (int r = 0; r < 4; r++) {
                const float pv = __builtin_amdgcn_exp2f(sc[rb][r] - m_run);  // masked rows: 0
                psum += pv;
                pw[r] = pv * (rr[rb][r] * rs);
            }
            pb[2 * rb] = pack_f16x2(pw[0], pw[1]);
            pb[2 * rb + 1] = pack_f16x2(pw[2], pw[3]);
        }
        l_part += psum;
        const f16x8_t bop = as_f16x8(make_uint4(pb[0], pb[1], pb[2], pb[3]));
        // ---- the next tile's share (after the last tile: the last one again,
        // into the free buffer), then the loads of the one after
        decode_share(buf ^ 1);
        load_share(min(t + 2, ntiles - 1));
        // ---- PV from the tile, the transposed reads four column blocks ahead
        auto pv_read = [&](int mb) __attribute__((always_inline)) {
            const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) s16x4_t*)&xt[buf][trow][16 * mb + tcol]);
            const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) s16x4_t*)&xt[buf][16 + trow][16 * mb + tcol]);
            const uint2 lo2 = __builtin_bit_cast(uint2, lo), hi2 = __builtin_bit_cast(uint2, hi);
            return as_f16x8(make_uint4(lo2.x, lo2.y, hi2.x, hi2.y));
        };
        f16x8_t pvq[4];
#pragma unroll
        for (int i = 0; i < 4; i++) pvq[i] = pv_read(i);
#pragma unroll
        for (int mb = 0; mb < 32; mb++) {
            const f16x8_t aop = pvq[mb & 3];
            if (mb + 4 < 32) pvq[mb & 3] = pv_read(mb + 4);
            acc_o[mb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(aop, bop, acc_o[mb], 0, 0, 0);
        }
        t++;
        again = vote(t);
    } while (!again && t < ntiles);
    }
    if (!again) break;
    over = false;
    if (ntiles > 0) load_share(0);
    }
    // ---- the partials of this wave's heads, staged in LDS (the tiles are free
    // after the last vote) half a row at a time and stored as whole rows
    l_part += __shfl_xor(l_part, 16, 64);
    l_part += __shfl_xor(l_part, 32, 64);
    if (g == 0 && head < a.n_heads) {
        p.part_m[c * a.n_heads + head] = m_run;  // log2 units
        p.part_l[c * a.n_heads + head] = l_part;
    }
    constexpr int SR = DL / 2 + 4;  // floats per staged half row
    static_assert(sizeof(xt) >= MF_WAVES * MF_HEADS * SR * sizeof(float), "staging fits in the tiles");
    float* stg = reinterpret_cast<float*>(&xt[0][0][0]) + wave * (MF_HEADS * SR);
    const float so = 1.0f / rs;  // exact (a power of two)
#pragma unroll
    for (int hf = 0; hf < 2; hf++) {
#pragma unroll
        for (int mb = 0; mb < 16; mb++) {
            const f32x4_t v = acc_o[16 * hf + mb];
            *reinterpret_cast<float4*>(stg + n * SR + 16 * mb + 4 * g) = make_float4(v[0] * so, v[1] * so, v[2] * so, v[3] * so);
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
        for (int k = 0; k < MF_HEADS; k++) {
            const int h = hg * TQ4_HEADS + MF_HEADS * wave + k;
            if (h < a.n_heads)
                *reinterpret_cast<float4*>(p.part_o + (c * a.n_heads + h) * DL + DL / 2 * hf + 4 * lane) =
                    *reinterpret_cast<const float4*>(stg + k * SR + 4 * lane);
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
}

// ---- 3. merge --------------------------------------------------------------------------------
// NDH workgroups per (sequence, head), each over DL / NDH output dims (TQ4: the
// whole row, which the un-rotation needs).  A thread owns one float4 column and
// every NGRP-th split; it merges its splits online (running max, rescaled sums),
// then the NGRP groups are combined through LDS.
template <bool TQ4, bool LOG2, int NT>
__global__ __launch_bounds__(NT) void k_merge(kvq_attn_args a, Plan p) {
    constexpr int NDH = TQ4 ? 1 : 2;
    constexpr int DW = DL / NDH;       // dims per workgroup
    constexpr int COLS = DW / 4;       // float4 columns
    constexpr int NGRP = NT / COLS;    // split groups
    constexpr int U = 8;               // splits in flight per thread
    __shared__ __align__(16) float4 o_s[NGRP][COLS];
    __shared__ float m_s[NGRP], l_s[NGRP];
    __shared__ __align__(16) float vec[DL];
    const int tid = threadIdx.x;
    const int64_t item = blockIdx.x / NDH;
    const int part = (int)(blockIdx.x % NDH);
    const int s = (int)(item / a.n_heads), h = (int)(item % a.n_heads);
    const int64_t c0 = min(p.chunk_prefix[s], p.max_chunks), c1 = min(p.chunk_prefix[s + 1], p.max_chunks);
    const int col = tid % COLS, grp = tid / COLS;
    auto ex = [](float x) { return LOG2 ? exp2f(x) : expf(x); };
    float m = -INFINITY, l = 0.0f;
    float4 o = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    // batches of U splits: all loads first (no branch between them), then the
    // online update with selects
    for (int64_t cb = c0 + grp; cb < c1; cb += U * NGRP) {
        float mc[U], lc[U];
        float4 v[U];
#pragma unroll
        for (int u = 0; u < U; u++) {
            const int64_t c = cb + u * NGRP;
            const int64_t ch = (c < c1 ? c : cb) * a.n_heads + h;
            mc[u] = p.part_m[ch];
            lc[u] = p.part_l[ch];
            v[u] = *reinterpret_cast<const float4*>(p.part_o + ch * DL + part * DW + 4 * col);
            if (c >= c1) mc[u] = -INFINITY;
        }
#pragma unroll
        for (int u = 0; u < U; u++) {
            const float mn = fmaxf(m, mc[u]);
            const float sc = m == -INFINITY ? 0.0f : ex(m - mn);
            const float w = mc[u] == -INFINITY ? 0.0f : ex(mc[u] - mn);
            o.x = o.x * sc + w * v[u].x;
            o.y = o.y * sc + w * v[u].y;
            o.z = o.z * sc + w * v[u].z;
            o.w = o.w * sc + w * v[u].w;
            l = l * sc + w * lc[u];
            m = mn;
        }
    }
    o_s[grp][col] = o;
    if (col == 0) {
        m_s[grp] = m;
        l_s[grp] = l;
    }
    __syncthreads();
    float M = -INFINITY;
#pragma unroll
    for (int k = 0; k < NGRP; k++) M = fmaxf(M, m_s[k]);
    float L = 0.0f;
    float wg[NGRP];
#pragma unroll
    for (int k = 0; k < NGRP; k++) {
        wg[k] = m_s[k] == -INFINITY ? 0.0f : ex(m_s[k] - M);
        L += wg[k] * l_s[k];
    }
    const float inv = L > 0.0f ? 1.0f / L : 0.0f;
    if (grp == 0) {
        float4 r = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
#pragma unroll
        for (int k = 0; k < NGRP; k++) {
            const float4 u = o_s[k][col];
            r.x += wg[k] * u.x; r.y += wg[k] * u.y; r.z += wg[k] * u.z; r.w += wg[k] * u.w;
        }
        r = make_float4(r.x * inv, r.y * inv, r.z * inv, r.w * inv);
        if (TQ4) *reinterpret_cast<float4*>(&vec[4 * col]) = r;
        else *reinterpret_cast<float4*>(a.out + item * DL + part * DW + 4 * col) = r;
    }
    if (TQ4) {
        __syncthreads();
        if (tid < 64) {  // o = D H o~ / sqrt(512), 8 consecutive per lane
            const int lane = tid;
            float v[8];
#pragma unroll
            for (int i = 0; i < 8; i++) v[i] = vec[8 * lane + i];
#pragma unroll
            for (int hh = 1; hh < 8; hh <<= 1)
#pragma unroll
                for (int i = 0; i < 8; i++)
                    if (!(i & hh)) {
                        const float x = v[i], y = v[i + hh];
                        v[i] = x + y;
                        v[i + hh] = x - y;
                    }
#pragma unroll
            for (int mm = 1; mm < 64; mm <<= 1)
#pragma unroll
                for (int i = 0; i < 8; i++) v[i] = fwht_xlane(v[i], lane, mm);
            const uint32_t sm = a.sign_mask[lane];
#pragma unroll
            for (int i = 0; i < 8; i++) {
                v[i] *= INV_SQRT_DL;
                if ((sm >> i) & 1u) v[i] = -v[i];
            }
            float4* dst = reinterpret_cast<float4*>(a.out + item * DL + 8 * lane);
            dst[0] = make_float4(v[0], v[1], v[2], v[3]);
            dst[1] = make_float4(v[4], v[5], v[6], v[7]);
        }
    }
    if (a.lse && part == 0 && tid == 0) {
        float v;
        if (!(L > 0.0f)) v = -INFINITY;
        else v = LOG2 ? (M + log2f(L)) * LN2 : M + logf(L);
        a.lse[item] = v;
    }
}

}  // namespace

int64_t attn_workspace_bytes(const kvq_attn_args& a) { return plan_bytes(a); }

hipError_t launch_decode_attn_stage(const kvq_attn_args& a, int stage, void* ws, hipStream_t st) {
    Plan p = make_plan(a, ws, nullptr);
    const bool f32 = a.precision == KVQ_PREC_FP32;
    const bool tq4 = a.qmode == KVQ_QMODE_TQ4;
    switch (stage) {
        case KVQ_STAGE_PREP:
            // the matrix-core split kernels plan their chunk themselves; the fp8 one
            // also prepares its query, TQ4 rotates it here once per head
            if (!f32) {
                if (tq4) {
                    const int64_t rows = (int64_t)a.n_seqs * p.heads_padded;
                    hipLaunchKernelGGL(k_qprep_tq4, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, st, a, p);
                }
                break;
            }
            hipLaunchKernelGGL(k_plan, dim3(1), dim3(256), 0, st, a.seq_offsets, a.n_seqs, p.split_rows, a.total_rows,
                               p.chunk_prefix);
            if (tq4) {
                const int64_t rows = (int64_t)a.n_seqs * a.n_heads;
                hipLaunchKernelGGL(k_qrot, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, st, a.q_lat, a.sign_mask,
                                   rows, p.q_rot);
            }
            break;
        case KVQ_STAGE_SPLITS:
            if (f32) {
                const dim3 grid((unsigned)p.max_chunks, (unsigned)p.n_groups);
                const float* qsrc = tq4 ? p.q_rot : a.q_lat;
                if (tq4) hipLaunchKernelGGL(k_attn_f32<KVQ_QMODE_TQ4>, grid, dim3(256), 0, st, a, p, qsrc);
                else hipLaunchKernelGGL(k_attn_f32<KVQ_QMODE_FP8>, grid, dim3(256), 0, st, a, p, qsrc);
            } else {
                const dim3 grid((unsigned)(p.chunks_per_xcd * N_XCD * p.n_groups));
                if (tq4) hipLaunchKernelGGL(k_attn_mfma_tq4, grid, dim3(MF_WAVES * 64), 0, st, a, p);
                else hipLaunchKernelGGL(k_attn_mfma_fp8, grid, dim3(MF_WAVES * 64), 0, st, a, p);
            }
            break;
        default: {
            const int64_t items = (int64_t)a.n_seqs * a.n_heads;
            // more split groups per workgroup when there are many splits per sequence,
            // a single one (one thread per float4 column) when there are few
            const bool wide = p.max_chunks >= 16 * (int64_t)a.n_seqs;
            const bool narrow = p.max_chunks <= 4 * (int64_t)a.n_seqs;
            if (tq4) {
                if (!f32 && wide) hipLaunchKernelGGL((k_merge<true, true, 1024>), dim3((unsigned)items), dim3(1024), 0, st, a, p);
                else if (!f32 && narrow) hipLaunchKernelGGL((k_merge<true, true, 128>), dim3((unsigned)items), dim3(128), 0, st, a, p);
                else if (!f32) hipLaunchKernelGGL((k_merge<true, true, 256>), dim3((unsigned)items), dim3(256), 0, st, a, p);
                else hipLaunchKernelGGL((k_merge<true, false, 256>), dim3((unsigned)items), dim3(256), 0, st, a, p);
            } else {
                if (!f32 && wide) hipLaunchKernelGGL((k_merge<false, true, 512>), dim3((unsigned)(2 * items)), dim3(512), 0, st, a, p);
                else if (!f32 && narrow) hipLaunchKernelGGL((k_merge<false, true, 64>), dim3((unsigned)(2 * items)), dim3(64), 0, st, a, p);
                else if (!f32) hipLaunchKernelGGL((k_merge<false, true, 256>), dim3((unsigned)(2 * items)), dim3(256), 0, st, a, p);
                else hipLaunchKernelGGL((k_merge<false, false, 256>), dim3((unsigned)(2 * items)), dim3(256), 0, st, a, p);
            }
            break;
        }
    }
    return hipGetLastError();
}

hipError_t launch_decode_attn(const kvq_attn_args& a, void* ws, int64_t ws_bytes, hipStream_t st) {
    (void)ws_bytes;
    for (int stage = KVQ_STAGE_PREP; stage <= KVQ_STAGE_MERGE; stage++) {
        const hipError_t e = launch_decode_attn_stage(a, stage, ws, st);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace kvq
