/*
 * kvq.h -- C ABI of libkvq.so: quantized KV-cache rows and decode attention
 * over them, native on AMD MI355X (gfx950).
 *
 * Conventions (all entry points):
 *  - Buffer pointers are DEVICE pointers unless the comment says "host".
 *    Every buffer is owned by the caller; the library keeps no reference to it
 *    after the call returns and allocates no device memory.
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *    Calls only enqueue work on it and return; no call synchronizes.
 *  - Arguments are validated before anything is enqueued: a call that returns
 *    an error has launched nothing.  There is no fallback to another precision
 *    or to the CPU.
 *  - Alignment (KVQ_ERR_INVALID_ARG otherwise): fp32 row inputs (x, k_src,
 *    v_src), code arrays read by the attention, pools, rope keys, outputs of
 *    the gather and of the attention: 16 bytes; fp8 codes written by the
 *    encoder: 8 bytes; codes written by the rotated-codec encoders: 4 bytes;
 *    every other buffer: the natural
 *    alignment of its element type.
 *  - NaN and Inf in floating-point inputs are outside the contract.
 *  - Calls are thread-safe; the library holds only immutable state.
 *
 * Sources cited below, by page title and section:
 *  [KV8]  colibri PR #399 "KV cache quantization: fp8 (KV8) + 4-bit TurboQuant
 *         (KV_TQ) on CPU, CUDA, and Metal".
 *  [Q4]   Strata PR #2533 "metal: q4_0 KV cache on the Mac engine".
 */
#ifndef KVQ_H
#define KVQ_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KVQ_ABI_VERSION 1

/* ---- status codes ------------------------------------------------------- */
#define KVQ_OK 0
#define KVQ_ERR_INVALID_ARG 1 /* null pointer, negative count, misalignment, bad shape    */
#define KVQ_ERR_UNSUPPORTED 2 /* valid but not provided: non-power-of-two TQ4 width, ...  */
#define KVQ_ERR_WORKSPACE 3   /* workspace smaller than kvq_decode_attn_workspace_bytes() */
#define KVQ_ERR_LAUNCH 4      /* the HIP runtime reported an error at launch             */
#define KVQ_ERR_TOO_LARGE 5   /* needs more than KVQ_NOALLOC_SCRATCH_BYTES of workspace   */

/* ---- modes ---------------------------------------------------------------- */
#define KVQ_QMODE_FP8 1      /* e4m3 codes [rows][dim] + fp32 scale per row           */
#define KVQ_QMODE_TQ4 2      /* 4-bit codebook indices [rows][dim/2] + fp32 radius    */
#define KVQ_QMODE_TQ3 3      /* 3-bit indices [rows][3*dim/8] + fp32 radius           */
#define KVQ_QMODE_TQ6 4      /* 6-bit indices [rows][6*dim/8] + fp32 radius           */
/* KVQ_PREC_MFMA: 16-bit matrix-core contractions with fp32 accumulation,
 * softmax and per-row scales.  [KV8]'s matrix-core wording names bf16
 * operands; it is read as "16-bit operands, fp32 accumulation", and the
 * latent codes and query are fp16 (exact for every e4m3 code and codebook
 * level, 3 more mantissa bits than bf16 for the query and probabilities, the
 * range handled by power-of-two scaling), the rope term bf16 (k_rope is
 * stored bf16) with a two-term bf16 query.  Hence the name: not _BF16. */
#define KVQ_PREC_MFMA 0
#define KVQ_PREC_FP32 1      /* fp32 vector arithmetic throughout (check path)        */
#define KVQ_Q4_NO_ROTATE 1u  /* append: rows are already in the rotated domain        */

/* ABI version of the loaded library (KVQ_ABI_VERSION at build time). */
int kvq_abi_version(void);

/* Static text for a status code; never NULL. */
const char* kvq_status_string(int status);

/* Bytes per stored row: KVQ_QMODE_FP8 -> dim + 4 (codes + scale),
 * KVQ_QMODE_TQ4 -> dim/2 + 4 (nibbles + radius), KVQ_QMODE_TQ3 -> 3*dim/8 + 4,
 * KVQ_QMODE_TQ6 -> 6*dim/8 + 4.  Returns -1 for an unknown mode or a dim the
 * encoders refuse.  Host only. */
int64_t kvq_row_bytes(int qmode, int dim);

/* The 4-bit codec's codebook ([KV8] "Why rotated-int4 for the 4-bit tier":
 * a fixed 16-level Lloyd-Max quantizer for N(0,1)).  levels: host float[16],
 * ascending, each a bfloat16 value; thresholds: host float[15], the exact
 * midpoints of neighbouring levels.  Either may be NULL.  Host only. */
int kvq_tq4_codebook(float* levels, float* thresholds);

/* The codebook of the rotated codec's b-bit tier, b = 3, 4 or 6 ([KV8]: the
 * 4-bit tier above; the 6-bit tier of the teacher-forcing table, TQ6; the
 * 3-bit tier of the .coli_kv reply, "codec 1, 3-bit"): the 2^b-level Lloyd-Max
 * quantizer for N(0,1), levels rounded to bfloat16, thresholds their exact
 * midpoints.  levels: host float[2^b]; thresholds: host float[2^b - 1]; either
 * may be NULL.  KVQ_ERR_UNSUPPORTED for another b.  Host only. */
int kvq_tq_codebook(int bits, float* levels, float* thresholds);

/* ---- a1: fp8 e4m3 per-row encoder ([KV8] Summary, commit 1) -------------
 * For each row r of x (fp32 [n_rows][dim], row-major):
 *   amax = max_i |x_i|,  scales[r] = fl32(amax / 448),
 *   codes[r][i] = e4m3(fl32(x_i / scales[r])), round to nearest even on the
 *   OCP e4m3 grid, |value| saturated to 448; the NaN code is never written.
 *   An all-zero row gets scales[r] = 0 and all codes 0x00.
 * Decode: x_hat = e4m3_value(code) * scale.
 * codes: u8 [n_rows][dim]; scales: fp32 [n_rows].
 * dim: a multiple of 8, 8 <= dim <= 2048.  n_rows == 0 is a no-op. */
int kvq_encode_fp8(const float* x, int64_t n_rows, int dim, uint8_t* codes, float* scales,
                   void* stream);

/* ---- a2: TQ4 row encoder ([KV8] Why rotated-int4; refusal of
 * non-power-of-two widths in the 85852e2 rebase note) ----------------------
 * For each row x (fp32 [n_rows][dim]):
 *   z_i = -x_i if bit i of sign_mask is set (bit i = byte i/8, bit i%8), else x_i;
 *   w = FWHT(z), unnormalized, stages h = 1, 2, 4, ... with (a, b) -> (a+b, a-b);
 *   radii[r] = sqrt(sum_i x_i^2), the sum a pairwise tree over i (fp32);
 *   idx_i = #{k : w_i > fl32(t_k * radii[r])}, t_k the codebook thresholds;
 *   codes[r][j] = idx_{2j} | idx_{2j+1} << 4.
 * Decode: y_i = level[idx_i] * r / sqrt(dim); x_hat = D H y / sqrt(dim).
 * sign_mask: u8 [dim/8]; codes: u8 [n_rows][dim/2]; radii: fp32 [n_rows].
 * dim: a power of two, 8 <= dim <= 512 (KVQ_ERR_UNSUPPORTED otherwise). */
int kvq_encode_tq4(const float* x, int64_t n_rows, int dim, const uint8_t* sign_mask,
                   uint8_t* codes, float* radii, void* stream);

/* The same codec at b = 3, 4 or 6 bits (TQ3, TQ4, TQ6; codebook:
 * kvq_tq_codebook(b)).  Identical steps with 2^b - 1 thresholds; the indices
 * of a row form a little-endian bit stream, index i in bits b*i .. b*i + b - 1
 * (least significant first; bit j of the stream is bit j % 8 of byte j / 8),
 * so codes is u8 [n_rows][dim*b/8] (b = 4: the nibble layout above; b = 4
 * gives exactly kvq_encode_tq4's output).  dim: a power of two, 8 <= dim <=
 * 512.  KVQ_ERR_UNSUPPORTED for another b or dim. */
int kvq_encode_tq(int bits, const float* x, int64_t n_rows, int dim, const uint8_t* sign_mask,
                  uint8_t* codes, float* radii, void* stream);

/* ---- a9/a10: q4_0 paged tier ([Q4]) ---------------------------------------
 * Pools: u8 [n_cells][n_kv_heads][144]; each 144-byte head-row is 8 blocks of
 * 18 bytes: binary16 scale d (little-endian) then 16 nibble bytes,
 * byte 2+j = q_j | q_{j+16} << 4.  Position p of sequence s lives in cell
 * block_table[s][p / page_size] * page_size + p % page_size. */
typedef struct kvq_q4_cache {
    uint8_t* k_pool;            /* device, [n_cells][n_kv_heads][144]            */
    uint8_t* v_pool;            /* device, [n_cells][n_kv_heads][144]            */
    const int32_t* block_table; /* device, [n_seqs][max_pages] physical page ids */
    int64_t n_cells;            /* cells in each pool (a multiple of page_size)  */
    int32_t max_pages;          /* columns of block_table                        */
    int32_t page_size;          /* cells per page, >= 1                          */
    int32_t n_kv_heads;         /* >= 1                                          */
    int32_t head_dim;           /* must be 256                                   */
} kvq_q4_cache;

/* Append new K and V rows ([Q4] first commit: kv_append_q4 single-step and
 * batch paths).  For sequence s the new rows are src_off[s] .. src_off[s+1]-1
 * of k_src/v_src (fp32 [total_new][n_kv_heads][256]); row i of s goes to
 * position pos0[s] + i.  Each head-row is rotated by FWHT-256 x 1/16 (skipped
 * with KVQ_Q4_NO_ROTATE) and quantized in blocks of 32:
 *   mval = element of largest |x| (a tie goes to the larger signed value,
 *          +0 over -0);  d = mval / -8;  id = d != 0 ? 1/d : 0;
 *   q_j  = min(15, max(0, trunc(fma(x_j, id, 8.5))))  (NaN -> 0);
 *   the scale is stored as binary16(d), round to nearest even.
 * pos0: device int32 [n_seqs]; src_off: device int64 [n_seqs+1], ascending,
 * src_off[0] = 0, src_off[n_seqs] = total_new (host).  Rows whose page is
 * outside block_table's columns, whose table entry is negative, or whose cell
 * is outside the pool are not written (never an out-of-bounds store).
 * Appends of the same cell in one call race; callers do not do that. */
int kvq_append_q4_0(const kvq_q4_cache* cache, int n_seqs, const int32_t* pos0,
                    const int64_t* src_off, int64_t total_new, const float* k_src,
                    const float* v_src, uint32_t flags, void* stream);

/* Gather positions 0 .. len_s-1 of every sequence (len_s = dst_off[s+1] -
 * dst_off[s]) to binary16 rows in the rotated domain ([Q4] kv_gather_q4 and
 * the QSA_KV_Q4 commit: dequant (nibble - 8) * f32(d)):
 *   out_j = binary16_rne((q_j - 8) * f32(d)).
 * dst_off: device int64 [n_seqs+1] (dst_off[n_seqs] = total_rows, host);
 * k_dst/v_dst: binary16 bits [total_rows][n_kv_heads][256].  Rows whose cell is
 * invalid (as for append) are left untouched. */
int kvq_gather_q4_0(const kvq_q4_cache* cache, int n_seqs, const int64_t* dst_off,
                    int64_t total_rows, uint16_t* k_dst, uint16_t* v_dst, void* stream);

/* ---- a3..a8: absorbed-MLA decode attention over quantized rows ------------
 * ([KV8] commit 6: fused decode with a 3-way qmode, score a_score8 and context
 * a_clat8 over fp8 rows; commit 2: split-T kernels; "Ready for review": the
 * native 4-bit consumer rotates q once per head, dots the codes through the
 * codebook and un-rotates the weighted sum; the 3- and 6-bit tiers of the
 * same codec are consumed the same way.)
 * For sequence s (rows seq_offsets[s] .. seq_offsets[s+1]-1) and head h:
 *   x_hat_t = the decoded latent row (fp8: e4m3(code)*scale; TQ3/4/6: the
 *             decode of kvq_encode_tq);
 *   s_t = sm_scale * (q_lat[s,h] . x_hat_t + q_rope[s,h] . k_rope_t);
 *   out[s,h] = sum_t softmax(s)_t x_hat_t;  lse[s,h] = log sum_t exp(s_t).
 * The latent rows are not reconstructed: fp8 codes (and codebook levels)
 * are converted exactly to fp16 matrix-core operands (KVQ_PREC_MFMA) or to
 * fp32 (KVQ_PREC_FP32), and the per-row scale is applied in fp32; the rotated
 * codec (TQ3/4/6) uses the rotated query R q and un-rotates the merged output
 * (R = H D / sqrt(dim)).
 * A sequence with no rows gets out = 0 and lse = -Inf.
 * Tolerance against an fp64 evaluation on the same codes:
 *   max|err| / max|ref| <= 2e-3 (KVQ_PREC_MFMA), <= 1e-5 (KVQ_PREC_FP32).
 * KVQ_PREC_MFMA operands: latent codes in fp16 (exact for every e4m3 value and
 * codebook level); the latent query scaled per head by a power of two and
 * rounded to fp16 (TQ3/4/6: R q, as two fp16 terms, the rounding and its
 * remainder); the rope query split into two bf16 terms (k_rope is
 * bf16); the probabilities p * rho_t scaled by a power of two per work item
 * and rounded to fp16; fp32 accumulation, softmax and per-row scales. */
typedef struct kvq_attn_args {
    int32_t qmode;              /* KVQ_QMODE_FP8, _TQ4, _TQ3 or _TQ6              */
    int32_t precision;          /* KVQ_PREC_MFMA or KVQ_PREC_FP32                 */
    int32_t n_seqs;             /* >= 1                                           */
    int32_t n_heads;            /* 1 .. 256                                       */
    int32_t dim_lat;            /* must be 512                                    */
    int32_t dim_rope;           /* must be 64                                     */
    int32_t split_rows;         /* rows per work item, a multiple of 32; 0 =
                                   automatic.  fp8 matrix-core path: rounded up to
                                   whole 128-row tiles, dealt over the sequences in
                                   order (a work item may span several) */
    int32_t reserved0;          /* must be 0                                      */
    int64_t total_rows;         /* host copy of seq_offsets[n_seqs]               */
    const int64_t* seq_offsets; /* device int64 [n_seqs+1], ascending, [0] = 0    */
    const uint8_t* codes;       /* device, fp8 [rows][512], TQ4 [rows][256],
                                   TQ3 [rows][192] or TQ6 [rows][384]             */
    const float* row_scale;     /* device fp32 [rows]: fp8 scale or the radius    */
    const uint16_t* k_rope;     /* device bf16 bits [rows][64]                    */
    const uint8_t* sign_mask;   /* device u8 [64] (TQ3/4/6; ignored for fp8)      */
    const float* q_lat;         /* device fp32 [n_seqs][n_heads][512]             */
    const float* q_rope;        /* device fp32 [n_seqs][n_heads][64]              */
    float* out;                 /* device fp32 [n_seqs][n_heads][512]             */
    float* lse;                 /* device fp32 [n_seqs][n_heads], or NULL         */
    float sm_scale;             /* softmax scale, finite                          */
    int32_t reserved1;          /* must be 0                                      */
} kvq_attn_args;

/* Device workspace bytes kvq_decode_attn needs for these arguments (partial
 * softmax states of the T-splits and the split plan); depends on qmode,
 * precision, n_seqs, n_heads, total_rows and split_rows only.  Host only;
 * returns -1 for arguments kvq_decode_attn would refuse. */
int64_t kvq_decode_attn_workspace_bytes(const kvq_attn_args* a);

/* Runs decode attention.  workspace: device, >= the queried size, 256-byte
 * aligned, contents need not be initialised; the call overwrites it.  Two
 * calls that share a workspace must be ordered (same stream). */
int kvq_decode_attn(const kvq_attn_args* a, void* workspace, int64_t ws_bytes, void* stream);

/* Appends n_new rows and runs decode attention, in one call: the same as the
 * row encoder of a->qmode (kvq_encode_fp8, or kvq_encode_tq with a->sign_mask)
 * on x_new (fp32 [n_new][512]) into codes_new (u8 [n_new][code bytes]) and
 * scale_new (fp32 [n_new]), followed by kvq_decode_attn(a, ...) -- a decode
 * step's append of the new token's latent row and its attention over the
 * cache ([KV8] commit 6, the fused layer decode).  codes_new and scale_new
 * normally point at the rows the new tokens take in the cache that a->codes and
 * a->row_scale describe; the attention reads them after the encode.  On the
 * fp8 matrix-core path the encode runs inside the attention's query-preparation
 * launch (one launch fewer); other modes launch the encoder first.  Results are
 * bit-identical to the two calls.  n_new = 0 is kvq_decode_attn.  Alignment:
 * x_new 16 bytes, codes_new 8 (fp8) or 4 bytes, scale_new 4. */
int kvq_decode_attn_append(const kvq_attn_args* a, const float* x_new, int64_t n_new, uint8_t* codes_new,
                           float* scale_new, void* workspace, int64_t ws_bytes, void* stream);

/* ---- decode attention without allocation ----------------------------------
 * For callers that cannot allocate device memory or pass a workspace: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation.  Same arguments, kernels, results and errors as kvq_decode_attn,
 * but the workspace is a static array inside the library, one per GPU, of
 * KVQ_NOALLOC_SCRATCH_BYTES bytes, held until the process ends (each GPU the
 * library runs on gets its own copy at its own address, looked up on the first
 * call on that device).  The call allocates nothing.
 *  - KVQ_ERR_TOO_LARGE when kvq_decode_attn_workspace_bytes(a) exceeds the
 *    scratch (32 MiB covers, e.g., one 32768-row sequence or 400k rows over 33
 *    sequences with 128 heads; the T-split partial states dominate).
 *  - `stream` must belong to the current device.
 *  - Every call on one GPU shares that GPU's scratch and leaves it holding the
 *    last call's contents (nothing in it must start at zero).  Calls that may
 *    overlap on one GPU (different streams, or threads without ordering) race
 *    and give wrong results: order them on one stream. */
#define KVQ_NOALLOC_SCRATCH_BYTES (32u << 20)
int kvq_decode_attn_noalloc(const kvq_attn_args* a, void* stream);

/* One stage of kvq_decode_attn; running stages 0..2 in order on one stream is
 * exactly kvq_decode_attn.  Running a stage gives profilers and timers one
 * stage per call:
 *   KVQ_STAGE_PREP   KVQ_PREC_FP32: the per-sequence T-split prefix and, TQ3/4/6,
 *                    R q in the workspace; KVQ_PREC_MFMA: the fp16 query
 *                    operands of every (sequence, head) with their per-head
 *                    power-of-two scales (TQ3/4/6: of R q) and the rope query
 *                    terms, and for fp8 with several sequences the split
 *                    kernel's tile plan (tiles per sequence, their prefix and
 *                    the tiles per work item);
 *   KVQ_STAGE_SPLITS the attention over every T-split (partial softmax states);
 *   KVQ_STAGE_MERGE  merge of the splits (+ un-rotation for TQ3/4/6) into out / lse. */
#define KVQ_STAGE_PREP 0
#define KVQ_STAGE_SPLITS 1
#define KVQ_STAGE_MERGE 2
int kvq_decode_attn_stage(const kvq_attn_args* a, int stage, void* workspace, int64_t ws_bytes,
                          void* stream);

/* ---- sparse (DSA-style) decode ----------------------------------------------
 * [KV8] commit list, item 2 ("split-T kernels, DSA-aware gather"), and the
 * rebase note on the DSA gather: a top-k selection picks the cache rows a
 * query attends to.  The selected rows are gathered by absolute row index into
 * a compact buffer, and the dense decode kernels consume that buffer.
 *
 * kvq_gather_rows copies rows row_index[0 .. n_index) of a quantized cache
 * (codes, row_scale, k_rope: cache_rows rows; code bytes per row: 512 for
 * KVQ_QMODE_FP8, 256 for KVQ_QMODE_TQ4, 192 for KVQ_QMODE_TQ3, 384 for
 * KVQ_QMODE_TQ6) unchanged to row i of codes_out,
 * scale_out and rope_out.
 *  - row_index: device int64.  An index outside [0, cache_rows) is clamped
 *    to the nearest valid row (0 or cache_rows - 1), so the call never reads
 *    outside the cache.
 *  - All buffers are device memory.  codes, k_rope, codes_out and rope_out
 *    must be 16-byte aligned.
 *  - n_index = 0 launches nothing. */
int kvq_gather_rows(int qmode, const uint8_t* codes, const float* row_scale, const uint16_t* k_rope,
                    int64_t cache_rows, const int64_t* row_index, int64_t n_index, uint8_t* codes_out,
                    float* scale_out, uint16_t* rope_out, void* stream);

/* kvq_decode_attn_sparse: decode attention of sequence s over the cache rows
 * row_index[seq_offsets[s] .. seq_offsets[s+1]).
 *  - a->seq_offsets partitions the index list, and a->total_rows = n_index is
 *    its host copy of seq_offsets[n_seqs].
 *  - a->codes, a->row_scale and a->k_rope describe the whole cache of
 *    cache_rows rows, 1 <= cache_rows < 2^32 (KVQ_ERR_INVALID_ARG otherwise;
 *    0 is accepted when the index list is empty).  Indices are clamped as in
 *    kvq_gather_rows.
 *  - The result equals kvq_decode_attn over the gathered rows, bit for bit.
 *    On the fp8 matrix-core path (KVQ_QMODE_FP8, KVQ_PREC_MFMA) the split
 *    kernel reads the selected rows in place through the index list; the
 *    other paths gather them into the workspace (kvq_gather_rows) and run the
 *    dense kernels over the copy.
 *  - A repeated index counts once per occurrence.
 *  - The workspace is device memory, 256-byte aligned, of at least
 *    kvq_decode_attn_sparse_workspace_bytes(a) bytes.  That function returns
 *    -1 for arguments the call would refuse. */
int64_t kvq_decode_attn_sparse_workspace_bytes(const kvq_attn_args* a);
int kvq_decode_attn_sparse(const kvq_attn_args* a, const int64_t* row_index, int64_t cache_rows, void* workspace,
                           int64_t ws_bytes, void* stream);

/* ---- fused decode attention over the q4_0 pools ([Q4], QSA_KV_Q4 commit) ---
 * The decode attention of the paged q4_0 tier, read straight from the pools:
 * for sequence s and query head h (KV head g = h / G, G = n_q_heads /
 * n_kv_heads, so query heads g*G .. g*G+G-1 share KV head g):
 *   q~      = FWHT256(q[s,h]) / 16 (the append's rotation; orthonormal);
 *   x_t     = (nibble - 8) * f32(d) for every block of the K and V head-rows
 *             of position t (fp32, exact: no rounding to binary16);
 *   s_t     = sm_scale * (q~ . k_t);  p = softmax(s) over the positions;
 *   out     = FWHT256(sum_t p_t v_t) / 16 (rotated back), lse = log sum exp s_t.
 * Sequence s attends positions 0 .. n_s - 1, n_s = min(len_off[s+1], total_rows)
 * - max(len_off[s], 0) (the device offsets are clamped to the host total, so
 * a stale device copy never makes the call read past its workspace), through
 * cache.block_table (cell = table[s][pos / page_size] * page_size + pos %
 * page_size); positions whose page column is past max_pages, whose table entry
 * is negative or whose cell is past n_cells take no part.  A sequence with no
 * position gets out = 0 and lse = -Inf.  The sigmoid gate that follows in the
 * pages' model is the caller's.
 * Arithmetic: fp32 accuracy on the matrix cores -- exact fp16 products of the
 * codes minus 8 with three fp16 terms of q~ (times a power of two) summed in
 * fp32 and multiplied by d in fp32; the value sum from (nibble - 8) * d as two
 * exact fp16 terms times p as two fp16 terms; sm_scale * log2(e) folded into
 * q~, exp2.  Tolerance against an fp64 evaluation on the same pool bytes:
 * max|err| / max|ref| <= 1e-5. */
typedef struct kvq_q4_attn_args {
    int32_t n_seqs;             /* >= 1                                              */
    int32_t n_q_heads;          /* n_kv_heads * G with G in {1, 2, 4, 8, 16}          */
    int32_t split_rows;         /* positions per work item: 0 = automatic, else a
                                   multiple of 256 up to 2^24                         */
    int32_t reserved0;          /* must be 0                                         */
    int64_t total_rows;         /* host copy of len_off[n_seqs]                      */
    const int64_t* len_off;     /* device int64 [n_seqs+1], non-decreasing, [0] = 0  */
    const float* q;             /* device fp32 [n_seqs][n_q_heads][256], unrotated   */
    float* out;                 /* device fp32 [n_seqs][n_q_heads][256]              */
    float* lse;                 /* device fp32 [n_seqs][n_q_heads], or NULL          */
    float sm_scale;             /* softmax scale, finite                             */
    int32_t reserved1;          /* must be 0                                         */
} kvq_q4_attn_args;

/* Device workspace bytes for kvq_decode_attn_q4_0 (rotated queries, the T-split
 * prefix and the partial softmax states); depends on n_kv_heads, n_seqs,
 * n_q_heads, total_rows and split_rows only.  Host only; -1 for arguments the
 * call would refuse. */
int64_t kvq_decode_attn_q4_0_workspace_bytes(const kvq_q4_cache* cache, const kvq_q4_attn_args* a);

/* Runs the fused decode attention on `stream` (three launches: query rotation
 * and split plan, split kernel, merge and rotation back).  workspace: device,
 * 256-byte aligned, >= the queried size (KVQ_ERR_WORKSPACE otherwise); two
 * calls sharing it must be ordered.  q and out 16-byte aligned, len_off 8-byte
 * aligned; pools as for kvq_append_q4_0.  KVQ_ERR_UNSUPPORTED for a head ratio
 * other than 1, 2, 4, 8 or 16 or head_dim != 256. */
int kvq_decode_attn_q4_0(const kvq_q4_cache* cache, const kvq_q4_attn_args* a, void* workspace,
                         int64_t ws_bytes, void* stream);

/* ---- conformance probe -------------------------------------------------------
 * Element-wise conversions exactly as the kernels perform them, so a caller
 * can check them against the format definitions (for instance over every
 * fp32 bit pattern):
 *   KVQ_CVT_F32_TO_E4M3   fp32 -> e4m3 byte, round to nearest even, |v| saturated
 *                         to 448 (the fp8 encoder's step after the division:
 *                         v_med3_f32, then v_cvt_scalef32_pk_fp8_f32, scale 1);
 *   KVQ_CVT_E4M3_TO_BF16  e4m3 byte -> bf16 bits, exact (the attention's dequant;
 *                         S.1111.111 reads as +0, [KV8] HIP portability note);
 *   KVQ_CVT_F32_TO_F16    fp32 -> binary16 bits, round to nearest even (the q4_0
 *                         scale and gather outputs: v_cvt_f16_f32);
 *   KVQ_CVT_F32_TO_BF16   fp32 -> bf16 bits, round to nearest even (the rope
 *                         query terms of the matrix-core path);
 *   KVQ_CVT_E4M3_TO_F16   e4m3 byte -> binary16 bits with the instruction the
 *                         matrix-core path uses (v_cvt_scalef32_pk_f16_fp8, scale
 *                         1): exact for the 254 finite codes; the two NaN codes,
 *                         which kvq_encode_fp8 never writes, are outside the
 *                         attention's contract.
 * in/out: device arrays of n elements of the source/destination type. */
#define KVQ_CVT_F32_TO_E4M3 1
#define KVQ_CVT_E4M3_TO_BF16 2
#define KVQ_CVT_F32_TO_F16 3
#define KVQ_CVT_F32_TO_BF16 4
#define KVQ_CVT_E4M3_TO_F16 5
int kvq_convert(int kind, const void* in, int64_t n, void* out, void* stream);

/* ---- binding support ------------------------------------------------------
 * Layout of the argument structs, so a foreign-language binding can check its
 * mirror: which = 0 -> kvq_attn_args, 1 -> kvq_q4_cache, 2 -> kvq_q4_attn_args;
 * out[0] = sizeof, then
 * the offsetof of every field in declaration order.  Returns the number of
 * values written (at most n), or -1 for an unknown struct.  Host only. */
int kvq_struct_layout(int which, int64_t* out, int n);

#ifdef __cplusplus
}
#endif

#endif /* KVQ_H */
