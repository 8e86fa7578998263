/*
 * sage_attn.h -- C ABI of the MI355X (gfx950) SageAttention2 quantized attention forward.
 *
 * Pages cited:
 *   [SA2]   "SageAttention2: Efficient Attention with Thorough Outlier Smoothing and
 *           Per-thread INT4 Quantization" (mlsanity.com page for arXiv 2411.10958),
 *           section "Abstract (arXiv)".
 *   [SA2c]  zhaifeiyue.github.io commentary on arXiv 2411.10958: the paragraphs on the
 *           paper's Sec. 3.4 (two-level accumulation), on per-thread quantization and on
 *           smoothing K.
 *   [SA2pp] pith.science verdict on arXiv 2505.21136 (SageAttention2++), JSON keys
 *           "key_machinery" and "supporting_citations".
 *   [BLOG]  "SageAttention：大模型量化注意力加速实践指南" (blog.gitcode.com), sections on the
 *           core API call and precision control: the method is a drop-in for PyTorch's
 *           scaled_dot_product_attention selected by a head_dim / is_causal / quant mode;
 *           the quant modes "qk_int8_pv_fp8" (fast) and "qk_int8_pv_fp16" (high fidelity:
 *           V kept in fp16) select the P~V precision.  Its feature section on adapting
 *           generation models names automatic tensor-layout conversion for the models'
 *           attention interfaces, and its precision-control section a causal variable-length
 *           (varlen) kernel for batches whose sequence lengths differ.
 *
 * What the library computes: O = softmax(Q K^T / sqrt(d)) V, approximated as in [SA2]:
 * K is smoothed by its per-channel mean over tokens, Q by its per-block mean with the
 * mean(Q) . gamma(K)^T term added back in fp32; smoothed Q and K are quantized to INT8
 * (qk_bits = 8, codes in [-127, 127]) or to INT4-range values (qk_bits = 4, codes in
 * [-7, 7] carried in int8 lanes) with one scale per MFMA lane group; QK^T runs on the
 * integer MFMA with exact int32 accumulation; an online softmax produces P~, which is
 * quantized to FP8 E4M3 with the static range P_r = 448; V is quantized per channel to
 * FP8 E4M3 with V_r = 448 [SA2pp key_machinery]; P~V runs on the FP8 MFMA with two-level
 * accumulation [SA2], [SA2c]: each instruction sums its 64 products in the matrix unit (the
 * narrow, block-local level) and adds them to the fp32 output accumulator it takes as its C
 * operand (the global level).  With pv_bits = 16 (the [BLOG] high-fidelity mode) V is not
 * quantized: P and V enter the fp16 MFMA (fp32 accumulation) and only QK^T is quantized.
 *
 * Tensors (all device pointers, caller-owned, never freed or retained by the library):
 *   q, o : fp16, contiguous [B, H, N, d]           (o is overwritten)
 *   k, v : fp16, contiguous [B, Hkv, N, d]; query head h reads kv head h / (H / Hkv)
 *   causal: 0 or 1; 1 masks key j > query i (top-left aligned, N_q == N_k)
 *   d    : 64 or 128; softmax scale 1/sqrt(d)
 *   qk_bits: 8 (INT8 codes) or 4 (INT4-range codes)
 *   pv_bits: 8 (FP8 P~ and V, two-level accumulation) or 16 (fp16 P and V)
 *   workspace: device memory of at least sage_attn_workspace_bytes(...) bytes, 256-byte
 *          aligned; its contents on entry are ignored.
 *   stream: a hipStream_t (NULL = the legacy default stream).  Every call is stream
 *          ordered and returns after enqueueing; the library makes no device
 *          synchronisation, allocates no memory and keeps no state between calls, so
 *          concurrent calls with distinct workspaces are safe.
 *
 * Errors: every argument check happens before anything is enqueued; on error nothing is
 * enqueued and a negative status is returned.  SAGE_ERR_HIP reports a failed HIP call or
 * launch; sage_last_error() then holds the HIP message for the calling thread.
 */
#ifndef SAGE_ATTN_H
#define SAGE_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SAGE_OK 0
#define SAGE_ERR_INVALID_ARG (-1) /* null pointer, size < 1, H % Hkv != 0, size overflow,
                                     bad layout/dtype code, cu_seqlens not from 0 upwards  */
#define SAGE_ERR_UNSUPPORTED (-2) /* d not in {64, 128}, qk_bits not in {4, 8},
                                     pv_bits not in {8, 16}, N > 2^23                       */
#define SAGE_ERR_WORKSPACE (-3)   /* workspace missing, too small or not 256-byte aligned */
#define SAGE_ERR_HIP (-4)         /* a HIP runtime call or kernel launch failed          */

/*
 * Compile-time constants of the library: the block sizes and quantization-group geometry that
 * fix the codes and scales, readable by callers (and by tests that check a reference against
 * them).
 *   bq      : query rows per workgroup and per Q-smoothing block (mu_Q is per bq rows)
 *   bk      : keys per KV block: online-softmax block, block-local PV accumulation span,
 *             and the slice of K sharing quantization scales
 *   A quantization group of rows is the set sharing (row / slice, (row % period) / run):
 *   q_*     : Q groups; (1, 1, 1) = one scale per query row.  In S^T = K Q^T on the
 *             32x32 integer MFMA each lane holds one query column [SA2 thread granularity].
 *   k_*     : K groups; (bk, 8, 4): keys 8a + 4h + r (r < 4) of a KV block share the
 *             scale of lane half h, the keys one lane accumulates.
 *   p_range, v_range : static FP8 ranges P_r, V_r
 *   fp8_format : 1 = OCP E4M3FN (max 448, RNE)
 */
typedef struct sage_config {
  int version;
  int bq, bk;
  int q_slice, q_period, q_run;
  int k_slice, k_period, k_run;
  float p_range, v_range;
  int fp8_format;
} sage_config_t;

int sage_get_config(sage_config_t* out);

/*
 * Extended problem description ([BLOG] layout conversion and varlen batches).
 *
 *   layout  SAGE_LAYOUT_HND: q, o [B, H, N, d]; k, v [B, Hkv, N, d]  (as sage_attn_fwd)
 *           SAGE_LAYOUT_NHD: q, o [B, N, H, d]; k, v [B, N, Hkv, d]  (token-major)
 *   cu_seqlens  NULL: B sequences of N tokens each, in `layout`.
 *           Otherwise a varlen batch: a HOST int32 array of B + 1 entries with
 *           cu_seqlens[0] = 0 and cu_seqlens[s] < cu_seqlens[s + 1]; sequence s holds tokens
 *           cu_seqlens[s] .. cu_seqlens[s + 1] - 1 of packed tensors q, o [T, H, d] and
 *           k, v [T, Hkv, d], T = cu_seqlens[B] (N and layout are ignored).  Each sequence is
 *           attended on its own (queries see only keys of the same sequence; causal is
 *           top-left aligned within it) and has its own smoothing means and quantization
 *           groups, exactly as if it were a batch of one.  The array is read during the
 *           call only.  Sequence lengths are at most 2^23.
 *   dtype   SAGE_DTYPE_FP16 or SAGE_DTYPE_BF16: q, k, v and o all of that type.  With bf16
 *           the smoothing means stay exact (column sums in a multi-limb integer accumulator,
 *           then RN32(RN64(sum) / n) as for fp16), O is rounded to bf16, and with pv_bits = 16
 *           P and V enter the bf16 MFMA (V keeps its input type; P is rounded to bf16).
 *           Inputs must be finite.
 * Every tensor is contiguous in its stated shape.  All other fields as for sage_attn_fwd.
 */
#define SAGE_LAYOUT_HND 0
#define SAGE_LAYOUT_NHD 1
#define SAGE_DTYPE_FP16 0
#define SAGE_DTYPE_BF16 1

typedef struct {
  int B;                  /* batch size, or number of sequences when cu_seqlens != NULL */
  int H, Hkv, N, d;
  int causal, qk_bits, pv_bits;
  int layout;             /* SAGE_LAYOUT_* */
  int dtype;              /* SAGE_DTYPE_* */
  const int* cu_seqlens;  /* host int32 [B + 1] or NULL */
} sage_problem_t;

/* Workspace bytes for *p (written to *bytes); the _ex calls below take at least this much.
 * (A sizing helper: the pages define no workspace; it holds the codes, scales, means and
 * Delta_S of the steps cited above.)  Errors as for the _ex calls' validation. */
int sage_attn_workspace_bytes_ex(const sage_problem_t* p, size_t* bytes);

/* sage_attn_fwd / sage_attn_prologue / sage_attn_attend for any problem *p (same error and
 * stream rules): the same method on varlen batches, the NHD layout and bf16 inputs, which the
 * blog page [BLOG] names in its precision-control tips (the arithmetic per sequence is that of
 * [SA2]).  The prologue and attend halves must be given the same *p and workspace. */
int sage_attn_fwd_ex(const sage_problem_t* p, const void* q, const void* k, const void* v,
                     void* o, void* workspace, size_t workspace_bytes, void* stream);
int sage_attn_prologue_ex(const sage_problem_t* p, const void* q, const void* k, const void* v,
                          void* workspace, size_t workspace_bytes, void* stream);
int sage_attn_attend_ex(const sage_problem_t* p, void* o, void* workspace,
                        size_t workspace_bytes, void* stream);

/* Bytes of workspace sage_attn_fwd needs for this problem (written to *bytes).  A sizing helper
 * (no passage defines it); SAGE_ERR_INVALID_ARG / SAGE_ERR_UNSUPPORTED as for sage_attn_fwd. */
int sage_attn_workspace_bytes(int B, int H, int Hkv, int N, int d, int causal, int qk_bits,
                              int pv_bits, size_t* bytes);

/*
 * The whole forward pass: quantize/smooth prologue kernels, then the fused attention
 * kernel, all enqueued on `stream`.  Replaces F.scaled_dot_product_attention(q, k, v,
 * is_causal=causal) for fp16 inputs [BLOG core API; SA2].
 */
int sage_attn_fwd(const void* q, const void* k, const void* v, void* o, int B, int H, int Hkv,
                  int N, int d, int causal, int qk_bits, int pv_bits, void* workspace,
                  size_t workspace_bytes, void* stream);

/*
 * The two halves of sage_attn_fwd, for callers that time or schedule them separately.
 * sage_attn_prologue smooths and quantizes q, k, v into `workspace` (K/Q/V codes, scales,
 * means and the Delta_S bias: [SA2] abstract on smoothing Q and thread-granular quantization,
 * [SA2c] on smoothing K, [SA2pp key_machinery] on per-channel FP8 V); sage_attn_attend is
 * the online softmax, FP8 P~ and two-level P~V of [SA2] and [SA2c].  sage_attn_attend runs the fused attention kernel on a
 * workspace the prologue filled for the same (B, H, Hkv, N, d, causal, qk_bits, pv_bits) and writes
 * o; a workspace filled for another problem gives meaningless output.  Stream ordered;
 * same argument and error rules as sage_attn_fwd.
 */
int sage_attn_prologue(const void* q, const void* k, const void* v, int B, int H, int Hkv, int N,
                       int d, int causal, int qk_bits, int pv_bits, void* workspace,
                       size_t workspace_bytes, void* stream);
int sage_attn_attend(void* o, int B, int H, int Hkv, int N, int d, int causal, int qk_bits,
                     int pv_bits, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Test/debug: run the prologue only and copy its results, in plain layouts, to the
 * caller's device buffers (any pointer may be NULL to skip it).  The quantities are those of
 * [SA2] (smoothing, thread-granular codes and scales, the mean(q) gamma(K)^T correction),
 * [SA2c] (K smoothing) and [SA2pp key_machinery] (per-channel V):
 *   mu_k     fp32 [B, Hkv, d]            mean of K over all N keys
 *   k_codes  int8 [B, Hkv, N, d]         quantized smoothed K
 *   k_scales fp32 [B, Hkv, N]            scale of each key's group
 *   v_codes  uint8 [B, Hkv, N, d]        FP8 E4M3 codes of V (must be NULL when pv_bits = 16)
 *   v_scales fp32 [B, Hkv, d]            delta_V = max|V[:, c]| / V_r (NULL when pv_bits = 16)
 *   mu_q     fp32 [B, H, ceil(N/bq), d]  per-block mean of Q
 *   q_codes  int8 [B, H, N, d]           quantized smoothed Q
 *   q_scales fp32 [B, H, N]              scale of each query's group
 *   delta_s  fp32 [B, H, ceil(N/bq), N] mu_Q . gamma_K^T (natural units, not log2); when
 *            causal, row qb holds only keys j < (qb + 1) * bq (the keys that block can see)
 *            and zeros beyond
 * Same tensor/workspace/stream rules as sage_attn_fwd.
 */
int sage_quant_debug(const void* q, const void* k, const void* v, int B, int H, int Hkv, int N,
                     int d, int causal, int qk_bits, int pv_bits, void* workspace,
                     size_t workspace_bytes, void* stream, void* mu_k, void* k_codes,
                     void* k_scales, void* v_codes, void* v_scales, void* mu_q, void* q_codes,
                     void* q_scales, void* delta_s);

/* sage_quant_debug for a fixed-length problem *p in any layout and dtype (varlen problems
 * return SAGE_ERR_INVALID_ARG); the outputs have the plain layouts above. */
int sage_quant_debug_ex(const sage_problem_t* p, const void* q, const void* k, const void* v,
                        void* workspace, size_t workspace_bytes, void* stream, void* mu_k,
                        void* k_codes, void* k_scales, void* v_codes, void* v_scales, void* mu_q,
                        void* q_codes, void* q_scales, void* delta_s);

/*
 * Test/debug: run the prologue, then the attention kernel's own integer-MFMA QK^T code
 * path ([SA2] abstract: QK^T on the low-bit integer codes) for query block qb of (b, h)
 * against KV block kb, and copy the raw int32
 * accumulators to tile_out (device, int32 [bq, bk], row = query, column = key; keys past N
 * hold products with K's zero padding codes, rows past N products of the padded query rows'
 * codes, which no output reads).
 */
int sage_qk_tile_debug(const void* q, const void* k, const void* v, int B, int H, int Hkv, int N,
                       int d, int causal, int qk_bits, int pv_bits, void* workspace,
                       size_t workspace_bytes, void* stream, int b, int h, int qb, int kb,
                       int32_t* tile_out);

/*
 * Allocation-free forward pass, for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): sage_attn_fwd_ex for a
 * fixed-length problem (p->cu_seqlens must be NULL), with the workspace taken from a device
 * array inside the library instead of the caller.
 *   The array holds 128 MiB (134217728 bytes) on every GPU the library runs on, from the first
 *   call on that GPU until the process ends; problems whose sage_attn_workspace_bytes_ex exceeds
 *   it return SAGE_ERR_WORKSPACE (sage_last_error() states both sizes) before anything is
 *   enqueued.  Example: B1 H16 N8192 d128 non-causal needs about 85 MB.
 *   The current device must be the device of q, k, v, o and stream (a stream on another device
 *   returns SAGE_ERR_INVALID_ARG); its copy of the array is used.
 *   Every call on one GPU shares that GPU's array, and the library makes no synchronisation:
 *   calls on one GPU whose executions overlap (different streams, or host threads racing on one
 *   stream) race on it and give meaningless output.  Calls ordered on one stream are safe.  The
 *   array keeps the last call's contents; each call re-initialises what it reads.
 *   No hipMalloc, hipFree or other allocating call is made; the first call on a device looks up
 *   the array's device address (hipGetSymbolAddress) and keeps it.
 * Errors as for sage_attn_fwd_ex.
 */
int sage_attn_fwd_noalloc(const sage_problem_t* p, const void* q, const void* k, const void* v, void* o,
                          void* stream);

/*
 * Measurement utility (not part of the method): enqueue a launch that keeps every SIMD's matrix
 * unit busy with one dense MFMA instruction, register operands only, two waves per SIMD, so that
 * timing it gives the sustained matrix rate at the clock the chip runs at.
 *   kind  0: v_mfma_i32_32x32x32_i8 (INT8), 1: v_mfma_f32_32x32x64_f8f6f4 with FP8 E4M3,
 *         2: the same with FP6 E2M3, 3: v_mfma_f32_32x32x16_f16
 *   iters rounds of four independent accumulator chains per wave (>= 1)
 *   sink  device buffer of at least 512 KiB; overwritten with the accumulator sums
 *   *ops  (host) receives the number of multiply-add operations (x2) the launch performs
 * Errors: SAGE_ERR_INVALID_ARG (kind, iters, null pointer), SAGE_ERR_WORKSPACE (sink too
 * small), SAGE_ERR_HIP (launch failed).  Stream ordered; returns after enqueueing.
 */
int sage_mfma_rate_probe(int kind, int iters, void* sink, size_t sink_bytes, double* ops, void* stream);

/* Static text for a status code (library plumbing; no passage). */
const char* sage_status_string(int status);

/* Detail of the last SAGE_ERR_HIP on the calling thread ("" if none; library plumbing). */
const char* sage_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* SAGE_ATTN_H */
