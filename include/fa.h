/*
 * fa.h — C ABI of the MI355X (gfx950) exact-attention library, libfa.so.
 *
 * The library computes exact attention O = softmax(scale · Q Kᵀ) · V with the tiled, IO-aware method:
 * the N×N scores S and probabilities P exist only as on-chip tiles and are never written to device
 * memory ("Anatomy of a FlashAttention Kernel", section "Why is attention memory-bound, and how does
 * FlashAttention fix it?"; "flash attention" glossary entry, comparison table).  The forward streams
 * key/value tiles with the online softmax (same page, section "What is online softmax and how does
 * tiling keep it exact?") and keeps one statistic per query row; the backward recomputes S and P tile
 * by tile from Q, K, V and that statistic (section "How does FlashAttention save memory in the
 * backward pass?").
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  Layout     Q, K, V, O, dO, dQ, dK, dV are contiguous [B, H, N, d] arrays, d innermost, 16-bit
 *             elements unless stated; element (b,h,i,t) is at ((b·H + h)·N + i)·d + t.  LSE is a
 *             contiguous fp32 [B, H, N] array.  Queries and keys share the sequence length N.
 *  LSE        LSE_i = ln Σ_j exp(scale · q_i·k_j) over the keys query i may use: natural log of the
 *             scaled scores.  It stands for the pair (row maximum, softmax denominator).
 *  Causal     causal != 0 lets query i use key j only when j ≤ i; causal == 0 lets it use all keys.
 *  Supported  d ∈ {64, 96, 128, 256}; N ≥ 1; B, H ≥ 1; B·H·N·d < 2^40.  bf16 values are IEEE
 *             bfloat16.
 *  Memory     Every pointer is a device pointer owned by the caller and 16-byte aligned.  The library
 *             never allocates or frees device memory and keeps no state between calls, except for the
 *             fixed device array behind fa_bwd_noalloc (see there).
 *  Streams    Every call only enqueues work on `stream` and returns; results are ready when the stream
 *             reaches that point.  Calls are re-entrant and may be made on several streams at once.
 *  Errors     Arguments are checked before any HIP call; a failed check returns its status and enqueues
 *             nothing.  A launch failure reported by the HIP runtime returns FA_ERR_LAUNCH.  Faults
 *             inside a kernel surface at the caller's next synchronisation of the stream.
 */
#ifndef FA_H_
#define FA_H_

#include <stddef.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FA_OK = 0,
  FA_ERR_NULL = 1,        /* a required pointer is NULL                                   */
  FA_ERR_SHAPE = 2,       /* B, H or N < 1, or the element count is out of range           */
  FA_ERR_UNSUPPORTED = 3, /* d not in {64, 96, 128, 256}, or a bad scale / descale     */
  FA_ERR_ALIGN = 4,       /* a pointer is not 16-byte aligned                              */
  FA_ERR_WORKSPACE = 5,   /* backward workspace is NULL or smaller than fa_bwd_workspace_bytes */
  FA_ERR_LAUNCH = 6       /* the HIP runtime rejected a kernel launch                      */
} fa_status;

/*
 * Forward pass, bf16 in, bf16 out ("Anatomy of a FlashAttention Kernel", sections "Why is attention
 * memory-bound ..." and "What is online softmax ...").
 *   q, k, v   [B,H,N,d] bf16 inputs.
 *   o         [B,H,N,d] bf16 output, O = softmax(scale · Q Kᵀ) V (fp32 accumulation, rounded once).
 *   lse       [B,H,N] fp32 output, the per-row logsumexp defined above.
 *   softmax_scale  multiplier of Q Kᵀ (1/√d for standard attention); finite and > 0.
 */
fa_status fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                 int B, int H, int N, int d, int causal, float softmax_scale, hipStream_t stream);

/*
 * Forward pass as fa_fwd, with a workspace that lets the library split each query tile's key range
 * when B·H·⌈N/128⌉ is too small to fill the device (few heads, long sequences: the long-context case
 * of "FlashAttention: where it matters", section "Where It Matters").  Each key segment's partial
 * result (unnormalised output, reference maximum, row sums) goes to the workspace and a second kernel
 * combines a row's segments by their softmax mass: the recurrence of "Anatomy of a FlashAttention
 * Kernel", section "What is online softmax and how does tiling keep it exact?", applied to whole key
 * ranges.  The result is the same attention, within rounding of fa_fwd's: each segment rounds its
 * probabilities to bf16 against its own reference maximum, and the sums run in another order.
 *   workspace  device memory of at least fa_fwd_split_workspace_bytes(B, H, N, d, causal) bytes,
 *              256-byte aligned, owned by the caller, contents undefined after the call.  May be NULL
 *              when that size is 0: the shape is not split and the call is fa_fwd.
 * Split rule: with d ≤ 128, T = the number of 64-key tiles summed over every (batch·head, 128-query
 * tile) pair (under the causal mask a query tile's keys end at its last query) and kt = ⌈N/64⌉, the
 * shape is split when 2·kt·512 ≥ 5·T, or 2·kt·512 ≥ 3·T and kt ≥ 256 (512: two workgroups on each
 * of the device's 256 compute units), into segments of seg = min(128, max(16, ⌊kt/8⌋)) tiles,
 * provided seg < kt; nseg = ⌈kt/seg⌉ segments, and the workspace is nseg·B·H·N·(d + 3) fp32 values
 * rounded up to 256 bytes.  Otherwise the workspace is 0.
 * Errors: as fa_fwd; FA_ERR_WORKSPACE when the workspace is needed and NULL or too small,
 * FA_ERR_ALIGN when it is not 256-byte aligned.  Head dimension 256 is never split.
 */
size_t fa_fwd_split_workspace_bytes(int B, int H, int N, int d, int causal);
fa_status fa_fwd_split(const void* q, const void* k, const void* v, void* o, float* lse,
                       void* workspace, size_t workspace_bytes, int B, int H, int N, int d,
                       int causal, float softmax_scale, hipStream_t stream);

/*
 * Forward pass with FP8 matrix products ("Anatomy ...", section "What changed between FlashAttention
 * 1, 2, and 3?": low-precision FP8).  Q, K, V are OCP e4m3fn codes with one fp32 scale per tensor:
 * the value of a code c in tensor X is c · x_descale.  Both products (Q Kᵀ and P V) run on fp8 matrix
 * cores with fp32 accumulation; P is rounded to e4m3 before P V and the softmax denominator is summed
 * from those same rounded values.
 *   q8, k8, v8   [B,H,N,d] e4m3fn codes (1 byte each), 16-byte aligned.
 *   q_descale, k_descale, v_descale   finite, > 0.
 *   o            [B,H,N,d] bf16 output;  lse  [B,H,N] fp32 output (natural log, scaled scores).
 */
fa_status fa_fwd_fp8(const void* q8, const void* k8, const void* v8,
                     float q_descale, float k_descale, float v_descale, void* o, float* lse,
                     int B, int H, int N, int d, int causal, float softmax_scale, hipStream_t stream);

/*
 * FP8 forward as fa_fwd_fp8, with the key-range split of fa_fwd_split for shapes with too few query
 * tiles to fill the device: the same rule, segments and workspace size
 * (fa_fwd_split_workspace_bytes(B, H, N, d, causal); NULL allowed when that is 0, and then the call
 * is fa_fwd_fp8).  Each segment's partial output is kept in fp32 with V's descale applied, beside its
 * reference maximum and the sum of its e4m3-rounded probabilities, and the rows are merged as in
 * fa_fwd_split; each segment rounds P to e4m3 against its own reference maximum, so the result is
 * fa_fwd_fp8's within that rounding.  Errors: as fa_fwd_fp8, plus FA_ERR_WORKSPACE / FA_ERR_ALIGN
 * for the workspace.
 */
fa_status fa_fwd_fp8_split(const void* q8, const void* k8, const void* v8, float q_descale,
                           float k_descale, float v_descale, void* o, float* lse, void* workspace,
                           size_t workspace_bytes, int B, int H, int N, int d, int causal,
                           float softmax_scale, hipStream_t stream);

/*
 * Bytes of device workspace fa_bwd needs for a shape: an fp32 [B,H,N] array for D_i = dO_i · O_i,
 * rounded up to 256 bytes.  Returns 0 for an unsupported shape.
 */
size_t fa_bwd_workspace_bytes(int B, int H, int N, int d);

/*
 * Backward pass ("Anatomy ...", section "How does FlashAttention save memory in the backward pass?"):
 * recomputes the score and probability tiles from q, k, v and lse and produces the gradients of
 * O = softmax(scale · Q Kᵀ) V for the upstream gradient dout.
 *   q, k, v, o, dout  [B,H,N,d] bf16 inputs (o and lse as returned by fa_fwd for the same inputs).
 *   lse               [B,H,N] fp32 input.
 *   dq, dk, dv        [B,H,N,d] bf16 outputs (fp32 accumulation, rounded once).
 *   workspace         device scratch of at least fa_bwd_workspace_bytes(B,H,N,d) bytes, 256-byte
 *                     aligned, owned by the caller; its contents on entry do not matter and on return
 *                     are unspecified.  It must not be shared by calls in flight at the same time.
 * The result is deterministic: no atomics, fixed summation order.
 */
fa_status fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
                 const void* dout, void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes,
                 int B, int H, int N, int d, int causal, float softmax_scale, hipStream_t stream);

/*
 * The backward pass in phases, for callers that schedule or time them separately.  Arguments mean
 * what they mean for fa_bwd and are checked the same way.
 *   fa_bwd_preprocess  D_i = dO_i · O_i (fp32) into the workspace (stored as −D_i; the layout of
 *                      the workspace is internal to these calls).
 *   fa_bwd_dkdv        recomputes S and P per key tile (key/value-stationary) and writes dK and dV;
 *                      needs D in the workspace.
 *   fa_bwd_dq          recomputes S, P and dP per query tile (query-stationary) and writes dQ; needs
 *                      D in the workspace.
 *   fa_bwd_delta_dq    D into the workspace and dQ, bit for bit what fa_bwd_preprocess followed by
 *                      fa_bwd_dq give; for d ∈ {64, 128, 256} one kernel (each query tile forms its
 *                      own rows' D from O and dO), for d = 96 those two calls.
 * fa_bwd enqueues fa_bwd_delta_dq, then fa_bwd_dkdv; fa_bwd_preprocess, fa_bwd_dkdv, fa_bwd_dq in
 * that order (or with the last two swapped) give the same gradients bit for bit.
 */
fa_status fa_bwd_preprocess(const void* o, const void* dout, void* workspace, size_t workspace_bytes,
                            int B, int H, int N, int d, hipStream_t stream);
fa_status fa_bwd_dkdv(const void* q, const void* k, const void* v, const float* lse,
                      const void* dout, void* dk, void* dv, const void* workspace,
                      size_t workspace_bytes, int B, int H, int N, int d, int causal,
                      float softmax_scale, hipStream_t stream);
fa_status fa_bwd_dq(const void* q, const void* k, const void* v, const float* lse,
                    const void* dout, void* dq, const void* workspace, size_t workspace_bytes,
                    int B, int H, int N, int d, int causal, float softmax_scale,
                    hipStream_t stream);
fa_status fa_bwd_delta_dq(const void* q, const void* k, const void* v, const void* o,
                          const float* lse, const void* dout, void* dq, void* workspace,
                          size_t workspace_bytes, int B, int H, int N, int d, int causal,
                          float softmax_scale, hipStream_t stream);

/*
 * Backward pass as fa_bwd, with a workspace that lets the library split the loops of both backward
 * kernels for the same shapes fa_fwd_split splits (few heads, long sequences).  The dQ kernel splits
 * each 128-query tile's key range into fa_fwd_split's segments of seg 64-key tiles; the dK/dV kernel
 * splits each 128-key block's query range into segments of 2·seg 32-query steps.  Each segment writes
 * fp32 partial sums of its gradients to the workspace and a last kernel adds a row's segments, applies
 * the scale and rounds to bf16 (the gradients of "Anatomy of a FlashAttention Kernel", section "How
 * does FlashAttention save memory in the backward pass?", summed over key or query ranges in another
 * grouping).  Each probability is recomputed exactly as fa_bwd does; only the order of the
 * gradient sums differs, so results can differ from fa_bwd's in the last bits.
 *   workspace  at least fa_bwd_split_workspace_bytes(B, H, N, d, causal) bytes, 256-byte aligned,
 *              owned by the caller, contents undefined after the call: −D_i (as fa_bwd), then, when
 *              split, nseg_q·B·H·N·d fp32 partial dQ sums and nseg_k·B·H·N·d each for dK and dV,
 *              each array rounded up to 256 bytes, with nseg_q = fa_fwd_split's nseg and nseg_k =
 *              ⌈⌈N/32⌉ / (2·seg)⌉.  Without a split the size is fa_bwd_workspace_bytes and the call is
 *              fa_bwd.
 * Errors: as fa_bwd.
 */
size_t fa_bwd_split_workspace_bytes(int B, int H, int N, int d, int causal);
fa_status fa_bwd_split(const void* q, const void* k, const void* v, const void* o,
                       const float* lse, const void* dout, void* dq, void* dk, void* dv,
                       void* workspace, size_t workspace_bytes, int B, int H, int N, int d,
                       int causal, float softmax_scale, hipStream_t stream);

/*
 * Backward pass of the FP8 forward (fa_fwd_fp8): the gradients of O = softmax(scale · Q Kᵀ) V with
 * respect to the dequantised inputs Q = q8 · q_descale, K = k8 · k_descale, V = v8 · v_descale
 * ("Anatomy ...", sections "How does FlashAttention save memory in the backward pass?" and "What
 * changed between FlashAttention 1, 2, and 3?").  The e4m3 codes are widened exactly to bf16 images
 * in the workspace and the bf16 backward runs on them with the descales folded into its scalar
 * factors; the products run on bf16 matrix cores with fp32 accumulation.
 *   q8, k8, v8   [B,H,N,d] e4m3fn codes as given to fa_fwd_fp8; descales finite and > 0.
 *   o, lse       fa_fwd_fp8's outputs for those inputs;  dout [B,H,N,d] bf16 upstream gradient.
 *   dq, dk, dv   [B,H,N,d] bf16 outputs.
 *   workspace    at least fa_bwd_fp8_workspace_bytes(B,H,N,d) bytes, 256-byte aligned, owned by the
 *                caller (D, then the bf16 images of q8, k8, v8); contents on entry do not matter.
 * d as for fa_bwd.  Errors as for fa_bwd; FA_ERR_UNSUPPORTED also when a descale, or a product of the
 * softmax scale with two descales, is not a positive normal fp32 number.
 */
size_t fa_bwd_fp8_workspace_bytes(int B, int H, int N, int d);
fa_status fa_bwd_fp8(const void* q8, const void* k8, const void* v8, float q_descale,
                     float k_descale, float v_descale, const void* o, const float* lse,
                     const void* dout, void* dq, void* dk, void* dv, void* workspace,
                     size_t workspace_bytes, int B, int H, int N, int d, int causal,
                     float softmax_scale, hipStream_t stream);

/* ---------------------------------------------------------------------------------------------------
 * Decoding against a key/value cache: a few new queries per (batch, head) attend over Nk cached keys,
 * the inference use the pages pair FlashAttention with ("flash attention" glossary entry, paragraph on
 * long-context training and serving; "FlashAttention: where it matters", section "Where It Matters":
 * long-context inference and speculative decoding).
 *
 *   q, o     [B, H, Nq, d] bf16, 1 ≤ Nq ≤ 32 (one new token, or a few draft tokens verified at once)
 *   k, v     [B, H, Nk, d] bf16, the cache, Nk ≥ Nq
 *   lse      [B, H, Nq] fp32, natural-log logsumexp of the scaled scores over the keys each query uses
 *   causal   the queries are the last Nq positions of the sequence: causal != 0 lets query i use key j
 *            only when j ≤ Nk − Nq + i; causal == 0 lets every query use all Nk keys
 *   workspace  device buffer of at least fa_decode_workspace_bytes(B, H, Nq, Nk, d) bytes, 256-byte
 *            aligned, owned by the caller; it receives per-chunk partial results (the keys are split
 *            into chunks attended to in parallel and merged by their softmax mass, the online-softmax
 *            recurrence of "Anatomy of a FlashAttention Kernel" applied to whole chunks) and needs no
 *            initialisation; its contents after the call are unspecified.
 *   d ∈ {64, 96, 128, 256}; other conventions as above.  Results are deterministic.
 *
 * Errors: FA_ERR_NULL (a tensor pointer is NULL), FA_ERR_SHAPE (B or H < 1, Nq outside [1, 32], Nk < Nq,
 * or the cache too large for 32-bit per-head offsets), FA_ERR_UNSUPPORTED (d, or a scale that is not
 * finite and positive), FA_ERR_WORKSPACE (workspace NULL or too small), FA_ERR_ALIGN, FA_ERR_LAUNCH.
 * fa_decode_workspace_bytes returns 0 for shapes fa_decode rejects. */
size_t fa_decode_workspace_bytes(int B, int H, int Nq, int Nk, int d);
fa_status fa_decode(const void* q, const void* k, const void* v, void* o, float* lse,
                    void* workspace, size_t workspace_bytes, int B, int H, int Nq, int Nk, int d,
                    int causal, float softmax_scale, hipStream_t stream);

/*
 * fa_bwd without a workspace argument, for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation).  The D array lives in a
 * fixed 16 MiB device array inside the library (one copy per device, held until the process ends), so
 * the call allocates nothing.  Arguments and results as for fa_bwd, plus one limit: B·H·N ≤
 * fa_bwd_noalloc_max_rows() (= 2^22); larger shapes return FA_ERR_WORKSPACE before any HIP call.
 * Every call on one device shares that device's array: calls that overlap in time on one device
 * (several streams or host threads) race and must be serialised by the caller.  The array needs no
 * initialisation: each call writes every row of D it reads.
 */
size_t fa_bwd_noalloc_max_rows(void);
fa_status fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                         const float* lse, const void* dout, void* dq, void* dk, void* dv,
                         int B, int H, int N, int d, int causal, float softmax_scale,
                         hipStream_t stream);

/* A static, human-readable name for a status code (never NULL). */
const char* fa_status_str(fa_status status);

/* Device facts for pricing measurements against the hardware: the number of compute units and the
 * peak shader clock (kHz) of HIP device `device`, as the HIP runtime reports them
 * (hipDeviceGetAttribute).  Writes both outputs and returns FA_OK; FA_ERR_NULL if an output pointer
 * is NULL; FA_ERR_LAUNCH if the runtime query fails (no such device).  Allocates nothing and
 * launches nothing.  Not part of the attention computation. */
fa_status fa_device_info(int device, int* compute_units, int* peak_clock_khz);

#ifdef __cplusplus
}
#endif

#endif /* FA_H_ */
