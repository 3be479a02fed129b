/*
 * qdm.h — C ABI of the Q4_K / Q5_K / Q6_K / Q8_0 dequantize-fused matmul
 * library for MI355X (gfx950), with the top-k router in front of its MoE
 * grouped matmul. Shared library: libqdm.so.
 *
 * What it computes. GGUF k-quant weights stay packed in HBM and are decoded on
 * the fly inside the matmul: a GEMV for decode and a matrix-core GEMM for
 * prefill over the same weights (hipEngine README, "Quickstart": WMMA prefill
 * and GEMV decode; "GGUF Support": Q4_K and Q6_K tensor families of a Q4_K_M
 * file, read by GGUF-specific quant readers), and an expert-grouped matmul for
 * a routed MoE FFN (hipster README, "Verify the claims": MoE grouped GEMM
 * micro-benchmark).
 *
 * Weight layout. A weight tensor W has N output rows of K weights; each row is
 * K/256 consecutive super-blocks (Q8_0: K/32 blocks of 32 weights) and rows
 * are contiguous (row n starts at byte n * (K/256) * block_bytes; Q8_0:
 * n * (K/32) * 34). The value of weight (n, k) is:
 *   Q4_K (144-byte block): fp16 d @0, fp16 dmin @2, 12 bytes of packed 6-bit
 *     scales/mins @4, 128 bytes of 4-bit codes @16 (chunk c of 32 bytes holds
 *     sub-block 2c in its low nibbles and 2c+1 in its high nibbles);
 *     w = d * sc_j * q - dmin * m_j for the 32-weight sub-block j.
 *   Q5_K (176-byte block): the Q4_K header (d @0, dmin @2, packed scales/mins
 *     @4), 32 bytes of fifth code bits @16 (bit j of byte l belongs to weight l
 *     of sub-block j), and the Q4_K arrangement of 128 bytes of low 4 bits
 *     @48; q = low | fifth << 4 in 0..31 and w = d * sc_j * q - dmin * m_j.
 *     The pages name Q5_K as the expert-down type of a Q4_K_M file (hipEngine
 *     README, "GGUF Support", payload table) without its byte layout; this
 *     layout is the reading the library and its tests share.
 *   Q6_K (210-byte block): 128 bytes of low 4 bits @0, 64 bytes of high 2 bits
 *     @128, 16 int8 scales @192 (one per 16 weights), fp16 d @208;
 *     w = d * scale * (q - 32), q in 0..63.
 *   Q8_0 (34-byte block of 32 weights): fp16 d @0, 32 two's-complement int8
 *     codes @2; w = d * q. Named in the same payload table without a layout;
 *     this is the reading the library and its tests share.
 *
 * Matmul convention. X is [M][K] row-major (fp32 or bf16), Y = X * W^T is
 * [M][N] fp32 row-major and is overwritten (no accumulation into Y).
 *
 * Conventions for every entry point:
 *  - All data pointers are device pointers; `stream` is a hipStream_t passed
 *    as void* (NULL = the null stream). Work is enqueued asynchronously; the
 *    library never synchronizes, never allocates, never frees and never reads
 *    device data on the host. The caller owns every buffer.
 *  - Arguments are validated on the host before anything is launched. On a
 *    failed check the call returns a negative status and enqueues nothing
 *    (outputs are untouched). A launch error reported by the HIP runtime maps
 *    to QDM_ERR_HIP. There is no fallback path of any kind.
 *  - Alignment: w, x, y, out and workspace must be 16-byte aligned (the
 *    router's logits, ids and weights: 4-byte aligned).
 *  - Calls are stateless and may overlap on different streams as long as
 *    their outputs and workspaces do not overlap.
 */
#ifndef QDM_H
#define QDM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* activation dtypes */
#define QDM_F32 0
#define QDM_BF16 1

/* weight types (moe_grouped_gemm_from_logits down experts) */
#define QDM_Q4_K 4
#define QDM_Q5_K 5

/* status codes */
#define QDM_OK 0
#define QDM_ERR_NULL (-1)      /* a required pointer is NULL */
#define QDM_ERR_SHAPE (-2)     /* bad size (K % 256, non-positive, limits) */
#define QDM_ERR_ALIGN (-3)     /* a pointer is not 16-byte aligned */
#define QDM_ERR_DTYPE (-4)     /* unknown or unsupported activation dtype or weight type */
#define QDM_ERR_WORKSPACE (-5) /* workspace missing or too small */
#define QDM_ERR_HIP (-6)       /* the HIP runtime reported an error */
#define QDM_ERR_SCRATCH (-7)   /* more scratch than moe_q4k_grouped_gemm_noalloc holds */

/* Bytes of the static scratch array behind moe_q4k_grouped_gemm_noalloc. */
#define QDM_MOE_SCRATCH_BYTES (16u << 20)

/* Human-readable text for a status code (static storage). */
const char *qdm_status_string(int status);

/* Library ABI version (major * 100 + minor). */
int qdm_version(void);

/*
 * q4k_dequantize / q5k_dequantize / q6k_dequantize: out[n][k] (fp32, [N][K]
 * row-major) = the value of weight (n, k), bit-identical to the format formula
 * evaluated in fp32 (every product in it is exact in fp32, so the result is
 * the single correctly rounded value; Q6_K values are exact). Test-facing.
 * Source: hipEngine README, "GGUF Support" (payload table: the Q4_K, Q5_K and
 * Q6_K tensor families of a Q4_K_M file, read by GGUF-specific quant readers);
 * the formulas are those of the layout preamble above.
 * w: the packed tensor (read only); out: caller-owned, fully overwritten.
 * N >= 1, K >= 256, K % 256 == 0, else QDM_ERR_SHAPE; NULL pointers give
 * QDM_ERR_NULL, pointers not 16-byte aligned QDM_ERR_ALIGN.
 */
int q4k_dequantize(const void *w, float *out, int64_t N, int64_t K, void *stream);
int q5k_dequantize(const void *w, float *out, int64_t N, int64_t K, void *stream);
int q6k_dequantize(const void *w, float *out, int64_t N, int64_t K, void *stream);

/*
 * q80_dequantize: as above for Q8_0 (the type is named in the hipEngine
 * README, "GGUF Support", payload table; the layout is a reading): 34-byte
 * blocks of 32 weights, fp16 d @0 then 32 two's-complement int8 codes q @2,
 * w = d * q (exact in fp32). A row of W is K/32 consecutive blocks.
 * N >= 1, K >= 256, K % 256 == 0 (a row is then a whole number of 16-byte
 * chunks).
 */
int q80_dequantize(const void *w, float *out, int64_t N, int64_t K, void *stream);

/*
 * q4k_gemv / q5k_gemv / q6k_gemv: decode-regime matmul,
 * y[m][n] = sum_k x[m][k] * w(n,k)
 * for 1 <= M <= 16. Source: hipEngine README, "Quickstart" (decode runs a
 * GEMV over the quantized weights) and hipster README, "Verify the claims"
 * (the GEMV micro-benchmark, reported in GB/s).
 * w: packed [N][K/256] blocks (read only); x: [M][K] row-major, fp32 or bf16
 * (read only); y: [M][N] fp32, caller-owned, fully overwritten.
 * x_dtype is QDM_F32 or QDM_BF16 (else QDM_ERR_DTYPE). Accumulation is fp32.
 * N >= 1, K >= 256, K % 256 == 0, K <= 65536 (bf16 x) or K <= 32768 (fp32 x):
 * one activation row is staged in the 160 KiB LDS of a compute unit.
 * q4k_gemv, q5k_gemv and q6k_gemv with bf16 x and M >= 2 run on the matrix
 * cores: each weight is decoded in fp32 (exact, or the single rounding of
 * d*sc*q - dmin*m) and rounded to bf16 (nearest even) before the
 * bf16 x bf16 -> fp32 contraction, as in q4k_gemm. Every other case keeps the
 * weights in fp32. Results are deterministic.
 */
int q4k_gemv(const void *w, const void *x, int x_dtype, float *y,
             int64_t M, int64_t N, int64_t K, void *stream);
int q5k_gemv(const void *w, const void *x, int x_dtype, float *y,
             int64_t M, int64_t N, int64_t K, void *stream);
int q6k_gemv(const void *w, const void *x, int x_dtype, float *y,
             int64_t M, int64_t N, int64_t K, void *stream);

/*
 * q80_gemv: the same decode-regime matmul with Q8_0 weights (w: [N][K/32]
 * 34-byte blocks, layout as in q80_dequantize). Arguments, limits and status
 * codes as q4k_gemv; x is staged per column chunk. With fp32 x, or M = 1,
 * weights are applied in fp32 (exact); with bf16 x and M >= 2 the call runs
 * on the matrix cores with the weights rounded to bf16 (nearest even), as
 * q4k_gemv does. Accumulation is fp32. Results are deterministic.
 */
int q80_gemv(const void *w, const void *x, int x_dtype, float *y,
             int64_t M, int64_t N, int64_t K, void *stream);

/*
 * q4k_gemm: prefill-regime matmul on the matrix cores. Source: hipEngine
 * README, "Quickstart" (prefill runs on the matrix cores, decode on a GEMV)
 * and "GGUF Support" (a bulk-prefill path over the GGUF quant readers).
 * x is bf16 [M][K] (read only); the Q4_K weights w [N][K/256] (read only) are
 * decoded in fp32 and rounded to bf16 (nearest even) before the
 * bf16 x bf16 -> fp32 MFMA contraction; y is fp32 [M][N], fully overwritten.
 * M >= 1, 1 <= N <= 2^20, K >= 256, K % 256 == 0 (else QDM_ERR_SHAPE).
 * When that gives every compute unit at least two of the K/128 stage pairs,
 * the 256 x 256 tiles x K iteration space is split evenly over one workgroup
 * per compute unit, and a tile computed by several workgroups is summed in a
 * fixed order (results are deterministic); otherwise each tile is one
 * workgroup.
 * workspace: q4k_gemm_workspace_bytes(M, N, K) bytes, 16-byte aligned, on the
 * device of the call; 0 bytes (workspace may be NULL) when no tile is split
 * (few tiles and short K).
 * Otherwise: a 256-byte status block, a flag word per workgroup, then one fp32
 * 256 x 256 partial tile per workgroup (a too-small or NULL workspace gives
 * QDM_ERR_WORKSPACE). It must be zero-filled before its first use; every call
 * leaves the flag words zero again, so one buffer serves any number of calls
 * in stream order. Two calls that overlap in time (different streams) need
 * different workspaces. The size depends on the current device's
 * compute-unit count (256 if no device is visible).
 * Status word (32-bit word 0 of the workspace): the number of split-tile
 * waits that gave up (a partial tile that did not arrive within about a
 * second of polling), counted across calls and never cleared by the library.
 * Such a tile of y is written as NaN. The caller reads the word after the
 * stream has synchronized; it stays 0 in normal operation.
 */
size_t q4k_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K);
int q4k_gemm(const void *w, const void *x, float *y, int64_t M, int64_t N, int64_t K,
             void *workspace, size_t workspace_bytes, void *stream);

/*
 * qdm_set_gemm_spin_limit: polls a q4k_gemm owner makes before giving up on a
 * split-tile partial (0 restores the default, about a second). A test hook of
 * the give-up path of the workspace status word: with a tiny limit the
 * kernels still end normally, some tiles are written as NaN and counted, and
 * the flags are left zero. Process-wide; set it only while no q4k_gemm call is
 * being enqueued on another thread. Returns QDM_OK.
 */
int qdm_set_gemm_spin_limit(uint32_t polls);

/*
 * moe_q4k_grouped_gemm: routed MoE FFN with Q4_K experts, one call for the
 * whole layer. Source: hipster README, "Verify the claims" (the MoE grouped
 * GEMM micro-benchmark over an expert tensor) and hipEngine README, "Status"
 * (a routed MoE model, Qwen3.6-35B-A3B); the activation between the two
 * expert matmuls (SwiGLU, gate rows before up rows) is a reading, the pages
 * do not state it:
 *   for every token t and slot s, e = topk_ids[t][s]:
 *     u = W13[e] * x_t                  (2F values; W13[e] is [2F][H])
 *     h = silu(u[0:F]) * u[F:2F]        (gate rows first, then up rows)
 *     y_t += topk_w[t][s] * (W2[e] * h) (W2[e] is [H][F])
 *   x: bf16 [T][H]; w_gate_up: E tensors of [2F][H/256] Q4_K blocks back to
 *   back; w_down: E tensors of [H][F/256]; topk_ids int32 [T][top_k] (each in
 *   [0, E), distinct within a row); topk_w fp32 [T][top_k]; y fp32 [T][H]
 *   (overwritten). x, the weights, ids and gate weights are read only. Tokens
 *   are grouped by expert on the device (histogram, scan, scatter) so every
 *   expert's weights are streamed once per call.
 *   Ids outside [0, E) are skipped (they contribute nothing) and counted:
 *   32-bit word 0 of the workspace holds, after the call, the number of
 *   (t, s) entries of this call whose id was outside [0, E) (stored by the
 *   call's routing step; the caller reads it after the stream synchronizes).
 *   Ids repeated within a row are a precondition violation (not detected).
 *   1 <= T <= 2^24, 1 <= E <= 1024, 1 <= top_k <= 16, H and F multiples of
 *   256 and at most 65536, and each expert's tensors below 2 GiB
 *   (2F * H/256 * 176 and H * F/256 * 176 bytes under 2^31); else
 *   QDM_ERR_SHAPE.
 *   workspace: moe_q4k_workspace_bytes(T, E, top_k, H, F) bytes, 16-byte
 *   aligned, on the device of the call (scratch; no initial contents
 *   needed; too small or NULL gives QDM_ERR_WORKSPACE). Calls that overlap in
 *   time need different workspaces.
 *   With T * top_k <= 64 (decode) the call is three kernels: gate+up+SwiGLU
 *   and down, each of which routes the few entries itself, and the combine.
 *   Above that: a routing kernel, two grouped matrix-core kernels and the
 *   combine.
 */
size_t moe_q4k_workspace_bytes(int64_t T, int64_t E, int64_t top_k, int64_t H, int64_t F);
int moe_q4k_grouped_gemm(const void *x, const void *w_gate_up, const void *w_down,
                         const int32_t *topk_ids, const float *topk_w, float *y,
                         int64_t T, int64_t E, int64_t top_k, int64_t H, int64_t F,
                         void *workspace, size_t workspace_bytes, void *stream);

/*
 * moe_q4k_grouped_gemm_noalloc: moe_q4k_grouped_gemm for callers that cannot
 * allocate (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc). Same arguments and results without the workspace: the
 * call's workspace lives in a static device array of QDM_MOE_SCRATCH_BYTES
 * (16 MiB) that each GPU the library runs on holds until the process ends. A
 * call whose moe_q4k_workspace_bytes(T, E, top_k, H, F) exceeds it returns
 * QDM_ERR_SCRATCH and enqueues nothing (at H = 2048, F = 768, top-8 that is
 * above 160 tokens). The call allocates and frees nothing. All calls on one
 * GPU share its array: two calls that overlap in time on one GPU (different
 * streams) race and give wrong results; calls in stream order are safe. The
 * stream must belong to the current device. The skipped-id count is kept in
 * the array and not exposed.
 */
int moe_q4k_grouped_gemm_noalloc(const void *x, const void *w_gate_up, const void *w_down,
                                 const int32_t *topk_ids, const float *topk_w, float *y,
                                 int64_t T, int64_t E, int64_t top_k, int64_t H, int64_t F,
                                 void *stream);

/*
 * moe_q4k_q5k_grouped_gemm: the same routed MoE FFN with Q4_K gate+up experts
 * and Q5_K down experts (w_down: E tensors of [H][F/256] Q5_K blocks), the
 * expert arrangement of a Q4_K_M file (hipEngine README, "GGUF Support":
 * Q5_K holds the MoE expert-down payload). Arguments, limits, workspace
 * (moe_q4k_workspace_bytes) and status codes are those of
 * moe_q4k_grouped_gemm.
 */
int moe_q4k_q5k_grouped_gemm(const void *x, const void *w_gate_up, const void *w_down,
                             const int32_t *topk_ids, const float *topk_w, float *y,
                             int64_t T, int64_t E, int64_t top_k, int64_t H, int64_t F,
                             void *workspace, size_t workspace_bytes, void *stream);

/*
 * moe_router_topk: the router in front of the MoE grouped matmul (hipEngine
 * README, "Status", names a routed MoE model, Qwen3.6-35B-A3B, but not its
 * router; this is the plainest reading of one). For each token t of the
 * logits [T][E] (fp32, finite): topk_ids[t] = the top_k experts with the
 * largest logits, largest first, the smaller index first among equal logits;
 * topk_w[t][s] = exp(l_s - l_0) / sum_j exp(l_j - l_0) over the selected
 * logits (the softmax of the selection), fp32. Integer results are exact;
 * the weights are within a few fp32 ulps of the float64 softmax.
 * 1 <= T <= 2^24, 1 <= E <= 1024, 1 <= top_k <= min(16, E). topk_ids int32
 * [T][top_k] and topk_w fp32 [T][top_k] are overwritten. The three arrays
 * need only 4-byte alignment.
 */
int moe_router_topk(const float *logits, int64_t T, int64_t E, int64_t top_k,
                    int32_t *topk_ids, float *topk_w, void *stream);

/*
 * moe_grouped_gemm_from_logits: moe_router_topk followed by the routed MoE
 * FFN in one call (gate+up experts Q4_K; down experts QDM_Q4_K or QDM_Q5_K
 * by down_qtype). The ids and gate weights live in the workspace:
 * moe_from_logits_workspace_bytes(T, E, top_k, H, F) bytes (scratch, no
 * initial contents). router_logits: fp32 [T][E], 4-byte aligned. Arguments
 * and limits otherwise as moe_q4k_grouped_gemm; top_k <= E. A down_qtype
 * other than the two returns QDM_ERR_DTYPE.
 */
size_t moe_from_logits_workspace_bytes(int64_t T, int64_t E, int64_t top_k, int64_t H,
                                       int64_t F);
int moe_grouped_gemm_from_logits(const void *x, const float *router_logits,
                                 const void *w_gate_up, const void *w_down, int down_qtype,
                                 float *y, int64_t T, int64_t E, int64_t top_k, int64_t H,
                                 int64_t F, void *workspace, size_t workspace_bytes,
                                 void *stream);

/*
 * qdm_probe_copy: streaming copy of n_bytes from src to dst (n_bytes % 16 ==
 * 0). A plain, known-size kernel used to calibrate memory-traffic counters
 * and to measure the achievable HBM bandwidth of the device (hipster README,
 * "Hardware and software this was measured on": measured roofs beside the
 * nominal ones).
 */
int qdm_probe_copy(const void *src, void *dst, int64_t n_bytes, void *stream);

/*
 * Roofline probes (the same source: measured roofs beside the nominal ones).
 * qdm_probe_read: reads the n_bytes of src once (n_bytes % 16 == 0, src
 *   16-byte aligned), a read-only HBM (or, for a buffer re-read while it fits
 *   the 256 MB last-level cache, cache) stream, each of up to 1024
 *   workgroups reading one contiguous slice; sink is a 4-byte device word
 *   the kernel may write (so no load can be dropped).
 * qdm_probe_mfma: `workgroups` workgroups of four waves, each wave issuing
 *   iters x 8 back-to-back bf16 MFMAs of 32 x 32 x 16 (32768 flops each);
 *   1 <= iters <= 2^24, 1 <= workgroups <= 65536. clocks (8-byte aligned,
 *   2 * workgroups uint64) receives per workgroup the shader-clock and the
 *   100 MHz reference-clock ticks of its first wave's loop (their ratio is the
 *   shader clock under MFMA load); sink is a 4-byte device word as above.
 * qdm_probe_empty: a launch of `workgroups` workgroups that do nothing (the
 *   per-launch cost), 1 <= workgroups <= 65536.
 * Status codes as elsewhere (NULL, size, alignment checked first).
 */
int qdm_probe_read(const void *src, int64_t n_bytes, void *sink, void *stream);
int qdm_probe_mfma(int64_t iters, int64_t workgroups, float *sink, uint64_t *clocks,
                   void *stream);
int qdm_probe_empty(int64_t workgroups, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* QDM_H */
