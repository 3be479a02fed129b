// C ABI of libqdm (declared in include/qdm.h): host-side validation, then the
// launches. Nothing here allocates, synchronizes or reads device memory.
//
// Unsupported arguments fail with a status code instead of falling back to
// another path (hipEngine README, "Quickstart": unsupported combinations fail
// instead of falling back).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/qdm.h"
#include "launch.h"

#define QDM_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

constexpr int64_t kMaxK = 65536;      // bf16 activations (x staged in LDS)
constexpr int64_t kMaxKF32 = 32768;   // fp32 activations

inline bool misaligned(const void *p) { return ((uintptr_t)p & 15u) != 0; }
inline bool misaligned4(const void *p) { return ((uintptr_t)p & 3u) != 0; }

inline int finish_launch() {
  return hipGetLastError() == hipSuccess ? QDM_OK : QDM_ERR_HIP;
}

inline bool bad_k(int64_t K) { return K < 256 || K % 256 != 0; }

}  // namespace

QDM_EXPORT const char *qdm_status_string(int status) {
  switch (status) {
    case QDM_OK: return "ok";
    case QDM_ERR_NULL: return "a required pointer is NULL";
    case QDM_ERR_SHAPE: return "invalid size argument";
    case QDM_ERR_ALIGN: return "pointer not 16-byte aligned";
    case QDM_ERR_DTYPE: return "unsupported activation dtype or weight type";
    case QDM_ERR_WORKSPACE: return "workspace missing or too small";
    case QDM_ERR_HIP: return "HIP runtime error at launch";
    case QDM_ERR_SCRATCH: return "the call needs more scratch than the static array holds";
    default: return "unknown status";
  }
}

QDM_EXPORT int qdm_version(void) { return 100; }

QDM_EXPORT int q4k_dequantize(const void *w, float *out, int64_t N, int64_t K, void *stream) {
  if (!w || !out) return QDM_ERR_NULL;
  if (N < 1 || bad_k(K)) return QDM_ERR_SHAPE;
  if (misaligned(w) || misaligned(out)) return QDM_ERR_ALIGN;
  qdm::launch_q4k_dequantize(w, out, N, K, (hipStream_t)stream);
  return finish_launch();
}

QDM_EXPORT int q5k_dequantize(const void *w, float *out, int64_t N, int64_t K, void *stream) {
  if (!w || !out) return QDM_ERR_NULL;
  if (N < 1 || bad_k(K)) return QDM_ERR_SHAPE;
  if (misaligned(w) || misaligned(out)) return QDM_ERR_ALIGN;
  qdm::launch_q5k_dequantize(w, out, N, K, (hipStream_t)stream);
  return finish_launch();
}

QDM_EXPORT int q6k_dequantize(const void *w, float *out, int64_t N, int64_t K, void *stream) {
  if (!w || !out) return QDM_ERR_NULL;
  if (N < 1 || bad_k(K)) return QDM_ERR_SHAPE;
  if (misaligned(w) || misaligned(out)) return QDM_ERR_ALIGN;
  qdm::launch_q6k_dequantize(w, out, N, K, (hipStream_t)stream);
  return finish_launch();
}

QDM_EXPORT int q80_dequantize(const void *w, float *out, int64_t N, int64_t K, void *stream) {
  if (!w || !out) return QDM_ERR_NULL;
  if (N < 1 || bad_k(K)) return QDM_ERR_SHAPE;
  if (misaligned(w) || misaligned(out)) return QDM_ERR_ALIGN;
  qdm::launch_q80_dequantize(w, out, N, K, (hipStream_t)stream);
  return finish_launch();
}

static int check_gemv(const void *w, const void *x, int x_dtype, float *y, int64_t M,
                      int64_t N, int64_t K) {
  if (!w || !x || !y) return QDM_ERR_NULL;
  if (M < 1 || M > 16 || N < 1 || N > INT32_MAX || bad_k(K) || K > kMaxK) return QDM_ERR_SHAPE;
  if (x_dtype != QDM_F32 && x_dtype != QDM_BF16) return QDM_ERR_DTYPE;
  if (x_dtype == QDM_F32 && K > kMaxKF32) return QDM_ERR_SHAPE;
  if (misaligned(w) || misaligned(x) || misaligned(y)) return QDM_ERR_ALIGN;
  return QDM_OK;
}

QDM_EXPORT int q4k_gemv(const void *w, const void *x, int x_dtype, float *y, int64_t M,
                        int64_t N, int64_t K, void *stream) {
  const int rc = check_gemv(w, x, x_dtype, y, M, N, K);
  if (rc) return rc;
  qdm::launch_q4k_gemv(w, x, x_dtype == QDM_BF16, y, M, N, K, (hipStream_t)stream);
  return finish_launch();
}

QDM_EXPORT int q5k_gemv(const void *w, const void *x, int x_dtype, float *y, int64_t M,
                        int64_t N, int64_t K, void *stream) {
  const int rc = check_gemv(w, x, x_dtype, y, M, N, K);
  if (rc) return rc;
  qdm::launch_q5k_gemv(w, x, x_dtype == QDM_BF16, y, M, N, K, (hipStream_t)stream);
  return finish_launch();
}

QDM_EXPORT int q6k_gemv(const void *w, const void *x, int x_dtype, float *y, int64_t M,
                        int64_t N, int64_t K, void *stream) {
  const int rc = check_gemv(w, x, x_dtype, y, M, N, K);
  if (rc) return rc;
  qdm::launch_q6k_gemv(w, x, x_dtype == QDM_BF16, y, M, N, K, (hipStream_t)stream);
  return finish_launch();
}

QDM_EXPORT int q80_gemv(const void *w, const void *x, int x_dtype, float *y, int64_t M,
                        int64_t N, int64_t K, void *stream) {
  const int rc = check_gemv(w, x, x_dtype, y, M, N, K);
  if (rc) return rc;
  if (!qdm::q80_gemv_fits(N, K)) return QDM_ERR_SHAPE;
  qdm::launch_q80_gemv(w, x, x_dtype == QDM_BF16, y, M, N, K, (hipStream_t)stream);
  return finish_launch();
}

QDM_EXPORT size_t q4k_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  if (M < 1 || N < 1 || bad_k(K)) return 0;
  return qdm::q4k_gemm_workspace(M, N, K);
}

QDM_EXPORT int q4k_gemm(const void *w, const void *x, float *y, int64_t M, int64_t N,
                        int64_t K, void *workspace, size_t workspace_bytes, void *stream) {
  if (!w || !x || !y) return QDM_ERR_NULL;
  // N <= 2^20: 256 rows of y are addressed with 32-bit offsets
  if (M < 1 || M > INT32_MAX || N < 1 || N > (1 << 20) || bad_k(K) || K > INT32_MAX ||
      ((M + 127) / 128) * ((N + 127) / 128) > INT32_MAX)
    return QDM_ERR_SHAPE;
  if (misaligned(w) || misaligned(x) || misaligned(y)) return QDM_ERR_ALIGN;
  const size_t need = qdm::q4k_gemm_workspace(M, N, K);
  if (need && (!workspace || workspace_bytes < need)) return QDM_ERR_WORKSPACE;
  if (need && misaligned(workspace)) return QDM_ERR_ALIGN;
  qdm::launch_q4k_gemm(w, x, y, M, N, K, workspace, (hipStream_t)stream);
  return finish_launch();
}

QDM_EXPORT int qdm_set_gemm_spin_limit(uint32_t polls) {
  qdm::set_gemm_spin_limit(polls);
  return QDM_OK;
}

QDM_EXPORT size_t moe_q4k_workspace_bytes(int64_t T, int64_t E, int64_t top_k, int64_t H,
                                          int64_t F) {
  if (T < 1 || E < 1 || top_k < 1 || top_k > 16 || bad_k(H) || bad_k(F)) return 0;
  return qdm::moe_workspace(T, E, top_k, H, F);
}

// Arguments of the MoE FFN shared by the entry points (the routing inputs,
// ids and gate weights or router logits, are checked by each caller).
static int check_moe(const void *x, const void *w_gate_up, const void *w_down, float *y,
                     int64_t T, int64_t E, int64_t top_k, int64_t H, int64_t F,
                     void *workspace, size_t workspace_bytes) {
  if (!x || !w_gate_up || !w_down || !y) return QDM_ERR_NULL;
  if (T < 1 || T > (1 << 24) || E < 1 || E > 1024 || top_k < 1 || top_k > 16 || bad_k(H) ||
      bad_k(F) || H > kMaxK || F > kMaxK)
    return QDM_ERR_SHAPE;
  // one expert's tensor must stay below 2 GiB (the kernels address it with
  // 32-bit offsets); 176 bytes per 256 weights covers Q4_K and Q5_K
  if (2 * F * (H / 256) * 176 >= ((int64_t)1 << 31) || H * (F / 256) * 176 >= ((int64_t)1 << 31))
    return QDM_ERR_SHAPE;
  if (misaligned(x) || misaligned(w_gate_up) || misaligned(w_down) || misaligned(y))
    return QDM_ERR_ALIGN;
  const size_t need = qdm::moe_workspace(T, E, top_k, H, F);
  if (!workspace || workspace_bytes < need) return QDM_ERR_WORKSPACE;
  if (misaligned(workspace)) return QDM_ERR_ALIGN;
  return QDM_OK;
}

QDM_EXPORT int moe_q4k_grouped_gemm(const void *x, const void *w_gate_up, const void *w_down,
                                    const int32_t *topk_ids, const float *topk_w, float *y,
                                    int64_t T, int64_t E, int64_t top_k, int64_t H, int64_t F,
                                    void *workspace, size_t workspace_bytes, void *stream) {
  if (!topk_ids || !topk_w) return QDM_ERR_NULL;
  const int rc = check_moe(x, w_gate_up, w_down, y, T, E, top_k, H, F, workspace,
                           workspace_bytes);
  if (rc) return rc;
  qdm::launch_moe_q4k(x, w_gate_up, w_down, topk_ids, topk_w, y, T, E, top_k, H, F, workspace,
                      (hipStream_t)stream);
  return finish_launch();
}

QDM_EXPORT int moe_q4k_grouped_gemm_noalloc(const void *x, const void *w_gate_up,
                                            const void *w_down, const int32_t *topk_ids,
                                            const float *topk_w, float *y, int64_t T, int64_t E,
                                            int64_t top_k, int64_t H, int64_t F, void *stream) {
  if (!topk_ids || !topk_w) return QDM_ERR_NULL;
  // the argument checks of moe_q4k_grouped_gemm, with a stand-in for the
  // workspace (its size is checked against the scratch array just below)
  const int rc = check_moe(x, w_gate_up, w_down, y, T, E, top_k, H, F, (void *)x,
                           qdm::moe_workspace(T, E, top_k, H, F));
  if (rc) return rc;
  if (qdm::moe_workspace(T, E, top_k, H, F) > qdm::MOE_SCRATCH_BYTES) return QDM_ERR_SCRATCH;
  void *ptr = qdm::moe_scratch_ptr();
  if (!ptr) return QDM_ERR_HIP;
  qdm::launch_moe_q4k_scratch(x, w_gate_up, w_down, topk_ids, topk_w, y, T, E, top_k, H, F, ptr,
                              (hipStream_t)stream);
  return finish_launch();
}

QDM_EXPORT int moe_q4k_q5k_grouped_gemm(const void *x, const void *w_gate_up,
                                        const void *w_down, const int32_t *topk_ids,
                                        const float *topk_w, float *y, int64_t T, int64_t E,
                                        int64_t top_k, int64_t H, int64_t F, void *workspace,
                                        size_t workspace_bytes, void *stream) {
  if (!topk_ids || !topk_w) return QDM_ERR_NULL;
  const int rc = check_moe(x, w_gate_up, w_down, y, T, E, top_k, H, F, workspace,
                           workspace_bytes);
  if (rc) return rc;
  qdm::launch_moe_q4k_q5k(x, w_gate_up, w_down, topk_ids, topk_w, y, T, E, top_k, H, F,
                          workspace, (hipStream_t)stream);
  return finish_launch();
}

QDM_EXPORT int moe_router_topk(const float *logits, int64_t T, int64_t E, int64_t top_k,
                               int32_t *topk_ids, float *topk_w, void *stream) {
  if (!logits || !topk_ids || !topk_w) return QDM_ERR_NULL;
  if (T < 1 || T > (1 << 24) || E < 1 || E > 1024 || top_k < 1 || top_k > 16 || top_k > E)
    return QDM_ERR_SHAPE;
  if (misaligned4(logits) || misaligned4(topk_ids) || misaligned4(topk_w)) return QDM_ERR_ALIGN;
  qdm::launch_router_topk(logits, T, E, top_k, topk_ids, topk_w, (hipStream_t)stream);
  return finish_launch();
}

QDM_EXPORT size_t moe_from_logits_workspace_bytes(int64_t T, int64_t E, int64_t top_k, int64_t H,
                                                  int64_t F) {
  if (T < 1 || E < 1 || E > 1024 || top_k < 1 || top_k > 16 || top_k > E || bad_k(H) ||
      bad_k(F))
    return 0;
  return qdm::moe_logits_workspace(T, E, top_k, H, F);
}

QDM_EXPORT int moe_grouped_gemm_from_logits(const void *x, const float *router_logits,
                                            const void *w_gate_up, const void *w_down,
                                            int down_qtype, float *y, int64_t T, int64_t E,
                                            int64_t top_k, int64_t H, int64_t F,
                                            void *workspace, size_t workspace_bytes,
                                            void *stream) {
  if (!router_logits) return QDM_ERR_NULL;
  if (down_qtype != QDM_Q4_K && down_qtype != QDM_Q5_K) return QDM_ERR_DTYPE;
  // ids and gate weights are produced here, into the workspace
  const int rc = check_moe(x, w_gate_up, w_down, y, T, E, top_k, H, F, workspace,
                           workspace_bytes);
  if (rc) return rc;
  if (top_k > E) return QDM_ERR_SHAPE;
  if (misaligned4(router_logits)) return QDM_ERR_ALIGN;
  if (workspace_bytes < qdm::moe_logits_workspace(T, E, top_k, H, F)) return QDM_ERR_WORKSPACE;
  qdm::launch_moe_from_logits(x, router_logits, w_gate_up, w_down, down_qtype == QDM_Q5_K, y, T,
                              E, top_k, H, F, workspace, (hipStream_t)stream);
  return finish_launch();
}

QDM_EXPORT int qdm_probe_copy(const void *src, void *dst, int64_t n_bytes, void *stream) {
  if (!src || !dst) return QDM_ERR_NULL;
  if (n_bytes < 16 || n_bytes % 16) return QDM_ERR_SHAPE;
  if (misaligned(src) || misaligned(dst)) return QDM_ERR_ALIGN;
  qdm::launch_probe_copy(src, dst, n_bytes, (hipStream_t)stream);
  return finish_launch();
}

QDM_EXPORT int qdm_probe_read(const void *src, int64_t n_bytes, void *sink, void *stream) {
  if (!src || !sink) return QDM_ERR_NULL;
  if (n_bytes < 16 || n_bytes % 16) return QDM_ERR_SHAPE;
  if (misaligned(src) || misaligned4(sink)) return QDM_ERR_ALIGN;
  qdm::launch_probe_read(src, n_bytes, (uint32_t *)sink, (hipStream_t)stream);
  return finish_launch();
}

QDM_EXPORT int qdm_probe_mfma(int64_t iters, int64_t workgroups, float *sink, uint64_t *clocks,
                              void *stream) {
  if (!sink || !clocks) return QDM_ERR_NULL;
  if (iters < 1 || iters > (1 << 24) || workgroups < 1 || workgroups > (1 << 16))
    return QDM_ERR_SHAPE;
  if (misaligned4(sink) || ((uintptr_t)clocks & 7u)) return QDM_ERR_ALIGN;
  qdm::launch_probe_mfma(iters, workgroups, sink, clocks, (hipStream_t)stream);
  return finish_launch();
}

QDM_EXPORT int qdm_probe_empty(int64_t workgroups, void *stream) {
  if (workgroups < 1 || workgroups > (1 << 16)) return QDM_ERR_SHAPE;
  qdm::launch_probe_empty(workgroups, (hipStream_t)stream);
  return finish_launch();
}
