// Host-side launchers (internal to libqdm; the public ABI is include/qdm.h).
// Each launcher assumes validated arguments and only enqueues work.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace qdm {

void launch_q4k_dequantize(const void *w, float *out, int64_t N, int64_t K, hipStream_t s);
void launch_q5k_dequantize(const void *w, float *out, int64_t N, int64_t K, hipStream_t s);
void launch_q6k_dequantize(const void *w, float *out, int64_t N, int64_t K, hipStream_t s);
void launch_q80_dequantize(const void *w, float *out, int64_t N, int64_t K, hipStream_t s);

void launch_q4k_gemv(const void *w, const void *x, bool x_bf16, float *y, int64_t M,
                     int64_t N, int64_t K, hipStream_t s);
void launch_q5k_gemv(const void *w, const void *x, bool x_bf16, float *y, int64_t M,
                     int64_t N, int64_t K, hipStream_t s);
void launch_q6k_gemv(const void *w, const void *x, bool x_bf16, float *y, int64_t M,
                     int64_t N, int64_t K, hipStream_t s);
// Q4_K (or Q5_K when q5) GEMV on the matrix cores, bf16 x, any M >= 1.
void launch_q4k_mfma_gemv(const void *w, const uint16_t *x, float *y, int64_t M, int64_t N,
                          int64_t K, bool q5, hipStream_t s);
// Q8_0 GEMV on the matrix cores, bf16 x, any M >= 1 (K % 256 == 0).
void launch_q80_mfma_gemv(const void *w, const uint16_t *x, float *y, int64_t M, int64_t N,
                          int64_t K, hipStream_t s);
bool q80_gemv_fits(int64_t N, int64_t K);
void launch_q80_gemv(const void *w, const void *x, bool x_bf16, float *y, int64_t M,
                     int64_t N, int64_t K, hipStream_t s);

size_t q4k_gemm_workspace(int64_t M, int64_t N, int64_t K);
void set_gemm_spin_limit(uint32_t limit);
void launch_q4k_gemm(const void *w, const void *x, float *y, int64_t M, int64_t N, int64_t K,
                     void *workspace, hipStream_t s);

size_t moe_workspace(int64_t T, int64_t E, int64_t top_k, int64_t H, int64_t F);
// Bytes of the static scratch array behind moe_q4k_grouped_gemm_noalloc.
constexpr size_t MOE_SCRATCH_BYTES = (size_t)16 << 20;
// The current device's copy of that array (looked up once per device), or
// nullptr if the runtime could not provide it.
void *moe_scratch_ptr();
void launch_moe_q4k_scratch(const void *x, const void *w13, const void *w2, const int32_t *ids,
                            const float *gw, float *y, int64_t T, int64_t E, int64_t top_k,
                            int64_t H, int64_t F, void *scratch_ptr, hipStream_t s);
void launch_moe_q4k(const void *x, const void *w13, const void *w2, const int32_t *ids,
                    const float *gw, float *y, int64_t T, int64_t E, int64_t top_k, int64_t H,
                    int64_t F, void *workspace, hipStream_t s);
void launch_moe_q4k_q5k(const void *x, const void *w13, const void *w2, const int32_t *ids,
                        const float *gw, float *y, int64_t T, int64_t E, int64_t top_k,
                        int64_t H, int64_t F, void *workspace, hipStream_t s);

void launch_router_topk(const float *logits, int64_t T, int64_t E, int64_t k, int32_t *ids,
                        float *gw, hipStream_t s);
size_t moe_logits_workspace(int64_t T, int64_t E, int64_t top_k, int64_t H, int64_t F);
void launch_moe_from_logits(const void *x, const float *logits, const void *w13, const void *w2,
                            bool down_q5, float *y, int64_t T, int64_t E, int64_t top_k,
                            int64_t H, int64_t F, void *workspace, hipStream_t s);

void launch_probe_copy(const void *src, void *dst, int64_t n_bytes, hipStream_t s);
void launch_probe_read(const void *src, int64_t n_bytes, uint32_t *sink, hipStream_t s);
void launch_probe_mfma(int64_t iters, int64_t workgroups, float *sink, uint64_t *clocks,
                       hipStream_t s);
void launch_probe_empty(int64_t workgroups, hipStream_t s);

}  // namespace qdm
