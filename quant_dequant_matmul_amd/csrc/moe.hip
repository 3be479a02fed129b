// Routed MoE FFN with Q4_K experts, one call per layer (expert-grouped
// matmul; hipster README, "Verify the claims": MoE grouped GEMM).
//
//   y_t = sum_s gw[t][s] * W2[e] * (silu(W13[e][0:F] x_t) * W13[e][F:2F] x_t),
//   e = ids[t][s].
//
// Pipeline (all on one stream, no host round trip):
//  1. route: histogram of the ids over experts, exclusive scan, then a stable
//     scatter of the (token, slot) entries into expert order (ties keep
//     (t, s) order), plus the compact list of experts that received entries.
//  2. gate+up: for each active expert, every W13 row is streamed once and
//     multiplied with all the gathered tokens of that expert -> U [8T][2F].
//  3. SwiGLU: h = silu(U[:, :F]) * U[:, F:] (fp32).
//  4. down: for each active expert, W2 rows times its h rows -> O [8T][H].
//  5. combine: y_t = sum over s in slot order of gw[t][s] * O[pos(t, s)];
//     deterministic, no atomics.
#include "common.h"
#include "launch.h"

namespace qdm {

namespace {

constexpr int ROUTE_THREADS = 1024;
constexpr int MOE_GEMV_THREADS = 256;
constexpr int MOE_WAVES = MOE_GEMV_THREADS / WAVE;
constexpr int MOE_MT = 4;  // tokens per pass in the gathered GEMV

inline size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

struct MoeWs {
  int32_t *counts;   // [E]
  int32_t *offsets;  // [E+1]
  int32_t *active;   // [E] compact list of experts with entries
  int32_t *meta;     // [0] = number of active experts, [1] = skipped (bad) ids
  int32_t *perm;     // [n] sorted position -> entry (t*top_k + s)
  int32_t *pos;      // [n] entry -> sorted position, -1 if skipped
  float *u;          // [n][2F]
  float *h;          // [n][F]
  float *o;          // [n][H]
  size_t total;
};

MoeWs carve(void *base, int64_t T, int64_t E, int64_t top_k, int64_t H, int64_t F) {
  const int64_t n = T * top_k;
  MoeWs ws;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off += align256(bytes);
    return o;
  };
  const size_t o_counts = take(sizeof(int32_t) * E);
  const size_t o_offsets = take(sizeof(int32_t) * (E + 1));
  const size_t o_active = take(sizeof(int32_t) * E);
  const size_t o_meta = take(sizeof(int32_t) * 4);
  const size_t o_perm = take(sizeof(int32_t) * n);
  const size_t o_pos = take(sizeof(int32_t) * n);
  const size_t o_u = take(sizeof(float) * n * 2 * F);
  const size_t o_h = take(sizeof(float) * n * F);
  const size_t o_o = take(sizeof(float) * n * H);
  char *b = (char *)base;
  ws.counts = (int32_t *)(b + o_counts);
  ws.offsets = (int32_t *)(b + o_offsets);
  ws.active = (int32_t *)(b + o_active);
  ws.meta = (int32_t *)(b + o_meta);
  ws.perm = (int32_t *)(b + o_perm);
  ws.pos = (int32_t *)(b + o_pos);
  ws.u = (float *)(b + o_u);
  ws.h = (float *)(b + o_h);
  ws.o = (float *)(b + o_o);
  ws.total = off;
  return ws;
}

// Single workgroup: counts, scan, active list and the stable scatter.
__global__ __launch_bounds__(ROUTE_THREADS) void moe_route_kernel(
    const int32_t *__restrict__ ids, int n, int E, int32_t *__restrict__ counts,
    int32_t *__restrict__ offsets, int32_t *__restrict__ active, int32_t *__restrict__ meta,
    int32_t *__restrict__ perm, int32_t *__restrict__ pos) {
  extern __shared__ int32_t sm[];
  int32_t *cnt = sm;          // [E]
  int32_t *run = sm + E;      // [E] running write position
  __shared__ int32_t bad;
  const int tid = threadIdx.x;
  for (int e = tid; e < E; e += ROUTE_THREADS) cnt[e] = 0;
  if (tid == 0) bad = 0;
  __syncthreads();
  for (int i = tid; i < n; i += ROUTE_THREADS) {
    const int e = ids[i];
    if (e >= 0 && e < E)
      atomicAdd(&cnt[e], 1);
    else
      atomicAdd(&bad, 1);
  }
  __syncthreads();
  if (tid == 0) {
    int acc = 0, na = 0;
    for (int e = 0; e < E; e++) {
      const int c = cnt[e];
      offsets[e] = acc;
      run[e] = acc;
      counts[e] = c;
      if (c > 0) active[na++] = e;
      acc += c;
    }
    offsets[E] = acc;
    meta[0] = na;
    meta[1] = bad;
  }
  __syncthreads();
  // Stable scatter by wave 0: 64 entries at a time, in entry order. Within a
  // batch, lanes with the same expert are ranked by lane index via ballots.
  if (tid < WAVE) {
    const int lane = tid;
    const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int base = 0; base < n; base += WAVE) {
      const int i = base + lane;
      int e = i < n ? ids[i] : -1;
      const bool valid = i < n && e >= 0 && e < E;
      if (i < n && !valid) pos[i] = -1;
      bool pending = valid;
      while (__ballot(pending) != 0ull) {
        const uint64_t pmask = __ballot(pending);
        const int leader = __builtin_ctzll(pmask);
        const int ev = __shfl(e, leader, WAVE);
        const bool mine = pending && e == ev;
        const uint64_t mmask = __ballot(mine);
        const int start = run[ev];
        if (mine) {
          const int p = start + __popcll(mmask & lt);
          pos[i] = p;
          perm[p] = i;
          pending = false;
        }
        if (lane == leader) run[ev] = start + __popcll(mmask);
      }
    }
  }
}

// Gathered Q4_K GEMV over the rows of one expert: for the a-th active expert
// e and the sorted entries p in [offsets[e], offsets[e+1]):
//   out[p][r] = sum_k xrow(p)[k] * W_e(r, k)
// xrow(p) = x[perm[p] / top_k] (bf16, gate+up) or x[p] (fp32, down).
// Lane mapping as in the dense GEMV: 4 lanes per block, G groups per row.
template <bool XBF16>
__global__ __launch_bounds__(MOE_GEMV_THREADS) void moe_gemv_kernel(
    const uint8_t *__restrict__ wbase, int64_t expert_stride, int Nr, int K,
    const void *__restrict__ x, const int32_t *__restrict__ perm, int top_k,
    const int32_t *__restrict__ offsets, const int32_t *__restrict__ active,
    const int32_t *__restrict__ meta, float *__restrict__ out, int G) {
  const int a = blockIdx.y;
  if (a >= meta[0]) return;
  const int e = active[a];
  const int p_begin = offsets[e], p_end = offsets[e + 1];
  const uint8_t *w = wbase + (int64_t)e * expert_stride;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 2, c = lane & 3;
  const int R = 16 / G;
  const int row = (blockIdx.x * MOE_WAVES + wave) * R + g / G;
  const int gg = g % G;
  const int nb = K / QK;
  const int iters = nb / G;
  const bool active_row = row < Nr;
  const uint8_t *rowp = w + (int64_t)(active_row ? row : 0) * nb * Q4K_BYTES;
  const int j0 = 2 * c;

  for (int p0 = p_begin; p0 < p_end; p0 += MOE_MT) {
    float acc[MOE_MT];
    int64_t xoff[MOE_MT];
#pragma unroll
    for (int m = 0; m < MOE_MT; m++) {
      acc[m] = 0.f;
      const int p = p0 + m < p_end ? p0 + m : p_end - 1;
      xoff[m] = XBF16 ? (int64_t)(perm[p] / top_k) * K : (int64_t)p * K;
    }
    if (active_row) {
      for (int it = 0; it < iters; it++) {
        const int kb = it * G + gg;
        const uint8_t *blk = rowp + (int64_t)kb * Q4K_BYTES;
        const u32x4 hdr = *(const u32x4 *)blk;
        const u32x4 qa = *(const u32x4 *)(blk + 16 + 32 * c);
        const u32x4 qb = *(const u32x4 *)(blk + 32 + 32 * c);
        const uint32_t q[8] = {qa.x, qa.y, qa.z, qa.w, qb.x, qb.y, qb.z, qb.w};
        const float d = half_bits_to_float(hdr.x), dmin = half_bits_to_float(hdr.x >> 16);
        uint32_t sc0, m0, sc1, m1;
        q4k_scale_min(hdr.y, hdr.z, hdr.w, j0, sc0, m0);
        q4k_scale_min(hdr.y, hdr.z, hdr.w, j0 + 1, sc1, m1);
        const float a0 = d * (float)sc0, b0 = dmin * (float)m0;
        const float a1 = d * (float)sc1, b1 = dmin * (float)m1;
        const int k0 = kb * QK + 32 * j0;
#pragma unroll
        for (int m = 0; m < MOE_MT; m++) {
          float s0 = 0.f, s1 = 0.f, x0s = 0.f, x1s = 0.f;
#pragma unroll
          for (int i = 0; i < 8; i++) {
            float xa[4], xb[4];
            if constexpr (XBF16) {
              const u32x2 va = *(const u32x2 *)((const uint16_t *)x + xoff[m] + k0 + 4 * i);
              const u32x2 vb = *(const u32x2 *)((const uint16_t *)x + xoff[m] + k0 + 32 + 4 * i);
              xa[0] = bf16_bits_to_float(va.x); xa[1] = bf16_bits_to_float(va.x >> 16);
              xa[2] = bf16_bits_to_float(va.y); xa[3] = bf16_bits_to_float(va.y >> 16);
              xb[0] = bf16_bits_to_float(vb.x); xb[1] = bf16_bits_to_float(vb.x >> 16);
              xb[2] = bf16_bits_to_float(vb.y); xb[3] = bf16_bits_to_float(vb.y >> 16);
            } else {
              const f32x4 va = *(const f32x4 *)((const float *)x + xoff[m] + k0 + 4 * i);
              const f32x4 vb = *(const f32x4 *)((const float *)x + xoff[m] + k0 + 32 + 4 * i);
              xa[0] = va.x; xa[1] = va.y; xa[2] = va.z; xa[3] = va.w;
              xb[0] = vb.x; xb[1] = vb.y; xb[2] = vb.z; xb[3] = vb.w;
            }
#pragma unroll
            for (int t = 0; t < 4; t++) {
              s0 = fmaf(xa[t], (float)((q[i] >> (8 * t)) & 15u), s0);
              s1 = fmaf(xb[t], (float)((q[i] >> (8 * t + 4)) & 15u), s1);
              x0s += xa[t];
              x1s += xb[t];
            }
          }
          acc[m] += a0 * s0 - b0 * x0s + a1 * s1 - b1 * x1s;
        }
      }
    }
#pragma unroll
    for (int m = 0; m < MOE_MT; m++) {
      const float v = group_sum(acc[m], 4 * G);
      if (active_row && p0 + m < p_end && (lane & (4 * G - 1)) == 0)
        out[(int64_t)(p0 + m) * Nr + row] = v;
    }
  }
}

__global__ void moe_swiglu_kernel(const float *__restrict__ u, float *__restrict__ h,
                                  const int32_t *__restrict__ offsets, int E, int F) {
  const int64_t n = offsets[E];
  const int64_t total = n * F;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t p = i / F, f = i % F;
    const float gt = u[p * 2 * F + f], up = u[p * 2 * F + F + f];
    h[i] = gt / (1.0f + __expf(-gt)) * up;
  }
}

__global__ void moe_combine_kernel(const float *__restrict__ o, const int32_t *__restrict__ pos,
                                   const float *__restrict__ gw, float *__restrict__ y, int T,
                                   int top_k, int H) {
  const int64_t total = (int64_t)T * H;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t t = i / H, r = i % H;
    float acc = 0.f;
    for (int s = 0; s < top_k; s++) {
      const int p = pos[t * top_k + s];
      if (p >= 0) acc = fmaf(gw[t * top_k + s], o[(int64_t)p * H + r], acc);
    }
    y[i] = acc;
  }
}

int gcd16(int nb) {
  int g = 16;
  while (g > 1 && nb % g) g >>= 1;
  return g;
}

}  // namespace

size_t moe_workspace(int64_t T, int64_t E, int64_t top_k, int64_t H, int64_t F) {
  return carve(nullptr, T, E, top_k, H, F).total;
}

void launch_moe_q4k(const void *x, const void *w13, const void *w2, const int32_t *ids,
                    const float *gw, float *y, int64_t T, int64_t E, int64_t top_k, int64_t H,
                    int64_t F, void *workspace, hipStream_t s) {
  const MoeWs ws = carve(workspace, T, E, top_k, H, F);
  const int n = (int)(T * top_k);
  const size_t route_lds = sizeof(int32_t) * 2 * E;
  hipLaunchKernelGGL(moe_route_kernel, dim3(1), dim3(ROUTE_THREADS), route_lds, s, ids, n,
                     (int)E, ws.counts, ws.offsets, ws.active, ws.meta, ws.perm, ws.pos);
  const int e_cap = (int)(E < n ? E : n);

  // gate+up: rows 2F, K = H
  {
    const int nb = (int)(H / QK), G = gcd16(nb), R = 16 / G;
    const int rows_wg = MOE_WAVES * R;
    const dim3 grid((unsigned)((2 * F + rows_wg - 1) / rows_wg), (unsigned)e_cap);
    hipLaunchKernelGGL(moe_gemv_kernel<true>, grid, dim3(MOE_GEMV_THREADS), 0, s,
                       (const uint8_t *)w13, (int64_t)2 * F * nb * Q4K_BYTES, (int)(2 * F),
                       (int)H, x, ws.perm, (int)top_k, ws.offsets, ws.active, ws.meta, ws.u, G);
  }
  hipLaunchKernelGGL(moe_swiglu_kernel, dim3(1024), dim3(256), 0, s, ws.u, ws.h, ws.offsets,
                     (int)E, (int)F);
  // down: rows H, K = F
  {
    const int nb = (int)(F / QK), G = gcd16(nb), R = 16 / G;
    const int rows_wg = MOE_WAVES * R;
    const dim3 grid((unsigned)((H + rows_wg - 1) / rows_wg), (unsigned)e_cap);
    hipLaunchKernelGGL(moe_gemv_kernel<false>, grid, dim3(MOE_GEMV_THREADS), 0, s,
                       (const uint8_t *)w2, (int64_t)H * nb * Q4K_BYTES, (int)H, (int)F, ws.h,
                       ws.perm, (int)top_k, ws.offsets, ws.active, ws.meta, ws.o, G);
  }
  hipLaunchKernelGGL(moe_combine_kernel, dim3(1024), dim3(256), 0, s, ws.o, ws.pos, gw, y,
                     (int)T, (int)top_k, (int)H);
}

}  // namespace qdm
