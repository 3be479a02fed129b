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

// ---------------------------------------------------------------------------
// Decode regime (n = T * top_k <= 64 entries).
// ---------------------------------------------------------------------------
constexpr int DEC_THREADS = 256;
constexpr int DEC_WAVES = DEC_THREADS / WAVE;
constexpr int DEC_MAX_N = 64;
#ifndef QDM_DEC_PF
#define QDM_DEC_PF 3
#endif
#ifndef QDM_DEC_FR
#define QDM_DEC_FR 16
#endif
#ifndef QDM_DEC_RW
#define QDM_DEC_RW 64
#endif
constexpr int DEC_PF = QDM_DEC_PF;  // wave iterations of weight loads in flight
constexpr int DEC_FR = QDM_DEC_FR;  // gate/up row pairs per gate+up workgroup
constexpr int DEC_RW = QDM_DEC_RW;  // W2 rows per down workgroup

// A value the compiler cannot see through (keeps v_and_or_b32 forms).
__device__ __forceinline__ uint32_t opaque_u32(uint32_t v) {
  asm volatile("" : "+v"(v));
  return v;
}

// Routing of at most 64 entries, derived by every workgroup from the ids:
// the number of distinct valid experts, the a-th of them in increasing id
// order (-1 past the end) and its entries in increasing (t, s) order.
struct SmallRoute {
  int nact, e, cnt;
  int ent[DEC_MAX_N];
};

__device__ void small_route(const int32_t *__restrict__ ids, int n, int E, int a, SmallRoute &sr,
                            uint32_t *bitmap) {
  const int tid = threadIdx.x;
  if (tid < 32) bitmap[tid] = 0u;  // E <= 1024 experts: 32 words
  __syncthreads();
  int myid = -1;
  if (tid < WAVE) {
    if (tid < n) myid = ids[tid];
    if (myid >= 0 && myid < E) atomicOr(&bitmap[myid >> 5], 1u << (myid & 31));
  }
  __syncthreads();
  if (tid < WAVE) {
    const uint32_t word = tid < 32 ? bitmap[tid] : 0u;
    const int c = __popc(word);
    int incl = c;  // inclusive prefix of set bits over words
#pragma unroll
    for (int o = 1; o < 32; o <<= 1) {
      const int v = __shfl_up(incl, o, WAVE);
      if (tid >= o) incl += v;
    }
    const int total = __shfl(incl, 31, WAVE);
    const int excl = incl - c;
    const uint64_t hm = __ballot(tid < 32 && a >= excl && a < incl);
    int e = -1;
    if (hm != 0ull) {
      const int L = __builtin_ctzll(hm);
      uint32_t wl = (uint32_t)__shfl((int)word, L, WAVE);
      const int r = a - __shfl(excl, L, WAVE);
      for (int i = 0; i < r; i++) wl &= wl - 1u;  // drop the r lowest set bits
      e = 32 * L + __builtin_ctz(wl);
    }
    const bool mine = e >= 0 && tid < n && myid == e;
    const uint64_t mm = __ballot(mine);
    if (mine) sr.ent[__popcll(mm & ((1ull << tid) - 1ull))] = tid;
    if (tid == 0) {
      sr.nact = total;
      sr.e = e;
      sr.cnt = __popcll(mm);
    }
  }
  __syncthreads();
}

// Stages mt input rows of length K into LDS: bf16 rows as (x0, x2, x1, x3)
// groups (to match the code pairs of the dot below) or fp32 rows as they are,
// plus every row's 32-element sums. Row m is src_row(m). Every 64-element
// piece (what one lane reads for its code chunk) is padded by 16 bytes, so
// the 16 (column block, chunk) pieces a wave reads at once start on 16
// different LDS bank groups.
constexpr int PIECE_BF16 = 128 + 16, REC_BF16 = 4 * PIECE_BF16;  // bytes per 64 / 256 bf16
constexpr int PIECE_F32 = 256 + 16, REC_F32 = 4 * PIECE_F32;     // bytes per 64 / 256 fp32

template <bool XBF16, typename SrcRow>
__device__ __forceinline__ void stage_rows(SrcRow src_row, int mt, int K, uint8_t *lds_in,
                                           float *lds_sum) {
  constexpr int PER_CHUNK = XBF16 ? 8 : 4;   // elements per 16-byte chunk
  constexpr int CH_PER_SUM = 32 / PER_CHUNK;
  constexpr int CH_PER_PIECE = 64 / PER_CHUNK;
  constexpr int PIECE = XBF16 ? PIECE_BF16 : PIECE_F32;
  const int rchunks = K / PER_CHUNK;
  const int nchunk = mt * rchunks;
  const int rowb = (K / 64) * PIECE;
  for (int base = 0; base < nchunk; base += DEC_THREADS) {
    const int cidx = base + threadIdx.x;
    float s = 0.f;
    if (cidx < nchunk) {
      const int m = cidx / rchunks, cc = cidx - m * rchunks;
      const u32x4 v = ((const u32x4 *)src_row(m))[cc];
      uint8_t *dst = lds_in + m * rowb + (cc / CH_PER_PIECE) * PIECE + (cc % CH_PER_PIECE) * 16;
      if constexpr (XBF16) {
        u32x4 p;
        p.x = (v.x & 0xFFFFu) | (v.y << 16);
        p.y = (v.x >> 16) | (v.y & 0xFFFF0000u);
        p.z = (v.z & 0xFFFFu) | (v.w << 16);
        p.w = (v.z >> 16) | (v.w & 0xFFFF0000u);
        *(u32x4 *)dst = p;
        s = bf16_bits_to_float(v.x) + bf16_bits_to_float(v.x >> 16) +
            bf16_bits_to_float(v.y) + bf16_bits_to_float(v.y >> 16) +
            bf16_bits_to_float(v.z) + bf16_bits_to_float(v.z >> 16) +
            bf16_bits_to_float(v.w) + bf16_bits_to_float(v.w >> 16);
      } else {
        *(u32x4 *)dst = v;
        const f32x4 f = __builtin_bit_cast(f32x4, v);
        s = (f.x + f.y) + (f.z + f.w);
      }
    }
#pragma unroll
    for (int o = 1; o < CH_PER_SUM; o <<= 1) s += __shfl_xor(s, o, WAVE);
    if (cidx < nchunk && (cidx % CH_PER_SUM) == 0) lds_sum[cidx / CH_PER_SUM] = s;
  }
}

// part[m][b] = sum over block b's 256 weights of w * in_m, for the nblk blocks
// blk_ptr(0 .. nblk-1) (block b covers input columns (b % nb) * 256 ..) and
// the mt staged rows. 4 lanes per block (lane c owns code chunk c, sub-blocks
// 2c and 2c+1), 16 blocks per wave iteration, DEC_PF iterations of loads in
// flight; loads are unconditional (clamped) so waits are exact. prefetch()
// issues the first loads (before the inputs are staged), run() the rest.
template <bool XBF16, int MT, typename BlkPtr>
struct RowsDot {
  BlkPtr blk_ptr;
  int nblk, wb0, wb1, iters, g, c;
  u32x4 Hd[DEC_PF], A[DEC_PF], Bq[DEC_PF];

  __device__ __forceinline__ RowsDot(BlkPtr bp, int nblk_) : blk_ptr(bp), nblk(nblk_) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    g = lane >> 2;
    c = lane & 3;
    wb0 = wave * nblk / DEC_WAVES;
    wb1 = (wave + 1) * nblk / DEC_WAVES;
    iters = (wb1 - wb0 + 15) >> 4;
  }

  __device__ __forceinline__ void load(int slot, int it) {
    const uint8_t *blk = blk_ptr(min(wb0 + g + 16 * it, wb1 - 1));
    Hd[slot] = *(const u32x4 *)blk;
    A[slot] = *(const u32x4 *)(blk + 16 + 32 * c);
    Bq[slot] = *(const u32x4 *)(blk + 32 + 32 * c);
  }

  __device__ __forceinline__ void prefetch() {
    if (iters == 0) return;
#pragma unroll
    for (int p = 0; p < DEC_PF; p++) load(p, min(p, iters - 1));
  }

  __device__ __forceinline__ void run(int nb, int K, int mt, const uint8_t *lds_in,
                                      const float *lds_sum, float *part) {
    constexpr int REC = XBF16 ? REC_BF16 : REC_F32;
    constexpr int PIECE = XBF16 ? PIECE_BF16 : PIECE_F32;
    if (iters == 0) return;
    const uint32_t MASK = opaque_u32(0x000F000Fu), MAGIC = opaque_u32(0x43004300u);
    for (int it0 = 0; it0 < iters; it0 += DEC_PF) {
#pragma unroll
      for (int p = 0; p < DEC_PF; p++) {
        const int it = it0 + p;
        if (it < iters) {
          const int b = wb0 + g + 16 * it;
          const bool valid = b < wb1;
          const u32x4 hdr = Hd[p];
          const uint32_t q[8] = {A[p].x, A[p].y, A[p].z, A[p].w,
                                 Bq[p].x, Bq[p].y, Bq[p].z, Bq[p].w};
          load(p, min(it + DEC_PF, iters - 1));  // refill the slot right away
          const float d = half_bits_to_float(hdr.x), dmin = half_bits_to_float(hdr.x >> 16);
          uint32_t sc0, m0, sc1, m1;
          q4k_scale_min(hdr.y, hdr.z, hdr.w, 2 * c, sc0, m0);
          q4k_scale_min(hdr.y, hdr.z, hdr.w, 2 * c + 1, sc1, m1);
          const float a0 = d * (float)sc0, b0 = dmin * (float)m0;
          const float a1 = d * (float)sc1, b1 = dmin * (float)m1;
          const int kb = b % nb;
          const int e0 = kb * QK + 64 * c;  // first input column of sub-block 2c
#pragma unroll
          for (int m = 0; m < MT; m++) {
            if (m < mt) {
              const float2 xs = *(const float2 *)(lds_sum + m * (K / 32) + (e0 >> 5));
              float s0 = 0.f, s1 = 0.f, r;
              if constexpr (XBF16) {
                const u32x4 *xv = (const u32x4 *)(lds_in + (m * nb + kb) * REC + PIECE * c);
#pragma unroll
                for (int i = 0; i < 4; i++) {
                  const u32x4 x0 = xv[i], x1 = xv[4 + i];
                  const uint32_t qa = q[2 * i], qb = q[2 * i + 1];
                  const uint32_t qa4 = qa >> 4, qb4 = qb >> 4;
                  s0 = dot2_bf16((qa & MASK) | MAGIC, x0.x, s0);
                  s0 = dot2_bf16(((qa >> 8) & MASK) | MAGIC, x0.y, s0);
                  s0 = dot2_bf16((qb & MASK) | MAGIC, x0.z, s0);
                  s0 = dot2_bf16(((qb >> 8) & MASK) | MAGIC, x0.w, s0);
                  s1 = dot2_bf16((qa4 & MASK) | MAGIC, x1.x, s1);
                  s1 = dot2_bf16(((qa4 >> 8) & MASK) | MAGIC, x1.y, s1);
                  s1 = dot2_bf16((qb4 & MASK) | MAGIC, x1.z, s1);
                  s1 = dot2_bf16(((qb4 >> 8) & MASK) | MAGIC, x1.w, s1);
                }
                r = a0 * s0;
                r = fmaf(-fmaf(128.f, a0, b0), xs.x, r);
                r = fmaf(a1, s1, r);
                r = fmaf(-fmaf(128.f, a1, b1), xs.y, r);
              } else {
                const f32x4 *xv = (const f32x4 *)(lds_in + (m * nb + kb) * REC + PIECE * c);
#pragma unroll
                for (int i = 0; i < 8; i++) {
                  const f32x4 x0 = xv[i], x1 = xv[8 + i];
                  const uint32_t lo = q[i] & 0x0F0F0F0Fu, hi = (q[i] >> 4) & 0x0F0F0F0Fu;
                  s0 = fmaf(x0.x, (float)(lo & 255u), s0);
                  s0 = fmaf(x0.y, (float)((lo >> 8) & 255u), s0);
                  s0 = fmaf(x0.z, (float)((lo >> 16) & 255u), s0);
                  s0 = fmaf(x0.w, (float)(lo >> 24), s0);
                  s1 = fmaf(x1.x, (float)(hi & 255u), s1);
                  s1 = fmaf(x1.y, (float)((hi >> 8) & 255u), s1);
                  s1 = fmaf(x1.z, (float)((hi >> 16) & 255u), s1);
                  s1 = fmaf(x1.w, (float)(hi >> 24), s1);
                }
                r = a0 * s0;
                r = fmaf(-b0, xs.x, r);
                r = fmaf(a1, s1, r);
                r = fmaf(-b1, xs.y, r);
              }
              r += __shfl_xor(r, 1, WAVE);
              r += __shfl_xor(r, 2, WAVE);
              if (valid && c == 0) part[m * nblk + b] = r;
            }
          }
        }
      }
    }
  }
};

template <bool XBF16, int MT, typename BlkPtr>
__device__ __forceinline__ RowsDot<XBF16, MT, BlkPtr> make_rows_dot(BlkPtr bp, int nblk) {
  return RowsDot<XBF16, MT, BlkPtr>(bp, nblk);
}

// Decode gate+up+SwiGLU: workgroup (f chunk, a) with e = the a-th active
// expert; rows f0 .. f0+fr-1 (gate) and F+f0 .. (up) of W13[e], all entries
// of e; h[entry][f] = silu(g) * u (fp32).
template <int MT>
__global__ __launch_bounds__(DEC_THREADS) void moe_dec_gateup_kernel(
    const uint16_t *__restrict__ x, const uint8_t *__restrict__ w13,
    const int32_t *__restrict__ ids, int n, int top_k, int E, int H, int F,
    float *__restrict__ h) {
  extern __shared__ __attribute__((aligned(16))) uint32_t lds[];
  __shared__ SmallRoute sr;
  __shared__ uint32_t bitmap[32];
  small_route(ids, n, E, blockIdx.y, sr, bitmap);
  if (sr.e < 0) return;
  const int e = sr.e, cnt = sr.cnt;
  const int nb = H / QK;
  const int f0 = blockIdx.x * DEC_FR, fr = min(DEC_FR, F - f0);
  const int nrows = 2 * fr, nblk = nrows * nb;
  uint8_t *lds_in = (uint8_t *)lds;                       // [MT][nb][REC_BF16]
  float *lds_sum = (float *)(lds_in + MT * nb * REC_BF16);  // [MT][H / 32]
  float *part = lds_sum + MT * (H / 32);                  // [MT][2 DEC_FR nb]
  float *res = part + MT * 2 * DEC_FR * nb;               // [MT][2 DEC_FR]
  const uint8_t *we = w13 + (int64_t)e * 2 * F * nb * Q4K_BYTES;
  auto blk_ptr = [&](int b) {  // gate rows first, then the matching up rows
    const int r = b / nb;
    const int row = r < fr ? f0 + r : F + f0 + (r - fr);
    return we + ((int64_t)row * nb + (b - r * nb)) * Q4K_BYTES;
  };
  auto rd = make_rows_dot<true, MT>(blk_ptr, nblk);
  for (int c0 = 0; c0 < cnt; c0 += MT) {
    const int mt = min(MT, cnt - c0);
    rd.prefetch();  // weight loads fly while the x rows are staged
    stage_rows<true>([&](int m) { return x + (int64_t)(sr.ent[c0 + m] / top_k) * H; }, mt, H,
                     lds_in, lds_sum);
    __syncthreads();
    rd.run(nb, H, mt, lds_in, lds_sum, part);
    __syncthreads();
    for (int t = threadIdx.x; t < mt * nrows; t += DEC_THREADS) {  // rows in block order
      const int m = t / nrows, r = t - m * nrows;
      const float *pp = part + m * nblk + r * nb;
      float sacc = 0.f;
      for (int k = 0; k < nb; k++) sacc += pp[k];
      res[m * nrows + r] = sacc;
    }
    __syncthreads();
    for (int t = threadIdx.x; t < mt * fr; t += DEC_THREADS) {
      const int m = t / fr, f = t - m * fr;
      const float gt = res[m * nrows + f], up = res[m * nrows + fr + f];
      h[(int64_t)sr.ent[c0 + m] * F + f0 + f] = gt / (1.0f + expf(-gt)) * up;
    }
    __syncthreads();
  }
}

// Decode down: workgroup (row chunk, a): o[entry][r] for rows r0 .. r0+rw-1
// of W2[e] and every entry of e (fp32).
template <int MT>
__global__ __launch_bounds__(DEC_THREADS) void moe_dec_down_kernel(
    const float *__restrict__ h, const uint8_t *__restrict__ w2, const int32_t *__restrict__ ids,
    float *__restrict__ o, int n, int top_k, int E, int H, int F) {
  extern __shared__ __attribute__((aligned(16))) uint32_t lds[];
  __shared__ SmallRoute sr;
  __shared__ uint32_t bitmap[32];
  small_route(ids, n, E, blockIdx.y, sr, bitmap);
  const int r0 = blockIdx.x * DEC_RW, rw = min(DEC_RW, H - r0);
  if (sr.e < 0) return;
  const int e = sr.e, cnt = sr.cnt;
  const int nb = F / QK, nblk = rw * nb;
  uint8_t *lds_in = (uint8_t *)lds;                       // [MT][nb][REC_F32]
  float *lds_sum = (float *)(lds_in + MT * nb * REC_F32);  // [MT][F / 32]
  float *part = lds_sum + MT * (F / 32);           // [MT][DEC_RW nb]
  const uint8_t *rows = w2 + ((int64_t)e * H + r0) * nb * Q4K_BYTES;
  auto blk_ptr = [&](int b) { return rows + (int64_t)b * Q4K_BYTES; };
  auto rd = make_rows_dot<false, MT>(blk_ptr, nblk);
  for (int c0 = 0; c0 < cnt; c0 += MT) {
    const int mt = min(MT, cnt - c0);
    rd.prefetch();  // weight loads fly while the h rows are staged
    stage_rows<false>([&](int m) { return h + (int64_t)sr.ent[c0 + m] * F; }, mt, F, lds_in,
                      lds_sum);
    __syncthreads();
    rd.run(nb, F, mt, lds_in, lds_sum, part);
    __syncthreads();
    for (int t = threadIdx.x; t < mt * rw; t += DEC_THREADS) {
      const int m = t / rw, r = t - m * rw;
      const float *pp = part + m * nblk + r * nb;
      float sacc = 0.f;
      for (int k = 0; k < nb; k++) sacc += pp[k];
      o[(int64_t)sr.ent[c0 + m] * H + r0 + r] = sacc;
    }
    __syncthreads();
  }
}

// y[t][r] = sum over slots s in order of gw[t][s] * o[t*top_k+s][r], slots
// with an id outside [0, E) skipped (o is indexed by entry).
__global__ void moe_combine_entries_kernel(const float *__restrict__ o,
                                           const int32_t *__restrict__ ids,
                                           const float *__restrict__ gw, float *__restrict__ y,
                                           int T, int top_k, int E, int H) {
  const int64_t total = (int64_t)T * H;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t t = i / H, r = i - t * H;
    float acc = 0.f;
    for (int s = 0; s < top_k; s++) {
      const int64_t en = t * top_k + s;
      const int id = ids[en];
      if (id >= 0 && id < E) acc = fmaf(gw[en], o[en * H + r], acc);
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

// Workspace: h [n][F] and o [n][H] (fp32, by entry) of the decode regime,
// then the regions of the matrix-core regime.
size_t moe_workspace(int64_t T, int64_t E, int64_t top_k, int64_t H, int64_t F) {
  const int64_t n = T * top_k;
  return align256(sizeof(float) * n * F) + align256(sizeof(float) * n * H) +
         carve(nullptr, T, E, top_k, H, F).total;
}

// Entries processed per pass by the decode kernels, or 0 if the decode regime
// does not apply (too many entries, or inputs too long for LDS).
// An expert has at most T entries when the ids of a token are distinct, so
// passes of min(8, T) entries (rounded up to a power of two) cover it at once.
int dec_mt(int64_t T, int64_t n, int64_t H, int64_t F, size_t &lds1, size_t &lds2) {
  if (n > DEC_MAX_N) return 0;
  int start = 1;
  while (start < 8 && start < T) start <<= 1;
  for (int mt = start; mt >= 1; mt >>= 1) {
    lds1 = (size_t)mt * (H / QK) * REC_BF16 + (size_t)mt * (H / 8) +
           (size_t)mt * 2 * DEC_FR * (H / QK) * 4 + (size_t)mt * 2 * DEC_FR * 4;
    lds2 = (size_t)mt * (F / QK) * REC_F32 + (size_t)mt * (F / 8) +
           (size_t)mt * DEC_RW * (F / QK) * 4;
    if (lds1 <= 96 * 1024 && lds2 <= 96 * 1024) return mt;
  }
  return 0;
}

template <int MT>
void launch_dec(const void *x, const void *w13, const void *w2, const int32_t *ids,
                const float *gw, float *y, int64_t T, int64_t E, int64_t top_k, int64_t H,
                int64_t F, float *hbuf, float *obuf, size_t lds1, size_t lds2,
                hipStream_t s) {
  const int n = (int)(T * top_k);
  const unsigned slots = (unsigned)(E < n ? E : n);
  auto k1 = moe_dec_gateup_kernel<MT>;
  auto k2 = moe_dec_down_kernel<MT>;
  (void)hipFuncSetAttribute((const void *)k1, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds1);
  (void)hipFuncSetAttribute((const void *)k2, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds2);
  hipLaunchKernelGGL(k1, dim3((unsigned)((F + DEC_FR - 1) / DEC_FR), slots), dim3(DEC_THREADS),
                     lds1, s, (const uint16_t *)x, (const uint8_t *)w13, ids, n, (int)top_k,
                     (int)E, (int)H, (int)F, hbuf);
  hipLaunchKernelGGL(k2, dim3((unsigned)((H + DEC_RW - 1) / DEC_RW), slots), dim3(DEC_THREADS),
                     lds2, s, hbuf, (const uint8_t *)w2, ids, obuf, n, (int)top_k, (int)E,
                     (int)H, (int)F);
  const int64_t total = T * H;
  hipLaunchKernelGGL(moe_combine_entries_kernel,
                     dim3((unsigned)((total + 255) / 256 < 2048 ? (total + 255) / 256 : 2048)),
                     dim3(256), 0, s, obuf, ids, gw, y, (int)T, (int)top_k, (int)E, (int)H);
}

void launch_moe_q4k(const void *x, const void *w13, const void *w2, const int32_t *ids,
                    const float *gw, float *y, int64_t T, int64_t E, int64_t top_k, int64_t H,
                    int64_t F, void *workspace, hipStream_t s) {
  const int64_t n64 = T * top_k;
  char *base = (char *)workspace;
  float *hbuf = (float *)base;
  float *obuf = (float *)((char *)hbuf + align256(sizeof(float) * n64 * F));
  size_t lds1 = 0, lds2 = 0;
  switch (dec_mt(T, n64, H, F, lds1, lds2)) {
    case 8: launch_dec<8>(x, w13, w2, ids, gw, y, T, E, top_k, H, F, hbuf, obuf, lds1, lds2, s); return;
    case 4: launch_dec<4>(x, w13, w2, ids, gw, y, T, E, top_k, H, F, hbuf, obuf, lds1, lds2, s); return;
    case 2: launch_dec<2>(x, w13, w2, ids, gw, y, T, E, top_k, H, F, hbuf, obuf, lds1, lds2, s); return;
    case 1: launch_dec<1>(x, w13, w2, ids, gw, y, T, E, top_k, H, F, hbuf, obuf, lds1, lds2, s); return;
    default: break;
  }
  const MoeWs ws = carve((char *)obuf + align256(sizeof(float) * n64 * H), T, E, top_k, H, F);
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
