// Q4_K prefill GEMM on the matrix cores: y = x * W^T, x bf16 [M][K], y fp32.
//
// Prefill over GGUF weights runs on matrix cores (hipEngine README,
// "Quickstart": WMMA prefill, GEMV decode). On gfx950 the equivalent is the
// bf16 MFMA: Q4_K tiles are decoded in fp32 (w = d*sc*q - dmin*m, exact
// products, one rounding), rounded to bf16 (nearest even, v_cvt_pk_bf16_f32)
// into LDS next to the bf16 activation tile, and contracted with
// v_mfma_f32_32x32x16_bf16 into fp32 accumulators.
//
// Tiling: a 256-thread workgroup (one per compute unit) owns a 256 x 256 tile
// of y; each of its 4 waves owns a 128 x 128 quadrant = 4 x 4 MFMA tiles of
// 32 x 32, i.e. 256 fp32 accumulators per lane. Every weight a workgroup
// decodes feeds 256 rows of x, which keeps the decode (about 3 VALU
// operations per weight) well below the MFMA time. K advances in stages of 64:
// stage (b, c) is code chunk c (sub-blocks 2c, 2c+1) of super-block b, so each
// thread decodes one row's 32 code bytes per stage. Stages are double-buffered
// in LDS (rows padded to 144 bytes so that 16 consecutive rows hit distinct
// banks); the global loads of stage s+1 are in flight during the MFMAs of
// stage s. All global loads are unconditional (rows past M or N are clamped
// and their values zeroed), so the compiler waits for exactly the loads it
// needs.
//
// Work split (stream-K): the 256 x 256 tiles times the K/128 stage pairs of
// each form one iteration space that is cut into equal contiguous ranges, one
// per workgroup. With at least as many tiles as compute units there is one
// workgroup per unit; a range then covers the end of one tile, whole tiles,
// and the start of another, so every unit gets the same number of MFMAs and
// the last wave of tiles is not left to a few units. With fewer tiles than
// units, each workgroup gets exactly one tile (no split). The unit that computes the last stage pair of
// a tile owns it. A contributor (a unit that computed earlier pairs of the
// tile) leaves its fp32 partial tile in the workspace in the accumulators' own
// register order, so its stores and the owner's loads are whole 4 KiB lines
// per instruction. The owner writes its accumulators into LDS, half a tile at a
// time, adds there the partials of the contributors (always units with a
// smaller index, in decreasing index order, so the sum is deterministic), and
// stores y from LDS in 16-byte pieces of rows; a tile with no contributor goes
// from the accumulators straight to y. A
// contributor writes its partial, fences at device scope and raises its flag;
// the owner waits on the flag (bounded), reads the partial and lowers the flag
// again, so the workspace flags are zero between calls. Workgroups start in
// index order and a unit only waits on units with a smaller index, which have
// started before it; each unit computes the segment others wait for before
// the one that waits: the waits cannot deadlock and do not form chains.
//
// MFMA operand layout (32x32x16 bf16, wave64): lane l holds, for A, row l%32
// and k = 8*(l/32) .. +7; for B, column l%32 and the same k. The 32x32 fp32
// result gives lane l column l%32 and, in accumulator r, row
// 8*(r/4) + 4*(l/32) + r%4.
#include "common.h"
#include "launch.h"
#include "q4k_tile.h"

namespace qdm {

namespace {

constexpr int BM = 256, BN = 256, BK = 64;
constexpr int LROW = TILE_LROW;  // bf16 per LDS row (144 bytes)
constexpr int GEMM_THREADS = 256;
constexpr int TILE_ELEMS = BM * LROW;  // per operand and stage (BM == BN)


struct XRegs {
  u32x4 v[8];  // x tile: 8 x 16 bytes per thread
};
static_assert(BM == BN && BM == GEMM_THREADS, "one W row per thread");

// Per-lane 32-bit byte offsets of this thread's loads, relative to the
// tile's uniform base addresses (the loads then use a scalar base and a vector
// offset). Rows past M or N are clamped to the last row.
struct LoadOffsets {
  uint32_t x[8];  // x chunk i: row (tid/8 + 32i) of the tile, 16-byte column tid%8
  uint32_t w;     // this thread's W row
};

__device__ __forceinline__ LoadOffsets make_offsets(int M, int N, int K, int m0, int n0) {
  LoadOffsets o;
#pragma unroll
  for (int i = 0; i < 8; i++) {
    const int q = threadIdx.x + GEMM_THREADS * i;
    const int row = min(m0 + (q >> 3), M - 1) - m0;
    o.x[i] = (uint32_t)row * (uint32_t)K * 2u + (uint32_t)(q & 7) * 16u;
  }
  o.w = (uint32_t)(min(n0 + (int)threadIdx.x, N - 1) - n0) * (uint32_t)(K / QK) * Q4K_BYTES;
  return o;
}

__device__ __forceinline__ void load_x(XRegs &r, const LoadOffsets &o,
                                       const uint8_t *__restrict__ xtile, int stage) {
  const uint8_t *base = xtile + ((stage >> 2) * QK + (stage & 3) * BK) * 2;
#pragma unroll
  for (int i = 0; i < 8; i++) r.v[i] = *(const u32x4 *)(base + o.x[i]);
}

__device__ __forceinline__ void load_w(WRegs &r, const LoadOffsets &o,
                                       const uint8_t *__restrict__ wtile, int stage) {
  const int b = stage >> 2, c = stage & 3;
  const uint8_t *blk = wtile + b * Q4K_BYTES + o.w;
  r.hdr = *(const u32x4 *)blk;
  r.qa = *(const u32x4 *)(blk + 16 + 32 * c);
  r.qb = *(const u32x4 *)(blk + 32 + 32 * c);
}

__device__ __forceinline__ void store_x(const XRegs &r, uint16_t *sx, int M, int m0) {
  if (m0 + BM <= M) {  // uniform: the whole tile is inside M
#pragma unroll
    for (int i = 0; i < 8; i++) {
      const int q = threadIdx.x + GEMM_THREADS * i;
      *(u32x4 *)(sx + (q >> 3) * LROW + (q & 7) * 8) = r.v[i];
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; i++) {
      const int q = threadIdx.x + GEMM_THREADS * i;
      const int row = q >> 3;
      const u32x4 v = (m0 + row < M) ? r.v[i] : u32x4{0, 0, 0, 0};
      *(u32x4 *)(sx + row * LROW + (q & 7) * 8) = v;
    }
  }
}

// One stage of MFMAs from LDS buffer (sx, swb), with the W decode of the next
// stage (regs nw, stage ns, into nws; skipped when store_next is false) woven
// between them: per 16 MFMAs, a quarter of the decode.
__device__ __forceinline__ void mfma_stage(f32x16 (&acc)[4][4], const uint16_t *sx,
                                           const uint16_t *swb, const WRegs &nw,
                                           bool store_next, int ns, uint16_t *nws, int N,
                                           int n0, int wm, int wn, int lane) {
  const int arow = lane & 31, akoff = 8 * (lane >> 5);
  const RowScales sc = row_scales(nw, n0 + (int)threadIdx.x < N, ns & 3);
  const uint16_t *pa = sx + (wm * 128 + arow) * LROW + akoff;
  const uint16_t *pb = swb + (wn * 128 + arow) * LROW + akoff;
  // operand fragments of k-step kk are read one k-step ahead of their MFMAs
  bf16x8 af[2][4], bfr[2][4];
#pragma unroll
  for (int i = 0; i < 4; i++) {
    af[0][i] = *(const bf16x8 *)(pa + i * 32 * LROW);
    bfr[0][i] = *(const bf16x8 *)(pb + i * 32 * LROW);
  }
#pragma unroll
  for (int kk = 0; kk < 4; kk++) {
    const int cur = kk & 1;
    if (kk < 3) {
#pragma unroll
      for (int i = 0; i < 4; i++) {
        af[cur ^ 1][i] = *(const bf16x8 *)(pa + i * 32 * LROW + (kk + 1) * 16);
        bfr[cur ^ 1][i] = *(const bf16x8 *)(pb + i * 32 * LROW + (kk + 1) * 16);
      }
    }
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
      for (int j = 0; j < 4; j++)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[cur][i], bfr[cur][j], acc[i][j],
                                                            0, 0, 0);
    if (store_next) store_w_part(nw, sc, kk, nws);
#pragma unroll
    for (int t = 0; t < 16; t++) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);  // three VALU
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Multiplies stage range [s0, s1) (s1 - s0 even, >= 2) of tile (m0, n0) into acc.
__device__ __forceinline__ void run_segment(f32x16 (&acc)[4][4], uint16_t *smem,
                                            const uint8_t *__restrict__ w,
                                            const uint16_t *__restrict__ x, int M, int N, int K,
                                            int m0, int n0, int s0, int s1, uint32_t *publish) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
#pragma unroll
  for (int i = 0; i < 4; i++)
#pragma unroll
    for (int j = 0; j < 4; j++)
#pragma unroll
      for (int v = 0; v < 16; v++) acc[i][j][v] = 0.f;

  // Stage s lives in LDS buffer (s - s0) & 1. While stage s is multiplied: x
  // and W of stage s+2 are in flight, W of stage s+1 is decoded into the other
  // buffer and x of stage s+1 (loaded two stages earlier) is stored there.
  const LoadOffsets lo = make_offsets(M, N, K, m0, n0);
  const uint8_t *xtile = (const uint8_t *)(x + (int64_t)m0 * K);
  const uint8_t *wtile = w + (int64_t)n0 * (K / QK) * Q4K_BYTES;
  const int last = s1 - 1;
  XRegs xa, xb;
  WRegs wa, wb;
  load_x(xa, lo, xtile, s0);
  load_w(wa, lo, wtile, s0);
  load_x(xb, lo, xtile, s0 + 1);
  load_w(wb, lo, wtile, s0 + 1);
  __syncthreads();  // the previous segment's last MFMAs have read the buffers
  store_x(xa, smem, M, m0);
  {
    const RowScales sc = row_scales(wa, n0 + (int)threadIdx.x < N, s0 & 3);
#pragma unroll
    for (int kk = 0; kk < 4; kk++) store_w_part(wa, sc, kk, smem + TILE_ELEMS);
  }
  __syncthreads();

  // The loop body covers an even and an odd stage. Past the segment's last
  // stage, loads are clamped to it and the decodes/stores go to the buffer
  // that is no longer read.
  for (int s = s0; s < s1; s += 2) {
    // even stage s (buffer 0): W of s+1 (wb) decoded and x of s+1 (xb) stored into buffer 1
    load_x(xa, lo, xtile, min(s + 2, last));
    load_w(wa, lo, wtile, min(s + 2, last));
    mfma_stage(acc, smem, smem + TILE_ELEMS, wb, true, s + 1, smem + 3 * TILE_ELEMS, N, n0, wm,
               wn, lane);
    store_x(xb, smem + 2 * TILE_ELEMS, M, m0);
    __syncthreads();
    // odd stage s+1 (buffer 1): W of s+2 (wa) and x of s+2 (xa) into buffer 0
    load_x(xb, lo, xtile, min(s + 3, last));
    load_w(wb, lo, wtile, min(s + 3, last));
    mfma_stage(acc, smem + 2 * TILE_ELEMS, smem + 3 * TILE_ELEMS, wa, true, min(s + 2, last),
               smem + TILE_ELEMS, N, n0, wm, wn, lane);
    store_x(xa, smem, M, m0);
    __syncthreads();
    if (publish != nullptr && s == s0) {
      // the partial tile stored before this segment has long been written:
      // make it visible device-wide and raise its flag
      __threadfence();
      __syncthreads();
      if (threadIdx.x == 0)
        __hip_atomic_store(publish, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

constexpr uint32_t SPIN_LIMIT = 1u << 24;  // ~1 s of polling before giving up

// A partial tile in the accumulators' own layout: accumulator group
// g = (i*4 + j)*4 + v/4 (64 groups of 4 floats per thread) of thread t sits at
// float4 index g*256 + t, so each store or load instruction of the workgroup
// covers 4 KiB of consecutive bytes.
__device__ __forceinline__ void store_partial(const f32x16 (&acc)[4][4], float *__restrict__ slot) {
  f32x4 *dst = (f32x4 *)slot;
  int t = (int)threadIdx.x;
  asm volatile("" : "+v"(t));
#pragma unroll
  for (int i = 0; i < 4; i++)
#pragma unroll
    for (int j = 0; j < 4; j++)
#pragma unroll
      for (int q = 0; q < 4; q++)
        dst[((i * 4 + j) * 4 + q) * GEMM_THREADS + t] =
            f32x4{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                  acc[i][j][4 * q + 3]};
}

// y tile store straight from the accumulators (a tile no other unit worked
// on): each lane writes its 32-column runs of rows; rows and columns past M, N
// skipped.
__device__ __forceinline__ void store_direct(const f32x16 (&acc)[4][4], float *yt, int ldy,
                                             int rows, int cols) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  // lane coordinates pass through an opaque move, so the per-element address
  // arithmetic is not hoisted out of the tile loop (where it would hold a
  // register per element for the whole kernel)
  int col = wn * 128 + (lane & 31), rq = wm * 128 + 4 * (lane >> 5);
  asm volatile("" : "+v"(col), "+v"(rq));
#pragma unroll
  for (int i = 0; i < 4; i++)
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const int c = j * 32 + col;
#pragma unroll
      for (int v = 0; v < 16; v++) {
        const int r = i * 32 + 8 * (v >> 2) + rq + (v & 3);
        if (r < rows && c < cols) yt[(int64_t)r * ldy + c] = acc[i][j][v];
      }
    }
}

// y tile store through LDS (a tile with contributors): the two 128-row halves of the tile in turn are
// written into LDS by the waves that hold them, plus the partial tiles of the
// contributors (each thread adds the values at its own accumulator positions,
// contributor by contributor in a fixed order), then every thread writes
// whole 16-byte pieces of rows to y (rows and columns past M, N skipped).
constexpr int EPI_LD = BN + 4;  // floats per LDS row (16 bytes of bank padding)

__device__ __forceinline__ void store_tile(const f32x16 (&acc)[4][4], float *yt, int ldy,
                                           int rows, int cols, uint16_t *smem, bool vec,
                                           bool bad, const float *__restrict__ part0,
                                           int nparts) {
  float *st = (float *)smem;  // [128][EPI_LD]
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
#pragma unroll
  for (int h = 0; h < 2; h++) {
    __syncthreads();  // the LDS is free (MFMAs done / previous half written out)
    if (wm == h) {
      // lane coordinates pass through an opaque move so the per-element
      // address arithmetic is not hoisted (it would pin a register per element)
      int col = wn * 128 + (lane & 31), rq = 4 * (lane >> 5);
      asm volatile("" : "+v"(col), "+v"(rq));
#pragma unroll
      for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < 4; j++)
#pragma unroll
          for (int v = 0; v < 16; v++)
            st[(i * 32 + 8 * (v >> 2) + rq + (v & 3)) * EPI_LD + j * 32 + col] = acc[i][j][v];
      for (int k = 0; k < nparts; k++) {
        const f32x4 *src = (const f32x4 *)(part0 - (size_t)k * BM * BN);
#pragma unroll
        for (int i = 0; i < 4; i++)
#pragma unroll
          for (int j = 0; j < 4; j++) {
            int off = (i * 4 + j) * 4 * GEMM_THREADS + (int)threadIdx.x;
            asm volatile("" : "+v"(off));
            f32x4 t[4];
#pragma unroll
            for (int q = 0; q < 4; q++) t[q] = src[off + q * GEMM_THREADS];
#pragma unroll
            for (int v = 0; v < 16; v++)
              st[(i * 32 + 8 * (v >> 2) + rq + (v & 3)) * EPI_LD + j * 32 + col] += t[v >> 2][v & 3];
          }
      }
    }
    __syncthreads();
    // 128 rows x 64 pieces of 16 bytes, 32 per thread
    for (int e = threadIdx.x; e < 128 * (BN / 4); e += GEMM_THREADS) {
      const int r = e / (BN / 4), c = 4 * (e % (BN / 4));
      const int gr = 128 * h + r;
      if (gr >= rows) continue;
      f32x4 v = *(const f32x4 *)(st + r * EPI_LD + c);
      if (bad) v = f32x4{__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""), __builtin_nanf("")};
      float *py = yt + (int64_t)gr * ldy + c;
      if (vec && c + 3 < cols) {
        *(f32x4 *)py = v;
      } else {
#pragma unroll
        for (int q = 0; q < 4; q++)
          if (c + q < cols) py[q] = v[q];
      }
    }
  }
}

__global__ __launch_bounds__(GEMM_THREADS) void q4k_gemm_kernel(
    const uint8_t *__restrict__ w, const uint16_t *__restrict__ x, float *__restrict__ y, int M,
    int N, int K, float *__restrict__ partials, uint32_t *__restrict__ flags, int units) {
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];
  // stage buffer p: x tile at smem + 2p*TILE_ELEMS, W tile right after it
  __shared__ uint32_t timed_out;

  const int ntm = (M + BM - 1) / BM, ntn = (N + BN - 1) / BN;
  const int P = K / (2 * BK);  // stage pairs per tile
  const int64_t total = (int64_t)ntm * ntn * P;
  const int unit = blockIdx.x;
  const int64_t begin = total * unit / units, end = total * (unit + 1) / units;

  f32x16 acc[4][4];
  uint32_t *pending = nullptr;  // flag of a partial tile stored but not yet published
  // The range is walked from its end: the segment that starts a later tile
  // (the only one whose partial another unit waits for) comes first, the
  // segment that finishes an earlier tile (the only one that waits) comes last.
  // So no unit's partial waits behind its own wait, and waits do not chain.
  for (int64_t hi = end; hi > begin;) {
    // tiles are ordered with the two (or more) M tiles of one N tile adjacent,
    // so the units sharing a W tile run at the same time
    const int tile = (int)((hi - 1) / P);
    const int pe = (int)(hi - (int64_t)tile * P);
    const int pb = (int)max(begin - (int64_t)tile * P, (int64_t)0);
    const int m0 = (tile % ntm) * BM, n0 = (tile / ntm) * BN;
    run_segment(acc, smem, w, x, M, N, K, m0, n0, 2 * pb, 2 * pe, pending);
    pending = nullptr;
    hi = (int64_t)tile * P + pb;

    if (pe != P) {
      // A contributor (its range does not reach the tile's last stage pair)
      // stores its part in its workspace slot; the flag is raised during the
      // next segment (after its first stage pair), so the stores drain
      // behind MFMA work; if there is no next segment, right after the loop.
      store_partial(acc, partials + (size_t)unit * BM * BN);
      pending = &flags[unit];
      continue;
    }
    float *yt = y + (int64_t)m0 * N + n0;
    if (pb == 0) {  // the owner computed the whole tile
      store_direct(acc, yt, N, M - m0, N - n0);
      continue;
    }
    // Earlier units [lowest, unit) worked on this tile: wait for their flags;
    // their partials are added while the tile goes out (highest unit first, a
    // fixed order).
    int lowest = unit;
    while (lowest > 0 && total * lowest / units > (int64_t)tile * P) lowest--;
    if (threadIdx.x == 0) {
      uint32_t spins = 0;
      for (int u = unit - 1; u >= lowest; u--) {
        while (__hip_atomic_load(&flags[u], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT) == 0u &&
               ++spins < SPIN_LIMIT)
          __builtin_amdgcn_s_sleep(2);
        __hip_atomic_store(&flags[u], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      timed_out = spins >= SPIN_LIMIT;
    }
    __syncthreads();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    const bool bad = timed_out != 0u;  // a partial that never arrived poisons the tile
    store_tile(acc, yt, N, M - m0, N - n0, smem, (N & 3) == 0, bad,
               partials + (size_t)(unit - 1) * BM * BN, unit - lowest);
  }
  if (pending != nullptr) {  // the last segment left a partial: publish it now
    __threadfence();
    __syncthreads();
    if (threadIdx.x == 0)
      __hip_atomic_store(pending, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
  }
}


constexpr size_t GEMM_LDS = 4 * TILE_ELEMS * sizeof(uint16_t);  // 147456 bytes

inline size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

// Compute units of the current device (one workgroup each); 256 if unknown.
int device_units() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
      cus = 256;
    cached[dev] = cus;
  }
  return cached[dev];
}

// Workgroups of a call. With fewer tiles than compute units, one workgroup
// per tile: splitting them costs more in partial-tile traffic and in clock
// (every unit busy) than the idle units leave on the table (measured at
// M = 512, N = 17408, K = 5120: 136 tiles, 166 us whole versus 190 us split).
// With at least as many tiles as units, the stream-K split evens out the
// last wave of tiles.
int gemm_units(int64_t M, int64_t N, int64_t K) {
  const int64_t tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  const int64_t cus = device_units();
  if (tiles < cus) return (int)tiles;
  const int64_t total = tiles * (K / (2 * BK));
  return (int)(total < cus ? total : cus);
}

}  // namespace

// Workspace: one flag word per unit (256-byte aligned block), then one fp32
// partial tile per unit.
size_t q4k_gemm_workspace(int64_t M, int64_t N, int64_t K) {
  const size_t units = (size_t)gemm_units(M, N, K);
  return align256(units * sizeof(uint32_t)) + units * BM * BN * sizeof(float);
}

void launch_q4k_gemm(const void *w, const void *x, float *y, int64_t M, int64_t N, int64_t K,
                     void *workspace, hipStream_t s) {
  const int units = gemm_units(M, N, K);
  uint32_t *flags = (uint32_t *)workspace;
  float *partials = (float *)((char *)workspace + align256((size_t)units * sizeof(uint32_t)));
  (void)hipFuncSetAttribute((const void *)q4k_gemm_kernel,
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)GEMM_LDS);
  hipLaunchKernelGGL(q4k_gemm_kernel, dim3((unsigned)units), dim3(GEMM_THREADS), GEMM_LDS, s,
                     (const uint8_t *)w, (const uint16_t *)x, y, (int)M, (int)N, (int)K, partials,
                     flags, units);
}

}  // namespace qdm
