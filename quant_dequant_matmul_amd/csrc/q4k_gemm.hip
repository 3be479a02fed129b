// Q4_K prefill GEMM on the matrix cores: y = x * W^T, x bf16 [M][K], y fp32.
//
// Prefill over GGUF weights runs on matrix cores (hipEngine README,
// "Quickstart": WMMA prefill, GEMV decode). On gfx950 the equivalent is the
// bf16 MFMA: Q4_K weights are decoded in fp32 (w = d*sc*q - dmin*m, exact
// products, one rounding), rounded to bf16 (nearest even, v_cvt_pk_bf16_f32)
// and contracted with v_mfma_f32_32x32x16_bf16 into fp32 accumulators.
//
// Tiling: a 256-thread workgroup (one per compute unit) owns a 256 x 256 tile
// of y. Wave v owns all 256 rows of x and the 64 weight rows 64v .. 64v+63:
// 8 x 2 MFMA tiles of 32 x 32, i.e. 256 fp32 accumulators per lane. Each
// weight row is needed by one wave only, so every lane decodes its own two
// rows straight into MFMA operand registers: weights never pass through LDS.
// Only the x tile does (it is shared by the four waves): it is written once
// and read four times per stage, which halves the LDS write traffic of a
// layout that stages both operands (LDS writes run at half the read rate).
// Every weight a workgroup decodes feeds 256 rows of x, which keeps the
// decode (about 3 VALU operations per weight) below the MFMA time.
//
// K advances in stages of 64: stage (b, c) is code chunk c (sub-blocks 2c and
// 2c+1) of super-block b. The k order inside a stage is permuted (the
// contraction does not depend on it) so that each lane reads one contiguous
// 16-byte run of codes per row: lanes 0..31 take code bytes 0..15, lanes
// 32..63 bytes 16..31 of the chunk. In k-step kk (16 k per MFMA) lane half h
// holds the low nibbles (kk = 0, 1) or high nibbles (kk = 2, 3) of code bytes
// 16h + 8(kk&1) .. +7, i.e. k = 32(kk>>1) + 16h + 8(kk&1) .. +7 of the stage,
// and reads x at the same k.
//
// Pipeline (one barrier per stage): x of stage s+2 and the codes of stage s+2
// are loaded while stage s is multiplied; x of stage s+1 is stored into the
// other LDS buffer during stage s; the weight operands of k-step kk+1 are
// decoded while the MFMAs of k-step kk run. All global loads are
// unconditional (rows past M or N are clamped; weight rows past N decode to
// zero, x rows past M only feed y rows that are not stored), so the compiler
// waits for exactly the loads it needs, and a stage has no branch that would
// split its MFMA schedule.
//
// Work split (stream-K): the 256 x 256 tiles times the K/128 stage pairs of
// each form one iteration space that is cut into equal contiguous ranges, one
// per workgroup. With at least as many tiles as compute units there is one
// workgroup per unit; a range then covers the end of one tile, whole tiles,
// and the start of another, so every unit gets the same number of MFMAs and
// the last wave of tiles is not left to a few units. With fewer tiles than
// units the space is still split over every unit when it holds at least two
// stage pairs per unit and a tile per 16 units (M = 512, N = 17408: 136
// tiles on 256 units); smaller calls take one whole tile per workgroup. The
// unit that
// computes the last stage pair of a tile owns it. A contributor (a unit that
// computed earlier pairs of the tile) leaves its fp32 partial tile in the
// workspace in the accumulators' own register order, so its stores and the
// owner's loads are whole 4 KiB lines per instruction. The owner adds the
// partials of the contributors (always units with a smaller index, in
// decreasing index order, so the sum is deterministic) to its accumulators a
// quarter tile at a time in registers and stores y as a whole tile is stored. A
// contributor writes its partial and, once every store of the workgroup has
// completed, one thread raises its flag with a device-scope release; the owner
// polls the flag (bounded), acquires once, reads the partial and lowers the
// flag again, so the workspace flags are zero between calls. (A device-scope
// fence in every thread would invalidate the L2 of its XCD each time.) Workgroups start in
// index order and a unit only waits on units with a smaller index, which have
// started before it; each unit computes the segment others wait for before
// the one that waits: the waits cannot deadlock and do not form chains.
// If a wait runs out of its bound anyway, the handshake stays two-sided: the
// owner marks the flag abandoned (compare-and-swap 0 -> 2; if the swap finds
// 1 the partial did arrive and is used), writes the tile as NaN and counts the
// event in the workspace status word; a contributor raises its flag with an
// exchange and, finding the abandoned mark, lowers it to 0. Every flag is
// then zero when the kernel ends, whatever the timing.
//
// MFMA operand layout (32x32x16 bf16, wave64): lane l holds, for A, row l%32
// and 8 consecutive k; for B, column l%32 and the same 8 k (lane halves take
// the two 8-k halves of the k-step). The 32x32 fp32 result gives lane l
// column l%32 and, in accumulator r, row 8*(r/4) + 4*(l/32) + r%4.
#include "common.h"
#include "launch.h"
#include "q4k_tile.h"

namespace qdm {

namespace {

constexpr int BM = 256, BN = 256, BK = 64;
constexpr int LROW = TILE_LROW;  // bf16 per LDS x row (144 bytes)
constexpr int GEMM_THREADS = 256;
constexpr int XTILE = BM * LROW;  // bf16 per LDS x buffer
constexpr int WAVE_ROWS = BN / 4;  // weight rows per wave
// VALU instructions placed after each MFMA in k-steps 0..2 and in k-step 3
// (which also forms the next stage's scales); measured best of 2..4 / 4..8.
constexpr int SCHED_VALU = 3, SCHED_VALU_K3 = 6;

struct XRegs {
  u32x4 v[8];  // x tile: 8 x 16 bytes per thread
};
static_assert(BM == GEMM_THREADS, "x tile loads assume one row-eighth per thread and chunk");

// This lane's two weight rows (j = 0, 1) for one stage: the block header and
// the lane's 16 code bytes of the stage's chunk.
struct WRaw {
  u32x4 hdr[2], q[2];
};

// Scales of both rows for one stage (a0, a1 carry the factor 2^9 that the fp8
// reading of the codes leaves out).
struct Scales2 {
  RowScales r[2];
};

// Per-lane 32-bit byte offsets of this thread's loads, relative to the
// tile's uniform base addresses (the loads then use a scalar base and a vector
// offset). Rows past M or N are clamped to the last row.
struct LoadOffsets {
  uint32_t x[8];  // x chunk i: row (tid/8 + 32i) of the tile, 16-byte column tid%8
  uint32_t w[2];  // weight row j of this lane: 64*wave + 32j + lane%32
  uint32_t q;     // code bytes of this lane half within a stage's 32-byte chunk
};

__device__ __forceinline__ LoadOffsets make_offsets(int M, int N, int K, int m0, int n0,
                                                    int wave, int lane) {
  LoadOffsets o;
#pragma unroll
  for (int i = 0; i < 8; i++) {
    const int q = threadIdx.x + GEMM_THREADS * i;
    const int row = min(m0 + (q >> 3), M - 1) - m0;
    o.x[i] = (uint32_t)row * (uint32_t)K * 2u + (uint32_t)(q & 7) * 16u;
  }
#pragma unroll
  for (int j = 0; j < 2; j++) {
    const int row = min(n0 + WAVE_ROWS * wave + 32 * j + (lane & 31), N - 1) - n0;
    o.w[j] = (uint32_t)row * (uint32_t)(K / QK) * Q4K_BYTES;
  }
  o.q = 16u + 16u * (uint32_t)(lane >> 5);
  return o;
}

__device__ __forceinline__ void load_x(XRegs &r, const LoadOffsets &o,
                                       const uint8_t *__restrict__ xtile, int stage) {
  const uint8_t *base = xtile + ((stage >> 2) * QK + (stage & 3) * BK) * 2;
#pragma unroll
  for (int i = 0; i < 8; i++) r.v[i] = *(const u32x4 *)(base + o.x[i]);
}

__device__ __forceinline__ void load_w(WRaw &r, const LoadOffsets &o,
                                       const uint8_t *__restrict__ wtile, int stage) {
  const uint8_t *blk = wtile + (stage >> 2) * Q4K_BYTES;
  const uint32_t qo = o.q + 32u * (uint32_t)(stage & 3);
#pragma unroll
  for (int j = 0; j < 2; j++) {
    r.hdr[j] = *(const u32x4 *)(blk + o.w[j]);
    r.q[j] = *(const u32x4 *)(blk + o.w[j] + qo);
  }
}

// Scale and min of sub-block j (0..7) of a block header, without a branch on
// j (the stage, hence j, is known only at run time, and a branch would split
// the MFMA schedule): both packings are formed and the right one selected.
__device__ __forceinline__ void scale_min_sel(const u32x4 &hdr, int j, uint32_t &sc,
                                              uint32_t &m) {
  const int sh = 8 * (j & 3);
  const uint32_t b0 = hdr.y >> sh, b1 = hdr.z >> sh, b2 = hdr.w >> sh;
  const uint32_t lo_sc = b0 & 63u, lo_m = b1 & 63u;
  const uint32_t hi_sc = (b2 & 15u) | ((b0 >> 2) & 48u);
  const uint32_t hi_m = ((b2 >> 4) & 15u) | ((b1 >> 2) & 48u);
  sc = j < 4 ? lo_sc : hi_sc;
  m = j < 4 ? lo_m : hi_m;
}

__device__ __forceinline__ Scales2 stage_scales(const WRaw &r, const bool (&live)[2], int stage) {
  Scales2 s;
  const int c = stage & 3;
#pragma unroll
  for (int j = 0; j < 2; j++) {
    const float d = live[j] ? half_bits_to_float(r.hdr[j].x) : 0.f;
    const float dmin = live[j] ? half_bits_to_float(r.hdr[j].x >> 16) : 0.f;
    uint32_t sc0, m0s, sc1, m1s;
    scale_min_sel(r.hdr[j], 2 * c, sc0, m0s);
    scale_min_sel(r.hdr[j], 2 * c + 1, sc1, m1s);
    const float d9 = d * 512.f;  // the fp8 code scale 2^-9 undone (exact)
    s.r[j] = RowScales{d9 * (float)sc0, dmin * (float)m0s, d9 * (float)sc1, dmin * (float)m1s};
  }
  return s;
}

// Weight operand of k-step kk for one row: 8 codes (two code words) scaled by
// the sub-block's scale and min, rounded to bf16. A code byte 0..15 read as an
// fp8 e4m3 value is exactly q * 2^-9 (the small ones as subnormals), so one
// conversion turns two codes into floats; the scale a carries the factor 2^9
// (exact), and a * (q * 2^-9) - b is the same single-rounding fma as
// a * q - b.
__device__ __forceinline__ bf16x8 decode_b(const u32x4 &q, const RowScales &sc, int kk) {
  const bool hi = kk >= 2;
  const uint32_t c0 = (kk & 1) ? q.z : q.x, c1 = (kk & 1) ? q.w : q.y;
  const float a = hi ? sc.a1 : sc.a0, b = hi ? sc.b1 : sc.b0;
  const uint32_t n0 = (hi ? c0 >> 4 : c0) & 0x0F0F0F0Fu, n1 = (hi ? c1 >> 4 : c1) & 0x0F0F0F0Fu;
  const auto p0 = __builtin_amdgcn_cvt_pk_f32_fp8((int)n0, false);
  const auto p1 = __builtin_amdgcn_cvt_pk_f32_fp8((int)n0, true);
  const auto p2 = __builtin_amdgcn_cvt_pk_f32_fp8((int)n1, false);
  const auto p3 = __builtin_amdgcn_cvt_pk_f32_fp8((int)n1, true);
  u32x4 o;
  o.x = pack_bf16(a * p0[0] - b, a * p0[1] - b);
  o.y = pack_bf16(a * p1[0] - b, a * p1[1] - b);
  o.z = pack_bf16(a * p2[0] - b, a * p2[1] - b);
  o.w = pack_bf16(a * p3[0] - b, a * p3[1] - b);
  return __builtin_bit_cast(bf16x8, o);
}

// x chunks i0 .. i0+3 of this thread into an LDS x buffer. Rows past M hold
// copies of row M-1 (clamped loads): finite, and their y rows are never
// stored, so they need no masking (and the stage has no branch).
__device__ __forceinline__ void store_x_part(const XRegs &r, uint16_t *sx, int i0) {
#pragma unroll
  for (int i = i0; i < i0 + 4; i++) {
    const int q = threadIdx.x + GEMM_THREADS * i;
    *(u32x4 *)(sx + (q >> 3) * LROW + (q & 7) * 8) = r.v[i];
  }
}

// LDS offset (in bf16) of this lane's x operand for k-step kk, row tile 0.
__device__ __forceinline__ int a_koff(int kk, int lane) {
  return 32 * (kk >> 1) + 16 * (lane >> 5) + 8 * (kk & 1);
}

// One stage. On entry bf[0] holds the weight operands of k-step 0 and
// sc_cur the scales of this stage; the x tile of this stage is complete in sx.
// During the stage: x of stage s+2 is loaded into xl, x of stage s+1 (xs) is
// stored into nsx, the codes of stage s+2 are loaded into wcur once its last
// operands are decoded, and the scales and k-step-0 operands of stage s+1
// (wnext) are formed, so that on exit bf[0] and sc_next are ready.
__device__ __forceinline__ void gemm_stage(f32x16 (&acc)[8][2], bf16x8 (&bf)[2][2],
                                           const Scales2 &sc_cur, Scales2 &sc_next,
                                           WRaw &wcur, const WRaw &wnext, int s_next,
                                           int s_load, const XRegs &xs, XRegs &xl,
                                           const uint16_t *sx, uint16_t *nsx,
                                           const LoadOffsets &lo, const bool (&live)[2],
                                           const uint8_t *__restrict__ xtile,
                                           const uint8_t *__restrict__ wtile, int M, int m0,
                                           int lane) {
  load_x(xl, lo, xtile, s_load);
  const uint16_t *pa = sx + (lane & 31) * LROW;
  bf16x8 af[8];
#pragma unroll
  for (int i = 0; i < 8; i++) af[i] = *(const bf16x8 *)(pa + i * 32 * LROW + a_koff(0, lane));
#pragma unroll
  for (int kk = 0; kk < 4; kk++) {
    const int cur = kk & 1;
    if (kk < 3) {
#pragma unroll
      for (int j = 0; j < 2; j++) bf[cur ^ 1][j] = decode_b(wcur.q[j], sc_cur.r[j], kk + 1);
    } else {
      sc_next = stage_scales(wnext, live, s_next);
#pragma unroll
      for (int j = 0; j < 2; j++) bf[cur ^ 1][j] = decode_b(wnext.q[j], sc_next.r[j], 0);
      load_w(wcur, lo, wtile, s_load);
    }
#pragma unroll
    for (int i = 0; i < 8; i++) {
      acc[i][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bf[cur][0], acc[i][0], 0, 0, 0);
      acc[i][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bf[cur][1], acc[i][1], 0, 0, 0);
      if (kk < 3) af[i] = *(const bf16x8 *)(pa + i * 32 * LROW + a_koff(kk + 1, lane));
    }
    if (kk < 2) store_x_part(xs, nsx, 4 * kk);
    // k-steps 0..2 carry one row pair's decode, k-step 3 also the next
    // stage's scales: their VALU work is spread over the 16 MFMAs
    if (kk < 3) {
#pragma unroll
      for (int t = 0; t < 16; t++) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);            // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, SCHED_VALU, 0);  // VALU
      }
    } else {
#pragma unroll
      for (int t = 0; t < 16; t++) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, SCHED_VALU_K3, 0);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  __syncthreads();  // x of stage s+1 complete in nsx; sx free for stage s+2
}

// Flag states: 0 idle, 1 partial published, 2 abandoned by an owner whose
// wait ran out (the contributor then resets it).
constexpr uint32_t FLAG_PUBLISHED = 1u, FLAG_ABANDONED = 2u;

__device__ __forceinline__ void raise_flag(uint32_t *flag) {
  const uint32_t old =
      __hip_atomic_exchange(flag, FLAG_PUBLISHED, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
  if (old == FLAG_ABANDONED)  // nobody will read this partial: leave the flag idle
    __hip_atomic_store(flag, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Makes this workgroup's partial tile visible to the other XCDs and raises
// its flag: every thread waits for its own stores to reach the L2, then one
// release (an L2 write-back, no invalidate) precedes the flag. A device-wide
// fence in every thread would also invalidate the L2 that the other compute
// units of the XCD read x and the weights through (measured: M = 512 split over
// 256 units 152 -> 126 us without it).
__device__ __forceinline__ void publish_partial(uint32_t *flag) {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (threadIdx.x == 0) raise_flag(flag);
}

// Multiplies stage range [s0, s1) (s1 - s0 even, >= 2) of tile (m0, n0) into acc.
__device__ __forceinline__ void run_segment(f32x16 (&acc)[8][2], uint16_t *smem,
                                            const uint8_t *__restrict__ w,
                                            const uint16_t *__restrict__ x, int M, int N, int K,
                                            int m0, int n0, int s0, int s1, uint32_t *publish) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
#pragma unroll
  for (int i = 0; i < 8; i++)
#pragma unroll
    for (int j = 0; j < 2; j++)
#pragma unroll
      for (int v = 0; v < 16; v++) acc[i][j][v] = 0.f;

  const LoadOffsets lo = make_offsets(M, N, K, m0, n0, wave, lane);
  bool live[2];
#pragma unroll
  for (int j = 0; j < 2; j++) live[j] = n0 + WAVE_ROWS * wave + 32 * j + (lane & 31) < N;
  const uint8_t *xtile = (const uint8_t *)(x + (int64_t)m0 * K);
  const uint8_t *wtile = w + (int64_t)n0 * (K / QK) * Q4K_BYTES;
  const int last = s1 - 1;
  uint16_t *sx0 = smem, *sx1 = smem + XTILE;
  XRegs xa, xb;
  WRaw wa, wb;
  Scales2 sca, scb;
  bf16x8 bf[2][2];
  load_x(xa, lo, xtile, s0);
  load_w(wa, lo, wtile, s0);
  load_x(xb, lo, xtile, s0 + 1);
  load_w(wb, lo, wtile, s0 + 1);
  __syncthreads();  // the previous segment's last reads of the buffers are done
  store_x_part(xa, sx0, 0);
  store_x_part(xa, sx0, 4);
  sca = stage_scales(wa, live, s0);
#pragma unroll
  for (int j = 0; j < 2; j++) bf[0][j] = decode_b(wa.q[j], sca.r[j], 0);
  __syncthreads();

  // The loop body covers an even and an odd stage; register sets alternate.
  // Past the segment's last stage, loads are clamped to it and the stores go
  // to the buffer that is no longer read.
  for (int s = s0; s < s1; s += 2) {
    // even stage s: codes wa, x in sx0; x of s+1 (xb) into sx1; loads of s+2 into xa, wa
    gemm_stage(acc, bf, sca, scb, wa, wb, s + 1, min(s + 2, last), xb, xa, sx0, sx1, lo, live,
               xtile, wtile, M, m0, lane);
    // odd stage s+1: codes wb, x in sx1; x of s+2 (xa) into sx0; loads of s+3 into xb, wb
    gemm_stage(acc, bf, scb, sca, wb, wa, min(s + 2, last), min(s + 3, last), xa, xb, sx1, sx0,
               lo, live, xtile, wtile, M, m0, lane);
    if (publish != nullptr && s == s0) publish_partial(publish);
  }
}

// Polls of a flag before an owner gives up (about 1 s of polling); the host
// can lower it (qdm_set_gemm_spin_limit) to exercise the give-up path.
constexpr uint32_t SPIN_LIMIT = 1u << 24;

// A partial tile in the accumulators' own layout: accumulator group
// g = (i*2 + j)*4 + v/4 (64 groups of 4 floats per thread) of thread t sits at
// float4 index g*256 + t, so each store or load instruction of the workgroup
// covers 4 KiB of consecutive bytes.
__device__ __forceinline__ void store_partial(const f32x16 (&acc)[8][2], float *__restrict__ slot) {
  f32x4 *dst = (f32x4 *)slot;
  int t = (int)threadIdx.x;
  asm volatile("" : "+v"(t));
#pragma unroll
  for (int i = 0; i < 8; i++)
#pragma unroll
    for (int j = 0; j < 2; j++)
#pragma unroll
      for (int q = 0; q < 4; q++)
        dst[((i * 2 + j) * 4 + q) * GEMM_THREADS + t] =
            f32x4{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                  acc[i][j][4 * q + 3]};
}

// y stores go through a buffer resource over the tile's rows: the lane's
// column (and lane-half row offset) is the vector offset and each row's
// offset is a scalar, so a store costs no vector address arithmetic; bytes
// past the tile's last valid row (rows past M) are dropped by the hardware's
// range check, and lanes whose column is past N are masked. The host limits
// N to 2^20, so 256 rows of y stay within 2^31 bytes.
constexpr int BUF_DWORD3 = 0x00020000;  // raw 32-bit buffer access (gfx9 family)

struct YOut {
  __amdgpu_buffer_rsrc_t rsrc;
  int voff;     // (lane-half row offset * ldy + column) * 4 for this lane, column tile 0
  int ldy4;     // ldy * 4
  bool live0, live1;  // column tile 0 / 1 of this lane inside N
};

__device__ __forceinline__ YOut y_out(float *yt, int ldy, int rows, int cols) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = WAVE_ROWS * wave + (lane & 31), rq = 4 * (lane >> 5);
  YOut o;
  o.rsrc = __builtin_amdgcn_make_buffer_rsrc(yt, (short)0, min(rows, BM) * ldy * 4, BUF_DWORD3);
  o.voff = (rq * ldy + col) * 4;
  o.ldy4 = ldy * 4;
  o.live0 = col < cols;
  o.live1 = col + 32 < cols;
  return o;
}

// Value v (accumulator index 0..15) of MFMA tile (i, j): row
// i*32 + 8*(v/4) + (lane-half offset) + v%4, column j*32 + (lane column).
__device__ __forceinline__ void y_put(const YOut &o, float val, int i, int j, int v) {
  if (j == 0 ? o.live0 : o.live1)
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, val), o.rsrc,
                                          o.voff + j * 128,
                                          (i * 32 + 8 * (v >> 2) + (v & 3)) * o.ldy4, 0);
}

// A tile no other unit worked on: straight from the accumulators.
__device__ __forceinline__ void store_direct(const f32x16 (&acc)[8][2], float *yt, int ldy,
                                             int rows, int cols) {
  const YOut o = y_out(yt, ldy, rows, cols);
#pragma unroll
  for (int i = 0; i < 8; i++)
#pragma unroll
    for (int j = 0; j < 2; j++)
#pragma unroll
      for (int v = 0; v < 16; v++) y_put(o, acc[i][j][v], i, j, v);
}

// A tile with contributors: its y values are the owner's accumulators plus
// the contributors' partial tiles (stored in accumulator order, so thread t
// finds its own values as whole 16-byte pieces), added in a fixed order (the
// owner's, then unit - 1, unit - 2, ...: deterministic). A quarter of the tile
// (two row tiles, 64 values per thread) at a time: the sums live in registers
// beside the accumulators, which are only read, and the quarter goes out as
// store_direct writes a whole tile. A tile whose partial never arrived is
// written as NaN.
// PREFETCH: the next quarter of the first partial (unit - 1's) is loaded while
// the current one is added and stored, so the quarters cost one memory latency
// instead of four. That pays when owners finish at different times (at least
// as many tiles as units: M = 4096, N = 17408, 725 -> 706 us); when every owner
// finishes at once (M = 512) the epilogues share HBM and the deeper queue was
// slower (14 -> 24 us per epilogue), so those calls keep one quarter in flight.
template <bool PREFETCH>
__device__ __forceinline__ void store_summed(const f32x16 (&acc)[8][2], float *yt, int ldy,
                                             int rows, int cols, const float *__restrict__ part0,
                                             int nparts, bool poison) {
  const YOut o = y_out(yt, ldy, rows, cols);
  int t = (int)threadIdx.x;
  asm volatile("" : "+v"(t));
  const f32x4 *src0 = (const f32x4 *)part0 + t;
  f32x4 pn[16];
  if constexpr (PREFETCH) {
#pragma unroll
    for (int gg = 0; gg < 16; gg++) pn[gg] = src0[gg * GEMM_THREADS];
  }
#pragma unroll
  for (int qt = 0; qt < 4; qt++) {
    f32x4 sum[16];
#pragma unroll
    for (int gg = 0; gg < 16; gg++) {
      const int i = 2 * qt + (gg >> 3), j = (gg >> 2) & 1, v0 = 4 * (gg & 3);
      sum[gg] = f32x4{acc[i][j][v0], acc[i][j][v0 + 1], acc[i][j][v0 + 2], acc[i][j][v0 + 3]};
    }
    int k = 0;
    if constexpr (PREFETCH) {
      // nparts >= 1: the owner's sum plus unit - 1's partial, then the next
      // quarter of that partial goes in flight
#pragma unroll
      for (int gg = 0; gg < 16; gg++) sum[gg] += pn[gg];
      if (qt < 3) {
#pragma unroll
        for (int gg = 0; gg < 16; gg++) pn[gg] = src0[(16 * (qt + 1) + gg) * GEMM_THREADS];
      }
      k = 1;
    }
    for (; k < nparts; k++) {
      const f32x4 *src = (const f32x4 *)(part0 - (size_t)k * BM * BN) + t;
      f32x4 p[16];
#pragma unroll
      for (int gg = 0; gg < 16; gg++) p[gg] = src[(16 * qt + gg) * GEMM_THREADS];
#pragma unroll
      for (int gg = 0; gg < 16; gg++) sum[gg] += p[gg];
    }
    if (poison) {
#pragma unroll
      for (int gg = 0; gg < 16; gg++)
        sum[gg] = f32x4{__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""),
                        __builtin_nanf("")};
    }
#pragma unroll
    for (int gg = 0; gg < 16; gg++) {
      const int i = 2 * qt + (gg >> 3), j = (gg >> 2) & 1, q = gg & 3;
#pragma unroll
      for (int e = 0; e < 4; e++) y_put(o, sum[gg][e], i, j, 4 * q + e);
    }
  }
}

__global__ __launch_bounds__(GEMM_THREADS) void q4k_gemm_kernel(
    const uint8_t *__restrict__ w, const uint16_t *__restrict__ x, float *__restrict__ y, int M,
    int N, int K, float *__restrict__ partials, uint32_t *__restrict__ flags,
    uint32_t *__restrict__ status, int units, uint32_t spin_limit) {
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];  // x stage buffer p at smem + p*XTILE
  __shared__ uint32_t timed_out;

  const int ntm = (M + BM - 1) / BM, ntn = (N + BN - 1) / BN;
  const int P = K / (2 * BK);  // stage pairs per tile
  const int64_t total = (int64_t)ntm * ntn * P;
  const int unit = blockIdx.x;
  const int64_t begin = total * unit / units, end = total * (unit + 1) / units;
  const bool spread = (int64_t)ntm * ntn >= units;  // at least one whole tile per unit

  f32x16 acc[8][2];
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
      bool lost = false;
      for (int u = unit - 1; u >= lowest; u--) {
        // relaxed polls (an acquire load would invalidate the L2 on every poll)
        while (__hip_atomic_load(&flags[u], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0u &&
               ++spins < spin_limit)
          __builtin_amdgcn_s_sleep(2);
        uint32_t seen = 0u;
        if (spins >= spin_limit &&
            __hip_atomic_compare_exchange_strong(&flags[u], &seen, FLAG_ABANDONED,
                                                 __ATOMIC_ACQ_REL, __ATOMIC_ACQUIRE,
                                                 __HIP_MEMORY_SCOPE_AGENT)) {
          lost = true;  // the contributor resets the abandoned flag when it publishes
          continue;
        }
        __hip_atomic_store(&flags[u], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      timed_out = lost;
      if (lost) atomicAdd(status, 1u);
      // one acquire for the partials seen (drops stale cached copies of them)
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    }
    __syncthreads();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    // the first partial is unit - 1's; spread: owners finish at different times
    if (spread)
      store_summed<true>(acc, yt, N, M - m0, N - n0, partials + (size_t)(unit - 1) * BM * BN,
                         unit - lowest, timed_out != 0u);
    else
      store_summed<false>(acc, yt, N, M - m0, N - n0, partials + (size_t)(unit - 1) * BM * BN,
                          unit - lowest, timed_out != 0u);
  }
  if (pending != nullptr) publish_partial(pending);  // the last segment left a partial
}

// Dynamic LDS: two x stage buffers (73728 bytes).
constexpr size_t GEMM_LDS = 2 * XTILE * sizeof(uint16_t);

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

// Workgroups of a call: the stream-K split over one workgroup per compute
// unit when there are at least as many tiles as units, or when the split
// gives every unit at least two stage pairs and no tile more than 16 units
// (an owner adds its contributors' partial tiles one after another). With
// fewer tiles than units this puts the idle units to work (M = 512,
// N = 17408, K = 5120: 136 tiles, 140 -> 122 us). Otherwise one workgroup per
// tile.
int gemm_units(int64_t M, int64_t N, int64_t K) {
  const int64_t tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  const int64_t cus = device_units();
  const int64_t total = tiles * (K / (2 * BK));
  if (tiles >= cus || (total >= 2 * cus && 16 * tiles >= cus))
    return (int)(total < cus ? total : cus);
  return (int)tiles;
}

// Whether a call splits tiles between workgroups (then it needs the flags and
// partial tiles of the workspace).
bool gemm_splits(int64_t M, int64_t N, int64_t K) {
  const int64_t tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  return gemm_units(M, N, K) != tiles;
}

uint32_t g_spin_limit = SPIN_LIMIT;

}  // namespace

void set_gemm_spin_limit(uint32_t limit) { g_spin_limit = limit ? limit : SPIN_LIMIT; }

// Workspace of a call that splits tiles (none otherwise): a 256-byte status
// block (word 0: split-tile waits that gave up, counted across calls), one
// flag word per unit (256-byte aligned block) and one fp32 partial tile per
// unit.
size_t q4k_gemm_workspace(int64_t M, int64_t N, int64_t K) {
  if (!gemm_splits(M, N, K)) return 0;  // whole tiles: no flags, partials or waits
  const size_t units = (size_t)gemm_units(M, N, K);
  return 256 + align256(units * sizeof(uint32_t)) + units * BM * BN * sizeof(float);
}

void launch_q4k_gemm(const void *w, const void *x, float *y, int64_t M, int64_t N, int64_t K,
                     void *workspace, hipStream_t s) {
  const int units = gemm_units(M, N, K);
  uint32_t *status = (uint32_t *)workspace;
  uint32_t *flags = (uint32_t *)((char *)workspace + 256);
  float *partials =
      (float *)((char *)workspace + 256 + align256((size_t)units * sizeof(uint32_t)));
  (void)hipFuncSetAttribute((const void *)q4k_gemm_kernel,
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)GEMM_LDS);
  hipLaunchKernelGGL(q4k_gemm_kernel, dim3((unsigned)units), dim3(GEMM_THREADS), GEMM_LDS, s,
                     (const uint8_t *)w, (const uint16_t *)x, y, (int)M, (int)N, (int)K, partials,
                     flags, status, units, g_spin_limit);
}

}  // namespace qdm
