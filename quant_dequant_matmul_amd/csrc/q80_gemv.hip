// Q8_0 GEMV: y[m][n] = sum_k x[m][k] * w(n, k) for M in 1..16.
//
// Q8_0 (hipEngine README, "GGUF Support", payload table) holds 32 weights in
// 34 bytes: fp16 d, then 32 two's-complement int8 codes q; w = d * q. A row of
// K columns is K/32 blocks, and with K % 256 == 0 it is a whole number of
// 16-byte chunks.
//
// Mapping. A quad is 4 consecutive blocks of a row: 136 bytes, 128 columns.
// A row holds an even number of quads, so quads never straddle rows. A
// workgroup owns a contiguous range of rows, i.e. of quads. Its waves take
// spans of 32 quads (4352 bytes) from a workgroup counter and load each span
// with 16-byte non-temporal loads (1 KiB per wave instruction). The next span
// stays in flight in registers while the wave computes the current one from
// its own LDS buffer, where lanes 2i and 2i + 1 share quad i: lane 2i + h
// reads blocks 2h and 2h + 1 (68 bytes, 4-byte aligned), and the two halves
// are added in a fixed order. Blocks 0 and 2 of a quad have their codes 2
// bytes into a dword and are realigned with v_alignbyte; blocks 1 and 3 have
// them dword-aligned. Half-size spans keep the first burst of weight loads
// small (x, loaded first, is ready sooner) and the last span's math short.
//
// Per code, q + 128 = byte ^ 0x80 is converted with v_cvt_f32_ubyte and
// multiplied by fp32 x from LDS; per block sum_k x_k q_k = s - 128 sum_k x_k,
// with the 32-column sums of x staged beside x.
//
// x lives in LDS as 528-byte records per 128 columns: 128 fp32 values and the
// four 32-column sums. The record stride is 132 dwords, so lanes reading
// consecutive records hit distinct banks. Long K is split into equal column
// chunks of at least 8192 columns, one launch each; every chunk after the
// first adds its partial sums to y.
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace qdm {

namespace {

constexpr int Q8_QUAD = 4 * Q80_BYTES;                 // 136 bytes, 128 columns
constexpr int Q8_SPAN = 32;                            // quads per span, two lanes each
constexpr int Q8_SPAN_BYTES = Q8_SPAN * Q8_QUAD;       // 4352 = 4.25 KiB
constexpr int Q8_NCH = (Q8_SPAN_BYTES + 1023) / 1024;  // 5 loads per lane, the last partly used
constexpr int Q8_SPAN_BUF = 1024 * Q8_NCH;             // LDS per wave
constexpr int Q8_XREC = 528;                           // LDS bytes per 128-column x record
constexpr int Q8_NB = 1;                               // spans in flight per wave
constexpr int Q8_TARGET_WGS = 256;                     // one workgroup per compute unit
constexpr int Q8_MIN_CHUNK = 8192;                     // columns of a chunk when K is split
constexpr size_t Q8_LDS_LIMIT = 160 * 1024;

struct Q8Span {
  u32x4 r[Q8_NCH];
};

// x records of MT tokens for columns kc0 .. kc0+kcn-1: token m, record q,
// element e at byte m * xstr + 528 q + 4 e; the sum of elements 32i .. 32i+31
// at byte m * xstr + 528 q + 512 + 4 i. A task is 4 consecutive columns; 8
// consecutive tasks make one 32-column sum. bf16 tasks keep their raw 8 bytes
// in registers until they are stored.
template <bool XBF16>
struct Q8XTask {
  typedef typename std::conditional<XBF16, u32x2, u32x4>::type Raw;
  Raw v;

  __device__ __forceinline__ void load(const void *__restrict__ x, int ldx, int kc0, int tpt,
                                       int task) {
    const int m = task / tpt, c4 = task - m * tpt;
    const int64_t e = (int64_t)m * ldx + kc0 + 4 * c4;
    if constexpr (XBF16)
      v = *(const u32x2 *)((const uint16_t *)x + e);
    else
      v = *(const u32x4 *)((const float *)x + e);
  }

  // valid: the task exists. Every lane takes part in the shuffles.
  __device__ __forceinline__ void store(uint8_t *xrec, int xstr, int tpt, int task,
                                        bool valid) const {
    f32x4 f;
    if constexpr (XBF16)
      f = __builtin_bit_cast(f32x4, u32x4{v.x << 16, v.x & 0xFFFF0000u, v.y << 16,
                                          v.y & 0xFFFF0000u});
    else
      f = __builtin_bit_cast(f32x4, v);
    float s = valid ? (f.x + f.y) + (f.z + f.w) : 0.f;
    s = lane_group_sum<8>(s);
    if (valid) {
      const int m = task / tpt, c4 = task - m * tpt;
      uint8_t *rec = xrec + m * xstr + (c4 >> 5) * Q8_XREC;
      *(f32x4 *)(rec + 16 * (c4 & 31)) = f;
      if ((c4 & 7) == 0) *(float *)(rec + 512 + 4 * ((c4 & 31) >> 3)) = s;
    }
  }
};

// sum_k x_k q_k over the 32 codes of one block (code words cw, q + 128
// converted per byte) against x at xb, for MT tokens (record stride xstr).
template <int MT>
__device__ __forceinline__ void q8_block(const uint32_t (&cw)[8], float d, const uint8_t *xb,
                                         int xstr, float (&acc)[MT]) {
  float f[32];
#pragma unroll
  for (int c = 0; c < 8; c++) {
    const uint32_t u = cw[c] ^ 0x80808080u;
    f[4 * c + 0] = (float)(u & 255u);
    f[4 * c + 1] = (float)((u >> 8) & 255u);
    f[4 * c + 2] = (float)((u >> 16) & 255u);
    f[4 * c + 3] = (float)(u >> 24);
  }
#pragma unroll
  for (int m = 0; m < MT; m++) {
    const uint8_t *xm = xb + m * xstr;
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < 8; c++) {
      const f32x4 xv = *(const f32x4 *)(xm + 16 * c);
      s = fmaf(xv.x, f[4 * c + 0], s);
      s = fmaf(xv.y, f[4 * c + 1], s);
      s = fmaf(xv.z, f[4 * c + 2], s);
      s = fmaf(xv.w, f[4 * c + 3], s);
    }
    acc[m] = fmaf(d, s, acc[m]);
  }
}

// Partial dot products of half h of one quad (blocks 2h and 2h + 1: the 68
// bytes at q, 4-byte aligned LDS) against the quad's x record xr, for MT
// tokens.
template <int MT>
__device__ __forceinline__ void q8_half_quad(const uint8_t *q, const uint8_t *xr, int h, int xstr,
                                             float (&out)[MT]) {
  uint32_t D[17];
#pragma unroll
  for (int i = 0; i < 17; i++) D[i] = *(const uint32_t *)(q + 4 * i);
  float acc[MT];
  float dsum[MT];  // sum over blocks of d_b * (32-column sum of x)
#pragma unroll
  for (int m = 0; m < MT; m++) acc[m] = dsum[m] = 0.f;
#pragma unroll
  for (int bb = 0; bb < 2; bb++) {
    // block bb of the half starts at byte 34 bb: dword 8 bb, at byte 0 of it
    // (bb = 0) or byte 2 (bb = 1)
    const int w0 = 8 * bb, b = 2 * h + bb;
    uint32_t cw[8];
    float d;
    if (bb == 0) {
      d = half_bits_to_float(D[w0]);
#pragma unroll
      for (int c = 0; c < 8; c++) cw[c] = __builtin_amdgcn_alignbyte(D[w0 + c + 1], D[w0 + c], 2);
    } else {
      d = half_bits_to_float(D[w0] >> 16);
#pragma unroll
      for (int c = 0; c < 8; c++) cw[c] = D[w0 + 1 + c];
    }
    q8_block<MT>(cw, d, xr + 128 * b, xstr, acc);
#pragma unroll
    for (int m = 0; m < MT; m++)
      dsum[m] = fmaf(d, *(const float *)(xr + m * xstr + 512 + 4 * b), dsum[m]);
  }
#pragma unroll
  for (int m = 0; m < MT; m++) out[m] = fmaf(-128.f, dsum[m], acc[m]);
}

// One launch: rows of this workgroup, columns kc0 .. kc0+kcn-1 (the whole row
// when kcn == K). Rows r0 .. r1-1 of the workgroup occupy (r1 - r0) * segb
// bytes of "virtual" span space, segment r holding row r0 + r's chunk; a span
// crosses at most one segment boundary (segb >= span bytes, or the segments
// are whole, consecutive rows).
// floor(v / d) for 0 <= v < 2^16 and 2 <= d < 2^16 with magic = ceil(2^32 / d)
// (here d = K/128 quads per row is at least 2):
// the error of magic * v / 2^32 against v / d is below v / 2^32 < 1 / d.
__device__ __forceinline__ int q8_div(int v, uint32_t magic) {
  return (int)__umulhi((uint32_t)v, magic);
}

// XC: x tasks per thread, all loaded before the first weight load (loads
// complete in order, so an x load issued behind weight loads would wait for
// them).
template <bool XBF16, int MT, int XC, int WAVES>
__global__ __launch_bounds__(WAVES * WAVE) void q80_gemv_kernel(
    const uint8_t *__restrict__ w, const void *__restrict__ x, float *__restrict__ y, int K,
    int ldx, int ldy, int kc0, int kcn, int rows_q, int rows_rem, int pq, uint32_t qpr_magic,
    int accumulate) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  __shared__ int next_span;
  const int qpr = kcn / 128;                                  // quads per row in the chunk
  const int xstr = qpr * Q8_XREC;                             // bytes per token's records
  constexpr int Q8_THREADS = WAVES * WAVE;
  uint8_t *spanbuf = smem;                                    // [waves][Q8_NCH KiB]
  uint8_t *xrec = smem + WAVES * Q8_SPAN_BUF;                 // [MT][qpr][528]
  float *part = (float *)(xrec + MT * xstr);                  // [MT][pq]

  const int bid = blockIdx.x;
  const int r0 = bid * rows_q + min(bid, rows_rem);
  const int r1 = r0 + rows_q + (bid < rows_rem ? 1 : 0);
  const int nquads = (r1 - r0) * qpr;
  const int rb = (K / 32) * Q80_BYTES;                        // bytes per row
  const int segb = qpr * Q8_QUAD;                             // bytes per row chunk
  const int gap = rb - segb;                                  // 0 for whole rows
  const int vtotal = (r1 - r0) * segb;                        // < 2^31: the quads fit LDS
  const int nspan = (nquads + Q8_SPAN - 1) / Q8_SPAN;
  const uint8_t *wbase = w + (int64_t)r0 * rb + (int64_t)(kc0 / 32) * Q80_BYTES;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

  // Virtual byte v of segment s is physical byte v + s * gap. Span si past
  // the end reloads the last span (already on its way), so every wave issues
  // the same loads in every iteration. A full span inside one segment takes
  // plain loads; otherwise chunks past the end re-read the span's last 16
  // bytes and chunks past the segment boundary take the next segment's offset.
  // Both branches load the same registers, so waits count exactly.
  auto issue = [&](Q8Span &sp, int sidx) {
    const int si = __builtin_amdgcn_readfirstlane(min(sidx, nspan - 1));
    const int v0 = si * Q8_SPAN_BYTES;
    const int vend = min(v0 + Q8_SPAN_BYTES, vtotal);
    const int seg = v0 / segb;
    const int bnd = (seg + 1) * segb;
    const int ph0 = seg * gap;
    if (vend == v0 + Q8_SPAN_BYTES && (gap == 0 || vend <= bnd)) {
      const uint8_t *p = wbase + (v0 + ph0) + 16 * lane;
#pragma unroll
      for (int j = 0; j < Q8_NCH; j++) {
        const int off = min(1024 * j + 16 * lane, Q8_SPAN_BYTES - 16) - 16 * lane;
        sp.r[j] = __builtin_nontemporal_load((const u32x4 *)(p + off));
      }
    } else {
#pragma unroll
      for (int j = 0; j < Q8_NCH; j++) {
        const int v = min(v0 + 1024 * j + 16 * lane, vend - 16);
        const int ph = v < bnd ? ph0 : ph0 + gap;
        sp.r[j] = __builtin_nontemporal_load((const u32x4 *)(wbase + (v + ph)));
      }
    }
  };
  auto grab = [&]() {
    int v = 0;
    if (lane == 0) v = atomicAdd(&next_span, 1);
    return __builtin_amdgcn_readfirstlane(v);
  };

  // x loads, the first span, the x records (storing waits for the x loads
  // only), then the second span: x does not queue behind both spans. Tasks
  // past the end re-read the last task and store nothing.
  const int tpt = kcn / 4;
  const int ntask = MT * tpt;
  Q8XTask<XBF16> xt[XC];
#pragma unroll
  for (int i = 0; i < XC; i++) {
    const int task = min(i * Q8_THREADS + (int)threadIdx.x, ntask - 1);
    xt[i].load(x, ldx, kc0, tpt, task);
  }
  if (threadIdx.x == 0) next_span = Q8_NB * WAVES;
  int sidx[Q8_NB];
#pragma unroll
  for (int b = 0; b < Q8_NB; b++) sidx[b] = b * WAVES + wave;
  Q8Span R[Q8_NB];
  issue(R[0], sidx[0]);
#pragma unroll
  for (int i = 0; i < XC; i++) {
    if (i * Q8_THREADS < ntask) {  // uniform
      const int task = i * Q8_THREADS + (int)threadIdx.x;
      xt[i].store(xrec, xstr, tpt, task, task < ntask);
    }
  }
#pragma unroll
  for (int b = 1; b < Q8_NB; b++) issue(R[b], sidx[b]);
  __syncthreads();

  uint8_t *mybuf = spanbuf + wave * Q8_SPAN_BUF;
  const int h = lane & 1;
  auto more = [&]() {
    bool m = false;
#pragma unroll
    for (int b = 0; b < Q8_NB; b++) m |= sidx[b] < nspan;
    return m;
  };
  while (more()) {
#pragma unroll
    for (int p = 0; p < Q8_NB; p++) {
      const int cur = sidx[p];
      const int nbytes = cur < nspan ? min(Q8_SPAN_BYTES, vtotal - cur * Q8_SPAN_BYTES) : 0;
#pragma unroll
      for (int j = 0; j < Q8_NCH; j++) {
        const int off = 1024 * j + 16 * lane;
        if (off < nbytes) *(u32x4 *)(mybuf + off) = R[p].r[j];
      }
      // refill this slot right away: the other spans stay in flight during the math
      const int nxt = cur < nspan ? grab() : nspan;
      issue(R[p], nxt);
      sidx[p] = nxt;
      // lanes 2i and 2i + 1 share quad i: half h is blocks 2h and 2h + 1, and
      // the halves are added in a fixed order
      const int g = Q8_SPAN * cur + (lane >> 1);
      float o[MT];
#pragma unroll
      for (int m = 0; m < MT; m++) o[m] = 0.f;
      if (cur < nspan && g < nquads) {
        const int qc = g - q8_div(g, qpr_magic) * qpr;
        q8_half_quad<MT>(mybuf + Q8_QUAD * (lane >> 1) + 68 * h, xrec + qc * Q8_XREC, h, xstr,
                         o);
      }
#pragma unroll
      for (int m = 0; m < MT; m++) o[m] += __shfl_xor(o[m], 1, WAVE);
      if (cur < nspan && g < nquads && h == 0) {
#pragma unroll
        for (int m = 0; m < MT; m++) part[m * pq + g] = o[m];
      }
    }
  }
  __syncthreads();

  // Row sums: one thread per (token, row), four interleaved partial sums
  // (independent LDS loads and adds), combined in a fixed order.
  const int nrows = r1 - r0;
  for (int t = threadIdx.x; t < MT * nrows; t += Q8_THREADS) {
    const int m = t / nrows, r = t - m * nrows;
    const float *pp = part + m * pq + r * qpr;  // qpr is even
    float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
    int k = 0;
    for (; k + 4 <= qpr; k += 4) {
      s0 += pp[k];
      s1 += pp[k + 1];
      s2 += pp[k + 2];
      s3 += pp[k + 3];
    }
    for (; k < qpr; k += 2) {
      s0 += pp[k];
      s1 += pp[k + 1];
    }
    const float sacc = (s0 + s1) + (s2 + s3);
    float *yo = y + (int64_t)m * ldy + r0 + r;
    *yo = accumulate ? *yo + sacc : sacc;
  }
}

size_t q8_lds(int waves, int mt, int64_t kcn, int64_t pq) {
  return (size_t)waves * Q8_SPAN_BUF + (size_t)mt * (kcn / 128) * Q8_XREC +
         (size_t)mt * pq * 4;
}

// Workgroups for N rows: one per compute unit, more when a workgroup's quad
// slots would not fit beside the spans and x. False if nothing fits.
bool q8_plan(int waves, int mt, int64_t N, int64_t kcn, int64_t &nwg, int &rows_q,
             int &rows_rem, int &pq, size_t &lds) {
  const int64_t qpr = kcn / 128;
  const size_t fixed = q8_lds(waves, mt, kcn, 0);
  if (fixed + (size_t)mt * 2 * qpr * 4 > Q8_LDS_LIMIT) return false;
  const int64_t cap_rows = (int64_t)((Q8_LDS_LIMIT - fixed) / ((size_t)mt * qpr * 4)) - 1;
  nwg = Q8_TARGET_WGS;
  const int64_t need = (N + cap_rows - 1) / cap_rows;
  if (need > nwg) nwg = need;
  if (nwg > N) nwg = N;
  rows_q = (int)(N / nwg);
  rows_rem = (int)(N % nwg);
  pq = (int)((rows_q + (rows_rem ? 1 : 0)) * qpr);
  lds = q8_lds(waves, mt, kcn, pq);
  return lds <= Q8_LDS_LIMIT;
}

template <bool XBF16, int MT, int XC, int WAVES>
void q8_launch_xc(const void *w, const void *x, float *y, int64_t N, int64_t K, int64_t ldy,
                  int64_t kc0, int64_t kcn, bool accumulate, hipStream_t s) {
  int64_t nwg;
  int rows_q, rows_rem, pq;
  size_t lds;
  if (!q8_plan(WAVES, MT, N, kcn, nwg, rows_q, rows_rem, pq, lds)) return;  // checked before
  auto kern = q80_gemv_kernel<XBF16, MT, XC, WAVES>;
  (void)hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)lds);
  const uint32_t qpr = (uint32_t)(kcn / 128);
  const uint32_t magic = (uint32_t)((((uint64_t)1 << 32) + qpr - 1) / qpr);
  hipLaunchKernelGGL(kern, dim3((unsigned)nwg), dim3(WAVES * WAVE), lds, s, (const uint8_t *)w, x,
                     y, (int)K, (int)K, (int)ldy, (int)kc0, (int)kcn, rows_q, rows_rem, pq, magic,
                     accumulate ? 1 : 0);
}

// The smallest instantiated task count per thread that covers MT * kcn / 4
// tasks. The LDS plan bounds MT * kcn by (160 KiB - spans) / 4.125 bytes per
// column, about 31K, i.e. at most 31 tasks per thread (4 waves).
template <bool XBF16, int MT, int WAVES>
void q8_launch_w(const void *w, const void *x, float *y, int64_t N, int64_t K, int64_t ldy,
                 int64_t kc0, int64_t kcn, bool accumulate, hipStream_t s) {
  const int64_t need = (MT * kcn / 4 + WAVES * WAVE - 1) / (WAVES * WAVE);
  if (need <= 4)
    q8_launch_xc<XBF16, MT, 4, WAVES>(w, x, y, N, K, ldy, kc0, kcn, accumulate, s);
  else if (need <= 8)
    q8_launch_xc<XBF16, MT, 8, WAVES>(w, x, y, N, K, ldy, kc0, kcn, accumulate, s);
  else if (WAVES == 8 || need <= 16)  // 8 waves: x is at most about 21K columns
    q8_launch_xc<XBF16, MT, 16, WAVES>(w, x, y, N, K, ldy, kc0, kcn, accumulate, s);
  else if constexpr (WAVES == 4)
    q8_launch_xc<XBF16, MT, 32, WAVES>(w, x, y, N, K, ldy, kc0, kcn, accumulate, s);
}

// One token per launch takes 8 waves (more spans in flight; measured faster
// for decode-sized tensors) when that still makes one workgroup per compute
// unit; several tokens (more registers per lane) and larger tensors take 4.
template <bool XBF16, int MT>
void q8_launch(const void *w, const void *x, float *y, int64_t N, int64_t K, int64_t ldy,
               int64_t kc0, int64_t kcn, bool accumulate, hipStream_t s) {
  int64_t nwg;
  int rq, rr, pq;
  size_t lds;
  if constexpr (MT == 1) {
    if (kcn / 4 <= 16 * 8 * WAVE && q8_plan(8, MT, N, kcn, nwg, rq, rr, pq, lds) &&
        nwg <= Q8_TARGET_WGS) {
      q8_launch_w<XBF16, MT, 8>(w, x, y, N, K, ldy, kc0, kcn, accumulate, s);
      return;
    }
  }
  q8_launch_w<XBF16, MT, 4>(w, x, y, N, K, ldy, kc0, kcn, accumulate, s);
}

// Column chunks for mt tokens: the fewest equal chunks (multiples of 256
// columns, widths within 256 of each other) whose widest one fits; 1 when K
// fits whole, 0 when no split with chunks of at least Q8_MIN_CHUNK fits.
int q8_nchunks(int mt, int64_t N, int64_t K) {
  int64_t nwg;
  int rq, rr, pq;
  size_t lds;
  const int64_t units = K / 256;
  for (int nch = 1; nch <= units; nch++) {
    const int64_t widest = (units + nch - 1) / nch * 256, narrowest = units / nch * 256;
    if (nch > 1 && narrowest < Q8_MIN_CHUNK) return 0;
    if (q8_plan(4, mt, N, widest, nwg, rq, rr, pq, lds)) return nch;
  }
  return 0;
}

template <bool XBF16, int MT>
void q8_tokens(const void *w, const void *x, float *y, int64_t N, int64_t K, int nch,
               hipStream_t s) {
  const int64_t units = K / 256;
  int64_t kc0 = 0;
  for (int c = 0; c < nch; c++) {
    const int64_t n = (units / nch + (c < units % nch ? 1 : 0)) * 256;
    q8_launch<XBF16, MT>(w, x, y, N, K, N, kc0, n, c > 0, s);
    kc0 += n;
  }
}

template <bool XBF16>
void q8_gemv(const void *w, const void *x, float *y, int64_t M, int64_t N, int64_t K,
             hipStream_t s) {
  const size_t elt = XBF16 ? 2 : 4;
  int64_t m0 = 0;
  while (m0 < M) {
    // the most tokens per launch whose x fits without splitting K, else one
    int mt = 8;
    while (mt > 1 && (mt > M - m0 || q8_nchunks(mt, N, K) != 1)) mt >>= 1;
    const int nch = q8_nchunks(mt, N, K);
    const void *xm = (const char *)x + (size_t)m0 * K * elt;
    float *ym = y + m0 * N;
    switch (mt) {
      case 8: q8_tokens<XBF16, 8>(w, xm, ym, N, K, nch, s); break;
      case 4: q8_tokens<XBF16, 4>(w, xm, ym, N, K, nch, s); break;
      case 2: q8_tokens<XBF16, 2>(w, xm, ym, N, K, nch, s); break;
      default: q8_tokens<XBF16, 1>(w, xm, ym, N, K, nch, s); break;
    }
    m0 += mt;
  }
}

// Bit-exact dequantization: one thread per 8 weights (a quarter block); the
// fields sit at even offsets, so they are read as 16-bit words.
__global__ __launch_bounds__(256) void q80_dequant_kernel(const uint8_t *__restrict__ w,
                                                          float *__restrict__ out,
                                                          int64_t nblocks) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t blk = t >> 2;
  if (blk >= nblocks) return;
  const int part = (int)(t & 3);
  const uint16_t *B = (const uint16_t *)(w + blk * Q80_BYTES);
  const float d = half_bits_to_float(B[0]);
  f32x4 r0, r1;
#pragma unroll
  for (int h = 0; h < 4; h++) {
    const uint32_t two = B[1 + 4 * part + h];  // codes 8 part + 2h, 8 part + 2h + 1
    const float a = d * (float)(int8_t)(two & 255u), b = d * (float)(int8_t)(two >> 8);
    if (h < 2) {
      r0[2 * h] = a;
      r0[2 * h + 1] = b;
    } else {
      r1[2 * h - 4] = a;
      r1[2 * h - 3] = b;
    }
  }
  f32x4 *o = (f32x4 *)(out + blk * 32 + 8 * part);
  o[0] = r0;
  o[1] = r1;
}

}  // namespace

bool q80_gemv_fits(int64_t N, int64_t K) { return q8_nchunks(1, N, K) > 0; }

// bf16 x with M >= 2: the matrix-core GEMV (weights rounded to bf16 once);
// the kernel here spends M FMAs per code (59.8 us at M = 8 for the QKV shape).
void launch_q80_gemv(const void *w, const void *x, bool x_bf16, float *y, int64_t M, int64_t N,
                     int64_t K, hipStream_t s) {
  if (x_bf16 && M >= 2 && ((uintptr_t)w & 15) == 0) {
    launch_q80_mfma_gemv(w, (const uint16_t *)x, y, M, N, K, s);
    return;
  }
  if (x_bf16)
    q8_gemv<true>(w, x, y, M, N, K, s);
  else
    q8_gemv<false>(w, x, y, M, N, K, s);
}

void launch_q80_dequantize(const void *w, float *out, int64_t N, int64_t K, hipStream_t s) {
  const int64_t nblocks = N * (K / 32);
  const int64_t threads = nblocks * 4;
  hipLaunchKernelGGL(q80_dequant_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0,
                     s, (const uint8_t *)w, out, nblocks);
}

}  // namespace qdm
