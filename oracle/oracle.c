/*
 * CPU oracle for the GGUF k-quant (Q4_K, Q5_K, Q6_K) and Q8_0
 * dequantize-fused matmul and the top-k router in front of its MoE grouped
 * matmul.
 *
 * TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the benchmark's
 * CPU-baseline leg may load this library. It shares no code, header or table
 * with the HIP library; it is written from the format definitions alone and is
 * deliberately plain: no blocking, no fusion, no reordering.
 *
 * What the method computes (hipEngine README, "GGUF Support": the GGUF path
 * reads Q4_K / Q6_K tensors with its own quant readers and multiplies with
 * them; "Quickstart": WMMA prefill and GEMV decode over the same weights) is,
 * exactly, a dense matmul with the dequantized weights. So the oracle is that
 * definition: dequantize every weight to fp32 with the format's formula, then
 * accumulate X * W^T in float64, in increasing k.
 *
 * Formats (little-endian; 256 weights per super-block; a weight tensor has N
 * rows of K/256 consecutive super-blocks):
 *
 * Q4_K, 144 bytes: fp16 d @0, fp16 dmin @2, 12 packed bytes S @4, 128 code
 *   bytes Q @16. Eight sub-blocks of 32 weights, each with a 6-bit scale sc_j
 *   and a 6-bit min m_j:
 *     S[0..3]  low 6 bits: sc_0..sc_3        top 2 bits: high bits of sc_4..sc_7
 *     S[4..7]  low 6 bits: m_0..m_3          top 2 bits: high bits of m_4..m_7
 *     S[8..11] low nibble: low 4 bits of sc_4..sc_7
 *              high nibble: low 4 bits of m_4..m_7
 *   32-byte chunk c of Q gives its low nibbles to sub-block 2c and its high
 *   nibbles to sub-block 2c+1 (weight l of a sub-block sits in byte 32c+l).
 *   w = d*sc_j*q - dmin*m_j.
 *
 * Q5_K, 176 bytes (a reading: the pages name the type and its share of a
 *   Q4_K_M file only): the Q4_K header (fp16 d @0, fp16 dmin @2, the same 12
 *   packed scale/min bytes @4), a high-bit plane QH @16 (32 B) and the Q4_K
 *   code bytes Q @48 (128 B). Weight l of sub-block j takes its low 4 bits as
 *   in Q4_K and its fifth bit from bit j of QH[l]: q = lo | hi << 4 in 0..31.
 *   w = d*sc_j*q - dmin*m_j.
 *
 * Q6_K, 210 bytes: low-nibble plane QL @0 (128 B), high-2-bit plane QH @128
 *   (64 B), sixteen int8 scales @192 (one per 16 weights), fp16 d @208.
 *   Placement of the code bits (a reading; the pages name the type only):
 *   weight i of the block, with h = i/128, r = i%128, g = r/32, l = r%32,
 *   takes its low 4 bits from QL[64h + 32(g%2) + l] (low nibble if g < 2,
 *   high nibble otherwise) and its high 2 bits from bits 2g..2g+1 of
 *   QH[32h + l]. q = lo | hi << 4 in 0..63;  w = d*scale[i/16]*(q - 32).
 *
 * Q8_0, 34 bytes per 32 weights (a reading: the pages name the type and its
 *   share of a Q4_K_M file only): fp16 d @0, then 32 int8 codes q[i] @2+i
 *   (two's complement); w = d*q[i]. A tensor row is K/32 consecutive blocks.
 *
 * fp32 exactness of the dequant (why one fp32 formula is the reference):
 *   every product here is exact in fp32 (Q4_K d*sc*q has at most 11+6+4 = 21
 *   significant bits, Q5_K d*sc*q at most 11+6+5 = 22, dmin*m at most 17;
 *   Q6_K d*scale*(q-32) at most 11+7+5, Q8_0 d*q at most 11+7), so a Q4_K or Q5_K weight is the
 *   single correctly rounded value of the exact d*sc*q - dmin*m, whatever the
 *   evaluation order or FMA contraction, and the Q6_K and Q8_0 weights are
 *   exact. Any
 *   correct fp32 implementation is bit-identical.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define QK 256
#define Q4K_BYTES 144
#define Q5K_BYTES 176
#define Q6K_BYTES 210
#define Q80_WEIGHTS 32
#define Q80_BYTES 34

/* IEEE 754 binary16 -> float, from the definition:
 *   e in 1..30: (-1)^s 2^(e-15) (1 + m/1024);  e = 0: (-1)^s 2^-14 (m/1024). */
static float fp16_value(uint16_t h)
{
    int s = h >> 15, e = (h >> 10) & 31, m = h & 1023;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + m), e - 25);
    return (float)(s ? -v : v); /* exact: 11 significant bits */
}

/* bf16 -> float: the bf16 bits are the top half of the fp32 pattern. */
static float bf16_value(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* The 6-bit scales and mins of the eight sub-blocks (Q4_K and Q5_K). */
static void kq_scales_mins(const uint8_t *S, int *sc, int *mn)
{
    for (int j = 0; j < 4; j++) {
        sc[j] = S[j] & 63;
        mn[j] = S[j + 4] & 63;
    }
    for (int j = 4; j < 8; j++) {
        sc[j] = (S[j + 4] & 15) | ((S[j - 4] >> 6) << 4);
        mn[j] = (S[j + 4] >> 4) | ((S[j] >> 6) << 4);
    }
}

/* w = d*sc_j*q - dmin*m_j for the 256 codes q[i] (sub-block j = i/32). */
static void kq_apply(const uint8_t *B, const int *q, float *w)
{
    const float d = fp16_value((uint16_t)(B[0] | B[1] << 8));
    const float dmin = fp16_value((uint16_t)(B[2] | B[3] << 8));
    int sc[8], mn[8];
    kq_scales_mins(B + 4, sc, mn);
    for (int i = 0; i < QK; i++) {
        int j = i / 32;
        float a = d * (float)sc[j];    /* exact */
        float aq = a * (float)q[i];    /* exact */
        float b = dmin * (float)mn[j]; /* exact */
        w[i] = aq - b;                 /* the one rounding */
    }
}

static void q4k_block_dequant(const uint8_t *B, float *w)
{
    const uint8_t *Q = B + 16;
    int q[QK];
    for (int i = 0; i < QK; i++) {
        int j = i / 32, l = i % 32;
        q[i] = (Q[32 * (j / 2) + l] >> (4 * (j % 2))) & 15;
    }
    kq_apply(B, q, w);
}

static void q5k_block_dequant(const uint8_t *B, float *w)
{
    const uint8_t *QH = B + 16, *Q = B + 48;
    int q[QK];
    for (int i = 0; i < QK; i++) {
        int j = i / 32, l = i % 32;
        int lo = (Q[32 * (j / 2) + l] >> (4 * (j % 2))) & 15;
        int hi = (QH[l] >> j) & 1;
        q[i] = lo | (hi << 4);
    }
    kq_apply(B, q, w);
}

static void q6k_block_dequant(const uint8_t *B, float *w)
{
    const uint8_t *QL = B, *QH = B + 128;
    const int8_t *SC = (const int8_t *)(B + 192);
    const float d = fp16_value((uint16_t)(B[208] | B[209] << 8));
    for (int i = 0; i < QK; i++) {
        int h = i / 128, r = i % 128, g = r / 32, l = r % 32;
        int lo = (QL[64 * h + 32 * (g % 2) + l] >> (4 * (g / 2))) & 15;
        int hi = (QH[32 * h + l] >> (2 * g)) & 3;
        int q = lo | (hi << 4);
        float a = d * (float)SC[i / 16]; /* exact */
        w[i] = a * (float)(q - 32);      /* exact */
    }
}

/* Dequantize a whole tensor: blocks [N][K/256] -> out fp32 [N][K]. */
void oracle_q4k_dequantize(const uint8_t *blocks, int64_t N, int64_t K, float *out)
{
    const int64_t nb = K / QK;
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; n++)
        for (int64_t b = 0; b < nb; b++)
            q4k_block_dequant(blocks + (n * nb + b) * Q4K_BYTES, out + n * K + b * QK);
}

void oracle_q5k_dequantize(const uint8_t *blocks, int64_t N, int64_t K, float *out)
{
    const int64_t nb = K / QK;
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; n++)
        for (int64_t b = 0; b < nb; b++)
            q5k_block_dequant(blocks + (n * nb + b) * Q5K_BYTES, out + n * K + b * QK);
}

/* Q8_0: w[i] = d * q[i], q[i] the int8 at byte 2 + i. */
static void q80_block_dequant(const uint8_t *B, float *w)
{
    const float d = fp16_value((uint16_t)(B[0] | B[1] << 8));
    for (int i = 0; i < Q80_WEIGHTS; i++)
        w[i] = d * (float)(int8_t)B[2 + i]; /* exact */
}

void oracle_q80_dequantize(const uint8_t *blocks, int64_t N, int64_t K, float *out)
{
    const int64_t nb = K / Q80_WEIGHTS;
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; n++)
        for (int64_t b = 0; b < nb; b++)
            q80_block_dequant(blocks + (n * nb + b) * Q80_BYTES,
                              out + n * K + b * Q80_WEIGHTS);
}

void oracle_q6k_dequantize(const uint8_t *blocks, int64_t N, int64_t K, float *out)
{
    const int64_t nb = K / QK;
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; n++)
        for (int64_t b = 0; b < nb; b++)
            q6k_block_dequant(blocks + (n * nb + b) * Q6K_BYTES, out + n * K + b * QK);
}

/* Activations X [M][K]: x_is_bf16 = 1 for bf16 bit patterns, 0 for fp32. */
static void widen_x(const void *x, int x_is_bf16, int64_t M, int64_t K, double *xd)
{
    for (int64_t i = 0; i < M * K; i++)
        xd[i] = x_is_bf16 ? (double)bf16_value(((const uint16_t *)x)[i])
                          : (double)((const float *)x)[i];
}

/* Y [M][N] float64 = X [M][K] * W^T for a quantized W [N][K].
 * qtype 4 = Q4_K, 5 = Q5_K, 6 = Q6_K (K % 256 == 0), 8 = Q8_0 (K % 32 == 0).
 * Each row of W is dequantized once into fp32, then
 * Y[m][n] = sum_k X[m][k] * W[n][k] in float64, k increasing. */
int oracle_qmatmul(int qtype, const uint8_t *blocks, const void *x, int x_is_bf16,
                   int64_t M, int64_t N, int64_t K, double *y)
{
    if (qtype != 4 && qtype != 5 && qtype != 6 && qtype != 8)
        return -1;
    const int64_t qk = qtype == 8 ? Q80_WEIGHTS : QK;
    if (K % qk || M < 0 || N < 0)
        return -1;
    const int64_t nb = K / qk;
    const int64_t bb = qtype == 4   ? Q4K_BYTES
                       : qtype == 5 ? Q5K_BYTES
                       : qtype == 6 ? Q6K_BYTES
                                    : Q80_BYTES;
    double *xd = (double *)malloc(sizeof(double) * (size_t)(M * K > 0 ? M * K : 1));
    if (!xd)
        return -2;
    widen_x(x, x_is_bf16, M, K, xd);
#pragma omp parallel
    {
        float *w = (float *)malloc(sizeof(float) * (size_t)K);
#pragma omp for schedule(static)
        for (int64_t n = 0; n < N; n++) {
            for (int64_t b = 0; b < nb; b++) {
                const uint8_t *blk = blocks + (n * nb + b) * bb;
                if (qtype == 4)
                    q4k_block_dequant(blk, w + b * qk);
                else if (qtype == 5)
                    q5k_block_dequant(blk, w + b * qk);
                else if (qtype == 6)
                    q6k_block_dequant(blk, w + b * qk);
                else
                    q80_block_dequant(blk, w + b * qk);
            }
            for (int64_t m = 0; m < M; m++) {
                double acc = 0.0;
                for (int64_t k = 0; k < K; k++)
                    acc += xd[m * K + k] * (double)w[k];
                y[m * N + n] = acc;
            }
        }
        free(w);
    }
    free(xd);
    return 0;
}

static double silu(double z) { return z / (1.0 + exp(-z)); }

/*
 * Routed MoE FFN with Q4_K gate+up experts, in float64.
 *   x      [T][H]  activations (bf16 bits or fp32)
 *   w13    [E][2F][H/256] Q4_K blocks: rows 0..F-1 are the gate projection,
 *          rows F..2F-1 the up projection (concatenated)
 *   w2     [E][H][F/256] blocks of type down_qtype (4 = Q4_K, 5 = Q5_K): the
 *          down projection
 *   ids    [T][top_k] expert index per (token, slot), distinct within a row
 *   gw     [T][top_k] fp32 gate weight per (token, slot)
 *   y      [T][H] float64 output
 * For each token t and slot s with e = ids[t][s]:
 *   u = W13[e] x_t (2F values), h_f = silu(u_f) * u_{F+f}, o = W2[e] h,
 * and y_t = sum over s, in slot order, of gw[t][s] * o. Everything after the
 * fp32 dequant is float64; silu(z) = z / (1 + exp(-z)).
 * Returns 0, or -1 for bad sizes / out-of-range ids.
 */
int oracle_moe(const void *x, int x_is_bf16, const uint8_t *w13, const uint8_t *w2,
               int down_qtype, const int32_t *ids, const float *gw, int64_t T, int64_t E,
               int64_t top_k, int64_t H, int64_t F, double *y)
{
    if (H % QK || F % QK || T < 0 || E <= 0 || top_k <= 0 ||
        (down_qtype != 4 && down_qtype != 5))
        return -1;
    const int64_t b2 = down_qtype == 4 ? Q4K_BYTES : Q5K_BYTES;
    for (int64_t i = 0; i < T * top_k; i++)
        if (ids[i] < 0 || ids[i] >= E)
            return -1;
    const int64_t nbH = H / QK, nbF = F / QK;
    double *xd = (double *)malloc(sizeof(double) * (size_t)(T * H > 0 ? T * H : 1));
    double *o = (double *)calloc((size_t)(T * top_k * H > 0 ? T * top_k * H : 1), sizeof(double));
    float *W13 = (float *)malloc(sizeof(float) * (size_t)(2 * F * H));
    float *W2 = (float *)malloc(sizeof(float) * (size_t)(H * F));
    if (!xd || !o || !W13 || !W2) {
        free(xd); free(o); free(W13); free(W2);
        return -2;
    }
    widen_x(x, x_is_bf16, T, H, xd);
    /* Expert by expert: dequantize its two tensors once, then compute the
     * expert output o[t][s] of every (token, slot) routed to it. */
    for (int64_t e = 0; e < E; e++) {
        int used = 0;
        for (int64_t i = 0; i < T * top_k && !used; i++)
            used = ids[i] == e;
        if (!used)
            continue;
        oracle_q4k_dequantize(w13 + e * 2 * F * nbH * Q4K_BYTES, 2 * F, H, W13);
        if (down_qtype == 4)
            oracle_q4k_dequantize(w2 + e * H * nbF * b2, H, F, W2);
        else
            oracle_q5k_dequantize(w2 + e * H * nbF * b2, H, F, W2);
#pragma omp parallel
        {
            double *u = (double *)malloc(sizeof(double) * (size_t)(2 * F));
            double *hbuf = (double *)malloc(sizeof(double) * (size_t)F);
#pragma omp for schedule(dynamic)
            for (int64_t i = 0; i < T * top_k; i++) {
                if (ids[i] != e)
                    continue;
                const double *xt = xd + (i / top_k) * H;
                for (int64_t r = 0; r < 2 * F; r++) {
                    double acc = 0.0;
                    for (int64_t k = 0; k < H; k++)
                        acc += xt[k] * (double)W13[r * H + k];
                    u[r] = acc;
                }
                for (int64_t f = 0; f < F; f++)
                    hbuf[f] = silu(u[f]) * u[F + f];
                double *ot = o + i * H;
                for (int64_t r = 0; r < H; r++) {
                    double acc = 0.0;
                    for (int64_t f = 0; f < F; f++)
                        acc += (double)W2[r * F + f] * hbuf[f];
                    ot[r] = acc;
                }
            }
            free(u);
            free(hbuf);
        }
    }
    for (int64_t t = 0; t < T; t++)
        for (int64_t r = 0; r < H; r++) {
            double acc = 0.0;
            for (int64_t s = 0; s < top_k; s++)
                acc += (double)gw[t * top_k + s] * o[(t * top_k + s) * H + r];
            y[t * H + r] = acc;
        }
    free(xd); free(o); free(W13); free(W2);
    return 0;
}

int oracle_moe_q4k(const void *x, int x_is_bf16, const uint8_t *w13, const uint8_t *w2,
                   const int32_t *ids, const float *gw, int64_t T, int64_t E,
                   int64_t top_k, int64_t H, int64_t F, double *y)
{
    return oracle_moe(x, x_is_bf16, w13, w2, 4, ids, gw, T, E, top_k, H, F, y);
}

/*
 * MoE router: top-k selection and softmax from router logits (a reading: the
 * pages name a routed MoE model but not its router). For each token t the k
 * experts with the largest logits are taken, largest first; of equal logits
 * the smaller expert index comes first. The gate weights are the softmax of
 * the selected logits, in float64:
 *   w_s = exp(l_s - l_0) / sum_{j<k} exp(l_j - l_0),  l_0 the largest.
 * logits [T][E] fp32 (finite), ids [T][k] int32, w [T][k] float64.
 * Returns 0, or -1 for bad sizes (k < 1 or k > E).
 */
int oracle_router_topk(const float *logits, int64_t T, int64_t E, int64_t k, int32_t *ids,
                       double *w)
{
    if (T < 0 || E < 1 || k < 1 || k > E)
        return -1;
    char *taken = (char *)malloc((size_t)E);
    if (!taken)
        return -2;
    for (int64_t t = 0; t < T; t++) {
        const float *l = logits + t * E;
        memset(taken, 0, (size_t)E);
        for (int64_t s = 0; s < k; s++) {
            int64_t best = -1;
            for (int64_t e = 0; e < E; e++)
                if (!taken[e] && (best < 0 || l[e] > l[best]))
                    best = e; /* strict '>': the first of equal logits stays */
            taken[best] = 1;
            ids[t * k + s] = (int32_t)best;
        }
        const double l0 = (double)l[ids[t * k]];
        double sum = 0.0;
        for (int64_t s = 0; s < k; s++)
            sum += exp((double)l[ids[t * k + s]] - l0);
        for (int64_t s = 0; s < k; s++)
            w[t * k + s] = exp((double)l[ids[t * k + s]] - l0) / sum;
    }
    free(taken);
    return 0;
}
