/*
 * csa2_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, scalar CPU oracle of the CSA2 decode path (compressed sparse
 * attention as described for DeepSeek-V4 / V4.1-Flash).  Only the test suite,
 * the smoke check and the benchmark's CPU-baseline leg may load it; the HIP
 * library never does, and the two share no code.
 *
 * Every function follows the plain definition of what it computes:
 *   - element codecs E2M1 (FP4), E4M3 (FP8) and E8M0 written from the format
 *     definitions (OCP 8-bit floating point and Microscaling v1.0 specs);
 *   - the three entry formats of the pages: FP4 main latent KV with one E4M3
 *     scale per 16 channels (288 B), MXFP4 indexer keys with one E8M0 scale
 *     per 32 channels (68 B) [V4.1-Flash architecture page, "890 bytes/token"
 *     section; KV-cache-diet page, "890 ... 10,324" section], and the 8-bit
 *     sliding-window KV [same pages: SWA kept in FP8];
 *   - the lightning-indexer score I = sum_h w_h * ReLU(q_h . K_s)
 *     [DeepSeek-V4 paper page, section 2.3.1, index-score equation], with the
 *     indexer dot product taken exactly in the FP4 domain and rounded once;
 *   - exact top-k with ties to the lower id [section 2.3.1, top-k selector];
 *   - joint softmax attention in fp64 over the selected entries and the
 *     sliding-window entries, with an optional sink logit [section 2.3.3].
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fno-fast-math -shared -fPIC.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------ */
/* Element codecs                                                      */
/* ------------------------------------------------------------------ */

/* E2M1: bit 3 sign, bits 2:1 exponent (bias 1), bit 0 mantissa.
 * Exponent field 0 is subnormal: 0.5 * m. */
double orc_e2m1_value(unsigned code)
{
    unsigned s = (code >> 3) & 1u, e = (code >> 1) & 3u, m = code & 1u;
    double mag = (e == 0) ? 0.5 * m : (1.0 + 0.5 * m) * ldexp(1.0, (int)e - 1);
    return s ? -mag : mag;
}

/* Round-to-nearest-even onto E2M1, saturating at 6; the sign bit is copied. */
unsigned orc_e2m1_encode(double x)
{
    unsigned sign = signbit(x) ? 8u : 0u;
    double a = fabs(x);
    if (a >= 6.0) return sign | 7u;
    if (a < 1.0) {                      /* subnormal spacing 0.5 */
        double q = nearbyint(a * 2.0);  /* 0, 1 or 2 (2 is the code of 1.0) */
        return sign | (unsigned)q;
    }
    int ex;
    frexp(a, &ex);
    int E = ex - 1;                     /* floor(log2 a): 0, 1 or 2 */
    double q = nearbyint(ldexp(a, 1 - E));   /* 2 .. 4 */
    if (q == 4.0) { E += 1; q = 2.0; }
    unsigned code = ((unsigned)(E + 1) << 1) | (unsigned)(q - 2.0);
    if (code > 7u) code = 7u;
    return sign | code;
}

/* E4M3 ("FN" variant): bias 7, no infinities, S.1111.111 is NaN. */
double orc_e4m3_value(unsigned code)
{
    unsigned s = (code >> 7) & 1u, e = (code >> 3) & 15u, m = code & 7u;
    double mag;
    if (e == 15u && m == 7u) return NAN;
    if (e == 0) mag = m * ldexp(1.0, -9);
    else mag = (1.0 + m / 8.0) * ldexp(1.0, (int)e - 7);
    return s ? -mag : mag;
}

/* Round-to-nearest-even onto E4M3, saturating at 448. */
unsigned orc_e4m3_encode(double x)
{
    unsigned sign = signbit(x) ? 0x80u : 0u;
    double a = fabs(x);
    if (a >= 448.0) return sign | 0x7Eu;
    if (a < ldexp(1.0, -6)) {           /* subnormal spacing 2^-9 */
        double q = nearbyint(a * 512.0);    /* 0 .. 8 (8 is the smallest normal) */
        return sign | (unsigned)q;
    }
    int ex;
    frexp(a, &ex);
    int E = ex - 1;                     /* -6 .. 8 */
    double q = nearbyint(ldexp(a, 3 - E));   /* 8 .. 16 */
    if (q == 16.0) { E += 1; q = 8.0; }
    unsigned code = ((unsigned)(E + 7) << 3) | (unsigned)(q - 8.0);
    if (code > 0x7Eu) code = 0x7Eu;
    return sign | code;
}

/* E8M0: 2^(code - 127); 255 is NaN. */
double orc_e8m0_value(unsigned code)
{
    if (code == 255u) return NAN;
    return ldexp(1.0, (int)code - 127);
}

/* floor(log2(a)) for a finite a > 0, exactly (from the binary exponent). */
static int floor_log2(double a)
{
    int ex;
    frexp(a, &ex);
    return ex - 1;
}

/* ------------------------------------------------------------------ */
/* Group quantisers                                                    */
/* ------------------------------------------------------------------ */

static void put_nibble(uint8_t* codes, int i, unsigned c)
{
    /* channel 2j in the low nibble of byte j, channel 2j+1 in the high one */
    if (i & 1) codes[i >> 1] = (uint8_t)((codes[i >> 1] & 0x0Fu) | (c << 4));
    else codes[i >> 1] = (uint8_t)((codes[i >> 1] & 0xF0u) | c);
}

static unsigned get_nibble(const uint8_t* codes, int i)
{
    return (i & 1) ? (codes[i >> 1] >> 4) & 15u : codes[i >> 1] & 15u;
}

/* Main latent KV, one group of 16 channels: scale s = E4M3(fl32(amax / 6)),
 * codes = E2M1(fl32(x / s)).  A scale that encodes to zero gives all-zero
 * codes.  Writes 8 code bytes and one scale byte. */
void orc_quant_main_group(const float* x, uint8_t* codes, uint8_t* scale)
{
    float amax = 0.0f;
    for (int i = 0; i < 16; i++) amax = fmaxf(amax, fabsf(x[i]));
    float t = amax / 6.0f;
    unsigned sc = orc_e4m3_encode((double)t);
    float s = (float)orc_e4m3_value(sc);
    *scale = (uint8_t)sc;
    memset(codes, 0, 8);
    if (s == 0.0f) return;
    for (int i = 0; i < 16; i++) {
        float y = x[i] / s;
        put_nibble(codes, i, orc_e2m1_encode((double)y));
    }
}

/* MXFP4 (indexer keys and indexer queries), one group of 32 channels:
 * e = floor(log2 amax) - 2 clamped to [-127, 127] (-127 for an all-zero
 * group), codes = E2M1(x * 2^-e).  Writes 16 code bytes and one E8M0 byte. */
void orc_quant_index_group(const float* x, uint8_t* codes, uint8_t* scale)
{
    float amax = 0.0f;
    for (int i = 0; i < 32; i++) amax = fmaxf(amax, fabsf(x[i]));
    int e = (amax == 0.0f) ? -127 : floor_log2((double)amax) - 2;
    if (e < -127) e = -127;
    if (e > 127) e = 127;
    *scale = (uint8_t)(e + 127);
    memset(codes, 0, 16);
    for (int i = 0; i < 32; i++)
        put_nibble(codes, i, orc_e2m1_encode(ldexp((double)x[i], -e)));
}

/* 8-bit sliding-window KV, one group of 16 channels (MX-style FP8):
 * e = floor(log2 amax) - 8 clamped to [-127, 127], codes = E4M3(x * 2^-e)
 * saturating.  Writes 16 code bytes and one E8M0 byte. */
void orc_quant_swa_group(const float* x, uint8_t* codes, uint8_t* scale)
{
    float amax = 0.0f;
    for (int i = 0; i < 16; i++) amax = fmaxf(amax, fabsf(x[i]));
    int e = (amax == 0.0f) ? -127 : floor_log2((double)amax) - 8;
    if (e < -127) e = -127;
    if (e > 127) e = 127;
    *scale = (uint8_t)(e + 127);
    for (int i = 0; i < 16; i++)
        codes[i] = (uint8_t)orc_e4m3_encode(ldexp((double)x[i], -e));
}

/* Row packers.  Main: 512 ch -> 256 code bytes + 32 scales (288 B).
 * Index: 128 ch -> 64 + 4 (68 B).  SWA: 512 ch -> 512 + 32 (544 B). */
void orc_pack_main(const float* src, int64_t n, uint8_t* codes, uint8_t* scales)
{
    for (int64_t r = 0; r < n; r++)
        for (int g = 0; g < 32; g++)
            orc_quant_main_group(src + r * 512 + 16 * g, codes + r * 256 + 8 * g,
                                 scales + r * 32 + g);
}

void orc_pack_index(const float* src, int64_t n, uint8_t* codes, uint8_t* scales)
{
    for (int64_t r = 0; r < n; r++)
        for (int g = 0; g < 4; g++)
            orc_quant_index_group(src + r * 128 + 32 * g, codes + r * 64 + 16 * g,
                                  scales + r * 4 + g);
}

void orc_pack_swa(const float* src, int64_t n, uint8_t* codes, uint8_t* scales)
{
    for (int64_t r = 0; r < n; r++)
        for (int g = 0; g < 32; g++)
            orc_quant_swa_group(src + r * 512 + 16 * g, codes + r * 512 + 16 * g,
                                scales + r * 32 + g);
}

void orc_dequant_main(const uint8_t* codes, const uint8_t* scales, int64_t n, float* out)
{
    for (int64_t r = 0; r < n; r++)
        for (int i = 0; i < 512; i++)
            out[r * 512 + i] = (float)(orc_e2m1_value(get_nibble(codes + r * 256, i)) *
                                       orc_e4m3_value(scales[r * 32 + i / 16]));
}

void orc_dequant_index(const uint8_t* codes, const uint8_t* scales, int64_t n, float* out)
{
    for (int64_t r = 0; r < n; r++)
        for (int i = 0; i < 128; i++)
            out[r * 128 + i] = (float)(orc_e2m1_value(get_nibble(codes + r * 64, i)) *
                                       orc_e8m0_value(scales[r * 4 + i / 32]));
}

void orc_dequant_swa(const uint8_t* codes, const uint8_t* scales, int64_t n, float* out)
{
    for (int64_t r = 0; r < n; r++)
        for (int i = 0; i < 512; i++)
            out[r * 512 + i] = (float)(orc_e4m3_value(codes[r * 512 + i]) *
                                       orc_e8m0_value(scales[r * 32 + i / 16]));
}

/* ------------------------------------------------------------------ */
/* Exact sum of signed powers-of-two terms, rounded once to fp32        */
/* ------------------------------------------------------------------ */

#define ACC_LIMBS 20      /* 640-bit two's complement fixed point */
#define ACC_OFFSET 300    /* bit index that carries weight 2^0     */

static void acc_add(uint32_t* acc, int64_t S, int pos)
{
    int L = pos >> 5, b = pos & 31;
    __int128 t = (__int128)S * ((__int128)1 << b);
    uint32_t ext = (S < 0) ? 0xFFFFFFFFu : 0u;
    uint64_t carry = 0;
    for (int k = L; k < ACC_LIMBS; k++) {
        int j = k - L;
        uint32_t part = (j < 4) ? (uint32_t)(t >> (32 * j)) : ext;
        uint64_t s = (uint64_t)acc[k] + part + carry;
        acc[k] = (uint32_t)s;
        carry = s >> 32;
    }
}

static int acc_bit(const uint32_t* acc, int k)
{
    return (int)((acc[k >> 5] >> (k & 31)) & 1u);
}

/* RN-even fp32 of sum_i S[i] * 2^E[i].  Needs |S| < 2^40 and
 * -ACC_OFFSET <= E <= 250, which every caller here respects. */
float orc_round_pow2_sum(const int64_t* S, const int* E, int n)
{
    uint32_t acc[ACC_LIMBS];
    memset(acc, 0, sizeof acc);
    for (int i = 0; i < n; i++)
        if (S[i] != 0) acc_add(acc, S[i], E[i] + ACC_OFFSET);
    int neg = (int)(acc[ACC_LIMBS - 1] >> 31);
    if (neg) {                                  /* magnitude = -acc */
        uint64_t carry = 1;
        for (int k = 0; k < ACC_LIMBS; k++) {
            uint64_t s = (uint64_t)(uint32_t)~acc[k] + carry;
            acc[k] = (uint32_t)s;
            carry = s >> 32;
        }
    }
    int top = -1;
    for (int k = ACC_LIMBS * 32 - 1; k >= 0; k--)
        if (acc_bit(acc, k)) { top = k; break; }
    if (top < 0) return 0.0f;
    int ulp = top - ACC_OFFSET - 23;            /* exponent of the fp32 ulp */
    if (ulp < -149) ulp = -149;
    int cut = ulp + ACC_OFFSET;                 /* bit index of that ulp */
    uint64_t q = 0;
    for (int k = top; k >= cut; k--) q = (q << 1) | (uint64_t)acc_bit(acc, k);
    int guard = acc_bit(acc, cut - 1);
    int sticky = 0;
    for (int k = cut - 2; k >= 0 && !sticky; k--) sticky = acc_bit(acc, k);
    if (guard && (sticky || (q & 1u))) q++;
    float r = ldexpf((float)q, ulp);
    return neg ? -r : r;
}

/* ------------------------------------------------------------------ */
/* Lightning-indexer score                                             */
/* ------------------------------------------------------------------ */

/* q_h . K_s for one MXFP4 query head and one MXFP4 key, exact, rounded once.
 * Each 32-channel group contributes 2^(eq+ek) * sum(E2M1 * E2M1); with the
 * E2M1 values doubled (integers) the group sum is an integer S and the term
 * is S * 2^(eq + ek - 2). */
float orc_head_dot(const uint8_t* qc, const uint8_t* qs, const uint8_t* kc, const uint8_t* ks)
{
    int64_t S[4];
    int E[4];
    for (int g = 0; g < 4; g++) {
        int64_t acc = 0;
        for (int i = 32 * g; i < 32 * g + 32; i++) {
            int64_t a = (int64_t)(2.0 * orc_e2m1_value(get_nibble(qc, i)));
            int64_t b = (int64_t)(2.0 * orc_e2m1_value(get_nibble(kc, i)));
            acc += a * b;
        }
        S[g] = acc;
        E[g] = ((int)qs[g] - 127) + ((int)ks[g] - 127) - 2;
    }
    return orc_round_pow2_sum(S, E, 4);
}

/* Scores of n keys for one query row: for each key,
 * acc = +0; acc = fma(w_h, ReLU(d_h), acc) for h = 0 .. Hi-1 in order. */
void orc_index_score(const uint8_t* qc, const uint8_t* qs, const float* w, int Hi,
                     const uint8_t* kc, const uint8_t* ks, int64_t n, float* out)
{
    for (int64_t s = 0; s < n; s++) {
        float acc = 0.0f;
        for (int h = 0; h < Hi; h++) {
            float d = orc_head_dot(qc + 64 * h, qs + 4 * h, kc + 64 * s, ks + 4 * s);
            float r = (d > 0.0f) ? d : 0.0f;
            acc = fmaf(w[h], r, acc);
        }
        if (acc == 0.0f) acc = 0.0f;    /* canonical +0 */
        out[s] = acc;
    }
}

/* Max over each aligned group of 8 scores (the last group may be partial). */
void orc_block_max(const float* scores, int64_t n, float* out)
{
    for (int64_t j = 0; 8 * j < n; j++) {
        float m = scores[8 * j];
        for (int64_t s = 8 * j + 1; s < 8 * j + 8 && s < n; s++)
            if (scores[s] > m) m = scores[s];
        out[j] = m;
    }
}

/* ------------------------------------------------------------------ */
/* Top-k                                                               */
/* ------------------------------------------------------------------ */

typedef struct { float key; int32_t id; } orc_item;

static int cmp_rank(const void* a, const void* b)
{
    const orc_item* x = (const orc_item*)a;
    const orc_item* y = (const orc_item*)b;
    if (x->key > y->key) return -1;
    if (x->key < y->key) return 1;
    return (x->id < y->id) ? -1 : (x->id > y->id);
}

static int cmp_i32(const void* a, const void* b)
{
    int32_t x = *(const int32_t*)a, y = *(const int32_t*)b;
    return (x > y) - (x < y);
}

/* The min(k, n) items ranked first by (key descending, id ascending);
 * their ids are written in ascending order.  Returns the count, or -1 if
 * memory runs out. */
int64_t orc_topk(const float* keys, const int32_t* ids, int64_t n, int64_t k, int32_t* out)
{
    if (n <= 0 || k <= 0) return 0;
    orc_item* it = (orc_item*)malloc((size_t)n * sizeof(orc_item));
    if (!it) return -1;
    for (int64_t i = 0; i < n; i++) {
        it[i].key = keys[i];
        it[i].id = ids ? ids[i] : (int32_t)i;
    }
    qsort(it, (size_t)n, sizeof(orc_item), cmp_rank);
    int64_t m = (k < n) ? k : n;
    for (int64_t i = 0; i < m; i++) out[i] = it[i].id;
    qsort(out, (size_t)m, sizeof(int32_t), cmp_i32);
    free(it);
    return m;
}

/* ------------------------------------------------------------------ */
/* Attention                                                           */
/* ------------------------------------------------------------------ */

/* Joint softmax attention for one query row, fp64 throughout.
 *   q     [H][C]   query heads (absorbed query in the latent space)
 *   K     [n][C]   selected entries, each used as key and value
 *   W     [m][C]   sliding-window entries, used the same way
 *   sink  [H] or NULL: extra exp(sink_h) in the denominator
 * z = sigma * q_h . entry;  out_h = sum e^(z - mu) entry / D,
 * D = sum e^(z - mu) (+ e^(sink - mu)),  lse_h = mu + ln D.
 * No entry and no sink: out = 0, lse = -inf. */
void orc_attention(const float* q, int H, int C, const float* K, int64_t n,
                   const float* W, int64_t m, const float* sink, double sigma,
                   float* out, float* lse)
{
    double* z = (double*)malloc((size_t)(n + m + 1) * sizeof(double));
    double* o = (double*)malloc((size_t)C * sizeof(double));
    for (int h = 0; h < H; h++) {
        const float* qh = q + (int64_t)h * C;
        double mu = -INFINITY;
        for (int64_t j = 0; j < n + m; j++) {
            const float* e = (j < n) ? K + j * C : W + (j - n) * C;
            double dot = 0.0;
            for (int c = 0; c < C; c++) dot += (double)qh[c] * (double)e[c];
            z[j] = sigma * dot;
            if (z[j] > mu) mu = z[j];
        }
        if (sink && (double)sink[h] > mu) mu = (double)sink[h];
        if (mu == -INFINITY) {
            for (int c = 0; c < C; c++) out[(int64_t)h * C + c] = 0.0f;
            lse[h] = -INFINITY;
            continue;
        }
        double D = 0.0;
        for (int c = 0; c < C; c++) o[c] = 0.0;
        for (int64_t j = 0; j < n + m; j++) {
            const float* e = (j < n) ? K + j * C : W + (j - n) * C;
            double p = exp(z[j] - mu);
            D += p;
            for (int c = 0; c < C; c++) o[c] += p * (double)e[c];
        }
        if (sink) D += exp((double)sink[h] - mu);
        for (int c = 0; c < C; c++) out[(int64_t)h * C + c] = (float)(o[c] / D);
        lse[h] = (float)(mu + log(D));
    }
    free(z);
    free(o);
}
