/*
 * oracle_driver.c -- runs every function of the C oracle (compiled into this
 * program) over edge inputs under AddressSanitizer and UndefinedBehavior-
 * Sanitizer: all E2M1/E4M3/E8M0 codes, packing and unpacking of zero, signed
 * zero, subnormal, huge and saturating values, exact power-of-two sums at
 * extreme exponents, index scores, block maxima of partial blocks, top-k with
 * ties and empty inputs, attention with empty sets and a sink.  A few cheap
 * invariants are checked on the way; the sanitizers report any memory or
 * undefined-behaviour error.  Exit status 0 = clean.
 */
#include "../../oracle/csa2_oracle.c"

#include <stdio.h>

static unsigned long long rng_state = 88172645463325252ULL;
static double urand(void) {   /* xorshift64 */
    rng_state ^= rng_state << 13;
    rng_state ^= rng_state >> 7;
    rng_state ^= rng_state << 17;
    return (double)(rng_state >> 11) * (1.0 / 9007199254740992.0);
}

static int fails = 0;
#define CHECK(c) do { if (!(c)) { fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__); fails++; } } while (0)

int main(void) {
    /* codecs: every code, and encode(decode(code)) = code where the value is canonical */
    for (unsigned c = 0; c < 16; c++) CHECK(orc_e2m1_encode(orc_e2m1_value(c)) == c);
    for (unsigned c = 0; c < 256; c++) {
        if ((c & 0x7F) == 0x7F) continue;                       /* NaN codes are never produced */
        CHECK(orc_e4m3_encode(orc_e4m3_value(c)) == c);
    }
    for (unsigned c = 0; c < 255; c++) CHECK(orc_e8m0_value(c) > 0.0);
    /* pack / dequant of edge rows (512 and 128 channels) */
    enum { N = 9 };
    static float src[N * 512];
    for (int r = 0; r < N; r++)
        for (int i = 0; i < 512; i++) {
            double v = urand() * 2 - 1;
            switch (r) {
                case 0: v = 0.0; break;
                case 1: v = -0.0; break;
                case 2: v *= 1e-40; break;         /* fp32 subnormal */
                case 3: v *= 3e38; break;          /* near the fp32 maximum */
                case 4: v *= 2688.0; break;        /* the FP4 maximum */
                case 5: v = (i % 16 == 0) ? 6.0 : 0.25 * (i % 7); break;   /* rounding midpoints */
                case 6: v *= 1e-3; break;          /* subnormal E4M3 scales */
                default: v *= ldexp(1.0, (int)(urand() * 60) - 30); break;
            }
            src[r * 512 + i] = (float)v;
        }
    static uint8_t mc[N * 256], ms[N * 32], ic[N * 4 * 64], is[N * 4 * 4], sc[N * 512], ss[N * 32];
    static float out[N * 512];
    orc_pack_main(src, N, mc, ms);
    orc_dequant_main(mc, ms, N, out);
    for (int i = 0; i < N * 512; i++) CHECK(fabsf(out[i]) <= 2688.0f);
    for (int i = 0; i < 512; i++) CHECK(out[i] == 0.0f);
    orc_pack_index(src, 4 * N, ic, is);     /* the same floats seen as 4N rows of 128 */
    orc_dequant_index(ic, is, 4 * N, out);
    orc_pack_swa(src, N, sc, ss);
    orc_dequant_swa(sc, ss, N, out);
    /* exact sums at extreme exponents */
    int64_t S[4] = {1, -1, (int64_t)1 << 39, -((int64_t)1 << 39)};
    int E[4] = {-300, -300, 250, 250};
    CHECK(orc_round_pow2_sum(S, E, 4) == 0.0f);
    int64_t S2[2] = {3, 1};
    int E2[2] = {-149, -150};
    CHECK(orc_round_pow2_sum(S2, E2, 2) == ldexpf(4.0f, -149));   /* 3.5 ulp ties to even: 4 */
    /* index scores of random MXFP4 keys, 8 heads */
    enum { NK = 37, HI = 8 };
    static float kf[NK * 128], qf[HI * 128], w[HI], scr[NK], bm[(NK + 7) / 8];
    for (int i = 0; i < NK * 128; i++) kf[i] = (float)(urand() * 4 - 2);
    for (int i = 0; i < HI * 128; i++) qf[i] = (float)(urand() * 4 - 2);
    for (int h = 0; h < HI; h++) w[h] = (float)urand();
    static uint8_t kc[NK * 64], ks[NK * 4], qc[HI * 64], qs[HI * 4];
    orc_pack_index(kf, NK, kc, ks);
    orc_pack_index(qf, HI, qc, qs);
    orc_index_score(qc, qs, w, HI, kc, ks, NK, scr);
    for (int s = 0; s < NK; s++) CHECK(scr[s] >= 0.0f && !signbit(scr[s]));
    orc_block_max(scr, NK, bm);
    for (int j = 0; j < (NK + 7) / 8; j++) CHECK(bm[j] >= scr[8 * j]);
    /* top-k: ties, k > n, empty */
    float keys[10] = {1, 3, 3, -INFINITY, 2, 3, 0, -0.0f, 3, 1};
    int32_t ids[10], got[10];
    for (int i = 0; i < 10; i++) ids[i] = 100 + 2 * i;
    CHECK(orc_topk(keys, ids, 10, 3, got) == 3 && got[0] == 102 && got[1] == 104 && got[2] == 110);
    CHECK(orc_topk(keys, NULL, 10, 20, got) == 10);
    CHECK(orc_topk(keys, NULL, 0, 5, got) == 0);
    /* attention: selected + window + sink; empty sets */
    enum { H = 3, C = 512, NS = 5, NW = 2 };
    static float q[H * C], K[NS * C], W[NW * C], o[H * C], lse[H], sink[H] = {0.5f, -1.0f, 2.0f};
    for (int i = 0; i < H * C; i++) q[i] = (float)(urand() - 0.5);
    for (int i = 0; i < NS * C; i++) K[i] = (float)(urand() - 0.5);
    for (int i = 0; i < NW * C; i++) W[i] = (float)(urand() - 0.5);
    orc_attention(q, H, C, K, NS, W, NW, sink, 1.0 / sqrt(512.0), o, lse);
    for (int h = 0; h < H; h++) CHECK(isfinite(lse[h]));
    orc_attention(q, H, C, NULL, 0, NULL, 0, NULL, 1.0 / sqrt(512.0), o, lse);
    for (int h = 0; h < H; h++) CHECK(isinf(lse[h]) && lse[h] < 0 && o[h * C] == 0.0f);
    orc_attention(q, H, C, NULL, 0, NULL, 0, sink, 1.0 / sqrt(512.0), o, lse);
    for (int h = 0; h < H; h++) CHECK(lse[h] == sink[h] && o[h * C] == 0.0f);
    if (fails) { fprintf(stderr, "%d check(s) failed\n", fails); return 1; }
    printf("oracle driver clean\n");
    return 0;
}
