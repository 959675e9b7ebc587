/*
 * Host driver for the fp64 oracle (oracle/wkv_oracle.c) built with the
 * address and undefined-behaviour sanitizers: every input kind, decay form,
 * variant, slice mask, ragged offsets with an empty sequence, carried states,
 * and a rejected offsets array.  Checks the hand-worked D = 2, T = 3 example
 * (tests/golden/hand_worked_d2_t3.json: GoldFinch architecture summary,
 * section 3.4, state equation with base Finch's bonus) exactly, and the
 * split-and-carry identity exactly.  Exits 0 when all checks hold.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_wkv_f64_ex(int kind, int decay_kind, int variant, const void *r, const void *k, const void *v,
                      const void *w, const float *u, const void *u2, const double *state_in,
                      const int64_t *cu_seqlens, int64_t N, int H, int D, const uint8_t *slice_mask,
                      double *o, double *state_out, int threads);

static int fails = 0;
#define CHECK(c) do { if (!(c)) { printf("FAIL line %d: %s\n", __LINE__, #c); ++fails; } } while (0)

static uint16_t to_bf16(float f) {            /* round to nearest even */
    uint32_t x;
    memcpy(&x, &f, 4);
    x += 0x7FFF + ((x >> 16) & 1);
    return (uint16_t)(x >> 16);
}

static double lcg(uint64_t *s) {              /* uniform in [-1, 1) */
    *s = *s * 6364136223846793005ull + 1442695040888963407ull;
    return (double)(*s >> 11) / 9007199254740992.0 * 2.0 - 1.0;
}

int main(void) {
    /* hand-worked example, fp32 inputs */
    {
        const float r[6] = {1, 1, 1, 1, 1, -1}, k[6] = {1, 0, 1, 1, 0, 2}, v[6] = {2, 1, 1, -1, 0.5f, 0};
        const float w[6] = {0.5f, 0.25f, 0.5f, 1, 1, 0.5f}, u[2] = {1, 0};
        const double s0[4] = {1, 0, 0, 2};
        const int64_t cu[2] = {0, 3};
        double o[6], s[4];
        CHECK(oracle_wkv_f64_ex(0, 0, 0, r, k, v, w, u, NULL, s0, cu, 1, 1, 2, NULL, o, s, 1) == 0);
        const double eo[6] = {3, 3, 3.5, 0.5, 1.25, 0}, es[4] = {2.25, -0.5, 1.5, -0.25};
        for (int i = 0; i < 6; ++i) CHECK(o[i] == eo[i]);
        for (int i = 0; i < 4; ++i) CHECK(s[i] == es[i]);
    }
    /* random bf16 inputs: 3 sequences (5, 0, 7 tokens), H = 2, D = 8, every form */
    {
        enum { N = 3, H = 2, D = 8, TOK = 12 };
        const int64_t cu[N + 1] = {0, 5, 5, 12};
        uint16_t r[TOK * H * D], k[TOK * H * D], v[TOK * H * D], w[TOK * H * D], d[TOK * H * D], u2[TOK * H * D];
        float u[H * D];
        double s0[N * H * D * D];
        uint64_t seed = 12345;
        for (int i = 0; i < TOK * H * D; ++i) {
            r[i] = to_bf16((float)lcg(&seed));
            k[i] = to_bf16((float)lcg(&seed));
            v[i] = to_bf16((float)lcg(&seed));
            const double x = -3.5 + 2.5 * lcg(&seed);                  /* d in [-6, -1) */
            d[i] = to_bf16((float)x);
            w[i] = to_bf16((float)exp(-exp(x)));
            u2[i] = to_bf16((float)lcg(&seed));
        }
        for (int i = 0; i < H * D; ++i) u[i] = (float)lcg(&seed);
        for (int i = 0; i < N * H * D * D; ++i) s0[i] = 0.1 * lcg(&seed);
        const uint8_t mask[N * H] = {1, 0, 1, 1, 1, 1};     /* (sequence 0, head 1) not computed */
        for (int form = 0; form < 4; ++form) {
            const int dk = form & 1, var = form >> 1;
            const uint16_t *dec = dk ? d : w;
            double o[TOK * H * D], s[N * H * D * D];
            memset(o, 0, sizeof o);
            memset(s, 0, sizeof s);
            CHECK(oracle_wkv_f64_ex(1, dk, var, r, k, v, dec, u, var ? u2 : NULL, s0, cu, N, H, D, mask, o, s, 2) == 0);
            for (int i = 0; i < TOK * H * D; ++i) CHECK(isfinite(o[i]));
            /* split sequence 2 (tokens 5..12) after 3 tokens and carry the state */
            const int64_t cu_a[2] = {0, 3}, cu_b[2] = {0, 4};
            double oa[3 * H * D], ob[4 * H * D], sa[H * D * D], sb[H * D * D];
            const size_t off = 5 * H * D, off_b = 8 * H * D;
            const double *s0_2 = s0 + 2 * H * D * D;
            CHECK(oracle_wkv_f64_ex(1, dk, var, r + off, k + off, v + off, dec + off, u, var ? u2 + off : NULL, s0_2,
                                    cu_a, 1, H, D, NULL, oa, sa, 1) == 0);
            CHECK(oracle_wkv_f64_ex(1, dk, var, r + off_b, k + off_b, v + off_b, dec + off_b, u,
                                    var ? u2 + off_b : NULL, sa, cu_b, 1, H, D, NULL, ob, sb, 1) == 0);
            for (int i = 0; i < 3 * H * D; ++i) CHECK(oa[i] == o[off + i]);
            for (int i = 0; i < 4 * H * D; ++i) CHECK(ob[i] == o[off_b + i]);
            for (int i = 0; i < H * D * D; ++i) CHECK(sb[i] == s[2 * H * D * D + i]);
            /* the empty sequence hands its state through */
            for (int i = 0; i < H * D * D; ++i) CHECK(s[H * D * D + i] == s0[H * D * D + i]);
        }
        /* offsets that decrease are rejected */
        const int64_t bad[N + 1] = {0, 5, 4, 12};
        double o[TOK * H * D], s[N * H * D * D];
        CHECK(oracle_wkv_f64_ex(1, 0, 0, r, k, v, w, u, NULL, NULL, bad, N, H, D, NULL, o, s, 1) == -1);
    }
    printf("%s (%d failure(s))\n", fails ? "FAILED" : "all checks passed", fails);
    return fails ? 1 : 0;
}
