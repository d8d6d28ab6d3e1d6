/* Drives the C oracle through its batch drivers on small random inputs, with
 * padding rows, out-of-range slots, bad token ranges, accepted lengths past a
 * row and checkpoints before, inside, past and absent, so that a sanitized
 * build (AddressSanitizer, UndefinedBehaviorSanitizer) sees every branch.
 * Exits 0 when every call returns the status the inputs call for. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int kda_oracle_decode(float *, int64_t, int64_t, const int32_t *, int32_t, int32_t, int32_t, int32_t,
                      const uint16_t *, const uint16_t *, const uint16_t *, const float *, const float *, float *,
                      const uint16_t *, const float *, double, int32_t, int32_t, int32_t);
int kda_oracle_verify(float *, int64_t, int64_t, const int32_t *, const int32_t *, int32_t, int32_t, int32_t,
                      int32_t, int32_t, int32_t, const uint16_t *, const uint16_t *, const uint16_t *,
                      const float *, const float *, float *, const uint16_t *, const float *, double, int32_t,
                      int32_t, uint16_t *, uint16_t *, float *, float *, float *, int32_t, int32_t, int32_t);
int kda_oracle_commit(float *, int64_t, int64_t, const int32_t *, const int32_t *, const int32_t *, int32_t,
                      int32_t, int32_t, int32_t, int32_t, int32_t, const uint16_t *, const uint16_t *,
                      const float *, const float *, int32_t, int32_t, int32_t);
int kda_oracle_prefill(float *, int64_t, int64_t, const int32_t *, const int32_t *, int32_t, int32_t, int32_t,
                       int32_t, int32_t, const uint16_t *, const uint16_t *, const uint16_t *, const float *,
                       const float *, float *, const int32_t *, float *, int32_t, int32_t, int32_t);

static uint32_t rng = 12345u;
static float frand(void) {
    rng = rng * 1664525u + 1013904223u;
    return (float)((rng >> 8) & 0xffff) / 65536.0f - 0.5f;
}
static uint16_t bf(float x) {
    uint32_t u;
    memcpy(&u, &x, 4);
    return (uint16_t)(u >> 16);
}

#define CHECK(cond)                                                     \
    do {                                                                \
        if (!(cond)) {                                                  \
            fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
            return 1;                                                   \
        }                                                               \
    } while (0)

int main(void) {
    enum { B = 5, H = 2, DK = 4, DV = 3, NS = 7, TMAX = 4, NTOK = 11 };
    const int64_t stride = (int64_t)H * DV * DK;
    float *cache = malloc(sizeof(float) * NS * stride);
    for (int i = 0; i < NS * stride; ++i) cache[i] = frand();
    uint16_t q[NTOK * H * DK], k[NTOK * H * DK], v[NTOK * H * DV], gate[NTOK * H * DV];
    float alpha[NTOK * H * DK], beta[NTOK * H], out[NTOK * H * DV], w[DV];
    for (int i = 0; i < NTOK * H * DK; ++i) {
        q[i] = bf(frand());
        k[i] = bf(frand());
        alpha[i] = 0.5f + frand();
    }
    for (int i = 0; i < NTOK * H * DV; ++i) {
        v[i] = bf(frand());
        gate[i] = bf(frand());
    }
    for (int i = 0; i < NTOK * H; ++i) beta[i] = 0.5f + frand();
    for (int i = 0; i < DV; ++i) w[i] = 1.0f + frand();

    const int32_t slots[B] = {3, -1, 0, 6, 2};
    const int32_t bad_slots[B] = {3, 7, 0, 6, 2};
    const int32_t cu[B + 1] = {0, 2, 3, 7, 8, 11};
    const int32_t bad_cu[B + 1] = {0, 2, 1, 7, 8, 11};
    uint16_t rk[B * TMAX * H * DK], rv[B * TMAX * H * DV];
    float ra[B * TMAX * H * DK], rb[B * TMAX * H];
    float *draft = malloc(sizeof(float) * B * TMAX * stride);

    for (int prologue = 0; prologue < 2; ++prologue) {
        for (int fp32 = 0; fp32 < 2; ++fp32) {
            CHECK(kda_oracle_decode(cache, NS, stride, slots, B, H, DK, DV, q, k, v, alpha, beta, out, NULL, NULL,
                                    1e-6, prologue, fp32, 2) == 0);
            CHECK(kda_oracle_decode(cache, NS, stride, slots, B, H, DK, DV, q, k, v, alpha, beta, out, gate, w,
                                    1e-6, prologue, fp32, 3) == 0);
            CHECK(kda_oracle_decode(cache, NS, stride, bad_slots, B, H, DK, DV, q, k, v, alpha, beta, out, NULL,
                                    NULL, 1e-6, prologue, fp32, 1) == 1);
            for (int mode = 0; mode < 2; ++mode)
                for (int inplace = 0; inplace < 2; ++inplace) {
                    CHECK(kda_oracle_verify(cache, NS, stride, slots, cu, B, TMAX, NTOK, H, DK, DV, q, k, v, alpha,
                                            beta, out, inplace ? gate : NULL, w, 1e-6, mode, inplace, rk, rv, ra, rb,
                                            draft, prologue, fp32, 2) == 0);
                    CHECK(kda_oracle_verify(cache, NS, stride, slots, bad_cu, B, TMAX, NTOK, H, DK, DV, q, k, v,
                                            alpha, beta, out, NULL, NULL, 1e-6, mode, inplace, rk, rv, ra, rb, draft,
                                            prologue, fp32, 2) == 2);
                }
            const int32_t acc[B] = {2, 1, 0, 1, 3};
            const int32_t bad_acc[B] = {3, 1, 0, 1, 3};
            CHECK(kda_oracle_commit(cache, NS, stride, slots, cu, acc, B, TMAX, NTOK, H, DK, DV, k, v, alpha, beta,
                                    prologue, fp32, 2) == 0);
            CHECK(kda_oracle_commit(cache, NS, stride, slots, cu, bad_acc, B, TMAX, NTOK, H, DK, DV, k, v, alpha,
                                    beta, prologue, fp32, 2) == 4);
            float ckpt[B * H * DV * DK];
            const int32_t pos[B] = {1, 0, -1, 0, 3};
            const int32_t bad_pos[B] = {3, 0, 0, 0, 3};
            CHECK(kda_oracle_prefill(cache, NS, stride, slots, cu, B, NTOK, H, DK, DV, q, k, v, alpha, beta, out, pos,
                                     ckpt, prologue, fp32, 2) == 0);
            CHECK(kda_oracle_prefill(cache, NS, stride, slots, cu, B, NTOK, H, DK, DV, q, k, v, alpha, beta, out,
                                     NULL, NULL, prologue, fp32, 4) == 0);
            CHECK(kda_oracle_prefill(cache, NS, stride, slots, cu, B, NTOK, H, DK, DV, q, k, v, alpha, beta, out,
                                     bad_pos, ckpt, prologue, fp32, 2) == 8);
        }
    }
    /* empty batch and invalid arguments */
    CHECK(kda_oracle_decode(cache, NS, stride, slots, 0, H, DK, DV, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL,
                            1e-6, 0, 1, 1) == 0);
    CHECK(kda_oracle_decode(cache, NS, stride - 1, slots, B, H, DK, DV, q, k, v, alpha, beta, out, NULL, NULL, 1e-6,
                            0, 1, 1) == -1);
    CHECK(kda_oracle_verify(cache, NS, stride, slots, cu, B, TMAX, NTOK, H, DK, DV, q, k, v, alpha, beta, out, NULL,
                            NULL, 1e-6, 2, 0, rk, rv, ra, rb, draft, 0, 1, 1) == -1);
    free(cache);
    free(draft);
    printf("oracle driver: ok\n");
    return 0;
}
