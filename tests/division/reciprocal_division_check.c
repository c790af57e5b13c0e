/* Check of the cache writer's division: for FP16 x and a scale b in
 * [2^-110, 2^126], with y = RN(1/b),
 *     q = RN(x y),  r = fma(-q, b, x),  c = copysign(RN(r y + q), x)
 * must equal the IEEE single-precision quotient RN(x / b) bit for bit
 * (Markstein's correction of a quotient from a correctly rounded reciprocal).
 * Every finite FP16 x is tried against every scale given: special mantissas at
 * every exponent of the range, plus n seeded random scales.
 * Usage: reciprocal_division_check N_RANDOM_SCALES THREADS
 * Prints the counts; exits 1 on any mismatch. */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static float xs[65536];
static int nx;
static float *scales;
static int ns;
static int nthreads;
static long long bad[64];

static float from_bits(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t to_bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

static float fp16_value(uint16_t h)
{
    const int e = (h >> 10) & 31, m = h & 1023;
    float v = e == 0 ? ldexpf((float)m, -24) : e == 31 ? (m ? NAN : INFINITY)
                                                      : ldexpf((float)(m | 1024), e - 25);
    return (h & 0x8000) ? -v : v;
}

static void *run(void *arg)
{
    const int t = (int)(intptr_t)arg;
    for (int j = t; j < ns; j += nthreads) {
        const float b = scales[j], y = 1.0f / b;
        for (int i = 0; i < nx; ++i) {
            const float x = xs[i];
            const float q = x * y;
            const float r = fmaf(-q, b, x);
            const float c = copysignf(fmaf(r, y, q), x);
            if (to_bits(c) != to_bits(x / b)) {
                if (bad[t] < 3)
                    fprintf(stderr, "x=%a b=%a: %a, IEEE %a\n", x, b, c, x / b);
                bad[t]++;
            }
        }
    }
    return NULL;
}

int main(int argc, char **argv)
{
    const int nrand = argc > 1 ? atoi(argv[1]) : 2000;
    nthreads = argc > 2 ? atoi(argv[2]) : 4;
    if (nthreads < 1 || nthreads > 64)
        return 2;
    for (int h = 0; h < 65536; ++h) {
        const float v = fp16_value((uint16_t)h);
        if (isfinite(v))
            xs[nx++] = v;
    }
    static const uint32_t mant[] = {0x000000, 0x000001, 0x7FFFFF, 0x7FFFFE, 0x400000,
                                    0x3FFFFF, 0x555555, 0x2AAAAA, 0x0CCCCD, 0x3D70A4};
    /* the range is [2^-110, 2^126]: every binade from 2^-110 up to 2^126 itself */
    const int nspecial = (125 + 110 + 1) * (int)(sizeof mant / sizeof mant[0]) + 1;
    scales = malloc(sizeof(float) * (size_t)(nspecial + nrand));
    for (int e = -110; e <= 125; ++e)
        for (size_t k = 0; k < sizeof mant / sizeof mant[0]; ++k)
            scales[ns++] = from_bits(((uint32_t)(e + 127) << 23) | mant[k]);
    scales[ns++] = 0x1p126f;
    uint64_t s = 0x5CA1E5EEDull;
    for (int i = 0; i < nrand; ++i) {
        s = s * 6364136223846793005ull + 1442695040888963407ull;   /* LCG, seeded */
        const int e = -110 + (int)((s >> 33) % 236);
        scales[ns++] = from_bits(((uint32_t)(e + 127) << 23) | (uint32_t)((s >> 8) & 0x7FFFFF));
    }
    pthread_t th[64];
    for (int t = 0; t < nthreads; ++t)
        pthread_create(&th[t], NULL, run, (void *)(intptr_t)t);
    long long total = 0;
    for (int t = 0; t < nthreads; ++t) {
        pthread_join(th[t], NULL);
        total += bad[t];
    }
    printf("fp16 values %d, scales %d, pairs %lld, mismatches %lld\n", nx, ns,
           (long long)nx * ns, total);
    free(scales);
    return total != 0;
}
