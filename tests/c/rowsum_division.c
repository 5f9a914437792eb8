/* The ordered softmax kernels write e / s, the IEEE quotient, as
 *   y = RN(1 / s),  q = RN(e y),  r = RN(e - s q),  q' = RN(q + r y)
 * (two fused multiply-adds; P. Markstein, IBM J. Res. Dev. 34(1), 1990),
 * for a row sum s >= 1 and numerators e == 0 or e >= 2^-96, and switch to
 * the division when some e lies in (0, 2^-96).  This program checks, against
 * the host's IEEE division and its correctly rounded fmaf:
 *   1. q' == e / s on structured pairs (significands 1.0, all ones, all
 *      ones but the last bit, ... for every exponent of e in [-96, 0] and of
 *      s in [0, 23]), on e = 1, 1/2 and 1 - 2^-24 over integer sums
 *      1 .. 2^20, and on seeded random pairs;
 *   2. the guard: the bit pattern minus one, unsigned, is below
 *      0x0F7FFFFF exactly for e in (0, 2^-96);
 *   3. below 2^-96 the form does differ from the division for some pairs,
 *      so the guard is needed.
 * Usage: rowsum_division <random pairs> <seed>.  Exit status 0 when all
 * hold. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static uint64_t splitmix(uint64_t* x) {
    uint64_t z = (*x += 0x9e3779b97f4a7c15ull);
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
    return z ^ (z >> 31);
}
static float from_bits(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t to_bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

static float quotient(float e, float s) {
    volatile float y = 1.0f / s;
    const float q = e * y;
    return fmaf(fmaf(-q, s, e), y, q);
}

static long long checked = 0, wrong = 0;
static void check(float e, float s) {
    const float want = e / s, got = quotient(e, s);
    ++checked;
    if (to_bits(got) != to_bits(want)) {
        if (wrong < 5) printf("e=%a s=%a: %a, division %a\n", e, s, got, want);
        ++wrong;
    }
}

int main(int argc, char** argv) {
    const long long n = argc > 1 ? atoll(argv[1]) : 1000000;
    uint64_t st = argc > 2 ? strtoull(argv[2], 0, 10) : 1;
    const uint32_t sig[] = {0x000000, 0x7fffff, 0x7ffffe, 0x400000, 0x3fffff, 0x000001, 0x555555, 0x2aaaab};
    const int nsig = (int)(sizeof sig / sizeof sig[0]);
    for (int ee = -96; ee <= 0; ++ee)
        for (int i = 0; i < nsig; ++i)
            for (int es = 0; es < 24; ++es)
                for (int j = 0; j < nsig; ++j) {
                    const float e = from_bits(((uint32_t)(ee + 127) << 23) | sig[i]);
                    if (e <= 1.0f) check(e, from_bits(((uint32_t)(es + 127) << 23) | sig[j]));
                }
    for (uint32_t k = 1; k <= (1u << 20); ++k) {
        check(1.0f, (float)k);
        check(0.5f, (float)k);
        check(from_bits(0x3f7fffff), (float)k);
    }
    check(0.0f, 3.0f);
    for (long long i = 0; i < n; ++i) {
        const uint64_t u = splitmix(&st), v = splitmix(&st);
        float e = from_bits(((uint32_t)(127 - (int)(u % 97)) << 23) | ((uint32_t)(u >> 8) & 0x7fffff));
        if (e > 1.0f) e = 1.0f;
        check(e, from_bits(((uint32_t)(127 + (int)(v % 24)) << 23) | ((uint32_t)(v >> 8) & 0x7fffff)));
    }
    printf("identity: %lld pairs, %lld differ from the division\n", checked, wrong);

    /* the guard */
    long long guard_bad = 0;
    const uint32_t edges[] = {0u, 1u, 0x007fffffu, 0x00800000u, 0x0F7FFFFEu, 0x0F7FFFFFu, 0x0F800000u,
                              0x0F800001u, 0x3f800000u};
    for (size_t i = 0; i < sizeof edges / sizeof edges[0]; ++i) {
        const float e = from_bits(edges[i]);
        const int flagged = (uint32_t)(edges[i] - 1u) < 0x0F7FFFFFu;
        const int tiny = e > 0.0f && e < 0x1p-96f;
        if (flagged != tiny) { printf("guard wrong at %a\n", e); ++guard_bad; }
    }

    /* below 2^-96 */
    long long below = 0;
    for (long long i = 0; i < 2000000; ++i) {
        const uint64_t u = splitmix(&st), v = splitmix(&st);
        const float e = from_bits(1u + (uint32_t)(u % (37ull << 23)));
        const float s = from_bits(((uint32_t)(127 + (int)(v % 24)) << 23) | ((uint32_t)(v >> 8) & 0x7fffff));
        if (to_bits(quotient(e, s)) != to_bits(e / s)) ++below;
    }
    printf("below 2^-96: %lld of 2000000 pairs differ; guard errors %lld\n", below, guard_bad);
    return (wrong == 0 && guard_bad == 0 && below > 0) ? 0 : 1;
}
