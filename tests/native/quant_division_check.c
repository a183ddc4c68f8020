/* Host check of the division-free quantiser step used by the matrix-core encode kernel.
 *
 * The quantiser (SPECTRA technical summary, SPECTRA pipeline stage 3; the code formula is this
 * library's reading) divides a float32 latent c by an fp16 scale s with correct rounding.  The
 * kernel instead forms r = RN(1/s) once per group and, per element,
 *     q0 = RN(c r),   t = RN(q0 + RN-exact(c - q0 s) r)      (two fused multiply-adds)
 * (Markstein's correction step).  This program compares t with the IEEE quotient c / s for every
 * float32 significand of c in [1, 2) against the fp16 significands s in [1, 2) named on the
 * command line (fraction f / 1024 for f in [first, last) stepping by stride).  Both sides scale
 * exactly by powers of two while no intermediate is subnormal, so the significands decide.
 * Prints the number of mismatches; exit status 1 if any.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static float from_bits(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t to_bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

int main(int argc, char** argv) {
    const int first = argc > 1 ? atoi(argv[1]) : 0;
    const int last = argc > 2 ? atoi(argv[2]) : 1024;
    const int stride = argc > 3 ? atoi(argv[3]) : 1;
    long bad = 0, checked = 0;
#pragma omp parallel for reduction(+ : bad, checked) schedule(dynamic)
    for (int f = first; f < last; f += stride) {
        const float s = from_bits(0x3f800000u | ((uint32_t)f << 13));
        const float r = 1.0f / s;
        for (uint32_t m = 0; m < (1u << 23); ++m) {
            const float c = from_bits(0x3f800000u | m);
            const float want = c / s;
            const float q0 = c * r;
            const float t = fmaf(fmaf(-q0, s, c), r, q0);
            if (to_bits(t) != to_bits(want)) ++bad;
            ++checked;
        }
    }
    printf("checked %ld mismatches %ld\n", checked, bad);
    return bad ? 1 : 0;
}
