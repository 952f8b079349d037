/* Exhaustive check of the q8_1 block scale computed without a division (MMQ page, "dp4a path
 * Q4_K": the activation scale d of a 32-value block; read as d32 = amax / 127 in fp32).
 *
 * The kernels form d32 from amax with one multiply by c = RN(1/127) and one fma correction,
 *     q1 = RN(amax * c);  r = fma(-q1, 127, amax);  d32 = fma(r, c, q1),
 * and fall back to the IEEE division whenever the result lies outside [2^-100, 2^100].  This
 * program walks every positive finite fp32 amax, applies the same three operations (C99 fmaf:
 * one rounding, as the GPU's v_fma_f32), and counts the values inside that window where the
 * result differs from amax / 127.0f.  Exit status 0 and "mismatches 0" means the shortcut never
 * changes a scale.  Build: gcc -O2 -mfma -ffp-contract=off -fopenmp (with -DPLANT_NO_CORRECTION the
 * correction is dropped, and the check must then fail).
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static float bits_to_float(uint32_t b) {
    float f;
    memcpy(&f, &b, sizeof f);
    return f;
}

int main(void) {
    const float c = 1.0f / 127.0f;
    const float lo = 0x1p-100f, hi = 0x1p100f;
    long long checked = 0, mismatches = 0;
    uint32_t first_bad = 0;
#pragma omp parallel for schedule(static, 1 << 16) reduction(+ : checked, mismatches)
    for (long long i = 1; i < 0x7F800000LL; ++i) {   /* every positive finite float */
        const float amax = bits_to_float((uint32_t)i);
        const float q1 = amax * c;
#ifdef PLANT_NO_CORRECTION
        const float d = q1;   /* planted mistake: the product alone, without the correction */
#else
        const float d = fmaf(fmaf(-q1, 127.0f, amax), c, q1);
#endif
        if (!(d >= lo && d <= hi)) continue;           /* the kernels divide there */
        ++checked;
        if (d != amax / 127.0f) {
            ++mismatches;
#pragma omp critical
            if (!first_bad) first_bad = (uint32_t)i;
        }
    }
    printf("checked %lld mismatches %lld first 0x%08x\n", checked, mismatches, first_bad);
    return mismatches == 0 && checked > 0 ? 0 : 1;
}
