/*
 * Exhaustive check of the quotient identity the HIP quantizer uses in place of
 * one IEEE division per element:
 *
 *   s  = fl32(a / qmax)            (block scale, a = block absmax)
 *   r  = fl32(1 / s)               (correctly rounded reciprocal, once per block)
 *   q0 = fl32(x * r)
 *   e  = fma(-q0, s, x)            (exact remainder)
 *   q1 = fma(e, r, q0)
 *
 * Markstein's theorem says q1 == fl32(x / s) when r is the correctly rounded
 * reciprocal and nothing over- or underflows. The activations and weights of
 * the layer are fp16, so this program proves the identity for every input the
 * quantizer can see: every positive fp16 absmax a and every fp16 x with
 * |x| <= a, for qmax = 7 (INT4) and qmax = 127 (INT8). It also checks that
 * |rint(q1)| <= qmax, i.e. that the clamp of the definition never changes a
 * code, so a kernel may leave it out.
 *
 * Build: gcc -O2 -fopenmp -ffp-contract=off -fno-fast-math (fmaf is the
 * correctly rounded fused multiply-add of C99).
 * Prints the number of mismatches for each qmax and exits 1 if any.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static float half_to_float(uint16_t h)
{
    /* exact fp16 -> fp32 widening, written from the binary16 definition */
    uint32_t sign = (uint32_t)(h >> 15) << 31;
    int exp = (h >> 10) & 0x1F;
    uint32_t man = h & 0x3FF;
    float f;
    if (exp == 0) {
        f = ldexpf((float)man, -24);           /* subnormal: man * 2^-24 */
    } else if (exp == 31) {
        f = man ? NAN : INFINITY;
    } else {
        f = ldexpf((float)(man | 0x400), exp - 25);
    }
    uint32_t bits;
    memcpy(&bits, &f, 4);
    bits |= sign;
    memcpy(&f, &bits, 4);
    return f;
}

int main(void)
{
    long total_bad = 0;
    const int qmaxes[2] = {7, 127};
    for (int qi = 0; qi < 2; ++qi) {
        const float qmax = (float)qmaxes[qi];
        long bad = 0, checked = 0, clamped = 0;
#pragma omp parallel for schedule(dynamic, 64) reduction(+ : bad, checked, clamped)
        for (int ha = 1; ha < 0x7C00; ++ha) {           /* positive finite fp16 absmax */
            const float a = half_to_float((uint16_t)ha);
            const float s = a / qmax;
            const float r = 1.0f / s;
            for (int hx = 0; hx <= ha; ++hx) {          /* 0 <= |x| <= a, both signs */
                for (int sg = 0; sg < 2; ++sg) {
                    const float x = sg ? -half_to_float((uint16_t)hx) : half_to_float((uint16_t)hx);
                    const float q0 = x * r;
                    const float e = fmaf(-q0, s, x);
                    const float q1 = fmaf(e, r, q0);
                    const float q = x / s;
                    uint32_t b1, b2;
                    memcpy(&b1, &q1, 4);
                    memcpy(&b2, &q, 4);
                    if (b1 != b2 && !(q1 == 0.0f && q == 0.0f))
                        ++bad;
                    if (fabsf(rintf(q1)) > qmax)
                        ++clamped;
                    ++checked;
                }
            }
        }
        printf("qmax=%d checked=%ld mismatches=%ld beyond_qmax=%ld\n", qmaxes[qi], checked, bad, clamped);
        total_bad += bad + clamped;
    }
    return total_bad ? 1 : 0;
}
