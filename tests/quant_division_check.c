/* Host check of the route-BS quantiser's quotient (csrc/quant.hip): for a scale s = RN(amax/448)
 * of at least 2^-90 the kernel computes RN(x/s) as Markstein's correction of a product,
 *     y = RN(1/s),  q0 = RN(x*y),  r = x - q0*s (one fused multiply-add),  q = RN(q0 + r*y),
 * which is the correctly rounded quotient when y is correctly rounded and the residual r is
 * exact (P. Markstein, "Computation of elementary functions on the IBM RISC System/6000
 * processor", IBM J. Res. Dev. 34(1), 1990). This program compares q with the IEEE quotient x/s
 * (a) for every finite bf16 x with |x| <= amax under every positive finite bf16 amax whose scale
 * is at least 2^-90, and (b) on random fp32 pairs, counting a difference only where it could
 * change the e4m3 code: both values below the code's zero-rounding threshold 2^-10 map to zero.
 * Exit status 0: no difference. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static float from_bits(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t to_bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

static int differs(float x, float s)
{
    const float y = 1.0f / s;
    const float q0 = x * y;
    const float q = fmaf(fmaf(-q0, s, x), y, q0);
    const float ref = x / s;
    if (to_bits(q) == to_bits(ref))
        return 0;
    return !(fabsf(ref) < 0x1p-11f && fabsf(q) < 0x1p-10f);
}

int main(void)
{
    long long pairs = 0, bad = 0;
    for (uint32_t ha = 1; ha < 0x7f80u; ++ha) { /* every positive finite bf16 amax */
        const float amax = from_bits(ha << 16);
        const float s = amax / 448.0f;
        if (s < 0x1p-90f)
            continue;
        for (uint32_t hx = 0; hx < 0x7f80u; ++hx) { /* |x| <= amax, both signs */
            const float x = from_bits(hx << 16);
            if (x > amax)
                break;
            pairs += 2;
            bad += differs(x, s) + differs(-x, s);
        }
    }
    printf("bf16 pairs %lld, differences %lld\n", pairs, bad);
    /* random fp32 pairs: amax with a random finite exponent, x uniform in [-amax, amax] */
    uint64_t st = 0x9E3779B97F4A7C15ull;
    long long rpairs = 0, rbad = 0;
    for (long long i = 0; i < 100000000LL; ++i) {
        st ^= st << 13; st ^= st >> 7; st ^= st << 17;
        const uint32_t ea = (uint32_t)(st % 254u) + 1u, ma = (uint32_t)(st >> 9) & 0x7fffffu;
        const float amax = from_bits((ea << 23) | ma);
        const float s = amax / 448.0f;
        if (s < 0x1p-90f || !isfinite(s))
            continue;
        st ^= st << 13; st ^= st >> 7; st ^= st << 17;
        const float x = amax * ((float)(st >> 40) * 0x1p-24f) * ((st & 1) ? -1.0f : 1.0f);
        ++rpairs;
        rbad += differs(x, s);
    }
    printf("random fp32 pairs %lld, differences %lld\n", rpairs, rbad);
    return (bad || rbad) ? 1 : 0;
}
