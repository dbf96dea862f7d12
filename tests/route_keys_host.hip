// Host-side check of the two helpers the top-k selections rank logits with
// (selection_value, f32_order_key in moe_internal.h): built by hipcc as an
// ordinary host program and run on the CPU by tests/test_route_keys_cpu.py.
// Prints one line per failed check and exits with the number of failures.
#include <math.h>
#include <stdio.h>
#include <string.h>

#include "moe_internal.h"

using bqmoe::f32_order_key;
using bqmoe::selection_value;

static int failures = 0;

static void expect(bool ok, const char *what, float a, float b) {
    if (!ok) {
        printf("FAIL %s: %a %a\n", what, a, b);
        ++failures;
    }
}

static float bits(uint32_t u) {
    float f;
    memcpy(&f, &u, 4);
    return f;
}

int main() {
    // NaN of either sign and any payload ranks as -inf; numbers are unchanged
    const float nans[] = {NAN, -NAN, bits(0x7F800001u), bits(0xFFFFFFFFu), bits(0x7FC00123u)};
    for (float n : nans) {
        const float v = selection_value(n);
        expect(v == -INFINITY, "NaN ranks as -inf", n, v);
        expect(f32_order_key(v) == f32_order_key(-INFINITY), "NaN key is the -inf key", n, v);
    }
    // ascending values (the zeros tie); every key is above 0, the key of
    // padded slots past the last expert
    const float asc[] = {-INFINITY, -3.4028235e38f, -1.0f, -1e-30f, -1.4e-45f, -0.0f, 0.0f,
                         1.4e-45f, 1.1754942e-38f, 1e-30f, 1.0f, 1.0000001f, 3.4028235e38f,
                         INFINITY};
    const int n = sizeof(asc) / sizeof(asc[0]);
    for (int i = 0; i < n; ++i) {
        expect(selection_value(asc[i]) == asc[i], "numbers keep their value", asc[i], asc[i]);
        expect(f32_order_key(asc[i]) > 0u, "keys are above the padding key", asc[i], asc[i]);
        for (int j = 0; j < n; ++j) {
            const bool gt = asc[i] > asc[j], eq = asc[i] == asc[j];
            expect((f32_order_key(asc[i]) > f32_order_key(asc[j])) == gt, "key order is float order",
                   asc[i], asc[j]);
            expect((f32_order_key(asc[i]) == f32_order_key(asc[j])) == eq, "equal keys iff equal",
                   asc[i], asc[j]);
        }
    }
    printf("%d failures\n", failures);
    return failures;
}
