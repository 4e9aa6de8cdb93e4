/* consumer.c -- a plain C99 program against the Echo C ABI (include/echo.h).
 * It uses only the calls that need no GPU: sizes, error strings, and
 * argument checks that the library performs before any HIP call.  Prints
 * "ok" and exits 0 when every check holds, else names the first failure. */
#include <stdio.h>
#include <string.h>

#include "echo.h"

static int failures = 0;
#define CHECK(cond)                                                   \
    do {                                                              \
        if (!(cond)) {                                                \
            printf("FAIL line %d: %s\n", __LINE__, #cond);           \
            ++failures;                                               \
        }                                                             \
    } while (0)

int main(void) {
    echo_config c;
    echo_seg segs[ECHO_MAX_RANKS];
    static uint16_t x[64] __attribute__((aligned(16)));
    static float state[128] __attribute__((aligned(16)));
    static uint8_t codes[64] __attribute__((aligned(16)));
    static uint32_t params[4] __attribute__((aligned(16)));
    int p;

    memset(&c, 0, sizeof c);
    c.bits = 4;
    c.group = ECHO_GROUP;
    c.in_dtype = ECHO_IN_BF16;
    c.out_dtype = ECHO_OUT_BF16;
    c.state_dtype = ECHO_STATE_F32;
    c.eta = 1.0f;
    c.beta_short = 0.5f;
    c.beta_long = 0.9f;
    c.mix_long = 0.0125f;
    for (p = 0; p < ECHO_MAX_RANKS; ++p) {
        segs[p].codes = codes;
        segs[p].params = params;
    }

    /* segment length: whole groups, ceil(ceil(n/P)/group)*group */
    CHECK(echo_segment_len(8 * 128 * 5, 8, 128) == 640);
    CHECK(echo_segment_len(1000, 4, 128) == 256);
    CHECK(echo_segment_len(1, 16, 32) == 32);
    CHECK(echo_segment_len(536870912LL, 8, 128) == 67108864LL);
    CHECK(echo_segment_len(0, 8, 128) == 0);
    CHECK(echo_segment_len(100, 17, 128) == 0);
    CHECK(echo_segment_len(100, 4, 96) == 0);

    /* payload and state sizes */
    CHECK(echo_codes_bytes(67108864LL, 4) == 33554432u);
    CHECK(echo_codes_bytes(256, 8) == 256u);
    CHECK(echo_codes_bytes(256, 5) == 0u);
    CHECK(echo_params_bytes(67108864LL, 128) == 2097152u);
    CHECK(echo_params_bytes(256, 32) == 32u);
    CHECK(echo_state_bytes(1000, ECHO_STATE_F32) == 8000u);
    CHECK(echo_state_bytes(1000, ECHO_STATE_BF16) == 4000u);

    /* argument checks that return before any GPU work */
    CHECK(echo_quantize_feedback(NULL, 2, 0, 256, x, state, segs, NULL) == ECHO_ERR_ARG);
    c.bits = 5;
    CHECK(echo_quantize_feedback(&c, 2, 0, 256, x, state, segs, NULL) == ECHO_ERR_ARG);
    c.bits = 4;
    CHECK(echo_quantize_feedback(&c, 2, 2, 256, x, state, segs, NULL) == ECHO_ERR_ARG);
    CHECK(echo_quantize_feedback(&c, 17, 0, 256, x, state, segs, NULL) == ECHO_ERR_ARG);
    CHECK(echo_quantize_feedback(&c, 2, 0, 0, x, state, segs, NULL) == ECHO_ERR_SHAPE);
    CHECK(echo_quantize_feedback(&c, 2, 0, 256, (const uint8_t*)x + 2, state, segs, NULL)
          == ECHO_ERR_ALIGN);
    CHECK(echo_owner_reduce_requant(&c, 2, 0, 256, x, state, segs, NULL, NULL) == ECHO_ERR_ARG);
    CHECK(echo_dequant_gather(&c, 2, 256, NULL, x, NULL) == ECHO_ERR_ARG);
    c.beta_short = 1.0f;
    CHECK(echo_dequant_gather(&c, 2, 256, segs, x, NULL) == ECHO_ERR_ARG);
    c.beta_short = 0.5f;
    CHECK(echo_state_reset(&c, state, -1, NULL) == ECHO_ERR_ARG);
    CHECK(echo_state_reset(&c, (uint8_t*)state + 4, 16, NULL) == ECHO_ERR_ALIGN);

    /* error strings are static and distinct */
    CHECK(strlen(echo_error_string(ECHO_OK)) > 0);
    CHECK(strcmp(echo_error_string(ECHO_ERR_ARG), echo_error_string(ECHO_ERR_SHAPE)) != 0);
    CHECK(strcmp(echo_error_string(ECHO_ERR_ALIGN), echo_error_string(ECHO_ERR_HIP)) != 0);
    CHECK(echo_error_string(12345) != NULL);

    if (failures) return 1;
    printf("ok\n");
    return 0;
}
