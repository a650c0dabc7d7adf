/* The C ABI used from C99: compiles against include/fa355.h alone, links
 * against libfa355.so, and exercises the calls that need no GPU (sizes,
 * status strings and host-side validation).  Prints one line per check and
 * exits non-zero on the first failure. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "fa355.h"

static int fails = 0;
#define CHECK(cond, what)                                   \
    do {                                                    \
        if (!(cond)) {                                      \
            printf("FAIL %s\n", what);                      \
            fails++;                                        \
        } else {                                            \
            printf("ok   %s\n", what);                      \
        }                                                   \
    } while (0)

int main(void)
{
    CHECK(fa_version() == FA355_VERSION, "version matches the header");
    CHECK(strcmp(fa_status_str(FA_ERR_WORKSPACE), "FA_ERR_WORKSPACE") == 0, "status string");
    CHECK(fa_decode_workspace_size(2, 3, 1000, 128, 4) == (size_t)2 * 3 * 4 * 129 * 4, "decode workspace size");
    CHECK(fa_bwd_workspace_size(1, 2, 100) == (size_t)1 * 2 * 100 * 8, "backward workspace size");
    /* a rejected call: head dim 96, no device pointer is touched */
    void *fake = (void *)(uintptr_t)(1ull << 32);
    int rc = fa_fwd(fake, fake, fake, fake, NULL, 1, 1, 64, 64, 96, 0, 0.125f, FA_F16, NULL);
    CHECK(rc == FA_ERR_UNSUPPORTED, "fa_fwd rejects d=96");
    CHECK(strstr(fa_last_error(), "d=96") != NULL, "last error names the cause");
    rc = fa_decode_paged(fake, fake, fake, (const int32_t *)fake, (const int32_t *)fake, fake, NULL, 1, 1, 128, 4, 16,
                         2, 7, 32, 0.1f, FA_F16, 0, fake, 1 << 20, NULL);
    CHECK(rc == FA_ERR_INVALID, "fa_decode_paged rejects an unknown layout");
    rc = fa_quantize_e4m3(fake, fake, 100, FA_BF16, NULL);
    CHECK(rc == FA_ERR_INVALID, "fa_quantize_e4m3 rejects overlapping buffers");
    return fails ? 1 : 0;
}
