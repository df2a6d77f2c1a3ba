/* A plain C99 client of the boundary, compiled against include/streamattn.h alone and linked to
 * libstreamattn.so. It does host work only: the rolling-cache slot rule and position map, and
 * argument validation (every device call below is rejected before anything is launched, or is
 * an empty no-op). Prints "ok" and exits 0 when every check holds. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "streamattn.h"

static int fails = 0;
#define CHECK(c)                                                              \
    do {                                                                      \
        if (!(c)) {                                                           \
            fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c);   \
            ++fails;                                                          \
        }                                                                     \
    } while (0)

int main(void) {
    /* chunks of 4 rows, one 4-row sink chunk, a 3-chunk (12-row) window: the sink chunk stays at
       row 0, later chunks cycle over rows 4, 8, 12 and evict the oldest window chunk */
    const int64_t slot[8] = {0, 4, 8, 12, 4, 8, 12, 4};
    for (int c = 0; c < 8; ++c) {
        int64_t base = -1;
        int vis = -1;
        CHECK(kv_cache_slot(c, 4, 4, 12, &base, &vis) == SA_OK);
        CHECK(base == slot[c]);
        CHECK(vis == ((c + 1) * 4 < 16 ? (c + 1) * 4 : 16));
    }
    /* after chunk 5 the visible chunks in arrival order are 0 (sink), 3, 4, 5, stored in rows
       0-3, 12-15, 4-7 and 8-11 */
    int64_t rows[16];
    const int64_t logical[16] = {0, 1, 2, 3, 8, 9, 10, 11, 12, 13, 14, 15, 4, 5, 6, 7};
    CHECK(kv_cache_positions(5, 4, 4, 12, rows, 16) == SA_OK);
    CHECK(memcmp(rows, logical, sizeof(rows)) == 0);
    CHECK(kv_cache_positions(5, 4, 4, 12, rows, 15) == SA_ERR_RANGE);
    CHECK(kv_cache_slot(-1, 4, 4, 12, rows, (int*)rows) == SA_ERR_RANGE);
    CHECK(kv_cache_slot(0, 4, 4, 12, NULL, NULL) == SA_ERR_NULL);

    /* validation: fake but aligned device addresses, rejected before any launch */
    void* p = (void*)(uintptr_t)4096;
    CHECK(attn_forward(p, p, p, p, 1, 8, 8, 16, 16, 96, 0.1f, 0, NULL) == SA_ERR_UNSUPPORTED);
    CHECK(strlen(sa_last_error()) > 0);
    CHECK(attn_forward(NULL, p, p, p, 1, 8, 8, 16, 16, 128, 0.1f, 0, NULL) == SA_ERR_NULL);
    CHECK(attn_forward(p, p, p, p, 1, 6, 4, 16, 16, 128, 0.1f, 0, NULL) == SA_ERR_SHAPE);
    CHECK(attn_forward((char*)p + 2, p, p, p, 1, 8, 8, 16, 16, 128, 0.1f, 0, NULL) == SA_ERR_ALIGN);
    CHECK(attn_forward_window(p, p, p, p, 1, 8, 8, 16, 16, 128, 0.1f, 3, -2, 16 * 8 * 128, SA_DTYPE_BF16, NULL) ==
          SA_ERR_RANGE);
    CHECK(attn_forward_qnorm(p, p, p, p, NULL, 1e-6f, NULL, SA_ROPE_NONE, 1, 8, 8, 16, 16, 128, 0.1f, -1, -1,
                             16 * 8 * 128, SA_DTYPE_BF16, NULL, 0, NULL) == SA_ERR_NULL);
    CHECK(qk_norm_rope_v(NULL, NULL, 0, NULL, NULL, 0, NULL, NULL, 0, NULL, NULL, NULL, NULL, 1, 16, 8, 8, 128, 1e-6f,
                         SA_NORM_HEAD, SA_ROPE_NONE, SA_DTYPE_BF16, NULL) == SA_ERR_NULL);
    CHECK(attn_forward_workspace_bytes(96) == SA_ERR_UNSUPPORTED);
    /* empty problems are successful no-ops, whatever the pointers */
    CHECK(attn_forward(NULL, NULL, NULL, NULL, 1, 8, 8, 0, 16, 128, 0.1f, 0, NULL) == SA_OK);
    CHECK(strlen(sa_last_error()) == 0);

    if (fails) return 1;
    printf("ok\n");
    return 0;
}
