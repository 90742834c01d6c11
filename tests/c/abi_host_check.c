/*
 * Plain C consumer of the q4 C ABI (no Python, no torch): compiled with gcc
 * against include/q4.h and linked to libq4stream.so.  Host-only calls, so
 * it runs without a GPU: version, argument validation of every product
 * entry point (nothing is enqueued on invalid arguments), the layer blob
 * layout, the offload placement rule and the decoder workspace size.
 * Exit status 0 when every check holds; prints the first failure.
 */
#include <stdio.h>
#include <string.h>

#include "q4.h"

#define CHECK(cond)                                                                   \
    do {                                                                              \
        if (!(cond)) {                                                                \
            fprintf(stderr, "check failed at line %d: %s (last error: %s)\n", __LINE__, \
                    #cond, q4_last_error());                                          \
            return 1;                                                                 \
        }                                                                             \
    } while (0)

int main(void) {
    CHECK(q4_abi_version() == Q4_ABI_VERSION);
    /* argument errors come back before any GPU work */
    CHECK(q4_pack(NULL, (uint8_t *)4096, 4, 64, NULL) == Q4_ERR_INVALID_ARG);
    CHECK(q4_gemv((const uint8_t *)4096, (const uint16_t *)4096, (const uint16_t *)4096,
                  (float *)4096, 4, 48, NULL) == Q4_ERR_INVALID_ARG); /* K % 32 */
    CHECK(strstr(q4_last_error(), "q4_gemv") != NULL);
    CHECK(q4_gemm_smallbatch((const uint8_t *)4096, (const uint16_t *)4096,
                             (const uint16_t *)4096, (float *)4096, 4, 64, 17, NULL) ==
          Q4_ERR_INVALID_ARG); /* B > 16 */
    CHECK(q4_quantize((const void *)4096, 7, (uint8_t *)4096, (uint16_t *)4096, 4, 64, NULL) ==
          Q4_ERR_INVALID_ARG); /* dtype */

    /* layer blob layout: eight 256-byte aligned sections in order */
    q4_layer shapes;
    memset(&shapes, 0, sizeof shapes);
    shapes.qkv.N = 128; shapes.qkv.K = 64;
    shapes.o.N = 64; shapes.o.K = 64;
    shapes.gate_up.N = 192; shapes.gate_up.K = 64;
    shapes.down.N = 64; shapes.down.K = 96;
    size_t off[8], bytes = 0;
    CHECK(q4_layer_blob_layout(&shapes, off, &bytes) == Q4_OK);
    for (int i = 0; i < 8; ++i) {
        CHECK(off[i] % 256 == 0);
        if (i)
            CHECK(off[i] > off[i - 1]);
    }
    CHECK(off[1] == 4096);          /* qkv codes 128 * 32 bytes */
    CHECK(bytes % 256 == 0 && bytes > off[7]);

    /* placement: 10 layers of 100 bytes, budget of 6 layers -> 4 resident */
    int32_t resident[10], k = -1;
    CHECK(q4_offload_plan(10, 100, 600, resident, &k) == Q4_OK);
    CHECK(k == 4);
    int count = 0;
    for (int l = 0; l < 10; ++l)
        count += resident[l];
    CHECK(count == 4 && resident[1] && resident[3] && resident[6] && resident[8]);
    CHECK(q4_offload_plan(10, 100, 150, resident, &k) == Q4_ERR_UNSUPPORTED);

    /* decoder workspace size: 2 layers, d 64, 4 heads, 2 kv heads, hd 16, dff 96 */
    q4_model_desc m;
    memset(&m, 0, sizeof m);
    m.n_layers = 2; m.d_model = 64; m.n_heads = 4; m.n_kv_heads = 2; m.head_dim = 16;
    m.d_ff = 96; m.eps = 1e-5f;
    size_t ws = 0;
    CHECK(q4_decoder_workspace_bytes(&m, &ws) == Q4_OK);
    CHECK(ws == 256 + 512 + 256 + 256 + 16896 + 256);
    m.n_heads = 3;
    CHECK(q4_decoder_workspace_bytes(&m, &ws) == Q4_ERR_INVALID_ARG);
    printf("q4 C ABI host checks passed (ABI version %d)\n", q4_abi_version());
    return 0;
}
