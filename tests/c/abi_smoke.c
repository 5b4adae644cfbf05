/* A plain C99 caller of libgdn: includes gdn.h with no HIP or C++ headers,
 * links against libgdn.so and checks the host-side contract (version, status
 * strings, validation before any device work). */
#include <stdio.h>
#include <string.h>

#include "gdn.h"

int main(void) {
    if (gdn_abi_version() != GDN_ABI_VERSION) {
        printf("abi version %d, header %d\n", gdn_abi_version(), GDN_ABI_VERSION);
        return 1;
    }
    if (strlen(gdn_strerror(GDN_ERR_ALIAS)) == 0) return 2;
    /* every required pointer NULL: rejected on the host, nothing launched */
    int rc = gdn_record(NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL,
                        1, 1, 1, 1, 128, 128, GDN_BF16, GDN_GQA_BLOCK, NULL);
    if (rc != GDN_ERR_NULL || strncmp(gdn_last_error(), "gdn_record:", 11) != 0) return 3;
    rc = gdn_replay(NULL, NULL, NULL, NULL, NULL, NULL, 1, 1, 1, 128, 128, 1, GDN_F16, NULL);
    if (rc != GDN_ERR_NULL) return 4;
    rc = gqa_expand((const void*)64, (void*)4096, 0, 1, 2, 8, GDN_F32, GDN_GQA_TILED, NULL);
    if (rc != GDN_ERR_ZERO_DIM) return 5;
    rc = rms_norm_bf16(NULL, NULL, NULL, 1, 8, 1e-6f, NULL);
    if (rc != GDN_ERR_NULL) return 6;
    printf("c abi ok\n");
    return 0;
}
