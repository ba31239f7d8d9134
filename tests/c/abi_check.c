/* A plain C99 consumer of include/dwconv.h: the header compiles as C, the
 * library links and its host-side validation answers without a GPU (every
 * call below fails or returns before anything would be enqueued). */
#include <stdio.h>
#include <string.h>

#include "dwconv.h"

static int failures = 0;

static void expect(int cond, const char *what) {
    if (!cond) {
        printf("FAIL %s (last error: %s)\n", what, dw_last_error());
        ++failures;
    }
}

int main(void) {
    void *p = (void *)0x1000, *q = (void *)0x2000, *r = (void *)0x3000, *ws = (void *)0x4000;
    size_t need;

    expect(dw_abi_version() == DW_ABI_VERSION, "abi version");
    expect(strcmp(dw_last_error(), "") == 0, "no error yet");

    expect(dwconv1d_fwd(p, p, NULL, NULL, q, 2, 8, 4, 0, DW_PAD_SYMMETRIC, DW_F32, NULL) == DW_ERR_INVALID_ARG,
           "1-D K = 0");
    expect(strstr(dw_last_error(), "K=0") != NULL, "1-D K = 0 message");
    expect(dwconv1d_fwd(p, p, NULL, NULL, p, 2, 8, 4, 3, DW_PAD_CAUSAL, DW_BF16, NULL) == DW_ERR_INVALID_ARG,
           "1-D aliasing");
    expect(dwconv1d_fwd(p, p, NULL, NULL, q, 0, 8, 4, 3, DW_PAD_CAUSAL, DW_F32, NULL) == DW_OK, "1-D empty batch");

    expect(dwconv1d_stream_fwd(p, p, NULL, NULL, r, q, r, 2, 8, 4, 9, DW_BF16, NULL) == DW_ERR_INVALID_ARG,
           "stream cache in place");

    need = dwconv1d_bwd_workspace_bytes(32, 1500, 512, 9);
    expect(need > 0, "1-D bwd workspace");
    expect(dwconv1d_bwd(p, p, NULL, q, r, (float *)ws, NULL, ws, need - 1, 32, 1500, 512, 9, DW_PAD_CAUSAL, DW_F32,
                        NULL) == DW_ERR_WORKSPACE, "1-D bwd short workspace");
    expect(dwconv1d_bwd(p, p, NULL, q, r, NULL, NULL, NULL, 0, 32, 1500, 512, 6, DW_PAD_CAUSAL, DW_F32, NULL)
               == DW_ERR_UNSUPPORTED, "1-D bwd width 6");

    expect(dwsub_fused_fwd_ex(p, p, NULL, p, NULL, NULL, q, 4, 1000, 80, 256, (dw_pad)7, DW_BF16, NULL)
               == DW_ERR_INVALID_ARG, "front bad pad");
    need = dwsub_fused_bwd_workspace_bytes_ex(4, 1000, 80, 256, DW_PAD_CAUSAL);
    expect(need > 0 && need == dwsub_fused_bwd_workspace_bytes_ex(4, 1000, 80, 256, DW_PAD_CAUSAL), "front ws");

    expect(dwconv2d_fwd_ex(p, p, NULL, NULL, q, 2, 8, 8, 4, 3, 3, 2, 0, 1, 1, 1, DW_F32, NULL) == DW_ERR_UNSUPPORTED,
           "2-D pad before 0");
    expect(dwconv2d_fwd(p, p, NULL, NULL, q, 2, 8, 8, 4, 3, 3, 1, 1, NULL) == DW_ERR_UNSUPPORTED, "2-D stride 1");
    need = dwconv2d_bwd_workspace_bytes_ex(32, 1500, 64, 256, 3, 3, 2, 2, 1, 2, 1);
    expect(need > 0, "2-D bwd workspace");
    expect(dwconv2d_bwd_ex(p, p, NULL, q, r, (float *)ws, NULL, ws, need - 1, 32, 1500, 64, 256, 3, 3, 2, 2, 1, 2, 1,
                           DW_BF16, NULL) == DW_ERR_WORKSPACE, "2-D bwd short workspace");
    expect(dwconv2d_bwd(p, p, NULL, q, NULL, NULL, NULL, NULL, 0, 32, 1500, 64, 256, 3, 3, 2, 1, NULL) == DW_OK,
           "2-D bwd nothing requested");

    /* extents and size products that would overflow int64 are refused, not wrapped */
    const int64_t big = INT64_MAX;
    expect(dwconv1d_fwd(p, p, NULL, NULL, q, big, big, big, 9, DW_PAD_CAUSAL, DW_F32, NULL) == DW_ERR_UNSUPPORTED,
           "1-D huge extents");
    expect(dwconv1d_fwd(p, p, NULL, NULL, q, 2, (int64_t)1 << 30, (int64_t)1 << 30, 9, DW_PAD_CAUSAL, DW_F32,
                        NULL) == DW_ERR_UNSUPPORTED, "1-D item past 2^31 bytes");
    expect(dwconv2d_fwd(p, p, NULL, NULL, q, 1, (int64_t)1 << 30, (int64_t)1 << 30, 1 << 30, 3, 3, 2, 1, NULL)
               == DW_ERR_UNSUPPORTED, "2-D huge product");
    expect(dwconv2d_bwd_workspace_bytes(big, big, big, big, 3, 3, 2, 1) == 0, "2-D workspace of huge sizes");
    expect(dwconv1d_bwd_workspace_bytes(big, 1, 1, 9) == 0, "1-D workspace of huge B");
    expect(dwsub_fused_bwd_workspace_bytes(4, big, 80, 256) == 0, "front workspace of huge T");
    expect(dwsub_fused_fwd_ex(p, p, NULL, p, NULL, NULL, q, big, big, big, big, DW_PAD_SYMMETRIC, DW_F32, NULL)
               == DW_ERR_UNSUPPORTED, "front huge extents");
    /* enum values outside the named ones are refused */
    expect(dwconv1d_fwd(p, p, NULL, NULL, q, 2, 8, 4, 3, (dw_pad)-5, DW_F32, NULL) == DW_ERR_INVALID_ARG,
           "1-D negative pad");
    expect(dwconv1d_fwd(p, p, NULL, NULL, q, 2, 8, 4, 3, DW_PAD_CAUSAL, (dw_dtype)2, NULL) == DW_ERR_INVALID_ARG,
           "1-D dtype 2");
    expect(dwsub_fused_bwd_workspace_bytes_ex(4, 1000, 80, 256, (dw_pad)2) == 0, "front ws bad pad");

    if (failures == 0) printf("c abi check: ok\n");
    return failures == 0 ? 0 : 1;
}
