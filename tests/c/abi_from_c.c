/* A plain C11 caller of the library: compiles against include/dfp.h alone,
 * links libdfp.so, and calls host-side entry points (no GPU needed). */
#include <stdio.h>

#include "dfp.h"

int main(void) {
    double c_x = 0.0, c_e = 0.0;
    if (dfp_ddim_coeffs(0.5, 0.75, &c_x, &c_e) != DFP_OK) return 1;
    printf("ddim %.17g %.17g\n", c_x, c_e);
    if (dfp_euler_coeffs(0.5, 0.25, &c_x, &c_e) != DFP_OK) return 2;
    printf("euler %.17g %.17g\n", c_x, c_e);
    printf("status %s\n", dfp_status_string(DFP_ERR_INVALID_ARG));
    printf("ws %zu\n", dfp_workspace_bytes(DFP_OP_CFG_STEP, 921600, 1, 0, 0, 0, 0, 0));
    printf("ldv %lld\n", (long long)dfp_v_ld(57600, DFP_BF16));
    /* validation happens before any launch: null tensors are refused */
    if (dfp_cfg_step(NULL, NULL, NULL, 16, 1, 7.5f, 1.0, 0.0, NULL, NULL, 0, NULL) !=
        DFP_ERR_INVALID_ARG)
        return 3;
    if (dfp_patch_attention(NULL, NULL, NULL, NULL, 1, 1, 8, 64, 64, 0.125f, DFP_BF16, NULL, 0,
                            NULL) != DFP_ERR_INVALID_ARG)
        return 4;
    printf("ok\n");
    return 0;
}
