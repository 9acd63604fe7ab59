// host.cpp -- host-only helpers of the C ABI: status text, buffer strides,
// workspace sizes, and the fp64 sampler coefficients the fused step consumes.
#include <algorithm>
#include <cmath>
#include <cstdint>

#include "dfp.h"
#include "dfp_internal.h"

extern "C" {

const char *dfp_status_string(dfp_status s) {
    switch (s) {
    case DFP_OK: return "DFP_OK";
    case DFP_ERR_INVALID_ARG: return "DFP_ERR_INVALID_ARG: invalid argument";
    case DFP_ERR_UNSUPPORTED: return "DFP_ERR_UNSUPPORTED: shape or dtype not implemented";
    case DFP_ERR_HIP: return "DFP_ERR_HIP: the HIP runtime rejected a launch";
    case DFP_ERR_TOO_LARGE:
        return "DFP_ERR_TOO_LARGE: the request exceeds the library's static scratch buffer";
    }
    return "unknown dfp_status";
}

int64_t dfp_v_ld(int64_t N_buf, dfp_dtype dt) {
    if (N_buf <= 0) return 0;
    int64_t vec;
    if (dt == DFP_BF16) vec = 8;
    else if (dt == DFP_F32) vec = 4;
    else return 0;
    return (N_buf + vec - 1) / vec * vec;
}

// Sampler coefficients.  DDIM with eta = 0 (section 3 of "AIGC 文生图系统如何
// 优化扩散模型推理速度"): x0 = (x - sqrt(1-a_t) g) / sqrt(a_t) followed by
// x' = sqrt(a_p) x0 + sqrt(1-a_p) g is affine in (x, g); expanding it gives
// the two coefficients below.  a_p = 1 reproduces the final "return x0" step.
dfp_status dfp_ddim_coeffs(double abar_t, double abar_prev, double *c_x, double *c_e) {
    if (!c_x || !c_e) return DFP_ERR_INVALID_ARG;
    if (!(abar_t > 0.0 && abar_t <= 1.0) || !(abar_prev > 0.0 && abar_prev <= 1.0))
        return DFP_ERR_INVALID_ARG;
    const double st = std::sqrt(abar_t), sp = std::sqrt(abar_prev);
    *c_x = sp / st;
    *c_e = std::sqrt(1.0 - abar_prev) - sp * std::sqrt(1.0 - abar_t) / st;
    return DFP_OK;
}

dfp_status dfp_ddim_eta_coeffs(double abar_t, double abar_prev, double eta, double *c_x,
                               double *c_e, double *c_z) {
    if (!c_x || !c_e || !c_z) return DFP_ERR_INVALID_ARG;
    if (!(abar_t > 0.0 && abar_t < 1.0) || !(abar_prev > 0.0 && abar_prev <= 1.0) ||
        !(abar_t <= abar_prev) || !(eta >= 0.0) || !std::isfinite(eta))
        return DFP_ERR_INVALID_ARG;
    const double st = std::sqrt(abar_t), sp = std::sqrt(abar_prev);
    const double s2 = eta * eta * (1.0 - abar_prev) / (1.0 - abar_t) * (1.0 - abar_t / abar_prev);
    const double keep = 1.0 - abar_prev - s2;
    if (keep < 0.0) return DFP_ERR_INVALID_ARG;
    *c_x = sp / st;
    *c_e = std::sqrt(keep) - sp * std::sqrt(1.0 - abar_t) / st;
    *c_z = std::sqrt(s2);
    return DFP_OK;
}

dfp_status dfp_switch_points(const float *relmae, int S, int L, double g_slope, int k,
                             int *tau1, int *tau2) {
    if (!relmae || !tau1 || !tau2 || S < 1 || L < 1 || k < 0 || !std::isfinite(g_slope))
        return DFP_ERR_INVALID_ARG;
    int cap = 0;  // first step of the global minimum
    for (int t = 0; t < S; ++t) {
        if (!std::isfinite(relmae[t])) return DFP_ERR_INVALID_ARG;
        if (relmae[t] < relmae[cap]) cap = t;
    }
    int t1 = cap;
    for (int t = L; t < cap; ++t) {   // a flat point only matters before the cap
        const double G = ((double)relmae[t] - (double)relmae[t - L]) / (double)L;
        if (G >= 0.0 && G < g_slope) {
            t1 = t;
            break;
        }
    }
    *tau1 = t1;
    *tau2 = (int)std::min<int64_t>((int64_t)t1 + k, S);
    return DFP_OK;
}

dfp_status dfp_euler_coeffs(double sigma, double sigma_next, double *c_x, double *c_e) {
    if (!c_x || !c_e) return DFP_ERR_INVALID_ARG;
    if (!std::isfinite(sigma) || !std::isfinite(sigma_next)) return DFP_ERR_INVALID_ARG;
    *c_x = 1.0;
    *c_e = sigma_next - sigma;
    return DFP_OK;
}

dfp_status dfp_scaled_linear_abar(int T, double beta_start, double beta_end, double *abar) {
    if (!abar || T < 2 || !(beta_start >= 0.0) || !(beta_end >= 0.0) ||
        !(beta_start < 1.0) || !(beta_end < 1.0))
        return DFP_ERR_INVALID_ARG;
    const double r0 = std::sqrt(beta_start), r1 = std::sqrt(beta_end);
    double run = 1.0;
    for (int t = 0; t < T; ++t) {
        const double r = r0 + (r1 - r0) * (double)t / (double)(T - 1);
        run *= 1.0 - r * r;
        abar[t] = run;
    }
    return DFP_OK;
}

// Round-half-even of (T-1) i / (S-1) in exact integer arithmetic.
dfp_status dfp_ddim_timesteps(int T, int S, int *ts) {
    if (!ts || T < 1 || S < 1) return DFP_ERR_INVALID_ARG;
    if (S == 1) { ts[0] = 0; return DFP_OK; }
    const int64_t den = S - 1;
    for (int i = 0; i < S; ++i) {
        const int64_t num = (int64_t)(T - 1) * i;
        int64_t q = num / den;
        const int64_t twice_rem = 2 * (num % den);
        if (twice_rem > den || (twice_rem == den && (q & 1))) ++q;
        ts[i] = (int)q;
    }
    return DFP_OK;
}

size_t dfp_workspace_bytes(int op, int64_t n_per_image, int batch, int B, int H, int n_q,
                           int N_kv, int d) {
    switch (op) {
    case DFP_OP_CFG_STEP:
    case DFP_OP_RELMAE:
        return dfp_cfg_workspace_bytes(n_per_image, batch);
    case DFP_OP_PATCH_ATTENTION:
        return dfp_attn_workspace_bytes(B, H, n_q, N_kv, d);
    }
    return 0;
}

}  // extern "C"
