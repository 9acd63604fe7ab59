// dfp_internal.h -- sizes shared between the C-ABI translation units of
// libdfp (workspace planning).  Not part of the public ABI.
#pragma once

#include <stddef.h>
#include <stdint.h>

size_t dfp_cfg_workspace_bytes(int64_t n_per_image, int batch);
size_t dfp_attn_workspace_bytes(int B, int H, int n_q, int N_kv, int d);

#include "dfp.h"

// bf16 MFMA attention launcher (attention_bf16.hip); arguments already
// validated by dfp_patch_attention.
dfp_status dfp_attn_bf16_launch(void *o, const void *q, const void *k, const void *vt, int BH,
                                int n_q, int N_kv, int d, float scale, void *ws, size_t ws_bytes,
                                hipStream_t stream);
