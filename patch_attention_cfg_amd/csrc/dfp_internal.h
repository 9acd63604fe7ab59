// dfp_internal.h -- sizes shared between the C-ABI translation units of
// libdfp (workspace planning).  Not part of the public ABI.
#pragma once

#include <stddef.h>
#include <stdint.h>

size_t dfp_cfg_workspace_bytes(int64_t n_per_image, int batch);
size_t dfp_attn_workspace_bytes(int B, int H, int n_q, int N_kv, int d);
// The bf16 launcher's plan for these sizes (attention_bf16.hip): key groups
// per workgroup, workgroups per query tile, attention workgroups.
void dfp_attn_bf16_plan(int BH, int n_q, int N_kv, int d, bool can_split, int *key_groups,
                        int *splits, int64_t *workgroups);

#include "dfp.h"

// Fresh rows of a dfp_patch_attention_fresh call: up to two validated,
// non-overlapping ranges of whole 64-key tiles, read instead of the buffer
// and, when land is set, copied into k_buf / v_buf_t by the same launch.
struct dfp_fresh_launch {
    const dfp_fresh_rows *ranges;
    int count;
    void *k_buf;   // the buffer, written when land is set
    void *v_buf_t;
    int land;
};

// bf16 MFMA attention launcher (attention_bf16.hip); arguments already
// validated by the ABI entry points.  fresh is NULL for plain attention
// over the buffer.
dfp_status dfp_attn_bf16_launch(void *o, const void *q, const void *k, const void *vt, int BH,
                                int n_q, int N_kv, int d, float scale, void *ws, size_t ws_bytes,
                                const dfp_fresh_launch *fresh, hipStream_t stream);
