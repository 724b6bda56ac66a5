// router_select.h -- top-k selection of one token by one wave (internal).
//
// Top-k of a token's router logits by (logit desc, expert asc), the
// normalised weights of the selected experts and the shared gate (Qwen3.8-
// Flash-Next anatomy page on frontier-model-atlas, "Decoder microscope",
// Feed-forward panel: router logits, softmax, top-k, selected-weight
// normalisation).  The weights use softmax(l)_i / sum_sel softmax(l) =
// exp(l_i - l_max) / sum_sel exp(l_j - l_max): the full denominator cancels.
#pragma once

#include "moe_device.h"

#include <math.h>

namespace moe {

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_max_step(float x) {
    const int o = __builtin_amdgcn_update_dpp(__float_as_int(x), __float_as_int(x), CTRL, ROW_MASK,
                                              0xF, false);
    return fmaxf(x, __int_as_float(o));
}

// Maximum of v over the wave, in every lane: quad permutes, row rotates and
// row broadcasts (DPP) leave the full maximum in lane 63.
__device__ __forceinline__ float wave_max_dpp(float v) {
    v = dpp_max_step<0xB1, 0xF>(v);   // quad_perm [1,0,3,2]
    v = dpp_max_step<0x4E, 0xF>(v);   // quad_perm [2,3,0,1]
    v = dpp_max_step<0x124, 0xF>(v);  // row_ror:4
    v = dpp_max_step<0x128, 0xF>(v);  // row_ror:8
    v = dpp_max_step<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
    v = dpp_max_step<0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// One wave selects for the token whose E (+1 gate) logits start at l.  Lane L
// holds the logits of experts L, L+64, ..., so a lane's candidates are
// already in ascending expert order.  Writes idx[0..k) (descending logit),
// w[0..k), and *gate_t / *gate_user_t (when non-null) = sigmoid(l[E]);
// idx_copy (non-null) receives idx too.  Returns, in lane j < k, the j-th
// selected expert.
template <int NV>
__device__ __forceinline__ int select_topk(const float *__restrict__ l, int E, int k, int lane,
                                           int32_t *idx, float *w, float *gate_t,
                                           float *gate_user_t, int32_t *idx_copy) {
#pragma clang fp contract(off)
    // Candidates still in play hold their logit; taken ones (and padding
    // past E) hold NaN, which fmaxf skips and == never matches.  NaN logits
    // are read as -inf first, so NaN marks only "not a candidate".  The gate
    // logit goes out with the others.
    float v[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int e = lane + 64 * i;
        const float val = e < E ? l[e] : __builtin_nanf("");
        v[i] = e < E && val != val ? -INFINITY : val;
    }
    const float lg = gate_t ? l[E] : 0.0f;

    float my_l = 0.0f;
    int my_e = 0;
    for (int j = 0; j < k; ++j) {
        // largest remaining logit (a DPP max over the wave) ...
        float lm = v[0];
#pragma unroll
        for (int i = 1; i < NV; ++i) lm = fmaxf(lm, v[i]);
        const float m = wave_max_dpp(lm);
        // ... and the lowest expert holding it: expert lane + 64 i grows with
        // i first, then with the lane
        int e = 0;
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const uint64_t hit = __ballot(v[i] == m);
            if (hit) {
                e = 64 * i + (int)__builtin_ctzll(hit);
                break;
            }
        }
#pragma unroll
        for (int i = 0; i < NV; ++i)
            if (e == lane + 64 * i) v[i] = __builtin_nanf("");
        if (lane == j) {
            my_l = m;
            my_e = e;
        }
    }
    const float lmax = __shfl(my_l, 0, kWave);
    const float ex = lane < k ? expf(my_l - lmax) : 0.0f;
    const float z = wave_sum(ex);
    if (lane < k) {
        idx[lane] = my_e;
        w[lane] = ex / z;
        if (idx_copy) idx_copy[lane] = my_e;
    }
    if (gate_t && lane == 0) {
        const float s = 1.0f / (1.0f + expf(-lg));
        *gate_t = s;
        if (gate_user_t) *gate_user_t = s;
    }
    return my_e;
}

}  // namespace moe
