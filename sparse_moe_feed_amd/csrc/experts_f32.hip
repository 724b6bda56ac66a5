// experts_f32.hip -- grouped SwiGLU experts for binary32 layers (plain FMA).
//
// Same maths as the bfloat16 path (gated MLP with SiLU per expert, weighted
// combine plus the sigmoid-gated shared expert; anatomy page on
// frontier-model-atlas, "Decoder microscope", Feed-forward panel) for small
// binary32 layers: one block per permuted row, threads across the outputs.
// h stays binary32.  Routed rows land in y (weighted), the shared expert's
// term in out; the combine kernel adds them.
#include "moe_device.h"
#include "moe_kernels.h"

namespace moe {

struct F32Args {
    const float *x, *w_gu, *w_dn, *w_sgu, *w_sdn;
    float *h, *h_sh, *out, *y;
    float *au, *au_sh;  // pre-activations [a | u] (training forward), or null
    const int32_t *perm, *offsets;
    const float *topk_w, *gate;
    int64_t T;
    int d, E, k, F, Fs;
};

// Row r of the routed region belongs to the largest g with offsets[g] <= r.
__device__ int group_of_row(const int32_t *offsets, int E, int r) {
    int lo = 0, hi = E;
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (offsets[mid] <= r) lo = mid;
        else hi = mid;
    }
    return lo;
}

// Resolve block row -> (token, expert weights, h row, width); false if the
// row is unused.  Routed rows come first ([0, T*k)), then the T shared rows.
__device__ bool resolve_row(const F32Args &a, int64_t r, int64_t &tok, int &grp, int &width,
                            float *&hrow, float &wgt, float *&dst) {
    const int64_t routed = a.T * a.k;
    if (r < routed) {
        if (r >= a.offsets[a.E]) return false;
        grp = group_of_row(a.offsets, a.E, (int)r);
        const int pair = a.perm[r];
        tok = pair / a.k;
        wgt = a.topk_w[pair];
        width = a.F;
        hrow = a.h + r * a.F;
        dst = a.y + r * a.d;
    } else {
        if (a.Fs == 0) return false;
        tok = r - routed;
        grp = a.E;
        wgt = a.gate[tok];
        width = a.Fs;
        hrow = a.h_sh + tok * a.Fs;
        dst = a.out + tok * a.d;
    }
    return true;
}

__global__ __launch_bounds__(256) void f32_gateup_kernel(F32Args a) {
    int64_t tok;
    int grp, width;
    float *hrow, *dst;
    float wgt;
    if (!resolve_row(a, blockIdx.x, tok, grp, width, hrow, wgt, dst)) return;
    const float *W = grp < a.E ? a.w_gu + (int64_t)grp * 2 * a.F * a.d : a.w_sgu;
    const float *xr = a.x + tok * a.d;
    for (int n = threadIdx.x; n < width; n += blockDim.x) {
        const float *wg = W + (int64_t)n * a.d;
        const float *wu = W + (int64_t)(width + n) * a.d;
        float g = 0.f, u = 0.f;
        for (int kk = 0; kk < a.d; ++kk) {
            g = fmaf(wg[kk], xr[kk], g);
            u = fmaf(wu[kk], xr[kk], u);
        }
        hrow[n] = silu_mul(g, u);
        if (a.au) {  // training forward: the pre-activations too
            float *arow = grp < a.E ? a.au + (int64_t)blockIdx.x * 2 * a.F : a.au_sh + tok * 2 * a.Fs;
            arow[n] = g;
            arow[width + n] = u;
        }
    }
}

__global__ __launch_bounds__(256) void f32_down_kernel(F32Args a) {
    int64_t tok;
    int grp, width;
    float *hrow, *dst;
    float wgt;
    if (!resolve_row(a, blockIdx.x, tok, grp, width, hrow, wgt, dst)) return;
    const float *W = grp < a.E ? a.w_dn + (int64_t)grp * a.d * a.F : a.w_sdn;
    for (int m = threadIdx.x; m < a.d; m += blockDim.x) {
        const float *wr = W + (int64_t)m * width;
        float y = 0.f;
        for (int n = 0; n < width; ++n) y = fmaf(wr[n], hrow[n], y);
        dst[m] = wgt * y;
    }
}

hipError_t launch_experts_f32(const Problem &p, hipStream_t s,
                               const std::function<void(int)> &mark) {
    F32Args a;
    a.x = static_cast<const float *>(p.x);
    a.w_gu = static_cast<const float *>(p.w_gate_up);
    a.w_dn = static_cast<const float *>(p.w_down);
    a.w_sgu = static_cast<const float *>(p.w_sh_gate_up);
    a.w_sdn = static_cast<const float *>(p.w_sh_down);
    a.h = static_cast<float *>(p.h);
    a.h_sh = static_cast<float *>(p.h_shared);
    a.au = static_cast<float *>(p.au);
    a.au_sh = static_cast<float *>(p.au_sh);
    a.out = p.out;
    a.y = static_cast<float *>(p.y);
    a.perm = p.perm;
    a.offsets = p.offsets;
    a.topk_w = p.topk_w;
    a.gate = p.gate;
    a.T = p.T;
    a.d = p.d;
    a.E = p.E;
    a.k = p.k;
    a.F = p.F;
    a.Fs = p.Fs;
    const int64_t rows = p.T * p.k + p.T;
    hipLaunchKernelGGL(f32_gateup_kernel, dim3((unsigned)rows), dim3(64), 0, s, a);
    mark(3);
    hipLaunchKernelGGL(f32_down_kernel, dim3((unsigned)rows), dim3(256), 0, s, a);
    mark(4);
    return hipGetLastError();
}

}  // namespace moe
