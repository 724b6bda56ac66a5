// router.hip -- router logits, top-k selection, normalised weights and the
// shared-expert gate.
//
// The layer's first four steps (Qwen3.8-Flash-Next anatomy page on
// frontier-model-atlas, "Decoder microscope", Feed-forward panel): router
// logits, softmax, top-k routed experts, normalisation of the selected
// weights; plus the shared expert's own sigmoid gate.
//
// Logits are accumulated in binary32 in a fixed order so that the integer
// top-k decision is reproducible bit for bit: 64 partial sums, element kk
// feeds partial (kk mod 512) div 8, each partial folds its elements in
// ascending kk with one fused multiply-add, partials are combined by
// acc[j] += acc[j+s] for s = 32..1, the bias is added last.  On a wave64 this
// is lane j holding partial j and reading 8 consecutive elements per 512-wide
// chunk: one coalesced 16-byte load per lane.
//
// For many tokens the exact logits of all experts cost E dot products per
// token on the vector ALUs.  The shortlist router instead computes
// f = x W_r^T on MFMA (binary32 accumulate, the hardware's own order), which
// is within Delta_e of the exact canonical logit l_e, and recomputes l_e
// exactly only for experts that can still reach the top k:
//   tau = k-th largest f_e, Delta_A = max Delta over those k experts,
//   S = { e : f_e + Delta_e >= tau - Delta_A }.
// The k experts with the largest f have l >= tau - Delta_A, so the k-th
// largest l is at least that; any expert of the exact top k then has
// f_e >= l_e - Delta_e >= tau - Delta_A - Delta_e, i.e. it is in S.  The
// top k of S under the exact order (l desc, e asc) is therefore the exact
// top k.  Delta_e = coef ||x_t|| ||W_r[e]|| + 2^-22 |f_e| bounds the two
// summation errors (each at most n u sum|x_k w_k| <= n u ||x|| ||w||, with
// u = 2^-23 allowing truncating adds in the MFMA) plus the bias roundings,
// with a factor 2 to spare.  When S has more than 32 experts the exact
// logits of all experts are computed instead.
//
// The selected weights use the identity softmax(l)_i / sum_sel softmax(l) =
// exp(l_i - l_max) / sum_sel exp(l_j - l_max): the full softmax denominator
// cancels, so only the k selected logits are needed.
#include "moe_device.h"
#include "moe_kernels.h"
#include "router_select.h"

#include <math.h>

#pragma clang fp contract(off)

namespace moe {

// Rows 0..E-1 of the extended router matrix are W_r, row E is the shared gate
// vector g (absent when g == nullptr).  Block (tx, ry) owns tokens
// [TT tx, TT tx + TT) and rows [4 RW ry, 4 RW ry + 4 RW); each wave owns RW rows.
// The grid is one-dimensional over ntg token groups and nry_pad (a multiple
// of 8) row groups.  Workgroups go to the 8 XCDs round robin (block b on XCD
// b % 8), so block b takes row group 8 ((b / 8) / ntg) + b % 8 and token
// group (b / 8) mod ntg: every row group stays on one XCD, whose L2 serves its
// W_r rows to all token groups (one HBM read of W_r instead of one per XCD).
// Row groups at or past nry have nothing to do.  A grid capped below the
// number of blocks (a multiple of 8, so b and blockIdx.x share an XCD) walks
// the blocks with a stride of gridDim.x.
// The block's token rows are staged in LDS.  For bf16 rows of at most
// kMaxChunks 512-element chunks, all of a row's chunk loads are issued before
// any arithmetic, so a row costs one memory round trip.
constexpr int kMaxChunks = 8;

//
// touch (null unless the select step marks the touched experts): block (0, 0)
// clears its 32-word map for the select launch that follows.
template <typename T, int TT, int RW>
__device__ __forceinline__ void router_logits_block(
    const T *__restrict__ x, const T *__restrict__ w_router, const T *__restrict__ g,
    const float *__restrict__ bias, float *__restrict__ logits, int64_t ntok, int d, int E,
    int64_t tx, int ry, T *xs) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int64_t t0 = tx * TT;
    const int ntt = (int)min<int64_t>(TT, ntok - t0);

    const bool vec = (d % 8) == 0;
    const bool preload = vec && sizeof(T) == 2 && d <= 512 * kMaxChunks;
    // The first row's weight chunks do not depend on x: their loads go out
    // before the token rows are staged.
    uint4 wq[kMaxChunks];
    if (preload) {
        const int row = ry * 4 * RW + wave * RW;
        const T *wrow = row < E ? w_router + (int64_t)row * d : (row == E ? g : nullptr);
#pragma unroll
        for (int c = 0; c < kMaxChunks; ++c) {
            const int kk0 = 512 * c + 8 * lane;
            wq[c] = wrow && kk0 < d ? *reinterpret_cast<const uint4 *>(wrow + kk0)
                                    : make_uint4(0, 0, 0, 0);
        }
    }

    if ((d * (int)sizeof(T)) % 16 == 0) {
        // whole rows are 16-byte multiples: copy the contiguous [ntt, d] slab,
        // eight loads in flight per thread before their stores
        const int per_row = d * (int)sizeof(T) / 16;
        const uint4 *src = reinterpret_cast<const uint4 *>(x + t0 * d);
        uint4 *dst = reinterpret_cast<uint4 *>(xs);
        for (int i0 = threadIdx.x; i0 < TT * per_row; i0 += 256 * 8) {
            uint4 v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int i = i0 + 256 * u;
                v[u] = i < ntt * per_row ? src[i] : make_uint4(0, 0, 0, 0);
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int i = i0 + 256 * u;
                if (i < TT * per_row) dst[i] = v[u];
            }
        }
    } else {
        for (int i = threadIdx.x; i < TT * d; i += 256) {
            int tt = i / d;
            xs[i] = tt < ntt ? x[(t0 + tt) * d + (i - tt * d)] : T(0);
        }
    }
    __syncthreads();

    for (int rr = 0; rr < RW; ++rr) {
        const int row = ry * 4 * RW + wave * RW + rr;
        if (row > E || (row == E && g == nullptr)) break;
        const T *wrow = row < E ? w_router + (int64_t)row * d : g;
        float acc[TT];
#pragma unroll
        for (int tt = 0; tt < TT; ++tt) acc[tt] = 0.0f;
        if (preload) {
            if (rr > 0) {
#pragma unroll
                for (int c = 0; c < kMaxChunks; ++c) {
                    const int kk0 = 512 * c + 8 * lane;
                    wq[c] = kk0 < d ? *reinterpret_cast<const uint4 *>(wrow + kk0)
                                    : make_uint4(0, 0, 0, 0);
                }
            }
#pragma unroll
            for (int c = 0; c < kMaxChunks; ++c) {
                const int kk0 = 512 * c + 8 * lane;
                if (512 * c >= d) break;
                if (kk0 < d) {
                    const uint32_t q4[4] = {wq[c].x, wq[c].y, wq[c].z, wq[c].w};
#pragma unroll
                    for (int tt = 0; tt < TT; ++tt) {
                        float xv[8];
                        load8(xs + tt * d + kk0, xv);
#pragma unroll
                        for (int q = 0; q < 8; ++q) {
                            const float wv = (q & 1) ? bf16_hi(q4[q >> 1]) : bf16_lo(q4[q >> 1]);
                            acc[tt] = __builtin_fmaf(xv[q], wv, acc[tt]);
                        }
                    }
                }
            }
        } else {
            for (int chunk = 0; chunk < d; chunk += 512) {
                const int kk0 = chunk + 8 * lane;
                if (kk0 >= d) continue;
                float wv[8];
                if (vec) {
                    load8(wrow + kk0, wv);
                } else {
#pragma unroll
                    for (int q = 0; q < 8; ++q) wv[q] = kk0 + q < d ? to_f32(wrow[kk0 + q]) : 0.0f;
                }
#pragma unroll
                for (int tt = 0; tt < TT; ++tt) {
                    float xv[8];
                    if (vec) {
                        load8(xs + tt * d + kk0, xv);
                    } else {
#pragma unroll
                        for (int q = 0; q < 8; ++q)
                            xv[q] = kk0 + q < d ? to_f32(xs[tt * d + kk0 + q]) : 0.0f;
                    }
#pragma unroll
                    for (int q = 0; q < 8; ++q)
                        if (kk0 + q < d) acc[tt] = __builtin_fmaf(xv[q], wv[q], acc[tt]);
                }
            }
        }
#pragma unroll
        for (int tt = 0; tt < TT; ++tt) {
            float a = acc[tt];
            for (int s = 32; s >= 1; s >>= 1) {
                float o = __shfl_down(a, s, kWave);
                a = a + o;
            }
            acc[tt] = a;
        }
        if (lane == 0) {
            const float b = (row < E && bias) ? bias[row] : 0.0f;
            for (int tt = 0; tt < ntt; ++tt)
                logits[(t0 + tt) * (E + 1) + row] = acc[tt] + b;
        }
    }
}

template <typename T, int TT, int RW>
__global__ __launch_bounds__(256) void router_logits_kernel(
    const T *__restrict__ x, const T *__restrict__ w_router, const T *__restrict__ g,
    const float *__restrict__ bias, float *__restrict__ logits, int64_t ntok, int d, int E,
    int64_t ntg, int nry, int64_t nblk, int32_t *__restrict__ touch) {
    extern __shared__ __align__(16) unsigned char smem_raw[];
    T *xs = reinterpret_cast<T *>(smem_raw);  // [TT][d]
    for (int64_t b = blockIdx.x; b < nblk; b += gridDim.x) {
        const int64_t bj = b >> 3;
        const int64_t tx = bj % ntg;
        const int ry = (int)(8 * (bj / ntg) + (b & 7));
        if (ry >= nry) continue;  // uniform over the block
        if (touch && tx == 0 && ry == 0 && threadIdx.x < 32) touch[threadIdx.x] = 0;
        if (b != blockIdx.x) __syncthreads();  // the last block's reads of xs are done
        router_logits_block<T, TT, RW>(x, w_router, g, bias, logits, ntok, d, E, tx, ry, xs);
    }
}

// One wave per token: top-k by (logit desc, expert asc), weights, gate
// (select_topk in router_select.h).  With touch (its 32 words cleared by the
// logits launch, E <= 1024): every selected expert e sets bit e % 32 of word
// e / 32, the map of touched experts that the weight-streaming kernels read.
// The block's four tokens are merged in LDS first, so each block sends at
// most one atomic OR per word.
template <int NV>
__global__ __launch_bounds__(256) void router_select_kernel(
    const float *__restrict__ logits, int64_t ntok, int E, int k, int has_gate,
    int32_t *__restrict__ topk_idx, float *__restrict__ topk_w, float *__restrict__ gate,
    float *__restrict__ gate_user, int32_t *__restrict__ touch) {
    __shared__ uint32_t map[32];
    const int lane = threadIdx.x & 63;
    const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (touch) {
        if (threadIdx.x < 32) map[threadIdx.x] = 0;
        __syncthreads();
    }
    if (t < ntok) {
        const int e = select_topk<NV>(logits + t * (E + 1), E, k, lane, topk_idx + t * k,
                                      topk_w + t * k, has_gate ? gate + t : nullptr,
                                      has_gate && gate_user ? gate_user + t : nullptr, nullptr);
        if (touch && lane < k) atomicOr(&map[e >> 5], 1u << (e & 31));
    }
    if (touch) {
        __syncthreads();
        if (threadIdx.x < 32 && map[threadIdx.x])
            atomicOr(reinterpret_cast<unsigned int *>(touch) + threadIdx.x, map[threadIdx.x]);
    }
}

// Exact canonical logit for the token whose 512-chunk slices this wave holds
// (lane j: elements 512 c + 8 j .. + 8 of chunk c), from the matching slices
// wq of one router row; the same order as router_logits_kernel, so the bits
// agree.
template <int NC>
__device__ __forceinline__ float canonical_dot(const uint4 (&xs)[NC], const uint4 (&wq)[NC],
                                               int d, int lane, float b) {
    float acc = 0.0f;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        const int kk0 = 512 * c + 8 * lane;
        if (kk0 < d) {
            const uint32_t x4[4] = {xs[c].x, xs[c].y, xs[c].z, xs[c].w};
            const uint32_t w4[4] = {wq[c].x, wq[c].y, wq[c].z, wq[c].w};
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const float xv = (q & 1) ? bf16_hi(x4[q >> 1]) : bf16_lo(x4[q >> 1]);
                const float wv = (q & 1) ? bf16_hi(w4[q >> 1]) : bf16_lo(w4[q >> 1]);
                acc = __builtin_fmaf(xv, wv, acc);
            }
        }
    }
    for (int s = 32; s >= 1; s >>= 1) {
        float o = __shfl_down(acc, s, kWave);
        acc = acc + o;
    }
    return __shfl(acc, 0, kWave) + b;
}

// This lane's slices of router row wrow; slices past d read slice 0 (a valid
// address; canonical_dot never uses them).
template <int NC>
__device__ __forceinline__ void load_row_slices(const uint16_t *wrow, int d, int lane,
                                                uint4 (&wq)[NC]) {
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        const int kk0 = 512 * c + 8 * lane;
        wq[c] = *reinterpret_cast<const uint4 *>(wrow + (kk0 < d ? kk0 : 0));
    }
}

template <int NC>
__device__ __forceinline__ float canonical_logit(const uint4 (&xs)[NC], const uint16_t *wrow,
                                                 int d, int lane, float b) {
    uint4 wq[NC];
    load_row_slices<NC>(wrow, d, lane, wq);
    return canonical_dot<NC>(xs, wq, d, lane, b);
}

// Shortlist candidates whose exact logits are computed together: their row
// loads are all in flight before the first dot product.  Two (one for rows
// longer than 4096), with the kernel held to 128 VGPRs (4 waves per SIMD) for
// d <= 2560, measured fastest at T = 4096, d = 2560: larger batches cost
// occupancy, and this kernel is latency-bound.
template <int NC> constexpr int cand_batch() { return NC <= 8 ? 2 : 1; }

// Wave-wide argmax under (value desc, expert asc); every lane gets the result.
__device__ __forceinline__ void wave_best(float &bv, int &be) {
    for (int o = 32; o >= 1; o >>= 1) {
        const float ov = __shfl_xor(bv, o, kWave);
        const int oe = __shfl_xor(be, o, kWave);
        if (ov > bv || (ov == bv && oe < be)) {
            bv = ov;
            be = oe;
        }
    }
}

// One wave per token; NV = ceil(E / 64) logits per lane, NC >= ceil(d / 512).
template <int NV, int NC>
__global__ __launch_bounds__(256, NC <= 5 ? 4 : 1) void router_select_shortlist_kernel(
    float *__restrict__ f, const float *__restrict__ wnorm, const uint16_t *__restrict__ x,
    const uint16_t *__restrict__ w_router, const uint16_t *__restrict__ g,
    const float *__restrict__ bias, int64_t ntok, int d, int E, int k, int nsplit, float coef,
    int32_t *__restrict__ topk_idx, float *__restrict__ topk_w, float *__restrict__ gate,
    float *__restrict__ gate_user) {
    __shared__ int s_cand[4][32];
    const int lane = threadIdx.x & 63;
    const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= ntok) return;

    // this lane's slices of x_t, ||x_t||^2 and g . x_t
    uint4 xs[NC];
    float xx = 0.f, zg = 0.f;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        const int kk0 = 512 * c + 8 * lane;
        xs[c] = make_uint4(0, 0, 0, 0);
        if (kk0 < d) {
            xs[c] = *reinterpret_cast<const uint4 *>(x + t * d + kk0);
            float xv[8];
            load8(x + t * d + kk0, xv);
#pragma unroll
            for (int q = 0; q < 8; ++q) xx += xv[q] * xv[q];
            if (g) {
                float gv[8];
                load8(g + kk0, gv);
#pragma unroll
                for (int q = 0; q < 8; ++q) zg += xv[q] * gv[q];
            }
        }
    }
    const float xnorm = sqrtf(wave_sum(xx));
    if (g) zg = wave_sum(zg);

    const float *ft = f + t * (E + 1);
    // column E (not written by the GEMM): the shared gate's logit in slice
    // 0, zeros in the others, so that the logits buffer carries x [W_r; g]^T
    // as K-slice partials (the training forward keeps it for the backward)
    if (lane < nsplit) f[((int64_t)lane * ntok + t) * (E + 1) + E] = lane == 0 ? zg : 0.0f;
    float fb[NV], dl[NV];
    uint32_t removed = 0;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int e = lane + 64 * i;
        if (e < E) {
            // f: the K slices' partial sums, added in slice order
            float fe = ft[e];
            for (int s = 1; s < nsplit; ++s) fe = fe + ft[(int64_t)s * ntok * (E + 1) + e];
            const float v = fe + (bias ? bias[e] : 0.0f);
            fb[i] = (v == v) ? v : -INFINITY;
            dl[i] = coef * xnorm * wnorm[e] + 0x1p-22f * fabsf(fb[i]);
        } else {
            fb[i] = -INFINITY;
            dl[i] = 0.f;
            removed |= 1u << i;
        }
    }

    // tau and Delta_A from the k largest approximate logits: per round a DPP
    // wave maximum, the lowest expert holding it by ballot, and that expert's
    // Delta read from its lane (taken candidates become NaN)
    float tau = 0.f, dA = 0.f;
    {
        float fr[NV];
#pragma unroll
        for (int i = 0; i < NV; ++i) fr[i] = ((removed >> i) & 1u) ? __builtin_nanf("") : fb[i];
        for (int j = 0; j < k; ++j) {
            float lm = fr[0];
#pragma unroll
            for (int i = 1; i < NV; ++i) lm = fmaxf(lm, fr[i]);
            const float m = wave_max_dpp(lm);
            int e = 0;
#pragma unroll
            for (int i = 0; i < NV; ++i) {
                const uint64_t hit = __ballot(fr[i] == m);
                if (hit) {
                    e = 64 * i + (int)__builtin_ctzll(hit);
                    break;
                }
            }
            float mine = 0.f;
#pragma unroll
            for (int i = 0; i < NV; ++i) {
                if (i == (e >> 6)) mine = dl[i];
                if (e == lane + 64 * i) fr[i] = __builtin_nanf("");
            }
            dA = fmaxf(dA, __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mine), e & 63)));
            tau = m;
        }
    }
    const float theta = tau - dA;
    int count = 0;
    uint64_t pass[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        pass[i] = __ballot(!((removed >> i) & 1u) && fb[i] + dl[i] >= theta);
        count += __popcll(pass[i]);
    }

    float my_l = 0.f;
    int my_e = 0;
    // fewer than k candidates happens only when fewer than k approximate
    // logits are finite (an infinite bias makes f + Delta NaN): the exact
    // pass over every expert then decides, as it does for the oracle
    if (count >= k && count <= 32) {
        // the shortlist in ascending expert order, candidate c at cand[c]
        int *cand = s_cand[threadIdx.x >> 6];
        {
            int base = 0;
            const uint64_t below = (1ull << lane) - 1;
#pragma unroll
            for (int i = 0; i < NV; ++i) {
                if ((pass[i] >> lane) & 1ull) cand[base + __popcll(pass[i] & below)] = 64 * i + lane;
                base += __popcll(pass[i]);
            }
        }
        __builtin_amdgcn_wave_barrier();
        // exact logits of the shortlist, CB rows in flight at a time;
        // candidate c lives in lane c
        float lc = -INFINITY;
        int ec = 0x7FFFFFFF;
        constexpr int CB = cand_batch<NC>();
        for (int c0 = 0; c0 < count; c0 += CB) {
            int e[CB];
            uint4 wq[CB][NC];
            float b[CB];
#pragma unroll
            for (int u = 0; u < CB; ++u) {
                e[u] = cand[min(c0 + u, count - 1)];
                load_row_slices<NC>(w_router + (int64_t)e[u] * d, d, lane, wq[u]);
                b[u] = bias ? bias[e[u]] : 0.0f;
            }
#pragma unroll
            for (int u = 0; u < CB; ++u) {
                const float l = canonical_dot<NC>(xs, wq[u], d, lane, b[u]);
                if (lane == c0 + u) {
                    lc = (l == l) ? l : -INFINITY;
                    ec = e[u];
                }
            }
        }
        // top k of the shortlist: DPP maximum, lowest lane (= lowest expert,
        // candidates being in ascending order) holding it, which drops out
        if (lane >= count) lc = __builtin_nanf("");
        for (int j = 0; j < k; ++j) {
            const float mx = wave_max_dpp(lc);
            const int wl = (int)__builtin_ctzll(__ballot(lc == mx));
            const int be = __builtin_amdgcn_readlane(ec, wl);
            if (lane == wl) lc = __builtin_nanf("");
            if (lane == j) {
                my_l = mx;
                my_e = be;
            }
        }
    } else {
        // exact logits of every expert, lane-strided as in the plain router
        float lv[NV];
#pragma unroll
        for (int i = 0; i < NV; ++i) lv[i] = -INFINITY;
        for (int e = 0; e < E; ++e) {
            const float l = canonical_logit<NC>(xs, w_router + (int64_t)e * d, d, lane,
                                                bias ? bias[e] : 0.0f);
            if ((e & 63) == lane) {
#pragma unroll
                for (int i = 0; i < NV; ++i)
                    if (i == (e >> 6)) lv[i] = (l == l) ? l : -INFINITY;
            }
        }
        uint32_t rem = removed;
        for (int j = 0; j < k; ++j) {
            float bv = -INFINITY;
            int be = 0x7FFFFFFF;
#pragma unroll
            for (int i = 0; i < NV; ++i) {
                const int e = lane + 64 * i;
                if (!((rem >> i) & 1u) && (lv[i] > bv || (lv[i] == bv && e < be))) {
                    bv = lv[i];
                    be = e;
                }
            }
            wave_best(bv, be);
            if ((be & 63) == lane) rem |= 1u << (be >> 6);
            if (lane == j) {
                my_l = bv;
                my_e = be;
            }
        }
    }
    const float lmax = __shfl(my_l, 0, kWave);
    const float ex = lane < k ? expf(my_l - lmax) : 0.0f;
    const float z = wave_sum(ex);
    if (lane < k) {
        topk_idx[t * k + lane] = my_e;
        topk_w[t * k + lane] = ex / z;
    }
    if (g && lane == 0) {
        const float s = 1.0f / (1.0f + expf(-zg));
        gate[t] = s;
        if (gate_user) gate_user[t] = s;
    }
}

// s_t = sigmoid(g . x_t): one wave per token (routing-given entry point).
template <typename T>
__global__ __launch_bounds__(256) void shared_gate_kernel(const T *__restrict__ x,
                                                          const T *__restrict__ g,
                                                          float *__restrict__ gate,
                                                          int64_t ntok, int d) {
    const int lane = threadIdx.x & 63;
    const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= ntok) return;
    float a = 0.0f;
    for (int kk = lane; kk < d; kk += 64) a += to_f32(x[t * d + kk]) * to_f32(g[kk]);
    a = wave_sum(a);
    if (lane == 0) gate[t] = 1.0f / (1.0f + expf(-a));
}

// Pre-FFN RMSNorm, one wave per row (4 rows per block), evaluated in a fixed
// binary32 order so that the routed bits match the definition's reading:
// lane j holds partial j of sum h_k^2 exactly as in the router logit
// (element kk feeds partial (kk mod 512) / 8, ascending kk, fused
// multiply-adds from +0, then the halving tree); mean = ss / d,
// v = mean + eps, r = 1 / sqrtf(v) with the division and square root
// correctly rounded (HIP's default binary32 semantics, which the build keeps);
// x_k = (h_k r) gamma_k, each product rounded, then rounded to the dtype.
template <typename T>
__global__ __launch_bounds__(256) void rmsnorm_kernel(const T *__restrict__ h,
                                                      const T *__restrict__ gamma, float eps,
                                                      T *__restrict__ x, int64_t ntok, int d) {
    const int lane = threadIdx.x & 63;
    const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= ntok) return;
    const T *hr = h + t * d;
    T *xr = x + t * d;
    const bool vec = (d % 8) == 0;
    if (vec && d <= 512 * kMaxChunks) {
        // the whole row and gamma in registers: one load round trip, vector stores
        float v[kMaxChunks][8], gw[kMaxChunks][8];
        float acc = 0.0f;
#pragma unroll
        for (int c = 0; c < kMaxChunks; ++c) {
            const int kk0 = 512 * c + 8 * lane;
            if (kk0 < d) {
                load8(hr + kk0, v[c]);
                load8(gamma + kk0, gw[c]);
            }
        }
#pragma unroll
        for (int c = 0; c < kMaxChunks; ++c)
            if (512 * c + 8 * lane < d)
#pragma unroll
                for (int q = 0; q < 8; ++q) acc = __builtin_fmaf(v[c][q], v[c][q], acc);
        for (int s = 32; s >= 1; s >>= 1) {
            float o = __shfl_down(acc, s, kWave);
            acc = acc + o;
        }
        const float r = 1.0f / sqrtf(__shfl(acc, 0, kWave) / (float)d + eps);
#pragma unroll
        for (int c = 0; c < kMaxChunks; ++c) {
            const int kk0 = 512 * c + 8 * lane;
            if (kk0 >= d) continue;
            float o[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) o[q] = (v[c][q] * r) * gw[c][q];
            if constexpr (sizeof(T) == 2) {
                *reinterpret_cast<uint4 *>(xr + kk0) =
                    make_uint4(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]),
                               pack_bf16x2(o[4], o[5]), pack_bf16x2(o[6], o[7]));
            } else {
                *reinterpret_cast<float4 *>(xr + kk0) = make_float4(o[0], o[1], o[2], o[3]);
                *reinterpret_cast<float4 *>(xr + kk0 + 4) = make_float4(o[4], o[5], o[6], o[7]);
            }
        }
        return;
    }
    float acc = 0.0f;
    for (int c = 0; c < d; c += 512) {
        const int kk0 = c + 8 * lane;
        if (kk0 >= d) continue;
        float v[8];
        if (vec) {
            load8(hr + kk0, v);
        } else {
#pragma unroll
            for (int q = 0; q < 8; ++q) v[q] = kk0 + q < d ? to_f32(hr[kk0 + q]) : 0.0f;
        }
#pragma unroll
        for (int q = 0; q < 8; ++q)
            if (kk0 + q < d) acc = __builtin_fmaf(v[q], v[q], acc);
    }
    for (int s = 32; s >= 1; s >>= 1) {
        float o = __shfl_down(acc, s, kWave);
        acc = acc + o;
    }
    const float ss = __shfl(acc, 0, kWave);
    const float mean = ss / (float)d;
    const float r = 1.0f / sqrtf(mean + eps);
    for (int kk = lane; kk < d; kk += 64) {
        const float xv = (to_f32(hr[kk]) * r) * to_f32(gamma[kk]);
        if constexpr (sizeof(T) == 2) xr[kk] = f32_to_bf16_rne(xv);
        else xr[kk] = xv;
    }
}

hipError_t launch_rmsnorm(const void *h, const void *gamma, float eps, void *x, int64_t T, int d,
                          bool bf16, hipStream_t s) {
    const dim3 grid((unsigned)((T + 3) / 4)), block(256);
    if (bf16)
        hipLaunchKernelGGL((rmsnorm_kernel<uint16_t>), grid, block, 0, s,
                           static_cast<const uint16_t *>(h), static_cast<const uint16_t *>(gamma),
                           eps, static_cast<uint16_t *>(x), T, d);
    else
        hipLaunchKernelGGL((rmsnorm_kernel<float>), grid, block, 0, s,
                           static_cast<const float *>(h), static_cast<const float *>(gamma), eps,
                           static_cast<float *>(x), T, d);
    return hipGetLastError();
}

// Few tokens: one row per wave (more blocks in flight); many: four.
template <typename T>
static hipError_t launch_logits(const Problem &p, hipStream_t s) {
    const size_t row_bytes = (size_t)p.d * sizeof(T);
    const dim3 block(256);
    const T *x = static_cast<const T *>(p.x);
    const T *wr = static_cast<const T *>(p.w_router);
    const T *g = static_cast<const T *>(p.sh_gate);
#define MOE_LOGITS(TT, RW)                                                                       \
    do {                                                                                         \
        const int64_t ntg = (p.T + TT - 1) / TT;                                                 \
        const int nry = (p.E + 1 + 4 * RW - 1) / (4 * RW);                                        \
        const int64_t nblk = ntg * ((nry + 7) / 8 * 8);                                           \
        const dim3 gr((unsigned)(nblk < ((int64_t)1 << 22) ? nblk : ((int64_t)1 << 22)));         \
        hipLaunchKernelGGL((router_logits_kernel<T, TT, RW>), gr, block, TT * row_bytes, s, x,   \
                           wr, g, p.router_bias, p.logits, p.T, p.d, p.E, ntg, nry, nblk,        \
                           p.direct ? p.counts : nullptr);                                       \
    } while (0)
    if (p.T <= 64) {
        // fewer tokens per block: more blocks in flight for a small batch
        if (4 * row_bytes <= 65536) MOE_LOGITS(4, 1);
        else if (2 * row_bytes <= 65536) MOE_LOGITS(2, 1);
        else MOE_LOGITS(1, 1);
    } else if (p.T <= 256) {
        if (8 * row_bytes <= 65536) MOE_LOGITS(8, 1);
        else if (4 * row_bytes <= 65536) MOE_LOGITS(4, 1);
        else if (2 * row_bytes <= 65536) MOE_LOGITS(2, 1);
        else MOE_LOGITS(1, 1);
    } else {
        if (8 * row_bytes <= 65536) MOE_LOGITS(8, 4);
        else if (4 * row_bytes <= 65536) MOE_LOGITS(4, 4);
        else if (2 * row_bytes <= 65536) MOE_LOGITS(2, 4);
        else MOE_LOGITS(1, 4);
    }
#undef MOE_LOGITS
    return hipGetLastError();
}

static hipError_t launch_shortlist(const Problem &p, float *sh_gate_user, hipStream_t s) {
    hipError_t err = launch_router_gemm(p, s);  // logits and row norms
    if (err != hipSuccess) return err;
    const int nchunk = (p.d + 511) / 512;
    const int nc = (p.d + 511) / 512;
    const double u = 1.0 / 8388608.0;  // 2^-23
    const float coef = (float)(2.0 * (p.d * u + (8.0 * nchunk + 7.0) * u));
    const int nv = (p.E + 63) / 64;
    const dim3 grid((unsigned)((p.T + 3) / 4)), block(256);
    const uint16_t *x = static_cast<const uint16_t *>(p.x);
    const uint16_t *wr = static_cast<const uint16_t *>(p.w_router);
    const uint16_t *g = static_cast<const uint16_t *>(p.sh_gate);
#define MOE_SL(NV, NC)                                                                          \
    hipLaunchKernelGGL((router_select_shortlist_kernel<NV, NC>), grid, block, 0, s, p.logits,   \
                       p.wnorm, x, wr, g, p.router_bias, p.T, p.d, p.E, p.k, p.router_split,    \
                       coef, p.topk_idx,                                                        \
                       p.topk_w, p.gate, sh_gate_user)
#define MOE_SL_NV(NC)                                                                           \
    do {                                                                                        \
        if (nv <= 1) MOE_SL(1, NC);                                                             \
        else if (nv <= 2) MOE_SL(2, NC);                                                        \
        else if (nv <= 4) MOE_SL(4, NC);                                                        \
        else if (nv <= 8) MOE_SL(8, NC);                                                        \
        else MOE_SL(16, NC);                                                                    \
    } while (0)
    if (nc <= 1) MOE_SL_NV(1);
    else if (nc <= 2) MOE_SL_NV(2);
    else if (nc <= 5) MOE_SL_NV(5);
    else if (nc <= 8) MOE_SL_NV(8);
    else if (nc <= 16) MOE_SL_NV(16);
    else MOE_SL_NV(32);
#undef MOE_SL_NV
#undef MOE_SL
    return hipGetLastError();
}

hipError_t launch_router(const Problem &p, float *sh_gate_user, hipStream_t s) {
    if (p.router == 1) return launch_shortlist(p, sh_gate_user, s);
    hipError_t err = p.bf16 ? launch_logits<uint16_t>(p, s) : launch_logits<float>(p, s);
    if (err != hipSuccess) return err;
    const int nv = (p.E + 63) / 64;
    const dim3 grid((unsigned)((p.T + 3) / 4)), block(256);
    const int has_gate = p.sh_gate != nullptr;
#define MOE_SELECT(NV)                                                                        \
    hipLaunchKernelGGL((router_select_kernel<NV>), grid, block, 0, s, p.logits, p.T, p.E, p.k, \
                       has_gate, p.topk_idx, p.topk_w, p.gate, sh_gate_user,                  \
                       p.direct ? p.counts : nullptr)
    if (nv <= 1) MOE_SELECT(1);
    else if (nv <= 2) MOE_SELECT(2);
    else if (nv <= 4) MOE_SELECT(4);
    else if (nv <= 8) MOE_SELECT(8);
    else MOE_SELECT(16);
#undef MOE_SELECT
    return hipGetLastError();
}

hipError_t launch_shared_gate(const Problem &p, hipStream_t s) {
    const dim3 grid((unsigned)((p.T + 3) / 4)), block(256);
    if (p.bf16)
        hipLaunchKernelGGL((shared_gate_kernel<uint16_t>), grid, block, 0, s,
                           static_cast<const uint16_t *>(p.x),
                           static_cast<const uint16_t *>(p.sh_gate), p.gate, p.T, p.d);
    else
        hipLaunchKernelGGL((shared_gate_kernel<float>), grid, block, 0, s,
                           static_cast<const float *>(p.x), static_cast<const float *>(p.sh_gate),
                           p.gate, p.T, p.d);
    return hipGetLastError();
}

}  // namespace moe
