// experts_mx4_gemm.hip -- grouped SwiGLU expert GEMMs with packed MXFP4
// expert weights, for batches with many rows per expert (prefill).
//
// Same maths, tiles and epilogues as experts_dma.hip (gated MLP with SiLU,
// weighted rows y, the shared expert scaled by its sigmoid gate; anatomy page
// on frontier-model-atlas, "Decoder microscope", Feed-forward panel): tiles of
// 128 permuted rows of one group by 256 output columns (gate/up: 128 gate
// columns over the matching 128 up columns), 8 waves of 64 x 64 on
// v_mfma_f32_32x32x16_bf16 (two per SIMD, so one wave's LDS reads and fp4
// conversions overlap the other's MFMAs), three stage buffers filled by
// direct global -> LDS loads (global_load_lds), a barrier per K step.
//
// A K step is 128 elements, one packed weight tile column: the B stage is the
// 16 tiles (16 rows x 128 elements each) of the step's 256 weight rows, 1 KB
// of codes per tile copied verbatim (one 64-lane load each: the packed form is
// already in wave-load order) and the tiles' 64 scale bytes (one 4-byte load
// per lane covers four tiles; waves 4-7 repeat the loads of waves 0-3, which
// write the same bytes to the same place, so every wave issues the same
// number of loads and one wait count serves all).  Weights stay 4-bit in LDS: a B fragment (8
// consecutive k of one weight row) is 4 bytes of one 16-byte LDS chunk plus
// its scale byte, decoded exactly to bf16 by v_cvt_scalef32_pk_bf16_fp4 just
// before the MFMA.  The A stage holds 128 token rows of 256 bytes; chunk c of row R
// sits at chunk c ^ (R & 15), so the 16 rows of one read phase at one logical
// chunk cover all 64 banks.
#include "moe_device.h"
#include "moe_kernels.h"

#include <string.h>

namespace moe {

namespace {
constexpr int XBM = 128, XBN = 256, XBK = 128;  // tile rows, tile columns, K per step
constexpr int XNS = 3;                          // stage buffers
constexpr int XW = 8;                           // waves per block
constexpr int XNB = 2;                          // 32-column blocks per wave
constexpr int XMI = XBM / 64;                   // 32-row sub-tiles per wave
constexpr int XQ = XBK / 16;                    // k16 sub-steps per stage
constexpr int A_ROWB = XBK * 2;                 // bytes of a staged A row
constexpr int X_OPA = XBM * A_ROWB;             // 32 KB of A
constexpr int X_CODES = X_OPA;                  // 16 tiles x 1 KB of codes
constexpr int X_SCALES = X_OPA + 16 * 1024;     // 16 tiles x 64 scale bytes
constexpr int X_STB = X_SCALES + 16 * 64;       // stage bytes (50176)
constexpr int X_AL = X_OPA / (XW * 1024);       // A loads (1 KB each) per wave per stage
constexpr int X_CL = 16 / XW;                   // code tiles per wave per stage
constexpr int X_LOADS = X_AL + X_CL + 1;        // + 1 scale load
constexpr int XTILE = 1088;                     // bytes of one packed tile

typedef __attribute__((address_space(3))) void lds_void_t;
typedef const __attribute__((address_space(1))) void global_void_t;

constexpr int xvmcnt_imm(int n) { return (n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8); }
constexpr int xvmcnt_lgkm0_imm(int n) { return xvmcnt_imm(n) & ~(0xF << 8); }

__device__ __forceinline__ int a_off(int R, int c) { return R * A_ROWB + ((c ^ (R & 15)) << 4); }
__device__ __forceinline__ void xfence() { asm volatile("" ::: "memory"); }

struct XStages {
    unsigned char *s[XNS];
};

// Per-lane load addresses: A rows (element offsets, 32-bit: the host checks
// that they fit), the four code tiles of this wave and its scale piece (byte
// pointers at K step 0; step kt adds kt * XTILE).
struct XAddr {
    uint32_t aoff[X_AL];
    const uint8_t *code[X_CL];
    const uint8_t *scale;
};

__device__ __forceinline__ void x_dma_stage(unsigned char *stage, const uint16_t *abase,
                                            const XAddr &ad, int kt, int wave) {
#pragma unroll
    for (int j = 0; j < X_AL; ++j)
        __builtin_amdgcn_global_load_lds((const global_void_t *)(abase + ad.aoff[j] + XBK * kt),
                                         (lds_void_t *)(stage + (X_AL * wave + j) * 1024), 16, 0,
                                         0);
#pragma unroll
    for (int j = 0; j < X_CL; ++j)
        __builtin_amdgcn_global_load_lds((const global_void_t *)(ad.code[j] + (int64_t)XTILE * kt),
                                         (lds_void_t *)(stage + X_CODES + (X_CL * wave + j) * 1024),
                                         16, 0, 0);
    __builtin_amdgcn_global_load_lds((const global_void_t *)(ad.scale + (int64_t)XTILE * kt),
                                     (lds_void_t *)(stage + X_SCALES + 256 * (wave & 3)), 4, 0, 0);
}

struct XFrags {
    bf16x8 a[XMI], b[XNB];
};

// Codes and scale of the odd sub-step, kept from the even one: both read the
// same 16-byte chunk and scale byte.
struct XCarry {
    uint32_t w[XNB], x[XNB];
};

// Fragments of k16 sub-step ks: lane half h takes k = 16 ks + 8 h .. + 7 of
// its A row and of its B row (weight row n = brow + lane % 32: tile n / 16,
// row n % 16; those 8 codes are bytes 8 (ks & 1) + 4 h .. + 3 of chunk ks / 2).
template <int MACT>
__device__ __forceinline__ void x_read_frags(const unsigned char *stage, int ks, int wm,
                                             const int (&brow)[XNB], int fr, int half,
                                             XFrags &f, XCarry &cr) {
    if (MACT == 0) return;
#pragma unroll
    for (int mi = 0; mi < MACT; ++mi)
        f.a[mi] = *reinterpret_cast<const bf16x8 *>(stage + a_off(XBM / 2 * wm + 32 * mi + fr,
                                                                  2 * ks + half));
    const int c = ks >> 1;
#pragma unroll
    for (int ni = 0; ni < XNB; ++ni) {
        uint32_t w, x;
        if ((ks & 1) == 0) {
            const int n = brow[ni] + fr, tb = n >> 4, r = n & 15;
            // the whole 16-byte chunk (a 4-byte LDS read here makes the compiler
            // wait for every direct-to-LDS load in flight): dword half now,
            // dword 2 + half for the odd sub-step
            const uint4 q4 =
                *reinterpret_cast<const uint4 *>(stage + X_CODES + tb * 1024 + 16 * (r + 16 * c));
            x = stage[X_SCALES + 64 * tb + r + 16 * c];
            w = half ? q4.y : q4.x;
            cr.w[ni] = half ? q4.w : q4.z;
            cr.x[ni] = x;
        } else {
            w = cr.w[ni];
            x = cr.x[ni];
        }
        f.b[ni] = mx4_decode8(w, mx4_scale(x));
    }
}

template <int MACT>
__device__ __forceinline__ void x_mfma(const XFrags &f, f32x16 (&acc)[XMI][XNB]) {
#pragma unroll
    for (int mi = 0; mi < MACT; ++mi)
#pragma unroll
        for (int ni = 0; ni < XNB; ++ni)
            acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.b[ni], f.a[mi], acc[mi][ni], 0, 0, 0);
}

// MFMAs on cur while sub-step ks of stage goes to nxt.
template <int MACT>
__device__ __forceinline__ void x_sub(const unsigned char *stage, int ks, int wm,
                                      const int (&brow)[XNB], int fr, int half, const XFrags &cur,
                                      XFrags &nxt, XCarry &cr, f32x16 (&acc)[XMI][XNB]) {
    if (MACT > 0) {
        x_mfma<MACT>(cur, acc);
        x_read_frags<MACT>(stage, ks, wm, brow, fr, half, nxt, cr);
    }
    __builtin_amdgcn_sched_barrier(0);
}

// Sub-steps QQ .. XQ - 1 of one stage, fragments alternating between a and b.
template <int MACT, int QQ>
__device__ __forceinline__ void x_subs(const unsigned char *stage, int wm, const int (&brow)[XNB],
                                       int fr, int half, XFrags &a, XFrags &b, XCarry &cr,
                                       f32x16 (&acc)[XMI][XNB]) {
    if constexpr (QQ < XQ) {
        x_sub<MACT>(stage, QQ, wm, brow, fr, half, a, b, cr, acc);
        x_subs<MACT, QQ + 1>(stage, wm, brow, fr, half, b, a, cr, acc);
    }
}

// One K step kt on buffer S (as k_step in experts_dma.hip): MFMAs on sub-steps
// 0 .. XQ-2 while the next fragments are read; wait for this wave's LDS reads
// and for stage kt+1, barrier; refill buffer S with stage kt+XNS; last
// sub-step's MFMAs while stage kt+1's first fragments are read.  XQ is even,
// so the last sub-step's fragments are in f1.
template <int MACT, int S>
__device__ __forceinline__ void x_step(const XStages &st, int kt, int last, const uint16_t *abase,
                                       const XAddr &ad, int wave, int wm, const int (&brow)[XNB],
                                       int fr, int half, XFrags &f0, XFrags &f1, XCarry &cr,
                                       f32x16 (&acc)[XMI][XNB]) {
    x_subs<MACT, 1>(st.s[S], wm, brow, fr, half, f0, f1, cr, acc);
    xfence();
    __builtin_amdgcn_s_waitcnt(xvmcnt_lgkm0_imm((XNS - 2) * X_LOADS));
    __builtin_amdgcn_s_barrier();
    xfence();
    x_dma_stage(st.s[S], abase, ad, min(kt + XNS, last), wave);
    __builtin_amdgcn_sched_barrier(0);
    x_sub<MACT>(st.s[(S + 1) % XNS], 0, wm, brow, fr, half, f1, f0, cr, acc);
}

template <int MACT, int S>
__device__ __forceinline__ void x_steps(const XStages &st, int kt, int cnt, int last,
                                        const uint16_t *abase, const XAddr &ad, int wave, int wm,
                                        const int (&brow)[XNB], int fr, int half, XFrags &f0,
                                        XFrags &f1, XCarry &cr, f32x16 (&acc)[XMI][XNB]) {
    if constexpr (S < XNS) {
        if (S < cnt) {
            x_step<MACT, S>(st, kt + S, last, abase, ad, wave, wm, brow, fr, half, f0, f1, cr,
                            acc);
            x_steps<MACT, S + 1>(st, kt, cnt, last, abase, ad, wave, wm, brow, fr, half, f0, f1,
                                 cr, acc);
        }
    }
}

template <int MACT>
__device__ __forceinline__ void x_loop(const XStages &st, const uint16_t *abase, const XAddr &ad,
                                       int nk, int wave, int wm, const int (&brow)[XNB], int fr,
                                       int half, f32x16 (&acc)[XMI][XNB]) {
    const int last = nk - 1;
#pragma unroll
    for (int i = 0; i < XNS; ++i) x_dma_stage(st.s[i], abase, ad, min(i, last), wave);
    xfence();
    __builtin_amdgcn_s_waitcnt(xvmcnt_imm((XNS - 1) * X_LOADS));
    __builtin_amdgcn_s_barrier();
    xfence();
    XFrags f0, f1;
    XCarry cr;
    x_read_frags<MACT>(st.s[0], 0, wm, brow, fr, half, f0, cr);
    int kt = 0;
    for (; kt + XNS <= nk; kt += XNS)
        x_steps<MACT, 0>(st, kt, XNS, last, abase, ad, wave, wm, brow, fr, half, f0, f1, cr, acc);
    x_steps<MACT, 0>(st, kt, nk - kt, last, abase, ad, wave, wm, brow, fr, half, f0, f1, cr, acc);
    xfence();
    __builtin_amdgcn_s_waitcnt(xvmcnt_imm(0));  // no load may land after the block ends
    __builtin_amdgcn_s_barrier();
    xfence();
}
}  // namespace

struct Mx4GemmArgs {
    const uint16_t *x;
    const uint8_t *wp;     // packed routed weights: gate/up [E*2F, d], down [E*d, F]
    const uint8_t *wp_sh;  // packed shared weights: gate/up [2Fs, d], down [d, Fs]
    uint16_t *h, *h_sh;
    float *out;
    uint8_t *y;            // routed rows, weighted, y16 rows
    const int32_t *perm, *counts, *offsets, *tile_start, *tile_group;
    const float *topk_w, *gate;
    int64_t T;
    int d, E, k, F, Fs;
    int nm, nn;
};

template <int MODE>
__global__ __launch_bounds__(64 * XW, 1) void gemm_mx4_kernel(Mx4GemmArgs a) {
    __shared__ __align__(1024) unsigned char st0[X_STB];
    __shared__ __align__(1024) unsigned char st1[X_STB];
    __shared__ __align__(1024) unsigned char st2[X_STB];
    __shared__ int32_t row_tok[XBM];
    __shared__ float row_w[XBM];

    int mt, nt;
    if (!raster_tile(a.nm, a.nn, -1, mt, nt)) return;
    if (mt >= a.tile_start[a.E + 1]) return;
    const int g = a.tile_group[mt];
    const bool shared = g == a.E;
    const int m_local = (mt - a.tile_start[g]) * XBM;
    int row0, nrows;
    if (!shared) {
        row0 = a.offsets[g] + m_local;
        nrows = min(XBM, a.counts[g] - m_local);
    } else {
        row0 = m_local;
        nrows = (int)min<int64_t>(XBM, a.T - m_local);
    }
    const int Fg = shared ? a.Fs : a.F;
    const int N = MODE == 0 ? Fg : a.d;
    const int K = MODE == 1 ? Fg : a.d;
    const int n0 = nt * (MODE == 0 ? XBN / 2 : XBN);
    if (n0 >= N) return;

    const int tid = threadIdx.x;
    if (tid < XBM) {
        const int r = min(tid, nrows - 1);  // padding rows repeat the last row; never stored
        int tok;
        float wgt = 0.f;
        if (!shared) {
            const int pair = a.perm[row0 + r];
            tok = pair / a.k;
            if (MODE == 1) wgt = a.topk_w[pair];
        } else {
            tok = row0 + r;
            if (MODE == 1) wgt = a.gate[tok];
        }
        row_tok[tid] = tok;
        row_w[tid] = wgt;
    }
    __syncthreads();

    const int lane = tid & 63, wave = wave_id();
    const uint16_t *abase = MODE == 1 ? (shared ? a.h_sh : a.h) : a.x;
    XAddr ad;
#pragma unroll
    for (int j = 0; j < X_AL; ++j) {
        const int R = (X_AL * wave + j) * 4 + (lane >> 4);  // 4 rows of 256 bytes per load
        const int c = (lane & 15) ^ (R & 15);
        ad.aoff[j] = (MODE == 1 ? (uint32_t)(row0 + min(R, nrows - 1)) * (uint32_t)Fg
                                : (uint32_t)row_tok[R] * (uint32_t)a.d) + 8 * c;
    }
    // the 16 weight row blocks of this N tile (gate/up: 8 gate blocks, then the
    // matching 8 up blocks; down: 16 consecutive blocks, the last ones clamped
    // to d when d % 256 != 0 -- their columns are never stored)
    const uint8_t *P = shared ? a.wp_sh : a.wp;
    const int64_t rb0 = shared ? 0 : (int64_t)g * (MODE == 0 ? 2 * a.F : a.d) / 16;
    const int64_t kt_tiles = K / XBK;
    auto tile_base = [&](int b) -> const uint8_t * {
        int64_t rb;
        if (MODE == 0) rb = rb0 + (b < 8 ? n0 / 16 + b : (Fg + n0) / 16 + (b - 8));
        else rb = rb0 + min(n0 / 16 + b, a.d / 16 - 1);
        return P + rb * kt_tiles * XTILE;
    };
#pragma unroll
    for (int j = 0; j < X_CL; ++j) ad.code[j] = tile_base(X_CL * wave + j) + 16 * lane;
    ad.scale = tile_base(4 * (wave & 3) + (lane >> 4)) + 1024 + 4 * (lane & 15);

    // wave (wm, wn): rows 64 wm .. + 63; gate/up: gate columns 32 wn .. + 31
    // (block 0) and the matching up columns (block 1); down: columns 64 wn ..
    const int wm = wave >> 2, wn = wave & 3;
    const int fr = lane & 31, half = lane >> 5;
    int brow[XNB];
#pragma unroll
    for (int ni = 0; ni < XNB; ++ni)
        brow[ni] = MODE == 0 ? ni * (XBN / 2) + 32 * wn : 64 * wn + 32 * ni;
    const int mact = min(XMI, max(0, (nrows - XBM / 2 * wm + 31) / 32));

    f32x16 acc[XMI][XNB];
#pragma unroll
    for (int i = 0; i < XMI; ++i)
#pragma unroll
        for (int j = 0; j < XNB; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

    const int nk = K / XBK;
    XStages st;
    st.s[0] = st0;
    st.s[1] = st1;
    st.s[2] = st2;
    switch (mact) {
    case 2: x_loop<2>(st, abase, ad, nk, wave, wm, brow, fr, half, acc); break;
    case 1: x_loop<1>(st, abase, ad, nk, wave, wm, brow, fr, half, acc); break;
    default: x_loop<0>(st, abase, ad, nk, wave, wm, brow, fr, half, acc); break;
    }

    // Accumulator layout (B A^T): lane holds token row 64 wm + 32 mi + lane % 32
    // and, in acc[mi][ni][4 g + q], output column brow[ni] + 8 g + 4 (lane / 32) + q.
    const int cq = 4 * (lane >> 5);
    if (MODE == 0) {
        uint16_t *H = shared ? a.h_sh : a.h;
#pragma unroll
        for (int mi = 0; mi < XMI; ++mi) {
            const int row = XBM / 2 * wm + 32 * mi + fr;
            if (mi >= mact || row >= nrows) continue;
            uint16_t *hrow = H + (int64_t)(row0 + row) * Fg + n0 + 32 * wn + cq;
            const f32x16 &gt = acc[mi][0], &up = acc[mi][1];
#pragma unroll
            for (int gg = 0; gg < 4; ++gg) {
                uint2 q;
                q.x = pack_bf16x2(silu_mul(gt[4 * gg], up[4 * gg]),
                                  silu_mul(gt[4 * gg + 1], up[4 * gg + 1]));
                q.y = pack_bf16x2(silu_mul(gt[4 * gg + 2], up[4 * gg + 2]),
                                  silu_mul(gt[4 * gg + 3], up[4 * gg + 3]));
                *reinterpret_cast<uint2 *>(hrow + 8 * gg) = q;
            }
        }
    } else {
#pragma unroll
        for (int mi = 0; mi < XMI; ++mi) {
            const int row = XBM / 2 * wm + 32 * mi + fr;
            if (mi >= mact || row >= nrows) continue;
            const float wgt = row_w[row];
            if (!shared) {
                uint8_t *yrow = a.y + (int64_t)(row0 + row) * y16_pitch(a.d);
                // a lane holds four consecutive columns of each 8-column
                // group, lane ^ 32 the other four (same row): the group's
                // exponent is their joint maximum, and the lane below 32
                // writes the four exponent bytes of a 32-column block at once
#pragma unroll
                for (int ni = 0; ni < XNB; ++ni) {
                    const int cb = n0 + brow[ni];
                    if (cb >= a.d) continue;
                    const f32x16 &c = acc[mi][ni];
                    uint32_t xw = 0;
#pragma unroll
                    for (int gg = 0; gg < 4; ++gg) {
                        const float v0 = wgt * c[4 * gg], v1 = wgt * c[4 * gg + 1];
                        const float v2 = wgt * c[4 * gg + 2], v3 = wgt * c[4 * gg + 3];
                        float am = absmax4(v0, v1, v2, v3);
                        am = fmaxf(am, __shfl_xor(am, 32, 64));
                        const uint32_t x = y16_exponent(am);
                        uint2 m;
                        m.x = y16_pack2(v0, v1, x);
                        m.y = y16_pack2(v2, v3, x);
                        *reinterpret_cast<uint2 *>(yrow + 2 * (int64_t)(cb + 8 * gg + cq)) = m;
                        xw |= x << (8 * gg);
                    }
                    if (cq == 0)
                        *reinterpret_cast<uint32_t *>(yrow + 2 * (int64_t)a.d + cb / 8) = xw;
                }
            } else {
                float *orow = a.out + (int64_t)row_tok[row] * a.d + n0 + cq;
#pragma unroll
                for (int ni = 0; ni < XNB; ++ni)
#pragma unroll
                    for (int gg = 0; gg < 4; ++gg) {
                        const int col = n0 + brow[ni] + 8 * gg + cq;
                        if (col >= a.d) continue;
                        const f32x16 &c = acc[mi][ni];
                        *reinterpret_cast<float4 *>(orow + brow[ni] + 8 * gg) =
                            make_float4(wgt * c[4 * gg], wgt * c[4 * gg + 1], wgt * c[4 * gg + 2],
                                        wgt * c[4 * gg + 3]);
                    }
            }
        }
    }
}

hipError_t launch_experts_mx4_gemm(const Problem &p, hipStream_t s,
                                   const std::function<void(int)> &mark) {
    Mx4GemmArgs a;
    memset(&a, 0, sizeof a);
    a.x = static_cast<const uint16_t *>(p.x);
    a.h = static_cast<uint16_t *>(p.h);
    a.h_sh = static_cast<uint16_t *>(p.h_shared);
    a.out = p.out;
    a.y = static_cast<uint8_t *>(p.y);
    a.perm = p.perm;
    a.counts = p.counts;
    a.offsets = p.offsets;
    a.tile_start = p.tile_start;
    a.tile_group = p.tile_group;
    a.topk_w = p.topk_w;
    a.gate = p.gate;
    a.T = p.T;
    a.d = p.d;
    a.E = p.E;
    a.k = p.k;
    a.F = p.F;
    a.Fs = p.Fs;
    a.nm = p.max_tiles;
    const int fmax = p.F > p.Fs ? p.F : p.Fs;
    a.wp = static_cast<const uint8_t *>(p.w_gate_up);
    a.wp_sh = static_cast<const uint8_t *>(p.w_sh_gate_up);
    a.nn = (fmax + XBN / 2 - 1) / (XBN / 2);
    hipLaunchKernelGGL(gemm_mx4_kernel<0>, dim3(raster_blocks(a.nm, a.nn, -1)), dim3(64 * XW), 0, s, a);
    mark(3);
    a.wp = static_cast<const uint8_t *>(p.w_down);
    a.wp_sh = static_cast<const uint8_t *>(p.w_sh_down);
    a.nn = (p.d + XBN - 1) / XBN;
    hipLaunchKernelGGL(gemm_mx4_kernel<1>, dim3(raster_blocks(a.nm, a.nn, -1)), dim3(64 * XW), 0, s, a);
    mark(4);
    return hipGetLastError();
}

}  // namespace moe
