// experts_bf16.hip -- grouped SwiGLU experts on MFMA (bfloat16 in, binary32
// accumulate) with the weighted scatter-combine.
//
// Experts are gated MLPs with SiLU (llm-architectures-explained
// "Qwen3.8-Flash-Next", "Every architecture field", ffns.moe.gated;
// llm-atlas "Qwen3.8-Flash-Next", "Raw config fields", hidden_act); each token
// sums its k routed experts weighted by the normalised router weights, plus
// the shared expert scaled by its sigmoid gate (anatomy page on
// frontier-model-atlas, "Decoder microscope", Feed-forward panel).
//
// Two launches over a tile list built by the permutation step.  A tile is
// up to BM consecutive permuted rows of one group; group E is the shared
// expert, whose rows are all tokens in order.
//   gate/up:  h[r, n] = bf16( silu(x_t . Wg[n]) * (x_t . Wu[n]) )   (t = token of row r)
//             A rows are gathered from x through the permutation; the block's
//             B tile stacks 64 gate rows on the matching 64 up rows, so the
//             SiLU*up product is formed in registers.
//   down:     y[r, n] = w_r * (h[r] . Wdn[n]) for routed rows (w_r the pair's
//             routing weight) and out[t, n] = s_t * (h_sh[t] . Wsdn[n]) for the
//             shared expert; a combine kernel then adds each token's k rows.
//             Plain stores only: no atomics, deterministic result.
// h is rounded to bfloat16 once; everything else stays binary32.
#include "moe_device.h"
#include "moe_kernels.h"

#include <string.h>

namespace moe {


constexpr int BM = kGemmBM, BN = 128, BK = 64, LDK = BK + 8;  // LDS row: 144 B, 9 x 16 B

// MODE 0: gate/up (K = d).  MODE 1: down (K = F).  MODE 2: dense router
// logits f = x W_r^T (K = d, N = E, rows = tokens, no tile map), binary32
// accumulate in the MFMA's own order (used only to shortlist experts).
// 256 threads = 4 waves in a 2 x 2 grid; wave (wm, wn) owns rows
// [64 wm, 64 wm + 64) and two 32-wide column blocks of B.  Each 32 x 32
// output block comes from v_mfma_f32_32x32x16_bf16.
template <int MODE>
__global__ __launch_bounds__(256) void grouped_gemm_kernel(GemmArgs a) {
    __shared__ __align__(16) uint16_t As[2][BM * LDK];
    __shared__ __align__(16) uint16_t Bs[2][BN * LDK];
    __shared__ int32_t row_tok[BM];
    __shared__ float row_w[BM];

    if (MODE == 2 && a.wnorm && (int)blockIdx.y == a.ksplit) {
#pragma clang fp contract(off)
        // router row norms ||W_r[e]|| for the shortlist bound, one wave per
        // row, beside the GEMM blocks (which do not fill the chip)
        const int lane = threadIdx.x & 63;
        for (int e = blockIdx.x * 4 + (threadIdx.x >> 6); e < a.E; e += gridDim.x * 4) {
            float s2 = 0.f;
            for (int kk = 8 * lane; kk < a.d; kk += 512) {
                float v[8];
                load8(a.w + (int64_t)e * a.d + kk, v);
#pragma unroll
                for (int q = 0; q < 8; ++q) s2 += v[q] * v[q];
            }
            s2 = wave_sum(s2);
            if (lane == 0) a.wnorm[e] = sqrtf(s2);
        }
        return;
    }
    int mt, nt;
    if (!raster_tile(a.nm, a.nn, a.gm, mt, nt)) return;
    int g = 0, row0, nrows;
    bool shared = false;
    if (MODE == 2) {
        row0 = mt * BM;
        if (row0 >= a.T) return;
        nrows = (int)min<int64_t>(BM, a.T - row0);
    } else {
        const int tile = mt;
        if (tile >= a.tile_start[a.E + 1]) return;
        g = a.tile_group[tile];
        shared = g == a.E;
        const int m_local = (tile - a.tile_start[g]) * BM;
        if (!shared) {
            row0 = a.offsets[g] + m_local;
            nrows = min(BM, a.counts[g] - m_local);
        } else {
            row0 = m_local;
            nrows = (int)min<int64_t>(BM, a.T - m_local);
        }
    }
    const int Fg = shared ? a.Fs : a.F;            // width of this group's expert
    // output columns (gate half for MODE 0) and contraction length; MODE 2
    // blocks with blockIdx.y = s cover K slice s of ksplit
    const int N = MODE == 0 ? Fg : MODE == 1 ? a.d : a.E;
    const int K = MODE == 1 ? Fg : MODE == 2 ? a.d / a.ksplit : a.d;
    const int kbeg = MODE == 2 ? (int)blockIdx.y * K : 0;
    const int n0 = nt * (MODE == 0 ? 64 : BN);
    if (n0 >= N) return;

    const int tid = threadIdx.x;
    for (int i = tid; i < BM; i += 256) {
        const int r = min(i, nrows - 1);  // padding rows repeat the last row; never stored
        int tok;
        float wgt = 0.f;
        if (MODE == 2) {
            tok = row0 + r;
        } else if (!shared) {
            const int pair = a.perm[row0 + r];
            tok = pair / a.k;
            if (MODE == 1) wgt = a.topk_w[pair];
        } else {
            tok = row0 + r;
            if (MODE == 1) wgt = a.gate[tok];
        }
        row_tok[i] = tok;
        row_w[i] = wgt;
    }
    __syncthreads();

    // Global -> register staging: thread owns 16-byte chunk (tid % 8) of rows
    // tid / 8 + 32 p, p = 0..3, for both A and B.
    const int lrow = tid >> 3, lchunk = tid & 7;
    const uint16_t *asrc[4];
    const uint16_t *bsrc[4];
    const uint16_t *wbase = MODE == 2 ? a.w
                            : shared  ? a.w_sh
                                      : a.w + (int64_t)g * (MODE == 0 ? (int64_t)2 * a.F * a.d
                                                                      : (int64_t)a.d * a.F);
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const int r = lrow + 32 * p;
        if (MODE == 0) {
            asrc[p] = a.x + (int64_t)row_tok[r] * a.d;
            const int wrow = r < 64 ? n0 + r : Fg + n0 + (r - 64);
            bsrc[p] = wbase + (int64_t)wrow * a.d;
        } else if (MODE == 2) {
            asrc[p] = a.x + (int64_t)row_tok[r] * a.d;
            bsrc[p] = wbase + (int64_t)min(n0 + r, a.E - 1) * a.d;
        } else {
            const int rr = min(r, nrows - 1);
            asrc[p] = shared ? a.h_sh + (int64_t)(row0 + rr) * a.Fs : a.h + (int64_t)(row0 + rr) * a.F;
            const int wrow = min(n0 + r, a.d - 1);
            bsrc[p] = wbase + (int64_t)wrow * Fg;
        }
        asrc[p] += kbeg + lchunk * 8;
        bsrc[p] += kbeg + lchunk * 8;
    }

    uint4 ra0, ra1, ra2, ra3, rb0, rb1, rb2, rb3;
#define MOE_LOAD_TILE(k0)                                                           \
    do {                                                                            \
        ra0 = *reinterpret_cast<const uint4 *>(asrc[0] + (k0));                     \
        ra1 = *reinterpret_cast<const uint4 *>(asrc[1] + (k0));                     \
        ra2 = *reinterpret_cast<const uint4 *>(asrc[2] + (k0));                     \
        ra3 = *reinterpret_cast<const uint4 *>(asrc[3] + (k0));                     \
        rb0 = *reinterpret_cast<const uint4 *>(bsrc[0] + (k0));                     \
        rb1 = *reinterpret_cast<const uint4 *>(bsrc[1] + (k0));                     \
        rb2 = *reinterpret_cast<const uint4 *>(bsrc[2] + (k0));                     \
        rb3 = *reinterpret_cast<const uint4 *>(bsrc[3] + (k0));                     \
    } while (0)
#define MOE_STORE_TILE(buf)                                                         \
    do {                                                                            \
        const int off = lrow * LDK + lchunk * 8;                                    \
        *reinterpret_cast<uint4 *>(&As[buf][off]) = ra0;                            \
        *reinterpret_cast<uint4 *>(&As[buf][off + 32 * LDK]) = ra1;                 \
        *reinterpret_cast<uint4 *>(&As[buf][off + 64 * LDK]) = ra2;                 \
        *reinterpret_cast<uint4 *>(&As[buf][off + 96 * LDK]) = ra3;                 \
        *reinterpret_cast<uint4 *>(&Bs[buf][off]) = rb0;                            \
        *reinterpret_cast<uint4 *>(&Bs[buf][off + 32 * LDK]) = rb1;                 \
        *reinterpret_cast<uint4 *>(&Bs[buf][off + 64 * LDK]) = rb2;                 \
        *reinterpret_cast<uint4 *>(&Bs[buf][off + 96 * LDK]) = rb3;                 \
    } while (0)

    const int lane = tid & 63, wave = wave_id();
    const int wm = wave >> 1, wn = wave & 1;
    const int brow0 = MODE == 0 ? 32 * wn : 64 * wn;
    const int brow1 = MODE == 0 ? 64 + 32 * wn : 64 * wn + 32;
    const int fr = lane & 31, fk = 8 * (lane >> 5);

    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

    const int nk = K / BK;
    MOE_LOAD_TILE(0);
    MOE_STORE_TILE(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < nk) MOE_LOAD_TILE((kt + 1) * BK);
#pragma unroll
        for (int ks = 0; ks < BK / 16; ++ks) {
            bf16x8 af[2], bf[2];
#pragma unroll
            for (int mi = 0; mi < 2; ++mi)
                af[mi] = *reinterpret_cast<const bf16x8 *>(
                    &As[cur][(64 * wm + 32 * mi + fr) * LDK + 16 * ks + fk]);
            bf[0] = *reinterpret_cast<const bf16x8 *>(&Bs[cur][(brow0 + fr) * LDK + 16 * ks + fk]);
            bf[1] = *reinterpret_cast<const bf16x8 *>(&Bs[cur][(brow1 + fr) * LDK + 16 * ks + fk]);
#pragma unroll
            for (int mi = 0; mi < 2; ++mi)
#pragma unroll
                for (int ni = 0; ni < 2; ++ni)
                    acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mi], bf[ni],
                                                                          acc[mi][ni], 0, 0, 0);
        }
        if (kt + 1 < nk) MOE_STORE_TILE(cur ^ 1);
        __syncthreads();
    }
#undef MOE_LOAD_TILE
#undef MOE_STORE_TILE

    // 32x32 accumulator layout: lane holds column (lane % 32) and rows
    // 8 (v / 4) + 4 (lane / 32) + (v % 4), v = 0..15.
    if (MODE == 0) {
        uint16_t *H = shared ? a.h_sh : a.h;
#pragma unroll
        for (int mi = 0; mi < 2; ++mi)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int row = 64 * wm + 32 * mi + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
                if (row < nrows) {
                    const int col = n0 + 32 * wn + fr;
                    H[(int64_t)(row0 + row) * Fg + col] =
                        f32_to_bf16_rne(silu_mul(acc[mi][0][v], acc[mi][1][v]));
                    if (a.au) {  // training forward: the pre-activations too
                        uint16_t *arow = (shared ? a.au_sh : a.au) + (int64_t)(row0 + row) * 2 * Fg;
                        arow[col] = f32_to_bf16_rne(acc[mi][0][v]);
                        arow[Fg + col] = f32_to_bf16_rne(acc[mi][1][v]);
                    }
                }
            }
    } else if (MODE == 2) {
#pragma unroll
        for (int mi = 0; mi < 2; ++mi)
#pragma unroll
            for (int ni = 0; ni < 2; ++ni)
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int row = 64 * wm + 32 * mi + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
                    const int col = n0 + (ni ? brow1 : brow0) + fr;
                    if (row < nrows && col < a.E)
                        a.f[((int64_t)blockIdx.y * a.T + row0 + row) * a.ldf + col] =
                            acc[mi][ni][v];
                }
    } else {
#pragma unroll
        for (int mi = 0; mi < 2; ++mi)
#pragma unroll
            for (int ni = 0; ni < 2; ++ni)
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int row = 64 * wm + 32 * mi + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
                    const int col = n0 + (ni ? brow1 : brow0) + fr;
                    const float val = row_w[row] * acc[mi][ni][v];
                    if (shared) {
                        if (row < nrows && col < a.d)
                            a.out[(int64_t)row_tok[row] * a.d + col] = val;
                    } else {
                        // eight consecutive lanes hold eight consecutive
                        // columns of one row: one y16 group
                        const uint32_t x = y16_octet_exponent(val);
                        if (row < nrows && col < a.d)
                            y16_store1(a.y + (int64_t)(row0 + row) * y16_pitch(a.d), a.d, col, val, x);
                    }
                }
    }
}

hipError_t launch_experts_bf16(const Problem &p, hipStream_t s,
                               const std::function<void(int)> &mark) {
    GemmArgs a;
    a.x = static_cast<const uint16_t *>(p.x);
    a.h = static_cast<uint16_t *>(p.h);
    a.h_sh = static_cast<uint16_t *>(p.h_shared);
    a.au = static_cast<uint16_t *>(p.au);
    a.au_sh = static_cast<uint16_t *>(p.au_sh);
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

    const int fmax = p.F > p.Fs ? p.F : p.Fs;
    auto grid = [](const GemmArgs &g) { return dim3(raster_blocks(g.nm, g.nn, g.gm)); };
    a.w = static_cast<const uint16_t *>(p.w_gate_up);
    a.w_sh = static_cast<const uint16_t *>(p.w_sh_gate_up);
    a.nm = p.max_tiles;
    a.nn = fmax / 64;
    a.gm = -1;  // M-tile m on XCD m % 8: its N-tiles share A through one L2
    hipLaunchKernelGGL(grouped_gemm_kernel<0>, grid(a), dim3(256), 0, s, a);
    mark(3);
    a.w = static_cast<const uint16_t *>(p.w_down);
    a.w_sh = static_cast<const uint16_t *>(p.w_sh_down);
    a.nn = (p.d + BN - 1) / BN;
    hipLaunchKernelGGL(grouped_gemm_kernel<1>, grid(a), dim3(256), 0, s, a);
    mark(4);
    return hipGetLastError();
}

hipError_t launch_router_gemm(const Problem &p, hipStream_t s) {
    GemmArgs a;
    memset(&a, 0, sizeof a);
    a.x = static_cast<const uint16_t *>(p.x);
    a.w = static_cast<const uint16_t *>(p.w_router);
    a.f = p.logits;
    a.ldf = p.E + 1;
    a.T = p.T;
    a.d = p.d;
    a.E = p.E;
    a.nm = (int)((p.T + BM - 1) / BM);
    a.nn = (p.E + BN - 1) / BN;
    a.gm = 8;
    a.ksplit = p.router_split;
    a.wnorm = p.wnorm;  // one more slice of blocks computes the row norms
    hipLaunchKernelGGL(grouped_gemm_kernel<2>,
                       dim3((unsigned)(8 * ((a.nm * a.nn + 7) / 8)), (unsigned)a.ksplit + 1),
                       dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace moe
