// experts_gemm256.hip -- grouped SwiGLU expert GEMMs with 256 x 256 tiles for
// many tokens per expert (long prefill chunks, skewed routing).
//
// Same maths and epilogues as experts_bf16.hip (gated MLP with SiLU, weighted
// rows y, the shared expert scaled by its sigmoid gate; anatomy page on
// frontier-model-atlas, "Decoder microscope", Feed-forward panel).  A tile is
// up to 256 consecutive permuted rows of one group (group E = the shared
// expert) against 256 output columns; gate/up tiles stack 128 gate rows on the
// matching 128 up rows.  8 waves (2 x 4), each owning 128 x 64 of the tile as
// 4 x 2 v_mfma_f32_32x32x16_bf16 blocks (128 accumulators per lane), so each
// staged byte feeds 128 FLOP (a 128 x 128 tile gives 64).  K advances in steps of 64 through double-buffered LDS rows of
// 72 elements (144 B: 16 lanes reading 16 consecutive rows hit 16 disjoint
// 4-bank groups).  Global loads for the next step are issued before the
// current step's MFMAs and are unconditional (the last step re-reads itself)
// so no branch sits around them.  32-row sub-tiles past the group's last row
// skip their MFMAs.
#include "moe_device.h"
#include "moe_kernels.h"

#include <string.h>

namespace moe {

namespace {
constexpr int BM = kGemm256BM, BN = 256, BK = 64, LDK = BK + 8;
}

// The K loop of one wave: MACT of its four 32-row sub-tiles do MFMAs; every
// wave loads, stores and synchronises alike.
template <int MACT>
__device__ __forceinline__ void k_loop(uint16_t (*As)[BM * LDK], uint16_t (*Bs)[BN * LDK],
                                       const uint16_t *abase, const uint16_t *wbase,
                                       const uint32_t (&aoff)[4], const uint32_t (&boff)[4],
                                       int sofs, int nk, int wm, const int (&brow)[2], int fr,
                                       int fk, f32x16 (&acc)[4][2]) {
    u32x4 ra[4], rb[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        ra[p] = *reinterpret_cast<const u32x4 *>(abase + aoff[p]);
        rb[p] = *reinterpret_cast<const u32x4 *>(wbase + boff[p]);
    }
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        *reinterpret_cast<u32x4 *>(&As[0][sofs + 64 * p * LDK]) = ra[p];
        *reinterpret_cast<u32x4 *>(&Bs[0][sofs + 64 * p * LDK]) = rb[p];
    }
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        const int knext = min(kt + 1, nk - 1) * BK;
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            ra[p] = *reinterpret_cast<const u32x4 *>(abase + aoff[p] + knext);
            rb[p] = *reinterpret_cast<const u32x4 *>(wbase + boff[p] + knext);
        }
        // keep the next step's loads above this step's MFMAs (the scheduler
        // otherwise sinks them to their LDS stores and nothing overlaps)
        __builtin_amdgcn_sched_barrier(0);
        if (MACT > 0) {
            const uint16_t *A = As[cur];
            const uint16_t *B = Bs[cur];
#pragma unroll
            for (int ks = 0; ks < BK / 16; ++ks) {
                bf16x8 af[4], bf[2];
#pragma unroll
                for (int mi = 0; mi < MACT; ++mi)
                    af[mi] = *reinterpret_cast<const bf16x8 *>(
                        &A[(128 * wm + 32 * mi + fr) * LDK + 16 * ks + fk]);
#pragma unroll
                for (int ni = 0; ni < 2; ++ni)
                    bf[ni] = *reinterpret_cast<const bf16x8 *>(&B[(brow[ni] + fr) * LDK + 16 * ks + fk]);
#pragma unroll
                for (int mi = 0; mi < MACT; ++mi)
#pragma unroll
                    for (int ni = 0; ni < 2; ++ni)
                        acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mi], bf[ni],
                                                                              acc[mi][ni], 0, 0, 0);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        if (kt + 1 < nk) {
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                *reinterpret_cast<u32x4 *>(&As[cur ^ 1][sofs + 64 * p * LDK]) = ra[p];
                *reinterpret_cast<u32x4 *>(&Bs[cur ^ 1][sofs + 64 * p * LDK]) = rb[p];
            }
        }
        __syncthreads();
    }
}

// MODE 0: gate/up (K = d).  MODE 1: down (K = F).  MODE 2: router logits.
template <int MODE>
__global__ __launch_bounds__(512, 1) void gemm256_kernel(GemmArgs a) {
    __shared__ __align__(16) uint16_t As[2][BM * LDK];
    __shared__ __align__(16) uint16_t Bs[2][BN * LDK];
    __shared__ int32_t row_tok[BM];
    __shared__ float row_w[BM];

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
    const int Fg = shared ? a.Fs : a.F;
    const int N = MODE == 0 ? Fg : MODE == 1 ? a.d : a.E;
    const int K = MODE == 1 ? Fg : a.d;
    const int n0 = nt * (MODE == 0 ? BN / 2 : BN);
    if (n0 >= N) return;

    const int tid = threadIdx.x;
    if (tid < BM) {
        const int r = min(tid, nrows - 1);  // padding rows repeat the last row; never stored
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
        row_tok[tid] = tok;
        row_w[tid] = wgt;
    }
    __syncthreads();

    // Thread owns 16-byte chunk (tid % 8) of rows tid / 8 + 64 p, p = 0..3,
    // of both the A and the B tile.
    const int lrow = tid >> 3, lchunk = tid & 7;
    const uint16_t *wbase = MODE == 2 ? a.w
                            : shared  ? a.w_sh
                                      : a.w + (int64_t)g * (MODE == 0 ? (int64_t)2 * a.F * a.d
                                                                      : (int64_t)a.d * a.F);
    // per-row element offsets from block-uniform bases (32-bit: the host
    // checks that every offset fits)
    const uint16_t *abase = MODE == 1 ? (shared ? a.h_sh : a.h) : a.x;
    uint32_t aoff[4], boff[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const int r = lrow + 64 * p;
        if (MODE == 1) {
            aoff[p] = (uint32_t)(row0 + min(r, nrows - 1)) * (uint32_t)Fg;
            boff[p] = (uint32_t)min(n0 + r, a.d - 1) * (uint32_t)Fg;
        } else {
            aoff[p] = (uint32_t)row_tok[r] * (uint32_t)a.d;
            if (MODE == 0)
                boff[p] = (uint32_t)(r < BN / 2 ? n0 + r : Fg + n0 + (r - BN / 2)) * (uint32_t)a.d;
            else
                boff[p] = (uint32_t)min(n0 + r, a.E - 1) * (uint32_t)a.d;
        }
        aoff[p] += lchunk * 8;
        boff[p] += lchunk * 8;
    }

    const int sofs = lrow * LDK + lchunk * 8;

    const int lane = tid & 63, wave = wave_id();
    const int wm = wave >> 2, wn = wave & 3;
    const int fr = lane & 31, fk = 8 * (lane >> 5);
    // B rows of this wave's two 32-column blocks: gate/up pairs gate column
    // block 32 wn with the matching up block; down takes 64 wn .. 64 wn + 63.
    int brow[2];
#pragma unroll
    for (int ni = 0; ni < 2; ++ni) brow[ni] = MODE == 0 ? ni * (BN / 2) + 32 * wn : 64 * wn + 32 * ni;
    // active 32-row sub-tiles of this wave's 128 rows
    const int mact = min(4, max(0, (nrows - 128 * wm + 31) / 32));

    f32x16 acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

    const int nk = K / BK;
    // mact is wave-uniform (scalar): the sub-tile skip is decided once, outside
    // the K loop, so the loop body is one straight block of loads and MFMAs.
    switch (mact) {
    case 4: k_loop<4>(As, Bs, abase, wbase, aoff, boff, sofs, nk, wm, brow, fr, fk, acc); break;
    case 3: k_loop<3>(As, Bs, abase, wbase, aoff, boff, sofs, nk, wm, brow, fr, fk, acc); break;
    case 2: k_loop<2>(As, Bs, abase, wbase, aoff, boff, sofs, nk, wm, brow, fr, fk, acc); break;
    case 1: k_loop<1>(As, Bs, abase, wbase, aoff, boff, sofs, nk, wm, brow, fr, fk, acc); break;
    default: k_loop<0>(As, Bs, abase, wbase, aoff, boff, sofs, nk, wm, brow, fr, fk, acc); break;
    }

    // 32x32 accumulator layout: lane holds column (lane % 32) and rows
    // 8 (v / 4) + 4 (lane / 32) + (v % 4), v = 0..15.
    if (MODE == 0) {
        uint16_t *H = shared ? a.h_sh : a.h;
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) {
            if (mi >= mact) continue;
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int row = 128 * wm + 32 * mi + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
                if (row < nrows) {
                    const int col = n0 + 32 * wn + fr;
                    H[(int64_t)(row0 + row) * Fg + col] =
                        f32_to_bf16_rne(silu_mul(acc[mi][0][v], acc[mi][1][v]));
                }
            }
        }
    } else {
        // one block-uniform base, 32-bit element offsets
        float *obase = MODE == 2 ? a.f : (shared ? a.out : a.y);
        const int ncol = MODE == 2 ? a.E : a.d;
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) {
            if (mi >= mact) continue;
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int row = 128 * wm + 32 * mi + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
                if (row >= nrows) continue;
                const uint32_t ro = MODE == 2 ? (uint32_t)(row0 + row) * (uint32_t)a.ldf
                                    : shared  ? (uint32_t)row_tok[row] * (uint32_t)a.d
                                              : (uint32_t)(row0 + row) * (uint32_t)a.d;
                const float wgt = MODE == 2 ? 1.0f : row_w[row];
#pragma unroll
                for (int ni = 0; ni < 2; ++ni) {
                    const int col = n0 + brow[ni] + fr;
                    if (col < ncol) obase[ro + col] = wgt * acc[mi][ni][v];
                }
            }
        }
    }
}

hipError_t launch_experts_gemm256(const Problem &p, hipStream_t s,
                                  const std::function<void(int)> &mark) {
    GemmArgs a;
    memset(&a, 0, sizeof a);
    a.x = static_cast<const uint16_t *>(p.x);
    a.h = static_cast<uint16_t *>(p.h);
    a.h_sh = static_cast<uint16_t *>(p.h_shared);
    a.out = p.out;
    a.y = p.y;
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
    auto grid = [](const GemmArgs &g) { return dim3((unsigned)(8 * ((g.nm * g.nn + 7) / 8))); };
    a.w = static_cast<const uint16_t *>(p.w_gate_up);
    a.w_sh = static_cast<const uint16_t *>(p.w_sh_gate_up);
    a.nm = p.max_tiles;
    a.nn = (fmax + BN / 2 - 1) / (BN / 2);
    a.gm = 0;  // N fastest (measured best; the XCD-grouped order is not faster here)
    hipLaunchKernelGGL(gemm256_kernel<0>, grid(a), dim3(512), 0, s, a);
    mark(3);
    a.w = static_cast<const uint16_t *>(p.w_down);
    a.w_sh = static_cast<const uint16_t *>(p.w_sh_down);
    a.nn = (p.d + BN - 1) / BN;
    hipLaunchKernelGGL(gemm256_kernel<1>, grid(a), dim3(512), 0, s, a);
    mark(4);
    return hipGetLastError();
}

}  // namespace moe
