// experts_dma.hip -- grouped SwiGLU expert GEMMs with tiles of BM = 256 or
// 128 rows by 256 output columns, staged by direct global -> LDS loads.
//
// Same maths and epilogues as experts_bf16.hip (gated MLP with SiLU, weighted
// rows y, the shared expert scaled by its sigmoid gate; anatomy page on
// frontier-model-atlas, "Decoder microscope", Feed-forward panel).  A tile is
// up to BM consecutive permuted rows of one group (group E = the shared
// expert) against 256 output columns; gate/up tiles stack 128 gate rows on the
// matching 128 up rows.  Waves in a (NW / 2) x 2 grid, each owning WR x 128 of
// the tile as (WR / 32) x 4 v_mfma_f32_32x32x16_bf16 blocks: 8 waves (two per
// SIMD) for 256-row tiles (WR = 64) and for the one-block-per-CU 128-row
// tiles (WR = 32).  BM = 256 serves
// many tokens per expert (each staged byte feeds 128 FLOP); BM = 128 serves
// the middle ground, where streaming the expert weights sets the time.
//
// Tiles go straight from global memory into LDS (global_load_lds_dwordx4:
// lane i of one load writes 16 bytes at the load's LDS base + 16 i), so no
// registers hold tiles in flight and the K loop runs up to three steps
// ahead through three stage buffers of BK = 32 or 64 (a buffer is refilled as
// soon as every wave has read it).  BK = 64 reads 128 contiguous bytes of
// each weight row per step, which HBM streams about 10% faster than 64-byte
// pieces; its 48 KB stages leave room for one block per CU (of 8 waves), so
// it serves the 128-row tiles of both GEMMs, and BK = 32 the 256-row tiles.  One load fills one KB of LDS:
// 16 rows of 64 bytes (BK = 32) or 8 rows of 128 bytes (BK = 64).  A 16-byte
// read by 64 lanes is served 16 lanes (256 bytes) per clock, so the 16 rows
// read together at one chunk must cover all 64 banks: chunk c of row R sits
// at chunk c ^ ((R >> 2) & 3) for 64-byte rows and c ^ ((R >> 1) & 7) for
// 128-byte rows (measured conflict-free for 64-byte rows; without the XOR
// each read takes 4x as long).  A step waits for its own stage with an
// explicit vmcnt and a bare s_barrier (a __syncthreads fence would drain
// every load in flight); the block drains all its loads before it ends.
#include "moe_device.h"
#include "moe_kernels.h"

#include <string.h>

#include <algorithm>

namespace moe {

namespace {
constexpr int BN = 256;
constexpr int NB = 4;  // 32-column blocks per wave

// Per tile height BM and K step BK (32 or 64): waves per block (each owns
// WR rows by 128 columns; 8 waves where one block fills a CU, measured faster
// than 4 there), bytes per staged row, 16-byte chunks per row, rows per 1 KB load, A
// and stage bytes (A then B), A and B loads per wave per stage, k16 sub-steps
// per stage, 32-row sub-tiles per wave.
template <int BM, int BK> struct Geo {
    static_assert(BK == 32 || BK == 64, "BK is 32 or 64");
    static constexpr int NW = BK == 64 ? 8 : BM / 32;
    static constexpr int WR = BM / (NW / 2);
    static constexpr int ROWB = BK * 2;
    static constexpr int CH = ROWB / 16;
    static constexpr int RPL = 64 / CH;
    static constexpr int OPA = BM * ROWB;
    static constexpr int STB = OPA + BN * ROWB;
    static constexpr int AL = BM / RPL / NW;
    static constexpr int BL = BN / RPL / NW;
    static constexpr int LOADS = AL + BL;
    static constexpr int Q = BK / 16;
    static constexpr int MI = WR / 32;
    static_assert(AL * RPL * NW == BM && BL * RPL * NW == BN, "loads cover the tile");
};

typedef __attribute__((address_space(3))) void lds_void_t;
typedef const __attribute__((address_space(1))) void global_void_t;

// s_waitcnt immediate that waits until at most n vector-memory operations are
// outstanding, leaving the other counters free (vmcnt is split over bits
// [3:0] and [15:14]); the second form also waits for every LDS access.
constexpr int vmcnt_imm(int n) { return (n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8); }
constexpr int vmcnt_lgkm0_imm(int n) { return vmcnt_imm(n) & ~(0xF << 8); }

// Chunk swizzle: the 16 rows that one 16-lane read phase touches at one
// logical chunk land on 16 distinct 16-byte bank groups.
template <int BK> __device__ __forceinline__ int swz(int R) {
    return BK == 32 ? (R >> 2) & 3 : (R >> 1) & 7;
}
template <int BK> __device__ __forceinline__ int tile_off(int R, int c) {
    return R * (2 * BK) + ((c ^ swz<BK>(R)) << 4);
}
__device__ __forceinline__ void compiler_fence() { asm volatile("" ::: "memory"); }
}  // namespace

// Issue one stage's loads: each load fills one contiguous KB of LDS, RPL
// tile rows.  This wave fills A rows RPL (AL wave + j) .., j < AL, and B rows
// RPL (BL wave + j) .., j < BL.  aoff/boff are this lane's element offsets
// (its row and swizzled chunk); k0 selects the K step.
template <int BM, int BK>
__device__ __forceinline__ void dma_stage(unsigned char *stage, const uint16_t *abase,
                                          const uint16_t *wbase,
                                          const uint32_t (&aoff)[Geo<BM, BK>::AL],
                                          const uint32_t (&boff)[Geo<BM, BK>::BL], int k0,
                                          int wave) {
    using G = Geo<BM, BK>;
#pragma unroll
    for (int j = 0; j < G::AL; ++j)
        __builtin_amdgcn_global_load_lds((const global_void_t *)(abase + aoff[j] + k0),
                                         (lds_void_t *)(stage + (G::AL * wave + j) * 1024), 16,
                                         0, 0);
#pragma unroll
    for (int j = 0; j < G::BL; ++j)
        __builtin_amdgcn_global_load_lds(
            (const global_void_t *)(wbase + boff[j] + k0),
            (lds_void_t *)(stage + G::OPA + (G::BL * wave + j) * 1024), 16, 0, 0);
}

// Operand fragments of one k16 step: MACT A blocks and the wave's NB B blocks.
struct Frags {
    bf16x8 a[4], b[NB];
};

template <int BM, int BK, int MACT>
__device__ __forceinline__ void read_frags(const unsigned char *stage, int ks, int wm,
                                           const int (&brow)[NB], int fr, int lane, Frags &f) {
    if (MACT == 0) return;
    const int c = 2 * ks + (lane >> 5);
#pragma unroll
    for (int mi = 0; mi < MACT; ++mi)
        f.a[mi] = *reinterpret_cast<const bf16x8 *>(stage +
                                                    tile_off<BK>(Geo<BM, BK>::WR * wm + 32 * mi + fr, c));
#pragma unroll
    for (int ni = 0; ni < NB; ++ni)
        f.b[ni] = *reinterpret_cast<const bf16x8 *>(stage + Geo<BM, BK>::OPA +
                                                    tile_off<BK>(brow[ni] + fr, c));
}

// acc[mi][ni] accumulates B_ni A_mi^T (output features by tokens), so each
// lane ends with one token row and runs of four consecutive output columns.
template <int MACT, int MI>
__device__ __forceinline__ void mfma_frags(const Frags &f, f32x16 (&acc)[MI][NB]) {
#pragma unroll
    for (int mi = 0; mi < MACT; ++mi)
#pragma unroll
        for (int ni = 0; ni < NB; ++ni)
            acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.b[ni], f.a[mi], acc[mi][ni], 0, 0, 0);
}

template <int NS> struct Stages {
    unsigned char *s[NS];
};

// Scheduling groups: one MFMA, then the fragment reads each followed by one
// MFMA, then the remaining MFMAs.  The first MFMA waits for the fragments it
// uses (read one half step earlier, so that wait is free); the reads for the
// next half step then overlap the MFMAs.
template <int MACT>
__device__ __forceinline__ void interleave_reads() {
    constexpr int reads = MACT + NB;
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
#pragma unroll
    for (int i = 0; i < reads; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, MACT * NB - 1 - reads, 0);
}

// MFMAs on the k16 fragments in cur while sub-step ks of stage goes to nxt.
template <int BM, int BK, int MACT>
__device__ __forceinline__ void sub_step(const unsigned char *stage, int ks, int wm,
                                         const int (&brow)[NB], int fr, int lane, const Frags &cur,
                                         Frags &nxt, f32x16 (&acc)[Geo<BM, BK>::MI][NB]) {
    if (MACT > 0) {
        mfma_frags<MACT>(cur, acc);
        read_frags<BM, BK, MACT>(stage, ks, wm, brow, fr, lane, nxt);
        interleave_reads<MACT>();
    }
    __builtin_amdgcn_sched_barrier(0);
}

// One K step kt on stage buffer S = kt % NS, entered with stage kt visible to
// all waves and its first k16 fragments in f0.  Stages kt+1 .. kt+NS-1 are in
// flight ((NS-1) LOADS loads per wave, oldest first).
//   1. MFMAs on each k16 sub-step but the last while the next one's
//      fragments are read (f0 and f1 alternate; Q is even, so the last
//      sub-step's fragments end in f1);
//   2. wait until this wave's reads of stage kt are done and its part of
//      stage kt+1 has landed (lgkmcnt 0, vmcnt <= (NS-2) LOADS), then
//      barrier: stage kt+1 is visible and no wave reads buffer S any more;
//   3. refill buffer S with stage kt+NS (past the last step the loads re-read
//      it into a buffer that is never computed);
//   4. MFMAs on f1 while the first k16 fragments of stage kt+1 go to f0.
// Every stage buffer is its own LDS array named by a constant index, so the
// compiler ties each LDS read to the loads of that buffer alone instead of
// waiting for every load in flight.
template <int BM, int BK, int NS, int MACT, int S>
__device__ __forceinline__ void k_step(const Stages<NS> &st, int kt, int last,
                                       const uint16_t *abase, const uint16_t *wbase,
                                       const uint32_t (&aoff)[Geo<BM, BK>::AL],
                                       const uint32_t (&boff)[Geo<BM, BK>::BL], int wave, int wm,
                                       const int (&brow)[NB], int fr, int lane, Frags &f0,
                                       Frags &f1, f32x16 (&acc)[Geo<BM, BK>::MI][NB]) {
    using G = Geo<BM, BK>;
    sub_step<BM, BK, MACT>(st.s[S], 1, wm, brow, fr, lane, f0, f1, acc);
    if constexpr (G::Q == 4) {
        sub_step<BM, BK, MACT>(st.s[S], 2, wm, brow, fr, lane, f1, f0, acc);
        sub_step<BM, BK, MACT>(st.s[S], 3, wm, brow, fr, lane, f0, f1, acc);
    }
    compiler_fence();
    __builtin_amdgcn_s_waitcnt(vmcnt_lgkm0_imm((NS - 2) * G::LOADS));
    __builtin_amdgcn_s_barrier();
    compiler_fence();
    dma_stage<BM, BK>(st.s[S], abase, wbase, aoff, boff, min((kt + NS) * BK, last), wave);
    __builtin_amdgcn_sched_barrier(0);
    sub_step<BM, BK, MACT>(st.s[(S + 1) % NS], 0, wm, brow, fr, lane, f1, f0, acc);
}

// Steps kt + S .. kt + cnt - 1 (cnt <= NS), each on its constant buffer.
template <int BM, int BK, int NS, int MACT, int S>
__device__ __forceinline__ void k_steps(const Stages<NS> &st, int kt, int cnt, int last,
                                        const uint16_t *abase, const uint16_t *wbase,
                                        const uint32_t (&aoff)[Geo<BM, BK>::AL],
                                        const uint32_t (&boff)[Geo<BM, BK>::BL], int wave, int wm,
                                        const int (&brow)[NB], int fr, int lane, Frags &f0,
                                        Frags &f1, f32x16 (&acc)[Geo<BM, BK>::MI][NB]) {
    if constexpr (S < NS) {
        if (S < cnt) {
            k_step<BM, BK, NS, MACT, S>(st, kt + S, last, abase, wbase, aoff, boff, wave, wm,
                                        brow, fr, lane, f0, f1, acc);
            k_steps<BM, BK, NS, MACT, S + 1>(st, kt, cnt, last, abase, wbase, aoff, boff, wave,
                                             wm, brow, fr, lane, f0, f1, acc);
        }
    }
}

// Issue stages S .. NS-1 of the prologue into their buffers.
template <int BM, int BK, int NS, int S>
__device__ __forceinline__ void prologue(const Stages<NS> &st, int last, const uint16_t *abase,
                                         const uint16_t *wbase,
                                         const uint32_t (&aoff)[Geo<BM, BK>::AL],
                                         const uint32_t (&boff)[Geo<BM, BK>::BL], int wave) {
    if constexpr (S < NS) {
        dma_stage<BM, BK>(st.s[S], abase, wbase, aoff, boff, min(S * BK, last), wave);
        prologue<BM, BK, NS, S + 1>(st, last, abase, wbase, aoff, boff, wave);
    }
}

template <int BM, int BK, int NS, int MACT>
__device__ __forceinline__ void k_loop(const Stages<NS> &st, const uint16_t *abase,
                                       const uint16_t *wbase,
                                       const uint32_t (&aoff)[Geo<BM, BK>::AL],
                                       const uint32_t (&boff)[Geo<BM, BK>::BL], int nk, int wave,
                                       int wm, const int (&brow)[NB], int fr, int lane,
                                       f32x16 (&acc)[Geo<BM, BK>::MI][NB]) {
    const int last = (nk - 1) * BK;
    prologue<BM, BK, NS, 0>(st, last, abase, wbase, aoff, boff, wave);
    compiler_fence();
    __builtin_amdgcn_s_waitcnt(vmcnt_imm((NS - 1) * Geo<BM, BK>::LOADS));
    __builtin_amdgcn_s_barrier();
    compiler_fence();
    Frags f0, f1;
    read_frags<BM, BK, MACT>(st.s[0], 0, wm, brow, fr, lane, f0);
    int kt = 0;
    for (; kt + NS <= nk; kt += NS)
        k_steps<BM, BK, NS, MACT, 0>(st, kt, NS, last, abase, wbase, aoff, boff, wave, wm, brow,
                                     fr, lane, f0, f1, acc);
    k_steps<BM, BK, NS, MACT, 0>(st, kt, nk - kt, last, abase, wbase, aoff, boff, wave, wm, brow,
                                 fr, lane, f0, f1, acc);
    compiler_fence();
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));  // no load may land after the block ends
    __builtin_amdgcn_s_barrier();
    compiler_fence();
}

// NS stage buffers; up to 80 KB of them leaves room for two blocks per CU, so
// one block's start-up and epilogue overlap the other's streaming.
template <int MODE, int BM, int BK, int NS>
__global__ __launch_bounds__((64 * Geo<BM, BK>::NW), (NS * Geo<BM, BK>::STB <= 80 * 1024 ? 2 : 1)) void gemm_dma_kernel(
    GemmArgs a) {
    using G = Geo<BM, BK>;
    static_assert(NS >= 3 && NS <= 6, "three to six stage buffers");
    __shared__ __align__(1024) unsigned char st0[G::STB];
    __shared__ __align__(1024) unsigned char st1[G::STB];
    __shared__ __align__(1024) unsigned char st2[G::STB];
    __shared__ __align__(1024) unsigned char st3[NS > 3 ? G::STB : 16];
    __shared__ __align__(1024) unsigned char st4[NS > 4 ? G::STB : 16];
    __shared__ __align__(1024) unsigned char st5[NS > 5 ? G::STB : 16];
    __shared__ int32_t row_tok[BM];
    __shared__ float row_w[BM];

    int mt, nt;
    if (!raster_tile(a.nm, a.nn, a.gm, mt, nt)) return;
    const int tile = mt;
    if (tile >= a.tile_start[a.E + 1]) return;
    const int g = a.tile_group[tile];
    const bool shared = g == a.E;
    const int m_local = (tile - a.tile_start[g]) * BM;
    int row0, nrows;
    if (!shared) {
        row0 = a.offsets[g] + m_local;
        nrows = min(BM, a.counts[g] - m_local);
    } else {
        row0 = m_local;
        nrows = (int)min<int64_t>(BM, a.T - m_local);
    }
    const int Fg = shared ? a.Fs : a.F;
    const int N = MODE == 0 ? Fg : a.d;
    const int K = MODE == 1 ? Fg : a.d;
    const int n0 = nt * (MODE == 0 ? BN / 2 : BN);
    if (n0 >= N) return;

    const int tid = threadIdx.x;
    if (tid < BM) {
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
    const uint16_t *wbase = shared ? a.w_sh
                                   : a.w + (int64_t)g * (MODE == 0 ? (int64_t)2 * a.F * a.d
                                                                   : (int64_t)a.d * a.F);
    const uint16_t *abase = MODE == 1 ? (shared ? a.h_sh : a.h) : a.x;
    // element offsets (32-bit: the host checks that every offset fits) of this
    // lane's row and swizzled chunk in each of its loads
    uint32_t aoff[G::AL], boff[G::BL];
#pragma unroll
    for (int j = 0; j < G::AL; ++j) {
        const int R = (G::AL * wave + j) * G::RPL + lane / G::CH;
        const int c = (lane % G::CH) ^ swz<BK>(R);
        aoff[j] = (MODE == 1 ? (uint32_t)(row0 + min(R, nrows - 1)) * (uint32_t)Fg
                             : (uint32_t)row_tok[R] * (uint32_t)a.d) + 8 * c;
    }
#pragma unroll
    for (int j = 0; j < G::BL; ++j) {
        const int R = (G::BL * wave + j) * G::RPL + lane / G::CH;
        const int c = (lane % G::CH) ^ swz<BK>(R);
        boff[j] = (MODE == 1 ? (uint32_t)min(n0 + R, a.d - 1) * (uint32_t)Fg
                             : (uint32_t)(R < BN / 2 ? n0 + R : Fg + n0 + (R - BN / 2)) *
                                   (uint32_t)a.d) + 8 * c;
    }

    const int wm = wave >> 1, wn = wave & 1;
    const int fr = lane & 31;
    // B rows of this wave's four 32-column blocks.  Gate/up: gate blocks
    // 64 wn and 64 wn + 32, then the matching up blocks, so block pr pairs
    // with pr + 2.  Down: 128 wn + 32 ni.
    int brow[NB];
#pragma unroll
    for (int ni = 0; ni < NB; ++ni)
        brow[ni] = MODE == 0 ? (ni >> 1) * (BN / 2) + 64 * wn + 32 * (ni & 1) : 128 * wn + 32 * ni;
    // active 32-row sub-tiles of this wave's BM/2 rows (wave-uniform)
    const int mact = min(G::MI, max(0, (nrows - G::WR * wm + 31) / 32));

    f32x16 acc[G::MI][NB];
#pragma unroll
    for (int i = 0; i < G::MI; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

    const int nk = K / BK;
    Stages<NS> st;
    {
        unsigned char *all[6] = {st0, st1, st2, st3, st4, st5};
#pragma unroll
        for (int i = 0; i < NS; ++i) st.s[i] = all[i];
    }
    // mact is decided once, outside the K loop, so the loop body is one
    // straight block of loads and MFMAs.
#define MOE_LOOP(M) k_loop<BM, BK, NS, M>(st, abase, wbase, aoff, boff, nk, wave, wm, brow, fr, lane, acc)
    if constexpr (G::MI == 4) {
        switch (mact) {
        case 4: MOE_LOOP(4); break;
        case 3: MOE_LOOP(3); break;
        case 2: MOE_LOOP(2); break;
        case 1: MOE_LOOP(1); break;
        default: MOE_LOOP(0); break;
        }
    } else {
        switch (mact) {
        case 2: MOE_LOOP(2); break;
        case 1: MOE_LOOP(1); break;
        default: MOE_LOOP(0); break;
        }
    }
#undef MOE_LOOP

    // Accumulator layout (B A^T): lane holds token row WR wm + 32 mi + lane % 32
    // and, in acc[mi][ni][4 g + q], output column brow[ni] + 8 g + 4 (lane / 32) + q.
    const int cq = 4 * (lane >> 5);
    if (MODE == 0) {
        uint16_t *H = shared ? a.h_sh : a.h;
#pragma unroll
        for (int mi = 0; mi < G::MI; ++mi) {
            const int row = G::WR * wm + 32 * mi + fr;
            if (mi >= mact || row >= nrows) continue;
            uint16_t *hrow = H + (int64_t)(row0 + row) * Fg + n0 + 64 * wn + cq;
#pragma unroll
            for (int pr = 0; pr < 2; ++pr)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const f32x16 &gt = acc[mi][pr], &up = acc[mi][pr + 2];
                    uint2 q;
                    q.x = pack_bf16x2(silu_mul(gt[4 * g], up[4 * g]), silu_mul(gt[4 * g + 1], up[4 * g + 1]));
                    q.y = pack_bf16x2(silu_mul(gt[4 * g + 2], up[4 * g + 2]),
                                      silu_mul(gt[4 * g + 3], up[4 * g + 3]));
                    *reinterpret_cast<uint2 *>(hrow + 32 * pr + 8 * g) = q;
                }
            if (a.au) {
                // training forward: the pre-activations too, gate half then up half
                uint16_t *arow = (shared ? a.au_sh : a.au) + (int64_t)(row0 + row) * 2 * Fg + n0 +
                                 64 * wn + cq;
#pragma unroll
                for (int pr = 0; pr < 2; ++pr)
#pragma unroll
                    for (int g = 0; g < 4; ++g)
#pragma unroll
                        for (int half = 0; half < 2; ++half) {
                            const f32x16 &v = acc[mi][pr + 2 * half];
                            uint2 q;
                            q.x = pack_bf16x2(v[4 * g], v[4 * g + 1]);
                            q.y = pack_bf16x2(v[4 * g + 2], v[4 * g + 3]);
                            *reinterpret_cast<uint2 *>(arow + half * Fg + 32 * pr + 8 * g) = q;
                        }
            }
        }
    } else {
#pragma unroll
        for (int mi = 0; mi < G::MI; ++mi) {
            const int row = G::WR * wm + 32 * mi + fr;
            if (mi >= mact || row >= nrows) continue;
            const float wgt = row_w[row];
            if (!shared) {
                // routed rows: weighted, into y (16-bit block floating point)
                uint8_t *yrow = a.y + (int64_t)(row0 + row) * y16_pitch(a.d);
                // a lane holds four consecutive columns of each 8-column
                // group, lane ^ 32 the other four (same row): the group's
                // exponent is their joint maximum, and the lane below 32
                // writes the four exponent bytes of a 32-column block at once
#pragma unroll
                for (int ni = 0; ni < NB; ++ni) {
                    const int cb = n0 + brow[ni];
                    if (cb >= a.d) continue;
                    const f32x16 &c = acc[mi][ni];
                    uint32_t xw = 0;
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        const float v0 = wgt * c[4 * g], v1 = wgt * c[4 * g + 1];
                        const float v2 = wgt * c[4 * g + 2], v3 = wgt * c[4 * g + 3];
                        float am = absmax4(v0, v1, v2, v3);
                        am = fmaxf(am, __shfl_xor(am, 32, 64));
                        const uint32_t x = y16_exponent(am);
                        uint2 m;
                        m.x = y16_pack2(v0, v1, x);
                        m.y = y16_pack2(v2, v3, x);
                        *reinterpret_cast<uint2 *>(yrow + 2 * (int64_t)(cb + 8 * g + cq)) = m;
                        xw |= x << (8 * g);
                    }
                    if (cq == 0)
                        *reinterpret_cast<uint32_t *>(yrow + 2 * (int64_t)a.d + cb / 8) = xw;
                }
            } else {
                // shared expert: gated term, binary32, straight into out
                float *orow = a.out + (int64_t)row_tok[row] * a.d + n0 + cq;
#pragma unroll
                for (int ni = 0; ni < NB; ++ni)
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        const int col = n0 + brow[ni] + 8 * g + cq;
                        if (col >= a.d) continue;
                        const f32x16 &c = acc[mi][ni];
                        *reinterpret_cast<float4 *>(orow + brow[ni] + 8 * g) =
                            make_float4(wgt * c[4 * g], wgt * c[4 * g + 1], wgt * c[4 * g + 2],
                                        wgt * c[4 * g + 3]);
                    }
            }
        }
    }
}

// One tile of a launch: M-tile m of the permutation's tile map and N-tile n.
struct DmaTile {
    int g, row0, nrows, n0, Fg;
    bool shared;
};

// Tile of virtual block v (raster_tile's XCD-aware order: M-tile m on XCD
// m % 8, its N-tiles 8 ids apart); false when v has no work.  ntiles is the
// tile map's length.
template <int MODE, int BM>
__device__ __forceinline__ bool dma_tile(const GemmArgs &a, int v, int ntiles, DmaTile &t) {
    const int x = v & 7, q = v >> 3;
    const int n = q % a.nn, m = 8 * (q / a.nn) + x;
    if (m >= a.nm || m >= ntiles) return false;
    t.g = a.tile_group[m];
    t.shared = t.g == a.E;
    const int m_local = (m - a.tile_start[t.g]) * BM;
    if (!t.shared) {
        t.row0 = a.offsets[t.g] + m_local;
        t.nrows = min(BM, a.counts[t.g] - m_local);
    } else {
        t.row0 = m_local;
        t.nrows = (int)min<int64_t>(BM, a.T - m_local);
    }
    t.Fg = t.shared ? a.Fs : a.F;
    t.n0 = n * (MODE == 0 ? BN / 2 : BN);
    return t.n0 < (MODE == 0 ? t.Fg : a.d);
}

// Token (the gathered A row) and combine weight of tile row r (padding rows
// repeat the last row and are never stored).
template <int MODE>
__device__ __forceinline__ void dma_row(const GemmArgs &a, const DmaTile &t, int r, int &tok,
                                        float &wgt) {
    r = min(r, t.nrows - 1);
    wgt = 0.f;
    if (!t.shared) {
        const int pair = a.perm[t.row0 + r];
        tok = pair / a.k;
        if (MODE == 1) wgt = a.topk_w[pair];
    } else {
        tok = t.row0 + r;
        if (MODE == 1) wgt = a.gate[tok];
    }
}

template <int MODE>
__device__ __forceinline__ const uint16_t *dma_wbase(const GemmArgs &a, const DmaTile &t) {
    return t.shared ? a.w_sh
                    : a.w + (int64_t)t.g * (MODE == 0 ? (int64_t)2 * a.F * a.d : (int64_t)a.d * a.F);
}
template <int MODE>
__device__ __forceinline__ const uint16_t *dma_abase(const GemmArgs &a, const DmaTile &t) {
    return MODE == 1 ? (t.shared ? a.h_sh : a.h) : a.x;
}

// The tile's outputs from the accumulators: gate/up writes h = silu(g) u
// (and, training, the pre-activations), down writes the weighted routed rows
// y or the gated shared-expert term into out.
template <int MODE, int BM, int BK>
__device__ __forceinline__ void dma_epilogue(const GemmArgs &a, const DmaTile &t,
                                             const int32_t *row_tok, const float *row_w,
                                             const f32x16 (&acc)[Geo<BM, BK>::MI][NB], int mact,
                                             int wm, int wn, const int (&brow)[NB], int fr,
                                             int lane) {
    using G = Geo<BM, BK>;
    const bool shared = t.shared;
    const int row0 = t.row0, nrows = t.nrows, n0 = t.n0, Fg = t.Fg;
    // Accumulator layout (B A^T): lane holds token row WR wm + 32 mi + lane % 32
    // and, in acc[mi][ni][4 g + q], output column brow[ni] + 8 g + 4 (lane / 32) + q.
    const int cq = 4 * (lane >> 5);
    if (MODE == 0) {
        uint16_t *H = shared ? a.h_sh : a.h;
#pragma unroll
        for (int mi = 0; mi < G::MI; ++mi) {
            const int row = G::WR * wm + 32 * mi + fr;
            if (mi >= mact || row >= nrows) continue;
            uint16_t *hrow = H + (int64_t)(row0 + row) * Fg + n0 + 64 * wn + cq;
#pragma unroll
            for (int pr = 0; pr < 2; ++pr)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const f32x16 &gt = acc[mi][pr], &up = acc[mi][pr + 2];
                    uint2 q;
                    q.x = pack_bf16x2(silu_mul(gt[4 * g], up[4 * g]), silu_mul(gt[4 * g + 1], up[4 * g + 1]));
                    q.y = pack_bf16x2(silu_mul(gt[4 * g + 2], up[4 * g + 2]),
                                      silu_mul(gt[4 * g + 3], up[4 * g + 3]));
                    *reinterpret_cast<uint2 *>(hrow + 32 * pr + 8 * g) = q;
                }
            if (a.au) {
                // training forward: the pre-activations too, gate half then up half
                uint16_t *arow = (shared ? a.au_sh : a.au) + (int64_t)(row0 + row) * 2 * Fg + n0 +
                                 64 * wn + cq;
#pragma unroll
                for (int pr = 0; pr < 2; ++pr)
#pragma unroll
                    for (int g = 0; g < 4; ++g)
#pragma unroll
                        for (int half = 0; half < 2; ++half) {
                            const f32x16 &v = acc[mi][pr + 2 * half];
                            uint2 q;
                            q.x = pack_bf16x2(v[4 * g], v[4 * g + 1]);
                            q.y = pack_bf16x2(v[4 * g + 2], v[4 * g + 3]);
                            *reinterpret_cast<uint2 *>(arow + half * Fg + 32 * pr + 8 * g) = q;
                        }
            }
        }
    } else {
#pragma unroll
        for (int mi = 0; mi < G::MI; ++mi) {
            const int row = G::WR * wm + 32 * mi + fr;
            if (mi >= mact || row >= nrows) continue;
            const float wgt = row_w[row];
            if (!shared) {
                // routed rows: weighted, into y (16-bit block floating point)
                uint8_t *yrow = a.y + (int64_t)(row0 + row) * y16_pitch(a.d);
                // a lane holds four consecutive columns of each 8-column
                // group, lane ^ 32 the other four (same row): the group's
                // exponent is their joint maximum, and the lane below 32
                // writes the four exponent bytes of a 32-column block at once
#pragma unroll
                for (int ni = 0; ni < NB; ++ni) {
                    const int cb = n0 + brow[ni];
                    if (cb >= a.d) continue;
                    const f32x16 &c = acc[mi][ni];
                    uint32_t xw = 0;
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        const float v0 = wgt * c[4 * g], v1 = wgt * c[4 * g + 1];
                        const float v2 = wgt * c[4 * g + 2], v3 = wgt * c[4 * g + 3];
                        float am = absmax4(v0, v1, v2, v3);
                        am = fmaxf(am, __shfl_xor(am, 32, 64));
                        const uint32_t x = y16_exponent(am);
                        uint2 m;
                        m.x = y16_pack2(v0, v1, x);
                        m.y = y16_pack2(v2, v3, x);
                        *reinterpret_cast<uint2 *>(yrow + 2 * (int64_t)(cb + 8 * g + cq)) = m;
                        xw |= x << (8 * g);
                    }
                    if (cq == 0)
                        *reinterpret_cast<uint32_t *>(yrow + 2 * (int64_t)a.d + cb / 8) = xw;
                }
            } else {
                // shared expert: gated term, binary32, straight into out
                float *orow = a.out + (int64_t)row_tok[row] * a.d + n0 + cq;
#pragma unroll
                for (int ni = 0; ni < NB; ++ni)
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        const int col = n0 + brow[ni] + 8 * g + cq;
                        if (col >= a.d) continue;
                        const f32x16 &c = acc[mi][ni];
                        *reinterpret_cast<float4 *>(orow + brow[ni] + 8 * g) =
                            make_float4(wgt * c[4 * g], wgt * c[4 * g + 1], wgt * c[4 * g + 2],
                                        wgt * c[4 * g + 3]);
                    }
            }
        }
    }
}

// Where a K step's refill comes from: the operands of one tile.
template <int BM, int BK> struct DmaSrc {
    const uint16_t *a, *w;
    uint32_t ao[Geo<BM, BK>::AL], bo[Geo<BM, BK>::BL];
};

// The tile's load sources: B rows of its weight slice, A rows of its tokens
// (gate/up: the gathered x rows, each lane looking up the tokens of its own
// loads) or of h (down).  Element offsets are 32-bit (the host checks that
// every offset fits).
template <int MODE, int BM, int BK>
__device__ __forceinline__ void dma_src(const GemmArgs &a, const DmaTile &t, int wave, int lane,
                                        DmaSrc<BM, BK> &src) {
    using G = Geo<BM, BK>;
    src.a = dma_abase<MODE>(a, t);
    src.w = dma_wbase<MODE>(a, t);
#pragma unroll
    for (int j = 0; j < G::AL; ++j) {
        const int R = (G::AL * wave + j) * G::RPL + lane / G::CH;
        const int c = (lane % G::CH) ^ swz<BK>(R);
        const int r = t.row0 + min(R, t.nrows - 1);
        if (MODE == 1) {
            src.ao[j] = (uint32_t)r * (uint32_t)t.Fg + 8 * c;
        } else {
            const int tok = t.shared ? r : a.perm[r] / a.k;
            src.ao[j] = (uint32_t)tok * (uint32_t)a.d + 8 * c;
        }
    }
#pragma unroll
    for (int j = 0; j < G::BL; ++j) {
        const int R = (G::BL * wave + j) * G::RPL + lane / G::CH;
        const int c = (lane % G::CH) ^ swz<BK>(R);
        src.bo[j] = (MODE == 1 ? (uint32_t)min(t.n0 + R, a.d - 1) * (uint32_t)t.Fg
                               : (uint32_t)(R < BN / 2 ? t.n0 + R : t.Fg + t.n0 + (R - BN / 2)) *
                                     (uint32_t)a.d) + 8 * c;
    }
}

// k_step (on buffer S) with the refill taken across tiles: stage kt + NS of
// this tile, or, past its last step, stage kt + NS - nk of the next tile
// (which lands in the buffer the next tile's K loop reads it from), or,
// with no next tile, this tile's last stage again (never computed).  The
// source is selected, the loads are issued either way, so every step keeps
// NS - 1 stages in flight and the waits are those of k_step.
template <int BM, int BK, int NS, int MACT, int S>
__device__ __forceinline__ void k_step_xt(const Stages<NS> &st, int kt, int nk, bool has,
                                          const DmaSrc<BM, BK> &cur, const DmaSrc<BM, BK> &nxt,
                                          int wave, int wm, const int (&brow)[NB], int fr,
                                          int lane, Frags &f0, Frags &f1,
                                          f32x16 (&acc)[Geo<BM, BK>::MI][NB]) {
    using G = Geo<BM, BK>;
    sub_step<BM, BK, MACT>(st.s[S], 1, wm, brow, fr, lane, f0, f1, acc);
    if constexpr (G::Q == 4) {
        sub_step<BM, BK, MACT>(st.s[S], 2, wm, brow, fr, lane, f1, f0, acc);
        sub_step<BM, BK, MACT>(st.s[S], 3, wm, brow, fr, lane, f0, f1, acc);
    }
    compiler_fence();
    __builtin_amdgcn_s_waitcnt(vmcnt_lgkm0_imm((NS - 2) * G::LOADS));
    __builtin_amdgcn_s_barrier();
    compiler_fence();
    const int sk = kt + NS;
    const bool in = sk < nk, to_next = !in && has;
    const int k0 = (in ? sk : (has ? sk - nk : nk - 1)) * BK;
    uint32_t ao[G::AL], bo[G::BL];
#pragma unroll
    for (int j = 0; j < G::AL; ++j) ao[j] = to_next ? nxt.ao[j] : cur.ao[j];
#pragma unroll
    for (int j = 0; j < G::BL; ++j) bo[j] = to_next ? nxt.bo[j] : cur.bo[j];
    dma_stage<BM, BK>(st.s[S], to_next ? nxt.a : cur.a, to_next ? nxt.w : cur.w, ao, bo, k0, wave);
    __builtin_amdgcn_sched_barrier(0);
    sub_step<BM, BK, MACT>(st.s[(S + 1) % NS], 0, wm, brow, fr, lane, f1, f0, acc);
}

// Local steps kt + I .. kt + cnt - 1 (cnt <= NS) of a tile whose stage 0
// sits in buffer P: local step j reads buffer (P + j) % NS, a constant here.
template <int BM, int BK, int NS, int MACT, int P, int I>
__device__ __forceinline__ void k_steps_xt(const Stages<NS> &st, int kt, int cnt, int nk, bool has,
                                           const DmaSrc<BM, BK> &cur, const DmaSrc<BM, BK> &nxt,
                                           int wave, int wm, const int (&brow)[NB], int fr,
                                           int lane, Frags &f0, Frags &f1,
                                           f32x16 (&acc)[Geo<BM, BK>::MI][NB]) {
    if constexpr (I < NS) {
        if (I < cnt) {
            k_step_xt<BM, BK, NS, MACT, (P + I) % NS>(st, kt + I, nk, has, cur, nxt, wave, wm,
                                                      brow, fr, lane, f0, f1, acc);
            k_steps_xt<BM, BK, NS, MACT, P, I + 1>(st, kt, cnt, nk, has, cur, nxt, wave, wm, brow,
                                                   fr, lane, f0, f1, acc);
        }
    }
}

// One tile's K loop, its stage 0 in buffer P: wait for that stage (issued by
// the prologue or by the previous tile's last steps), then every step.  A
// refill past the last step lands where the next tile reads it: the next
// tile's stage 0 in buffer (P + nk) % NS.  No drain at the end: the next
// tile's first stages stay in flight.
template <int BM, int BK, int NS, int MACT, int P>
__device__ __forceinline__ void k_loop_xt(const Stages<NS> &st, int nk, bool has,
                                          const DmaSrc<BM, BK> &cur, const DmaSrc<BM, BK> &nxt,
                                          int wave, int wm, const int (&brow)[NB], int fr,
                                          int lane, f32x16 (&acc)[Geo<BM, BK>::MI][NB]) {
    compiler_fence();
    __builtin_amdgcn_s_waitcnt(vmcnt_imm((NS - 1) * Geo<BM, BK>::LOADS));
    __builtin_amdgcn_s_barrier();
    compiler_fence();
    Frags f0, f1;
    read_frags<BM, BK, MACT>(st.s[P], 0, wm, brow, fr, lane, f0);
    int kt = 0;
    for (; kt + NS <= nk; kt += NS)
        k_steps_xt<BM, BK, NS, MACT, P, 0>(st, kt, NS, nk, has, cur, nxt, wave, wm, brow, fr, lane,
                                           f0, f1, acc);
    k_steps_xt<BM, BK, NS, MACT, P, 0>(st, kt, nk - kt, nk, has, cur, nxt, wave, wm, brow, fr,
                                       lane, f0, f1, acc);
}

template <int BM, int BK, int NS, int MACT>
__device__ __forceinline__ void k_loop_xt_at(int ph, const Stages<NS> &st, int nk, bool has,
                                             const DmaSrc<BM, BK> &cur, const DmaSrc<BM, BK> &nxt,
                                             int wave, int wm, const int (&brow)[NB], int fr,
                                             int lane, f32x16 (&acc)[Geo<BM, BK>::MI][NB]) {
#define MOE_XT(P) k_loop_xt<BM, BK, NS, MACT, P>(st, nk, has, cur, nxt, wave, wm, brow, fr, lane, acc)
    switch (ph) {
    case 0: MOE_XT(0); break;
    case 1: MOE_XT(1); break;
    case 2: MOE_XT(2); break;
    default:
        if constexpr (NS > 3) MOE_XT(3);
        break;
    }
#undef MOE_XT
}

// The grouped GEMM with its K pipeline running across tiles: persistent
// blocks (one per CU, a multiple of 8) walk the tiles v = blockIdx.x,
// + gridDim.x, ... in raster_tile's XCD-aware order; the last NS steps of a
// tile load the first NS stages of the block's next tile, so the next tile
// starts on landed data while this one's epilogue runs.  Every tile has the
// same number of K steps nk >= NS (the host checks); the next tile's stage 0
// then sits in buffer (ph + nk) % NS, and its K loop is the instantiation
// for that buffer.  The next
// tile's token and weight lookups go out at the start of this tile's K loop;
// its rows' tokens and weights reach row_tok / row_w (the half this tile's
// epilogue does not read) before this tile's epilogue.
template <int MODE, int BM, int BK, int NS>
__global__ __launch_bounds__((64 * Geo<BM, BK>::NW), 1) void gemm_dma_xt_kernel(GemmArgs a) {
    using G = Geo<BM, BK>;
    static_assert(NS >= 3 && NS <= 4, "three or four stage buffers");
    __shared__ __align__(1024) unsigned char st0[G::STB];
    __shared__ __align__(1024) unsigned char st1[G::STB];
    __shared__ __align__(1024) unsigned char st2[G::STB];
    __shared__ __align__(1024) unsigned char st3[NS > 3 ? G::STB : 16];
    __shared__ int32_t row_tok[2][BM];
    __shared__ float row_w[2][BM];

    const int ntiles = a.tile_start[a.E + 1];
    const int nv = 8 * ((a.nm + 7) / 8) * a.nn;  // raster_blocks(nm, nn, -1)
    const int stride = (int)gridDim.x;
    const int nk = (MODE == 1 ? a.F : a.d) / BK;  // the same for every tile
    int v = blockIdx.x;
    DmaTile cur;
    while (v < nv && !dma_tile<MODE, BM>(a, v, ntiles, cur)) v += stride;
    if (v >= nv) return;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = wave_id();
    const int wm = wave >> 1, wn = wave & 1;
    const int fr = lane & 31;
    int brow[NB];
#pragma unroll
    for (int ni = 0; ni < NB; ++ni)
        brow[ni] = MODE == 0 ? (ni >> 1) * (BN / 2) + 64 * wn + 32 * (ni & 1) : 128 * wn + 32 * ni;
    Stages<NS> st;
    {
        unsigned char *all[4] = {st0, st1, st2, st3};
#pragma unroll
        for (int i = 0; i < NS; ++i) st.s[i] = all[i];
    }

    int buf = 0, ph = 0;  // ph: the buffer holding the current tile's stage 0
    if (tid < BM) {
        int tok;
        float wgt;
        dma_row<MODE>(a, cur, tid, tok, wgt);
        row_tok[0][tid] = tok;
        row_w[0][tid] = wgt;
    }
    DmaSrc<BM, BK> cs, ns;
    dma_src<MODE, BM, BK>(a, cur, wave, lane, cs);
    prologue<BM, BK, NS, 0>(st, (nk - 1) * BK, cs.a, cs.w, cs.ao, cs.bo, wave);
    for (;;) {
        int vn = v + stride;
        DmaTile nxt;
        bool has = false;
        for (; vn < nv; vn += stride)
            if (dma_tile<MODE, BM>(a, vn, ntiles, nxt)) {
                has = true;
                break;
            }
        int ntok = 0;
        float nwgt = 0.f;
        if (has) {
            dma_src<MODE, BM, BK>(a, nxt, wave, lane, ns);
            if (tid < BM) dma_row<MODE>(a, nxt, tid, ntok, nwgt);
        } else {
            ns = cs;
        }

        f32x16 acc[G::MI][NB];
#pragma unroll
        for (int i = 0; i < G::MI; ++i)
#pragma unroll
            for (int j = 0; j < NB; ++j)
#pragma unroll
                for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;
        const int mact = min(G::MI, max(0, (cur.nrows - G::WR * wm + 31) / 32));
#define MOE_LOOP(M) k_loop_xt_at<BM, BK, NS, M>(ph, st, nk, has, cs, ns, wave, wm, brow, fr, lane, acc)
        if constexpr (G::MI == 2) {
            switch (mact) {
            case 2: MOE_LOOP(2); break;
            case 1: MOE_LOOP(1); break;
            default: MOE_LOOP(0); break;
            }
        } else {
            switch (mact) {
            case 1: MOE_LOOP(1); break;
            default: MOE_LOOP(0); break;
            }
        }
#undef MOE_LOOP
        // row_tok / row_w [buf ^ 1] were last read by the previous tile's
        // epilogue, before this tile's K-loop barriers; the next tile's
        // epilogue reads them after its own K-loop barriers
        if (has && tid < BM) {
            row_tok[buf ^ 1][tid] = ntok;
            row_w[buf ^ 1][tid] = nwgt;
        }
        dma_epilogue<MODE, BM, BK>(a, cur, row_tok[buf], row_w[buf], acc, mact, wm, wn, brow, fr,
                                   lane);
        if (!has) break;
        cur = nxt;
        cs = ns;
        v = vn;
        buf ^= 1;
        ph = (ph + nk) % NS;
    }
    // the last tile's refills re-read its own last stage: no load may land
    // after the block ends
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
}

// ---------------------------------------------------------------------------
// Backward products whose weight operand runs along the output axis (dX of
// the rows, [da | du] W_gu, and G = dOut W_dn; the backward's 128-row tile
// map), on the 128 x 256 tiles above (K in steps of 64, three direct-to-LDS
// stages, 8 waves).  A (rows contiguous along K) is staged as the forward's
// A.  Each K step's 64 weight rows of 256 columns (512 bytes) go to LDS as
// loaded, two rows per 1 KB load, with the 16-byte chunks of row k permuted
// by chunk ^ 4 (k & 3); the MFMA fragments are read with ds_read_b64_tr_b16,
// and the 64 bytes that one read touches in each of four consecutive rows
// then sit in four different quarters of the 256-byte bank space.
namespace {
constexpr int MC_ROWB = BN * 2;  // bytes per staged B row (one K index)
constexpr int MC_AROWB = 128 * 2; // bytes per staged A row when A runs along the output axis too
__device__ __forceinline__ int mc_swz(int k) { return 4 * (k & 3); }

// One stage: A as dma_stage (AMC: like B, K rows k0 .. k0 + 63 of lda
// elements, aoff of this lane's row and chunk); B rows k0 .. k0 + 63
// (element offsets boff of this lane's row and chunk, plus k0 rows of ldb
// elements).
template <bool AMC>
__device__ __forceinline__ void dma_stage_mc(unsigned char *stage, const uint16_t *abase,
                                             const uint16_t *wbase,
                                             const uint32_t (&aoff)[Geo<128, 64>::AL],
                                             const uint32_t (&boff)[Geo<128, 64>::BL], int k0,
                                             uint32_t lda, uint32_t ldb, int wave) {
    using G = Geo<128, 64>;
    const uint16_t *ak = AMC ? abase + (size_t)k0 * lda : abase + k0;
#pragma unroll
    for (int j = 0; j < G::AL; ++j)
        __builtin_amdgcn_global_load_lds((const global_void_t *)(ak + aoff[j]),
                                         (lds_void_t *)(stage + (G::AL * wave + j) * 1024), 16,
                                         0, 0);
    const uint16_t *wk = wbase + (size_t)k0 * ldb;
#pragma unroll
    for (int j = 0; j < G::BL; ++j)
        __builtin_amdgcn_global_load_lds(
            (const global_void_t *)(wk + boff[j]),
            (lds_void_t *)(stage + G::OPA + (G::BL * wave + j) * 1024), 16, 0, 0);
}

typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16_t lds_v4i16_t;

// Fragment of output columns nb .. nb + 31 at k16 step ks from a tile whose
// K rows are ROWB bytes: lane L gets column nb + L % 32, K rows 16 ks + 8 (L
// / 32) .. + 7.  Lane s of a 16-lane group addresses K row k + s / 4,
// columns 4 (s % 4) .. + 3 of its 16-column half; the transposing read hands
// lane s column s of those four rows, and a second read four rows down
// completes the eight.
template <int ROWB>
__device__ __forceinline__ bf16x8 mc_tfrag(const unsigned char *bst, int ks, int nb, int lane) {
    const int g = lane >> 4, s = lane & 15;
    const int k = 16 * ks + 8 * (g >> 1) + (s >> 2);
    const int m = nb + 16 * (g & 1) + 4 * (s & 3);
    const int off = (((m >> 3) ^ mc_swz(k)) << 4) + (m & 7) * 2;  // k and k + 4: same swizzle
    const unsigned char *p = bst + k * ROWB + off;
    const v4i16_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t *)p);
    const v4i16_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t *)(p + 4 * ROWB));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

template <int MACT, bool AMC>
__device__ __forceinline__ void read_frags_mc(const unsigned char *stage, int ks, int wm,
                                              const int (&brow)[NB], int fr, int lane, Frags &f) {
    if (MACT == 0) return;
    if (AMC) {
        f.a[0] = mc_tfrag<MC_AROWB>(stage, ks, 32 * wm, lane);
    } else {
        const int c = 2 * ks + (lane >> 5);
        f.a[0] = *reinterpret_cast<const bf16x8 *>(stage + tile_off<64>(32 * wm + fr, c));
    }
#pragma unroll
    for (int ni = 0; ni < NB; ++ni) f.b[ni] = mc_tfrag<MC_ROWB>(stage + Geo<128, 64>::OPA, ks, brow[ni], lane);
}

template <int MACT, bool AMC>
__device__ __forceinline__ void sub_step_mc(const unsigned char *stage, int ks, int wm,
                                            const int (&brow)[NB], int fr, int lane,
                                            const Frags &cur, Frags &nxt, f32x16 (&acc)[1][NB]) {
    if (MACT > 0) {
        mfma_frags<MACT>(cur, acc);
        read_frags_mc<MACT, AMC>(stage, ks, wm, brow, fr, lane, nxt);
        interleave_reads<MACT>();
    }
    __builtin_amdgcn_sched_barrier(0);
}

// Operands of one tile's K loop.
struct McOps {
    const uint16_t *abase, *wbase;
    uint32_t aoff[Geo<128, 64>::AL], boff[Geo<128, 64>::BL];
    uint32_t lda, ldb;
};

// One K step on constant buffer S (as k_step).
template <int MACT, bool AMC, int S>
__device__ __forceinline__ void k_step_mc(const Stages<3> &st, int kt, int last, const McOps &o,
                                          int wave, int wm, const int (&brow)[NB], int fr,
                                          int lane, Frags &f0, Frags &f1, f32x16 (&acc)[1][NB]) {
    using G = Geo<128, 64>;
    sub_step_mc<MACT, AMC>(st.s[S], 1, wm, brow, fr, lane, f0, f1, acc);
    sub_step_mc<MACT, AMC>(st.s[S], 2, wm, brow, fr, lane, f1, f0, acc);
    sub_step_mc<MACT, AMC>(st.s[S], 3, wm, brow, fr, lane, f0, f1, acc);
    compiler_fence();
    __builtin_amdgcn_s_waitcnt(vmcnt_lgkm0_imm(G::LOADS));
    __builtin_amdgcn_s_barrier();
    compiler_fence();
    dma_stage_mc<AMC>(st.s[S], o.abase, o.wbase, o.aoff, o.boff, min((kt + 3) * 64, last), o.lda,
                      o.ldb, wave);
    __builtin_amdgcn_sched_barrier(0);
    sub_step_mc<MACT, AMC>(st.s[(S + 1) % 3], 0, wm, brow, fr, lane, f1, f0, acc);
}

template <int MACT, bool AMC, int S>
__device__ __forceinline__ void k_steps_mc(const Stages<3> &st, int kt, int cnt, int last,
                                           const McOps &o, int wave, int wm,
                                           const int (&brow)[NB], int fr, int lane, Frags &f0,
                                           Frags &f1, f32x16 (&acc)[1][NB]) {
    if constexpr (S < 3) {
        if (S < cnt) {
            k_step_mc<MACT, AMC, S>(st, kt + S, last, o, wave, wm, brow, fr, lane, f0, f1, acc);
            k_steps_mc<MACT, AMC, S + 1>(st, kt, cnt, last, o, wave, wm, brow, fr, lane, f0, f1,
                                         acc);
        }
    }
}

template <int MACT, bool AMC>
__device__ __forceinline__ void k_loop_mc(const Stages<3> &st, const McOps &o, int nk, int wave,
                                          int wm, const int (&brow)[NB], int fr, int lane,
                                          f32x16 (&acc)[1][NB]) {
    const int last = (nk - 1) * 64;
#pragma unroll
    for (int i = 0; i < 3; ++i)
        dma_stage_mc<AMC>(st.s[i], o.abase, o.wbase, o.aoff, o.boff, min(i * 64, last), o.lda,
                          o.ldb, wave);
    compiler_fence();
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * Geo<128, 64>::LOADS));
    __builtin_amdgcn_s_barrier();
    compiler_fence();
    Frags f0, f1;
    read_frags_mc<MACT, AMC>(st.s[0], 0, wm, brow, fr, lane, f0);
    int kt = 0;
    for (; kt + 3 <= nk; kt += 3)
        k_steps_mc<MACT, AMC, 0>(st, kt, 3, last, o, wave, wm, brow, fr, lane, f0, f1, acc);
    k_steps_mc<MACT, AMC, 0>(st, kt, nk - kt, last, o, wave, wm, brow, fr, lane, f0, f1, acc);
    compiler_fence();
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));  // no load may land after the block ends
    __builtin_amdgcn_s_barrier();
    compiler_fence();
}
}  // namespace

// The two backward products on these tiles (B runs along the output axis):
//   BWD_DX: dX rows = [da | du] W_gu   (A: [da | du] rows, K = 2 Fg; bf16 out, N = d)
//   BWD_G:  G rows  = dOut W_dn        (A: the rows' tokens of dOut, rounded to
//           bf16 beforehand, K = d; N = Fg), consumed in the epilogue by the
//           SwiGLU backward: G never leaves the registers
enum { BWD_DX = 0, BWD_G = 1 };

struct BwdTileArgs {
    const uint16_t *a, *a_sh;      // DX: [da | du] [T k, 2F], [T, 2Fs]; G: dOut bf16 [T, d]
    const uint16_t *w, *w_sh;      // DX: W_gu [E, 2F, d], [2Fs, d]; G: W_dn [E, d, F], [d, Fs]
    void *c, *c_sh;                // DX: dX rows bf16 [T k, d], [T, d]
    const int32_t *perm, *counts, *offsets, *tile_start, *tile_group;
    int64_t T;
    int d, E, k, F, Fs;
    int nm, nn, gm;
    // BWD_G's SwiGLU backward (rows in the tile map's order, as G's)
    const uint16_t *au, *au_sh;    // [T k, 2F], [T, 2Fs]  gate | up pre-activations
    uint16_t *dgu, *dgu_sh;        // [T k, 2F], [T, 2Fs]  da | du
    uint16_t *hh, *hh_sh;          // [T k, F], [T, Fs]    w h
    const float *topk_w;           // [T k] routed rows' combine weights (pair order)
    const float *logits;           // [logit_split, T, ldl] router logit partials (column E: shared gate)
    float *gate;                   // [T] s_t = sigmoid of the shared gate's logit
    float *dwp, *ds;               // G . h per row and 128 columns: [T k, np] (pair order), [T, np]
    int ldl, logit_split, np;
};

template <int KIND>
__global__ __launch_bounds__(512, 1) void bwd_mc_dma_kernel(BwdTileArgs a) {
    using G = Geo<128, 64>;
    __shared__ __align__(1024) unsigned char st0[G::STB];
    __shared__ __align__(1024) unsigned char st1[G::STB];
    __shared__ __align__(1024) unsigned char st2[G::STB];
    int mt, nt;
    if (!raster_tile(a.nm, a.nn, a.gm, mt, nt)) return;
    if (mt >= a.tile_start[a.E + 1]) return;
    const int g = a.tile_group[mt];
    const bool shared = g == a.E;
    const int m_local = (mt - a.tile_start[g]) * 128;
    int row0, nrows;
    if (!shared) {
        row0 = a.offsets[g] + m_local;
        nrows = min(128, a.counts[g] - m_local);
    } else {
        row0 = m_local;
        nrows = (int)min<int64_t>(128, a.T - m_local);
    }
    const int Fg = shared ? a.Fs : a.F;
    const int K = KIND == BWD_DX ? 2 * Fg : a.d;
    const int N = KIND == BWD_DX ? a.d : Fg;
    const int n0 = nt * BN;
    if (n0 >= N) return;

    const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
    McOps o;
    o.abase = shared ? a.a_sh : a.a;
    o.wbase = shared ? a.w_sh : a.w + (int64_t)g * (KIND == BWD_DX ? 2 * a.F : a.F) * a.d;
    o.lda = (uint32_t)K;
    o.ldb = (uint32_t)N;
    uint32_t (&aoff)[G::AL] = o.aoff;
    uint32_t (&boff)[G::BL] = o.boff;
    // BWD_G: the SwiGLU backward in the epilogue gives thread tid the rows
    // 32 it + tid / 16 (it < 4) of the tile and, in each 128-column half, the
    // 8 columns 8 (tid % 16); their pairs are looked up with the A rows' (a
    // shared row reads some pair id, clamped to the valid range, unused)
    const int er = tid >> 4, ec = 8 * (tid & 15);
    int epair[4];
#pragma unroll
    for (int it = 0; it < 4; ++it)
        epair[it] = KIND == BWD_G ? (int)min<int64_t>(max(a.perm[row0 + min(32 * it + er, nrows - 1)], 0),
                                                      a.T * a.k - 1)
                                  : 0;
#pragma unroll
    for (int j = 0; j < G::AL; ++j) {
        const int R = (G::AL * wave + j) * G::RPL + lane / G::CH;
        const int c = (lane % G::CH) ^ swz<64>(R);
        const int r = row0 + min(R, nrows - 1);  // padding rows repeat the last row
        // G: the row's token (routed rows through the permutation)
        const int src = KIND == BWD_DX || shared ? r : a.perm[r] / a.k;
        aoff[j] = (uint32_t)src * (uint32_t)K + 8 * c;
    }
#pragma unroll
    for (int j = 0; j < G::BL; ++j) {
        // K row kr of the stage, physical chunk p: logical chunk p ^ swizzle;
        // columns past N read the last full chunk (never stored)
        const int kr = 2 * (G::BL * wave + j) + (lane >> 5);
        const int col = min(n0 + 8 * ((lane & 31) ^ mc_swz(kr)), N - 8);
        boff[j] = (uint32_t)kr * (uint32_t)N + (uint32_t)col;
    }
    const int wm = wave >> 1, wn = wave & 1, fr = lane & 31;
    int brow[NB];
#pragma unroll
    for (int ni = 0; ni < NB; ++ni) brow[ni] = 128 * wn + 32 * ni;
    const int mact = nrows > 32 * wm ? 1 : 0;  // this wave's 32 rows hold data
    // BWD_G: the epilogue's operands, issued before the K loop so that they
    // land with its first stages, all unconditionally (clamped to valid
    // addresses; a branch here makes the compiler wait for every load at its
    // join): the routed rows' weights, the shared rows' gate logits (at most
    // two K slices), and 8 gate and 8 up pre-activations per row and half
    uint4 pa[2][4], pu[2][4];
    float wpair[4], z0[4], z1[4];
    if (KIND == BWD_G) {
#pragma unroll
        for (int it = 0; it < 4; ++it) {
            const int64_t rc = row0 + min(32 * it + er, nrows - 1);
            wpair[it] = a.topk_w[epair[it]];
            const int64_t tok = shared ? rc : 0;
            z0[it] = a.logits[tok * a.ldl + a.E];
            z1[it] = a.logits[((a.logit_split > 1 ? a.T : 0) + tok) * a.ldl + a.E];
            const uint16_t *aur = (shared ? a.au_sh : a.au) + rc * 2 * Fg + ec;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int c0 = min(n0 + 128 * h, N - 128);
                pa[h][it] = *reinterpret_cast<const uint4 *>(aur + c0);
                pu[h][it] = *reinterpret_cast<const uint4 *>(aur + Fg + c0);
            }
        }
    }
    f32x16 acc[1][NB];
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[0][j][v] = 0.f;
    Stages<3> st;
    st.s[0] = st0;
    st.s[1] = st1;
    st.s[2] = st2;
    if (mact)
        k_loop_mc<1, false>(st, o, K / 64, wave, wm, brow, fr, lane, acc);
    else
        k_loop_mc<0, false>(st, o, K / 64, wave, wm, brow, fr, lane, acc);
    if (KIND == BWD_G) {
        // the K loop ended with every load complete; uses here let the
        // compiler know (else it waits for them again in the epilogue,
        // counting the epilogue's own stores)
#pragma unroll
        for (int it = 0; it < 4; ++it) {
            asm volatile("" ::"v"(wpair[it]), "v"(z0[it]), "v"(z1[it]), "v"(epair[it]));
#pragma unroll
            for (int h = 0; h < 2; ++h)
                asm volatile("" ::"v"(pa[h][it].x), "v"(pa[h][it].y), "v"(pa[h][it].z),
                             "v"(pa[h][it].w), "v"(pu[h][it].x), "v"(pu[h][it].y),
                             "v"(pu[h][it].z), "v"(pu[h][it].w));
        }
    }
    // lane holds row 32 wm + lane % 32 and, in acc[0][ni][4 q + i], column
    // brow[ni] + 8 q + 4 (lane / 32) + i
    if (KIND == BWD_DX) {
        // the tile goes out through the idle stage buffers (rows 0 .. 63 in
        // buffer 0, 64 .. 127 in buffer 1; 512-byte rows, chunk c of row r
        // at chunk c ^ (r & 31)) as whole 512-byte row pieces, nontemporal:
        // 8-byte pieces straight from the accumulators took 0.81 against
        // 0.73 ms for the 210 MB at T = 4096 (the dx combine, which reads
        // them next, is no slower for it)
        typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
        unsigned char *sbuf = wm < 2 ? st0 : st1;
        const int rl = 32 * (wm & 1) + fr;
#pragma unroll
        for (int ni = 0; ni < NB; ++ni)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const f32x16 &c4 = acc[0][ni];
                const int col = brow[ni] + 8 * q + 4 * (lane >> 5);
                int off = rl * 512 + (((col >> 3) ^ (rl & 31)) << 4) + (col & 7) * 2;
                asm volatile("" : "+v"(off));
                *reinterpret_cast<uint2 *>(sbuf + off) =
                    make_uint2(pack_bf16x2(c4[4 * q], c4[4 * q + 1]), pack_bf16x2(c4[4 * q + 2], c4[4 * q + 3]));
            }
        compiler_fence();
        __builtin_amdgcn_s_waitcnt(0xC07F);
        __builtin_amdgcn_s_barrier();
        compiler_fence();
        uint16_t *cb = static_cast<uint16_t *>(shared ? a.c_sh : a.c) + (int64_t)row0 * N + n0;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int pc = tid + 512 * i, r = pc >> 5, c = pc & 31, r2 = r & 63;
            const unsigned char *src = (i < 4 ? st0 : st1) + r2 * 512 + ((c ^ (r2 & 31)) << 4);
            const u32x4_t v = *reinterpret_cast<const u32x4_t *>(src);
            if (r < nrows && n0 + 8 * c < N) {
                uint16_t *dst = cb + (int64_t)r * N + 8 * c;
                __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t *>(dst));
            }
        }
        return;
    }
    if (KIND == BWD_G) {
        // SwiGLU backward on the tile, in two passes of 128 columns: pass h
        // stages G of the waves with wn == h in LDS (binary32, 512-byte rows,
        // rows 0 .. 63 in buffer 0 and 64 .. 127 in buffer 1, chunk c of row
        // r at chunk c ^ (r & 31)); then every thread takes its rows' 8
        // columns (only rows that hold data: the work is spread evenly over
        // the block whatever the tile's fill).  With s = sigmoid(a) (through
        // the hardware reciprocal, about 1 ulp), h = a s u, dh = w G:
        // da = dh u s (1 + a (1 - s)), du = dh a s, the stored H = w h; and
        // G . h of the row's 128 columns (16 lanes' sums in a fixed tree) as
        // one partial, 128 columns apart in dwp / ds.
        typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
        float ew[4];
#pragma unroll
        for (int it = 0; it < 4; ++it)
            ew[it] = shared ? 1.0f / (1.0f + __expf(-(z0[it] + (a.logit_split > 1 ? z1[it] : 0.f))))
                            : wpair[it];
        if (shared && nt == 0 && (tid & 15) == 0) {
#pragma unroll
            for (int it = 0; it < 4; ++it)
                if (32 * it + er < nrows) a.gate[row0 + 32 * it + er] = ew[it];
        }
        uint16_t *dgu = shared ? a.dgu_sh : a.dgu;
        uint16_t *hhp = shared ? a.hh_sh : a.hh;
        unsigned char *sbuf = wm < 2 ? st0 : st1;
        const int rl = 32 * (wm & 1) + fr;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            if (n0 + 128 * h >= N) break;  // block-uniform
            if (wn == h) {
#pragma unroll
                for (int ni = 0; ni < NB; ++ni)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const f32x16 &c4 = acc[0][ni];
                        const int col = 32 * ni + 8 * q + 4 * (lane >> 5);  // of the 128
                        int off = rl * 512 + (((col >> 2) ^ (rl & 31)) << 4);
                        asm volatile("" : "+v"(off));
                        *reinterpret_cast<float4 *>(sbuf + off) =
                            make_float4(c4[4 * q], c4[4 * q + 1], c4[4 * q + 2], c4[4 * q + 3]);
                    }
            }
            compiler_fence();
            __builtin_amdgcn_s_waitcnt(0xC07F);
            __builtin_amdgcn_s_barrier();
            compiler_fence();
            const int cb = (n0 >> 7) + h;  // the partial's 128-column block
#pragma unroll
            for (int it = 0; it < 4; ++it) {
                if (32 * it >= nrows) break;  // block-uniform
                const int row = 32 * it + er, r2 = row & 63;
                const unsigned char *gb = (row < 64 ? st0 : st1) + r2 * 512;
                const int ch = ec >> 2;
                const float4 g0 = *reinterpret_cast<const float4 *>(gb + ((ch ^ (r2 & 31)) << 4));
                const float4 g1 =
                    *reinterpret_cast<const float4 *>(gb + (((ch + 1) ^ (r2 & 31)) << 4));
                const float gv[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
                const uint32_t av2[4] = {pa[h][it].x, pa[h][it].y, pa[h][it].z, pa[h][it].w};
                const uint32_t uv2[4] = {pu[h][it].x, pu[h][it].y, pu[h][it].z, pu[h][it].w};
                const float w = ew[it];
                uint32_t da2[4], du2[4], hw2[4];
                float dot = 0.f;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    float da[2], du[2], hw[2];
#pragma unroll
                    for (int i = 0; i < 2; ++i) {
                        const float av = i ? bf16_hi(av2[e]) : bf16_lo(av2[e]);
                        const float uv = i ? bf16_hi(uv2[e]) : bf16_lo(uv2[e]);
                        const float g = gv[2 * e + i];
                        const float sg = __builtin_amdgcn_rcpf(1.0f + __expf(-av));
                        const float silu = av * sg;
                        const float hv = silu * uv;
                        dot = fmaf(g, hv, dot);
                        const float dh = w * g;
                        da[i] = dh * uv * (sg * fmaf(av, 1.0f - sg, 1.0f));
                        du[i] = dh * silu;
                        hw[i] = w * hv;
                    }
                    da2[e] = pack_bf16x2(da[0], da[1]);
                    du2[e] = pack_bf16x2(du[0], du[1]);
                    hw2[e] = pack_bf16x2(hw[0], hw[1]);
                }
#pragma unroll
                for (int o = 8; o >= 1; o >>= 1) dot += __shfl_xor(dot, o, kWave);
                if (row < nrows) {
                    const int64_t gr = row0 + row;
                    const int col = n0 + 128 * h + ec;
                    uint16_t *d0 = dgu + gr * 2 * Fg + col;
                    __builtin_nontemporal_store(u32x4_t{da2[0], da2[1], da2[2], da2[3]},
                                                reinterpret_cast<u32x4_t *>(d0));
                    __builtin_nontemporal_store(u32x4_t{du2[0], du2[1], du2[2], du2[3]},
                                                reinterpret_cast<u32x4_t *>(d0 + Fg));
                    __builtin_nontemporal_store(u32x4_t{hw2[0], hw2[1], hw2[2], hw2[3]},
                                                reinterpret_cast<u32x4_t *>(hhp + gr * Fg + col));
                    if ((tid & 15) == 0) {
                        if (!shared) a.dwp[(int64_t)epair[it] * a.np + cb] = dot;
                        else a.ds[gr * a.np + cb] = dot;
                    }
                }
            }
            compiler_fence();
            __builtin_amdgcn_s_waitcnt(0xC07F);
            __builtin_amdgcn_s_barrier();
            compiler_fence();
        }
        return;
    }
}

// dOut rounded to bf16 (nearest even, as the generic kernel rounds it when
// staging), n a multiple of 8.
__global__ __launch_bounds__(256) void round_bf16_kernel(const float *__restrict__ src,
                                                         uint16_t *__restrict__ dst, int64_t n) {
    const int64_t i = 8 * ((int64_t)blockIdx.x * 256 + threadIdx.x);
    if (i >= n) return;
    const float4 lo = *reinterpret_cast<const float4 *>(src + i);
    const float4 hi = *reinterpret_cast<const float4 *>(src + i + 4);
    uint4 v;
    v.x = pack_bf16x2(lo.x, lo.y);
    v.y = pack_bf16x2(lo.z, lo.w);
    v.z = pack_bf16x2(hi.x, hi.y);
    v.w = pack_bf16x2(hi.z, hi.w);
    *reinterpret_cast<uint4 *>(dst + i) = v;
}

// Weight gradients of the shared expert, whose reduction runs over all T
// tokens: token chunk sp on 128 x 256 tiles of the output, both operands
// running along the output axis (A [K, M] and B [K, N], K = the chunk's
// token rows), binary32 partials part[sp] for the chunk-order sum that
// follows (the number of chunks is chosen per gradient shape, so that the
// tiles fill the CUs in few rounds):
//   gate/up: dW_sgu [2Fs, d] <- [da | du]_sh^T X
//   down:    dW_sdn [d, Fs]  <- dOut^T (s H)_sh, dOut rounded to bf16 first
struct WshArgs {
    const uint16_t *a, *b;  // [T, M], [T, N]
    float *part;            // [S, M, N]
    int64_t T;
    int M, N, chunk, S;
};

__global__ __launch_bounds__(512, 1) void bwd_wsh_dma_kernel(WshArgs a) {
    using G = Geo<128, 64>;
    __shared__ __align__(1024) unsigned char st0[G::STB];
    __shared__ __align__(1024) unsigned char st1[G::STB];
    __shared__ __align__(1024) unsigned char st2[G::STB];
    const int mtn = a.M / 128, ntn = (a.N + BN - 1) / BN;
    int b = blockIdx.x;
    const int nt = b % ntn;
    b /= ntn;
    const int mt = b % mtn, sp = b / mtn;
    if (sp >= a.S) return;
    const int64_t rb = (int64_t)sp * a.chunk;
    const int64_t re = min<int64_t>(rb + a.chunk, a.T);
    if (re <= rb) return;
    const int K = (int)(re - rb);  // a multiple of 64
    const int m0 = 128 * mt, n0 = BN * nt;

    const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
    McOps o;
    o.abase = a.a + rb * a.M;
    o.wbase = a.b + rb * a.N;
    o.lda = (uint32_t)a.M;
    o.ldb = (uint32_t)a.N;
#pragma unroll
    for (int j = 0; j < G::AL; ++j) {
        // K row kr of the stage (16 lanes per 256-byte row), physical chunk p:
        // logical chunk p ^ swizzle
        const int kr = 4 * (G::AL * wave + j) + (lane >> 4);
        o.aoff[j] = (uint32_t)kr * (uint32_t)a.M + (uint32_t)(m0 + 8 * ((lane & 15) ^ mc_swz(kr)));
    }
#pragma unroll
    for (int j = 0; j < G::BL; ++j) {
        const int kr = 2 * (G::BL * wave + j) + (lane >> 5);
        const int col = min(n0 + 8 * ((lane & 31) ^ mc_swz(kr)), a.N - 8);
        o.boff[j] = (uint32_t)kr * (uint32_t)a.N + (uint32_t)col;
    }
    const int wm = wave >> 1, wn = wave & 1, fr = lane & 31;
    int brow[NB];
#pragma unroll
    for (int ni = 0; ni < NB; ++ni) brow[ni] = 128 * wn + 32 * ni;
    f32x16 acc[1][NB];
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[0][j][v] = 0.f;
    Stages<3> st;
    st.s[0] = st0;
    st.s[1] = st1;
    st.s[2] = st2;
    k_loop_mc<1, true>(st, o, K / 64, wave, wm, brow, fr, lane, acc);
    // lane holds output row m0 + 32 wm + lane % 32 and, in acc[0][ni][4 q + i],
    // column n0 + brow[ni] + 8 q + 4 (lane / 32) + i
    float *crow = a.part + ((int64_t)sp * a.M + m0 + 32 * wm + fr) * a.N + n0 + 4 * (lane >> 5);
#pragma unroll
    for (int ni = 0; ni < NB; ++ni)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            if (n0 + brow[ni] + 8 * q >= a.N) continue;
            const f32x16 &c4 = acc[0][ni];
            *reinterpret_cast<float4 *>(crow + brow[ni] + 8 * q) =
                make_float4(c4[4 * q], c4[4 * q + 1], c4[4 * q + 2], c4[4 * q + 3]);
        }
}

bool bwd_wsh_dma_ok(const BwdArgs &a) {
    // chunks of whole 64-row K steps; dOut in bf16 is G's copy
    return bwd_dma_ok(a) && a.sh_split > 0 && a.Fs > 0 && a.T % 64 == 0 && a.sh_chunk % 64 == 0;
}

// Token chunks for an M x N gradient on 128 x 256 tiles: of the splits into
// at most smax chunks of whole 64-row k-steps, the one with the fewest k-step
// rounds per CU (rounds of ncu tiles times steps per chunk), fewer chunks on
// ties (less binary32 partial traffic).
static int wsh_split(int64_t T, int M, int N, int smax, int ncu, int &chunk) {
    const int64_t base = (int64_t)(M / 128) * ((N + BN - 1) / BN);
    int best = 1;
    int64_t best_cost = INT64_MAX;
    chunk = (int)T;
    for (int sp = 1; sp <= smax; ++sp) {
        const int64_t c = (T + sp - 1) / sp;
        const int64_t ch = (c + 63) / 64 * 64;
        const int eff = (int)((T + ch - 1) / ch);  // every chunk holds rows
        const int64_t cost = (eff * base + ncu - 1) / ncu * (ch / 64);
        if (cost < best_cost || (cost == best_cost && eff < best)) {
            best_cost = cost;
            best = eff;
            chunk = (int)ch;
        }
    }
    return best;
}

hipError_t launch_bwd_wsh_dma(const BwdArgs &b, bool down, hipStream_t s, int *split) {
    WshArgs a;
    a.part = b.part;
    a.T = b.T;
    if (!down) {
        a.a = static_cast<const uint16_t *>(b.dgu_sh);
        a.b = static_cast<const uint16_t *>(b.x);
        a.M = 2 * b.Fs;
        a.N = b.d;
    } else {
        a.a = static_cast<const uint16_t *>(b.dob);
        a.b = static_cast<const uint16_t *>(b.hh_sh);
        a.M = b.d;
        a.N = b.Fs;
    }
    int dev = 0, ncu = 256;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || ncu <= 0)
        ncu = 256;
    a.S = wsh_split(b.T, a.M, a.N, b.sh_split, ncu, a.chunk);
    *split = a.S;
    const unsigned blocks = (unsigned)(a.S * (a.M / 128) * ((a.N + BN - 1) / BN));
    hipLaunchKernelGGL(bwd_wsh_dma_kernel, dim3(blocks), dim3(512), 0, s, a);
    return hipGetLastError();
}

// Down-projection weight gradients of the routed experts with at most 128
// rows (the usual case: T k / E rows on average), as a stream of output
// tiles: over the expert's K <= 128 rows,
//   dW_dn[e] [d, F] = Q^T P,  P = H_e,  Q = dOut_e
// (H_e: the rows' w h, the combine weight folded in by the SwiGLU backward;
// dOut_e: the rows' tokens through the permutation, dOut rounded to bf16
// once beforehand).  Output rows run along Q's columns (d), output columns
// along P's (F).
// Block (expert g, 128-column slice of P) loads that slice of P for the K
// rows once, keeps its MFMA fragments in registers, and walks 64-column
// tiles of Q through three direct-to-LDS buffers (two tiles in flight while
// one computes).  Only the k16 steps that hold rows are loaded and computed
// (rows past K inside the last step repeat row K - 1 and meet zeros in P).
// A finished 128 x 64 tile goes out through an LDS staging buffer as 64
// whole 256-byte row pieces, nontemporal (no later kernel of the call reads
// the gradient).  Two barriers per tile: one when the tile's buffer has
// landed (which also frees the staging buffer), one when the staging is
// complete (which also frees the tile's buffer for the load three tiles
// ahead).  4 waves in 2 x 2, each 64 columns of P by 32 of Q; 80 KB of LDS,
// so two blocks share a CU and one's loads, barriers and stores overlap the
// other's MFMAs.
struct DwArgs {
    const uint16_t *p;      // w H [T k, F]: row k of the expert is permuted row offsets[g] + k
    const uint16_t *q;      // dOut bf16 [T, d]: row k of the expert is its token's row
    uint16_t *out;          // dW_dn [E, d, F]
    const int32_t *perm, *counts, *offsets;
    int64_t estride;
    int E, k, ldp, ldq, ldo;
    int RT, CT;             // 128-column slices of P, 64-column tiles of Q
};

namespace {
constexpr int DW_QROWB = 128;             // one staged Q row: 64 bf16
constexpr int DW_QBUF = 128 * DW_QROWB;   // 128 K rows: 16 KB
constexpr int DW_STG = 128 * 256;         // P's K rows of 128 bf16, then 64 output rows

// Q rows of 128 bytes, 16-byte chunk c of row k at c ^ 4 ((k >> 1) & 1): a
// transposing read touches two chunks of each of four consecutive rows, and
// the two 16-lane groups that share a pass then cover all 64 banks.
__device__ __forceinline__ int q_swz(int k) { return 4 * ((k >> 1) & 1); }

// Fragment of Q columns nb .. nb + 31 at k16 step ks (as mc_tfrag, for
// 128-byte rows; k and k + 4 share the swizzle).
__device__ __forceinline__ bf16x8 q_frag(const unsigned char *qb, int ks, int nb, int lane) {
    const int g = lane >> 4, s = lane & 15;
    const int k = 16 * ks + 8 * (g >> 1) + (s >> 2);
    const int m = nb + 16 * (g & 1) + 4 * (s & 3);
    const int off = (((m >> 3) ^ q_swz(k)) << 4) + (m & 7) * 2;
    const unsigned char *p = qb + k * DW_QROWB + off;
    const v4i16_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t *)p);
    const v4i16_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t *)(p + 4 * DW_QROWB));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Staging of a finished tile: output row R (of 64), 16-byte chunk c at
// chunk c ^ (R & 15), so the 32 rows one accumulator write touches fall on
// distinct banks (two passes of 256 bytes) and a row read by 16 lanes too.
__device__ __forceinline__ int stg_off(int R, int c) { return R * 256 + ((c ^ (R & 15)) << 4); }

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// Output piece c (16 bytes) of staged row R of tile t: row 64 t + R,
// columns r0 + 8 c ..
__device__ __forceinline__ u32x4_t *dw_dst(const DwArgs &a, uint16_t *out, int t, int r0, int R,
                                           int c) {
    return reinterpret_cast<u32x4_t *>(out + (int64_t)(64 * t + R) * a.ldo + r0 + 8 * c);
}

// MFMAs of one tile over N k16 steps: this wave's Q fragments, then 2 N
// products with the P fragments held in registers (the accumulator's runs
// of four go along P's columns, i.e. along the output rows).
template <int N>
__device__ __forceinline__ void dw_tile_mfma(const unsigned char *qb, const bf16x8 (&pf)[8][2],
                                             int wc, int lane, f32x16 (&acc)[2]) {
    bf16x8 qf[N];
#pragma unroll
    for (int ks = 0; ks < N; ++ks) qf[ks] = q_frag(qb, ks, 32 * wc, lane);
#pragma unroll
    for (int ks = 0; ks < N; ++ks)
#pragma unroll
        for (int mi = 0; mi < 2; ++mi)
            acc[mi] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pf[ks][mi], qf[ks], acc[mi], 0, 0, 0);
}

__device__ __forceinline__ void dw_mfma(int nks, const unsigned char *qb, const bf16x8 (&pf)[8][2],
                                        int wc, int lane, f32x16 (&acc)[2]) {
    switch (nks) {
    case 1: dw_tile_mfma<1>(qb, pf, wc, lane, acc); break;
    case 2: dw_tile_mfma<2>(qb, pf, wc, lane, acc); break;
    case 3: dw_tile_mfma<3>(qb, pf, wc, lane, acc); break;
    case 4: dw_tile_mfma<4>(qb, pf, wc, lane, acc); break;
    case 5: dw_tile_mfma<5>(qb, pf, wc, lane, acc); break;
    case 6: dw_tile_mfma<6>(qb, pf, wc, lane, acc); break;
    case 7: dw_tile_mfma<7>(qb, pf, wc, lane, acc); break;
    case 8: dw_tile_mfma<8>(qb, pf, wc, lane, acc); break;
    default: break;
    }
}

// Q tile t (columns 64 t ..) into buffer qb: this wave's 32 K rows, four
// loads of eight 128-byte rows (qrow: this lane's row and swizzled chunk).
__device__ __forceinline__ void dw_load_q(unsigned char *qb, const uint16_t *const (&qrow)[4], int t,
                                          int wave) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
        __builtin_amdgcn_global_load_lds((const global_void_t *)(qrow[j] + 64 * t),
                                         (lds_void_t *)(qb + (4 * wave + j) * 1024), 16, 0, 0);
}

// One tile on constant buffer qb: wait until this wave's loads of it have
// landed (16 vector-memory operations follow them: two tiles' stores and
// loads) and the other waves' too (barrier), compute, stage, store, and load
// tile t + 3 into the same buffer (past the last tile the loads re-read
// tile CT - 1 into a buffer that is never computed).
__device__ __forceinline__ void dw_tile(const DwArgs &a, unsigned char *qb, unsigned char *stg,
                                        const uint16_t *const (&qrow)[4], bool dma,
                                        const bf16x8 (&pf)[8][2], int nks, int t, uint16_t *out,
                                        int r0, int wave, int wr, int wc, int lane, int tid) {
    compiler_fence();
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(16));
    __builtin_amdgcn_s_barrier();
    compiler_fence();
    f32x16 acc[2];
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[mi][v] = 0.f;
    dw_mfma(nks, qb, pf, wc, lane, acc);
    // accumulator layout: lane holds Q column 32 wc + lane % 32 (the output
    // row) and, in acc[mi][4 gq + i], P columns 64 wr + 32 mi + 8 gq +
    // 4 (lane / 32) + i (runs of four along the output row)
    const int fr = lane & 31, h = lane >> 5;
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
            const int R = 32 * wc + fr;
            const int C = 64 * wr + 32 * mi + 8 * gq + 4 * h;
            const f32x16 &c = acc[mi];
            // an offset the compiler cannot relate to the others: paired
            // LDS writes merged into one ds_write2 lose the buffer's alias
            // scope, and the compiler then waits for every load in flight
            int off = stg_off(R, C >> 3) + (C & 7) * 2;
            asm volatile("" : "+v"(off));
            *reinterpret_cast<uint2 *>(stg + off) =
                make_uint2(pack_bf16x2(c[4 * gq], c[4 * gq + 1]), pack_bf16x2(c[4 * gq + 2], c[4 * gq + 3]));
        }
    compiler_fence();
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's staging writes are done
    __builtin_amdgcn_s_barrier();
    compiler_fence();
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) {
        const int pc = tid + 256 * qq, R = pc >> 4, c = pc & 15;
        const u32x4_t v = *reinterpret_cast<const u32x4_t *>(stg + stg_off(R, c));
        __builtin_nontemporal_store(v, dw_dst(a, out, t, r0, R, c));
    }
    if (dma) dw_load_q(qb, qrow, min(t + 3, a.CT - 1), wave);
    __builtin_amdgcn_sched_barrier(0);
}
}  // namespace

__global__ __launch_bounds__(256, 2) void bwd_dwdn_stream_kernel(DwArgs a) {
    __shared__ __align__(1024) unsigned char qb0[DW_QBUF];
    __shared__ __align__(1024) unsigned char qb1[DW_QBUF];
    __shared__ __align__(1024) unsigned char qb2[DW_QBUF];
    __shared__ __align__(1024) unsigned char stg[DW_STG];
    // expert g on XCD g % 8 with its RT blocks consecutive (they share the
    // expert's Q rows through that XCD's L2)
    const int b = blockIdx.x, q8 = b >> 3;
    const int g = 8 * (q8 / a.RT) + (b & 7), rt = q8 % a.RT;
    if (g >= a.E) return;
    const int K = a.counts[g];
    if (K > 128) return;  // the tiled kernel's
    const int rb = a.offsets[g], nks = (K + 15) >> 4;
    const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
    const int wr = wave >> 1, wc = wave & 1;
    const int r0 = 128 * rt;
    uint16_t *out = a.out + (int64_t)g * a.estride;
    if (K == 0) {  // no rows: the gradient is zero
        const u32x4_t z = {0u, 0u, 0u, 0u};
        for (int t = 0; t < a.CT; ++t)
#pragma unroll
            for (int qq = 0; qq < 4; ++qq) {
                const int pc = tid + 256 * qq;
                __builtin_nontemporal_store(z, dw_dst(a, out, t, r0, pc >> 4, pc & 15));
            }
        return;
    }
    // this wave loads K rows 32 wave .. + 31: P in eight loads of four
    // 256-byte rows, Q in four loads of eight 128-byte rows per tile (lane:
    // its row, physical chunk <- logical chunk ^ swizzle); rows past K
    // repeat row K - 1
    const bool dma = 2 * wave < nks;
    // the permutation lookups of Q's tokens
    int qt[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) qt[j] = a.perm[rb + max(min(32 * wave + 8 * j + (lane >> 3), K - 1), 0)];
    // used here, so the compiler issues all four lookups before the first
    // wait (it would otherwise wait for them one at a time)
#pragma unroll
    for (int j = 0; j < 4; ++j) asm volatile("" ::"v"(qt[j]));
    const uint16_t *qrow[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int kr = 32 * wave + 8 * j + (lane >> 3);
        const int src = qt[j] / a.k;
        qrow[j] = a.q + (int64_t)src * a.ldq + 8 * ((lane & 7) ^ q_swz(kr));
    }
    const uint16_t *prow[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int kr = 32 * wave + 4 * j + (lane >> 4);
        const int row = rb + max(min(kr, K - 1), 0);
        prow[j] = a.p + (int64_t)row * a.ldp + r0 + 8 * ((lane & 15) ^ mc_swz(kr));
    }
    // every lookup has landed before the first load goes out (a wait for a
    // lookup issued after a load would wait for the load too)
    compiler_fence();
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    compiler_fence();
    // P into the staging buffer (free until the P fragments are in
    // registers) and the first three tiles; these loads go out on every wave
    // (rows past the expert's included) so that the compiler sees them on
    // every path
#pragma unroll
    for (int j = 0; j < 8; ++j)
        __builtin_amdgcn_global_load_lds((const global_void_t *)prow[j],
                                         (lds_void_t *)(stg + (8 * wave + j) * 1024), 16, 0, 0);
    dw_load_q(qb0, qrow, 0, wave);
    dw_load_q(qb1, qrow, min(1, a.CT - 1), wave);
    dw_load_q(qb2, qrow, min(2, a.CT - 1), wave);
    // P and the first three tiles are in LDS.  A full drain:
    // with loads in flight at the tile loop's entry the compiler can no
    // longer tell the buffers apart and waits for every load before each LDS
    // read in the loop.
    __syncthreads();
    // P fragments (P column 64 wr + 32 mi + lane % 32, K rows 16 ks + 8 (lane
    // / 32) .. + 7), zero past K
    bf16x8 pf[8][2];
    const int h = lane >> 5;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
#pragma unroll
        for (int mi = 0; mi < 2; ++mi) {
            bf16x8 v = {};
            if (ks < nks) {
                v = mc_tfrag<256>(stg, ks, 64 * wr + 32 * mi, lane);
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    if (16 * ks + 8 * h + e >= K) v[e] = (__bf16)0.f;
            }
            pf[ks][mi] = v;
        }
    // every wave's P reads are done before the first tile's staging writes
    // (the first tile's barrier follows this wait)
    compiler_fence();
    __builtin_amdgcn_s_waitcnt(0xC07F);
    compiler_fence();
    for (int t = 0; t < a.CT; t += 3) {
        dw_tile(a, qb0, stg, qrow, dma, pf, nks, t, out, r0, wave, wr, wc, lane, tid);
        if (t + 1 < a.CT) dw_tile(a, qb1, stg, qrow, dma, pf, nks, t + 1, out, r0, wave, wr, wc, lane, tid);
        if (t + 2 < a.CT) dw_tile(a, qb2, stg, qrow, dma, pf, nks, t + 2, out, r0, wave, wr, wc, lane, tid);
    }
    compiler_fence();
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));  // no load may land after the block ends
}

bool bwd_dwdn_stream_ok(const BwdArgs &a) {
    // the shared expert is left to the tiled kernels (split over token
    // chunks); dOut in bf16 is G's copy (the same condition)
    return bwd_dma_ok(a) && (a.Fs == 0 || a.sh_split > 0);
}

hipError_t launch_bwd_dwdn_stream(const BwdArgs &b, hipStream_t s) {
    // dOut rounded to bf16 again (the same bits G's copy holds): written
    // just before, the rows that the tiles gather stay in the caches
    // (T = 4096: reading G's copy from 1.5 ms earlier made the stage 30 us
    // slower than rounding again)
    const int64_t n = b.T * b.d;
    hipLaunchKernelGGL(round_bf16_kernel, dim3((unsigned)((n / 8 + 255) / 256)), dim3(256), 0, s,
                       b.dout, static_cast<uint16_t *>(b.dob), n);
    DwArgs a;
    a.p = static_cast<const uint16_t *>(b.hh);
    a.q = static_cast<const uint16_t *>(b.dob);
    a.out = static_cast<uint16_t *>(b.dw_dn);
    a.perm = b.perm;
    a.counts = b.counts;
    a.offsets = b.offsets;
    a.estride = (int64_t)b.d * b.F;
    a.E = b.E;
    a.k = b.k;
    a.ldp = b.F;
    a.ldq = b.d;
    a.ldo = b.F;
    a.RT = b.F / 128;
    a.CT = b.d / 64;
    const unsigned blocks = 8u * (unsigned)((b.E + 7) / 8) * (unsigned)a.RT;
    hipLaunchKernelGGL(bwd_dwdn_stream_kernel, dim3(blocks), dim3(256), 0, s, a);
    return hipGetLastError();
}

// dW_router (and the shared gate's gradient) on the same tiles: dL^T X with
// dL [T, ldd] (the router-logit gradient, zero padded to ldd, a multiple of
// 128) and X [T, d], token chunks with binary32 partials [S, ldd, d] in part
// (free by then: its last reader ran), summed in chunk order afterwards.
bool bwd_dwr_dma_ok(const BwdArgs &a) {
    return bwd_dma_ok(a) && a.T % 64 == 0 && a.ldd % 128 == 0 && a.sh_split > 0 && a.Fs > 0 &&
           (int64_t)a.sh_split * 2 * a.Fs >= 2 * (int64_t)a.ldd;
}

hipError_t launch_bwd_dwr_dma(const BwdArgs &b, hipStream_t s, int *split) {
    WshArgs a;
    a.a = static_cast<const uint16_t *>(b.dl);
    a.b = static_cast<const uint16_t *>(b.x);
    a.part = b.part;
    a.T = b.T;
    a.M = b.ldd;
    a.N = b.d;
    int dev = 0, ncu = 256;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || ncu <= 0)
        ncu = 256;
    const int smax = (int)std::min<int64_t>(16, (int64_t)b.sh_split * 2 * b.Fs / b.ldd);
    a.S = wsh_split(b.T, a.M, a.N, smax, ncu, a.chunk);
    *split = a.S;
    const unsigned blocks = (unsigned)(a.S * (a.M / 128) * ((a.N + BN - 1) / BN));
    hipLaunchKernelGGL(bwd_wsh_dma_kernel, dim3(blocks), dim3(512), 0, s, a);
    return hipGetLastError();
}

bool bwd_dma_ok(const BwdArgs &a) {
    if (!a.bf16 || a.F % 128 || a.Fs % 128 || a.d % 128 || a.logit_split > 2) return false;
    const int64_t rows = a.T * a.k;
    const int64_t wide = 2 * (int64_t)(a.F > a.Fs ? a.F : a.Fs);
    return rows * wide < ((int64_t)1 << 32) && wide * a.d < ((int64_t)1 << 32) &&
           a.T * a.d < ((int64_t)1 << 32);
}

static BwdTileArgs bwd_tile_args(const BwdArgs &b, int max_tiles) {
    BwdTileArgs a;
    a.perm = b.perm;
    a.counts = b.counts;
    a.offsets = b.offsets;
    a.tile_start = b.tile_start;
    a.tile_group = b.tile_group;
    a.T = b.T;
    a.d = b.d;
    a.E = b.E;
    a.k = b.k;
    a.F = b.F;
    a.Fs = b.Fs;
    a.nm = max_tiles;
    a.gm = -1;  // M-tile m on XCD m % 8 (its N-tiles share A through one L2)
    return a;
}

hipError_t launch_bwd_dx_dma(const BwdArgs &b, int max_tiles, hipStream_t s) {
    BwdTileArgs a = bwd_tile_args(b, max_tiles);
    a.a = static_cast<const uint16_t *>(b.dgu);
    a.a_sh = static_cast<const uint16_t *>(b.dgu_sh);
    a.w = static_cast<const uint16_t *>(b.w_gu);
    a.w_sh = static_cast<const uint16_t *>(b.w_sgu);
    a.c = b.dxp;
    a.c_sh = b.dxs;
    a.nn = (b.d + BN - 1) / BN;
    hipLaunchKernelGGL(bwd_mc_dma_kernel<BWD_DX>, dim3(raster_blocks(a.nm, a.nn, a.gm)), dim3(512), 0,
                       s, a);
    return hipGetLastError();
}

hipError_t launch_bwd_g_dma(const BwdArgs &b, int max_tiles, void *dout_bf16, hipStream_t s) {
    const int64_t n = b.T * b.d;  // d % 128 == 0
    hipLaunchKernelGGL(round_bf16_kernel, dim3((unsigned)((n / 8 + 255) / 256)), dim3(256), 0, s,
                       b.dout, static_cast<uint16_t *>(dout_bf16), n);
    BwdTileArgs a = bwd_tile_args(b, max_tiles);
    a.a = static_cast<const uint16_t *>(dout_bf16);
    a.a_sh = a.a;
    a.w = static_cast<const uint16_t *>(b.w_dn);
    a.w_sh = static_cast<const uint16_t *>(b.w_sdn);
    a.c = nullptr;
    a.c_sh = nullptr;
    a.au = static_cast<const uint16_t *>(b.au);
    a.au_sh = static_cast<const uint16_t *>(b.au_sh);
    a.dgu = static_cast<uint16_t *>(b.dgu);
    a.dgu_sh = static_cast<uint16_t *>(b.dgu_sh);
    a.hh = static_cast<uint16_t *>(b.hh);
    a.hh_sh = static_cast<uint16_t *>(b.hh_sh);
    a.topk_w = b.topk_w;
    a.logits = b.logits;
    a.gate = b.gate;
    a.dwp = b.dwp;
    a.ds = b.ds;
    a.ldl = b.ldl;
    a.logit_split = b.logit_split;
    a.np = b.gtile;  // cdiv(max(F, Fs), 128)
    const int fmax = b.F > b.Fs ? b.F : b.Fs;
    a.nn = (fmax + BN - 1) / BN;
    hipLaunchKernelGGL(bwd_mc_dma_kernel<BWD_G>, dim3(raster_blocks(a.nm, a.nn, a.gm)), dim3(512), 0,
                       s, a);
    return hipGetLastError();
}

hipError_t launch_experts_dma(const Problem &p, int bm, hipStream_t s,
                              const std::function<void(int)> &mark) {
    GemmArgs a;
    memset(&a, 0, sizeof a);
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
    a.nn = (fmax + BN / 2 - 1) / (BN / 2);
    a.gm = -1;  // M-tile m on XCD m % 8: its N-tiles share A through one L2
    // The K pipeline runs across tiles on persistent blocks wherever every
    // tile has the same number of K steps, at least the stage count: both
    // GEMMs on 128-row tiles (T = 4096: gate/up 0.683 -> 0.674 ms, down
    // 0.456 -> 0.442 ms), and the down projection on 256-row tiles with a
    // multiple of four steps (its 20-step tiles at F = 640 lose a larger
    // share to each tile's start and end than gate/up's 80-step tiles, which
    // measured faster on the dispatcher's dynamic order)
    const int d_steps128 = p.d / 64;
    const bool xt_dn128 = (p.Fs == 0 || p.Fs == p.F) && p.F / 64 >= 3;
    const bool xt_dn = bm == 256 && (p.Fs == 0 || p.Fs == p.F) && (p.F / 32) % 4 == 0 && p.F / 32 >= 4;
    int dev = 0, ncu = 256;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || ncu < 8)
        ncu = 256;
    auto xgrid = [ncu](const GemmArgs &g) {
        const unsigned n = raster_blocks(g.nm, g.nn, g.gm), cap = 8u * (unsigned)(ncu / 8);
        return dim3(n < cap ? n : cap);
    };
    if (bm == 256) hipLaunchKernelGGL((gemm_dma_kernel<0, 256, 32, 3>), grid(a), dim3(512), 0, s, a);
    else if (d_steps128 >= 3) hipLaunchKernelGGL((gemm_dma_xt_kernel<0, 128, 64, 3>), xgrid(a), dim3(512), 0, s, a);
    else hipLaunchKernelGGL((gemm_dma_kernel<0, 128, 64, 3>), grid(a), dim3(64 * Geo<128, 64>::NW), 0, s, a);
    mark(3);
    a.w = static_cast<const uint16_t *>(p.w_down);
    a.w_sh = static_cast<const uint16_t *>(p.w_sh_down);
    a.nn = (p.d + BN - 1) / BN;
    if (xt_dn) hipLaunchKernelGGL((gemm_dma_xt_kernel<1, 256, 32, 4>), xgrid(a), dim3(512), 0, s, a);
    else if (bm == 256) hipLaunchKernelGGL((gemm_dma_kernel<1, 256, 32, 3>), grid(a), dim3(512), 0, s, a);
    else if (xt_dn128) hipLaunchKernelGGL((gemm_dma_xt_kernel<1, 128, 64, 3>), xgrid(a), dim3(512), 0, s, a);
    else hipLaunchKernelGGL((gemm_dma_kernel<1, 128, 64, 3>), grid(a), dim3(64 * Geo<128, 64>::NW), 0, s, a);
    mark(4);
    return hipGetLastError();
}

}  // namespace moe
