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
                // routed rows: weighted, bf16, into y
                uint16_t *yrow = a.y + (int64_t)(row0 + row) * a.d + n0 + cq;
#pragma unroll
                for (int ni = 0; ni < NB; ++ni)
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        const int col = n0 + brow[ni] + 8 * g + cq;
                        if (col >= a.d) continue;
                        const f32x16 &c = acc[mi][ni];
                        uint2 q;
                        q.x = pack_bf16x2(wgt * c[4 * g], wgt * c[4 * g + 1]);
                        q.y = pack_bf16x2(wgt * c[4 * g + 2], wgt * c[4 * g + 3]);
                        *reinterpret_cast<uint2 *>(yrow + brow[ni] + 8 * g) = q;
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
    a.y = static_cast<uint16_t *>(p.y);
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
    if (bm == 256) hipLaunchKernelGGL((gemm_dma_kernel<0, 256, 32, 3>), grid(a), dim3(512), 0, s, a);
    else hipLaunchKernelGGL((gemm_dma_kernel<0, 128, 64, 3>), grid(a), dim3(64 * Geo<128, 64>::NW), 0, s, a);
    mark(3);
    a.w = static_cast<const uint16_t *>(p.w_down);
    a.w_sh = static_cast<const uint16_t *>(p.w_sh_down);
    a.nn = (p.d + BN - 1) / BN;
    if (bm == 256) hipLaunchKernelGGL((gemm_dma_kernel<1, 256, 32, 3>), grid(a), dim3(512), 0, s, a);
    else hipLaunchKernelGGL((gemm_dma_kernel<1, 128, 64, 3>), grid(a), dim3(64 * Geo<128, 64>::NW), 0, s, a);
    mark(4);
    return hipGetLastError();
}

}  // namespace moe
