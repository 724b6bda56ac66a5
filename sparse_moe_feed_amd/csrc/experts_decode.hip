// experts_decode.hip -- grouped SwiGLU experts when each expert sees only a
// few tokens (decode): weight streaming from HBM.
//
// Same maths as experts_bf16.hip (gated MLP with SiLU per expert, weighted
// rows y, shared expert scaled by its sigmoid gate; anatomy page on
// frontier-model-atlas, "Decoder microscope", Feed-forward panel and "Expert
// fan-out").  With about one token per touched expert, the work is reading
// every touched expert's 3 x F x d weights once; the arithmetic is a few
// MFMAs per 16-byte load.
//
// Tiles hold up to 32 rows of one group (two 16-row halves of
// v_mfma_f32_16x16x32_bf16): consecutive permuted rows, or, at T <= 32 with
// the exact router, the expert's pairs found in topk_idx.  Each wave owns NB blocks of 16 output columns
// and walks K with weights loaded straight from HBM into registers: 4 MFMA
// K-steps (128 elements, 256 contiguous bytes per weight row) per group, two
// groups in flight (ping-pong).  A fragments (token rows) come from L2.  No
// LDS staging of weights: every weight byte is used by exactly one wave.
#include "moe_device.h"
#include "moe_kernels.h"

#include <algorithm>

namespace moe {

constexpr int DBM = kDecodeBM;  // rows per decode tile
constexpr int KG = 128;         // K elements per pipeline group (4 MFMA steps)
constexpr int DW = 1;           // waves per block (finer blocks, a shorter tail: 4 / 2 / 1 waves
                                // gave gate/up 286 / 279 / 277 us at T = 32, d = 2560, top-10 of 512)
constexpr int DNB = 2;          // 16-column blocks per wave in the down projection (1 / 2 / 4:
                                // 152 / 145 / 153 us at T = 32, d = 2560, 512 experts top-10)

struct DecodeArgs {
    const uint16_t *x;
    const uint16_t *w;     // gate/up: [E, 2F, d]   down: [E, d, F]
    const uint16_t *w_sh;  // gate/up: [2Fs, d]     down: [d, Fs]
    uint16_t *h;           // [T*k, F]
    uint16_t *h_sh;        // [T, Fs]
    uint16_t *au, *au_sh;  // pre-activations [a | u] (training forward), or null
    float *out;
    float *y;              // [T*k, d] weighted routed rows (binary32)
    const int32_t *perm, *counts, *offsets, *tile_start, *tile_group;
    const int32_t *topk_idx;
    const float *topk_w, *gate;
    int64_t T;
    int d, E, k, F, Fs;
    int direct;            // tiles without the permutation step (decode_tile)
};

struct Frag {
    uint4 v[4];  // one 16-byte slice for each of the 4 MFMA steps of a group
};

// No per-lane conditions on loads (padding rows read a valid row): divergent
// branches around loads make the compiler's wait counts conservative and
// drain the pipeline every group.
template <int NB, int HALVES>
__device__ __forceinline__ void load_group(Frag (&b)[NB], Frag (&a)[HALVES],
                                           const uint16_t *const (&bp)[NB],
                                           const uint16_t *const (&ap)[HALVES], int g) {
    const int kb = g * KG;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
#pragma unroll
        for (int n = 0; n < NB; ++n) b[n].v[s] = *reinterpret_cast<const uint4 *>(bp[n] + kb + 32 * s);
#pragma unroll
        for (int h = 0; h < HALVES; ++h) a[h].v[s] = *reinterpret_cast<const uint4 *>(ap[h] + kb + 32 * s);
    }
}

template <int NB>
__device__ __forceinline__ void load_b(Frag (&b)[NB], const uint16_t *const (&bp)[NB], int g) {
    const int kb = g * KG;
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int n = 0; n < NB; ++n) b[n].v[s] = *reinterpret_cast<const uint4 *>(bp[n] + kb + 32 * s);
}

template <int HALVES>
__device__ __forceinline__ void load_a(Frag (&a)[HALVES], const uint16_t *const (&ap)[HALVES], int g) {
    const int kb = g * KG;
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int h = 0; h < HALVES; ++h) a[h].v[s] = *reinterpret_cast<const uint4 *>(ap[h] + kb + 32 * s);
}

template <int NB, int HALVES>
__device__ __forceinline__ void mfma_group(f32x4 (&acc)[HALVES][NB], const Frag (&b)[NB],
                                           const Frag (&a)[HALVES]) {
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int h = 0; h < HALVES; ++h)
#pragma unroll
            for (int n = 0; n < NB; ++n)
                acc[h][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    __builtin_bit_cast(bf16x8, a[h].v[s]), __builtin_bit_cast(bf16x8, b[n].v[s]),
                    acc[h][n], 0, 0, 0);
}

// Streams K (a multiple of KG) for NB weight-row blocks and HALVES row halves.
// bp[n]: this lane's weight row plus its 8-element k offset; ap[h]: this
// lane's token row plus k offset (padding rows point at a valid row; their
// results are never stored).  Two groups of loads are kept in flight
// (ping-pong register buffers).
// stream_k_from: the same with group 0 already loaded into b0 / a0 by the
// caller (which can then issue its B loads before the A addresses are known).
template <int NB, int HALVES>
__device__ __forceinline__ void stream_k_from(Frag (&b0)[NB], Frag (&a0)[HALVES],
                                              const uint16_t *const (&bp)[NB],
                                              const uint16_t *const (&ap)[HALVES], int K,
                                              f32x4 (&acc)[HALVES][NB]) {
    Frag b1[NB], a1[HALVES];
    const int ng = K / KG;
    // The steady-state body has no branches around loads (any branch makes
    // the compiler's wait counts fall back to zero), and sched_barrier keeps
    // the phases in program order, so a group's loads are in flight while the
    // previous group's MFMAs run.  The last one or two groups are peeled.
    int g = 0;
    for (; g + 2 < ng; g += 2) {
        load_group<NB, HALVES>(b1, a1, bp, ap, g + 1);
        __builtin_amdgcn_sched_barrier(0);
        mfma_group<NB, HALVES>(acc, b0, a0);
        __builtin_amdgcn_sched_barrier(0);
        load_group<NB, HALVES>(b0, a0, bp, ap, g + 2);
        __builtin_amdgcn_sched_barrier(0);
        mfma_group<NB, HALVES>(acc, b1, a1);
        __builtin_amdgcn_sched_barrier(0);
    }
    if (g + 1 < ng) {
        load_group<NB, HALVES>(b1, a1, bp, ap, g + 1);
        __builtin_amdgcn_sched_barrier(0);
        mfma_group<NB, HALVES>(acc, b0, a0);
        __builtin_amdgcn_sched_barrier(0);
        mfma_group<NB, HALVES>(acc, b1, a1);
    } else {
        mfma_group<NB, HALVES>(acc, b0, a0);
    }
}

template <int NB, int HALVES>
__device__ __forceinline__ void stream_k(const uint16_t *const (&bp)[NB],
                                         const uint16_t *const (&ap)[HALVES], int K,
                                         f32x4 (&acc)[HALVES][NB]) {
    Frag b0[NB], a0[HALVES];
    load_group<NB, HALVES>(b0, a0, bp, ap, 0);
    stream_k_from<NB, HALVES>(b0, a0, bp, ap, K, acc);
}

// A tile's rows: rows r < nrows of group g.  With the permutation step they
// are the consecutive permuted rows row0 + r; without it (direct) routed rows
// are the pairs rows[r] (h and y indexed by pair id); shared-expert rows are
// the tokens row0 + r either way.
struct TileInfo {
    int g, row0, nrows;
    bool shared;
    const int *rows;  // direct routed tiles: this wave's LDS list of pair ids, else null
};

__device__ __forceinline__ int tile_row(const TileInfo &ti, int r) {
    return ti.rows ? ti.rows[r] : ti.row0 + r;
}

// Pair (routed) or token (shared) of row r: what the gate/up A rows and the
// down epilogue's weights are looked up by.
template <class Args>
__device__ __forceinline__ int tile_src(const Args &a, const TileInfo &ti, int r) {
    return ti.shared ? ti.row0 + r : ti.rows ? ti.rows[r] : a.perm[ti.row0 + r];
}

constexpr int kScanChunks = DBM * 32 / 64;  // 64-pair chunks of topk_idx at T <= DBM, k <= 32

// Direct tiles (T <= DBM, so an expert has at most DBM pairs when the top-k
// experts of a token are distinct): the router set bit e % 32 of word e / 32
// of a 32-word map in counts for every touched expert e (the map cleared
// before it); block 0 serves the shared expert (if any; its tile has all T
// rows, so it starts first), block sh + x the x-th touched expert in
// ascending order, later blocks end.  The map is uniform over the block and
// read by scalar loads, which do not queue behind the weight streams of the
// CU's other blocks the way a vector load does.
// decode_tile finds the group (and, with the permutation, the rows); for a
// direct routed tile the rows come from tile_rows, after the block has its
// first weight loads in flight.
constexpr int kTouchWords = 32;  // 32-expert words of the touched map, E <= 1024

// Position of the x-th (from 0) set bit of w; w has more than x set bits.
__device__ __forceinline__ int nth_set_bit(uint32_t w, int x) {
    int pos = 0;
#pragma unroll
    for (int s = 16; s >= 1; s >>= 1) {
        const int c = __popc(w & ((1u << s) - 1));
        if (x >= c) {
            x -= c;
            w >>= s;
            pos += s;
        }
    }
    return pos;
}

__device__ __forceinline__ int touched_expert(const int *__restrict__ map, int x) {
    uint32_t w[kTouchWords];
#pragma unroll
    for (int j = 0; j < kTouchWords; ++j) w[j] = (uint32_t)map[j];
#pragma unroll
    for (int j = 0; j < kTouchWords; ++j) {
        const int c = __popc(w[j]);
        if (x < c) return 32 * j + nth_set_bit(w[j], x);
        x -= c;
    }
    return -1;  // fewer than x + 1 experts touched
}

template <class Args>
__device__ __forceinline__ bool decode_tile(const Args &a, TileInfo &ti, int tile) {
    ti.rows = nullptr;
    ti.row0 = 0;
    if (a.direct) {
        const int sh = a.Fs > 0 ? 1 : 0;
        ti.shared = sh && tile == 0;
        ti.g = ti.shared ? a.E : touched_expert(a.counts, tile - sh);
        if (ti.g < 0) return false;
        ti.nrows = ti.shared ? (int)a.T : 0;  // routed: tile_rows
        return true;
    }
    if (tile >= a.tile_start[a.E + 1]) return false;
    ti.g = a.tile_group[tile];
    ti.shared = ti.g == a.E;
    const int m_local = (tile - a.tile_start[ti.g]) * DBM;
    if (!ti.shared) {
        ti.row0 = a.offsets[ti.g] + m_local;
        ti.nrows = min(DBM, a.counts[ti.g] - m_local);
    } else {
        ti.row0 = m_local;
        ti.nrows = (int)min<int64_t>(DBM, a.T - m_local);
    }
    return true;
}

// Rows of a direct routed tile: each wave scans topk_idx and lists the
// expert's pairs in ascending pair id in its own LDS slots (no block
// barrier).  Other tiles already have their rows.  False (no rows) cannot
// happen for a listed expert; the caller then drains its loads and ends.
template <class Args>
__device__ __forceinline__ bool tile_rows(const Args &a, TileInfo &ti, int *rows) {
    if (!a.direct || ti.shared) return true;
    const int lane = threadIdx.x & 63;
    const int np = (int)a.T * a.k;  // <= DBM * 32 = 64 kScanChunks
    const uint64_t below = (1ull << lane) - 1;
    // every chunk's load issued before the first compare: one round trip
    // (addresses clamped into the array, so the loads need no branch)
    int v[kScanChunks];
#pragma unroll
    for (int i = 0; i < kScanChunks; ++i) v[i] = a.topk_idx[min(64 * i + lane, np - 1)];
    int n = 0;
#pragma unroll
    for (int i = 0; i < kScanChunks; ++i) {
        const int p = 64 * i + lane;
        const bool hit = v[i] == ti.g && p < np;
        const uint64_t m = __ballot(hit);
        const int at = n + __popcll(m & below);
        if (hit && at < DBM) rows[at] = p;
        n += __popcll(m);
    }
    if (n == 0) return false;
    __builtin_amdgcn_wave_barrier();
    ti.nrows = min(n, DBM);
    ti.rows = rows;
    return true;
}

// A block whose tile has no rows ends here, after its loads in flight land.
__device__ __forceinline__ void drain_and_end() { __builtin_amdgcn_s_waitcnt(0); }

// gate/up: block = DW waves, wave w owns gate columns n0 + 16 w .. + 16 and
// the matching up columns; grid.y walks 16 DW-column slabs of the expert width.
// Each lane looks up the token of its own A rows; the first group's weight
// loads are issued before those lookups are waited for.
template <int HALVES>
__device__ void decode_gateup_body(const DecodeArgs &a, const TileInfo &ti,
                                   const uint16_t *const (&bp)[2], Frag (&b0)[2]) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int Fg = ti.shared ? a.Fs : a.F;
    const int ncol = blockIdx.y * 16 * DW + wave * 16;  // first gate column of this wave
    const int rl = lane & 15, kq = 8 * (lane >> 4);
    int tok[HALVES];
#pragma unroll
    for (int h = 0; h < HALVES; ++h) {
        const int r = min(16 * h + rl, ti.nrows - 1);  // padding rows repeat the last row
        tok[h] = tile_src(a, ti, r);
    }
    Frag a0[HALVES];
    const uint16_t *ap[HALVES];
#pragma unroll
    for (int h = 0; h < HALVES; ++h)
        ap[h] = a.x + (int64_t)(ti.shared ? tok[h] : tok[h] / a.k) * a.d + kq;
    load_a<HALVES>(a0, ap, 0);
    f32x4 acc[HALVES][2];
#pragma unroll
    for (int h = 0; h < HALVES; ++h)
#pragma unroll
        for (int n = 0; n < 2; ++n) acc[h][n] = f32x4{0.f, 0.f, 0.f, 0.f};
    stream_k_from<2, HALVES>(b0, a0, bp, ap, a.d, acc);
    uint16_t *H = ti.shared ? a.h_sh : a.h;
    // 16x16 accumulator: lane holds column lane % 16, rows 4 (lane / 16) + i.
#pragma unroll
    for (int h = 0; h < HALVES; ++h)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = 16 * h + 4 * (lane >> 4) + i;
            if (row < ti.nrows) {
                const int64_t hr = tile_row(ti, row);
                H[hr * Fg + ncol + rl] = f32_to_bf16_rne(silu_mul(acc[h][0][i], acc[h][1][i]));
                if (a.au) {  // training forward: the pre-activations too
                    uint16_t *arow = (ti.shared ? a.au_sh : a.au) + hr * 2 * Fg;
                    arow[ncol + rl] = f32_to_bf16_rne(acc[h][0][i]);
                    arow[Fg + ncol + rl] = f32_to_bf16_rne(acc[h][1][i]);
                }
            }
        }
}

__global__ __launch_bounds__(64 * DW) void decode_gateup_kernel(DecodeArgs a) {
    __shared__ int rows[DW][DBM];
    TileInfo ti;
    if (!decode_tile(a, ti, blockIdx.x)) return;
    const int Fg = ti.shared ? a.Fs : a.F;
    if (blockIdx.y * 16 * DW >= Fg) return;
    // the first weight group goes out before the rows are looked up
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int ncol = blockIdx.y * 16 * DW + wave * 16;
    const int rl = lane & 15, kq = 8 * (lane >> 4);
    const uint16_t *W = ti.shared ? a.w_sh : a.w + (int64_t)ti.g * 2 * a.F * a.d;
    const uint16_t *bp[2] = {W + (int64_t)(ncol + rl) * a.d + kq,
                             W + (int64_t)(Fg + ncol + rl) * a.d + kq};
    Frag b0[2];
    load_b<2>(b0, bp, 0);
    if (!tile_rows(a, ti, rows[wave])) {
        drain_and_end();
        return;
    }
    if (ti.nrows > 16) decode_gateup_body<2>(a, ti, bp, b0);
    else decode_gateup_body<1>(a, ti, bp, b0);
}

// down: block = DW waves, wave w owns output columns n0 + 16 DNB w .. + 16 DNB
// (DNB 16-column blocks); grid.x walks 16 DNB DW-column slabs of d and grid.y
// the tiles, so the slabs of one expert run back to back (measured faster
// than tile-major order here; gate/up keeps tile-major order).  Nothing in the
// stream depends on the routing (h rows are the tile's own rows), so the
// lookups that the epilogue needs (pair ids, then weights) are issued first
// and resolved after the stream.
template <int HALVES>
__device__ void decode_down_body(const DecodeArgs &a, const TileInfo &ti,
                                 const uint16_t *const (&bp)[DNB], Frag (&b0)[DNB]) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int Fg = ti.shared ? a.Fs : a.F;
    const int ncol = blockIdx.x * 16 * DNB * DW + wave * 16 * DNB;
    const int rl = lane & 15, kq = 8 * (lane >> 4);
    // this lane's output rows 16 h + 4 (lane / 16) + i: routed rows need their
    // pair id (for the weight), shared rows are tokens row0 + row
    int src[HALVES][4];
#pragma unroll
    for (int h = 0; h < HALVES; ++h)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = min(16 * h + 4 * (lane >> 4) + i, ti.nrows - 1);
            src[h][i] = tile_src(a, ti, r);
        }
    const uint16_t *H = ti.shared ? a.h_sh : a.h;
    const uint16_t *ap[HALVES];
#pragma unroll
    for (int h = 0; h < HALVES; ++h) {
        const int r = 16 * h + rl;
        ap[h] = H + (int64_t)tile_row(ti, min(r, ti.nrows - 1)) * Fg + kq;
    }
    Frag a0[HALVES];
    load_a<HALVES>(a0, ap, 0);
    f32x4 acc[HALVES][DNB];
#pragma unroll
    for (int h = 0; h < HALVES; ++h)
#pragma unroll
        for (int n = 0; n < DNB; ++n) acc[h][n] = f32x4{0.f, 0.f, 0.f, 0.f};
    stream_k_from<DNB, HALVES>(b0, a0, bp, ap, Fg, acc);
    float wr[HALVES][4];
#pragma unroll
    for (int h = 0; h < HALVES; ++h)
#pragma unroll
        for (int i = 0; i < 4; ++i) wr[h][i] = ti.shared ? a.gate[src[h][i]] : a.topk_w[src[h][i]];
#pragma unroll
    for (int h = 0; h < HALVES; ++h)
#pragma unroll
        for (int n = 0; n < DNB; ++n)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = 16 * h + 4 * (lane >> 4) + i;
                const int col = ncol + 16 * n + rl;
                if (row < ti.nrows && col < a.d) {
                    const float v = wr[h][i] * acc[h][n][i];
                    if (ti.shared) a.out[(int64_t)(ti.row0 + row) * a.d + col] = v;
                    else a.y[(int64_t)tile_row(ti, row) * a.d + col] = v;
                }
            }
}

__global__ __launch_bounds__(64 * DW) void decode_down_kernel(DecodeArgs a) {
    __shared__ int rows[DW][DBM];
    TileInfo ti;
    if (!decode_tile(a, ti, blockIdx.y)) return;
    if (blockIdx.x * 16 * DNB * DW >= a.d) return;
    // the first weight group goes out before the rows are looked up
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int Fg = ti.shared ? a.Fs : a.F;
    const int ncol = blockIdx.x * 16 * DNB * DW + wave * 16 * DNB;
    const int rl = lane & 15, kq = 8 * (lane >> 4);
    const uint16_t *W = ti.shared ? a.w_sh : a.w + (int64_t)ti.g * a.d * a.F;
    const uint16_t *bp[DNB];
#pragma unroll
    for (int n = 0; n < DNB; ++n) bp[n] = W + (int64_t)min(ncol + 16 * n + rl, a.d - 1) * Fg + kq;
    Frag b0[DNB];
    load_b<DNB>(b0, bp, 0);
    if (!tile_rows(a, ti, rows[wave])) {
        drain_and_end();
        return;
    }
    if (ti.nrows > 16) decode_down_body<2>(a, ti, bp, b0);
    else decode_down_body<1>(a, ti, bp, b0);
}

// ---------------------------------------------------------------------------
// MXFP4 expert weights.  Same tiles, blocks and ping-pong pipeline; the
// weights arrive as E2M1 codes (two per byte, even element in the low nibble)
// with one E8M0 scale per 32 elements of a row, in the packed form of 16-row
// x 128-element tiles (1 KB of codes in wave-load order, then 64 scale
// bytes; mx4_pack_kernel below), and are decoded exactly to bf16 in
// registers by v_cvt_scalef32_pk_bf16_fp4.  That instruction uses
// only the exponent field of its binary32 scale operand, so scale byte X is
// passed as the bits X << 23 (2^(X-127) for every X < 255, 2^-127 included).
//
// A lane's 16-byte load is one whole 32-element block: in K group g (128
// elements, one packed tile per 16-row block) lane r + 16 q loads elements
// 128 g + 32 q .. + 31 of weight row r of the block -- bytes 16 (r + 16 q) of
// the tile, so a wave's load reads one contiguous KB -- and MFMA step s of
// the group takes, in lane q, elements
// 128 g + 32 q + 8 s .. + 7 of the weights and of the token row alike.  The
// four q lanes of a step still cover 32 distinct k and the four steps cover
// the group, so every dot product is the same sum; only the binary32
// summation order inside the MFMAs differs from the bf16 kernels'.  A wave
// owns NB4 blocks of 16 weight rows, so one group streams 4 KB of codes per
// wave (the bf16 kernels stream 8 KB of weights per group over 2 blocks).
// Each block's tiles follow each other along K, so a wave reads NB4
// sequential streams; with the row-major MX layout (64 bytes of each of 64
// rows 1280 bytes apart per group) the gate/up stage was 22% slower.

constexpr int NB4 = 4;
constexpr int TILE4 = 1088;  // bytes of one packed 16 x 128 tile: 1024 of codes, 64 of scales

struct Mx4Args {
    const uint8_t *wp;     // packed routed weights: gate/up [E*2F, d], down [E*d, F]
    const uint8_t *wp_sh;  // packed shared weights: gate/up [2Fs, d], down [d, Fs]
    const uint16_t *x;
    uint16_t *h, *h_sh;
    float *out;
    float *y;              // [T*k, d] weighted routed rows (binary32)
    const int32_t *perm, *counts, *offsets, *tile_start, *tile_group;
    const int32_t *topk_idx;
    const float *topk_w, *gate;
    int64_t T;
    int d, E, k, F, Fs;
    int direct;            // tiles without the permutation step (decode_tile)
};

struct Mx4Group {
    uint4 c[NB4];      // one 32-element block of codes per weight-row block
    uint32_t s[NB4];   // its scale byte
};

__device__ __forceinline__ void mx4_load_b(Mx4Group &b, const uint8_t *const (&cp)[NB4],
                                           const uint8_t *const (&sp)[NB4], int g) {
#pragma unroll
    for (int n = 0; n < NB4; ++n) {
        b.c[n] = *reinterpret_cast<const uint4 *>(cp[n] + TILE4 * g);
        b.s[n] = sp[n][TILE4 * g];
    }
}

template <int HALVES>
__device__ __forceinline__ void mx4_load_a(Frag (&a)[HALVES], const uint16_t *const (&ap)[HALVES],
                                           int g) {
#pragma unroll
    for (int h = 0; h < HALVES; ++h)
#pragma unroll
        for (int s = 0; s < 4; ++s)
            a[h].v[s] = *reinterpret_cast<const uint4 *>(ap[h] + 128 * g + 8 * s);
}

template <int HALVES>
__device__ __forceinline__ void mx4_mfma_group(f32x4 (&acc)[HALVES][NB4], const Mx4Group &b,
                                               const Frag (&a)[HALVES]) {
    float sc[NB4];
#pragma unroll
    for (int n = 0; n < NB4; ++n) sc[n] = __uint_as_float(b.s[n] << 23);
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int n = 0; n < NB4; ++n) {
            const uint32_t w = s == 0 ? b.c[n].x : s == 1 ? b.c[n].y : s == 2 ? b.c[n].z : b.c[n].w;
            const bf16x8 wb = mx4_decode8(w, sc[n]);
#pragma unroll
            for (int h = 0; h < HALVES; ++h)
                acc[h][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    __builtin_bit_cast(bf16x8, a[h].v[s]), wb, acc[h][n], 0, 0, 0);
        }
}

// K (a multiple of 128) streamed with group 0 already loaded into b0 / a0;
// two groups in flight, branch-free steady state, tail peeled (as stream_k_from).
template <int HALVES>
__device__ __forceinline__ void mx4_stream(Mx4Group &b0, Frag (&a0)[HALVES],
                                           const uint8_t *const (&cp)[NB4],
                                           const uint8_t *const (&sp)[NB4],
                                           const uint16_t *const (&ap)[HALVES], int K,
                                           f32x4 (&acc)[HALVES][NB4]) {
    Mx4Group b1;
    Frag a1[HALVES];
    const int ng = K / KG;
    int g = 0;
    for (; g + 2 < ng; g += 2) {
        mx4_load_b(b1, cp, sp, g + 1);
        mx4_load_a<HALVES>(a1, ap, g + 1);
        __builtin_amdgcn_sched_barrier(0);
        mx4_mfma_group<HALVES>(acc, b0, a0);
        __builtin_amdgcn_sched_barrier(0);
        mx4_load_b(b0, cp, sp, g + 2);
        mx4_load_a<HALVES>(a0, ap, g + 2);
        __builtin_amdgcn_sched_barrier(0);
        mx4_mfma_group<HALVES>(acc, b1, a1);
        __builtin_amdgcn_sched_barrier(0);
    }
    if (g + 1 < ng) {
        mx4_load_b(b1, cp, sp, g + 1);
        mx4_load_a<HALVES>(a1, ap, g + 1);
        __builtin_amdgcn_sched_barrier(0);
        mx4_mfma_group<HALVES>(acc, b0, a0);
        __builtin_amdgcn_sched_barrier(0);
        mx4_mfma_group<HALVES>(acc, b1, a1);
    } else {
        mx4_mfma_group<HALVES>(acc, b0, a0);
    }
}

// This lane's first packed tile of each weight-row block of the wave (gate/up:
// K = d, d / 128 tiles per 16-row block; the two gate blocks then the
// matching up blocks), codes and scales.
__device__ __forceinline__ void mx4_gateup_ptrs(const Mx4Args &a, const TileInfo &ti,
                                                const uint8_t *(&cp)[NB4], const uint8_t *(&sp)[NB4]) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int Fg = ti.shared ? a.Fs : a.F;
    const int c0 = blockIdx.y * 32 * DW + wave * 32;
    const int64_t row_base = ti.shared ? 0 : (int64_t)ti.g * 2 * a.F;
    const uint8_t *P = ti.shared ? a.wp_sh : a.wp;
#pragma unroll
    for (int n = 0; n < NB4; ++n) {
        const int64_t rb = (row_base + (n < 2 ? c0 + 16 * n : Fg + c0 + 16 * (n - 2))) / 16;
        const uint8_t *tile = P + rb * (a.d / 128) * TILE4;
        cp[n] = tile + 16 * lane;
        sp[n] = tile + 1024 + lane;
    }
}

// The same for the down projection (K = Fg: Fg / 128 tiles per block;
// d % 128 == 0, so every block of the slab lies inside d).
__device__ __forceinline__ void mx4_down_ptrs(const Mx4Args &a, const TileInfo &ti,
                                              const uint8_t *(&cp)[NB4], const uint8_t *(&sp)[NB4]) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int Fg = ti.shared ? a.Fs : a.F;
    const int c0 = blockIdx.x * 64 * DW + wave * 64;
    const int64_t row_base = ti.shared ? 0 : (int64_t)ti.g * a.d;
    const uint8_t *P = ti.shared ? a.wp_sh : a.wp;
#pragma unroll
    for (int n = 0; n < NB4; ++n) {
        const int64_t rb = (row_base + c0 + 16 * n) / 16;
        const uint8_t *tile = P + rb * (Fg / 128) * TILE4;
        cp[n] = tile + 16 * lane;
        sp[n] = tile + 1024 + lane;
    }
}

// gate/up: wave w owns gate columns c0 .. c0 + 31 (two 16-row blocks) and the
// matching up columns; grid.y walks 32 DW-column slabs of the expert width.
template <int HALVES>
__device__ void mx4_gateup_body(const Mx4Args &a, const TileInfo &ti,
                                const uint8_t *const (&cp)[NB4], const uint8_t *const (&sp)[NB4],
                                Mx4Group &b0) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int Fg = ti.shared ? a.Fs : a.F;
    const int c0 = blockIdx.y * 32 * DW + wave * 32;
    const int rl = lane & 15, q = lane >> 4;
    int tok[HALVES];
#pragma unroll
    for (int h = 0; h < HALVES; ++h) {
        const int r = min(16 * h + rl, ti.nrows - 1);  // padding rows repeat the last row
        tok[h] = tile_src(a, ti, r);
    }
    const uint16_t *ap[HALVES];
#pragma unroll
    for (int h = 0; h < HALVES; ++h)
        ap[h] = a.x + (int64_t)(ti.shared ? tok[h] : tok[h] / a.k) * a.d + 32 * q;
    Frag a0[HALVES];
    mx4_load_a<HALVES>(a0, ap, 0);
    f32x4 acc[HALVES][NB4];
#pragma unroll
    for (int h = 0; h < HALVES; ++h)
#pragma unroll
        for (int n = 0; n < NB4; ++n) acc[h][n] = f32x4{0.f, 0.f, 0.f, 0.f};
    mx4_stream<HALVES>(b0, a0, cp, sp, ap, a.d, acc);
    uint16_t *H = ti.shared ? a.h_sh : a.h;
    // 16x16 accumulator: lane holds column lane % 16, rows 4 (lane / 16) + i.
#pragma unroll
    for (int h = 0; h < HALVES; ++h)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = 16 * h + 4 * q + i;
            if (row < ti.nrows)
#pragma unroll
                for (int n = 0; n < 2; ++n)
                    H[(int64_t)tile_row(ti, row) * Fg + c0 + 16 * n + rl] =
                        f32_to_bf16_rne(silu_mul(acc[h][n][i], acc[h][n + 2][i]));
        }
}

__global__ __launch_bounds__(64 * DW) void decode_gateup_mx4_kernel(Mx4Args a) {
    __shared__ int rows[DW][DBM];
    TileInfo ti;
    if (!decode_tile(a, ti, blockIdx.x)) return;
    const int Fg = ti.shared ? a.Fs : a.F;
    if (blockIdx.y * 32 * DW >= Fg) return;
    // the first weight group goes out before the rows are looked up
    const uint8_t *cp[NB4], *sp[NB4];
    mx4_gateup_ptrs(a, ti, cp, sp);
    Mx4Group b0;
    mx4_load_b(b0, cp, sp, 0);
    if (!tile_rows(a, ti, rows[threadIdx.x >> 6])) {
        drain_and_end();
        return;
    }
    if (ti.nrows > 16) mx4_gateup_body<2>(a, ti, cp, sp, b0);
    else mx4_gateup_body<1>(a, ti, cp, sp, b0);
}

// down: wave w owns output columns c0 .. c0 + 63 (four 16-row blocks of
// W_dn); grid.y walks 64 DW-column slabs of d.  The epilogue's lookups (pair
// ids, then weights) are issued before the stream, as in decode_down_body.
template <int HALVES>
__device__ void mx4_down_body(const Mx4Args &a, const TileInfo &ti,
                                const uint8_t *const (&cp)[NB4], const uint8_t *const (&sp)[NB4],
                                Mx4Group &b0) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int Fg = ti.shared ? a.Fs : a.F;
    const int c0 = blockIdx.x * 64 * DW + wave * 64;
    const int rl = lane & 15, q = lane >> 4;
    int src[HALVES][4];
#pragma unroll
    for (int h = 0; h < HALVES; ++h)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = min(16 * h + 4 * q + i, ti.nrows - 1);
            src[h][i] = tile_src(a, ti, r);
        }
    const uint16_t *H = ti.shared ? a.h_sh : a.h;
    const uint16_t *ap[HALVES];
#pragma unroll
    for (int h = 0; h < HALVES; ++h)
        ap[h] = H + (int64_t)tile_row(ti, min(16 * h + rl, ti.nrows - 1)) * Fg + 32 * q;
    Frag a0[HALVES];
    mx4_load_a<HALVES>(a0, ap, 0);
    f32x4 acc[HALVES][NB4];
#pragma unroll
    for (int h = 0; h < HALVES; ++h)
#pragma unroll
        for (int n = 0; n < NB4; ++n) acc[h][n] = f32x4{0.f, 0.f, 0.f, 0.f};
    mx4_stream<HALVES>(b0, a0, cp, sp, ap, Fg, acc);
    float wr[HALVES][4];
#pragma unroll
    for (int h = 0; h < HALVES; ++h)
#pragma unroll
        for (int i = 0; i < 4; ++i) wr[h][i] = ti.shared ? a.gate[src[h][i]] : a.topk_w[src[h][i]];
#pragma unroll
    for (int h = 0; h < HALVES; ++h)
#pragma unroll
        for (int n = 0; n < NB4; ++n)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = 16 * h + 4 * q + i;
                const int col = c0 + 16 * n + rl;
                if (row < ti.nrows && col < a.d) {
                    const float v = wr[h][i] * acc[h][n][i];
                    if (ti.shared) a.out[(int64_t)(ti.row0 + row) * a.d + col] = v;
                    else a.y[(int64_t)tile_row(ti, row) * a.d + col] = v;
                }
            }
}

__global__ __launch_bounds__(64 * DW) void decode_down_mx4_kernel(Mx4Args a) {
    __shared__ int rows[DW][DBM];
    TileInfo ti;
    if (!decode_tile(a, ti, blockIdx.y)) return;
    if (blockIdx.x * 64 * DW >= a.d) return;
    // the first weight group goes out before the rows are looked up
    const uint8_t *cp[NB4], *sp[NB4];
    mx4_down_ptrs(a, ti, cp, sp);
    Mx4Group b0;
    mx4_load_b(b0, cp, sp, 0);
    if (!tile_rows(a, ti, rows[threadIdx.x >> 6])) {
        drain_and_end();
        return;
    }
    if (ti.nrows > 16) mx4_down_body<2>(a, ti, cp, sp, b0);
    else mx4_down_body<1>(a, ti, cp, sp, b0);
}

// Row-major MX (codes [R, K/2], scales [R, K/32]) -> packed tiles.  Block of
// 256 threads = 4 tiles; thread i of a tile copies the 16 code bytes of row
// i % 16, block i / 16 of the tile and that block's scale byte.
__global__ __launch_bounds__(256) void mx4_pack_kernel(const uint8_t *__restrict__ codes,
                                                       const uint8_t *__restrict__ scales,
                                                       int64_t ntiles, int64_t K,
                                                       uint8_t *__restrict__ packed) {
    const int64_t tile = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (tile >= ntiles) return;
    const int i = threadIdx.x & 63, r = i & 15, c = i >> 4;
    const int64_t kt = K / 128, b = tile / kt, t = tile - b * kt;
    const int64_t row = 16 * b + r;
    uint8_t *dst = packed + tile * TILE4;
    *reinterpret_cast<uint4 *>(dst + 16 * i) =
        *reinterpret_cast<const uint4 *>(codes + row * (K / 2) + 64 * t + 16 * c);
    dst[1024 + i] = scales[row * (K / 32) + 4 * t + c];
}

hipError_t launch_mx4_pack(const uint8_t *codes, const uint8_t *scales, int64_t rows, int64_t K,
                           void *packed, hipStream_t s) {
    const int64_t ntiles = rows / 16 * (K / 128);
    hipLaunchKernelGGL(mx4_pack_kernel, dim3((unsigned)((ntiles + 3) / 4)), dim3(256), 0, s, codes,
                       scales, ntiles, K, static_cast<uint8_t *>(packed));
    return hipGetLastError();
}

hipError_t launch_experts_decode_mx4(const Problem &p, hipStream_t s,
                                     const std::function<void(int)> &mark) {
    Mx4Args a;
    a.x = static_cast<const uint16_t *>(p.x);
    a.h = static_cast<uint16_t *>(p.h);
    a.h_sh = static_cast<uint16_t *>(p.h_shared);
    a.out = p.out;
    a.y = static_cast<float *>(p.y);
    a.perm = p.perm;
    a.counts = p.counts;
    a.offsets = p.offsets;
    a.tile_start = p.tile_start;
    a.tile_group = p.tile_group;
    a.topk_idx = p.topk_idx;
    a.direct = p.direct;
    a.topk_w = p.topk_w;
    a.gate = p.gate;
    a.T = p.T;
    a.d = p.d;
    a.E = p.E;
    a.k = p.k;
    a.F = p.F;
    a.Fs = p.Fs;
    const int fmax = p.F > p.Fs ? p.F : p.Fs;
    // direct: at most min(E, T k) touched experts, then the shared expert
    const unsigned gx = p.direct ? (unsigned)(std::min<int64_t>(p.E, p.T * p.k) + 1) : (unsigned)p.max_tiles;
    a.wp = static_cast<const uint8_t *>(p.w_gate_up);
    a.wp_sh = static_cast<const uint8_t *>(p.w_sh_gate_up);
    hipLaunchKernelGGL(decode_gateup_mx4_kernel, dim3(gx, (fmax + 32 * DW - 1) / (32 * DW)),
                       dim3(64 * DW), 0, s, a);
    mark(3);
    a.wp = static_cast<const uint8_t *>(p.w_down);
    a.wp_sh = static_cast<const uint8_t *>(p.w_sh_down);
    hipLaunchKernelGGL(decode_down_mx4_kernel, dim3((p.d + 64 * DW - 1) / (64 * DW), gx),
                       dim3(64 * DW), 0, s, a);
    mark(4);
    return hipGetLastError();
}

hipError_t launch_experts_decode(const Problem &p, hipStream_t s,
                                 const std::function<void(int)> &mark) {
    DecodeArgs a;
    a.x = static_cast<const uint16_t *>(p.x);
    a.h = static_cast<uint16_t *>(p.h);
    a.h_sh = static_cast<uint16_t *>(p.h_shared);
    a.au = static_cast<uint16_t *>(p.au);
    a.au_sh = static_cast<uint16_t *>(p.au_sh);
    a.out = p.out;
    a.y = static_cast<float *>(p.y);
    a.perm = p.perm;
    a.counts = p.counts;
    a.offsets = p.offsets;
    a.tile_start = p.tile_start;
    a.tile_group = p.tile_group;
    a.topk_idx = p.topk_idx;
    a.direct = p.direct;
    a.topk_w = p.topk_w;
    a.gate = p.gate;
    a.T = p.T;
    a.d = p.d;
    a.E = p.E;
    a.k = p.k;
    a.F = p.F;
    a.Fs = p.Fs;
    const int fmax = p.F > p.Fs ? p.F : p.Fs;
    // direct: at most min(E, T k) touched experts, then the shared expert
    const unsigned gx = p.direct ? (unsigned)(std::min<int64_t>(p.E, p.T * p.k) + 1) : (unsigned)p.max_tiles;
    a.w = static_cast<const uint16_t *>(p.w_gate_up);
    a.w_sh = static_cast<const uint16_t *>(p.w_sh_gate_up);
    hipLaunchKernelGGL(decode_gateup_kernel, dim3(gx, (fmax + 16 * DW - 1) / (16 * DW)), dim3(64 * DW), 0, s,
                       a);
    mark(3);
    a.w = static_cast<const uint16_t *>(p.w_down);
    a.w_sh = static_cast<const uint16_t *>(p.w_sh_down);
    hipLaunchKernelGGL(decode_down_kernel, dim3((p.d + 16 * DNB * DW - 1) / (16 * DNB * DW), gx), dim3(64 * DW), 0, s,
                       a);
    mark(4);
    return hipGetLastError();
}

}  // namespace moe
