// backward.hip -- the layer's backward pass: gradients of every input and
// weight for a given routing, plus the router's load-balancing loss.
//
// The pages give the router's auxiliary-loss coefficient only (llm-atlas
// "Qwen3.8-Flash-Next", "Raw config fields", router_aux_loss_coef); the loss
// is read as coef * E * sum_e f_e P_e, with f_e the share of the T*k routed
// assignments that went to expert e and P_e the mean router probability of e.
// The scalar differentiated is sum_t dout_t . out_t + L_aux, with the top-k
// selection held fixed (it is piecewise constant).  Per (token t, slot j)
// with expert e and routing weight w (experts are gated MLPs with SiLU:
// llm-architectures-explained "Qwen3.8-Flash-Next", "Every architecture
// field", ffns.moe.gated):
//   a, u = W_g x, W_u x;  h = silu(a) u;  G = W_dn^T dout_t;  dw = G . h
//   dh = w G;  da = dh u silu'(a);  du = dh silu(a)
//   dx_t += W_gu^T [da; du];  dW_gu += [da; du] x_t^T;  dW_dn += dout_t (w h)^T
// The shared expert is the same with w = s_t = sigmoid(g . x_t); its gate
// logit gets ds s (1 - s), ds = G_sh . h_sh.  The router logits get
//   dl_te = [e = idx_tj] w_j (dw_j - sum_j' w_j' dw_j') + coef (E/T) p_te (f_e - f . p_t)
// and dW_r = dL^T X, dx += dL W_r (the shared-gate logit rides along as
// column E, with g as router row E).
//
// Launch sequence (bfloat16 layers on MFMA; binary32 layers use the same jobs
// with a plain FMA kernel):
//   1. permutation and tile map of the given routing (permute.hip)
//   2. logits   [T, E+1]  = X [W_r; g]^T                       (binary32)
//   3. AU       [rows, 2F] = X_gathered W_gu^T  (pre-activations a | u)
//   4. G        [rows, F]  = dOut_gathered W_dn                 (binary32)
//   5. SwiGLU backward per row: dGU = [da | du], H = w h, dw (pair) or ds (token)
//   6. router backward per token: dL [T, E+1], q_t = f . p_t
//   7. dXp      [rows, d]  = dGU W_gu
//   8. dW_gu,e  = dGU_e^T X_e;   dW_dn,e = dOut_e^T H_e         (K = rows of e)
//   9. dW_r     = dL^T X;        dXr = dL [W_r; g]
//  10. dx[t] = sum_j dXp[row(t,j)] + dXs[t] + dXr[t];  L_aux = coef E/T sum_t q_t
//
// One grouped-GEMM kernel serves every contraction.  An operand is either
// contiguous along the reduction axis ("KC", e.g. a weight row of W_gu for
// X W_gu^T) or along the output axis ("MC", e.g. W_dn read as W_dn^T, or the
// token-major activations of a weight gradient, whose reduction runs over
// tokens).  KC tiles go to LDS as they are; MC tiles are transposed on the
// way through registers (two reduction indices packed per 32-bit LDS write),
// so the MFMA fragments always read eight consecutive reduction elements.
#include "moe_device.h"
#include "moe_kernels.h"

#include <limits.h>

#include <algorithm>

namespace moe {

enum BwdKind { K_LOGITS, K_AU, K_G, K_DX, K_DWGU, K_DWDN, K_DWR, K_DXR };

// Operand source.  The strided index s (the row for KC, the reduction index
// for MC) runs from `base` to `lim` (absolute); beyond `lim` a KC operand
// repeats its last row (its output is never stored) and an MC operand reads
// zeros.  With `map`, source row = map[s] / div and the value is scaled by
// scale[map[s]]; otherwise row = s and scale[s].  Rows at or past `alt` come
// from p_alt (row - alt).  MC operands read the columns cb .. cb + 127 of a
// row (tile-local i < ilim only).
struct Opnd {
    const char *p, *p_alt;
    int64_t ld;          // bytes per row
    const int32_t *map;
    int div;
    const float *scale;
    int base, lim, alt;
    int cb, ilim;
};

// One output tile: rows [0, mrows) x columns [0, ncols) of C at c (row
// stride ldc; tile rows >= c_alt go to c_alt_p + (row - c_alt) * ldc), K
// reduction steps of the job.
struct Job {
    Opnd a, b;
    char *c, *c_alt_p;
    int64_t ldc;
    int c_alt;
    int mrows, ncols, K;
    int N;       // output columns of the job (weight gradients)
    bool c_f32;  // binary32 output whatever the kind's (split reductions' partials)
};

constexpr int QB = 128;           // tile rows and columns
constexpr int QK = 64;            // reduction elements per step
constexpr int QLD = QK + 8;       // LDS row: 144 bytes

template <int KIND> struct Traits;
// A_KC / B_KC: operand contiguous along K; *_F32: binary32 source (rounded to
// bf16 when staged for the MFMA); C_F32: binary32 output (else bf16).
template <> struct Traits<K_LOGITS> { static constexpr bool A_KC = 1, B_KC = 1, A_F32 = 0, B_F32 = 0, C_F32 = 1; };
template <> struct Traits<K_AU>     { static constexpr bool A_KC = 1, B_KC = 1, A_F32 = 0, B_F32 = 0, C_F32 = 0; };
template <> struct Traits<K_G>      { static constexpr bool A_KC = 1, B_KC = 0, A_F32 = 1, B_F32 = 0, C_F32 = 1; };
template <> struct Traits<K_DX>     { static constexpr bool A_KC = 1, B_KC = 0, A_F32 = 0, B_F32 = 0, C_F32 = 0; };
template <> struct Traits<K_DWGU>   { static constexpr bool A_KC = 0, B_KC = 0, A_F32 = 0, B_F32 = 0, C_F32 = 0; };
template <> struct Traits<K_DWDN>   { static constexpr bool A_KC = 0, B_KC = 0, A_F32 = 1, B_F32 = 0, C_F32 = 0; };
template <> struct Traits<K_DWR>    { static constexpr bool A_KC = 0, B_KC = 0, A_F32 = 0, B_F32 = 0, C_F32 = 0; };
template <> struct Traits<K_DXR>    { static constexpr bool A_KC = 1, B_KC = 0, A_F32 = 0, B_F32 = 0, C_F32 = 1; };

__device__ __forceinline__ Opnd opnd(const void *p, int64_t ld, int base, int lim, int esize) {
    Opnd o;
    o.p = static_cast<const char *>(p);
    o.p_alt = o.p;
    o.ld = ld * esize;  // kept in bytes from here on
    o.map = nullptr;
    o.div = 1;
    o.scale = nullptr;
    o.base = base;
    o.lim = lim;
    o.alt = INT_MAX;
    o.cb = 0;
    o.ilim = QB;
    return o;
}

// Source row of strided index s, and its scale.
__device__ __forceinline__ const char *op_row(const Opnd &o, int s, float &sc) {
    int row = s;
    int si = s;
    if (o.map) {
        si = o.map[s];
        row = si / o.div;
    }
    sc = o.scale ? o.scale[si] : 1.0f;
    return row >= o.alt ? o.p_alt + (int64_t)(row - o.alt) * o.ld : o.p + (int64_t)row * o.ld;
}

// Tile decode shared by the grouped kinds that follow the permutation's tile
// map (tiles of QB rows of one group; group E is the shared expert).
struct MapTile {
    int g, row0, nrows, Fg;
    bool shared;
};
__device__ __forceinline__ bool map_tile(const BwdArgs &a, int tile, MapTile &t) {
    if (tile >= a.tile_start[a.E + 1]) return false;
    t.g = a.tile_group[tile];
    t.shared = t.g == a.E;
    const int m_local = (tile - a.tile_start[t.g]) * QB;
    if (!t.shared) {
        t.row0 = a.offsets[t.g] + m_local;
        t.nrows = min(QB, a.counts[t.g] - m_local);
    } else {
        t.row0 = m_local;
        t.nrows = (int)min<int64_t>(QB, a.T - m_local);
    }
    t.Fg = t.shared ? a.Fs : a.F;
    return t.nrows > 0;
}

// Block -> (bx, by) of the job grid, for a 1-D launch of nblocks(...) blocks.
// Workgroups go to the 8 XCDs round robin (block b on XCD b % 8) and each
// XCD has its own L2, so the blocks that share operands are kept on one XCD:
//   weight gradients: every tile of one expert (its rows of X / dOut and of
//     [da; du] / H, about 0.6-0.9 MB at the pages' shapes) on XCD g % 8, the
//     column tiles of one row tile consecutive;
//   the others: row tile m on XCD m % 8 with its column tiles consecutive
//     (the tile's gathered rows are read once per XCD).
template <int KIND>
__device__ __forceinline__ bool block_tile(int b, int nx, int ny, int groups, int &bx, int &by) {
    const int x = b & 7, q = b >> 3;
    if (KIND == K_DWGU || KIND == K_DWDN) {
        const int mtiles = nx / groups;          // row tiles per group
        const int per = mtiles * ny;             // tiles per group
        const int g = 8 * (q / per) + x;
        if (g >= groups) return false;
        const int r = q - (q / per) * per;
        bx = g * mtiles + r / ny;
        by = r - (r / ny) * ny;
        return true;
    }
    by = q % ny;
    bx = 8 * (q / ny) + x;
    return bx < nx;
}

__host__ __device__ inline unsigned bwd_blocks(int kind, int nx, int ny, int groups) {
    if (kind == K_DWGU || kind == K_DWDN)
        return 8u * (unsigned)((groups + 7) / 8) * (unsigned)(nx / groups) * (unsigned)ny;
    return 8u * (unsigned)((nx + 7) / 8) * (unsigned)ny;
}

// The job of block (bx, by) for a contraction kind; false: nothing to do.
// esize: bytes per element of the layer's dtype (2 bf16, 4 binary32).
template <int KIND>
__device__ bool make_job(const BwdArgs &a, int bx, int by, int es, Job &j) {
    const int E = a.E, d = a.d;
    const int sh_rows = a.Fs > 0 ? 1 : 0;  // router row E (the shared gate) exists
    j.c_alt = INT_MAX;
    j.c_alt_p = nullptr;
    j.c_f32 = false;
    if (KIND == K_LOGITS || KIND == K_DXR || KIND == K_DWR) {
        int m0 = QB * bx, n0 = QB * by;
        if (KIND == K_LOGITS) {
            // column tiles of K slice sl follow those of slice sl - 1
            const int ntn = (E + sh_rows + QB - 1) / QB;
            const int sl = by / ntn;
            if (sl >= a.logit_split) return false;
            n0 = QB * (by - sl * ntn);
            const int ks = d / a.logit_split;
            j.mrows = (int)min<int64_t>(QB, a.T - m0);
            j.ncols = min(QB, E + sh_rows - n0);
            j.K = ks;
            j.a = opnd(a.x, d, m0, (int)a.T, es);
            j.b = opnd(a.w_router, d, n0, E + sh_rows, es);
            j.b.alt = E;
            j.b.p_alt = static_cast<const char *>(a.sh_gate ? a.sh_gate : a.w_router);
            j.a.p += (int64_t)sl * ks * es;  // rows start at the slice's first element
            j.b.p += (int64_t)sl * ks * es;
            j.b.p_alt += (int64_t)sl * ks * es;
            j.c = reinterpret_cast<char *>(a.logits + (int64_t)sl * a.T * a.ldl + (int64_t)m0 * a.ldl + n0);
            j.ldc = (int64_t)a.ldl * 4;
        } else if (KIND == K_DXR) {
            j.mrows = (int)min<int64_t>(QB, a.T - m0);
            j.ncols = min(QB, d - n0);
            j.K = a.ldd;
            j.a = opnd(a.dl, a.ldd, m0, (int)a.T, es);
            j.b = opnd(a.w_router, d, 0, E + sh_rows, es);
            j.b.alt = E;
            j.b.p_alt = static_cast<const char *>(a.sh_gate ? a.sh_gate : a.w_router);
            j.b.cb = n0;
            j.b.ilim = j.ncols;
            j.c = reinterpret_cast<char *>(a.dxr + (int64_t)m0 * d + n0);
            j.ldc = (int64_t)d * 4;
        } else {  // K_DWR
            // with dwr_split > 1, column tiles of token chunk sl follow those
            // of chunk sl - 1, and each chunk writes a binary32 partial
            const int ntn = (d + QB - 1) / QB;
            const int sl = by / ntn;
            if (sl >= a.dwr_split) return false;
            n0 = QB * (by - sl * ntn);
            const int chunk = (int)((a.T + a.dwr_split - 1) / a.dwr_split);
            const int rb = sl * chunk, re = (int)min<int64_t>(a.T, (int64_t)rb + chunk);
            if (re <= rb) return false;
            j.mrows = min(QB, E + sh_rows - m0);
            j.ncols = min(QB, d - n0);
            j.K = re - rb;
            j.a = opnd(a.dl, a.ldd, rb, re, es);
            j.a.cb = m0;
            j.a.ilim = min(QB, E + 1 - m0);
            j.b = opnd(a.x, d, rb, re, es);
            j.b.cb = n0;
            j.b.ilim = j.ncols;
            if (a.dwr_split > 1) {
                j.c = reinterpret_cast<char *>(a.part + ((int64_t)sl * (E + sh_rows) + m0) * d + n0);
                j.ldc = (int64_t)d * 4;
                j.c_f32 = true;
            } else {
                j.c = static_cast<char *>(a.dw_router) + ((int64_t)m0 * d + n0) * es;
                j.ldc = (int64_t)d * es;
                if (a.dsh_gate) {
                    j.c_alt = E - m0;
                    j.c_alt_p = static_cast<char *>(a.dsh_gate) + (int64_t)n0 * es;
                }
            }
        }
        return j.mrows > 0 && j.ncols > 0;
    }
    if (KIND == K_AU || KIND == K_G || KIND == K_DX) {
        MapTile t;
        if (!map_tile(a, bx, t)) return false;
        const int N = KIND == K_AU ? 2 * t.Fg : KIND == K_G ? t.Fg : d;
        const int n0 = QB * by;
        if (n0 >= N) return false;
        j.mrows = t.nrows;
        j.ncols = min(QB, N - n0);
        const int64_t g = t.g;
        if (KIND == K_AU) {
            j.K = d;
            j.a = opnd(a.x, d, t.row0, t.row0 + t.nrows, es);
            j.b = opnd(t.shared ? a.w_sgu : static_cast<const char *>(a.w_gu) + g * 2 * a.F * d * es,
                       d, n0, N, es);
            j.c = static_cast<char *>(t.shared ? a.au_sh : a.au) + ((int64_t)t.row0 * N + n0) * es;
            j.ldc = (int64_t)N * es;
        } else if (KIND == K_G) {
            j.K = d;
            j.a = opnd(a.dout, d, t.row0, t.row0 + t.nrows, 4);
            j.b = opnd(t.shared ? a.w_sdn : static_cast<const char *>(a.w_dn) + g * d * a.F * es,
                       t.Fg, 0, d, es);
            j.b.cb = n0;
            j.b.ilim = j.ncols;
            j.c = reinterpret_cast<char *>((t.shared ? a.g_sh : a.g) + (int64_t)t.row0 * N + n0);
            j.ldc = (int64_t)N * 4;
        } else {  // K_DX
            j.K = 2 * t.Fg;
            j.a = opnd(t.shared ? a.dgu_sh : a.dgu, 2 * t.Fg, t.row0, t.row0 + t.nrows, es);
            j.b = opnd(t.shared ? a.w_sgu : static_cast<const char *>(a.w_gu) + g * 2 * a.F * d * es,
                       d, 0, 2 * t.Fg, es);
            j.b.cb = n0;
            j.b.ilim = j.ncols;
            j.c = static_cast<char *>(t.shared ? a.dxs : a.dxp) + ((int64_t)t.row0 * d + n0) * es;
            j.ldc = (int64_t)d * es;
        }
        if (!t.shared && (KIND == K_AU || KIND == K_G)) {
            j.a.map = a.perm;
            j.a.div = a.k;
        }
        return true;
    }
    // K_DWGU / K_DWDN: one group per run of M-tiles: the experts, then the
    // shared expert (groups E .. E + sh_split - 1: its reduction over the
    // tokens split into chunks of sh_chunk rows, each chunk's binary32
    // partial written to part[chunk], when sh_split > 0)
    const int Fmax = a.F > a.Fs ? a.F : a.Fs;
    const int mtiles = KIND == K_DWGU ? (2 * Fmax + QB - 1) / QB : (d + QB - 1) / QB;
    const int g = bx / mtiles, mt = bx - g * mtiles;
    if (g >= E + (a.sh_split > 0 ? a.sh_split : 1) || (g >= E && a.Fs == 0)) return false;
    const bool shared = g >= E;
    const int sp = g - E;
    const int Fg = shared ? a.Fs : a.F;
    const int M = KIND == K_DWGU ? 2 * Fg : d;
    const int N = KIND == K_DWGU ? d : Fg;
    const int m0 = QB * mt, n0 = QB * by;
    if (m0 >= M || n0 >= N) return false;
    j.mrows = min(QB, M - m0);
    j.ncols = min(QB, N - n0);
    int rb = 0, cnt = (int)a.T;
    if (!shared) {
        rb = a.offsets[g];
        cnt = a.counts[g];
    } else if (a.sh_split > 0) {
        rb = sp * a.sh_chunk;
        cnt = min(a.sh_chunk, (int)a.T - rb);
        if (cnt <= 0) return false;
    }
    // groups up to dw_kmin rows are done by the short-reduction kernel
    if ((!shared || a.sh_split == 0) && cnt <= a.dw_kmin) return false;
    j.K = cnt;
    j.N = N;
    if (KIND == K_DWGU) {
        j.a = opnd(shared ? a.dgu_sh : a.dgu, 2 * Fg, rb, rb + cnt, es);
        j.b = opnd(a.x, d, rb, rb + cnt, es);
        j.c = (shared ? static_cast<char *>(a.dw_sgu)
                      : static_cast<char *>(a.dw_gu) + (int64_t)g * 2 * a.F * d * es) +
              ((int64_t)m0 * d + n0) * es;
        j.ldc = (int64_t)d * es;
    } else {
        j.a = opnd(a.dout, d, rb, rb + cnt, 4);  // the weights are in H
        j.b = opnd(shared ? a.hh_sh : a.hh, Fg, rb, rb + cnt, es);
        j.c = (shared ? static_cast<char *>(a.dw_sdn)
                      : static_cast<char *>(a.dw_dn) + (int64_t)g * d * a.F * es) +
              ((int64_t)m0 * Fg + n0) * es;
        j.ldc = (int64_t)Fg * es;
    }
    if (shared && a.sh_split > 0) {
        j.c = reinterpret_cast<char *>(a.part + (int64_t)sp * M * N + (int64_t)m0 * N + n0);
        j.ldc = (int64_t)N * 4;
        j.c_f32 = true;
    }
    j.a.cb = m0;
    j.a.ilim = j.mrows;
    j.b.cb = n0;
    j.b.ilim = j.ncols;
    if (!shared) {
        // token-indexed operands of routed rows follow the permutation
        Opnd &tokop = KIND == K_DWGU ? j.b : j.a;
        tokop.map = a.perm;
        tokop.div = a.k;
    }
    return true;
}

// ---------------------------------------------------------------------------
// Staging of one operand tile (QB x QK) into LDS, for 256 threads.

// KC: chunk c = tid + 256 q (q < 4) is row c / 8, elements 8 (c % 8) .. +7.
template <bool F32>
struct StageKC {
    const char *src[4];
    uint4 r[4];
    uint4 r2[4];  // binary32 sources: second half of the 8 values
    __device__ void init(const Opnd &o, int tid) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int c = tid + 256 * q;
            int s = o.base + (c >> 3);
            if (s >= o.lim) s = o.lim - 1;
            float sc;
            src[q] = op_row(o, s, sc) + (int64_t)(8 * (c & 7)) * (F32 ? 4 : 2);
        }
    }
    __device__ void load(int k0) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            if (F32) {
                const float4 *p = reinterpret_cast<const float4 *>(src[q] + (int64_t)k0 * 4);
                r[q] = __builtin_bit_cast(uint4, p[0]);
                r2[q] = __builtin_bit_cast(uint4, p[1]);
            } else {
                r[q] = *reinterpret_cast<const uint4 *>(src[q] + (int64_t)k0 * 2);
            }
        }
    }
    __device__ void store(uint16_t *lds, int tid) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int c = tid + 256 * q;
            uint4 v = r[q];
            if (F32) {
                v.x = pack_bf16x2(__uint_as_float(r[q].x), __uint_as_float(r[q].y));
                v.y = pack_bf16x2(__uint_as_float(r[q].z), __uint_as_float(r[q].w));
                v.z = pack_bf16x2(__uint_as_float(r2[q].x), __uint_as_float(r2[q].y));
                v.w = pack_bf16x2(__uint_as_float(r2[q].z), __uint_as_float(r2[q].w));
            }
            *reinterpret_cast<uint4 *>(lds + (c >> 3) * QLD + 8 * (c & 7)) = v;
        }
    }
};

// MC: the tile goes to LDS as it lies in memory, reduction row k by output
// column m ([k][m], PM elements per row); the MFMA fragments are read back
// transposed with ds_read_b64_tr_b16 (mc_frag).  Thread piece c = tid + 256 q
// (q < 4) is row k = c / 16 of the step, columns 8 (c % 16) .. +7: sixteen
// lanes cover one 256-byte row piece, so each load instruction reads four
// whole row pieces.  The source rows of a step are looked up one step ahead
// (rows[], scl[]), so the data loads never wait on the permutation.
constexpr int PM = QB + 32;  // LDS row of an MC tile: 320 bytes (4 rows = 4 bank quarters)

template <bool F32>
struct StageMC {
    const char *rows[4];
    float scl[4];   // scales of the looked-up step
    float sld[4];   // scales of the step whose data is in r / r2
    bool live[4];
    bool okd[4];    // which of r / r2 hold data (else they are stored as zeros)
    uint4 r[4], r2[4];
    int k_in, m8;
    __device__ void init(int tid) {
        k_in = tid >> 4;
        m8 = 8 * (tid & 15);
    }
    // Branch-free: every lane looks up and loads a valid address (a row past
    // the end reads the last valid row, a column piece past the end reads
    // piece 0) and selects zero afterwards.  A branch around a load makes the
    // compiler wait for every memory operation in flight (stores included) at
    // the next use.
    __device__ void lookup(const Opnd &o, int k0) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int s = o.base + k0 + k_in + 16 * q;
            live[q] = s < o.lim;
            const int sc_idx = max(min(s, o.lim - 1), 0);
            float sc;
            rows[q] = op_row(o, sc_idx, sc);
            scl[q] = live[q] ? sc : 0.f;
        }
    }
    __device__ void load(const Opnd &o) {
        const bool mok = m8 < o.ilim;
        const int mc = mok ? m8 : 0;  // piece 0 of a row is always readable
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            sld[q] = scl[q];
            okd[q] = live[q] && mok;
            const char *p = rows[q] + (int64_t)(o.cb + mc) * (F32 ? 4 : 2);
            // the zero select waits until store(), so nothing waits for the
            // data before the step that writes it to LDS
            if (F32) {
                r[q] = __builtin_bit_cast(uint4, reinterpret_cast<const float4 *>(p)[0]);
                r2[q] = __builtin_bit_cast(uint4, reinterpret_cast<const float4 *>(p)[1]);
            } else {
                r[q] = *reinterpret_cast<const uint4 *>(p);
            }
        }
    }
    // rows k0 .. k0 + 63 of the LDS tile (k0 = 0 for a one-step tile)
    __device__ void store(uint16_t *lds, int k0 = 0) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const uint4 z = uint4{0, 0, 0, 0};
            uint4 v;
            if (F32) {
                const float sc = sld[q];
                const uint4 a = okd[q] ? r[q] : z, b = okd[q] ? r2[q] : z;
                v.x = pack_bf16x2(sc * __uint_as_float(a.x), sc * __uint_as_float(a.y));
                v.y = pack_bf16x2(sc * __uint_as_float(a.z), sc * __uint_as_float(a.w));
                v.z = pack_bf16x2(sc * __uint_as_float(b.x), sc * __uint_as_float(b.y));
                v.w = pack_bf16x2(sc * __uint_as_float(b.z), sc * __uint_as_float(b.w));
            } else {
                v = okd[q] ? r[q] : z;
            }
            *reinterpret_cast<uint4 *>(lds + (k0 + k_in + 16 * q) * PM + m8) = v;
        }
    }
};

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

// MFMA fragment of an MC tile: eight consecutive reduction rows k0 + 8 (lane
// / 32) .. + 7 of output column mb + lane % 32, as v_mfma_f32_32x32x16_bf16
// takes them.  ds_read_b64_tr_b16 works on groups of 16 lanes: lane 4 a + b
// of a group receives 16-bit element b of the 64-bit pieces addressed by
// lanes a, a + 4, a + 8, a + 12 of the group.  So lane s of the group points
// at row k + s / 4, columns 4 (s % 4) .. +3 of its 16-column block, and lane
// s receives rows k .. k + 3 of column 4 (s / 4) + ... = the block's column
// s; two reads (k and k + 4) give the eight rows.
__device__ __forceinline__ bf16x8 mc_frag(const uint16_t *lds, int k0, int mb, int lane) {
    const int g = lane >> 4, s = lane & 15;
    const int k = k0 + 8 * (g >> 1) + (s >> 2);
    const int m = mb + 16 * (g & 1) + 4 * (s & 3);
    const uint16_t *p = lds + k * PM + m;
    const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(p));
    const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(p + 4 * PM));
    const short __attribute__((ext_vector_type(8))) v =
        __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(bf16x8, v);
}

// Fragment of a KC tile (row m of the tile holds its reduction elements).
__device__ __forceinline__ bf16x8 kc_frag(const uint16_t *lds, int k0, int mb, int lane) {
    return *reinterpret_cast<const bf16x8 *>(&lds[(mb + (lane & 31)) * QLD + k0 + 8 * (lane >> 5)]);
}

template <bool KC>
__device__ __forceinline__ bf16x8 frag(const uint16_t *lds, int k0, int mb, int lane) {
    return KC ? kc_frag(lds, k0, mb, lane) : mc_frag(lds, k0, mb, lane);
}

// LDS elements of one QB x QK tile of either kind
constexpr int TILE_E = QB * QLD > QK * PM ? QB * QLD : QK * PM;

template <bool KC, bool F32> struct Stager;
template <bool F32> struct Stager<true, F32> {
    StageKC<F32> s;
    __device__ void init(const Opnd &o, int tid) { s.init(o, tid); }
    __device__ void lookup(const Opnd &, int) {}
    __device__ void load(const Opnd &, int k0) { s.load(k0); }
    __device__ void store(uint16_t *lds, int tid) { s.store(lds, tid); }
};
template <bool F32> struct Stager<false, F32> {
    StageMC<F32> s;
    __device__ void init(const Opnd &, int tid) { s.init(tid); }
    __device__ void lookup(const Opnd &o, int k0) { s.lookup(o, k0); }
    __device__ void load(const Opnd &o, int) { s.load(o); }
    __device__ void store(uint16_t *lds, int) { s.store(lds); }
};

// Store one accumulated tile (accumulator layout: lane holds column lane % 32
// and rows 8 (v / 4) + 4 (lane / 32) + (v % 4)).
template <bool C_F32>
__device__ __forceinline__ void store_tile(const Job &j, f32x16 (&acc)[2][2], int wm, int wn,
                                           int lane) {
    // accumulator layout (B A^T, mfma_step): lane holds row 64 wm + 32 mi +
    // lane % 32 and, in acc[mi][ni][4 g + q], column 64 wn + 32 ni + 8 g +
    // 4 (lane / 32) + q: runs of four columns go out as one 16- (binary32) or
    // 8-byte (bf16) store where the rows allow it
    const int fr = lane & 31;
    const bool f32 = C_F32 || j.c_f32;
    const int64_t vec_align = f32 ? 16 : 8;
    const bool vec = j.ldc % vec_align == 0 &&
                     reinterpret_cast<uintptr_t>(j.c) % vec_align == 0 &&
                     (j.c_alt >= j.mrows || reinterpret_cast<uintptr_t>(j.c_alt_p) % vec_align == 0);
#pragma unroll
    for (int mi = 0; mi < 2; ++mi) {
        const int row = 64 * wm + 32 * mi + fr;
        if (row >= j.mrows) continue;
        char *crow = row >= j.c_alt ? j.c_alt_p + (int64_t)(row - j.c_alt) * j.ldc
                                    : j.c + (int64_t)row * j.ldc;
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int col = 64 * wn + 32 * ni + 8 * g + 4 * (lane >> 5);
                const f32x16 &c4 = acc[mi][ni];
                if (vec && col + 3 < j.ncols) {
                    if (f32)
                        *reinterpret_cast<float4 *>(crow + (int64_t)col * 4) =
                            make_float4(c4[4 * g], c4[4 * g + 1], c4[4 * g + 2], c4[4 * g + 3]);
                    else
                        *reinterpret_cast<uint2 *>(crow + (int64_t)col * 2) =
                            make_uint2(pack_bf16x2(c4[4 * g], c4[4 * g + 1]),
                                       pack_bf16x2(c4[4 * g + 2], c4[4 * g + 3]));
                } else {
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        if (col + q >= j.ncols) continue;
                        if (f32)
                            reinterpret_cast<float *>(crow)[col + q] = c4[4 * g + q];
                        else
                            reinterpret_cast<uint16_t *>(crow)[col + q] = f32_to_bf16_rne(c4[4 * g + q]);
                    }
                }
            }
    }
}

// One QK step of the 128 x 128 tile from LDS: 4 waves in 2 x 2, each 64 x 64
// from v_mfma_f32_32x32x16_bf16, accumulated as B A^T (the layout store_tile
// takes).
template <bool A_KC, bool B_KC>
__device__ __forceinline__ void mfma_step(const uint16_t *As, const uint16_t *Bs,
                                          f32x16 (&acc)[2][2], int wm, int wn, int lane) {
#pragma unroll
    for (int ks = 0; ks < QK / 16; ++ks) {
        bf16x8 af[2], bfr[2];
#pragma unroll
        for (int mi = 0; mi < 2; ++mi) af[mi] = frag<A_KC>(As, 16 * ks, 64 * wm + 32 * mi, lane);
#pragma unroll
        for (int ni = 0; ni < 2; ++ni) bfr[ni] = frag<B_KC>(Bs, 16 * ks, 64 * wn + 32 * ni, lane);
#pragma unroll
        for (int mi = 0; mi < 2; ++mi)
#pragma unroll
            for (int ni = 0; ni < 2; ++ni)
                acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[ni], af[mi],
                                                                      acc[mi][ni], 0, 0, 0);
    }
}

// bfloat16 layers, long reductions: 128 x 128 tiles, register-staged double
// buffer in LDS (the next step's loads fly while this one computes); two
// blocks per CU.
template <int KIND>
__global__ __launch_bounds__(256, 2) void bwd_gemm_kernel(BwdArgs a, int nx, int ny, int groups,
                                                          int nvirt) {
    using Tr = Traits<KIND>;
    __shared__ __align__(16) uint16_t As[2][TILE_E];
    __shared__ __align__(16) uint16_t Bs[2][TILE_E];
    const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
    const int wm = wave >> 1, wn = wave & 1;
    // Weight gradients after the short-reduction kernel: when no routed
    // expert has more than dw_kmin rows, only the shared expert's groups
    // (E .. , after the routed ones in the virtual order) have work, so the
    // walk starts at their first virtual block instead of looking at every
    // routed tile.
    int b0 = blockIdx.x;
    if ((KIND == K_DWGU || KIND == K_DWDN) && a.dw_kmin >= 0) {
        bool big = false;
        for (int g = tid; g < a.E; g += 256) big |= a.counts[g] > a.dw_kmin;
        if (!__syncthreads_or(big)) {
            const int per = (nx / groups) * ny;  // virtual blocks per group
            b0 += 8 * per * (a.E / 8);
        }
    }
    // grid-stride over the virtual blocks (the grid is a multiple of 8, so a
    // block keeps its XCD's share of the tile map); tiles with nothing to do
    // cost one look at the tile map instead of a block launch each
    for (int b = b0; b < nvirt; b += gridDim.x) {
        Job j;
        int bx, by;
        if (!block_tile<KIND>(b, nx, ny, groups, bx, by) || !make_job<KIND>(a, bx, by, 2, j))
            continue;
        Stager<Tr::A_KC, Tr::A_F32> sa;
        Stager<Tr::B_KC, Tr::B_F32> sb;
        sa.init(j.a, tid);
        sb.init(j.b, tid);

        f32x16 acc[2][2];
#pragma unroll
        for (int mi = 0; mi < 2; ++mi)
#pragma unroll
            for (int ni = 0; ni < 2; ++ni)
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[mi][ni][v] = 0.f;

        const int nk = (j.K + QK - 1) / QK;
        if (nk > 0) {
            sa.lookup(j.a, 0);
            sb.lookup(j.b, 0);
            sa.load(j.a, 0);
            sb.load(j.b, 0);
            if (nk > 1) {
                sa.lookup(j.a, QK);
                sb.lookup(j.b, QK);
            }
            sa.store(As[0], tid);
            sb.store(Bs[0], tid);
            __syncthreads();
        }
        for (int kt = 0; kt < nk; ++kt) {
            const int cur = kt & 1;
            if (kt + 1 < nk) {
                sa.load(j.a, (kt + 1) * QK);
                sb.load(j.b, (kt + 1) * QK);
                if (kt + 2 < nk) {
                    sa.lookup(j.a, (kt + 2) * QK);
                    sb.lookup(j.b, (kt + 2) * QK);
                }
            }
            mfma_step<Tr::A_KC, Tr::B_KC>(As[cur], Bs[cur], acc, wm, wn, lane);
            if (kt + 1 < nk) {
                sa.store(As[cur ^ 1], tid);
                sb.store(Bs[cur ^ 1], tid);
            }
            __syncthreads();  // also: LDS free for the next tile of this block
        }
        store_tile<Tr::C_F32>(j, acc, wm, wn, lane);
    }
}

// Weight gradients of experts with at most KS rows (the usual case: T k / E
// rows per expert on average), bfloat16 layers.  Block (expert g, row tile
// mt) stages its A tile -- 128 output rows x all K <= KS reduction rows --
// in LDS once (with the row lookups through the permutation done once), then
// walks every column tile of its rows: the next tile's B rows are loaded into
// registers while the current one computes, and each finished tile goes out
// through LDS as 16-byte row pieces, so a tile costs 8 stores per thread and
// the next tile's loads do not wait behind a long tail of small stores.
constexpr int KS = 128;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
constexpr int SLD = QB + 8;  // output staging row: 272 bytes

template <int KIND>
__global__ __launch_bounds__(256, 2) void bwd_dw_small_kernel(BwdArgs a, int nx, int groups) {
    using Tr = Traits<KIND>;
    __shared__ __align__(16) uint16_t As[KS * PM];  // [k][m], as MC tiles
    __shared__ __align__(16) uint16_t Bs[KS * PM];  // [k][n]; also the output staging
    Job j;
    int bx, by;
    if (!block_tile<KIND>(blockIdx.x, nx, 1, groups, bx, by)) return;
    BwdArgs aa = a;
    aa.dw_kmin = -1;  // every group with at most KS rows
    if (!make_job<KIND>(aa, bx, 0, 2, j) || j.K > KS) return;
    const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
    const int wm = wave >> 1, wn = wave & 1;
    const int fr = lane & 31;
    const int ntiles = (j.N + QB - 1) / QB;

    StageMC<Tr::A_F32> sa0, sa1;
    StageMC<false> sb0, sb1;
    sa0.init(tid);
    sa1.init(tid);
    sb0.init(tid);
    sb1.init(tid);
    sa0.lookup(j.a, 0);
    sa1.lookup(j.a, QK);
    sb0.lookup(j.b, 0);
    sb1.lookup(j.b, QK);
    sa0.load(j.a);
    sa1.load(j.a);
    sb0.load(j.b);
    sb1.load(j.b);
    sa0.store(As, 0);
    sa1.store(As, QK);
    sb0.store(Bs, 0);
    sb1.store(Bs, QK);
    __syncthreads();

    for (int t = 0; t < ntiles; ++t) {
        const int n0 = QB * t, ncols = min(QB, j.N - n0);
        // the next tile's B rows (the last iteration reloads its own tile: no
        // branch, see StageMC)
        const int tn = t + 1 < ntiles ? t + 1 : t;
        j.b.cb = QB * tn;
        j.b.ilim = min(QB, j.N - QB * tn);
        sb0.load(j.b);
        sb1.load(j.b);
        // keep the loads ahead of the MFMAs and the next tile's packing after
        // them (interleaving them only raises register pressure)
        __builtin_amdgcn_sched_barrier(0);
        f32x16 acc[2][2];
#pragma unroll
        for (int mi = 0; mi < 2; ++mi)
#pragma unroll
            for (int ni = 0; ni < 2; ++ni)
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[mi][ni][v] = 0.f;
#pragma unroll
        for (int ks = 0; ks < KS / 16; ++ks) {
            bf16x8 af[2], bfr[2];
#pragma unroll
            for (int mi = 0; mi < 2; ++mi) af[mi] = mc_frag(As, 16 * ks, 64 * wm + 32 * mi, lane);
#pragma unroll
            for (int ni = 0; ni < 2; ++ni) bfr[ni] = mc_frag(Bs, 16 * ks, 64 * wn + 32 * ni, lane);
            // B A^T: each lane ends with one output row and runs of four
            // consecutive columns (8-byte LDS writes below)
#pragma unroll
            for (int mi = 0; mi < 2; ++mi)
#pragma unroll
                for (int ni = 0; ni < 2; ++ni)
                    acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[ni], af[mi],
                                                                          acc[mi][ni], 0, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
        __syncthreads();  // every wave is done reading Bs
        // the tile as bf16 rows in Bs (accumulator layout: lane holds row
        // 64 wm + 32 mi + lane % 32 and, in acc[mi][ni][4 g + q], column
        // 64 wn + 32 ni + 8 g + 4 (lane / 32) + q)
#pragma unroll
        for (int mi = 0; mi < 2; ++mi)
#pragma unroll
            for (int ni = 0; ni < 2; ++ni)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int row = 64 * wm + 32 * mi + fr;
                    const int col = 64 * wn + 32 * ni + 8 * g + 4 * (lane >> 5);
                    const f32x16 &c4 = acc[mi][ni];
                    *reinterpret_cast<uint2 *>(&Bs[row * SLD + col]) =
                        make_uint2(pack_bf16x2(c4[4 * g], c4[4 * g + 1]),
                                   pack_bf16x2(c4[4 * g + 2], c4[4 * g + 3]));
                }
        __syncthreads();
        char *c = j.c + (int64_t)n0 * 2;
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            // pieces outside the tile rewrite a piece inside it with its own
            // bytes (no branch around the store)
            const int ch = tid + 256 * q;
            const int row = min(ch >> 4, j.mrows - 1), c8 = min(8 * (ch & 15), ncols - 8);
            // the gradient is read by no later kernel of the call: streamed
            // past the caches (nontemporal) so it does not evict the rows
            // the next tiles read
            __builtin_nontemporal_store(*reinterpret_cast<const u32x4 *>(&Bs[row * SLD + c8]),
                                        reinterpret_cast<u32x4 *>(c + (int64_t)row * j.ldc + c8 * 2));
        }
        __syncthreads();  // the staged tile is read out
        sb0.store(Bs, 0);
        sb1.store(Bs, QK);
        __syncthreads();
    }
}

// binary32 layers: the same jobs, one output element per thread and step,
// plain binary32 fused multiply-adds over the reduction.
__device__ __forceinline__ float op_elem_kc(const Opnd &o, int i, int k) {
    int s = o.base + i;
    if (s >= o.lim) s = o.lim - 1;
    float sc;
    return reinterpret_cast<const float *>(op_row(o, s, sc))[k] * sc;
}
__device__ __forceinline__ float op_elem_mc(const Opnd &o, int i, int k) {
    const int s = o.base + k;
    if (s >= o.lim || i >= o.ilim) return 0.f;
    float sc;
    return reinterpret_cast<const float *>(op_row(o, s, sc))[o.cb + i] * sc;
}

template <int KIND>
__global__ __launch_bounds__(256) void bwd_gemm_f32_kernel(BwdArgs a) {
    using Tr = Traits<KIND>;
    Job j;
    if (!make_job<KIND>(a, blockIdx.x, blockIdx.y, 4, j)) return;
    for (int o = threadIdx.x; o < QB * QB; o += 256) {
        const int i = o / QB, c = o % QB;
        if (i >= j.mrows || c >= j.ncols) continue;
        float acc = 0.f;
        for (int k = 0; k < j.K; ++k) {
            const float av = Tr::A_KC ? op_elem_kc(j.a, i, k) : op_elem_mc(j.a, i, k);
            const float bv = Tr::B_KC ? op_elem_kc(j.b, c, k) : op_elem_mc(j.b, c, k);
            acc = fmaf(av, bv, acc);
        }
        char *crow = i >= j.c_alt ? j.c_alt_p + (int64_t)(i - j.c_alt) * j.ldc
                                  : j.c + (int64_t)i * j.ldc;
        reinterpret_cast<float *>(crow)[c] = acc;
    }
}

// ---------------------------------------------------------------------------
// SwiGLU backward, one wave per row: routed rows r < offsets[E] (pair
// perm[r], weight topk_w), then the T shared rows (weight s_t = sigmoid of
// logit column E, stored to gate[t]).  dw (routed, at the pair id) or ds
// (shared, at the token) is G . h summed in a fixed order.
template <typename Tv>
__global__ __launch_bounds__(256) void swiglu_bwd_kernel(BwdArgs a) {
    const int64_t routed = (int64_t)a.T * a.k;
    const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const bool shared = r >= routed;
    int64_t row;
    int Fg;
    float w;
    int pair = 0;
    if (!shared) {
        if (r >= a.offsets[a.E]) return;
        row = r;
        pair = a.perm[r];
        w = a.topk_w[pair];
        Fg = a.F;
    } else {
        if (a.Fs == 0 || r - routed >= a.T) return;
        row = r - routed;
        float z = a.logits[row * a.ldl + a.E];
        for (int sl = 1; sl < a.logit_split; ++sl) z += a.logits[(sl * a.T + row) * a.ldl + a.E];
        w = 1.0f / (1.0f + __expf(-z));
        Fg = a.Fs;
        if (lane == 0) a.gate[row] = w;
    }
    const Tv *au = static_cast<const Tv *>(shared ? a.au_sh : a.au) + row * 2 * Fg;
    const float *G = (shared ? a.g_sh : a.g) + row * Fg;
    Tv *dgu = static_cast<Tv *>(shared ? a.dgu_sh : a.dgu) + row * 2 * Fg;
    Tv *hh = static_cast<Tv *>(shared ? a.hh_sh : a.hh) + row * Fg;
    float acc = 0.f;
    for (int f = lane; f < Fg; f += 64) {
        const float av = to_f32(au[f]), uv = to_f32(au[Fg + f]), gv = G[f];
        const float sg = 1.0f / (1.0f + __expf(-av));
        const float silu = av * sg;
        const float h = silu * uv;
        acc = fmaf(gv, h, acc);
        const float dh = w * gv;
        const float da = dh * uv * (sg * (1.0f + av * (1.0f - sg)));
        const float du = dh * silu;
        // H carries the row's weight (w, or s_t for the shared expert): the
        // down-projection weight gradient is then dOut^T H alone
        if constexpr (sizeof(Tv) == 2) {
            dgu[f] = f32_to_bf16_rne(da);
            dgu[Fg + f] = f32_to_bf16_rne(du);
            hh[f] = f32_to_bf16_rne(w * h);
        } else {
            dgu[f] = da;
            dgu[Fg + f] = du;
            hh[f] = w * h;
        }
    }
    acc = wave_sum(acc);
    if (lane == 0) {
        if (!shared) a.dwp[pair] = acc;
        else a.ds[row] = acc;
    }
}

// Block-wide fixed-order sum over 256 threads (4 waves).
__device__ __forceinline__ float block_sum(float v, float *red) {
    v = wave_sum(v);
    const int w = threadIdx.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[w] = v;
    __syncthreads();
    return (red[0] + red[1]) + (red[2] + red[3]);
}

// Router backward, one wave per token (four per block), expert e in lane
// e % 64, slot e / 64 (NS slots, E <= 64 NS): softmax p over the E logits
// (+ bias), f . p, the load-balancing term, the selected experts' term and
// the shared-gate logit's gradient, written as a dL row zero padded to ldd
// columns (layer dtype).  Sums run over each lane's slots in order, then a
// fixed tree over the wave.
template <typename Tv, int NS>
__global__ __launch_bounds__(256) void router_bwd_kernel(BwdArgs a) {
    const int lane = threadIdx.x & 63;
    const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= a.T) return;
    // G . h of each pair (lane jj < k) and of the shared row (every lane):
    // one value, or partial sums over 128 columns of G each, added in column
    // order; loaded first, used after the softmax
    // (every load is issued here, none waits for another: the kernel's time
    // is one memory latency, not a chain of them)
    const int st = a.gtile > 0 ? a.gtile : 1;
    const int nr = a.gtile > 0 ? (a.F + 127) / 128 : 1;
    const int ns = a.gtile > 0 ? (a.Fs + 127) / 128 : 1;
    // (unconditional loads from clamped addresses: a load under a branch
    // makes the compiler wait for every load at the join)
    const bool pl = lane < a.k;
    const int64_t pj = t * a.k + (pl ? lane : 0);
    float wj = a.topk_w[pj];
    int ej = a.topk_idx[pj];
    constexpr int U = 8;  // partial sums loaded up front; more come one by one
    float dpart[U], spart[U];
#pragma unroll
    for (int i = 0; i < U; ++i) {
        dpart[i] = a.dwp[pj * st + min(i, nr - 1)];
        spart[i] = a.ds[t * st + min(i, max(ns, 1) - 1)];
    }
    float sg = a.gate[t];
    // the token's logits (the sum of the K slices' partials) plus the bias,
    // and f_e = counts_e / (T k)
    float v[NS], fe[NS];
    const float inv_pairs = 1.0f / (float)((int64_t)a.T * a.k);
#pragma unroll
    for (int j = 0; j < NS; ++j) {
        const int e = min(lane + 64 * j, a.E - 1);
        const float x0 = a.logits[t * a.ldl + e];
        const float x1 = a.logits[((a.logit_split > 1 ? a.T : 0) + t) * a.ldl + e];
        const float b = a.bias ? a.bias[e] : 0.f;
        fe[j] = (float)a.counts[e] * inv_pairs;
        v[j] = lane + 64 * j < a.E ? (a.logit_split > 1 ? x0 + x1 : x0) + b : -INFINITY;
    }
    ej = ej < 0 ? 0 : (ej >= a.E ? a.E - 1 : ej);
    float dwj = dpart[0], dsv = spart[0];
#pragma unroll
    for (int i = 1; i < U; ++i) {
        if (i < nr) dwj += dpart[i];
        if (i < ns) dsv += spart[i];
    }
    for (int i = U; i < nr; ++i) dwj += a.dwp[pj * st + i];
    for (int i = U; i < ns; ++i) dsv += a.ds[t * st + i];
    if (!pl) wj = dwj = 0.f;
    if (a.Fs == 0) dsv = sg = 0.f;
    float m = v[0];
#pragma unroll
    for (int j = 1; j < NS; ++j) m = fmaxf(m, v[j]);
    for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, kWave));
    float z = 0.f;
#pragma unroll
    for (int j = 0; j < NS; ++j) {
        v[j] = lane + 64 * j < a.E ? __expf(v[j] - m) : 0.f;
        z += v[j];
    }
    z = wave_sum(z);
    const float rz = 1.0f / z;
    float fp = 0.f;
#pragma unroll
    for (int j = 0; j < NS; ++j) {
        v[j] *= rz;  // 0 past E
        fp = fmaf(fe[j], v[j], fp);
    }
    fp = wave_sum(fp);
    const float c = a.coef * (float)a.E / (float)a.T;
#pragma unroll
    for (int j = 0; j < NS; ++j) v[j] = c * v[j] * (fe[j] - fp);
    // the selected experts' terms w_j (dw_j - sum_i w_i dw_i), added in slot
    // order (a repeated expert takes its terms in that order)
    float wdw = wj * dwj;
    for (int o = 32; o >= 1; o >>= 1) wdw += __shfl_xor(wdw, o, kWave);
    const float term = wj * (dwj - wdw);
    for (int jj = 0; jj < a.k; ++jj) {
        const int e = __shfl(ej, jj, kWave);
        const float tv = __shfl(term, jj, kWave);
        if ((e & 63) == lane) {
#pragma unroll
            for (int j = 0; j < NS; ++j)
                if (j == (e >> 6)) v[j] += tv;
        }
    }
    if (lane == 0) a.q[t] = fp;
    const float dgate = a.Fs > 0 ? dsv * sg * (1.0f - sg) : 0.f;
    Tv *out = static_cast<Tv *>(a.dl) + t * a.ldd;
    for (int e = lane; e < a.ldd; e += 64) {
        const int j = e >> 6;
        float x = 0.f;
#pragma unroll
        for (int jj = 0; jj < NS; ++jj)
            if (jj == j) x = v[jj];
        if (e >= a.E) x = e == a.E ? dgate : 0.f;
        if constexpr (sizeof(Tv) == 2) out[e] = f32_to_bf16_rne(x);
        else out[e] = x;
    }
}

// dx[t] = sum_j dXp[row(t, j)] + dXs[t] + dXr[t], binary32, slot order.
template <typename Tv>
__global__ __launch_bounds__(256) void dx_combine_kernel(BwdArgs a) {
    const int64_t t = blockIdx.x;
    const int c = blockIdx.y * 256 + threadIdx.x;
    if (c >= a.d) return;
    float acc = 0.f;
    const Tv *dxp = static_cast<const Tv *>(a.dxp);
    for (int jj = 0; jj < a.k; ++jj)
        acc += to_f32(dxp[(int64_t)a.rank[t * a.k + jj] * a.d + c]);
    if (a.Fs > 0) acc += to_f32(static_cast<const Tv *>(a.dxs)[t * a.d + c]);
    acc += a.dxr[t * a.d + c];
    a.dx[t * a.d + c] = acc;
}

// The same for bfloat16 layers (d % 8 == 0), eight columns per thread: block
// (t, c) handles token t and columns 512 c .. 512 c + 511.
__global__ __launch_bounds__(64) void dx_combine_bf16_kernel(BwdArgs a) {
    const int64_t t = blockIdx.x;
    const int c = (blockIdx.y * 64 + threadIdx.x) * 8;
    if (a.aux_loss && blockIdx.x == 0 && blockIdx.y == 0) {
        // the load-balancing loss, coef E / T sum_t q_t, summed in a fixed
        // order by this one block (a launch of its own cost more than the
        // sum; the other blocks of the grid run meanwhile)
        float sq = 0.f;
        for (int64_t u = threadIdx.x; u < a.T; u += 64) sq += a.q[u];
        sq = wave_sum(sq);
        if (threadIdx.x == 0) a.aux_loss[0] = a.coef * (float)a.E / (float)a.T * sq;
    }
    if (c >= a.d) return;
    float acc[8], v[8], vs[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.f;
    // the shared expert's and the router's terms are loaded first; the pair
    // rows in groups of four, every load of a group before its adds; the adds
    // keep the order rows (slot order), shared, router
    if (a.Fs > 0) load8(static_cast<const uint16_t *>(a.dxs) + t * a.d + c, vs);
    load8(a.dxr + t * a.d + c, v);
    const uint16_t *dxp = static_cast<const uint16_t *>(a.dxp);
    constexpr int G = 4;
    for (int j0 = 0; j0 < a.k; j0 += G) {
        uint4 q[G];
#pragma unroll
        for (int u = 0; u < G; ++u) {
            const int jj = min(j0 + u, a.k - 1);  // the tail re-reads the last row, unused
            q[u] = *reinterpret_cast<const uint4 *>(dxp + (int64_t)a.rank[t * a.k + jj] * a.d + c);
        }
#pragma unroll
        for (int u = 0; u < G; ++u) {
            if (j0 + u >= a.k) break;
            const uint32_t w4[4] = {q[u].x, q[u].y, q[u].z, q[u].w};
#pragma unroll
            for (int i = 0; i < 8; ++i)
                acc[i] += (i & 1) ? bf16_hi(w4[i >> 1]) : bf16_lo(w4[i >> 1]);
        }
    }
    if (a.Fs > 0) {
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] += vs[i];
    }
    float *o = a.dx + t * a.d + c;
    reinterpret_cast<float4 *>(o)[0] = make_float4(acc[0] + v[0], acc[1] + v[1], acc[2] + v[2],
                                                   acc[3] + v[3]);
    reinterpret_cast<float4 *>(o)[1] = make_float4(acc[4] + v[4], acc[5] + v[5], acc[6] + v[6],
                                                   acc[7] + v[7]);
}

// L_aux = coef (E / T) sum_t q_t (q_t = f . p_t), one block, fixed order.
__global__ __launch_bounds__(256) void aux_loss_kernel(BwdArgs a) {
    __shared__ float red[4];
    float s = 0.f;
    for (int64_t t = threadIdx.x; t < a.T; t += 256) s += a.q[t];
    s = block_sum(s, red);
    if (threadIdx.x == 0) a.aux_loss[0] = a.coef * (float)a.E / (float)a.T * s;
}

// ---------------------------------------------------------------------------

// nx row tiles (weight gradients: groups x row tiles per group) by ny column
// tiles.
// max_blocks > 0 caps the grid (the blocks then stride over the tiles).
template <int KIND>
static void launch_gemm(const BwdArgs &a, unsigned nx, unsigned ny, hipStream_t s,
                        int groups = 1, unsigned max_blocks = 0) {
    if (nx == 0 || ny == 0) return;
    const unsigned nvirt = bwd_blocks(KIND, (int)nx, (int)ny, groups);
    const unsigned grid = max_blocks && max_blocks < nvirt ? max_blocks : nvirt;
    if (!a.bf16)
        hipLaunchKernelGGL(bwd_gemm_f32_kernel<KIND>, dim3(nx, ny), dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL(bwd_gemm_kernel<KIND>, dim3(grid), dim3(256), 0, s, a, (int)nx,
                           (int)ny, groups, (int)nvirt);
}

// dW_router (rows 0 .. E-1) and the shared gate's gradient (row E, when a
// shared expert exists and its output is given) from the token chunks'
// binary32 partials (partial sp at part + sp pstride, rows of d): summed in
// chunk order, rounded to bf16.
__global__ __launch_bounds__(256) void dwr_reduce_kernel(const float *__restrict__ part, int S,
                                                         int64_t pstride, int E, int d, int rows,
                                                         uint16_t *__restrict__ dw_router,
                                                         uint16_t *__restrict__ dsh_gate) {
    const int64_t n = (int64_t)rows * d;
    const int64_t i = 4 * ((int64_t)blockIdx.x * 256 + threadIdx.x);
    if (i >= n) return;
    float4 acc = *reinterpret_cast<const float4 *>(part + i);
    for (int sp = 1; sp < S; ++sp) {
        const float4 v = *reinterpret_cast<const float4 *>(part + (int64_t)sp * pstride + i);
        acc.x += v.x;
        acc.y += v.y;
        acc.z += v.z;
        acc.w += v.w;
    }
    uint2 q;
    q.x = pack_bf16x2(acc.x, acc.y);
    q.y = pack_bf16x2(acc.z, acc.w);
    // d % 4 == 0: the four values share a row
    if (i < (int64_t)E * d) *reinterpret_cast<uint2 *>(dw_router + i) = q;
    else if (dsh_gate) *reinterpret_cast<uint2 *>(dsh_gate + (i - (int64_t)E * d)) = q;
}

// Shared expert's weight gradient from its split reduction: out = the sum of
// the S binary32 partials in chunk order, rounded to bf16.
__global__ __launch_bounds__(256) void sh_reduce_kernel(const float *__restrict__ part, int S,
                                                        int64_t n, uint16_t *__restrict__ out) {
    const int64_t i = 4 * ((int64_t)blockIdx.x * 256 + threadIdx.x);
    if (i >= n) return;
    float4 acc = *reinterpret_cast<const float4 *>(part + i);
    for (int sp = 1; sp < S; ++sp) {
        const float4 v = *reinterpret_cast<const float4 *>(part + (int64_t)sp * n + i);
        acc.x += v.x;
        acc.y += v.y;
        acc.z += v.z;
        acc.w += v.w;
    }
    uint2 q;
    q.x = pack_bf16x2(acc.x, acc.y);
    q.y = pack_bf16x2(acc.z, acc.w);
    *reinterpret_cast<uint2 *>(out + i) = q;
}

static unsigned cdiv(int64_t a, int64_t b) { return (unsigned)((a + b - 1) / b); }

// The router backward for E <= 64 NS (E <= 1024).
template <typename Tv> static hipError_t launch_router_bwd(const BwdArgs &a, hipStream_t s) {
    const dim3 grid(cdiv(a.T, 4)), block(256);
    const int slots = (a.E + 63) / 64;
    if (slots <= 1) hipLaunchKernelGGL((router_bwd_kernel<Tv, 1>), grid, block, 0, s, a);
    else if (slots <= 2) hipLaunchKernelGGL((router_bwd_kernel<Tv, 2>), grid, block, 0, s, a);
    else if (slots <= 4) hipLaunchKernelGGL((router_bwd_kernel<Tv, 4>), grid, block, 0, s, a);
    else if (slots <= 8) hipLaunchKernelGGL((router_bwd_kernel<Tv, 8>), grid, block, 0, s, a);
    else if (slots <= 16) hipLaunchKernelGGL((router_bwd_kernel<Tv, 16>), grid, block, 0, s, a);
    else return hipErrorInvalidValue;
    return hipSuccess;
}

hipError_t launch_backward(const Problem &pp, const BwdArgs &a, hipStream_t s,
                           const std::function<void(int)> &mark) {
    hipError_t err = a.counts_given ? launch_permute_tiles(pp, a.counts_given, QB, s)
                                    : launch_permute(pp, QB, s);
    if (err != hipSuccess) return err;
    const int Fmax = a.F > a.Fs ? a.F : a.Fs;
    const unsigned tiles = (unsigned)pp.max_tiles;
    if (!a.logits_given)
        launch_gemm<K_LOGITS>(a, cdiv(a.T, QB), cdiv(a.E + 1, QB) * a.logit_split, s);
    mark(1);
    if (!a.au_given) launch_gemm<K_AU>(a, tiles, cdiv(2 * Fmax, QB), s);
    // G rounds dOut to bf16 once (dob), for itself and for the
    // down-projection weight gradients; on the direct-to-LDS tiles the
    // SwiGLU backward runs in its epilogue (G . h as partial sums per 128
    // columns), elsewhere in a kernel of its own that reads G
    const bool dma = bwd_dma_ok(a);
    BwdArgs ag = a;
    ag.gtile = dma ? (int)cdiv(Fmax, 128) : 0;
    if (dma) {
        err = launch_bwd_g_dma(ag, (int)tiles, a.dob, s);
        if (err != hipSuccess) return err;
    } else {
        launch_gemm<K_G>(a, tiles, cdiv(Fmax, QB), s);
    }
    mark(2);
    const int64_t rows = (int64_t)a.T * a.k + (a.Fs > 0 ? a.T : 0);
    if (a.bf16) {
        if (!dma)
            hipLaunchKernelGGL(swiglu_bwd_kernel<uint16_t>, dim3(cdiv(rows, 4)), dim3(256), 0, s,
                               ag);
        err = launch_router_bwd<uint16_t>(ag, s);
    } else {
        hipLaunchKernelGGL(swiglu_bwd_kernel<float>, dim3(cdiv(rows, 4)), dim3(256), 0, s, ag);
        err = launch_router_bwd<float>(ag, s);
    }
    if (err != hipSuccess) return err;
    mark(3);
    if (dma) {
        err = launch_bwd_dx_dma(a, (int)tiles, s);
        if (err != hipSuccess) return err;
    } else {
        launch_gemm<K_DX>(a, tiles, cdiv(a.d, QB), s);
    }
    mark(4);
    // The weight gradients reduce over one expert's rows: experts (and a
    // shared expert over T <= KS tokens) with at most KS rows in the
    // short-reduction kernel, the rest in the tiled one; the shared expert
    // over more tokens splits its reduction into sh_split chunks.
    BwdArgs ab = a;
    ab.dw_kmin = a.bf16 ? KS : -1;
    const int g_small = a.E + (a.Fs > 0 && a.sh_split == 0 ? 1 : 0);
    const int g_all = a.E + (a.Fs > 0 ? (a.sh_split > 0 ? a.sh_split : 1) : 0);
    const unsigned gu_m = cdiv(2 * Fmax, QB), dn_m = cdiv(a.d, QB);
    if (a.bf16)
        hipLaunchKernelGGL(bwd_dw_small_kernel<K_DWGU>,
                           dim3(bwd_blocks(K_DWGU, g_small * gu_m, 1, g_small)), dim3(256), 0, s,
                           a, (int)(g_small * gu_m), g_small);
    // most groups were done above: a capped grid strides over the tile map
    // (the routed groups only when the shared expert's token chunks run on
    // the direct-to-LDS tiles)
    // one round of the two blocks per CU that fit: enough to fill the chip
    // for the grid-stride walk, and few when there is nothing to do (the
    // usual case when the shared expert runs on the direct-to-LDS tiles)
    int dev = 0, ncu = 256;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        ncu <= 0)
        ncu = 256;
    const unsigned cap = 8u * (unsigned)((ncu + 3) / 4);  // 2 ncu, a multiple of 8 (XCD order)
    const bool wsh = bwd_wsh_dma_ok(a);
    const int g_tiled = wsh ? a.E : g_all;
    launch_gemm<K_DWGU>(ab, g_tiled * gu_m, cdiv(a.d, QB), s, g_tiled, cap);
    int parts = a.sh_split;  // binary32 partials of the shared expert's gradient
    if (wsh) {
        err = launch_bwd_wsh_dma(a, false, s, &parts);
        if (err != hipSuccess) return err;
    }
    if (a.sh_split > 0) {
        const int64_t n = (int64_t)2 * a.Fs * a.d;
        hipLaunchKernelGGL(sh_reduce_kernel, dim3(cdiv(n / 4, 256)), dim3(256), 0, s, a.part,
                           parts, n, static_cast<uint16_t *>(a.dw_sgu));
    }
    mark(5);
    if (bwd_dwdn_stream_ok(a)) {
        err = launch_bwd_dwdn_stream(a, s);
        if (err != hipSuccess) return err;
    } else if (a.bf16) {
        hipLaunchKernelGGL(bwd_dw_small_kernel<K_DWDN>,
                           dim3(bwd_blocks(K_DWDN, g_small * dn_m, 1, g_small)), dim3(256), 0, s,
                           a, (int)(g_small * dn_m), g_small);
    }
    launch_gemm<K_DWDN>(ab, g_tiled * dn_m, cdiv(Fmax, QB), s, g_tiled, cap);
    parts = a.sh_split;
    if (wsh) {
        err = launch_bwd_wsh_dma(a, true, s, &parts);
        if (err != hipSuccess) return err;
    }
    if (a.sh_split > 0) {
        const int64_t n = (int64_t)a.d * a.Fs;
        hipLaunchKernelGGL(sh_reduce_kernel, dim3(cdiv(n / 4, 256)), dim3(256), 0, s, a.part,
                           parts, n, static_cast<uint16_t *>(a.dw_sdn));
    }
    mark(6);
    // dW_router reduces over all T tokens on few tiles: at larger T in token
    // chunks, their binary32 partials in part (free again: its last reader ran)
    BwdArgs ar = a;
    ar.dwr_split = 1;
    const int rrows = a.E + (a.Fs > 0 ? 1 : 0);  // router rows (row E: the shared gate)
    if (a.bf16 && a.T >= 1024 && a.d % 4 == 0 && a.sh_split > 0) {
        const int64_t cap = (int64_t)a.sh_split * 2 * a.Fs;  // rows of d binary32 in part
        ar.dwr_split = (int)std::min<int64_t>(4, cap / (a.E + 1));
        if (ar.dwr_split < 2) ar.dwr_split = 1;
    }
    if (bwd_dwr_dma_ok(a)) {
        // on the direct-to-LDS split-K tiles (both operands token-major)
        int parts = 1;
        err = launch_bwd_dwr_dma(a, s, &parts);
        if (err != hipSuccess) return err;
        const int64_t n = (int64_t)rrows * a.d;
        hipLaunchKernelGGL(dwr_reduce_kernel, dim3(cdiv(n / 4, 256)), dim3(256), 0, s, a.part,
                           parts, (int64_t)a.ldd * a.d, a.E, a.d, rrows,
                           static_cast<uint16_t *>(a.dw_router), static_cast<uint16_t *>(a.dsh_gate));
    } else {
        launch_gemm<K_DWR>(ar, cdiv(a.E + 1, QB), cdiv(a.d, QB) * ar.dwr_split, s);
        if (ar.dwr_split > 1) {
            const int64_t n = (int64_t)rrows * a.d;
            hipLaunchKernelGGL(dwr_reduce_kernel, dim3(cdiv(n / 4, 256)), dim3(256), 0, s, a.part,
                               ar.dwr_split, n, a.E, a.d, rrows,
                               static_cast<uint16_t *>(a.dw_router),
                               static_cast<uint16_t *>(a.dsh_gate));
        }
    }
    launch_gemm<K_DXR>(a, cdiv(a.T, QB), cdiv(a.d, QB), s);
    if (a.bf16)
        hipLaunchKernelGGL(dx_combine_bf16_kernel, dim3((unsigned)a.T, cdiv(a.d / 8, 64)), dim3(64),
                           0, s, a);
    else
        hipLaunchKernelGGL(dx_combine_kernel<float>, dim3((unsigned)a.T, cdiv(a.d, 256)),
                           dim3(256), 0, s, a);
    // (bf16 layers: the loss comes from the dx combine's first block)
    if (a.aux_loss && !a.bf16) hipLaunchKernelGGL(aux_loss_kernel, dim3(1), dim3(256), 0, s, a);
    mark(7);
    return hipGetLastError();
}

}  // namespace moe
