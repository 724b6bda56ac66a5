// permute.hip -- per-expert histogram, prefix scan and stable token
// permutation, plus the tile map of the grouped GEMMs.
//
// After routing every token t holds k (token, slot) pairs, pair id t*k+j,
// each naming one expert.  The expert GEMMs want the pairs of one expert in
// consecutive rows.  Row r of expert e lies in [offsets[e], offsets[e]+counts[e])
// and rows of one expert are in ascending pair id, so the permutation is
// deterministic (no atomics decide an order):
//   count:   blocks of 256 tokens set one bit per (expert, token) in LDS;
//            a pair's rank inside its block is a popcount of the lower bits;
//   scan:    per expert, exclusive prefix of the block counts; across experts,
//            exclusive prefix of the totals (offsets) and of the tile counts;
//   scatter: perm[offsets[e] + block_base[e] + rank] = pair id, and the
//            pair's row is kept for the combine.
// Every row a block reserves is written by some pair, so perm never holds
// stale entries, even when a routing given from outside repeats an expert
// within one token (that pair's copies then share one row).
#include "moe_device.h"
#include "moe_kernels.h"

namespace moe {

__device__ __forceinline__ int clamp_expert(int e, int E) { return e < 0 ? 0 : (e >= E ? E - 1 : e); }

constexpr int kWords = kCountBlock / 32;

__global__ __launch_bounds__(kCountBlock) void route_count_kernel(
    const int32_t *__restrict__ topk_idx, int64_t ntok, int k, int E, int nblk,
    int32_t *__restrict__ rank, int32_t *__restrict__ blk) {
    extern __shared__ uint32_t bits[];  // [E][kWords]
    for (int i = threadIdx.x; i < E * kWords; i += kCountBlock) bits[i] = 0;
    __syncthreads();
    const int64_t t = (int64_t)blockIdx.x * kCountBlock + threadIdx.x;
    const bool valid = t < ntok;
    const int word = threadIdx.x >> 5;
    const uint32_t bit = 1u << (threadIdx.x & 31);
    if (valid)
        for (int j = 0; j < k; ++j)
            atomicOr(&bits[clamp_expert(topk_idx[t * k + j], E) * kWords + word], bit);
    __syncthreads();
    if (valid)
        for (int j = 0; j < k; ++j) {
            const uint32_t *b = bits + clamp_expert(topk_idx[t * k + j], E) * kWords;
            int r = __popc(b[word] & (bit - 1u));
            for (int w = 0; w < word; ++w) r += __popc(b[w]);
            rank[t * k + j] = r;
        }
    for (int e = threadIdx.x; e < E; e += kCountBlock) {
        int c = 0;
#pragma unroll
        for (int w = 0; w < kWords; ++w) c += __popc(bits[e * kWords + w]);
        blk[(int64_t)e * nblk + blockIdx.x] = c;
    }
}

// Block-wide exclusive scan of one int per thread (1024 threads).
__device__ int block_exclusive_scan(int v, int *total) {
    __shared__ int warp_sums[16];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int incl = v;
    for (int o = 1; o < 64; o <<= 1) {
        int n = __shfl_up(incl, o, kWave);
        if (lane >= o) incl += n;
    }
    if (lane == 63) warp_sums[wave] = incl;
    __syncthreads();
    int before = 0, all = 0;
    for (int w = 0; w < 16; ++w) {
        if (w < wave) before += warp_sums[w];
        all += warp_sums[w];
    }
    __syncthreads();
    *total = all;
    return before + incl - v;
}

// One block of 1024 threads; thread e owns expert e (E <= 1024).
__global__ __launch_bounds__(1024) void route_scan_kernel(int32_t *__restrict__ blk, int nblk,
                                                          int E, int64_t ntok, int bm,
                                                          int has_shared,
                                                          int32_t *__restrict__ counts,
                                                          int32_t *__restrict__ offsets,
                                                          int32_t *__restrict__ tile_start,
                                                          int32_t *__restrict__ tile_group) {
    const int e = threadIdx.x;
    int total = 0;
    if (e < E) {
        int32_t *col = blk + (int64_t)e * nblk;
        int b = 0;
        for (; b + 8 <= nblk; b += 8) {
            int c[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) c[i] = col[b + i];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                col[b + i] = total;
                total += c[i];
            }
        }
        for (; b < nblk; ++b) {
            int c = col[b];
            col[b] = total;
            total += c;
        }
        counts[e] = total;
    }
    const int tiles = e < E ? (total + bm - 1) / bm : 0;
    int all_rows, all_tiles;
    const int off = block_exclusive_scan(e < E ? total : 0, &all_rows);
    const int ts = block_exclusive_scan(tiles, &all_tiles);
    if (e < E) {
        offsets[e] = off;
        tile_start[e] = ts;
        for (int i = 0; i < tiles; ++i) tile_group[ts + i] = e;
    }
    if (e == 0) {
        offsets[E] = all_rows;
        counts[E] = (int)ntok;
        tile_start[E] = all_tiles;
        tile_start[E + 1] = all_tiles + (has_shared ? (int)((ntok + bm - 1) / bm) : 0);
    }
    if (has_shared) {
        const int shared_tiles = (int)((ntok + bm - 1) / bm);
        for (int i = threadIdx.x; i < shared_tiles; i += 1024) tile_group[all_tiles + i] = E;
    }
}

// Also turns rank[pair] into the pair's row, for the combine.
__global__ __launch_bounds__(kCountBlock) void route_scatter_kernel(
    const int32_t *__restrict__ topk_idx, int64_t ntok, int k, int E, int nblk,
    int32_t *__restrict__ rank, const int32_t *__restrict__ blk,
    const int32_t *__restrict__ offsets, int32_t *__restrict__ perm) {
    const int64_t t = (int64_t)blockIdx.x * kCountBlock + threadIdx.x;
    if (t >= ntok) return;
    for (int j = 0; j < k; ++j) {
        const int e = clamp_expert(topk_idx[t * k + j], E);
        const int pos = offsets[e] + blk[(int64_t)e * nblk + blockIdx.x] + rank[t * k + j];
        perm[pos] = (int32_t)(t * k + j);
        rank[t * k + j] = pos;
    }
}

// All of the above in one block of 1024 threads when every token fits one
// histogram block (T <= 256): no block prefix is needed and one launch
// replaces three.  topk points at the routing (global memory or LDS); bits
// is [E][kWords] and s_off [E], both in LDS.
__device__ __forceinline__ void permute_small(const int32_t *topk, int ntok, int k, int E, int bm,
                                              int has_shared, uint32_t *bits, int32_t *s_off,
                                              int32_t *__restrict__ counts,
                                              int32_t *__restrict__ offsets,
                                              int32_t *__restrict__ tile_start,
                                              int32_t *__restrict__ tile_group,
                                              int32_t *__restrict__ row_of,
                                              int32_t *__restrict__ perm) {
    const int t = threadIdx.x;
    const bool valid = t < ntok;
    const int word = t >> 5;
    const uint32_t bit = 1u << (t & 31);
    if (valid)
        for (int j = 0; j < k; ++j)
            atomicOr(&bits[clamp_expert(topk[t * k + j], E) * kWords + word], bit);
    __syncthreads();
    const int e = threadIdx.x;
    int total = 0;
    if (e < E) {
#pragma unroll
        for (int w = 0; w < kWords; ++w) total += __popc(bits[e * kWords + w]);
        counts[e] = total;
    }
    const int tiles = e < E ? (total + bm - 1) / bm : 0;
    int all_rows, all_tiles;
    const int off = block_exclusive_scan(e < E ? total : 0, &all_rows);
    const int ts = block_exclusive_scan(tiles, &all_tiles);
    if (e < E) {
        offsets[e] = off;
        s_off[e] = off;
        tile_start[e] = ts;
        for (int i = 0; i < tiles; ++i) tile_group[ts + i] = e;
    }
    if (e == 0) {
        offsets[E] = all_rows;
        counts[E] = ntok;
        tile_start[E] = all_tiles;
        tile_start[E + 1] = all_tiles + (has_shared ? (ntok + bm - 1) / bm : 0);
    }
    if (has_shared)
        for (int i = threadIdx.x; i < (ntok + bm - 1) / bm; i += 1024) tile_group[all_tiles + i] = E;
    __syncthreads();
    if (valid)
        for (int j = 0; j < k; ++j) {
            const int ee = clamp_expert(topk[t * k + j], E);
            const uint32_t *b = bits + ee * kWords;
            int r = __popc(b[word] & (bit - 1u));
            for (int w = 0; w < word; ++w) r += __popc(b[w]);
            const int pos = s_off[ee] + r;
            perm[pos] = t * k + j;
            row_of[t * k + j] = pos;
        }
}

__global__ __launch_bounds__(1024) void route_permute_small_kernel(
    const int32_t *__restrict__ topk_idx, int ntok, int k, int E, int bm, int has_shared,
    int32_t *__restrict__ counts, int32_t *__restrict__ offsets, int32_t *__restrict__ tile_start,
    int32_t *__restrict__ tile_group, int32_t *__restrict__ row_of, int32_t *__restrict__ perm) {
    extern __shared__ uint32_t bits[];  // [E][kWords], then offsets [E]
    int32_t *s_off = reinterpret_cast<int32_t *>(bits + E * kWords);
    for (int i = threadIdx.x; i < E * kWords; i += 1024) bits[i] = 0;
    __syncthreads();
    permute_small(topk_idx, ntok, k, E, bm, has_shared, bits, s_off, counts, offsets, tile_start,
                  tile_group, row_of, perm);
}

// Offsets and the tile map of tile height bm from given per-expert counts
// (a permutation whose rank and perm are already there), as the scan step
// derives them.
__global__ __launch_bounds__(1024) void route_tiles_kernel(const int32_t *__restrict__ cnt, int E,
                                                           int64_t ntok, int bm, int has_shared,
                                                           int32_t *__restrict__ counts,
                                                           int32_t *__restrict__ offsets,
                                                           int32_t *__restrict__ tile_start,
                                                           int32_t *__restrict__ tile_group) {
    const int e = threadIdx.x;
    const int total = e < E ? cnt[e] : 0;
    if (e < E) counts[e] = total;
    const int tiles = e < E ? (total + bm - 1) / bm : 0;
    int all_rows, all_tiles;
    const int off = block_exclusive_scan(e < E ? total : 0, &all_rows);
    const int ts = block_exclusive_scan(tiles, &all_tiles);
    if (e < E) {
        offsets[e] = off;
        tile_start[e] = ts;
        for (int i = 0; i < tiles; ++i) tile_group[ts + i] = e;
    }
    if (e == 0) {
        offsets[E] = all_rows;
        counts[E] = (int)ntok;
        tile_start[E] = all_tiles;
        tile_start[E + 1] = all_tiles + (has_shared ? (int)((ntok + bm - 1) / bm) : 0);
    }
    if (has_shared) {
        const int shared_tiles = (int)((ntok + bm - 1) / bm);
        for (int i = threadIdx.x; i < shared_tiles; i += 1024) tile_group[all_tiles + i] = E;
    }
}

hipError_t launch_permute_tiles(const Problem &p, const int32_t *counts_in, int bm, hipStream_t s) {
    hipLaunchKernelGGL(route_tiles_kernel, dim3(1), dim3(1024), 0, s, counts_in, p.E, p.T, bm,
                       p.Fs > 0 ? 1 : 0, p.counts, p.offsets, p.tile_start, p.tile_group);
    return hipGetLastError();
}

hipError_t launch_permute(const Problem &p, int bm, hipStream_t s) {
    if (p.nblk == 1) {
        const size_t lds = (size_t)p.E * (kWords + 1) * sizeof(uint32_t);
        hipLaunchKernelGGL(route_permute_small_kernel, dim3(1), dim3(1024), lds, s, p.topk_idx,
                           (int)p.T, p.k, p.E, bm, p.Fs > 0 ? 1 : 0, p.counts, p.offsets,
                           p.tile_start, p.tile_group, p.rank, p.perm);
        return hipGetLastError();
    }
    const size_t lds = (size_t)p.E * kWords * sizeof(uint32_t);
    hipLaunchKernelGGL(route_count_kernel, dim3(p.nblk), dim3(kCountBlock), lds, s, p.topk_idx,
                       p.T, p.k, p.E, p.nblk, p.rank, p.blk);
    hipLaunchKernelGGL(route_scan_kernel, dim3(1), dim3(1024), 0, s, p.blk, p.nblk, p.E, p.T, bm,
                       p.Fs > 0 ? 1 : 0, p.counts, p.offsets, p.tile_start, p.tile_group);
    hipLaunchKernelGGL(route_scatter_kernel, dim3(p.nblk), dim3(kCountBlock), 0, s, p.topk_idx,
                       p.T, p.k, p.E, p.nblk, p.rank, p.blk, p.offsets, p.perm);
    return hipGetLastError();
}

// Weighted combine in a fixed order: the shared term already in out[t]
// (written by the down-projection's shared tiles), then the routed rows in
// slot order j = 0..k-1, all in binary32.  Deterministic: no atomics.
//
// Binary32 layers and the weight-streaming path keep the routed rows y in
// binary32.  Rows of a width that
// is a multiple of 8: block (t, c) handles token t and columns 512 c .. 512 c
// + 511, eight per thread.  row_of null: the rows are indexed by pair id (the
// permutation step was skipped), row t*k+j.  resid (nullable): the caller's
// binary32 residual stream, which gets the finished output added in the same
// pass, resid[t] = resid[t] + out[t].
constexpr int kCombineGroup = 8;

__device__ __forceinline__ void add8(float (&acc)[8], const float4 &lo, const float4 &hi) {
    acc[0] += lo.x; acc[1] += lo.y; acc[2] += lo.z; acc[3] += lo.w;
    acc[4] += hi.x; acc[5] += hi.y; acc[6] += hi.z; acc[7] += hi.w;
}

template <bool SHARED>
__global__ __launch_bounds__(64) void combine_rows_kernel(const float *__restrict__ y,
                                                          const int32_t *__restrict__ row_of,
                                                          float *__restrict__ out,
                                                          float *__restrict__ resid, int d, int k) {
    const int64_t t = blockIdx.x;
    const int c = (blockIdx.y * 64 + threadIdx.x) * 8;
    if (c >= d) return;
    float acc[8];
    float *o = out + t * d + c;
    if (SHARED) {
        const float4 lo = reinterpret_cast<const float4 *>(o)[0];
        const float4 hi = reinterpret_cast<const float4 *>(o)[1];
        acc[0] = lo.x; acc[1] = lo.y; acc[2] = lo.z; acc[3] = lo.w;
        acc[4] = hi.x; acc[5] = hi.y; acc[6] = hi.z; acc[7] = hi.w;
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = 0.f;
    }
    // rows in groups of kCombineGroup, every load of a group issued before
    // the first add; the adds stay in slot order (the tail group re-reads
    // slot k - 1 for its missing slots and skips them)
    for (int j0 = 0; j0 < k; j0 += kCombineGroup) {
        float4 q[kCombineGroup][2];
#pragma unroll
        for (int u = 0; u < kCombineGroup; ++u) {
            const int j = min(j0 + u, k - 1);
            const int64_t r = row_of ? row_of[t * k + j] : t * k + j;
            const float4 *src = reinterpret_cast<const float4 *>(y + r * d + c);
            q[u][0] = src[0];
            q[u][1] = src[1];
        }
#pragma unroll
        for (int u = 0; u < kCombineGroup; ++u) {
            if (j0 + u >= k) break;
            add8(acc, q[u][0], q[u][1]);
        }
    }
    reinterpret_cast<float4 *>(o)[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
    reinterpret_cast<float4 *>(o)[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
    if (resid) {
        float4 *r = reinterpret_cast<float4 *>(resid + t * d + c);
        const float4 lo = r[0], hi = r[1];
        r[0] = make_float4(lo.x + acc[0], lo.y + acc[1], lo.z + acc[2], lo.w + acc[3]);
        r[1] = make_float4(hi.x + acc[4], hi.y + acc[5], hi.z + acc[6], hi.w + acc[7]);
    }
}

// bfloat16 layers: the same, with the routed rows in 16-bit block floating
// point (y16_pitch bytes per row: mantissas, then one exponent byte per eight
// columns); a thread's eight columns are one group.
template <bool SHARED>
__global__ __launch_bounds__(64) void combine_y16_kernel(const uint8_t *__restrict__ y,
                                                         const int32_t *__restrict__ row_of,
                                                         float *__restrict__ out,
                                                         float *__restrict__ resid, int d, int k) {
    const int64_t t = blockIdx.x;
    const int c = (blockIdx.y * 64 + threadIdx.x) * 8;
    if (c >= d) return;
    const int64_t pitch = y16_pitch(d);
    float acc[8];
    float *o = out + t * d + c;
    if (SHARED) {
        const float4 lo = reinterpret_cast<const float4 *>(o)[0];
        const float4 hi = reinterpret_cast<const float4 *>(o)[1];
        acc[0] = lo.x; acc[1] = lo.y; acc[2] = lo.z; acc[3] = lo.w;
        acc[4] = hi.x; acc[5] = hi.y; acc[6] = hi.z; acc[7] = hi.w;
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = 0.f;
    }
    for (int j0 = 0; j0 < k; j0 += kCombineGroup) {
        uint4 m[kCombineGroup];
        uint32_t x[kCombineGroup];
#pragma unroll
        for (int u = 0; u < kCombineGroup; ++u) {
            const int j = min(j0 + u, k - 1);
            const int64_t r = row_of ? row_of[t * k + j] : t * k + j;
            const uint8_t *row = y + r * pitch;
            m[u] = *reinterpret_cast<const uint4 *>(row + 2 * (int64_t)c);
            x[u] = row[2 * (int64_t)d + c / 8];
        }
#pragma unroll
        for (int u = 0; u < kCombineGroup; ++u) {
            if (j0 + u >= k) break;
            const uint32_t xu = x[u];
            acc[0] += y16_value(m[u].x & 0xFFFFu, xu);
            acc[1] += y16_value(m[u].x >> 16, xu);
            acc[2] += y16_value(m[u].y & 0xFFFFu, xu);
            acc[3] += y16_value(m[u].y >> 16, xu);
            acc[4] += y16_value(m[u].z & 0xFFFFu, xu);
            acc[5] += y16_value(m[u].z >> 16, xu);
            acc[6] += y16_value(m[u].w & 0xFFFFu, xu);
            acc[7] += y16_value(m[u].w >> 16, xu);
        }
    }
    reinterpret_cast<float4 *>(o)[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
    reinterpret_cast<float4 *>(o)[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
    if (resid) {
        float4 *r = reinterpret_cast<float4 *>(resid + t * d + c);
        const float4 lo = r[0], hi = r[1];
        r[0] = make_float4(lo.x + acc[0], lo.y + acc[1], lo.z + acc[2], lo.w + acc[3]);
        r[1] = make_float4(hi.x + acc[4], hi.y + acc[5], hi.z + acc[6], hi.w + acc[7]);
    }
}

// Any width: one block per token.
template <bool SHARED>
__global__ __launch_bounds__(128) void combine_f32_kernel(const float *__restrict__ y,
                                                          const int32_t *__restrict__ row_of,
                                                          float *__restrict__ out,
                                                          float *__restrict__ resid, int d, int k) {
    const int64_t t = blockIdx.x;
    __shared__ int32_t rows[32];
    if (threadIdx.x < k) rows[threadIdx.x] = row_of ? row_of[t * k + threadIdx.x] : (int32_t)(t * k + threadIdx.x);
    __syncthreads();
    float *o = out + t * d;
    for (int c = threadIdx.x; c < d; c += 128) {
        float acc = SHARED ? o[c] : 0.f;
        for (int j = 0; j < k; ++j) acc += y[(int64_t)rows[j] * d + c];
        o[c] = acc;
        if (resid) resid[t * d + c] += acc;
    }
}

hipError_t launch_combine(const Problem &p, hipStream_t s) {
    const int32_t *rows = p.direct ? nullptr : p.rank;
    const dim3 grid8((unsigned)p.T, (unsigned)((p.d / 8 + 63) / 64));
    if (!p.y_f32) {
        const uint8_t *y = static_cast<const uint8_t *>(p.y);
        if (p.Fs > 0)
            hipLaunchKernelGGL(combine_y16_kernel<true>, grid8, dim3(64), 0, s, y, rows, p.out,
                               p.resid, p.d, p.k);
        else
            hipLaunchKernelGGL(combine_y16_kernel<false>, grid8, dim3(64), 0, s, y, rows, p.out,
                               p.resid, p.d, p.k);
        return hipGetLastError();
    }
    const float *y = static_cast<const float *>(p.y);
    if (p.d % 8 == 0) {
        if (p.Fs > 0)
            hipLaunchKernelGGL(combine_rows_kernel<true>, grid8, dim3(64), 0, s, y, rows, p.out,
                               p.resid, p.d, p.k);
        else
            hipLaunchKernelGGL(combine_rows_kernel<false>, grid8, dim3(64), 0, s, y, rows, p.out,
                               p.resid, p.d, p.k);
    } else {
        if (p.Fs > 0)
            hipLaunchKernelGGL(combine_f32_kernel<true>, dim3((unsigned)p.T), dim3(128), 0, s, y,
                               rows, p.out, p.resid, p.d, p.k);
        else
            hipLaunchKernelGGL(combine_f32_kernel<false>, dim3((unsigned)p.T), dim3(128), 0, s, y,
                               rows, p.out, p.resid, p.d, p.k);
    }
    return hipGetLastError();
}

}  // namespace moe
