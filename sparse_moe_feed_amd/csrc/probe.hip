// probe.hip -- a plain streaming read of a device buffer, used to measure the
// practical HBM read ceiling the layer's weight-streaming kernels are judged
// against.  Not part of the layer.
//
// The whole chip reads the buffer once in coalesced 16-byte loads: block b
// streams its own contiguous share, sixteen 4 KB steps in flight (every load
// of a step group issued before the first is used); each wave folds what it
// read into one XOR word, so every load is used and the result can be
// checked.  Measured on one MI355X over 1 GiB: this shape 6.16 TB/s; a
// grid-stride loop with four loads in flight, 5.26 TB/s.
#include "moe.h"
#include "moe_device.h"

namespace {

constexpr int kProbeBlock = 256;
constexpr int kProbeWaves = MOE_READ_PROBE_SINK_WORDS;
constexpr int kProbeGrid = kProbeWaves / (kProbeBlock / moe::kWave);
constexpr int kProbeDepth = 16;

__device__ __forceinline__ uint32_t fold(uint4 v) { return v.x ^ v.y ^ v.z ^ v.w; }

__global__ __launch_bounds__(kProbeBlock) void read_probe_kernel(const uint4 *__restrict__ p,
                                                                 int64_t n, uint32_t *sink) {
    const int64_t per = (n + gridDim.x - 1) / gridDim.x;
    const int64_t lo = (int64_t)blockIdx.x * per;
    const int64_t hi = min(n, lo + per);
    int64_t i = lo + threadIdx.x;
    uint32_t acc = 0;
    for (; i + (kProbeDepth - 1) * kProbeBlock < hi; i += kProbeDepth * kProbeBlock) {
        uint4 v[kProbeDepth];
#pragma unroll
        for (int u = 0; u < kProbeDepth; ++u) v[u] = p[i + u * kProbeBlock];
#pragma unroll
        for (int u = 0; u < kProbeDepth; ++u) acc ^= fold(v[u]);
    }
    for (; i < hi; i += kProbeBlock) acc ^= fold(p[i]);
    for (int o = moe::kWave / 2; o > 0; o >>= 1) acc ^= __shfl_xor(acc, o, moe::kWave);
    if ((threadIdx.x & (moe::kWave - 1)) == 0)
        sink[blockIdx.x * (kProbeBlock / moe::kWave) + threadIdx.x / moe::kWave] = acc;
}

}  // namespace

extern "C" moe_status moe_read_probe(const void *buf, size_t bytes, uint32_t *sink, void *stream) {
    if (!buf || !sink || (reinterpret_cast<uintptr_t>(buf) & 15u) ||
        (reinterpret_cast<uintptr_t>(sink) & 3u) || bytes % 16)
        return MOE_ERR_INVALID_ARG;
    hipLaunchKernelGGL(read_probe_kernel, dim3(kProbeGrid), dim3(kProbeBlock), 0,
                       static_cast<hipStream_t>(stream), static_cast<const uint4 *>(buf),
                       (int64_t)(bytes / 16), sink);
    const hipError_t err = hipGetLastError();
    return err == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}
