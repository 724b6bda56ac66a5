// probe.hip -- a plain streaming read of a device buffer, used to measure the
// practical HBM read ceiling the layer's weight-streaming kernels are judged
// against.  Not part of the layer.
//
// The whole chip reads the buffer once in coalesced 16-byte loads (lane i of a
// step reads bytes 16i..16i+15 of that step's 16 KB window, four steps in
// flight per lane); each wave folds what it read into one XOR word, so every
// load is used and the result can be checked.
#include "moe.h"
#include "moe_device.h"

namespace {

constexpr int kProbeBlock = 256;
constexpr int kProbeWaves = MOE_READ_PROBE_SINK_WORDS;
constexpr int kProbeGrid = kProbeWaves / (kProbeBlock / moe::kWave);

__device__ __forceinline__ uint32_t fold(uint4 v) { return v.x ^ v.y ^ v.z ^ v.w; }

__global__ __launch_bounds__(kProbeBlock) void read_probe_kernel(const uint4 *__restrict__ p,
                                                                 int64_t n, uint32_t *sink) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    uint32_t acc = 0;
    for (; i + 3 * stride < n; i += 4 * stride) {
        const uint4 a = p[i], b = p[i + stride], c = p[i + 2 * stride], d = p[i + 3 * stride];
        acc ^= fold(a) ^ fold(b) ^ fold(c) ^ fold(d);
    }
    for (; i < n; i += stride) acc ^= fold(p[i]);
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
