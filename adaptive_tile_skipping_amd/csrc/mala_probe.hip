// Measurement probes: what this part sustains, for reading the roofline
// figures of the attention kernels against the part as well as against its
// published peaks.  They compute nothing of the attention method.
//
// - mala_probe_mfma: every wave of a full grid (two 4-wave workgroups per
//   compute unit, the forward's occupancy) issues back-to-back 32x32x16 bf16
//   MFMAs on register operands, four independent accumulators per wave, with
//   no memory traffic.  Its rate is the bf16 MFMA rate at the clock the part
//   holds under that load.
// - mala_probe_read: a grid-stride streaming read of device memory (16-byte
//   loads, eight in flight per lane, one 8-wave workgroup per compute unit).
//   Its rate over a buffer larger than the last-level cache is the HBM read
//   bandwidth a plain kernel reaches.
#include "../../include/mala.h"
#include "mala_device.h"

namespace mala {
namespace {

constexpr int kProbeChains = 4;       // independent accumulators per wave
constexpr int kProbeReadUnroll = 8;   // 16-byte loads in flight per lane

int probe_cus() {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    return n;
}

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void probe_mfma_kernel(int iters, float* sink) {
    const int lane = threadIdx.x & 63;
    bf16x8 a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        a[e] = to_bf16(1e-3f * (float)(lane + e));
        b[e] = to_bf16(1e-3f * (float)(lane - e));
    }
    f32x16 c[kProbeChains];
#pragma unroll
    for (int j = 0; j < kProbeChains; ++j) c[j] = f32x16{};
#pragma unroll 4
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < kProbeChains; ++j) c[j] = mfma32x32x16(a, b, c[j]);
    }
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < kProbeChains; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) s += c[j][r];
    // one value per wave keeps every MFMA live
    if (lane == 0) sink[blockIdx.x * (blockDim.x / 64) + (threadIdx.x >> 6)] = s;
}

__global__ __launch_bounds__(512) void probe_read_kernel(const u32x4* src, int64_t n16, uint32_t* sink) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    u32x4 acc = {0u, 0u, 0u, 0u};
    for (; i + (kProbeReadUnroll - 1) * stride < n16; i += kProbeReadUnroll * stride) {
        u32x4 x[kProbeReadUnroll];
#pragma unroll
        for (int u = 0; u < kProbeReadUnroll; ++u) x[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
        for (int u = 0; u < kProbeReadUnroll; ++u) acc ^= x[u];
    }
    for (; i < n16; i += stride) acc ^= src[i];
    // one word per thread keeps every load live
    sink[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
}

}  // namespace
}  // namespace mala

extern "C" {

mala_status mala_probe_mfma(int iters, float* sink, void* stream) {
    if (iters < 1 || !sink) return MALA_ERR_INVALID_ARG;
    const int cus = mala::probe_cus();
    if (cus <= 0 || 2 * cus * 4 > MALA_PROBE_SINK_WORDS) return MALA_ERR_HIP;
    hipLaunchKernelGGL(mala::probe_mfma_kernel, dim3(2 * cus), dim3(256), 0, (hipStream_t)stream, iters, sink);
    return hipGetLastError() == hipSuccess ? MALA_OK : MALA_ERR_HIP;
}

double mala_probe_mfma_flop(int iters) {
    const int cus = mala::probe_cus();
    return (double)cus * 2 * 4 * mala::kProbeChains * (double)iters * (2.0 * 32 * 32 * 16);
}

mala_status mala_probe_read(const void* src, size_t bytes, uint32_t* sink, void* stream) {
    if (!src || !sink || bytes < 16 || bytes % 16 != 0 || ((uintptr_t)src & 15u) != 0) return MALA_ERR_INVALID_ARG;
    const int cus = mala::probe_cus();
    if (cus <= 0 || cus * 512 > MALA_PROBE_SINK_WORDS) return MALA_ERR_HIP;
    hipLaunchKernelGGL(mala::probe_read_kernel, dim3(cus), dim3(512), 0, (hipStream_t)stream,
                       (const mala::u32x4*)src, (int64_t)(bytes / 16), sink);
    return hipGetLastError() == hipSuccess ? MALA_OK : MALA_ERR_HIP;
}

}  // extern "C"
