// A plain read of device memory, for the benchmark only (not part of libr9k):
// the bandwidth ceiling that the weight-streaming GEMMs are compared with.
// Two access patterns over `bytes` (a multiple of 16):
//   mode 0  grid-stride: 1024 CTAs of 512 threads, each lane reads 16 bytes per
//           step, consecutive lanes consecutive bytes, 8 steps unrolled;
//   mode 1  slabs: each wave reads its own 16 KiB (16 loads of 1 KiB a wave, all
//           issued at once, as a decode wave reads its weight slice), starting at
//           load (5 w) mod 16 of its slab (w its index in the grid) and
//           wrapping; 8 waves a CTA.  Needs bytes to be a multiple of 16 KiB.
// The data are folded into one word per lane and stored only if it equals a
// value that random data practically never gives, so the loads cannot be dropped.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
constexpr uint32_t KEEP = 0x9E3779B9u;

__global__ __launch_bounds__(512) void k_read_stride(const u32x4 *__restrict__ p, int64_t n, uint32_t *out) {
    u32x4 acc = {0u, 0u, 0u, 0u};
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
#pragma unroll 8
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
        acc ^= __builtin_nontemporal_load(p + i);
    const uint32_t v = acc.x ^ acc.y ^ acc.z ^ acc.w;
    if (v == KEEP) out[threadIdx.x] = v;
}

__global__ __launch_bounds__(512) void k_read_slab(const uint8_t *__restrict__ p, int64_t nslab, uint32_t *out) {
    const int lane = threadIdx.x & 63;
    const int64_t w = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
    if (w >= nslab) return;
    const uint8_t *base = p + w * 16384 + 16 * lane;
    const int r = (int)((w * 5) & 15);
    u32x4 v[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = __builtin_nontemporal_load((const u32x4 *)(base + ((i + r) & 15) * 1024));
    u32x4 acc = v[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) acc ^= v[i];
    const uint32_t x = acc.x ^ acc.y ^ acc.z ^ acc.w;
    if (x == KEEP) out[threadIdx.x] = x;
}
}  // namespace

// out: at least 512 uint32 of device memory.  Returns 0, or -1 for a size the
// mode cannot read, or the HIP error of the launch.
extern "C" __attribute__((visibility("default"))) int r9kb_hbm_read(const void *p, int64_t bytes, int mode,
                                                                   uint32_t *out, void *stream) {
    if (!p || !out || bytes <= 0 || bytes % 16) return -1;
    if (mode == 0) {
        hipLaunchKernelGGL(k_read_stride, dim3(1024), dim3(512), 0, (hipStream_t)stream, (const u32x4 *)p,
                           bytes / 16, out);
    } else if (mode == 1) {
        if (bytes % 16384) return -1;
        const int64_t nslab = bytes / 16384;
        hipLaunchKernelGGL(k_read_slab, dim3((unsigned)((nslab + 7) / 8)), dim3(512), 0, (hipStream_t)stream,
                           (const uint8_t *)p, nslab, out);
    } else {
        return -1;
    }
    return (int)hipGetLastError();
}
