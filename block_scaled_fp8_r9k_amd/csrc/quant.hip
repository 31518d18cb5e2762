// Quantisation kernels: activation groups of 128 (per token along K), weight
// blocks of 128x128, and the elementwise e4m3 encoder.
//
// Activation quant is the per-token-group-128 quant of the r9700-stack release
// v0.3.1 ("What changed for someone running it"), here as its own launch (the
// split form); weight quant is the load-time conversion of release v0.3.2
// (same section).  All three are HBM-bound streaming kernels; each one's
// lane-to-data mapping is stated above it.
#include "r9k_device.h"
#include "r9k_internal.h"

namespace r9k {

// Group gid covers bf16 [gid*128, gid*128 + 128) of the row-major [M][K]
// array (row m, group g has gid = m*K/128 + g), which is also where its codes
// go; its scale goes to as[gid].  8 lanes (half a DPP row) per group, 32
// groups per 256-thread block: lane j of a group holds the 16-byte pieces j
// and j + 8, so that each load instruction reads whole 128-byte lines (8 lanes
// x 16 bytes a group) and each store writes 64 contiguous bytes of codes.
// With `transposed`, the scale of row m, group g goes to as[g*M + m] instead
// (the GEMMs read the scales of consecutive rows per group), and block b takes
// group g = b % G of the 32 rows from 32 (b / G) on: its 32 scales are then one
// 128-byte line, where in memory order (one row's G groups a block) each block
// wrote G lines 4 bytes apiece and the neighbouring rows, whose blocks run on
// other XCDs, filled the rest of each line from another L2.  Consecutive blocks
// take consecutive groups of the same rows, so that the loads and code stores
// still sweep memory in order across the grid.
__global__ __launch_bounds__(256) void k_quant_act(const uint4 *__restrict__ a, uint2 *__restrict__ aq,
                                                   float *__restrict__ as, int64_t ngroups, int64_t G, int64_t M,
                                                   bool transposed) {
    int64_t gid;
    if (transposed) {
        const int64_t m = (int64_t)(blockIdx.x / G) * 32 + (threadIdx.x >> 3);
        if (m >= M) return;  // uniform across the 8 lanes of a group
        gid = m * G + blockIdx.x % G;
    } else {
        gid = (int64_t)blockIdx.x * 32 + (threadIdx.x >> 3);
        if (gid >= ngroups) return;
    }
    const int l = threadIdx.x & 7;
    const uint4 v0 = a[gid * 16 + l], v1 = a[gid * 16 + 8 + l];
    // maximum over the group's 8 lanes: quad_perm [1,0,3,2], [2,3,0,1], then
    // row_half_mirror (lane i of each 8-lane half row reads lane 7 - i, which
    // lies in the other quad)
    uint32_t m = max(absmax8_bits(v0), absmax8_bits(v1));
    m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0xB1, 0xF, 0xF, false));
    m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0x4E, 0xF, 0xF, false));
    m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0x141, 0xF, 0xF, false));
    const float s = group_scale(__uint_as_float(m << 16));
    const float r = 1.0f / s;
    aq[gid * 16 + l] = quant8(v0, s, r);
    aq[gid * 16 + 8 + l] = quant8(v1, s, r);
    if (l == 0) as[transposed ? (gid % G) * M + gid / G : gid] = s;
}

hipError_t launch_quant_act(const uint16_t *a, int64_t M, int64_t K, uint8_t *aq, float *as, hipStream_t s,
                            bool scales_transposed) {
    const int64_t ngroups = M * (K / 128);
    const int64_t blocks = scales_transposed ? (M + 31) / 32 * (K / 128) : (ngroups + 31) / 32;
    hipLaunchKernelGGL(k_quant_act, dim3((unsigned)blocks), dim3(256), 0, s, (const uint4 *)a, (uint2 *)aq, as,
                       ngroups, K / 128, M, scales_transposed);
    return hipGetLastError();
}

// as [M][G] -> as_t [G][M], through LDS in tiles of 16 rows x 32 groups (one
// value per thread, 512 threads), so that the reads take 128-byte row pieces
// and the writes 64-byte column pieces, with enough CTAs to keep the memory
// system busy (256 for M = 4096, G = 32).  Grid: (ceil(M / 16), ceil(G / 32)).
__global__ __launch_bounds__(512) void k_transpose_scales(const float *__restrict__ as, float *__restrict__ as_t,
                                                          int64_t M, int64_t G) {
    __shared__ float tile[16][33];
    const int64_t m0 = (int64_t)blockIdx.x * 16, g0 = (int64_t)blockIdx.y * 32;
    const int t = threadIdx.x;
    {
        const int r = t >> 5, c = t & 31;
        if (m0 + r < M && g0 + c < G) tile[r][c] = as[(m0 + r) * G + g0 + c];
    }
    __syncthreads();
    {
        const int c = t >> 4, r = t & 15;
        if (m0 + r < M && g0 + c < G) as_t[(g0 + c) * M + m0 + r] = tile[r][c];
    }
}

// One thread per 16-byte chunk of the packed output (consecutive threads write
// consecutive chunks; the reads gather 16 rows).
__global__ __launch_bounds__(256) void k_pack_weight(const uint4 *__restrict__ wq, int64_t K, int64_t nchunks,
                                                     uint4 *__restrict__ wp) {
    const int64_t o = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (o >= nchunks) return;
    const int64_t G = K / 128;
    const int64_t blk = o >> 7;                  // 2 KiB block: (tile, group)
    const int h = (int)(o >> 6) & 1, l = (int)o & 63;
    const int64_t t = blk / G, g = blk % G;
    const int64_t n = t * 16 + (l & 15);
    const int64_t k = g * 128 + 64 * h + 16 * (l >> 4);
    wp[o] = wq[(n * K + k) >> 4];
}

hipError_t launch_pack_weight(const uint8_t *wq, int64_t N, int64_t K, uint8_t *wp, hipStream_t s) {
    const int64_t nchunks = N * K / 16;
    hipLaunchKernelGGL(k_pack_weight, dim3((unsigned)((nchunks + 255) / 256)), dim3(256), 0, s, (const uint4 *)wq, K,
                       nchunks, (uint4 *)wp);
    return hipGetLastError();
}

hipError_t launch_transpose_scales(const float *as, int64_t M, int64_t G, float *as_t, hipStream_t s) {
    hipLaunchKernelGGL(k_transpose_scales, dim3((unsigned)((M + 15) / 16), (unsigned)((G + 31) / 32)), dim3(512), 0,
                       s, as, as_t, M, G);
    return hipGetLastError();
}

// One 256-thread block per 128x128 weight block (grid: K/128 x N/128).
// Thread t handles rows t/16 + 16 i (i = 0..7) and columns 8 (t % 16) .. +7.
__global__ __launch_bounds__(256) void k_quant_weight(const uint16_t *__restrict__ w, int64_t K,
                                                      uint8_t *__restrict__ wq, float *__restrict__ ws) {
    const int64_t bk = blockIdx.x, bn = blockIdx.y;
    const int t = threadIdx.x;
    const int r0 = t >> 4, col = (t & 15) * 8;
    const uint16_t *blk = w + (bn * 128) * K + bk * 128 + col;
    uint4 v[8];
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        v[i] = *(const uint4 *)(blk + (int64_t)(r0 + 16 * i) * K);
        m = max(m, absmax8_bits(v[i]));
    }
    m = max16_dpp(m);
    __shared__ uint32_t red[16];
    if ((t & 15) == 0) red[t >> 4] = m;
    __syncthreads();
    uint32_t mm = red[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) mm = max(mm, red[i]);
    const float s = group_scale(__uint_as_float(mm << 16));
    const float r = 1.0f / s;
    uint8_t *qb = wq + (bn * 128) * K + bk * 128 + col;
#pragma unroll
    for (int i = 0; i < 8; ++i) *(uint2 *)(qb + (int64_t)(r0 + 16 * i) * K) = quant8(v[i], s, r);
    if (t == 0) ws[bn * (K / 128) + bk] = s;
}

hipError_t launch_quant_weight(const uint16_t *w, int64_t N, int64_t K, uint8_t *wq, float *ws, hipStream_t s) {
    hipLaunchKernelGGL(k_quant_weight, dim3((unsigned)(K / 128), (unsigned)(N / 128)), dim3(256), 0, s, w, K, wq,
                       ws);
    return hipGetLastError();
}

// Elementwise encoder: 4 values per thread, scalar tail.
__global__ __launch_bounds__(256) void k_encode_e4m3(const float *__restrict__ x, int64_t n,
                                                     uint8_t *__restrict__ out) {
    const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
    if (i + 4 <= n) {
        float4 v = *(const float4 *)(x + i);
        *(uint32_t *)(out + i) = e4m3x4(v.x, v.y, v.z, v.w);
    } else {
        for (int64_t j = i; j < n; ++j) out[j] = (uint8_t)(e4m3x4(x[j], 0.0f, 0.0f, 0.0f) & 0xFFu);
    }
}

hipError_t launch_encode_e4m3(const float *x, int64_t n, uint8_t *codes, hipStream_t s) {
    int64_t threads = (n + 3) / 4;
    int64_t blocks = (threads + 255) / 256;
    hipLaunchKernelGGL(k_encode_e4m3, dim3((unsigned)blocks), dim3(256), 0, s, x, n, codes);
    return hipGetLastError();
}

}  // namespace r9k
