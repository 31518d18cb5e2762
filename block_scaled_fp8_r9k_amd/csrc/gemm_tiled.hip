// Engine (b): the LDS-tiled block-scaled fp8 MFMA GEMM for prefill widths.
//
// The pages' tiled fp8 GEMMs take every row count above the decode kernels'
// 255 (r9700-stack release v0.3.2, "What changed for someone running it"), and
// their exact block-scaled variant (release v0.3.0, same section) is the
// semantics kept here: the K loop steps one 128-wide group at a time, and each
// group's MFMA sum is promoted with its own scales, acc += P * as[m,g] * ws[n/128,g].
//
// Activations arrive pre-quantised (codes + scales): at these widths the
// fused entry point quantises A once per call in a streaming pre-pass instead
// of once per column tile, which would cost more VALU time than the MFMAs.
//
// CTA tile: 128 output columns (one weight block row, so one ws per group)
// x 128 rows; 4 waves in 2 x 2, each 64 n x 64 m = 4 x 4 MFMA tiles of
// 16 x 16 x 128.  Both operand tiles are [128 rows][128 bytes] in LDS, double
// buffered (2 x 32 KiB); the next group's tiles are loaded into registers
// while the current one is multiplied.  The 16-byte chunk c of row r is stored
// at chunk c ^ ((r >> 1) & 7), so the 16 rows a lane column reads, and the
// 2 rows x 8 chunks a store instruction writes, fall on distinct banks.
#include <mutex>

#include "r9k_device.h"
#include "r9k_internal.h"

namespace r9k {

namespace {
constexpr int BN = 128, BM = 128;
constexpr int TILE_BYTES = 128 * 128;

__device__ __forceinline__ int swz(int row, int chunk) { return row * 128 + ((chunk ^ ((row >> 1) & 7)) << 4); }
}  // namespace

__global__ __launch_bounds__(256, 2) void k_gemm_tiled(TiledArgs p) {
    extern __shared__ __align__(16) uint8_t lds[];  // [2 stages][W tile, A tile]
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, l16 = lane & 15, q = lane >> 4;
    const int64_t K = p.K, N = p.N, M = p.M, G = K / 128;
    const int64_t ntn = N / BN, ntm = (M + BM - 1) / BM;

    // block -> tile: each XCD (blocks are dealt round-robin to 8) gets a
    // contiguous range of tiles, walked in groups of 8 row tiles so that
    // concurrently running blocks share weight and activation tiles in L2.
    const int64_t nblk = ntn * ntm;
    int64_t lid = blockIdx.x;
    if (nblk % 8 == 0) lid = (blockIdx.x % 8) * (nblk / 8) + blockIdx.x / 8;
    constexpr int GM = 8;
    const int64_t group = lid / (GM * ntn);
    const int64_t first_m = group * GM;
    const int64_t gsz = min<int64_t>(GM, ntm - first_m);
    const int64_t in_group = lid % (GM * ntn);
    const int64_t mt = first_m + in_group % gsz;
    const int64_t nt = in_group / gsz;
    const int64_t n0 = nt * BN, m0 = mt * BM;

    // global -> register loads: thread t moves rows t/8 + 32 i, chunk t % 8
    const int lrow = tid >> 3, lchunk = tid & 7;
    const uint8_t *wsrc[4];
    const uint8_t *asrc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = lrow + 32 * i;
        wsrc[i] = p.w + (n0 + r) * K + lchunk * 16;
        const int64_t am = min<int64_t>(m0 + r, M - 1);  // rows past M read row M-1; never stored
        asrc[i] = p.aq + am * K + lchunk * 16;
    }
    uint4 wreg[4], areg[4];
    auto load_tiles = [&](int64_t g) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            wreg[i] = *(const uint4 *)(wsrc[i] + g * 128);
            areg[i] = *(const uint4 *)(asrc[i] + g * 128);
        }
    };
    auto store_tiles = [&](int stage) {
        uint8_t *wt = lds + stage * 2 * TILE_BYTES;
        uint8_t *at = wt + TILE_BYTES;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = lrow + 32 * i;
            *(uint4 *)(wt + swz(r, lchunk)) = wreg[i];
            *(uint4 *)(at + swz(r, lchunk)) = areg[i];
        }
    };

    // per-lane activation scale rows: m = m0 + wm + 16 j + l16
    const int wn = (wave & 1) * 64, wm = (wave >> 1) * 64;
    const float *as_row[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) as_row[j] = p.as + min<int64_t>(m0 + wm + 16 * j + l16, M - 1) * G;
    const float *ws_row = p.ws + nt * G;

    v4f acc[4][4];  // [n tile][m tile]
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
    const v4f zero = {0.f, 0.f, 0.f, 0.f};

    load_tiles(0);
    store_tiles(0);
    float sa_next[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) sa_next[j] = as_row[j][0];
    __syncthreads();

    for (int64_t g = 0; g < G; ++g) {
        const int stage = (int)(g & 1);
        float sa[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) sa[j] = sa_next[j];
        const float swg = ws_row[g];
        if (g + 1 < G) {
            load_tiles(g + 1);
#pragma unroll
            for (int j = 0; j < 4; ++j) sa_next[j] = as_row[j][g + 1];
        }
        const uint8_t *wt = lds + stage * 2 * TILE_BYTES;
        const uint8_t *at = wt + TILE_BYTES;
        v8i af[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int r = wm + 16 * j + l16;
            af[j] = make_frag(*(const uint4 *)(at + swz(r, q)), *(const uint4 *)(at + swz(r, 4 + q)));
        }
        float sc[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) sc[j] = sa[j] * swg;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = wn + 16 * i + l16;
            const v8i wf = make_frag(*(const uint4 *)(wt + swz(r, q)), *(const uint4 *)(wt + swz(r, 4 + q)));
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const v4f pr = mfma_e4m3_16x16x128(wf, af[j], zero);
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[i][j][e] = __builtin_fmaf(pr[e], sc[j], acc[i][j][e]);
            }
        }
        if (g + 1 < G) store_tiles(stage ^ 1);
        __syncthreads();
    }

    // epilogue: lane holds C[m][n .. n+3] for m = m0 + wm + 16 j + l16, n = n0 + wn + 16 i + 4 q
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int64_t m = m0 + wm + 16 * j + l16;
        if (m < M) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int64_t n = n0 + wn + 16 * i + 4 * q;
                *(uint2 *)(p.c + m * N + n) = bf16x4_rne(acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]);
            }
        }
    }
}

hipError_t launch_gemm_tiled(const TiledArgs &a, hipStream_t s) {
    const size_t smem = 2 * 2 * TILE_BYTES;
    // the dynamic LDS limit is a per-device function attribute: set it once per device
    static std::once_flag once[64];
    static hipError_t attr_err[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    std::call_once(once[dev], [&] {
        attr_err[dev] = hipFuncSetAttribute((const void *)k_gemm_tiled, hipFuncAttributeMaxDynamicSharedMemorySize,
                                            (int)smem);
    });
    if (attr_err[dev] != hipSuccess) return attr_err[dev];
    const int64_t nblk = (a.N / BN) * ((a.M + BM - 1) / BM);
    hipLaunchKernelGGL(k_gemm_tiled, dim3((unsigned)nblk), dim3(256), smem, s, a);
    return hipGetLastError();
}

}  // namespace r9k
