// Engine (b): the LDS-tiled block-scaled fp8 MFMA GEMM for prefill widths.
//
// The pages' tiled fp8 GEMMs take every row count above the decode kernels'
// 255 (r9700-stack release v0.3.2, "What changed for someone running it"), and
// their exact block-scaled variant (release v0.3.0, same section) is the
// semantics kept here: the K loop steps one 128-wide group at a time, and each
// group's MFMA sum is promoted with its own scales, acc += P * as[m,g] * ws[n/128,g].
//
// Activations arrive pre-quantised, with the scales transposed to [K/128][M]
// so that a group's scales for consecutive rows are contiguous: at these
// widths the fused entry point quantises A once per call instead of once per
// column tile, which would cost more VALU time than the MFMAs.
//
// CTA tile: 128 rows of A x 256 columns (two weight block rows), 4 waves, one
// per SIMD, so that each wave has the whole register file (the 128 fp32
// accumulators, the fragments and the MFMA results in flight).  Wave w owns
// columns 128 (w & 1) .. +127 (one weight block row, so one weight scale per
// group) and rows 64 (w >> 1) .. +63: 8 x 4 MFMA tiles of 16 x 16 x 128,
// computed as C^T = W A^T so that a lane's four outputs of a tile share one
// row of A, and with it one activation scale.  The promotion is then one
// multiply per row tile and one FMA per output per group.
//
// A stage holds one group: the W tile [256 rows][128 bytes], the A tile
// [128 rows][128 bytes] and the wave's 64 activation scales; three stages
// (147 KiB of LDS), filled two groups ahead.  Everything moves from global
// memory straight into LDS (global_load_lds, no register staging), so one
// wait on the wave's load counter covers a stage.  A 16-byte load instruction
// fills 1 KiB of LDS, 8 rows; lane l writes physical chunk l % 8 of its row
// and fetches the logical chunk that belongs there: chunk c of row r lives at
// chunk c ^ ((r >> 1) & 7), so the 16 rows a fragment read touches in one LDS
// cycle fall on distinct banks.
#include <mutex>

#include "r9k_device.h"
#include "r9k_internal.h"

namespace r9k {

namespace {
constexpr int BN = 256;                 // output columns (W rows) per CTA
constexpr int BM = 128;                 // output rows (A rows) per CTA
constexpr int WBYTES = BN * 128;        // W tile of a stage
constexpr int ABYTES = BM * 128;        // A tile of a stage
constexpr int SBYTES = 4 * 2 * 64 * 4;  // per wave: 64 activation scales, the weight scale x 64
constexpr int STAGE = WBYTES + ABYTES + SBYTES;
constexpr int NST = 3;
constexpr int SMEM = NST * STAGE;
constexpr int THREADS = 256;
constexpr int LOADS_PER_STAGE = 8 + 4 + 2;  // per wave: W, A, activation scales, weight scale
static_assert(SMEM <= 160 * 1024, "LDS");

// Global -> LDS loads (lane l's bytes land at LDS address `l_addr` + size * l,
// the address taken from M0).  Issued from inline asm so that the compiler
// neither waits for them at every barrier nor before every LDS read (it cannot
// tell that the reads touch another stage); the kernel waits for them itself
// with wait_vm, counting this wave's load instructions.
__device__ __forceinline__ uint32_t lds_addr(const uint8_t *p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t *)p;
}
__device__ __forceinline__ void load_lds16(const uint8_t *g, uint32_t l_addr) {
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(l_addr) : "memory", "m0");
}
__device__ __forceinline__ void load_lds4(const float *g, uint32_t l_addr) {
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off" ::"v"(g), "s"(l_addr) : "memory", "m0");
}

__device__ __forceinline__ int swz(int row, int chunk) { return row * 128 + ((chunk ^ ((row >> 1) & 7)) << 4); }

__device__ __forceinline__ v8i frag(const uint8_t *tile, int row, int q) {
    return make_frag(*(const uint4 *)(tile + swz(row, q)), *(const uint4 *)(tile + swz(row, q + 4)));
}

// wait until at most VM of this wave's vector-memory instructions are in flight
template <int VM>
__device__ __forceinline__ void wait_vm() {
    static_assert(VM >= 0 && VM < 64, "vmcnt");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(VM) : "memory");
}
}  // namespace

__global__ __launch_bounds__(THREADS, 1) void k_gemm_tiled(TiledArgs p) {
    extern __shared__ __align__(16) uint8_t lds[];
    const int tid = threadIdx.x, lane = tid & 63, l16 = lane & 15, q = lane >> 4;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wn = wave & 1, wm = wave >> 1;
    const int64_t K = p.K, N = p.N, M = p.M, G = K / 128;
    const int64_t ntn = (N + BN - 1) / BN, ntm = (M + BM - 1) / BM;

    // block -> tile.  Blocks are dealt round-robin to the 8 XCDs; each XCD
    // takes a contiguous range of tiles, walked in groups of GM row tiles, so
    // that the blocks running together on one XCD share A and W tiles in its L2.
    const int64_t nblk = ntn * ntm;
    int64_t lid = blockIdx.x;
    if (nblk % 8 == 0) lid = (blockIdx.x % 8) * (nblk / 8) + blockIdx.x / 8;
    constexpr int GM = 8;
    const int64_t group = lid / (GM * ntn);
    const int64_t first_m = group * GM;
    const int64_t gsz = min<int64_t>(GM, ntm - first_m);
    const int64_t in_group = lid % (GM * ntn);
    const int64_t m0 = (first_m + in_group % gsz) * BM;
    const int64_t n0 = (in_group / gsz) * BN;

    // This wave's loads of a stage: W instructions 8 wave + u (u < 8) and A
    // instructions 4 wave + u (u < 4), each 8 rows from row 8 * index + lane / 8,
    // its 64 activation scales, and its weight scale (every lane the same).  W rows past N (the upper half of a last,
    // half-full column tile; an instruction's 8 rows are all on one side) read
    // the lower half instead; A rows past M read row M - 1.  Neither is stored.
    const uint8_t *wsrc[8];
    const uint8_t *asrc[4];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
        const int row = 8 * (8 * wave + u) + (lane >> 3);
        const int chunk = (lane & 7) ^ ((row >> 1) & 7);
        const int64_t wrow = (n0 + 8 * (8 * wave + u) < N) ? n0 + row : n0 + row - 128;
        wsrc[u] = p.w + wrow * K + 16 * chunk;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int row = 8 * (4 * wave + u) + (lane >> 3);
        const int chunk = (lane & 7) ^ ((row >> 1) & 7);
        asrc[u] = p.aq + min<int64_t>(m0 + row, M - 1) * K + 16 * chunk;
    }
    const float *ssrc = p.as_t + min<int64_t>(m0 + 64 * wm + lane, M - 1);
    const int64_t nb = min<int64_t>(n0 / 128 + wn, N / 128 - 1);
    const float *wssrc = p.ws + nb * G;
    const uint32_t lds0 = __builtin_amdgcn_readfirstlane(lds_addr(lds));
    auto issue = [&](int64_t g, int st) {
        const uint32_t sb = lds0 + st * STAGE;
#pragma unroll
        for (int u = 0; u < 8; ++u) load_lds16(wsrc[u] + g * 128, sb + (8 * wave + u) * 1024);
#pragma unroll
        for (int u = 0; u < 4; ++u) load_lds16(asrc[u] + g * 128, sb + WBYTES + (4 * wave + u) * 1024);
        load_lds4(ssrc + g * M, sb + WBYTES + ABYTES + wave * 512);
        load_lds4(wssrc + g, sb + WBYTES + ABYTES + wave * 512 + 256);
    };

    v4f acc[8][4];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
    const v4f zero = {0.f, 0.f, 0.f, 0.f};

    issue(0, 0);
    if (G > 1) issue(1, 1);
    for (int64_t g = 0; g < G; ++g) {
        const int st = (int)(g % NST);
        // group g's stage has landed: this wave's loads issued after it are
        // group g + 1's, if any; then every wave's, and every wave is done
        // with the stage that group g + 2 will overwrite
        if (g + 1 < G) wait_vm<LOADS_PER_STAGE>();
        else wait_vm<0>();
        __syncthreads();
        if (g + 2 < G) issue(g + 2, (int)((g + 2) % NST));

        const uint8_t *wt = lds + st * STAGE;
        const uint8_t *at = wt + WBYTES;
        const float *sl = (const float *)(at + ABYTES + wave * 512);
        const float wsg = sl[64 + lane];
        float sc[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) sc[j] = sl[16 * j + l16] * wsg;
        v8i af[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) af[j] = frag(at, 64 * wm + 16 * j + l16, q);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const v8i wf = frag(wt, 128 * wn + 16 * i + l16, q);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const v4f pr = mfma_e4m3_16x16x128(wf, af[j], zero);
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[i][j][e] = __builtin_fmaf(pr[e], sc[j], acc[i][j][e]);
            }
        }
    }

    // lane holds, per tile (i, j), row m = m0 + 64 wm + 16 j + l16 and the four
    // columns n = n0 + 128 wn + 16 i + 4 q .. +3
    const int64_t nbase = n0 + 128 * wn;
    if (nbase >= N) return;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int64_t m = m0 + 64 * wm + 16 * j + l16;
        if (m >= M) continue;
        uint16_t *crow = p.c + m * N + nbase + 4 * q;
#pragma unroll
        for (int i = 0; i < 8; ++i)
            *(uint2 *)(crow + 16 * i) = bf16x4_rne(acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]);
    }
}

hipError_t launch_gemm_tiled(const TiledArgs &a, hipStream_t s) {
    // the dynamic LDS limit is a per-device function attribute: set it once per device
    static std::once_flag once[64];
    static hipError_t attr_err[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    std::call_once(once[dev], [&] {
        attr_err[dev] = hipFuncSetAttribute((const void *)k_gemm_tiled, hipFuncAttributeMaxDynamicSharedMemorySize,
                                            SMEM);
    });
    if (attr_err[dev] != hipSuccess) return attr_err[dev];
    const int64_t nblk = ((a.N + BN - 1) / BN) * ((a.M + BM - 1) / BM);
    hipLaunchKernelGGL(k_gemm_tiled, dim3((unsigned)nblk), dim3(THREADS), SMEM, s, a);
    return hipGetLastError();
}

}  // namespace r9k
