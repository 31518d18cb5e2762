// The bf16-activation variant at decode widths (1 <= M <= 16): fp8 block
// weights against the unquantised bf16 activations.
//
// The r9700-stack release v0.3.1 notes ("What changed for someone running
// it") ship the decode GEMMs of fp8 weights as bf16 WMMA against unquantised
// activations.  Here, with the block scales applied per 128-K group:
//   C[m][n] = bf16( sum_g ws[n/128][g] * sum_{k in g} a[m][k] * dec(wq[n][k]) ).
// An e4m3 value has at most four significant bits, so it converts to bf16
// exactly (v_cvt_scalef32_pk_bf16_fp8 with scale 1), and a bf16 x bf16
// product is exact in the MFMA's fp32.
//
// Shape, like the fp8 decode kernel: a CTA's wn x wk waves own (16-column
// tile, K slice) pairs; each wave requests its whole weight slice into
// registers up front (16-byte loads, the weight stream) and holds it.  Per
// group the lane's 32 weight bytes become four bf16 MFMA fragments of
// v_mfma_f32_16x16x32_bf16.  A group's dot product does not depend on the
// order of K, so the lane's K positions follow the fragment-order weight
// layout (bytes [16q, +16) and [64 + 16q, +16) of the group for lane quarter
// q): MFMA i takes weight bytes 16q + 64 (i / 2) + 8 (i % 2) .. +7 and the
// activations at the same K positions, which the lane loads from global memory
// (L2) two groups ahead.  The four MFMAs of a group accumulate in fp32, then
// acc += P * ws[n/128][g].  The wk slices of a tile are summed through LDS in
// ascending slice order and stored as bf16.  Activation rows past M read row
// M - 1 again; their outputs are never stored.
#include <algorithm>
#include <cstdlib>
#include <mutex>

#include "r9k_device.h"
#include "r9k_internal.h"

namespace r9k {

namespace {
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef unsigned int v4u __attribute__((ext_vector_type(4)));

// four e4m3 codes (one 32-bit word) -> four bf16, two to a word: one
// converting instruction per pair, scale 1 (exact: an e4m3 value has at most
// four significant bits and its exponent range lies inside bf16's)
__device__ __forceinline__ void fp8x4_to_bf16(uint32_t x, uint32_t &lo, uint32_t &hi) {
    lo = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)x, 1.0f, false));  // bytes 0, 1
    hi = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)x, 1.0f, true));   // bytes 2, 3
}

// eight codes (two words) -> one MFMA fragment of eight bf16
__device__ __forceinline__ v8bf frag_bf16(uint32_t w0, uint32_t w1) {
    uint32_t a, b, c, d;
    fp8x4_to_bf16(w0, a, b);
    fp8x4_to_bf16(w1, c, d);
    return __builtin_bit_cast(v8bf, v4u{a, b, c, d});
}

__device__ __forceinline__ v8bf as_bf16(uint4 v) { return __builtin_bit_cast(v8bf, v4u{v.x, v.y, v.z, v.w}); }
}  // namespace

// ALDS: the CTA first copies the M activation rows (all of K) into LDS, with
// coalesced loads issued before the weight stream, so that the MFMA loop reads
// its fragments from LDS while the weights arrive; rows are padded by 16 bytes
// so that the 16 rows a fragment read touches fall on distinct banks.  Without
// it (rows too long for LDS) each lane loads its fragments from global memory,
// two groups ahead of their use.
template <bool PK, int GS, bool ALDS, int NT>
__global__ __launch_bounds__(NT) void k_gemm_bf16a(Bf16aArgs p, int wn, int wk) {
    (void)wk;
    extern __shared__ __align__(16) uint8_t lds[];
    const int64_t K = p.K, N = p.N, G = K / 128;
    const int M = (int)p.M;
    const int tid = threadIdx.x, nthreads = blockDim.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, l16 = lane & 15, q = lane >> 4;
    const int ct = wave % wn, slice = wave / wn;
    const int64_t n0 = ((int64_t)blockIdx.x * wn + ct) * 16;
    const int64_t gbeg = (int64_t)slice * GS;
    const int row = l16 < M ? l16 : M - 1;
    const int apitch = (int)K * 2 + 16;  // bytes per staged row

    // 1. the activation rows, M x K bf16 (16-byte loads, 8 per thread at a time)
    constexpr int AB = 8;
    const int chunks = M * (int)(K / 8);  // 16-byte chunks
    uint4 ab[AB];
    if (ALDS) {
#pragma unroll
        for (int u = 0; u < AB; ++u) {
            const int i = tid + u * nthreads;
            ab[u] = i < chunks ? ((const uint4 *)p.a)[i] : make_uint4(0, 0, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
    }

    // 2. the weight slice, 2 x 16 B per lane per group: the stream (packed weights
    //    through a per-wave buffer descriptor with the non-temporal hint, as in
    //    the decode kernel)
    uint4 wr[GS][2];
    const uint8_t *wrow = PK ? p.w + ((n0 / 16) * G + gbeg) * 2048 + 16 * lane
                             : p.w + (n0 + l16) * K + gbeg * 128 + 16 * q;
    __amdgpu_buffer_rsrc_t wdesc;
    if constexpr (PK)
        wdesc = __builtin_amdgcn_make_buffer_rsrc((void *)(p.w + ((n0 / 16) * G + gbeg) * 2048), (short)0,
                                                  GS * 2048, 0x00020000);
#pragma unroll
    for (int g = 0; g < GS; ++g) {
        if (PK) {
            wr[g][0] = load_buf_nt16(wdesc, 16 * lane + g * 2048);
            wr[g][1] = load_buf_nt16(wdesc, 16 * lane + g * 2048 + 1024);
        } else {
            wr[g][0] = *(const uint4 *)(wrow + g * 128);
            wr[g][1] = *(const uint4 *)(wrow + g * 128 + 64);
        }
    }
    // every weight load goes out before anything else (the compiler would
    // otherwise sink them to their uses and keep only a few in flight)
    __builtin_amdgcn_sched_barrier(0);

    // 3. the activation fragments: the lane's K positions of row min(l16, M - 1),
    // elements [16q, +16) and [64 + 16q, +16) of each group
    uint4 av[3][4];
    const uint16_t *arow = p.a + (int64_t)row * K + gbeg * 128 + 16 * q;
    const uint8_t *alds = lds + row * apitch + (gbeg * 128 + 16 * q) * 2;
    auto load_act = [&](int g, int slot) {
        if (ALDS) {
            const uint4 *src = (const uint4 *)(alds + g * 256);
            av[slot][0] = src[0];
            av[slot][1] = src[1];
            av[slot][2] = src[8];
            av[slot][3] = src[9];
        } else {
            const uint4 *src = (const uint4 *)(arow + g * 128);
            av[slot][0] = src[0];
            av[slot][1] = src[1];
            av[slot][2] = src[8];
            av[slot][3] = src[9];
        }
    };
    if (ALDS) {
        for (int u = 0; u < AB; ++u) {
            const int i = tid + u * nthreads;
            if (i < chunks) {
                const int r = i / (int)(K / 8), c = i % (int)(K / 8);
                *(uint4 *)(lds + r * apitch + c * 16) = ab[u];
            }
        }
        // rows longer than AB chunks a thread: the rest, loaded and stored directly
        for (int i = tid + AB * nthreads; i < chunks; i += nthreads) {
            const int r = i / (int)(K / 8), c = i % (int)(K / 8);
            *(uint4 *)(lds + r * apitch + c * 16) = ((const uint4 *)p.a)[i];
        }
        __syncthreads();
    }
    load_act(0, 0);
    if (GS > 1) load_act(1, 1);
    if (!ALDS) __builtin_amdgcn_sched_barrier(0);

    const int64_t nb = __builtin_amdgcn_readfirstlane((int)(n0 / 128));
    const float *wsrow = p.ws + nb * G + gbeg;
    v4f acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int g = 0; g < GS; ++g) {
        if (g + 2 < GS) load_act(g + 2, (g + 2) % 3);
        const int s = g % 3;
        v4f pr = {0.f, 0.f, 0.f, 0.f};
        pr = __builtin_amdgcn_mfma_f32_16x16x32_bf16(frag_bf16(wr[g][0].x, wr[g][0].y), as_bf16(av[s][0]), pr, 0, 0,
                                                    0);
        pr = __builtin_amdgcn_mfma_f32_16x16x32_bf16(frag_bf16(wr[g][0].z, wr[g][0].w), as_bf16(av[s][1]), pr, 0, 0,
                                                    0);
        pr = __builtin_amdgcn_mfma_f32_16x16x32_bf16(frag_bf16(wr[g][1].x, wr[g][1].y), as_bf16(av[s][2]), pr, 0, 0,
                                                    0);
        pr = __builtin_amdgcn_mfma_f32_16x16x32_bf16(frag_bf16(wr[g][1].z, wr[g][1].w), as_bf16(av[s][3]), pr, 0, 0,
                                                    0);
        const float wsg = wsrow[g];
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] = __builtin_fmaf(pr[i], wsg, acc[i]);
    }

    pin_acc(acc);  // the MFMAs run with every lane enabled

    // 4. sum the K slices in ascending order, round, store: lane holds row
    // l16, columns n0 + 4q .. +3 (the reduction reuses the LDS)
    if (ALDS) __syncthreads();  // every wave is done reading the staged rows
    v4f *red = (v4f *)lds;      // [wave][64 lanes]
    if (slice > 0) red[wave * 64 + lane] = acc;
    __syncthreads();
    if (slice == 0) {
        for (int sl = 1; sl * wn < nthreads / 64; ++sl) acc += red[(sl * wn + ct) * 64 + lane];
        if (l16 < M)
            *(uint2 *)(p.c + (int64_t)l16 * N + n0 + 4 * q) = bf16x4_rne(acc[0], acc[1], acc[2], acc[3]);
    }
}

// dynamic LDS of a launch: the staged rows (if they fit) and the slice sums
static size_t bf16a_lds(int64_t M, int64_t K, const Bf16aCfg &c, bool *alds) {
    const size_t red = sizeof(v4f) * 64 * c.wn * c.wk;
    const size_t rows = (size_t)M * (size_t)(K * 2 + 16);
    *alds = rows <= 144 * 1024;
    return *alds ? std::max(rows, red) : red;
}

// (wn, wk, gs): K-groups per wave preferably 8 (else 16, 4, 2, 1) in at most 8
// slices, then tiles per CTA while at least 256 CTAs remain (168 from 5 rows on;
// up to 4 rows, one tile a CTA where that evens out the compute units' shares).  When a CTA's
// staged rows take more than 72 KiB only one CTA fits on a compute unit, so the
// widest CTA is taken instead (16 groups a wave if that allows it): a single
// round of CTAs (measured at M = 16, K = 4096, N = 14336).
Bf16aCfg bf16a_config(int64_t M, int64_t K, int64_t N) {
    Bf16aCfg c{0, 0, 0};
    const int64_t G = K / 128, tiles = N / 16;
    if (M < 1 || M > 16 || K % 128 || N % 128 || G < 1) return c;
    int force = 0;
    force = tuning().bf16a_gs;
    const bool wide = (size_t)M * (size_t)(K * 2 + 16) > 72 * 1024;
    static const int pref[] = {8, 16, 4, 2, 1}, pref_wide[] = {16, 8, 4, 2, 1};
    // wide rows with eight groups a wave: sixteen-wave CTAs (1024 threads), four
    // slices of eight groups per column tile, so that one CTA per compute unit
    // runs the slices side by side (measured at M = 16, K = 4096, N = 14336)
    // (taken only where the slice count divides sixteen and the CTA's column
    // tiles divide N's, so that the grid covers every column)
    if (wide && !force && G % 8 == 0 && 16 % (G / 8) == 0 && tiles % (16 / (G / 8)) == 0) {
        const int wn16 = (int)(16 / (G / 8));
        // (where that leaves fewer than 168 CTAs, eight waves of half the column
        // tiles, twice the CTAs, as long as they still run in one round of one CTA
        // a compute unit: 6-16 rows at K = 4096 and 8192, N = 2048-8192, 12-42%
        // faster; at N = 10240, K = 4096 the 320 CTAs of two rounds were up to
        // 26% slower, and from 168 CTAs the sixteen-wave CTAs won by up to 27%)
        if (tiles / wn16 < 168 && wn16 >= 2 && tiles / (wn16 / 2) <= 256) return Bf16aCfg{wn16 / 2, (int)(G / 8), 8};
        return Bf16aCfg{wn16, (int)(G / 8), 8};
    }
    for (int gs : wide ? pref_wide : pref) {
        if (force && gs != force) continue;
        if (G % gs || G / gs > 8) continue;
        const int wk = (int)(G / gs);
        int wn = 1;
        // (from 5 rows each CTA stages more of A, and wider CTAs pay down to 168:
        // 5-8 rows at N = 5376-8064, K = 2048 and 4096, 5-26% faster than one tile a CTA)
        const int64_t min_ctas = M > 4 ? 168 : 256;
        while (wn * 2 * wk <= 8 && tiles % (wn * 2) == 0 && (wide || tiles / (wn * 2) >= min_ctas)) wn *= 2;
        // up to 4 rows the busiest compute unit's share of the column tiles sets
        // the time: one tile a CTA where that cuts the share by a fifth or more
        // (576 to 768 tiles: 3 against 4; 1 to 4 rows 3.5-12% faster, at 8 rows,
        // where every CTA stages more of A, 15-23% slower)
        if (!wide && M <= 4 && wn == 2 && 5 * ((tiles + 255) / 256) <= 4 * (2 * ((tiles / 2 + 255) / 256))) wn = 1;
        return Bf16aCfg{wn, wk, gs};
    }
    return c;
}

template <bool PK, int GS, bool ALDS, int NT>
static hipError_t launch_one(const Bf16aArgs &a, const Bf16aCfg &c, size_t lds, hipStream_t s) {
    // the dynamic-LDS limit is a per-device function attribute: set it once per device
    static std::once_flag once[64];
    static hipError_t attr_err[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    std::call_once(once[dev], [&] {
        attr_err[dev] = hipFuncSetAttribute((const void *)k_gemm_bf16a<PK, GS, ALDS, NT>,
                                            hipFuncAttributeMaxDynamicSharedMemorySize, 150 * 1024);
    });
    if (attr_err[dev] != hipSuccess) return attr_err[dev];
    const dim3 grid((unsigned)(a.N / 16 / c.wn)), block((unsigned)(64 * c.wn * c.wk));
    hipLaunchKernelGGL((k_gemm_bf16a<PK, GS, ALDS, NT>), grid, block, lds, s, a, c.wn, c.wk);
    return hipGetLastError();
}

template <bool PK, int GS>
static hipError_t launch_b(const Bf16aArgs &a, const Bf16aCfg &c, hipStream_t s) {
    bool alds = false;
    const size_t lds = bf16a_lds(a.M, a.K, c, &alds);
    if (c.wn * c.wk <= 8)
        return alds ? launch_one<PK, GS, true, 512>(a, c, lds, s) : launch_one<PK, GS, false, 512>(a, c, lds, s);
    if constexpr (GS <= 8)  // sixteen waves: at most 128 VGPRs a lane, so at most eight groups a wave
        if (c.wn * c.wk <= 16)
            return alds ? launch_one<PK, GS, true, 1024>(a, c, lds, s) : launch_one<PK, GS, false, 1024>(a, c, lds, s);
    return hipErrorInvalidValue;
}

template <bool PK>
static hipError_t launch_gs(const Bf16aArgs &a, const Bf16aCfg &c, hipStream_t s) {
    switch (c.gs) {
        case 1: return launch_b<PK, 1>(a, c, s);
        case 2: return launch_b<PK, 2>(a, c, s);
        case 4: return launch_b<PK, 4>(a, c, s);
        case 8: return launch_b<PK, 8>(a, c, s);
        case 16: return launch_b<PK, 16>(a, c, s);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_gemm_bf16a(const Bf16aArgs &a, const Bf16aCfg &c, hipStream_t s) {
    return a.packed ? launch_gs<true>(a, c, s) : launch_gs<false>(a, c, s);
}

}  // namespace r9k
