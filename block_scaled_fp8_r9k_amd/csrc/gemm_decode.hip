// Engine (a), decode widths (1 <= M <= 64): the weight-streaming skinny GEMM.
//
// The r9700-stack release v0.3.1 notes ("What changed for someone running
// it") describe the decode GEMMs as the step's largest weight stream and move
// the per-token-group-128 activation quant into the GEMM's A-load.  Here the
// kernel is shaped around that stream:
//   - a CTA's wn x wk waves own (16-column tile, K slice) pairs, 16 weight rows
//     by K/wk bytes each, and all of K is covered inside the CTA, so no CTA
//     ever waits for another and the result does not depend on timing;
//   - every wave first requests its share of the activation groups, then its
//     whole weight slice, straight into the registers that feed the MFMA
//     (16-byte loads, at most 32 per lane); a wave's loads complete in issue
//     order, so the activations are usable while the weights still stream;
//   - the CTA quantises the M activation rows over all of K into LDS, 4 lanes
//     (a DPP quad) per 128-value group: the fused A-load of
//     r9k_gemm_fp8_block_qa; the split form copies pre-quantised codes instead;
//   - per K-group one e4m3 16x16x128 MFMA, promoted as acc += P * as * ws;
//   - the wk K-slices of a tile are summed through LDS in ascending slice order
//     by the slice-0 wave, rounded to bf16 and stored.
// LDS holds the M activation rows only; the MFMA's rows M..15 read row M - 1
// again and their outputs are never stored.  MFMA roles: weight rows are the A operand (16 n), activation
// rows the B operand (16 m); a lane's four outputs are four consecutive n of
// row l % 16.  K order inside a group: lane quarter q feeds bytes [16q, +16)
// and [64+16q, +16) for both operands.
#include <algorithm>
#include <climits>
#include <cstdlib>
#include <mutex>

#include "r9k_device.h"
#include "r9k_internal.h"

namespace r9k {

namespace {
constexpr int MAX_GS = 16;  // K-groups per wave: 32 x 16-byte loads per lane
}

// GS = K-groups per wave, PASSES = activation groups per lane quad; both fixed
// at compile time so that every load is unconditional and each wait covers
// only the loads it needs.
//
// Issue schedule per wave.  A wave that has more loads than the memory system
// takes at once stalls at the load instruction itself, so anything placed
// after all of its weight loads would start only near the end of the stream.
// The weight slice therefore goes out in NCH chunks, and the activation side
// is worked on between them: activation batch 0, weight chunk 0, quantise
// batch 0, activation batch 1, weight chunk 1, quantise batch 1, remaining
// weight chunks.  Loads of one wave complete in issue order, so each quantise
// step waits only for its own batch and the chunks issued before it.
//
// PK: the weights are in fragment order (r9k_pack_weight), so a wave's slice
// is one contiguous run and every 16-byte load instruction reads 1 KiB of
// consecutive bytes; the registers receive exactly what the row-major loads
// would give them.
//
// MT: row tiles of 16 (M <= 16 * MT); each weight fragment feeds MT MFMAs.
//
// K split (gridDim.y = ksplit > 1): CTA (x, ks) covers K-groups
// [ks * wk * GS, (ks + 1) * wk * GS) only, quantises just those groups of
// the activations into LDS, and writes fp32 partial sums part[ks][m][n] that a
// second kernel adds in ascending ks.  Used where all of K does not fit in LDS
// or where every CTA quantising all of K would cost more than the stream.
template <bool QA, bool PK, int GS, int PASSES, int MT, int NT>
__global__ __launch_bounds__(NT) void k_gemm_decode(DecodeArgs p, int wn, int wk) {
    constexpr int SR = 16 * MT;                      // scale row stride
    constexpr int PB = PASSES < 4 ? PASSES : 4;      // passes per activation batch
    constexpr int NB = PASSES / PB;                  // activation batches (1 or 2)
    constexpr int NCH = GS < 4 ? GS : 4;             // weight chunks
    constexpr int CH = GS / NCH;                     // K-groups per chunk
    static_assert(NB <= NCH, "each activation batch follows a weight chunk");
    extern __shared__ __align__(16) uint8_t lds[];
    const int64_t K = p.K, N = p.N, G = K / 128;
    const int M = (int)p.M;
    const int GC = wk * GS;                           // K-groups of this CTA
    const int64_t g0 = (int64_t)blockIdx.y * GC;      // its first group
    const int pitch = GC * 128 + 16;                  // codes [M][GC * 128 + 16]
    float *scales = (float *)(lds + M * pitch);        // [GC][16 MT]
    const int tid = threadIdx.x, nthreads = blockDim.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, l16 = lane & 15, q = lane >> 4;
    const int ct = wave % wn, slice = wave / wn;
    const int64_t n0 = ((int64_t)blockIdx.x * wn + ct) * 16;  // first column of this wave's tile
    const int lbeg = slice * GS;                      // first local group of this wave
    const int64_t gbeg = g0 + lbeg;                   // ... as a global group

    // activation task (row r, local group g) per lane quad, 32 values a lane;
    // quads past M * GC load task 0 again and discard it
    const int quads = nthreads >> 2, quad = tid >> 2, sub = tid & 3;
    const int tasks = M * GC;
    // fused: bf16 values (four uint4 a lane); codes path: e4m3 codes (two
    // 16-byte vectors) and the group scale.  The codes are held as plain
    // vectors: copied as uint4 aggregates they would stay in scratch memory.
    uint4 av[PB][QA ? 4 : 1];
    u32x4 cv[PB][QA ? 1 : 2];
    float sv[PB];
    auto load_act = [&](int batch) {
#pragma unroll
        for (int j = 0; j < PB; ++j) {
            int task = quad + quads * (batch * PB + j);
            task = task < tasks ? task : 0;
            const int r = task / GC, g = task % GC;
            if constexpr (QA) {
                const uint4 *src = (const uint4 *)(p.a + (int64_t)r * K + (g0 + g) * 128 + sub * 32);
#pragma unroll
                for (int i = 0; i < 4; ++i) av[j][i] = src[i];
            } else {
                const u32x4 *src = (const u32x4 *)(p.aq + (int64_t)r * K + (g0 + g) * 128 + sub * 32);
                cv[j][0] = src[0];
                cv[j][1] = src[1];
                sv[j] = p.as[(int64_t)r * G + g0 + g];
            }
        }
    };
    auto quant_act = [&](int batch) {
#pragma unroll
        for (int j = 0; j < PB; ++j) {
            const int task = quad + quads * (batch * PB + j);
            if (task < tasks) {  // uniform across the 4 lanes of a quad
                const int r = task / GC, g = task % GC;
                u32x4 *dst = (u32x4 *)(lds + r * pitch + g * 128 + sub * 32);
                float sc;
                if constexpr (QA) {
                    uint4 v[4] = {av[j][0], av[j][1], av[j][2], av[j][3]};
                    uint4 codes[2];
                    quant_group4(v, codes, sc);
                    dst[0] = u32x4{codes[0].x, codes[0].y, codes[0].z, codes[0].w};
                    dst[1] = u32x4{codes[1].x, codes[1].y, codes[1].z, codes[1].w};
                } else {
                    dst[0] = cv[j][0];
                    dst[1] = cv[j][1];
                    sc = sv[j];
                }
                if (sub == 0) scales[g * SR + r] = sc;
            }
        }
    };

    // the weight slice: 16 rows x GS groups, 2 x 16 B per lane per group.  Packed
    // weights are read with buffer loads through a per-wave descriptor over the
    // wave's GS x 2 KiB slab (a 32-bit lane offset instead of a 64-bit address;
    // 2-3% faster than global loads) with the non-temporal hint (each 1 KiB
    // instruction reads whole lines once per call: 5-6% faster); row-major loads,
    // which read half lines, ran 10% slower with the hint and keep plain loads
    uint4 wr[GS][2];
    const uint8_t *wrow = PK ? p.w + ((n0 / 16) * G + gbeg) * 2048 + 16 * lane
                             : p.w + (n0 + l16) * K + gbeg * 128 + 16 * q;
    __amdgpu_buffer_rsrc_t wdesc;
    if constexpr (PK)  // base, stride 0, size in bytes, dword 3 of a raw byte buffer
        wdesc = __builtin_amdgcn_make_buffer_rsrc((void *)(p.w + ((n0 / 16) * G + gbeg) * 2048), (short)0,
                                                  GS * 2048, 0x00020000);
    auto load_w = [&](int chunk) {
#pragma unroll
        for (int j = 0; j < CH; ++j) {
            const int g = chunk * CH + j;
            if (PK) {
                wr[g][0] = load_buf_nt16(wdesc, 16 * lane + g * 2048);
                wr[g][1] = load_buf_nt16(wdesc, 16 * lane + g * 2048 + 1024);
            } else {
                wr[g][0] = *(const uint4 *)(wrow + g * 128);
                wr[g][1] = *(const uint4 *)(wrow + g * 128 + 64);
            }
        }
    };

    load_act(0);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int ch = 0; ch < NCH; ++ch) {
        load_w(ch);
        __builtin_amdgcn_sched_barrier(0);
        if (ch < NB) {
            quant_act(ch);
            __builtin_amdgcn_sched_barrier(0);
            if (ch + 1 < NB) {
                load_act(ch + 1);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    }
    __syncthreads();

    // ---- MFMA per group and row tile, and promotion; the weight block scale is
    // uniform per wave
    v4f acc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt] = v4f{0.f, 0.f, 0.f, 0.f};
    const v4f zero = {0.f, 0.f, 0.f, 0.f};
    const int64_t nb = __builtin_amdgcn_readfirstlane((int)(n0 / 128));
    const float *wsrow = p.ws + nb * G + gbeg;
#pragma unroll
    for (int g = 0; g < GS; ++g) {
        const int gg = lbeg + g;  // local group
        const v8i wf = make_frag(wr[g][0], wr[g][1]);
        const float wsg = wsrow[g];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            // the MFMA's rows past M read row M - 1 again; their outputs are never stored
            const int row = min(16 * mt + l16, M - 1);
            const uint8_t *ap = lds + row * pitch + gg * 128 + 16 * q;
            const v8i af = make_frag(*(const uint4 *)ap, *(const uint4 *)(ap + 64));
            const float sc = scales[gg * SR + row] * wsg;
            const v4f pr = mfma_e4m3_16x16x128(wf, af, zero);
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[mt][i] = __builtin_fmaf(pr[i], sc, acc[mt][i]);
        }
    }

#pragma unroll
    for (int mt = 0; mt < MT; ++mt) pin_acc(acc[mt]);  // the MFMAs run with every lane enabled

    // ---- sum the K slices in ascending order, round, store
    __syncthreads();                                   // every wave is done reading the codes
    v4f *red = (v4f *)lds;                             // [wave][MT][64 lanes]
    if (slice > 0) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) red[(wave * MT + mt) * 64 + lane] = acc[mt];
    }
    __syncthreads();
    if (slice == 0) {
        for (int s = 1; s < wk; ++s) {
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) acc[mt] += red[((s * wn + ct) * MT + mt) * 64 + lane];
        }
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const int row = 16 * mt + l16;
            if (row >= M) continue;
            if (gridDim.y > 1)
                *(v4f *)(p.part + ((int64_t)blockIdx.y * M + row) * N + n0 + 4 * q) = acc[mt];
            else
                *(uint2 *)(p.c + (int64_t)row * N + n0 + 4 * q) =
                    bf16x4_rne(acc[mt][0], acc[mt][1], acc[mt][2], acc[mt][3]);
        }
    }
}

// Is (wn, wk, gs, ksplit) a valid launch for M rows?  Fills c if so.
static bool decode_fits(int64_t M, int64_t K, int64_t N, int wn, int wk, int64_t gs, int64_t ksplit, DecodeCfg &c) {
    const int64_t G = K / 128, tiles = N / 16;
    if (tiles % wn || wn * wk > 16 || gs < 1 || gs > MAX_GS || (gs & (gs - 1))) return false;
    // sixteen-wave CTAs (1024 threads, at most 128 VGPRs a lane) for one row tile and at most eight
    // groups a wave: their weight slice must fit the smaller register budget
    if (wn * wk > 8 && ((M + 15) / 16 > 1 || gs > 8)) return false;
    if ((int64_t)wk * gs * ksplit != G) return false;
    const int mt = (int)((M + 15) / 16);
    const int64_t gc = wk * gs;
    const size_t lds = (size_t)M * (gc * 128 + 16) + (size_t)gc * 16 * mt * 4;
    const size_t red = (size_t)wn * wk * mt * 64 * 16;  // the slice reduction reuses the codes region
    if (std::max(lds, red) > 150 * 1024) return false;
    const int64_t quads = 16 * wn * wk;
    int passes = 1;
    while (passes * quads < M * gc) passes *= 2;
    if (passes > 8) return false;
    const int64_t nch = gs < 4 ? gs : 4;
    if ((passes < 4 ? 1 : passes / 4) > nch) return false;  // each activation batch follows a weight chunk
    c = DecodeCfg{wn, wk, (int)gs, passes, std::max(lds, red), mt, (int)ksplit};
    return true;
}

// (wn, wk, gs, ksplit) for a shape, M <= 64.  Measured on the MI355X (K = 4096,
// N = 14336): eight-wave CTAs stream fastest; the activation quant, which
// every CTA repeats, favours fewer and wider CTAs once M is large.
//  1. All of K in one CTA (ksplit = 1): wn = 4 from 9 rows on when that leaves
//     at least 168 CTAs, else wn = 2 when that leaves at least 256 CTAs (168
//     from 5 rows on), else 1, and up to 4 rows wn = 1 where it gives the
//     busiest compute unit a fifth fewer tiles; then the smallest K split into waves (K-groups per wave a power of
//     two, at most 16; the split any count up to 8, e.g. 7 for K = 14336) that
//     gives at least 8 waves per compute unit (4 on row-major weights, whose
//     16-row load pattern does better with fewer); on fragment-order weights
//     also at least as many slices as keep a wave's slab at 8 K-groups or fewer
//     (at 8 to 16 thousand column tiles two slices of 16 groups streamed 3-6%
//     slower than four of 8).  Taken when it fits and the CTAs together quantise
//     at most 2^24 activation values or a quarter of the weight bytes, whichever
//     is more: an LM head over a large vocabulary repeats the quant across
//     thousands of CTAs, but each CTA's share stays small next to its stream
//     (4 x 4096 x 128256 80 against 87 us with the K split, 8 rows 86.5 against
//     94.7 us on the skinny kernel; row-major 91 against 119 us).
//  2. Else a K split across CTAs: CTAs of 4 x 2 waves (fewer column tiles if
//     N is narrow), the largest K-groups per wave that still gives at least
//     256 CTAs, with the split's partial sums reduced by a second kernel.
// The activation side needs PASSES = M * (its K-groups) / (16 * waves)
// register passes, at most 8 (two batches of 4).
// R9K_DECODE_WN / R9K_DECODE_WK override step 1 (tuning).
DecodeCfg decode_config(int64_t M, int64_t K, int64_t N, bool packed) {
    DecodeCfg c{0, 0, 0, 0, 0, 0, 0};
    const int64_t G = K / 128, tiles = N / 16;
    if (M < 1 || M > 64) return c;
    // 1. all of K per CTA
    int wn = (tiles % 2 == 0 && tiles / 2 >= (M <= 4 ? 256 : 168)) ? 2 : 1;
    // (from 9 rows: at 9 to 11 rows and N = 14336 the half-width CTAs took 6-10%
    // longer on packed weights, at 10 and 11 rows because their repeated quant
    // passes the 2^24 budget below and sends the shape to a K split)
    if (M >= 9 && tiles % 4 == 0 && tiles / 4 >= 168) wn = 4;
    // up to 4 rows the repeated quant is small, and the busiest compute unit's
    // share of the column tiles sets the time: one tile a CTA where that cuts
    // the share by a fifth or more (640 to 768 tiles: 3 against 4)
    if (M <= 4 && wn == 2 && 5 * ((tiles + 255) / 256) <= 4 * (2 * ((tiles / 2 + 255) / 256))) wn = 1;
    if (const int v = tuning().decode_wn) {
        if (v >= 1 && v <= 4 && tiles % v == 0) wn = v;
    }
    const int force_wk = tuning().decode_wk;
    DecodeCfg best{0, 0, 0, 0, 0, 0, 0};
    for (int cand = 1; cand <= 16; ++cand) {
        if (force_wk && cand != force_wk) continue;
        if (G % cand) continue;
        DecodeCfg t;
        if (!decode_fits(M, K, N, wn, cand, G / cand, 1, t)) continue;
        best = t;
        if ((tiles / wn) * wn * cand >= (packed ? 8 : 4) * 256 && (!packed || G / cand <= 8)) break;
    }
    // (a whole-K grid of fewer than 192 CTAs leaves compute units idle; where each
    // CTA also re-quantises 12 x 8192 activation values or more, the K split below,
    // which spreads the stream and divides the quant, was faster: N = 1024 and 2048
    // at 12-16 rows and K = 8192, 8 rows and K = 14336-16384, 4-17%; with less
    // quant a CTA it lost up to 22%, its reduce launch costing more than it saved)
    const bool few_ctas = best.wn && tiles / best.wn < 192 && M * K >= 12 * 8192 && K >= 8192 && N >= 1024;
    if (best.wn && (force_wk || (!few_ctas && (tiles / best.wn) * M * K <=
                                                  std::max<int64_t>(int64_t(1) << 24, N * K / 4))))
        return best;
    // 2. a K split across CTAs
    const int wn2 = tiles % 4 == 0 && tiles / 4 >= 64 ? 4 : tiles % 2 == 0 && tiles / 2 >= 64 ? 2 : 1;
    const int wk2 = 8 / wn2 >= 2 ? 2 : 1;
    DecodeCfg split{0, 0, 0, 0, 0, 0, 0};
    for (int64_t gs = MAX_GS; gs >= 1; gs /= 2) {
        if (G % (wk2 * gs)) continue;
        const int64_t ks = G / (wk2 * gs);
        if (ks < 2) continue;
        DecodeCfg t;
        if (!decode_fits(M, K, N, wn2, wk2, gs, ks, t)) continue;
        split = t;
        if ((tiles / wn2) * ks >= 256) break;
    }
    // every n-tile CTA quantises its own copy of the activation slice: past
    // 2^25 such elements (M = 64 at K = 14336, N = 4096) the tiled engine is faster
    if (split.wn && (tiles / split.wn) * M * K <= (int64_t(1) << 25)) return split;
    return best.wn && (tiles / best.wn) * M * K <= (int64_t(1) << 26) ? best : c;
}

size_t decode_partial_bytes(int64_t M, int64_t K, int64_t N) {
    size_t b = 0;
    for (bool packed : {false, true}) {
        const DecodeCfg c = decode_config(M, K, N, packed);
        if (c.wn && c.ksplit > 1) b = std::max(b, sizeof(float) * (size_t)c.ksplit * M * N);
    }
    return align_up(b, 256);
}

// one instantiation: its 160 KiB dynamic-LDS limit is set once per device
template <bool QA, bool PK, int GS, int PS, int MT, int NT>
static hipError_t launch_nt(const DecodeArgs &a, const DecodeCfg &c, hipStream_t s, dim3 grid, dim3 block) {
    static std::once_flag once[64];
    static hipError_t attr_err[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    std::call_once(once[dev], [&] {
        attr_err[dev] = hipFuncSetAttribute((const void *)k_gemm_decode<QA, PK, GS, PS, MT, NT>,
                                            hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    });
    if (attr_err[dev] != hipSuccess) return attr_err[dev];
    hipLaunchKernelGGL((k_gemm_decode<QA, PK, GS, PS, MT, NT>), grid, block, c.lds, s, a, c.wn, c.wk);
    return hipGetLastError();
}

// eight-wave CTAs, or sixteen (one row tile, at most eight groups a wave)
template <bool QA, bool PK, int GS, int PS, int MT>
static hipError_t launch_one(const DecodeArgs &a, const DecodeCfg &c, hipStream_t s, dim3 grid, dim3 block) {
    if (c.wn * c.wk <= 8) return launch_nt<QA, PK, GS, PS, MT, 512>(a, c, s, grid, block);
    if constexpr (MT == 1 && GS <= 8) return launch_nt<QA, PK, GS, PS, MT, 1024>(a, c, s, grid, block);
    return hipErrorInvalidValue;
}

template <bool QA, bool PK, int GS, int MT>
static hipError_t launch_ps(const DecodeArgs &a, const DecodeCfg &c, hipStream_t s, dim3 grid, dim3 block) {
    switch (c.passes) {
        case 1: return launch_one<QA, PK, GS, 1, MT>(a, c, s, grid, block);
        case 2: return launch_one<QA, PK, GS, 2, MT>(a, c, s, grid, block);
        case 4: return launch_one<QA, PK, GS, 4, MT>(a, c, s, grid, block);
        case 8:
            if constexpr (GS >= 2) return launch_one<QA, PK, GS, 8, MT>(a, c, s, grid, block);
            break;
    }
    return hipErrorInvalidValue;
}

template <bool QA, bool PK, int GS>
static hipError_t launch_mt(const DecodeArgs &a, const DecodeCfg &c, hipStream_t s, dim3 grid, dim3 block) {
    switch (c.mt) {
        case 1: return launch_ps<QA, PK, GS, 1>(a, c, s, grid, block);
        case 2: return launch_ps<QA, PK, GS, 2>(a, c, s, grid, block);
        case 3: return launch_ps<QA, PK, GS, 3>(a, c, s, grid, block);
        case 4: return launch_ps<QA, PK, GS, 4>(a, c, s, grid, block);
    }
    return hipErrorInvalidValue;
}

template <bool QA, bool PK>
static hipError_t launch_gs(const DecodeArgs &a, const DecodeCfg &c, hipStream_t s, dim3 grid, dim3 block) {
    switch (c.gs) {
        case 1: return launch_mt<QA, PK, 1>(a, c, s, grid, block);
        case 2: return launch_mt<QA, PK, 2>(a, c, s, grid, block);
        case 4: return launch_mt<QA, PK, 4>(a, c, s, grid, block);
        case 8: return launch_mt<QA, PK, 8>(a, c, s, grid, block);
        case 16: return launch_mt<QA, PK, 16>(a, c, s, grid, block);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_gemm_decode(const DecodeArgs &a, const DecodeCfg &c, hipStream_t s) {
    const dim3 grid((unsigned)(a.N / 16 / c.wn), (unsigned)c.ksplit);
    const dim3 block((unsigned)(64 * c.wn * c.wk));
    hipError_t e;
    if (a.a) e = a.packed ? launch_gs<true, true>(a, c, s, grid, block) : launch_gs<true, false>(a, c, s, grid, block);
    else e = a.packed ? launch_gs<false, true>(a, c, s, grid, block) : launch_gs<false, false>(a, c, s, grid, block);
    if (e != hipSuccess || c.ksplit == 1) return e;
    return launch_splitk_reduce(a.part, a.c, a.M, a.N, c.ksplit, s);
}

}  // namespace r9k
