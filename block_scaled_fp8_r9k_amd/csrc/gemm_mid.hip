// Engine (a) at mid widths (17 to 256 rows): the block-scaled fp8 GEMM as one
// launch over all of K, with no partial sums leaving a CTA; at long K and up to
// 64 rows, a K split whose fp32 partials a second launch sums in order.
//
// The r9700-stack release v0.3.2 notes ("What changed for someone running it")
// run the fp8 decode kernels up to 255 rows.  At these widths the weight is
// still most of the bytes, but the activation codes (M x K) are read by every
// column block, and the product of the two is large enough that splitting K
// across CTAs means writing and re-reading fp32 partials of M x N.  Here a CTA
// covers a BM x BN output block over all of K:
//   - BM = 16 MT rows (MT = 1, 2 or 4 row tiles of 16), BN = 16 WN columns;
//     WN x WK waves, wave (ct, slice) owns column tile ct and the K-groups
//     g = s WK + slice of steps s = 0 .. G/WK - 1; the WK slices of a column
//     tile are summed through LDS at the end, in ascending slice order;
//   - the CTA count is about 256 (one per compute unit) and BM x BN is as square
//     as the shape allows, which minimises the bytes a compute unit reads
//     (BN + BM) x K;
//   - weight fragments stream straight into registers (16-byte loads, fragment
//     order or row-major), D steps ahead of their use;
//   - activation codes come quantised (the fused entry point quantises once per
//     call, like the tiled engine), with the scales transposed to [K/128][M] so
//     that the 16 rows of a row tile read one line of scales: with WN > 1 the CTA stages each step's
//     WK groups of its BM rows in LDS (loaded into registers D steps ahead,
//     written to one of two LDS buffers in a bank-swizzled layout, one barrier
//     per step), shared by the WN
//     column tiles; with WN = 1 nothing is shared and each wave loads its own
//     activation fragments into registers;
//   - per group one e4m3 16x16x128 MFMA per row tile, promoted with the group's
//     scales, acc += P * as[m,g] * ws[n/128,g].
// MFMA roles as in the decode kernel: weight rows are the A operand (16 n),
// activation rows the B operand (16 m); a lane's four outputs are four
// consecutive n of row l % 16, and lane quarter q feeds bytes [16q, +16) and
// [64 + 16q, +16) of a group.  Rows past M read row M - 1 and are never stored.
#include <algorithm>
#include <mutex>

#include "r9k_device.h"
#include "r9k_internal.h"

namespace r9k {

namespace {
// Staged activations: rows of one group, 128 bytes each, with the 16-byte chunk
// c of row R at chunk c ^ ((R >> 1) & 7).  A fragment read (16 rows, one chunk
// each) then falls on 16 distinct bank groups, and a staging write (8 lanes per
// row, two rows) too: the LDS bank-conflict counter reads 0 (with rows padded
// to 144 bytes instead it counted 4 extra cycles per fragment read).
constexpr int MID_PITCH = 128;
__device__ __forceinline__ int mid_chunk(int row, int c) { return c ^ ((row >> 1) & 7); }
}

template <int MT, int WN, int WK, int D, bool PK>
__global__ __launch_bounds__(64 * WN * WK) void k_gemm_mid(MidArgs p) {
    constexpr int NW = WN * WK, NT = 64 * NW, BM = 16 * MT;
    constexpr bool ALDS = WN > 1;
    constexpr int STAGE = WK * BM * MID_PITCH;        // one step's groups of the CTA's rows
    constexpr int CHUNKS = WK * BM * 8;               // 16-byte pieces of a step's activation codes
    constexpr int ACH = ALDS ? (CHUNKS + NT - 1) / NT : 2 * MT;  // per thread (staged) or per lane (direct)
    extern __shared__ __align__(16) uint8_t lds[];

    const int64_t K = p.K, N = p.N, M = p.M, G = K / 128;
    const int tid = threadIdx.x, lane = tid & 63, l16 = lane & 15, q = lane >> 4;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int ct = wave % WN, slice = wave / WN;

    // block -> (column block, row block).  Blocks are dealt round-robin to the
    // 8 XCDs; each XCD takes a contiguous range of local ids, and the row blocks
    // of one column block are consecutive ids, so they run together on one XCD
    // and share its weight bytes in L2.
    const int64_t nrb = (M + BM - 1) / BM, nblk = (N / (16 * WN)) * nrb;
    int64_t lid = blockIdx.x;
    if (nblk % 8 == 0) lid = (blockIdx.x % 8) * (nblk / 8) + blockIdx.x / 8;
    const int64_t cb = lid / nrb, rb = lid % nrb;
    const int64_t m0 = rb * BM, n0 = (cb * WN + ct) * 16;
    // K split (gridDim.y = S > 1): this CTA covers K-groups [ks G / S, (ks + 1) G / S)
    const int64_t S = gridDim.y, ks = blockIdx.y;
    const int64_t steps = G / (S * WK), gbase = ks * (G / S);
    const int64_t nbk = __builtin_amdgcn_readfirstlane((int)(n0 / 128));
    const float *wsrow = p.ws + nbk * G;

    // this lane's activation rows (one per row tile), clamped to M - 1
    int64_t arow[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) arow[mt] = min<int64_t>(m0 + 16 * mt + l16, M - 1);

    uint4 wr[D][2];        // weight fragments of a step
    // activation codes of a step (staged pieces, or this lane's fragments), held
    // as plain vectors: as uint4 aggregates the staged copies stay in scratch memory
    u32x4 ar[D][ACH];
    float sr[D][MT];       // the activation scales of this lane's rows for its group of a step
    float wsr[D];          // the weight block scale of a step's group (the same in every lane)

    const uint8_t *wtile = PK ? p.w + (n0 / 16) * G * 2048 + 16 * lane : p.w + (n0 + l16) * K + 16 * q;
    auto issue = [&](int64_t s, int slot) {
        __builtin_amdgcn_sched_barrier(0);
        const int64_t g = gbase + s * WK + slice;
        if (PK) {
            wr[slot][0] = load_nt16(wtile + g * 2048);
            wr[slot][1] = load_nt16(wtile + g * 2048 + 1024);
        } else {
            wr[slot][0] = *(const uint4 *)(wtile + g * 128);
            wr[slot][1] = *(const uint4 *)(wtile + g * 128 + 64);
        }
        if constexpr (ALDS) {
#pragma unroll
            for (int c = 0; c < ACH; ++c) {
                int id = tid + c * NT;
                id = id < CHUNKS ? id : CHUNKS - 1;
                const int kk = id / (BM * 8), r = (id / 8) % BM, c16 = id % 8;
                const int64_t row = min<int64_t>(m0 + r, M - 1);
                ar[slot][c] = *(const u32x4 *)(p.aq + row * K + (gbase + s * WK + kk) * 128 + c16 * 16);
            }
        } else {
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const uint8_t *src = p.aq + arow[mt] * K + g * 128 + 16 * q;
                ar[slot][2 * mt] = *(const u32x4 *)src;
                ar[slot][2 * mt + 1] = *(const u32x4 *)(src + 64);
            }
        }
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) sr[slot][mt] = p.as_t[g * M + arow[mt]];
        wsr[slot] = wsrow[g];  // wave-uniform: a scalar load, which the next step's wait before its barrier covers
        // keep every step's loads in this order, in the prologue as in the loop, so
        // that the waits the compiler derives for the loop hold from its first trip
        // (reordered in the prologue, they forced a drain of the ring every D steps)
        __builtin_amdgcn_sched_barrier(0);
    };

    v4f acc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt] = v4f{0.f, 0.f, 0.f, 0.f};
    const v4f zero = {0.f, 0.f, 0.f, 0.f};

    // step s from ring slot j: stage the activations (ALDS), then one MFMA per row tile
    auto consume = [&](int64_t s, int j) {
        const uint8_t *st = lds + (j & 1) * STAGE;  // D is even or 1 step per chunk: slot parity = step parity
        if constexpr (ALDS) {
#pragma unroll
            for (int c = 0; c < ACH; ++c) {
                const int id = tid + c * NT;
                if (CHUNKS % NT == 0 || id < CHUNKS) {
                    const int kk = id / (BM * 8), r = (id / 8) % BM, c16 = id % 8;
                    const int R = kk * BM + r;
                    *(u32x4 *)(lds + (j & 1) * STAGE + R * MID_PITCH + mid_chunk(R, c16) * 16) = ar[j][c];
                }
            }
            __syncthreads();
        }
        // all of the step's fragments first, then its MFMAs back to back, then the
        // promotions: each MFMA then waits for no LDS read of its own, and each
        // product is promoted MT - 1 MFMAs after it was issued
        const v8i wf = make_frag(wr[j][0], wr[j][1]);
        v8i af[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            if constexpr (ALDS) {
                // chunks q and q + 4 of row R: the second at the first's chunk ^ 4
                const int R = slice * BM + 16 * mt + l16, c0 = mid_chunk(R, q);
                const uint8_t *row = st + R * MID_PITCH;
                af[mt] = make_frag(*(const uint4 *)(row + 16 * c0), *(const uint4 *)(row + 16 * (c0 ^ 4)));
            } else {
                const u32x4 lo = ar[j][2 * mt], hi = ar[j][2 * mt + 1];
                af[mt] = v8i{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
            }
        }
        __builtin_amdgcn_sched_barrier(0);
        v4f pr[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) pr[mt] = mfma_e4m3_16x16x128(wf, af[mt], zero);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const float sc = sr[j][mt] * wsr[j];
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[mt][i] = __builtin_fmaf(pr[mt][i], sc, acc[mt][i]);
        }
    };

    // the planner guarantees steps % D == 0 and steps >= D
#pragma unroll
    for (int j = 0; j < D; ++j) issue(j, j);
    int64_t s0 = 0;
    for (; s0 + D < steps; s0 += D) {
#pragma unroll
        for (int j = 0; j < D; ++j) {
            consume(s0 + j, j);
            issue(s0 + j + D, j);
        }
    }
#pragma unroll
    for (int j = 0; j < D; ++j) consume(s0 + j, j);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) pin_acc(acc[mt]);  // the last step's MFMAs run with every lane enabled

    // ---- sum the K slices in ascending order, round, store
    if constexpr (WK > 1) {
        __syncthreads();  // every wave is done with the staged activations
        v4f *red = (v4f *)lds;  // [wave][MT][64 lanes]
        if (slice > 0) {
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) red[(wave * MT + mt) * 64 + lane] = acc[mt];
        }
        __syncthreads();
        if (slice > 0) return;
#pragma unroll
        for (int sl = 1; sl < WK; ++sl)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) acc[mt] += red[((sl * WN + ct) * MT + mt) * 64 + lane];
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const int64_t m = m0 + 16 * mt + l16;
        if (m >= M) continue;
        if (S > 1)  // fp32 partial [ks][M][N]; a second kernel adds the splits in ascending ks
            *(v4f *)(p.part + (ks * M + m) * N + n0 + 4 * q) = acc[mt];
        else
            *(uint2 *)(p.c + m * N + n0 + 4 * q) = bf16x4_rne(acc[mt][0], acc[mt][1], acc[mt][2], acc[mt][3]);
    }
}

// LDS of a launch: two activation stages (WN > 1) and the slice reduction
static size_t mid_lds(const MidCfg &c) {
    const size_t stages = c.wn > 1 ? 2 * (size_t)c.wk * 16 * c.mt * MID_PITCH : 0;
    const size_t red = c.wk > 1 ? (size_t)c.wn * c.wk * c.mt * 64 * 16 : 0;
    return std::max<size_t>(std::max(stages, red), 16);
}

// Does (mt, wn, wk, depth, ksplit) give a valid launch of this shape?
static bool mid_fits(int64_t M, int64_t K, int64_t N, const MidCfg &c) {
    const int64_t G = K / 128;
    if (M < 1 || (c.mt != 1 && c.mt != 2 && c.mt != 4) || (c.wn != 1 && c.wn != 2 && c.wn != 4) || c.wk < 1 || c.wn * c.wk > 8)
        return false;
    if ((c.wk & (c.wk - 1)) || (c.depth != 1 && c.depth != 2 && c.depth != 4)) return false;
    if (c.ksplit < 1 || c.ksplit > MID_MAX_KSPLIT || G % c.ksplit) return false;
    if (c.wn == 1 && c.mt > 2 && c.depth > 2) return false;  // direct fragments: 8 mt registers a step
    if (c.wn > 1 && c.depth == 1) return false;              // two LDS buffers alternate by step parity
    const int64_t gs = G / c.ksplit;  // K-groups of one split
    return N % (16 * c.wn) == 0 && gs % c.wk == 0 && gs / c.wk >= c.depth && (gs / c.wk) % c.depth == 0;
}

// (mt, wn, wk, depth) for a shape.  A compute unit takes in its CTAs' bytes at
// a rate of its own, so the busiest unit's bytes per K position, (CTAs it
// runs) x (BM + BN), set the time: among row tiles mt = 4, 2, 1 and column
// tiles wn = 4, 2, 1 the fewest such bytes, then the fewest CTAs, then the
// shapes that share activations through LDS (two or four column tiles a CTA),
// then the wider column block; eight waves a CTA (wk = 8 / wn), and the deepest
// load ring (4 steps, else 2) that divides the step count.  (The rule before,
// the fewest CTAs that still give 256, ran 448 CTAs of 32 x 32 at 32 x 4096 x
// 14336, two on most units, where 224 of 32 x 64 move a quarter fewer bytes a
// unit: 15.2 against 18.2 us; over 17 such shapes at K = 4096, N = 2048-14336
// and 24-192 rows, 8-29% faster, one GPU, interleaved runs.)
MidCfg mid_config(int64_t M, int64_t K, int64_t N) {
    MidCfg c{0, 0, 0, 0, 1};
    if (M < 1 || M > 256 || N % 16) return c;
    const int *f = tuning().mid_cfg;  // tuning override
    if (f[0]) {
        const MidCfg o{f[0], f[1], f[2], f[3], f[4] ? f[4] : 1};
        if (mid_fits(M, K, N, o)) return o;
    }
    // long K at up to 64 rows: one row block (BM >= M) of 64-column blocks, K split
    // over the fewest CTAs (2 to 8, dividing K/128) that make 256, its fp32
    // partials summed by the reduce launch: each compute unit then reads
    // (BM + 64) x K / S bytes instead of all of K for a narrower block (measured
    // at N = 4096, K = 14336: 32 rows 21.1 -> 18.3 us, 64 rows 24.2 -> 22.6 us;
    // at K = 4096 and at 128 rows the split does not pay)
    if (M <= 64 && K >= 8192 && N % 64 == 0) {
        const int mt = M <= 16 ? 1 : M <= 32 ? 2 : 4;
        const int64_t ncb = N / 64;
        for (int ks = 2; ks <= MID_MAX_KSPLIT; ++ks) {
            if (ncb * ks < 256) continue;
            for (const MidCfg t : {MidCfg{mt, 4, 1, 4, ks}, MidCfg{mt, 4, 1, 2, ks}, MidCfg{mt, 4, 2, 2, ks}})
                if (mid_fits(M, K, N, t)) return t;
        }
    }
    const int mtmax = (int)std::min<int64_t>((M + 15) / 16, 4);
    MidCfg best{0, 0, 0, 0, 1};
    int64_t best_ctas = 0, best_unit = 0;
    for (int mt : {4, 2, 1}) {
        if (mt > mtmax && mt != 1) continue;
        for (int wn : {4, 2, 1}) {
            MidCfg t{0, 0, 0, 0, 1};
            for (int wk = 8 / wn; wk >= 1 && !t.mt; wk /= 2)
                for (int d : {4, 2, 1})
                    if (!t.mt && mid_fits(M, K, N, MidCfg{mt, wn, wk, d, 1})) t = MidCfg{mt, wn, wk, d, 1};
            if (!t.mt) continue;
            const int64_t ctas = ((M + 16 * mt - 1) / (16 * mt)) * (N / (16 * wn));
            // bytes a K position costs the busiest compute unit (its CTAs' rows and columns)
            const int64_t unit = (ctas + 255) / 256 * (16 * mt + 16 * wn);
            bool better;
            if (!best.mt) better = true;
            else if (unit != best_unit) better = unit < best_unit;
            else if (ctas != best_ctas) better = ctas < best_ctas;
            else if ((best.wn > 1) != (wn > 1)) better = wn > 1;
            else better = wn > best.wn;
            if (better) {
                best = t;
                best_ctas = ctas;
                best_unit = unit;
            }
        }
    }
    return best;
}

template <int MT, int WN, int WK, int D, bool PK>
static hipError_t launch_mid_one(const MidArgs &a, const MidCfg &c, hipStream_t s) {
    static std::once_flag once[64];
    static hipError_t attr_err[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    std::call_once(once[dev], [&] {
        attr_err[dev] = hipFuncSetAttribute((const void *)k_gemm_mid<MT, WN, WK, D, PK>,
                                            hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    });
    if (attr_err[dev] != hipSuccess) return attr_err[dev];
    const int64_t nblk = (a.N / (16 * WN)) * ((a.M + 16 * MT - 1) / (16 * MT));
    if (c.ksplit > 1 && !a.part) return hipErrorInvalidValue;
    hipLaunchKernelGGL((k_gemm_mid<MT, WN, WK, D, PK>), dim3((unsigned)nblk, (unsigned)c.ksplit),
                       dim3(64 * WN * WK), mid_lds(c), s, a);
    return hipGetLastError();
}

template <int MT, int WN, int WK, bool PK>
static hipError_t launch_mid_d(const MidArgs &a, const MidCfg &c, hipStream_t s) {
    switch (c.depth) {
        case 4: if constexpr (WN > 1 || MT <= 2) return launch_mid_one<MT, WN, WK, 4, PK>(a, c, s); break;
        case 2: return launch_mid_one<MT, WN, WK, 2, PK>(a, c, s);
        case 1: if constexpr (WN == 1) return launch_mid_one<MT, WN, WK, 1, PK>(a, c, s); break;
    }
    return hipErrorInvalidValue;
}

template <int MT, int WN, bool PK>
static hipError_t launch_mid_wk(const MidArgs &a, const MidCfg &c, hipStream_t s) {
    switch (c.wk) {
        case 8: if constexpr (WN == 1) return launch_mid_d<MT, WN, 8, PK>(a, c, s); break;
        case 4: if constexpr (WN <= 2) return launch_mid_d<MT, WN, 4, PK>(a, c, s); break;
        case 2: return launch_mid_d<MT, WN, 2, PK>(a, c, s);
        case 1: return launch_mid_d<MT, WN, 1, PK>(a, c, s);
    }
    return hipErrorInvalidValue;
}

template <int MT, bool PK>
static hipError_t launch_mid_wn(const MidArgs &a, const MidCfg &c, hipStream_t s) {
    switch (c.wn) {
        case 4: return launch_mid_wk<MT, 4, PK>(a, c, s);
        case 2: return launch_mid_wk<MT, 2, PK>(a, c, s);
        case 1: return launch_mid_wk<MT, 1, PK>(a, c, s);
    }
    return hipErrorInvalidValue;
}

template <bool PK>
static hipError_t launch_mid_mt(const MidArgs &a, const MidCfg &c, hipStream_t s) {
    switch (c.mt) {
        case 1: return launch_mid_wn<1, PK>(a, c, s);
        case 2: return launch_mid_wn<2, PK>(a, c, s);
        case 4: return launch_mid_wn<4, PK>(a, c, s);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_gemm_mid(const MidArgs &a, const MidCfg &c, hipStream_t s) {
    const hipError_t e = a.packed ? launch_mid_mt<true>(a, c, s) : launch_mid_mt<false>(a, c, s);
    if (e != hipSuccess || c.ksplit == 1) return e;
    return launch_splitk_reduce(a.part, a.c, a.M, a.N, c.ksplit, s);
}

// Workspace bytes of the K split's fp32 partials [ksplit][M][N] (0 without one)
size_t mid_partial_bytes(int64_t M, int64_t K, int64_t N) {
    const MidCfg c = mid_config(M, K, N);
    return c.mt && c.ksplit > 1 ? align_up(sizeof(float) * (size_t)c.ksplit * M * N, 256) : 0;
}

}  // namespace r9k
