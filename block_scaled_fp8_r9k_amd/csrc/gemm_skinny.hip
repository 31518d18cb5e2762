// Engine (a): the skinny-M, weight-streaming block-scaled fp8 GEMM.
//
// Decode widths (the r9700-stack release v0.3.1 notes: up to 16 tokens; release
// v0.3.2: any row count up to 255) stream every weight byte from HBM once, so
// the kernel is built around the weight stream:
//   - a CTA owns 128 output columns (one row of 128x128 weight blocks) and kc
//     consecutive K-groups; all of its weight bytes are requested up front with
//     16-byte loads straight into the registers that feed the MFMA (no LDS for
//     weights), so a CTA keeps 16*kc KiB in flight;
//   - while those loads fly, the CTA quantises its few activation rows for its
//     K range into LDS, 16 lanes per 128-value group, reducing the group
//     maximum with DPP row operations (the fused A-load of r9k_gemm_fp8_block_qa),
//     or copies pre-quantised codes there (the split form);
//   - per K-group, one e4m3 16x16x128 MFMA per 16x16 output tile gives the
//     group's exact-product sum P in fp32, which is promoted into the fp32
//     accumulator as acc += P * as[m,g] * ws[n/128,g];
//   - ksplit CTAs share an output tile; each writes its fp32 partial to the
//     workspace and a second kernel sums the partials in ascending split order
//     (the result does not depend on which CTA finishes first) and rounds to
//     bf16.
// MFMA roles: the weight rows are the MFMA's A operand (16 n-rows), the
// activation rows its B operand (16 m-columns), so a lane's four outputs are
// four consecutive n of one row m: one 8-byte bf16 store.
// K order inside a 128-group: lane quarter q = l/16 feeds bytes [16q, 16q+16)
// and [64+16q, 64+16q+16) of the group for both operands.  Any order is the
// same sum; this one makes each of the two 16-byte weight loads cover 64
// contiguous bytes of a row across the four lane quarters.
#include "r9k_device.h"
#include "r9k_internal.h"

namespace r9k {

template <int MT, int KC>
struct SkinnySmem {
    static constexpr int ROWS = MT * 16;
    static constexpr int PITCH = KC * 128 + 16;  // +16 B: rows of a lane column fall on distinct banks
    uint8_t codes[ROWS * PITCH];
    float scales[KC * ROWS];
};

// PK: weights in fragment order (r9k_pack_weight); the same registers come
// from 1 KiB contiguous runs instead of 16 rows x 64 bytes.
template <int MT, int KC, bool QA, bool PK>
__global__ __launch_bounds__(256) void k_gemm_skinny(SkinnyArgs p, int ksplit, int nb) {
    using Smem = SkinnySmem<MT, KC>;
    constexpr int ROWS = Smem::ROWS, PITCH = Smem::PITCH;
    __shared__ Smem sm;

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, l16 = lane & 15, q = lane >> 4;
    const int64_t K = p.K, N = p.N, G = K / 128;
    const int64_t nt = blockIdx.x / ksplit;
    const int ks = blockIdx.x % ksplit;
    const int64_t m_base = (int64_t)blockIdx.y * ROWS;
    const int rows = (int)min<int64_t>(ROWS, p.M - m_base);
    const int64_t n_wave = nt * 128 + wave * 32;

    // rows past M: zero codes and zero scales, written once, never overwritten
    {
        const int pad_u4 = (ROWS - rows) * (KC * 8);
        for (int i = tid; i < pad_u4; i += 256) {
            const int r = rows + i / (KC * 8), c16 = i % (KC * 8);
            *(uint4 *)&sm.codes[r * PITCH + c16 * 16] = make_uint4(0, 0, 0, 0);
        }
        for (int i = tid; i < (ROWS - rows) * KC; i += 256) {
            const int r = rows + i / KC, g = i % KC;
            sm.scales[g * ROWS + r] = 0.0f;
        }
    }

    v4f acc[MT][2];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int c = 0; c < 2; ++c) acc[mt][c] = v4f{0.f, 0.f, 0.f, 0.f};
    const v4f zero = {0.f, 0.f, 0.f, 0.f};

    constexpr int PASSES = (ROWS * KC + 15) / 16;  // activation groups per 16-lane row, per batch
    const int tasks = rows * KC;

    for (int b = 0; b < nb; ++b) {
        const int64_t g0 = ((int64_t)ks * nb + b) * KC;
        if (b > 0) __syncthreads();  // the previous batch's LDS reads are done

        // ---- activation loads first (their wait then does not cover the weights)
        uint4 av[QA ? PASSES : 1];
        if (QA) {
#pragma unroll
            for (int it = 0; it < PASSES; ++it) {
                const int task = (tid >> 4) + 16 * it;
                if (task < tasks) {
                    const int r = task / KC, g = task % KC;
                    av[it] = *(const uint4 *)(p.a + (m_base + r) * K + (g0 + g) * 128 + l16 * 8);
                }
            }
        }

        // ---- the weight stream: this batch's bytes, straight into MFMA registers
        uint4 wr[KC][2][2];
#pragma unroll
        for (int g = 0; g < KC; ++g)
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                if (PK) {
                    const uint8_t *src = p.w + (((n_wave + 16 * c) / 16) * G + g0 + g) * 2048 + 16 * lane;
                    wr[g][c][0] = load_nt16(src);
                    wr[g][c][1] = load_nt16(src + 1024);
                } else {
                    const uint8_t *src = p.w + (n_wave + 16 * c + l16) * K + (g0 + g) * 128 + 16 * q;
                    // row-major: two half lines; plain loads (with the
                    // non-temporal hint these ran 13% slower)
                    wr[g][c][0] = *(const uint4 *)src;
                    wr[g][c][1] = *(const uint4 *)(src + 64);
                }
            }

        // ---- A side into LDS: codes [row][batch K range], scales [g][row]
        if (QA) {
#pragma unroll
            for (int it = 0; it < PASSES; ++it) {
                const int task = (tid >> 4) + 16 * it;
                if (task < tasks) {  // uniform across the 16 lanes of a group
                    const int r = task / KC, g = task % KC;
                    float s;
                    const uint2 codes = quant_group16(av[it], s);
                    *(uint2 *)&sm.codes[r * PITCH + g * 128 + l16 * 8] = codes;
                    if (l16 == 0) sm.scales[g * ROWS + r] = s;
                }
            }
        } else {
            const int n_u4 = rows * (KC * 8);
            for (int i = tid; i < n_u4; i += 256) {
                const int r = i / (KC * 8), c16 = i % (KC * 8);
                *(uint4 *)&sm.codes[r * PITCH + c16 * 16] =
                    *(const uint4 *)(p.aq + (m_base + r) * K + g0 * 128 + c16 * 16);
            }
            for (int i = tid; i < rows * KC; i += 256) {
                const int r = i / KC, g = i % KC;
                sm.scales[g * ROWS + r] = p.as[(m_base + r) * G + g0 + g];
            }
        }
        __syncthreads();

        // ---- MFMA per group, promotion acc += P * as * ws
        const float *wsrow = p.ws + nt * G + g0;
#pragma unroll
        for (int g = 0; g < KC; ++g) {
            const float swg = wsrow[g];
            const v8i wf0 = make_frag(wr[g][0][0], wr[g][0][1]);
            const v8i wf1 = make_frag(wr[g][1][0], wr[g][1][1]);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const int row = mt * 16 + l16;
                const uint8_t *ap = &sm.codes[row * PITCH + g * 128 + 16 * q];
                const v8i af = make_frag(*(const uint4 *)ap, *(const uint4 *)(ap + 64));
                const float sc = sm.scales[g * ROWS + row] * swg;
                const v4f p0 = mfma_e4m3_16x16x128(wf0, af, zero);
                const v4f p1 = mfma_e4m3_16x16x128(wf1, af, zero);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    acc[mt][0][i] = __builtin_fmaf(p0[i], sc, acc[mt][0][i]);
                    acc[mt][1][i] = __builtin_fmaf(p1[i], sc, acc[mt][1][i]);
                }
            }
        }
    }

#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int c = 0; c < 2; ++c) pin_acc(acc[mt][c]);  // the MFMAs run with every lane enabled

    // ---- epilogue
    // lane's outputs: rows m = m_base + 16 mt + l16, columns n = n_wave + 16 c + 4 q + i
    if (ksplit == 1) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const int r = mt * 16 + l16;
            if (r < rows) {
#pragma unroll
                for (int c = 0; c < 2; ++c) {
                    const int64_t n = n_wave + 16 * c + 4 * q;
                    *(uint2 *)(p.c + (m_base + r) * N + n) =
                        bf16x4_rne(acc[mt][c][0], acc[mt][c][1], acc[mt][c][2], acc[mt][c][3]);
                }
            }
        }
        return;
    }

    // split-K: this split's fp32 partial of the tile, part[ks][m][n]; the
    // reduce kernel sums the splits in ascending order
    float *mine = p.part + (int64_t)ks * p.M * N;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const int r = mt * 16 + l16;
        if (r < rows) {
#pragma unroll
            for (int c = 0; c < 2; ++c)
                *(v4f *)(mine + (m_base + r) * N + n_wave + 16 * c + 4 * q) = acc[mt][c];
        }
    }
}

// C[m][n] = bf16(sum over splits, ascending, of part[ks][m][n]); 8 columns a
// thread.  The partials of up to four splits are loaded before they are added,
// so that each thread keeps several loads in flight; the additions still go in
// ascending split order.
__global__ __launch_bounds__(256) void k_splitk_reduce(const float *__restrict__ part, uint16_t *__restrict__ c,
                                                       int64_t MN, int ksplit) {
    const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 8;
    if (i >= MN) return;
    v4f s0 = *(const v4f *)(part + i), s1 = *(const v4f *)(part + i + 4);
    int k = 1;
    for (; k + 4 <= ksplit; k += 4) {
        v4f x[4][2];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const float *pk = part + (int64_t)(k + u) * MN + i;
            x[u][0] = *(const v4f *)pk;
            x[u][1] = *(const v4f *)(pk + 4);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            s0 += x[u][0];
            s1 += x[u][1];
        }
    }
    for (; k < ksplit; ++k) {
        const float *pk = part + (int64_t)k * MN + i;
        s0 += *(const v4f *)pk;
        s1 += *(const v4f *)(pk + 4);
    }
    uint2 lo = bf16x4_rne(s0[0], s0[1], s0[2], s0[3]), hi = bf16x4_rne(s1[0], s1[1], s1[2], s1[3]);
    *(uint4 *)(c + i) = make_uint4(lo.x, lo.y, hi.x, hi.y);
}

// ---- configuration ----------------------------------------------------------

static int kc_max_for(int mt16) { return mt16 <= 2 ? 8 : mt16 == 4 ? 4 : mt16 == 8 ? 2 : 1; }

// Choice of (kc, ksplit, nb) with kc * ksplit * nb = K/128:
//  - a single chunk of rows (M <= 256): the largest kc within the register
//    budget whose smallest ksplit still gives at least two CTAs per compute
//    unit (512), nb = 1 where possible; else kc = 1 and ksplit = K/128;
//  - several row chunks (the skinny engine forced at M > 256): no split, each
//    CTA loops over K in batches of kc groups.
// R9K_SKINNY_KC and R9K_SKINNY_KSPLIT override the choice (tuning).
SkinnyCfg skinny_config(int64_t M, int64_t K, int64_t N) {
    SkinnyCfg c;
    const int64_t rows = M < 256 ? M : 256;
    int mt = 1;
    while (mt * 16 < rows) mt *= 2;
    c.mt16 = mt;
    c.mchunks = (int)((M + mt * 16 - 1) / (mt * 16));
    const int64_t G = K / 128, ntiles = N / 128;
    const int64_t target = 512;
    int kc = 1;
    int64_t ksplit = G;
    if (c.mchunks > 1) {
        for (int cand = kc_max_for(mt); cand >= 1; cand /= 2)
            if (G % cand == 0) { kc = cand; break; }
        ksplit = 1;
    } else {
        bool found = false;
        for (int cand = kc_max_for(mt); cand >= 1 && !found; cand /= 2) {
            if (G % cand) continue;
            const int64_t nk = G / cand;
            for (int64_t d = 1; d <= nk; ++d)
                if (nk % d == 0 && ntiles * d >= target) { kc = cand; ksplit = d; found = true; break; }
        }
        if (!found) { kc = 1; ksplit = G; }
    }
    if (int v = tuning().skinny_kc) {
        if (v >= 1 && v <= kc_max_for(mt) && (v & (v - 1)) == 0 && G % v == 0) {
            kc = v;
            if ((G / kc) % ksplit) ksplit = G / kc;
        }
    }
    if (int64_t v = tuning().skinny_ksplit) {
        if (v >= 1 && c.mchunks == 1 && (G / kc) % v == 0) ksplit = v;
    }
    c.kc = kc;
    c.ksplit = (int)ksplit;
    c.nb = (int)(G / kc / ksplit);
    return c;
}

size_t skinny_partial_bytes(const SkinnyCfg &c, int64_t M, int64_t N) {
    if (c.ksplit <= 1) return 0;
    return align_up(sizeof(float) * (size_t)c.ksplit * M * N, 256);
}

template <int MT, int KC>
static hipError_t launch_mk(const SkinnyArgs &a, const SkinnyCfg &c, hipStream_t s) {
    dim3 grid((unsigned)((a.N / 128) * c.ksplit), (unsigned)c.mchunks);
    if (a.a && a.packed)
        hipLaunchKernelGGL((k_gemm_skinny<MT, KC, true, true>), grid, dim3(256), 0, s, a, c.ksplit, c.nb);
    else if (a.a)
        hipLaunchKernelGGL((k_gemm_skinny<MT, KC, true, false>), grid, dim3(256), 0, s, a, c.ksplit, c.nb);
    else if (a.packed)
        hipLaunchKernelGGL((k_gemm_skinny<MT, KC, false, true>), grid, dim3(256), 0, s, a, c.ksplit, c.nb);
    else
        hipLaunchKernelGGL((k_gemm_skinny<MT, KC, false, false>), grid, dim3(256), 0, s, a, c.ksplit, c.nb);
    return hipGetLastError();
}

template <int MT>
static hipError_t launch_m(const SkinnyArgs &a, const SkinnyCfg &c, hipStream_t s) {
    switch (c.kc) {
        case 1: return launch_mk<MT, 1>(a, c, s);
        case 2: if constexpr (MT <= 8) return launch_mk<MT, 2>(a, c, s); break;
        case 4: if constexpr (MT <= 4) return launch_mk<MT, 4>(a, c, s); break;
        case 8: if constexpr (MT <= 2) return launch_mk<MT, 8>(a, c, s); break;
    }
    return hipErrorInvalidValue;
}

hipError_t launch_gemm_skinny(const SkinnyArgs &a, const SkinnyCfg &c, hipStream_t s) {
    hipError_t e = hipErrorInvalidValue;
    switch (c.mt16) {
        case 1: e = launch_m<1>(a, c, s); break;
        case 2: e = launch_m<2>(a, c, s); break;
        case 4: e = launch_m<4>(a, c, s); break;
        case 8: e = launch_m<8>(a, c, s); break;
        case 16: e = launch_m<16>(a, c, s); break;
    }
    if (e != hipSuccess || c.ksplit == 1) return e;
    return launch_splitk_reduce(a.part, a.c, a.M, a.N, c.ksplit, s);
}

hipError_t launch_splitk_reduce(const float *part, uint16_t *c, int64_t M, int64_t N, int ksplit, hipStream_t s) {
    const int64_t MN = M * N;
    hipLaunchKernelGGL(k_splitk_reduce, dim3((unsigned)((MN / 8 + 255) / 256)), dim3(256), 0, s, part, c, MN, ksplit);
    return hipGetLastError();
}

}  // namespace r9k
