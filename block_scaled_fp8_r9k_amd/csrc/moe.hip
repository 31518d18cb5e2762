// Engine (c): routed MoE decode with block-scaled fp8 experts.
//
// The r9700-stack release v0.3.3 notes ("What changed for someone running it")
// describe the fused MoE decode path: silu(gate) * up in the gate_up GEMM's
// epilogue and the fp8 row quant inside the down GEMM's A-load, bit-identical
// to the three-launch path (gate_up GEMM, silu*up with the quant, down GEMM).
// Both paths are here; both end with the weighted combine over the top-k.
//
// Decode MoE is a weight stream over the experts the tokens touch.  Every
// kernel's grid covers all E experts (it never depends on routing data); a
// CTA first collects, in ascending order, the (token, slot) pairs routed to its
// expert, and leaves at once if there are none.  The pairs are the rows of a
// skinny GEMM against that expert's weights, organised like the dense skinny
// engine: weight bytes straight into MFMA registers with 16-byte loads, the
// pairs' activation codes in LDS, one e4m3 16x16x128 MFMA per 16x16 tile and
// K-group, promotion acc += P * as * ws per group.
//   gate_up: CTA = (expert, 64-column tile j); each wave holds gate columns
//            [64 j + 16 w, +16) and the matching up columns I + the same, so
//            its lanes own gate and up of the same (pair, column).
//   down:    CTA = (expert, 128-column tile of H).
// A pair p = t * topk + j is a row everywhere; intermediates are indexed by p.
#include "r9k_device.h"
#include "r9k_internal.h"

namespace r9k {

namespace {

enum Mode { GATEUP_STORE = 0, GATEUP_SILU = 1, DOWN_QUANT = 2, DOWN_CODES = 3 };

// gate_up: column tiles of 16 per wave (half gate, half up) and the gate
// columns of a CTA (four waves).  A CTA of 64 gate + 64 up columns streams 256
// KiB of an expert's weights at H = 2048; at the decode workload (16 tokens,
// top-8 of 128 experts) its 1032 working CTAs spread over the compute units
// evenly enough, where 128 + 128 columns (516 CTAs of 512 KiB, two or three a
// unit) left the units with three behind: the MoE call took 75 us against 84.
constexpr int GU_NCT = 2, GU_COLS = 4 * 16 * GU_NCT / 2;
// down: column tiles of 16 per wave and the columns of a CTA (96 KiB of weights
// at I = 768; CTAs of 64 columns measured the same)
constexpr int DN_NCT = 2, DN_COLS = 4 * 16 * DN_NCT;

constexpr int MAX_PAIRS = 4096;

// silu(g) * u in fp32, rounded to bf16: the single definition both paths use.
__device__ __forceinline__ uint32_t silu_mul_bf16(float g, float u) {
    const float sg = g / (1.0f + expf(-g));
    return bf16_rne(sg * u);
}

// Collect the pairs routed to expert e, ascending, into list[]; returns count.
__device__ int gather_pairs(const int32_t *ids, int P, int e, int *list, int *wave_cnt) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    int base = 0;
    for (int c0 = 0; c0 < P; c0 += 256) {
        const int idx = c0 + tid;
        const bool hit = idx < P && ids[idx] == e;
        const unsigned long long bal = __ballot(hit);
        if (lane == 0) wave_cnt[wave] = __popcll(bal);
        __syncthreads();
        int off = base;
        for (int w = 0; w < wave; ++w) off += wave_cnt[w];
        if (hit) {
            off += __popcll(bal & ((1ull << lane) - 1ull));
            list[off] = idx;
        }
        int tot = 0;
        for (int w = 0; w < 4; ++w) tot += wave_cnt[w];
        base += tot;
        __syncthreads();
    }
    return base;
}

template <int KC, int MTR>
struct MoeSmem {
    static constexpr int PITCH = KC * 128 + 16;
    uint8_t codes[16 * MTR * PITCH];
    float scales[KC * 16 * MTR];
};

}  // namespace

// One expert GEMM pass.  NCT = column tiles of 16 per wave (GU_NCT for
// gate_up, half gate and half up; 2 for down).  Rows are the expert's pairs in
// tiles of 16, MTR of them a pass: the weight tile streams once per pass, so
// an expert with up to 16 MTR pairs reads its weights once.
// PK: expert weights in fragment order (r9k_pack_weight of [E * 2I][H] and
// [E * H][I]; 16-row tiles never straddle two experts), read in 1 KiB runs.
template <int MODE, int KC, int MTR, bool PK>
__global__ __launch_bounds__(256) void k_moe_gemm(MoeArgs p) {
    constexpr bool GATEUP = MODE == GATEUP_STORE || MODE == GATEUP_SILU;
    constexpr int NCT = GATEUP ? GU_NCT : DN_NCT, HALF = GATEUP ? NCT / 2 : NCT;
    constexpr int PITCH = MoeSmem<KC, MTR>::PITCH, ROWS = 16 * MTR;
    __shared__ MoeSmem<KC, MTR> sm;
    __shared__ int list[MAX_PAIRS];
    __shared__ int wave_cnt[4];

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, l16 = lane & 15, q = lane >> 4;
    const int64_t H = p.H, I = p.I, topk = p.topk;
    const int P = (int)(p.T * topk);
    const int64_t K = GATEUP ? H : I;          // contraction length
    const int64_t G = K / 128;
    const int64_t ntile = GATEUP ? I / GU_COLS : H / DN_COLS;
    const int e = (int)(blockIdx.x / ntile);
    const int64_t j = blockIdx.x % ntile;

    const int cnt = gather_pairs(p.ids, P, e, list, wave_cnt);
    if (cnt == 0) return;

    // weight rows this lane streams, per column tile c
    const uint8_t *wbase;
    const float *wsbase;
    int64_t wrow[NCT];
    if (GATEUP) {
        wbase = p.w13 + (int64_t)e * 2 * I * H;
        wsbase = p.w13s + (int64_t)e * (2 * I / 128) * G;
#pragma unroll
        for (int c = 0; c < NCT; ++c)
            wrow[c] = (c < HALF ? 0 : I) + GU_COLS * j + wave * 16 * HALF + 16 * (c % HALF) + l16;
    } else {
        wbase = p.w2 + (int64_t)e * H * I;
        wsbase = p.w2s + (int64_t)e * (H / 128) * G;
#pragma unroll
        for (int c = 0; c < NCT; ++c) wrow[c] = DN_COLS * j + wave * 16 * NCT + 16 * c + l16;
    }
    const int64_t jb = (GATEUP ? GU_COLS : DN_COLS) * j / 128;  // block row of the gate / down tile
    const float *ws_gate = wsbase + jb * G;
    const float *ws_up = GATEUP ? wsbase + (I / 128 + jb) * G : ws_gate;

    const v4f zero = {0.f, 0.f, 0.f, 0.f};
    const int nb = (int)(G / KC);
    for (int r0 = 0; r0 < cnt; r0 += ROWS) {
        const int rows = min(ROWS, cnt - r0);
        v4f acc[MTR][NCT];
#pragma unroll
        for (int rt = 0; rt < MTR; ++rt)
#pragma unroll
            for (int c = 0; c < NCT; ++c) acc[rt][c] = zero;

        for (int b = 0; b < nb; ++b) {
            const int64_t g0 = (int64_t)b * KC;
            __syncthreads();  // LDS free (previous batch / row tile done)

            // activation side: QA modes quantise a bf16 row group per 16 lanes
            constexpr bool QA = MODE != DOWN_CODES;
            const int task = tid >> 4;  // 16 row groups per pass, KC MTR passes cover 16 MTR rows x KC groups
            uint4 avs[KC * MTR];
            if (QA) {
#pragma unroll
                for (int it = 0; it < KC * MTR; ++it) {
                    const int tk = task + 16 * it;  // tk = row * KC + g
                    if (tk < rows * KC) {
                        const int r = tk / KC, g = tk % KC;
                        const int pr = list[r0 + r];
                        const uint16_t *src = GATEUP ? p.x + (int64_t)(pr / topk) * H : p.h + (int64_t)pr * I;
                        avs[it] = *(const uint4 *)(src + (g0 + g) * 128 + l16 * 8);
                    }
                }
            }

            uint4 wr[KC][NCT][2];
#pragma unroll
            for (int g = 0; g < KC; ++g)
#pragma unroll
                for (int c = 0; c < NCT; ++c) {
                    if (PK) {
                        const uint8_t *src = wbase + ((wrow[c] - l16) / 16 * G + g0 + g) * 2048 + 16 * lane;
                        wr[g][c][0] = load_nt16(src);
                        wr[g][c][1] = load_nt16(src + 1024);
                    } else {
                        const uint8_t *src = wbase + wrow[c] * K + (g0 + g) * 128 + 16 * q;
                        // row-major: two half lines; plain loads (with the
                        // non-temporal hint these ran 10% slower)
                        wr[g][c][0] = *(const uint4 *)src;
                        wr[g][c][1] = *(const uint4 *)(src + 64);
                    }
                }

            // zero rows past the pair count, then fill the valid rows
            for (int i = tid; i < (ROWS - rows) * KC * 8; i += 256) {
                const int r = rows + i / (KC * 8), c16 = i % (KC * 8);
                *(uint4 *)&sm.codes[r * PITCH + c16 * 16] = make_uint4(0, 0, 0, 0);
            }
            for (int i = tid; i < (ROWS - rows) * KC; i += 256) sm.scales[(i % KC) * ROWS + rows + i / KC] = 0.0f;
            if (QA) {
#pragma unroll
                for (int it = 0; it < KC * MTR; ++it) {
                    const int tk = task + 16 * it;
                    if (tk < rows * KC) {
                        const int r = tk / KC, g = tk % KC;
                        float s;
                        const uint2 codes = quant_group16(avs[it], s);
                        *(uint2 *)&sm.codes[r * PITCH + g * 128 + l16 * 8] = codes;
                        if (l16 == 0) sm.scales[g * ROWS + r] = s;
                    }
                }
            } else {
                for (int i = tid; i < rows * KC * 8; i += 256) {
                    const int r = i / (KC * 8), c16 = i % (KC * 8);
                    const int pr = list[r0 + r];
                    *(uint4 *)&sm.codes[r * PITCH + c16 * 16] =
                        *(const uint4 *)(p.hq + (int64_t)pr * I + g0 * 128 + c16 * 16);
                }
                for (int i = tid; i < rows * KC; i += 256) {
                    const int r = i / KC, g = i % KC;
                    sm.scales[g * ROWS + r] = p.hs[(int64_t)list[r0 + r] * G + g0 + g];
                }
            }
            __syncthreads();

#pragma unroll
            for (int g = 0; g < KC; ++g) {
                const float wsg = ws_gate[g0 + g], wsu = ws_up[g0 + g];
#pragma unroll
                for (int rt = 0; rt < MTR; ++rt) {
                    const uint8_t *ap = &sm.codes[(16 * rt + l16) * PITCH + g * 128 + 16 * q];
                    const v8i af = make_frag(*(const uint4 *)ap, *(const uint4 *)(ap + 64));
                    const float sa = sm.scales[g * ROWS + 16 * rt + l16];
                    const float sc_g = sa * wsg;
                    const float sc_u = sa * wsu;
#pragma unroll
                    for (int c = 0; c < NCT; ++c) {
                        const v4f pr = mfma_e4m3_16x16x128(make_frag(wr[g][c][0], wr[g][c][1]), af, zero);
                        const float sc = (GATEUP && c >= HALF) ? sc_u : sc_g;
#pragma unroll
                        for (int i = 0; i < 4; ++i) acc[rt][c][i] = __builtin_fmaf(pr[i], sc, acc[rt][c][i]);
                    }
                }
            }
        }

#pragma unroll
        for (int rt = 0; rt < MTR; ++rt)
#pragma unroll
            for (int c = 0; c < NCT; ++c) pin_acc(acc[rt][c]);  // the MFMAs run with every lane enabled
        // epilogue: lane holds rows (pairs) list[r0 + 16 rt + l16], columns 4q + i of each tile c
#pragma unroll
        for (int rt = 0; rt < MTR; ++rt) {
            if (16 * rt + l16 >= rows) continue;
            const int64_t pr = list[r0 + 16 * rt + l16];
            if (MODE == GATEUP_STORE) {
#pragma unroll
                for (int c = 0; c < NCT; ++c) {
                    const int64_t n = wrow[c] - l16 + 4 * q;  // first of the lane's 4 columns
                    *(uint2 *)(p.gu + pr * 2 * I + n) =
                        bf16x4_rne(acc[rt][c][0], acc[rt][c][1], acc[rt][c][2], acc[rt][c][3]);
                }
            } else if (MODE == GATEUP_SILU) {
#pragma unroll
                for (int c = 0; c < HALF; ++c) {
                    uint32_t hb[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const float g = __uint_as_float(bf16_rne(acc[rt][c][i]) << 16);
                        const float u = __uint_as_float(bf16_rne(acc[rt][c + HALF][i]) << 16);
                        hb[i] = silu_mul_bf16(g, u);
                    }
                    const int64_t n = wrow[c] - l16 + 4 * q;
                    *(uint2 *)(p.h + pr * I + n) = make_uint2(hb[0] | (hb[1] << 16), hb[2] | (hb[3] << 16));
                }
            } else {
#pragma unroll
                for (int c = 0; c < NCT; ++c) {
                    const int64_t n = wrow[c] - l16 + 4 * q;
                    *(v4f *)(p.y + pr * H + n) = acc[rt][c];
                }
            }
        }
    }
}

// Three-launch path, middle launch: h = bf16(silu(gate) * up) from the stored
// bf16 gu, then h's group-128 quant.  16 lanes per group, 16 groups per block.
__global__ __launch_bounds__(256) void k_moe_silu_quant(MoeArgs p) {
    const int64_t I = p.I, GI = I / 128;
    const int64_t P = p.T * p.topk;
    const int64_t gid = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
    const int l = threadIdx.x & 15;
    if (gid >= P * GI) return;
    const int64_t pr = gid / GI, g = gid % GI;
    const uint4 gv = *(const uint4 *)(p.gu + pr * 2 * I + g * 128 + l * 8);
    const uint4 uv = *(const uint4 *)(p.gu + pr * 2 * I + I + g * 128 + l * 8);
    uint4 hv;
    hv.x = silu_mul_bf16(bf16_lo(gv.x), bf16_lo(uv.x)) | (silu_mul_bf16(bf16_hi(gv.x), bf16_hi(uv.x)) << 16);
    hv.y = silu_mul_bf16(bf16_lo(gv.y), bf16_lo(uv.y)) | (silu_mul_bf16(bf16_hi(gv.y), bf16_hi(uv.y)) << 16);
    hv.z = silu_mul_bf16(bf16_lo(gv.z), bf16_lo(uv.z)) | (silu_mul_bf16(bf16_hi(gv.z), bf16_hi(uv.z)) << 16);
    hv.w = silu_mul_bf16(bf16_lo(gv.w), bf16_lo(uv.w)) | (silu_mul_bf16(bf16_hi(gv.w), bf16_hi(uv.w)) << 16);
    *(uint4 *)(p.h + pr * I + g * 128 + l * 8) = hv;
    float s;
    const uint2 codes = quant_group16(hv, s);
    *(uint2 *)(p.hq + pr * I + g * 128 + l * 8) = codes;
    if (l == 0) p.hs[pr * GI + g] = s;
}

// out[t][n] = bf16(sum_j w[t][j] * y[t*topk + j][n]), j ascending, fp32 fma.
// Pairs whose expert id is out of range contribute nothing.  4 columns per
// thread; the slots' loads go out 8 at a time, so that the sum waits for one
// round trip per 8 slots (a slot past topk, or with an invalid id, reads an
// existing y row and discards it).
__global__ __launch_bounds__(256) void k_moe_combine(MoeArgs p) {
    constexpr int SL = 8;
    const int64_t H = p.H, topk = p.topk;
    const int64_t t = blockIdx.y;
    const int64_t n = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
    if (n >= H) return;
    v4f acc = {0.f, 0.f, 0.f, 0.f};
    for (int64_t j0 = 0; j0 < topk; j0 += SL) {
        bool use[SL];
        float w[SL];
        v4f y[SL];
#pragma unroll
        for (int jj = 0; jj < SL; ++jj) {
            const int64_t j = j0 + jj;
            const int64_t pr = t * topk + (j < topk ? j : topk - 1);
            const int32_t e = p.ids[pr];
            use[jj] = j < topk && e >= 0 && e < p.E;
            w[jj] = p.tw[pr];
            y[jj] = *(const v4f *)(p.y + pr * H + n);
        }
#pragma unroll
        for (int jj = 0; jj < SL; ++jj)
            if (use[jj]) {
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[i] = __builtin_fmaf(w[jj], y[jj][i], acc[i]);
            }
    }
    if (p.shared) {  // the shared expert's term, g * s, added before the one rounding
        const float g = p.shared_w ? p.shared_w[t] : 1.0f;
        const uint2 sv = *(const uint2 *)(p.shared + t * H + n);
        acc[0] = __builtin_fmaf(g, bf16_lo(sv.x), acc[0]);
        acc[1] = __builtin_fmaf(g, bf16_hi(sv.x), acc[1]);
        acc[2] = __builtin_fmaf(g, bf16_lo(sv.y), acc[2]);
        acc[3] = __builtin_fmaf(g, bf16_hi(sv.y), acc[3]);
    }
    *(uint2 *)(p.out + t * H + n) = bf16x4_rne(acc[0], acc[1], acc[2], acc[3]);
}

// MoE routing in one launch (release v0.3.0, "What changed for someone running
// it": one-launch MoE routing), one wave per token.  The experts are the topk
// largest logits, a larger logit first and equal logits in ascending expert id
// (the softmax is increasing, so these are the topk largest probabilities).
// Round j takes the first expert, in that order, among those after round
// j - 1's choice, so nothing needs marking: each lane scans its strided share
// of the logits (the first 8 per lane held in registers), then the wave keeps
// the first of the 64 candidates.  Lane j keeps choice j (topk <= 64).  The
// weights are the probabilities renormalised over the chosen experts, in
// which the softmax's denominator cancels: w_j = exp(l_j - l_0) / sum_i
// exp(l_i - l_0), in fp32.
namespace {
constexpr int ROUTE_RV = 8;  // logits a lane holds in registers (E <= 512 needs no reload)

// (v, e) comes first: the larger logit, or the lower id among equal ones
__device__ __forceinline__ bool route_first(float v, int e, float bv, int be) {
    return v > bv || (v == bv && e < be);
}
__device__ __forceinline__ void route_keep(float v, int e, float &bv, int &be) {
    if (route_first(v, e, bv, be)) {
        bv = v;
        be = e;
    }
}
// One DPP step of the wave reduction: the partner lane's candidate, kept if it comes first.
template <int CTRL>
__device__ __forceinline__ void route_dpp(float &bv, int &be) {
    const float ov = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(bv), CTRL, 0xF, 0xF, false));
    const int oe = __builtin_amdgcn_mov_dpp(be, CTRL, 0xF, 0xF, false);
    route_keep(ov, oe, bv, be);
}
template <int CTRL>
__device__ __forceinline__ float sum_dpp(float x) {
    return x + __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, false));
}
// quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_half_mirror, row_mirror: after
// these every lane of a 16-lane row holds the row's result
constexpr int DPP_Q1 = 0xB1, DPP_Q2 = 0x4E, DPP_HALF_MIRROR = 0x141, DPP_MIRROR = 0x140;
}  // namespace

__global__ __launch_bounds__(256) void k_moe_route(const float *__restrict__ logits, int64_t T, int64_t E, int topk,
                                                   int32_t *__restrict__ ids, float *__restrict__ w) {
    const int lane = threadIdx.x & 63;
    const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;  // uniform across the wave
    const float *row = logits + t * E;
    float lv[ROUTE_RV];
#pragma unroll
    for (int r = 0; r < ROUTE_RV; ++r) {
        const int64_t e = lane + 64 * r;
        lv[r] = e < E ? row[e] : 0.0f;
    }
    float pv = __builtin_inff();  // the previous choice; every expert comes after (+inf, -1)
    int pe = -1;
    float my_v = 0.0f;
    int my_e = 0;
    for (int j = 0; j < topk; ++j) {
        float bv = -__builtin_inff();
        int be = 0x7fffffff;
        auto consider = [&](float v, int e) {
            if ((v < pv || (v == pv && e > pe)) && route_first(v, e, bv, be)) {
                bv = v;
                be = e;
            }
        };
#pragma unroll
        for (int r = 0; r < ROUTE_RV; ++r)
            if (lane + 64 * r < E) consider(lv[r], lane + 64 * r);
        for (int64_t e = lane + 64 * ROUTE_RV; e < E; e += 64) consider(row[e], (int)e);
        route_dpp<DPP_Q1>(bv, be);
        route_dpp<DPP_Q2>(bv, be);
        route_dpp<DPP_HALF_MIRROR>(bv, be);
        route_dpp<DPP_MIRROR>(bv, be);
        float cv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(bv), 0));
        int ce = __builtin_amdgcn_readlane(be, 0);
#pragma unroll
        for (int rr = 16; rr < 64; rr += 16)
            route_keep(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(bv), rr)),
                       __builtin_amdgcn_readlane(be, rr), cv, ce);
        pv = cv;
        pe = ce;
        if (lane == j) {
            my_v = cv;
            my_e = ce;
        }
    }
    const float l0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_v), 0));
    const float ex = lane < topk ? expf(my_v - l0) : 0.0f;
    // the sum over the chosen slots: the same value in every lane of a row,
    // then the four rows added in a fixed order
    float rs = sum_dpp<DPP_Q1>(ex);
    rs = sum_dpp<DPP_Q2>(rs);
    rs = sum_dpp<DPP_HALF_MIRROR>(rs);
    rs = sum_dpp<DPP_MIRROR>(rs);
    const float s01 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(rs), 0)) +
                      __int_as_float(__builtin_amdgcn_readlane(__float_as_int(rs), 16));
    const float s23 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(rs), 32)) +
                      __int_as_float(__builtin_amdgcn_readlane(__float_as_int(rs), 48));
    const float sum = s01 + s23;
    if (lane < topk) {
        ids[t * topk + lane] = my_e;
        w[t * topk + lane] = ex / sum;
    }
}

hipError_t launch_moe_route(const float *logits, int64_t T, int64_t E, int topk, int32_t *ids, float *w,
                            hipStream_t s) {
    hipLaunchKernelGGL(k_moe_route, dim3((unsigned)((T + 3) / 4)), dim3(256), 0, s, logits, T, E, topk, ids, w);
    return hipGetLastError();
}

MoeLayout moe_layout(int64_t T, int64_t H, int64_t E, int64_t I, int64_t topk) {
    (void)E;
    const size_t P = (size_t)(T * topk);
    MoeLayout L;
    size_t off = 0;
    L.gu = off; off = align_up(off + P * 2 * I * 2, 256);
    L.h = off;  off = align_up(off + P * I * 2, 256);
    L.hq = off; off = align_up(off + P * I, 256);
    L.hs = off; off = align_up(off + P * (I / 128) * 4, 256);
    L.y = off;  off = align_up(off + P * H * 4, 256);
    L.total = off;
    return L;
}

template <int MODE, int MTR, bool PK>
static hipError_t launch_kc(const MoeArgs &a, int kc, dim3 grid, hipStream_t s) {
    switch (kc) {
        // (two row tiles a pass take K batches of at most 3)
        case 8: if constexpr (MTR == 1) { hipLaunchKernelGGL((k_moe_gemm<MODE, 8, MTR, PK>), grid, dim3(256), 0, s, a); break; }
                return hipErrorInvalidValue;
        case 6: if constexpr (MTR == 1) { hipLaunchKernelGGL((k_moe_gemm<MODE, 6, MTR, PK>), grid, dim3(256), 0, s, a); break; }
                return hipErrorInvalidValue;
        case 4: if constexpr (MTR == 1) { hipLaunchKernelGGL((k_moe_gemm<MODE, 4, MTR, PK>), grid, dim3(256), 0, s, a); break; }
                return hipErrorInvalidValue;
        case 3: hipLaunchKernelGGL((k_moe_gemm<MODE, 3, MTR, PK>), grid, dim3(256), 0, s, a); break;
        case 2: hipLaunchKernelGGL((k_moe_gemm<MODE, 2, MTR, PK>), grid, dim3(256), 0, s, a); break;
        default: hipLaunchKernelGGL((k_moe_gemm<MODE, 1, MTR, PK>), grid, dim3(256), 0, s, a); break;
    }
    return hipGetLastError();
}

// Row tiles a pass: two once an expert gets 10 pairs on average (the launch
// cannot see the routing), with smaller K batches to keep two waves a SIMD.
// H = 2048, 128 experts of 768, top-8, fused call: 256 tokens 148.5 against
// 180.4 us, 192 tokens 136-139 against 145.6; 128 tokens (8 on average) the
// same; with the one-pass K batches two row tiles were slower below 256 tokens,
// and four row tiles slower everywhere.  R9K_MOE_MTR overrides (tuning).
static int moe_row_tiles(const MoeArgs &a) {
    if (const int v = tuning().moe_mtr) {
        if (v == 1 || v == 2) return v;
    }
    return a.T * a.topk >= 10 * a.E ? 2 : 1;
}

// compute units of the chip: a grid up to this many CTAs runs in one wave, one CTA each
constexpr int64_t MOE_ONE_PER_CU_CTAS = 256;

template <int MODE>
static hipError_t launch_gemm_mode(const MoeArgs &a, hipStream_t s) {
    constexpr bool GATEUP = MODE == GATEUP_STORE || MODE == GATEUP_SILU;
    const int64_t G = (GATEUP ? a.H : a.I) / 128;
    const int64_t ntile = GATEUP ? a.I / GU_COLS : a.H / DN_COLS;
    const dim3 grid((unsigned)(a.E * ntile));
    // the largest K batch within the register budget that divides K/128
    // (gate_up at 8: 254 VGPRs, one wave a SIMD, 10% slower; at 2: 1-2% slower;
    // down at 2 or 3 instead of 6: the same time).  When the CTAs that hold
    // pairs fit one a compute unit, occupancy buys nothing and gate_up takes 8
    // too: twice the bytes in flight a round trip (1-2 tokens over 128 experts
    // of 768: 4-6% faster; at 3 CTAs in 2 compute units, 6% slower).
    const int mtr = moe_row_tiles(a);
    const int64_t busy_ctas = std::min<int64_t>(a.E, a.T * a.topk) * ntile;  // at most
    const bool one_per_cu = mtr == 1 && busy_ctas <= MOE_ONE_PER_CU_CTAS;
    const int kcmax = mtr > 1 ? (GATEUP ? 2 : 3) : (GATEUP && !one_per_cu) ? 4 : 8;
    int kc = 1;
    for (int cand : {8, 6, 4, 3, 2, 1})
        if (cand <= kcmax && G % cand == 0) { kc = cand; break; }
    switch (mtr) {
        case 2: return a.packed ? launch_kc<MODE, 2, true>(a, kc, grid, s) : launch_kc<MODE, 2, false>(a, kc, grid, s);
        default: return a.packed ? launch_kc<MODE, 1, true>(a, kc, grid, s) : launch_kc<MODE, 1, false>(a, kc, grid, s);
    }
}

hipError_t launch_moe_decode(const MoeArgs &a, bool fused, hipStream_t s) {
    hipError_t e;
    if (fused) {
        if ((e = launch_gemm_mode<GATEUP_SILU>(a, s)) != hipSuccess) return e;
        if ((e = launch_gemm_mode<DOWN_QUANT>(a, s)) != hipSuccess) return e;
    } else {
        if ((e = launch_gemm_mode<GATEUP_STORE>(a, s)) != hipSuccess) return e;
        const int64_t ngroups = a.T * a.topk * (a.I / 128);
        hipLaunchKernelGGL(k_moe_silu_quant, dim3((unsigned)((ngroups + 15) / 16)), dim3(256), 0, s, a);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        if ((e = launch_gemm_mode<DOWN_CODES>(a, s)) != hipSuccess) return e;
    }
    hipLaunchKernelGGL(k_moe_combine, dim3((unsigned)((a.H / 4 + 255) / 256), (unsigned)a.T), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace r9k
