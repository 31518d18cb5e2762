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
// Work split: C^T = W A^T, so that a lane's four outputs of an MFMA tile
// share one row of A, and with it one activation scale; the promotion is one
// multiply per row tile and one FMA per output per group.  Each wave owns TN
// column tiles of 16 (all inside one weight block row: one weight scale per
// group) by four row tiles of 16, two waves per SIMD; the CTA shapes are
// listed with Cfg below.  Per group a wave keeps its four A fragments in
// registers and streams its weight fragments from LDS two column tiles ahead,
// and each MFMA is issued right after the promotion FMAs of the product it
// replaces, so that one register set holds every product in flight.
//
// A stage holds one group: the W tile [BN rows][128 bytes], the A tile
// [BM rows][128 bytes] and the scales; two or three stages, filled one or two
// groups ahead.  Everything moves from global memory straight into LDS
// (global_load_lds, no register staging), so one wait on the wave's load
// counter covers a stage.  A 16-byte load instruction fills 1 KiB of LDS, 8
// rows; lane l writes physical chunk l % 8 of its row and fetches the logical
// chunk that belongs there: chunk c of row r lives at chunk c ^ ((r >> 1) & 7),
// so the 16 rows a fragment read touches in one LDS cycle fall on distinct
// banks.
#include <algorithm>
#include <atomic>
#include <cstdlib>
#include <mutex>

#include "r9k_device.h"
#include "r9k_internal.h"

namespace r9k {

namespace {
// Tile shape: WN x WM waves, each TN x 4 MFMA tiles of 16 x 16 (TN * 16
// columns, 64 rows), two waves per SIMD so that one wave's LDS and barrier
// waits hide behind the other's MFMAs.  Two shapes are built:
//   C: 2 x 4 waves of 8 x 4 tiles, a 256 x 256 CTA tile, two LDS stages;
//   B: 4 x 2 waves of 4 x 4 tiles, a 256 x 128 CTA tile, three LDS stages;
//   M1, M2: 64 columns x 128 / 256 rows, for skinny widths with a K split.
// C reads 0.75 KiB of LDS per MFMA instead of 1 KiB and moves a third less
// from L2 per flop; B makes twice as many CTAs for shapes too small for C.
template <int WN_, int WM_, int TN_, int NST_>
struct Cfg {
    static constexpr int WN = WN_, WM = WM_, TN = TN_, TM = 4;
    static constexpr int NW = WN * WM, THREADS = 64 * NW;
    static constexpr int BN = WN * TN * 16;        // output columns (W rows) per CTA
    static constexpr int BM = WM * TM * 16;        // output rows (A rows) per CTA
    static constexpr int WBYTES = BN * 128;        // W tile of a stage
    static constexpr int ABYTES = BM * 128;        // A tile of a stage
    static constexpr int SBYTES = NW * 2 * 64 * 4; // per wave: 64 activation scales, the weight scale x 64
    static constexpr int STAGE = WBYTES + ABYTES + SBYTES;
    static constexpr int NST = NST_;  // stages in the LDS ring; loads run NST - 1 groups ahead
    static constexpr int SMEM = NST * STAGE;
    static constexpr int WLOADS = BN / 8 / NW, ALOADS = BM / 8 / NW;  // 1 KiB load instructions per wave
    static constexpr int LOADS_PER_STAGE = WLOADS + ALOADS + 2;
    static_assert(SMEM <= 160 * 1024, "LDS");
    static_assert(NST == 2 || NST == 3, "stages");
    static_assert(WLOADS * NW * 8 == BN && ALOADS * NW * 8 == BM, "loads split evenly");
    static_assert(TN * 16 <= 128 && 128 % (TN * 16) == 0, "a wave's columns lie in one weight block row");
};
using CfgB = Cfg<4, 2, 4, 3>;
using CfgC = Cfg<2, 4, 8, 2>;
// narrow tiles for skinny widths (64 columns; all of M up to 128 or 256 rows),
// where the K split, not the tile, gives the CTAs: fewer fp32 partials per
// output than wide tiles split further
using CfgM1 = Cfg<4, 2, 1, 3>;
using CfgM2 = Cfg<2, 4, 2, 3>;

// Global -> LDS loads (lane l's bytes land at LDS address `l_addr` + size * l,
// the address taken from M0).  Issued from inline asm so that the compiler
// neither waits for them at every barrier nor before every LDS read (it cannot
// tell that the reads touch another stage); the kernel waits for them itself
// with wait_vm, counting this wave's load instructions.
__device__ __forceinline__ uint32_t lds_addr(const uint8_t *p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t *)p;
}
// The global address is a wave-uniform base (SGPRs) plus a 32-bit lane offset;
// the LDS address goes in M0, which the compiler sets from the operand.
__device__ __forceinline__ void load_lds16(const void *base, uint32_t off, uint32_t l_addr) {
    asm volatile("global_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(base), "{m0}"(l_addr) : "memory");
}
__device__ __forceinline__ void load_lds4(const void *base, uint32_t off, uint32_t l_addr) {
    asm volatile("global_load_lds_dword %0, %1" ::"v"(off), "s"(base), "{m0}"(l_addr) : "memory");
}

__device__ __forceinline__ int swz(int row, int chunk) { return row * 128 + ((chunk ^ ((row >> 1) & 7)) << 4); }

// an MFMA fragment: 16 bytes at p0 and 16 at p1 (chunks q and q + 4 of a
// swizzled row; the swizzle leaves bit 6 of the chunk offset alone, so the
// second chunk's offset is the first one's with bit 6 flipped)
__device__ __forceinline__ v8i frag2(const uint8_t *p0, const uint8_t *p1) {
    return make_frag(*(const uint4 *)p0, *(const uint4 *)p1);
}

// acc += pr * sc, then pr = the e4m3 MFMA of a and b.  The plain form of the
// instruction, not the one with E8M0 block scales (which would be 1 here):
// back to back it issues every 32.5 clocks against 33.1 for the scaled form.
// Two volatile asm statements, which the compiler keeps in this order: the
// FMAs read the product that an MFMA four calls earlier wrote into pr (long
// done: the caller keeps that distance, which also covers the wait the
// hardware needs before VALU reads an MFMA result), at issue, so that this
// call's MFMA may overwrite the same registers; one register set thus holds
// every product in flight.  The FMAs run while the previous MFMA executes.
__device__ __forceinline__ void promote_mfma(v4f &pr, const v8i &a, const v8i &b, float sc, v4f &acc) {
    float a0 = acc[0], a1 = acc[1], a2 = acc[2], a3 = acc[3];
    asm volatile(
        "v_fmac_f32 %0, %4, %8\n\t"
        "v_fmac_f32 %1, %5, %8\n\t"
        "v_fmac_f32 %2, %6, %8\n\t"
        "v_fmac_f32 %3, %7, %8"
        : "+v"(a0), "+v"(a1), "+v"(a2), "+v"(a3)
        : "v"(pr[0]), "v"(pr[1]), "v"(pr[2]), "v"(pr[3]), "v"(sc));
    asm volatile("v_mfma_f32_16x16x128_f8f6f4 %0, %1, %2, 0" : "=&v"(pr) : "v"(a), "v"(b));
    acc = v4f{a0, a1, a2, a3};
}

// The order of a group's 4 TN MFMAs: MFMA k computes column tile mfma_i, row
// tile mfma_j.  With two or more column tiles, the first eight interleave
// tiles 0 and 1 on rows 0 and 1, then on rows 2 and 3; then tile by tile.
template <int TN>
__device__ constexpr int mfma_i(int k) {
    return TN == 1 ? 0 : k < 4 ? k >> 1 : k < 8 ? (k - 4) >> 1 : k >> 2;
}
template <int TN>
__device__ constexpr int mfma_j(int k) {
    return TN == 1 ? k : k < 4 ? k & 1 : k < 8 ? 2 + (k & 1) : k & 3;
}
// the MFMA after which weight tile t >= 2 is read into slot t % 3: tile 2
// into the free slot at once, tile 3 after tile 0's last MFMA (k = 5), then
// tile t during tile t - 2
__device__ constexpr int wread_k(int t) { return t == 2 ? 0 : t == 3 ? 6 : 4 * (t - 2); }

// wait until at most VM of this wave's vector-memory instructions are in flight
template <int VM>
__device__ __forceinline__ void wait_vm() {
    static_assert(VM >= 0 && VM < 64, "vmcnt");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(VM) : "memory");
}
}  // namespace

// PK: the weights are in fragment order (r9k_pack_weight).  The W tile of a
// stage is then 16 blocks of 2 KiB, [column tile][half][lane][16 bytes], each
// load instruction one half-block (1 KiB contiguous in memory and in LDS), and
// a fragment read is 16 bytes at lane * 16 (no swizzle needed).
template <class C, bool PK>
__global__ __launch_bounds__(C::THREADS, 1) void k_gemm_tiled(TiledArgs p) {
    constexpr int WN = C::WN, TN = C::TN, BN = C::BN, BM = C::BM;
    constexpr int WBYTES = C::WBYTES, ABYTES = C::ABYTES, STAGE = C::STAGE, NST = C::NST;
    extern __shared__ __align__(16) uint8_t lds[];
    const int tid = threadIdx.x, lane = tid & 63, l16 = lane & 15, q = lane >> 4;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wn = wave % WN, wm = wave / WN;
    const int64_t K = p.K, N = p.N, M = p.M, G = K / 128;
    const int64_t ntn = (N + BN - 1) / BN, ntm = (M + BM - 1) / BM;
    // this CTA's K range: groups gb .. gb + GL - 1 of split blockIdx.y
    const int ks = blockIdx.y;
    const int64_t gb = (int64_t)ks * G / p.ksplit, GL = (int64_t)(ks + 1) * G / p.ksplit - gb;

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

    // This wave's loads of a stage: W instructions WLOADS wave + u and A
    // instructions ALOADS wave + u, each 8 rows from row 8 * index + lane / 8,
    // its 64 activation scales, and its weight scale (every lane the same).
    // W rows past N (the upper half of a last, half-full column tile; an
    // instruction's 8 rows are all on one side) read the lower half instead;
    // A rows past M read row M - 1.  Neither is ever stored.
    uint32_t woff[C::WLOADS], aoff[C::ALOADS];
#pragma unroll
    for (int u = 0; u < C::WLOADS; ++u) {
        const int idx = C::WLOADS * wave + u;
        if (PK) {  // column tile idx / 2, half idx % 2
            int t = idx >> 1;
            if (n0 + 16 * t >= N) t -= 8;
            woff[u] = (uint32_t)t * (uint32_t)(G * 2048) + 1024 * (idx & 1) + 16 * lane;
        } else {
            const int row = 8 * idx + (lane >> 3);
            const int chunk = (lane & 7) ^ ((row >> 1) & 7);
            const int wrow = (n0 + 8 * idx < N) ? row : row - 128;
            woff[u] = (uint32_t)wrow * (uint32_t)K + 16 * chunk;
        }
    }
#pragma unroll
    for (int u = 0; u < C::ALOADS; ++u) {
        const int row = 8 * (C::ALOADS * wave + u) + (lane >> 3);
        const int chunk = (lane & 7) ^ ((row >> 1) & 7);
        aoff[u] = (uint32_t)min<int64_t>(row, M - 1 - m0) * (uint32_t)K + 16 * chunk;
    }
    const uint32_t soff = 4u * (uint32_t)min<int64_t>(m0 + 64 * wm + lane, M - 1);
    const int64_t nb = min<int64_t>((n0 + TN * 16 * wn) / 128, N / 128 - 1);
    const uint8_t *wbase = PK ? p.w + (n0 / 16) * G * 2048 : p.w + n0 * K;
    const uint8_t *abase = p.aq + m0 * K;
    const float *wsbase = p.ws + nb * G;
    const uint32_t lds0 = __builtin_amdgcn_readfirstlane(lds_addr(lds));
    // load instructions u0 .. u1 - 1 of this wave's share of group g, into
    // stage st: the W rows first, then the A rows, then the two scale loads
    constexpr int LPS = C::LOADS_PER_STAGE;
    auto issue = [&](int64_t g, int st, int u0, int u1) {
        const uint32_t sb = lds0 + st * STAGE + C::WLOADS * wave * 1024;
        const uint32_t sa = lds0 + st * STAGE + WBYTES + C::ALOADS * wave * 1024;
        const uint32_t ss = lds0 + st * STAGE + WBYTES + ABYTES + wave * 512;
        const uint8_t *wg = wbase + g * (PK ? 2048 : 128), *ag = abase + g * 128;
#pragma unroll
        for (int u = 0; u < C::WLOADS; ++u)
            if (u >= u0 && u < u1) load_lds16(wg, woff[u], sb + u * 1024);
#pragma unroll
        for (int u = 0; u < C::ALOADS; ++u)
            if (C::WLOADS + u >= u0 && C::WLOADS + u < u1) load_lds16(ag, aoff[u], sa + u * 1024);
        if (LPS - 2 >= u0 && LPS - 2 < u1) load_lds4(p.as_t + g * M, soff, ss);
        if (LPS - 1 >= u0 && LPS - 1 < u1) load_lds4(wsbase + g, 0u, ss + 256);
    };
    // With two stages (the 256 x 256 tile) the next stage's loads are spread
    // over the first SPREAD column tiles, PER instructions after each: the
    // compute unit's load unit takes 64 bytes a clock, so a whole stage issued
    // at once by every wave queues for about a thousand clocks, with each
    // wave's MFMAs behind its own loads; the last ones still go out early
    // enough to land before the next group starts (2-3% faster on the MI355X).
    // The three-stage tiles issue a stage at once, right after the barrier,
    // which measured as fast or faster for them.
    constexpr int SPREAD = (TN * 5 + 7) / 8;
    constexpr int PER = (LPS + SPREAD - 1) / SPREAD;

    // fragment addresses inside a stage: column tile i of this wave at
    // wfo + 2048 i (and ^ 64), row tile j at afo + 2048 j (rows 16 apart keep
    // their swizzle)
    const int wfo = PK ? TN * wn * 2048 + 16 * lane : swz(TN * 16 * wn + l16, q);
    const int wfo2 = PK ? wfo + 1024 : wfo ^ 64;
    const int afo = WBYTES + swz(64 * wm + l16, q), afo2 = afo ^ 64;

    v4f acc[TN][4];
#pragma unroll
    for (int i = 0; i < TN; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
    // products of the previous column tile and their scales, zero before the first
    v4f pr[4];
    float scp[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        pr[j] = v4f{0.f, 0.f, 0.f, 0.f};
        scp[j] = 0.f;
    }

#pragma unroll
    for (int k = 0; k < NST - 1; ++k)
        if (k < GL) issue(gb + k, k, 0, LPS);
    for (int64_t gl = 0; gl < GL; ++gl) {
        const int st = (int)(gl % NST);
        // local group gl's stage has landed: this wave's loads issued after it
        // are those of groups gl + 1 .. gl + NST - 2 (three stages: gl + 1, if
        // any); then every wave's, and every wave is done with the stage that
        // group gl + NST - 1 will overwrite
        if (NST == 3 && gl + 1 < GL) wait_vm<C::LOADS_PER_STAGE>();
        else wait_vm<0>();
        __syncthreads();
        const bool more = gl + NST - 1 < GL;
        const int64_t gn = gb + gl + NST - 1;
        const int stn = (int)((gl + NST - 1) % NST);
        if (NST == 3 && more) issue(gn, stn, 0, LPS);

        const uint8_t *wt = lds + st * STAGE;
        const uint8_t *at = wt + WBYTES;
        const float *sl = (const float *)(at + ABYTES + wave * 512);
        // Fragments at the group's start in the order of first use: weight
        // tile 0, A rows 0 and 1, weight tile 1, A rows 2 and 3; later weight
        // tiles are read during the group (wread_k).
        v8i wq[3], af[4];
        wq[0] = frag2(wt + wfo, wt + wfo2);
        af[0] = frag2(wt + afo, wt + afo2);
        af[1] = frag2(wt + afo + 2048, wt + afo2 + 2048);
        if (TN > 1) wq[1] = frag2(wt + wfo + 2048, wt + wfo2 + 2048);
        af[2] = frag2(wt + afo + 4096, wt + afo2 + 4096);
        af[3] = frag2(wt + afo + 6144, wt + afo2 + 6144);
        const float wsg = sl[64 + lane];
        float sc[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) sc[j] = sl[16 * j + l16] * wsg;

        // MFMA k of the group (order: mfma_i / mfma_j) runs together with
        // the promotion of the product of MFMA k - 4 (for k < 4, of the
        // previous group's last four), held in product slot k % 4, so an FMA
        // reads a product four MFMAs old.  The first eight MFMAs take column
        // tiles 0 and 1 with A rows 0 and 1 before rows 2 and 3, so that the
        // group starts on four LDS reads.  Weight tile t is read into slot
        // t % 3 once the tile that used the slot before is done (wread_k).
        // The fragment offsets are constants from one stage base, so every
        // read takes its offset in the instruction and costs no VALU work.
#pragma unroll
        for (int k = 0; k < 4 * TN; ++k) {
            const int i = mfma_i<TN>(k), j = mfma_j<TN>(k);
            const int kp = (k + 4 * TN - 4) % (4 * TN);  // the MFMA whose product this one's FMAs promote
            const int ip = mfma_i<TN>(kp), jp = mfma_j<TN>(kp);
            promote_mfma(pr[k & 3], wq[i % 3], af[j], k < 4 ? scp[jp] : sc[jp], acc[ip][jp]);
#pragma unroll
            for (int t = 2; t < TN; ++t)
                if (k == wread_k(t)) wq[t % 3] = frag2(wt + wfo + 2048 * t, wt + wfo2 + 2048 * t);
            if (NST == 2 && (k & 3) == 3 && (k >> 2) < SPREAD && more)
                issue(gn, stn, PER * (k >> 2), PER * ((k >> 2) + 1));
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) scp[j] = sc[j];
    }
    // the last group's last tile: wait out the MFMA latency, then promote
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
#pragma unroll
    for (int k = 4 * TN - 4; k < 4 * TN; ++k) {
        const int i = mfma_i<TN>(k), j = mfma_j<TN>(k);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[i][j][e] = __builtin_fmaf(pr[k & 3][e], scp[j], acc[i][j][e]);
    }

#pragma unroll
    for (int i = 0; i < TN; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) pin_acc(acc[i][j]);  // the MFMAs run with every lane enabled

    // lane holds, per tile (i, j), row m = m0 + 64 wm + 16 j + l16 and the four
    // columns n = n0 + TN 16 wn + 16 i + 4 q .. +3
    const int64_t nbase = n0 + TN * 16 * wn;
    if (p.ksplit == 1) {
        // bf16 output through LDS: each wave writes its tiles into a row-major
        // copy of the CTA's output tile (rows padded by 16 bytes against bank
        // conflicts), then the CTA stores it in 16-byte pieces, consecutive
        // lanes along a row, so that every store instruction writes whole
        // rows.  Stored straight from the MFMA layout, a store wrote 32
        // contiguous bytes of a row per 16 lanes, and the output write took
        // far longer than its bytes.
        constexpr int PITCH = BN * 2 + 16;
        static_assert(BM * PITCH <= C::SMEM, "the output tile fits in the stages' LDS");
        __syncthreads();  // every wave is done reading the last stage
        if (nbase < N) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = 64 * wm + 16 * j + l16;
#pragma unroll
                for (int i = 0; i < TN; ++i)
                    *(uint2 *)(lds + r * PITCH + 2 * (TN * 16 * wn + 16 * i + 4 * q)) =
                        bf16x4_rne(acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]);
            }
        }
        __syncthreads();
        constexpr int CPR = BN / 8;  // 16-byte pieces per row
        static_assert((BM * CPR) % C::THREADS == 0, "whole passes");
#pragma unroll
        for (int k = 0; k < BM * CPR / C::THREADS; ++k) {
            const int id = k * C::THREADS + tid, r = id / CPR, cc = id % CPR;
            const uint4 v = *(const uint4 *)(lds + r * PITCH + 16 * cc);
            if (m0 + r < M && n0 + 8 * cc < N) *(uint4 *)(p.c + (m0 + r) * N + n0 + 8 * cc) = v;
        }
        return;
    }
    if constexpr (BM * (BN * 4 + 16) <= C::SMEM) {
        // fp32 partials of a K split, through LDS in the same way
        constexpr int PITCH = BN * 4 + 16;
        __syncthreads();
        if (nbase < N) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = 64 * wm + 16 * j + l16;
#pragma unroll
                for (int i = 0; i < TN; ++i) *(v4f *)(lds + r * PITCH + 4 * (TN * 16 * wn + 16 * i + 4 * q)) = acc[i][j];
            }
        }
        __syncthreads();
        constexpr int CPR = BN / 4;
        static_assert((BM * CPR) % C::THREADS == 0, "whole passes");
        float *pbase = p.part + (int64_t)ks * M * N;
#pragma unroll
        for (int k = 0; k < BM * CPR / C::THREADS; ++k) {
            const int id = k * C::THREADS + tid, r = id / CPR, cc = id % CPR;
            const v4f v = *(const v4f *)(lds + r * PITCH + 16 * cc);
            if (m0 + r < M && n0 + 4 * cc < N) *(v4f *)(pbase + (m0 + r) * N + n0 + 4 * cc) = v;
        }
        return;
    }
    if (nbase >= N) return;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int64_t m = m0 + 64 * wm + 16 * j + l16;
        if (m >= M) continue;
        if (p.ksplit > 1) {
            float *prow = p.part + ((int64_t)ks * M + m) * N + nbase + 4 * q;
#pragma unroll
            for (int i = 0; i < TN; ++i) *(v4f *)(prow + 16 * i) = acc[i][j];
        } else {
            uint16_t *crow = p.c + m * N + nbase + 4 * q;
#pragma unroll
            for (int i = 0; i < TN; ++i)
                *(uint2 *)(crow + 16 * i) = bf16x4_rne(acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]);
        }
    }
}

template <class C, bool PK>
static hipError_t launch_cfg(const TiledArgs &a, hipStream_t s) {
    // the dynamic LDS limit is a per-device function attribute: set it once per device
    static std::once_flag once[64];
    static hipError_t attr_err[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    std::call_once(once[dev], [&] {
        attr_err[dev] = hipFuncSetAttribute((const void *)k_gemm_tiled<C, PK>,
                                            hipFuncAttributeMaxDynamicSharedMemorySize, C::SMEM);
    });
    if (attr_err[dev] != hipSuccess) return attr_err[dev];
    const int64_t nblk = ((a.N + C::BN - 1) / C::BN) * ((a.M + C::BM - 1) / C::BM);
    hipLaunchKernelGGL((k_gemm_tiled<C, PK>), dim3((unsigned)nblk, (unsigned)a.ksplit), dim3(C::THREADS), C::SMEM, s,
                       a);
    return hipGetLastError();
}

template <class C>
static int64_t ctas_of(int64_t M, int64_t N) {
    return ((N + C::BN - 1) / C::BN) * ((M + C::BM - 1) / C::BM);
}

// Above 256 rows: the tile shape and K split of the least estimated time.  A
// launch runs in rounds of up to 256 CTAs (one a compute unit); a round costs
// about the same whether it is full or not, per 128-K group (fused calls at K =
// 4096 on the MI355X, rounds of 168-256 CTAs): 256 x 256 1.875 us, 256 x 128
// 1.31 us, 256 x 64 1.02 us, 128 x 64 0.78 us.  Where a shape other than 256 x
// 256 leaves the chip partly idle, K is split so that about 256 CTAs run, and
// the split pays its fp32 partials at about 5 TB/s (written, then read with the
// output written by the reduce launch) and that launch, about 2 us.  The
// estimates matched the measured calls within about 10% (768 to 3072 rows at N
// = 4096 to 28672, and 1024 x 14336 x 4096) and picked the fastest shape at
// each: e.g. 1024 x 4096 x 14336 in one round of 256 x 256 tiles (224 CTAs)
// 63 us, where two rounds of 256 x 128 took 84 us.
struct TileCost {
    TileShape shape;
    double us_per_group;
    bool splits;
};
static int64_t ctas_for(TileShape shape, int64_t M, int64_t N) {
    switch (shape) {
        case TILE_C: return ctas_of<CfgC>(M, N);
        case TILE_B: return ctas_of<CfgB>(M, N);
        case TILE_M1: return ctas_of<CfgM1>(M, N);
        case TILE_M2: return ctas_of<CfgM2>(M, N);
    }
    return 0;
}
static TiledPlan tiled_plan_wide(int64_t M, int64_t K, int64_t N) {
    static constexpr TileCost costs[] = {
        {TILE_C, 1.875, false}, {TILE_B, 1.31, true}, {TILE_M2, 1.02, true}, {TILE_M1, 0.78, true}};
    const int64_t G = K / 128;
    TiledPlan best{TILE_C, 1};
    double best_us = 0.0;
    for (const TileCost &c : costs) {
        const int64_t ctas = ctas_for(c.shape, M, N);
        int64_t s = 1;
        if (c.splits && ctas < 256) s = std::max<int64_t>(std::min<int64_t>(256 / ctas, G / 2), 1);
        const int64_t rounds = (ctas * s + 255) / 256;
        double us = (double)rounds * c.us_per_group * (double)G / (double)s;
        if (s > 1) us += (8.0 * (double)s * (double)M * (double)N + 2.0 * (double)M * (double)N) / 5.0e6 + 2.0;
        if (best_us == 0.0 || us < best_us) {
            best_us = us;
            best = TiledPlan{c.shape, (int)s};
        }
    }
    return best;
}

namespace {
std::atomic<int> g_tile_shape{-1}, g_tile_ksplit{0};
std::once_flag g_tile_once;
void tile_override_init() {
    std::call_once(g_tile_once, [] {
        int sh = -1;
        switch (tuning().tiled_cfg) {  // b|c|1|2
            case 'b': sh = TILE_B; break;
            case 'c': sh = TILE_C; break;
            case '1': sh = TILE_M1; break;
            case '2': sh = TILE_M2; break;
        }
        g_tile_shape = sh;
        g_tile_ksplit = std::max(tuning().tiled_ksplit, 0);
    });
}
}  // namespace

void set_tiled_override(int shape, int ksplit) {
    tile_override_init();
    g_tile_shape = shape;
    g_tile_ksplit = ksplit;
}

void get_tiled_override(int *shape, int *ksplit) {
    tile_override_init();
    *shape = g_tile_shape.load();
    *ksplit = g_tile_ksplit.load();
}

TiledPlan tiled_plan(int64_t M, int64_t K, int64_t N) {
    TiledPlan t{TILE_B, 1};
    const int64_t G = K / 128;
    tile_override_init();
    const int force_shape = g_tile_shape.load(), force_ksplit = g_tile_ksplit.load();
    if (M > 256 && force_shape < 0 && force_ksplit == 0) return tiled_plan_wide(M, K, N);
    if (ctas_of<CfgC>(M, N) >= 256) t.shape = TILE_C;
    else if (ctas_of<CfgB>(M, N) >= 256) t.shape = TILE_B;
    else if (M <= 256) {
        // 64-column tiles: 128 rows a tile up to 128 rows, and above 128 rows too
        // where those tiles fill most of one round of the chip by themselves (no
        // split; 255 x 4096 x 8192 24.0 against 26.4 us for 256-row tiles split two
        // ways, 192 x 4096 x 8192 23.7 against 24.4), else 256 rows a tile; except
        // at K >= 12288 above 128 rows, where the 256 x 128 tile split about 8 ways
        // is faster (N = 4096, K = 14336: 35.3-37.9 against 36.0-39.6 us at 192 and
        // 255 rows; at K = 8192 the 256 x 64 tile split 4 ways is: 25.2 against 31.6)
        const int64_t m1 = ctas_of<CfgM1>(M, N);
        if (M > 128 && G >= 96) t.shape = TILE_B;
        else if (M <= 128 || (m1 >= 192 && m1 <= 256)) t.shape = TILE_M1;
        else t.shape = TILE_M2;
    }
    if (force_shape >= 0) t.shape = (TileShape)force_shape;
    int64_t ctas = 0;
    switch (t.shape) {
        case TILE_C: ctas = ctas_of<CfgC>(M, N); break;
        case TILE_B: ctas = ctas_of<CfgB>(M, N); break;
        case TILE_M1: ctas = ctas_of<CfgM1>(M, N); break;
        case TILE_M2: ctas = ctas_of<CfgM2>(M, N); break;
    }
    // split K so that about 256 CTAs run, each with at least two groups
    if (t.shape != TILE_C && ctas > 0 && ctas < 256) t.ksplit = (int)std::max<int64_t>(std::min<int64_t>(256 / ctas, G / 2), 1);
    if (force_ksplit >= 1 && t.shape != TILE_C) t.ksplit = (int)std::min<int64_t>(force_ksplit, G);
    return t;
}

size_t tiled_partial_bytes(const TiledPlan &t, int64_t M, int64_t N) {
    return t.ksplit > 1 ? align_up(sizeof(float) * (size_t)t.ksplit * M * N, 256) : 0;
}

hipError_t launch_gemm_tiled(const TiledArgs &a, const TiledPlan &plan, hipStream_t s) {
    TiledArgs b = a;
    b.ksplit = plan.ksplit;
    hipError_t e = hipErrorInvalidValue;
    switch (plan.shape) {
        case TILE_C: e = a.packed ? launch_cfg<CfgC, true>(b, s) : launch_cfg<CfgC, false>(b, s); break;
        case TILE_B: e = a.packed ? launch_cfg<CfgB, true>(b, s) : launch_cfg<CfgB, false>(b, s); break;
        case TILE_M1: e = a.packed ? launch_cfg<CfgM1, true>(b, s) : launch_cfg<CfgM1, false>(b, s); break;
        case TILE_M2: e = a.packed ? launch_cfg<CfgM2, true>(b, s) : launch_cfg<CfgM2, false>(b, s); break;
    }
    if (e != hipSuccess || plan.ksplit == 1) return e;
    return launch_splitk_reduce(b.part, b.c, b.M, b.N, plan.ksplit, s);
}

}  // namespace r9k
