// Host-side interfaces between the C ABI (api.hip) and the kernel files.
// Every launcher enqueues on `stream` and returns hipGetLastError().
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace r9k {

// Tuning overrides of the launch configuration, read from the environment once
// per process (the first call that needs them) and fixed after that, so that a
// workspace query and the call it sizes always plan the same launch.  0 (or
// an empty string) means "not set"; each planner ignores values it cannot use.
//   R9K_DECODE_WN, R9K_DECODE_WK    decode kernel: column tiles / K slices per CTA
//   R9K_TILED_CFG                   tiled engine tile shape: b, c, 1 or 2
//   R9K_TILED_KSPLIT                tiled engine K split
//   R9K_SKINNY_KC, R9K_SKINNY_KSPLIT skinny kernel K batch and K split
//   R9K_BF16A_GS                    bf16-activation variant: K-groups per wave
//   R9K_MID                         mid-width kernel: 0 never, 1 wherever it fits (else the planner's choice)
//   R9K_MID_CFG=mt,wn,wk,d[,ks]     mid-width kernel launch shape and K split (ignored where it does not fit)
//   R9K_MOE_MTR                     MoE expert GEMMs: row tiles of 16 pairs a pass (1 or 2)
struct Tuning {
    int decode_wn, decode_wk;
    char tiled_cfg;
    int tiled_ksplit;
    int skinny_kc;
    long long skinny_ksplit;
    int bf16a_gs;
    int mid;  // -1: not set
    int mid_cfg[5];
    int moe_mtr;  // MoE row tiles a pass (1 or 2; 0 = by the average pairs an expert gets)
};
const Tuning &tuning();

// ---- quantisation (quant.hip) ----
// scales_transposed: write as [K/128][M] instead of [M][K/128]
hipError_t launch_quant_act(const uint16_t *a, int64_t M, int64_t K, uint8_t *aq, float *as, hipStream_t s,
                            bool scales_transposed = false);
hipError_t launch_transpose_scales(const float *as, int64_t M, int64_t G, float *as_t, hipStream_t s);
// W [N][K] row-major -> the fragment-order layout every GEMM engine can read:
// for 16-row tile t and K-group g, the 2 KiB block at (t * K/128 + g) * 2048
// holds, at h * 1024 + 16 * l, the 16 bytes that MFMA lane l loads as its h-th
// chunk: row 16 t + l % 16, bytes 128 g + 64 h + 16 (l / 16) .. +15.
hipError_t launch_pack_weight(const uint8_t *wq, int64_t N, int64_t K, uint8_t *wp, hipStream_t s);
hipError_t launch_quant_weight(const uint16_t *w, int64_t N, int64_t K, uint8_t *wq, float *ws, hipStream_t s);
hipError_t launch_encode_e4m3(const float *x, int64_t n, uint8_t *codes, hipStream_t s);

// ---- decode engine, 1 <= M <= 64 (gemm_decode.hip) ----
struct DecodeCfg {
    int wn;      // 16-column tiles per CTA (0: the shape does not fit this engine)
    int wk;      // K slices per column tile (waves per CTA = wn * wk)
    int gs;      // K-groups per wave: (K / 128) / wk
    int passes;  // activation groups per lane quad
    size_t lds;  // dynamic LDS bytes
    int mt;      // row tiles of 16 (1 to 4)
    int ksplit;  // CTAs along K (> 1: fp32 partials in the workspace, then a reduce)
};
// fused: the kernel quantises the activations itself; otherwise it reads codes.
DecodeCfg decode_config(int64_t M, int64_t K, int64_t N, bool packed);
// Workspace the decode engine needs for its partial sums under either layout.
size_t decode_partial_bytes(int64_t M, int64_t K, int64_t N);
struct DecodeArgs {
    const uint16_t *a;  // bf16 activations (fused form), or NULL
    const uint8_t *aq;  // pre-quantised codes (split form)
    const float *as;
    const uint8_t *w;   // weight codes, row-major or fragment-order (packed)
    const float *ws;
    uint16_t *c;
    int64_t M, K, N;
    bool packed;
    float *part;        // fp32 partials [ksplit][M][N] when the config splits K
};
hipError_t launch_gemm_decode(const DecodeArgs &args, const DecodeCfg &cfg, hipStream_t s);

// ---- skinny weight-streaming engine (gemm_skinny.hip) ----
// One CTA covers 128 output columns (one weight block row), mt16 * 16 rows of
// A (a chunk of at most 256 rows) and kc * nb K-groups; `ksplit` CTAs share a
// tile, write fp32 partials, and a second kernel sums them in split order.
struct SkinnyCfg {
    int mt16;    // row tiles of 16 per CTA: 1, 2, 4, 8 or 16
    int kc;      // K-groups (of 128) per batch: the weight bytes one CTA holds in flight
    int ksplit;  // CTAs sharing an output tile along K
    int nb;      // batches per CTA; kc * ksplit * nb = K/128
    int mchunks; // ceil(M / (16 * mt16))
};
SkinnyCfg skinny_config(int64_t M, int64_t K, int64_t N);
// Workspace the skinny engine needs for this config: the split-K partials.
size_t skinny_partial_bytes(const SkinnyCfg &c, int64_t M, int64_t N);

struct SkinnyArgs {
    const uint16_t *a;  // bf16 activations when quantising in the A-load, else NULL
    const uint8_t *aq;  // fp8 activation codes when pre-quantised
    const float *as;    // their scales [M][K/128]
    const uint8_t *w;   // weight codes, row-major or fragment-order (packed)
    const float *ws;
    uint16_t *c;
    float *part;        // split-K partials [ksplit][M][N]
    int64_t M, K, N;
    bool packed;
};
hipError_t launch_gemm_skinny(const SkinnyArgs &args, const SkinnyCfg &cfg, hipStream_t s);

// ---- mid widths, one launch over all of K (gemm_mid.hip) ----
// Activations come quantised: codes [M][K] and scales transposed, as_t [K/128][M].
struct MidArgs {
    const uint8_t *aq;
    const float *as_t;
    const uint8_t *w;   // weight codes, row-major or fragment-order (packed)
    const float *ws;
    uint16_t *c;
    int64_t M, K, N;
    bool packed;
    float *part;  // K split: fp32 partials [ksplit][M][N]
};
struct MidCfg {
    int mt;      // row tiles of 16 per CTA (0: the shape does not fit)
    int wn;      // column tiles of 16 per CTA
    int wk;      // K slices per column tile (waves per CTA = wn * wk)
    int depth;   // steps of loads in flight per wave
    int ksplit;  // CTAs along K (> 1: fp32 partials, then the ordered reduce launch)
};
constexpr int MID_MAX_KSPLIT = 8;
MidCfg mid_config(int64_t M, int64_t K, int64_t N);
size_t mid_partial_bytes(int64_t M, int64_t K, int64_t N);
hipError_t launch_gemm_mid(const MidArgs &args, const MidCfg &cfg, hipStream_t s);

// ---- LDS-tiled MFMA engine (gemm_tiled.hip) ----
// Activations come pre-quantised, with their scales transposed: as_t [K/128][M].
struct TiledArgs {
    const uint8_t *aq;
    const float *as_t;
    const uint8_t *w;   // weight codes, row-major or fragment-order (packed)
    const float *ws;
    uint16_t *c;
    int64_t M, K, N;
    bool packed;
    float *part;        // ksplit > 1: fp32 partial sums [ksplit][M][N], summed by a second kernel
    int ksplit;
};
// The tile shape and K split for a shape: CTAs of 256 x 256 when there are
// enough of them, else 256 columns x 128 rows, else (skinny widths) 64
// columns x all rows, with the K range split so that about one CTA per
// compute unit runs (fp32 partials in the workspace).
enum TileShape { TILE_C, TILE_B, TILE_M1, TILE_M2 };
struct TiledPlan {
    TileShape shape;
    int ksplit;
};
TiledPlan tiled_plan(int64_t M, int64_t K, int64_t N);
// The forced tiled plan (r9k_set_tiled_plan; R9K_TILED_CFG and R9K_TILED_KSPLIT
// give the initial values): shape -1 = the planner's, else a TileShape; ksplit
// 0 = the planner's.
void set_tiled_override(int shape, int ksplit);
void get_tiled_override(int *shape, int *ksplit);
size_t tiled_partial_bytes(const TiledPlan &t, int64_t M, int64_t N);
hipError_t launch_gemm_tiled(const TiledArgs &args, const TiledPlan &plan, hipStream_t s);
hipError_t launch_splitk_reduce(const float *part, uint16_t *c, int64_t M, int64_t N, int ksplit, hipStream_t s);

// ---- bf16-activation variant at decode widths (gemm_bf16a.hip) ----
struct Bf16aArgs {
    const uint16_t *a;  // [M][K] bf16
    const uint8_t *w;   // [N][K] codes, or their fragment-order copy
    const float *ws;    // [N/128][K/128]
    uint16_t *c;        // [M][N] bf16
    int64_t M, K, N;
    bool packed;
};
struct Bf16aCfg {
    int wn;  // 16-column tiles per CTA (0: the shape does not fit)
    int wk;  // K slices per tile (waves per CTA = wn * wk)
    int gs;  // K-groups per wave
};
Bf16aCfg bf16a_config(int64_t M, int64_t K, int64_t N);
hipError_t launch_gemm_bf16a(const Bf16aArgs &args, const Bf16aCfg &cfg, hipStream_t s);

// ---- MoE decode (moe.hip) ----
struct MoeArgs {
    const uint16_t *x;
    const int32_t *ids;
    const float *tw;
    const uint8_t *w13;
    const float *w13s;
    const uint8_t *w2;
    const float *w2s;
    uint16_t *out;
    uint16_t *gu;   // [P][2I] bf16 (three-launch path)
    uint16_t *h;    // [P][I] bf16
    uint8_t *hq;    // [P][I] fp8 (three-launch path)
    float *hs;      // [P][I/128] (three-launch path)
    float *y;       // [P][H] fp32
    int64_t T, H, E, I, topk;
    bool packed;    // w13 and w2 in fragment order
    const uint16_t *shared;  // NULL, or the shared expert's output [T][H] bf16, added in the combine
    const float *shared_w;   // NULL (weight 1), or the shared term's weight per token [T]
};
struct MoeLayout {
    size_t gu, h, hq, hs, y, total;
};
MoeLayout moe_layout(int64_t T, int64_t H, int64_t E, int64_t I, int64_t topk);
hipError_t launch_moe_decode(const MoeArgs &args, bool fused, hipStream_t s);
hipError_t launch_moe_route(const float *logits, int64_t T, int64_t E, int topk, int32_t *ids, float *w,
                            hipStream_t s);

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

}  // namespace r9k
