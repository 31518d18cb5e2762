// The C ABI of libr9k.so: argument checks, the M-based dispatcher and the
// launches.  Declarations, argument meanings and error behaviour: r9k.h.
//
// The dispatcher follows the r9700-stack release v0.3.2 notes ("What changed
// for someone running it"): the decode (skinny) kernels take up to 255 rows,
// the tiled fp8 GEMMs everything above; the boundary is a setting, as it is on
// the pages (R9K_HC_FP8_DECODE_MAXM there, R9K_FP8_SKINNY_MAXM here).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdlib>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "r9k.h"
#include "r9k_internal.h"

using namespace r9k;

namespace {

std::atomic<int> g_skinny_max_m{255};
std::atomic<int> g_engine{R9K_ENGINE_AUTO};
std::atomic<int> g_qa_inload_max_m{64};
std::once_flag g_env_once;

void read_env() {
    std::call_once(g_env_once, [] {
        if (const char *e = getenv("R9K_FP8_SKINNY_MAXM")) {
            int v = atoi(e);
            if (v >= 0) g_skinny_max_m = v;
        }
        if (const char *e = getenv("R9K_FP8_ENGINE")) {
            if (!strcmp(e, "skinny")) g_engine = R9K_ENGINE_SKINNY;
            else if (!strcmp(e, "tiled")) g_engine = R9K_ENGINE_TILED;
            else g_engine = R9K_ENGINE_AUTO;
        }
        if (const char *e = getenv("R9K_QA_INLOAD_MAXM")) {
            int v = atoi(e);
            if (v >= 0) g_qa_inload_max_m = v;
        }
    });
}

}  // namespace

namespace r9k {
const Tuning &tuning() {
    static Tuning t;
    static std::once_flag once;
    std::call_once(once, [] {
        auto num = [](const char *name) -> long long {
            const char *e = getenv(name);
            return e ? atoll(e) : 0;
        };
        t.decode_wn = (int)num("R9K_DECODE_WN");
        t.decode_wk = (int)num("R9K_DECODE_WK");
        const char *cfg = getenv("R9K_TILED_CFG");
        t.tiled_cfg = cfg ? cfg[0] : 0;
        t.tiled_ksplit = (int)num("R9K_TILED_KSPLIT");
        t.skinny_kc = (int)num("R9K_SKINNY_KC");
        t.skinny_ksplit = num("R9K_SKINNY_KSPLIT");
        t.bf16a_gs = (int)num("R9K_BF16A_GS");
        t.mid = getenv("R9K_MID") ? (int)num("R9K_MID") : -1;
        t.moe_mtr = (int)num("R9K_MOE_MTR");
        if (const char *e = getenv("R9K_MID_CFG"))
            if (sscanf(e, "%d,%d,%d,%d,%d", &t.mid_cfg[0], &t.mid_cfg[1], &t.mid_cfg[2], &t.mid_cfg[3],
                       &t.mid_cfg[4]) < 4)
                t.mid_cfg[0] = 0;
    });
    return t;
}
}  // namespace r9k

namespace {

// Device check, cached per device id: 1 = gfx950, 2 = not usable.
constexpr int MAX_DEV = 64;
std::atomic<int> g_dev_ok[MAX_DEV];

int check_device() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
        (void)hipGetLastError();
        return R9K_ERR_DEVICE;
    }
    if (dev < MAX_DEV) {
        const int st = g_dev_ok[dev].load();
        if (st == 1) return R9K_OK;
        if (st == 2) return R9K_ERR_DEVICE;
    }
    hipDeviceProp_t prop;
    int ok = 0;
    if (hipGetDeviceProperties(&prop, dev) == hipSuccess) ok = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    (void)hipGetLastError();
    if (dev < MAX_DEV) g_dev_ok[dev] = ok ? 1 : 2;
    return ok ? R9K_OK : R9K_ERR_DEVICE;
}

inline bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

constexpr int64_t MAX_DIM = int64_t(1) << 24;

// The mid-width kernel's CTAs that one wave of the MI355X's 256 compute units holds
constexpr int64_t MID_ONE_WAVE_CTAS = 256;

int check_gemm_shape(int64_t M, int64_t K, int64_t N) {
    if (M < 0 || K <= 0 || N <= 0 || K % 128 || N % 128) return R9K_ERR_SHAPE;
    if (M > MAX_DIM || K > MAX_DIM || N > MAX_DIM) return R9K_ERR_SHAPE;
    return R9K_OK;
}

int engine_for(int64_t M) {
    read_env();
    const int e = g_engine.load();
    if (e == R9K_ENGINE_SPLITK) return M <= g_skinny_max_m.load() ? R9K_ENGINE_SPLITK : R9K_ENGINE_TILED;
    if (e != R9K_ENGINE_AUTO) return e;
    return M <= g_skinny_max_m.load() ? R9K_ENGINE_SKINNY : R9K_ENGINE_TILED;
}

// GEMM workspace: [split-K partials][A codes][A scales]
struct GemmWs {
    size_t part, aq, as, total;
};
GemmWs gemm_ws(int64_t M, int64_t K, int64_t N) {
    GemmWs w;
    if (M == 0) return GemmWs{0, 0, 0, 0};  // nothing is launched, nothing is needed
    const SkinnyCfg c = skinny_config(M, K, N);
    w.part = 0;
    w.aq = w.part + std::max({skinny_partial_bytes(c, M, N), tiled_partial_bytes(tiled_plan(M, K, N), M, N),
                              decode_partial_bytes(M, K, N), mid_partial_bytes(M, K, N)});
    w.as = w.aq + align_up((size_t)(M * K), 256);
    w.total = w.as + align_up((size_t)(M * (K / 128)) * sizeof(float), 256);
    return w;
}

int launch_result(hipError_t e) { return e == hipSuccess ? R9K_OK : R9K_ERR_LAUNCH; }

// Which kernel a GEMM call runs, with its configuration: the dispatcher's
// whole decision, shared by the launch path and r9k_gemm_fp8_block_plan.
struct GemmRoute {
    int kernel;  // R9K_KERNEL_*
    DecodeCfg dc;
    TiledPlan tp;
    MidCfg mc;
};
// From 17 rows both the whole-K decode kernel and the mid-width kernel take a
// shape, and what each compute unit must do decides between them.  The busiest
// unit of the decode launch streams W weight bytes and re-quantises Q activation
// values (every CTA quantises all of A); that of the mid-width launch reads B
// bytes of codes, quantised once by a launch of its own.  Fitted over 112 shapes
// (17 to 64 rows, K = 512 to 4096, N = 1024 to 28672, each kernel forced, fused
// calls on fragment-order weights in graphs, one GPU): decode 2.6 us + W /
// (36.2 KiB/us) + Q / (13.9 K values/us), mid-width 4.7 us + B / (38.6 KiB/us),
// within about 0.4-0.7 us.  Taking the lower estimate loses 9.7 us summed over
// those shapes against the faster kernel of each, where taking the decode kernel
// always lost 91.6 us (32 x 4096 x 2048: 7.4 against 12.4 us; 32 x 4096 x 28672:
// 25.4 against 35.1 us; the decode kernel keeps N = 14336 and short K).
bool mid_beats_decode(const DecodeCfg &d, int64_t M, int64_t K, int64_t N) {
    const MidCfg m = mid_config(M, K, N);
    if (!m.mt || m.ksplit != 1) return false;
    const int64_t dctas = N / 16 / d.wn, mctas = (M + 16 * m.mt - 1) / (16 * m.mt) * (N / (16 * m.wn));
    const double dc = double((dctas + 255) / 256), mc = double((mctas + 255) / 256);
    const double W = dc * 16 * d.wn * K, Q = dc * M * K, B = mc * (16 * m.mt + 16 * m.wn) * K;
    const double t_decode = 2.6 + W / (36.2 * 1024) + Q / (13.9 * 1024);
    const double t_mid = 4.7 + B / (38.6 * 1024);
    return t_mid < t_decode;
}

// The skinny engine (M <= the boundary) is three kernels: the decode kernel
// (all of K per CTA, the activation quant in its A-load) where it runs without
// a K split; else, from 17 rows on, the mid-width kernel (all of K per CTA on
// activations quantised once per call); else the decode kernel with a K split,
// or the split-K skinny kernel (very wide N).  Above the boundary: the tiled
// engine.
GemmRoute route_gemm(int64_t M, int64_t K, int64_t N, bool packed) {
    GemmRoute r{R9K_KERNEL_SKINNY, DecodeCfg{0, 0, 0, 0, 0, 0, 0}, TiledPlan{TILE_C, 1}, MidCfg{0, 0, 0, 0, 1}};
    const int engine = engine_for(M);
    if (engine == R9K_ENGINE_TILED) {
        r.kernel = R9K_KERNEL_TILED;
        r.tp = tiled_plan(M, K, N);
        return r;
    }
    if (engine == R9K_ENGINE_SPLITK) return r;  // the split-K skinny kernel, forced
    r.dc = decode_config(M, K, N, packed);
    const int mid = tuning().mid;
    if (r.dc.wn && r.dc.ksplit == 1 && mid != 1 && !(M >= 17 && mid != 0 && mid_beats_decode(r.dc, M, K, N))) {
        r.kernel = R9K_KERNEL_DECODE;
        return r;
    }
    // Above 64 rows the tiled engine (256-row tiles, a K split where they do not
    // fill the chip) is faster than the mid-width kernel at long K (65 to 128 rows
    // at K = 14336, N = 4096: 26.7-29.2 against 31.3-32.7 us) and wherever the mid
    // kernel's largest blocks (64 x 64) would need more than one CTA a compute unit
    // (at K = 4096: 65 to 255 rows at N = 14336, 23.8-32.7 against 26.9-50.4 us; 129
    // to 255 rows at N = 6144 to 12288, 6-21% faster); with at most one such CTA a
    // unit the mid kernel is faster (N = 4096 up to 255 rows, N = 6144 and 8192 up
    // to 128 rows: 3-14%).
    // (at long K only for weights past 2^24 bytes: narrower ones need the tiled
    // engine to split K 8 to 32 ways, and the mid-width kernel was faster, 65 to 255
    // rows at K = 8192, N = 1024 and 2048 by 8-27%, at K = 14336, N = 1024 by up to
    // 11%; at K = 8192, N = 3072 and K = 14336, N = 2048 the tiled engine by 6-34%)
    const bool tiled_faster =
        M > 64 && ((K >= 8192 && N * K > (int64_t(1) << 24)) || ((M + 63) / 64) * (N / 64) > MID_ONE_WAVE_CTAS);
    if (mid != 0 && ((M >= 17 && !tiled_faster) || mid == 1)) {
        r.mc = mid_config(M, K, N);
        if (r.mc.mt) {
            r.kernel = R9K_KERNEL_MID;
            return r;
        }
    }
    if (r.dc.wn) {
        r.kernel = R9K_KERNEL_DECODE;
    } else if (tiled_faster && g_engine.load() == R9K_ENGINE_AUTO) {
        r.kernel = R9K_KERNEL_TILED;
        r.tp = tiled_plan(M, K, N);
    } else if (mid != 0 && M >= 8) {
        // from 8 rows, where the decode kernel fits neither way (large K and N: its
        // LDS cannot hold M x K codes), the mid-width kernel with its K split streams
        // faster than the split-K skinny kernel: 8 x 16384 x 32768 89.3 against 97.4 us,
        // 12 and 16 x 8192 x 32768 50.0 / 51.0 against 54.4 / 57.5, 16 x 16384 x 16384
        // 49.4 against 53.6; below 8 rows the skinny kernel streams at the chip's
        // plain-read rate (4 x 16384 x 65536: 6.36 TB/s)
        const MidCfg mc = mid_config(M, K, N);
        if (mc.mt) {
            r.kernel = R9K_KERNEL_MID;
            r.mc = mc;
        }
    }
    return r;
}

int run_gemm(const uint16_t *a, const uint8_t *aq, const float *as, int64_t M, int64_t K, const uint8_t *w,
             const float *ws, int64_t N, uint16_t *c, void *workspace, size_t ws_bytes, hipStream_t s,
             bool packed) {
    if (M == 0) return R9K_OK;
    const GemmWs L = gemm_ws(M, K, N);
    if (ws_bytes < L.total) return R9K_ERR_WORKSPACE;
    int rc = check_device();
    if (rc) return rc;
    uint8_t *base = (uint8_t *)workspace;
    const GemmRoute route = route_gemm(M, K, N, packed);
    if (route.kernel == R9K_KERNEL_DECODE) {
        DecodeArgs d{a, aq, as, w, ws, c, M, K, N, packed, (float *)(base + L.part)};
        return launch_result(launch_gemm_decode(d, route.dc, s));
    }
    if (route.kernel == R9K_KERNEL_TILED || route.kernel == R9K_KERNEL_MID) {
        // the tiled and mid-width kernels read codes and transposed scales
        // [K/128][M]: quantise A once per call into the workspace, or transpose
        // the caller's scales there
        float *as_t = (float *)(base + L.as);
        if (a) {
            uint8_t *aq_w = base + L.aq;
            rc = launch_result(launch_quant_act(a, M, K, aq_w, as_t, s, true));
            aq = aq_w;
        } else {
            rc = launch_result(launch_transpose_scales(as, M, K / 128, as_t, s));
        }
        if (rc) return rc;
        if (route.kernel == R9K_KERNEL_MID) {
            MidArgs m{aq, as_t, w, ws, c, M, K, N, packed, (float *)(base + L.part)};
            return launch_result(launch_gemm_mid(m, route.mc, s));
        }
        TiledArgs t{aq, as_t, w, ws, c, M, K, N, packed, (float *)(base + L.part), 1};
        return launch_result(launch_gemm_tiled(t, route.tp, s));
    }
    if (a && M > g_qa_inload_max_m.load()) {
        // quantise A once per call into the workspace, then run on codes
        uint8_t *wq_a = base + L.aq;
        float *ws_a = (float *)(base + L.as);
        rc = launch_result(launch_quant_act(a, M, K, wq_a, ws_a, s));
        if (rc) return rc;
        a = nullptr;
        aq = wq_a;
        as = ws_a;
    }
    const SkinnyCfg cfg = skinny_config(M, K, N);
    SkinnyArgs sa{a, aq, as, w, ws, c, (float *)(base + L.part), M, K, N, packed};
    return launch_result(launch_gemm_skinny(sa, cfg, s));
}

// ---- the allocation-free entry point's scratch -------------------------------
// A file-scope device array that stands in for the workspace of
// r9k_gemm_fp8_block_qa_noalloc.  In host code its name is a host-side
// stand-in, not a device address: the address is taken once per device with
// hipGetSymbolAddress (that device current) and only that pointer is used.
constexpr size_t SCRATCH_BYTES = R9K_NOALLOC_SCRATCH_BYTES;
static_assert(SCRATCH_BYTES % 256 == 0, "scratch size");
__device__ __align__(256) uint8_t scratch[SCRATCH_BYTES];
std::once_flag g_scratch_once[MAX_DEV];
void *g_scratch_ptr[MAX_DEV];
hipError_t g_scratch_err[MAX_DEV];

int scratch_for_current_device(void **ptr) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEV) {
        (void)hipGetLastError();
        return R9K_ERR_DEVICE;
    }
    std::call_once(g_scratch_once[dev], [dev] {
        void *p = nullptr;
        g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        g_scratch_ptr[dev] = g_scratch_err[dev] == hipSuccess ? p : nullptr;
    });
    if (g_scratch_err[dev] != hipSuccess || !g_scratch_ptr[dev]) {
        (void)hipGetLastError();
        return R9K_ERR_DEVICE;
    }
    *ptr = g_scratch_ptr[dev];
    return R9K_OK;
}

}  // namespace

extern "C" {

int r9k_abi_version(void) { return R9K_ABI_VERSION; }

const char *r9k_strerror(int code) {
    switch (code) {
        case R9K_OK: return "success";
        case R9K_ERR_NULLPTR: return "a required pointer is NULL";
        case R9K_ERR_SHAPE: return "a size is out of range";
        case R9K_ERR_ALIGN: return "a base pointer is not 16-byte aligned";
        case R9K_ERR_DEVICE: return "no HIP device, or the current device is not gfx950";
        case R9K_ERR_LAUNCH: return "a kernel launch failed";
        case R9K_ERR_WORKSPACE: return "the workspace is smaller than required";
        case R9K_ERR_ARG: return "an enumerated argument has an unknown value";
        default: return "unknown r9k error code";
    }
}

int r9k_quant_act(const uint16_t *a, int64_t M, int64_t K, uint8_t *aq, float *as, void *stream) {
    if (!a || !aq || !as) return R9K_ERR_NULLPTR;
    if (M < 0 || K <= 0 || K % 128 || M > MAX_DIM || K > MAX_DIM) return R9K_ERR_SHAPE;
    if (!aligned16(a) || !aligned16(aq) || !aligned16(as)) return R9K_ERR_ALIGN;
    if (M == 0) return R9K_OK;
    if (int rc = check_device()) return rc;
    return launch_result(launch_quant_act(a, M, K, aq, as, (hipStream_t)stream));
}

int r9k_quant_weight(const uint16_t *w, int64_t N, int64_t K, uint8_t *wq, float *ws, void *stream) {
    if (!w || !wq || !ws) return R9K_ERR_NULLPTR;
    if (N <= 0 || K <= 0 || N % 128 || K % 128 || N > MAX_DIM || K > MAX_DIM) return R9K_ERR_SHAPE;
    if (!aligned16(w) || !aligned16(wq) || !aligned16(ws)) return R9K_ERR_ALIGN;
    if (int rc = check_device()) return rc;
    return launch_result(launch_quant_weight(w, N, K, wq, ws, (hipStream_t)stream));
}

int r9k_encode_e4m3(const float *x, int64_t n, uint8_t *codes, void *stream) {
    if (!x || !codes) return R9K_ERR_NULLPTR;
    if (n < 0 || n > (int64_t(1) << 40)) return R9K_ERR_SHAPE;
    if (!aligned16(x) || !aligned16(codes)) return R9K_ERR_ALIGN;
    if (n == 0) return R9K_OK;
    if (int rc = check_device()) return rc;
    return launch_result(launch_encode_e4m3(x, n, codes, (hipStream_t)stream));
}

int r9k_gemm_fp8_block_workspace(int64_t M, int64_t K, int64_t N, size_t *bytes) {
    if (!bytes) return R9K_ERR_NULLPTR;
    if (int rc = check_gemm_shape(M, K, N)) return rc;
    *bytes = gemm_ws(M, K, N).total;
    return R9K_OK;
}

int r9k_gemm_fp8_block(const uint8_t *aq, const float *as, int64_t M, int64_t K, const uint8_t *w,
                       const float *ws, int64_t N, uint16_t *c, void *workspace, size_t ws_bytes, void *stream) {
    if (!aq || !as || !w || !ws || !c || !workspace) return R9K_ERR_NULLPTR;
    if (int rc = check_gemm_shape(M, K, N)) return rc;
    if (!aligned16(aq) || !aligned16(as) || !aligned16(w) || !aligned16(ws) || !aligned16(c) || !aligned16(workspace))
        return R9K_ERR_ALIGN;
    return run_gemm(nullptr, aq, as, M, K, w, ws, N, c, workspace, ws_bytes, (hipStream_t)stream, false);
}

int r9k_gemm_fp8_block_packed(const uint8_t *aq, const float *as, int64_t M, int64_t K, const uint8_t *wp,
                              const float *ws, int64_t N, uint16_t *c, void *workspace, size_t ws_bytes,
                              void *stream) {
    if (!aq || !as || !wp || !ws || !c || !workspace) return R9K_ERR_NULLPTR;
    if (int rc = check_gemm_shape(M, K, N)) return rc;
    if (!aligned16(aq) || !aligned16(as) || !aligned16(wp) || !aligned16(ws) || !aligned16(c) ||
        !aligned16(workspace))
        return R9K_ERR_ALIGN;
    return run_gemm(nullptr, aq, as, M, K, wp, ws, N, c, workspace, ws_bytes, (hipStream_t)stream, true);
}

int r9k_gemm_fp8_block_qa(const uint16_t *a, int64_t M, int64_t K, const uint8_t *w, const float *ws, int64_t N,
                          uint16_t *c, void *workspace, size_t ws_bytes, void *stream) {
    if (!a || !w || !ws || !c || !workspace) return R9K_ERR_NULLPTR;
    if (int rc = check_gemm_shape(M, K, N)) return rc;
    if (!aligned16(a) || !aligned16(w) || !aligned16(ws) || !aligned16(c) || !aligned16(workspace))
        return R9K_ERR_ALIGN;
    return run_gemm(a, nullptr, nullptr, M, K, w, ws, N, c, workspace, ws_bytes, (hipStream_t)stream, false);
}

int r9k_gemm_fp8_block_qa_packed(const uint16_t *a, int64_t M, int64_t K, const uint8_t *wp, const float *ws,
                                 int64_t N, uint16_t *c, void *workspace, size_t ws_bytes, void *stream) {
    if (!a || !wp || !ws || !c || !workspace) return R9K_ERR_NULLPTR;
    if (int rc = check_gemm_shape(M, K, N)) return rc;
    if (!aligned16(a) || !aligned16(wp) || !aligned16(ws) || !aligned16(c) || !aligned16(workspace))
        return R9K_ERR_ALIGN;
    return run_gemm(a, nullptr, nullptr, M, K, wp, ws, N, c, workspace, ws_bytes, (hipStream_t)stream, true);
}

int r9k_gemm_fp8_block_qa_noalloc(const uint16_t *a, int64_t M, int64_t K, const uint8_t *w, const float *ws,
                                  int64_t N, uint16_t *c, int packed, void *stream) {
    if (!a || !w || !ws || !c) return R9K_ERR_NULLPTR;
    if (int rc = check_gemm_shape(M, K, N)) return rc;
    if (packed != 0 && packed != 1) return R9K_ERR_ARG;
    if (!aligned16(a) || !aligned16(w) || !aligned16(ws) || !aligned16(c)) return R9K_ERR_ALIGN;
    if (M == 0) return R9K_OK;
    const size_t need = gemm_ws(M, K, N).total;
    if (need > SCRATCH_BYTES) return R9K_ERR_WORKSPACE;  // beyond the fixed scratch: use r9k_gemm_fp8_block_qa
    if (int rc = check_device()) return rc;
    void *ptr = nullptr;
    if (int rc = scratch_for_current_device(&ptr)) return rc;
    return run_gemm(a, nullptr, nullptr, M, K, w, ws, N, c, ptr, SCRATCH_BYTES, (hipStream_t)stream, packed == 1);
}

static int run_bf16a(const uint16_t *a, int64_t M, int64_t K, const uint8_t *w, const float *ws, int64_t N,
                     uint16_t *c, void *stream, bool packed) {
    if (!a || !w || !ws || !c) return R9K_ERR_NULLPTR;
    if (int rc = check_gemm_shape(M, K, N)) return rc;
    if (M > 16) return R9K_ERR_SHAPE;
    if (!aligned16(a) || !aligned16(w) || !aligned16(ws) || !aligned16(c)) return R9K_ERR_ALIGN;
    if (M == 0) return R9K_OK;
    const Bf16aCfg cfg = bf16a_config(M, K, N);
    if (!cfg.wn) return R9K_ERR_SHAPE;
    if (int rc = check_device()) return rc;
    return launch_result(launch_gemm_bf16a(Bf16aArgs{a, w, ws, c, M, K, N, packed}, cfg, (hipStream_t)stream));
}

int r9k_gemm_fp8_block_bf16a(const uint16_t *a, int64_t M, int64_t K, const uint8_t *w, const float *ws, int64_t N,
                             uint16_t *c, void *stream) {
    return run_bf16a(a, M, K, w, ws, N, c, stream, false);
}

int r9k_gemm_fp8_block_bf16a_packed(const uint16_t *a, int64_t M, int64_t K, const uint8_t *wp, const float *ws,
                                    int64_t N, uint16_t *c, void *stream) {
    return run_bf16a(a, M, K, wp, ws, N, c, stream, true);
}

int r9k_pack_weight(const uint8_t *wq, int64_t N, int64_t K, uint8_t *wp, void *stream) {
    if (!wq || !wp) return R9K_ERR_NULLPTR;
    if (N <= 0 || K <= 0 || N % 128 || K % 128 || N > MAX_DIM || K > MAX_DIM) return R9K_ERR_SHAPE;
    if (!aligned16(wq) || !aligned16(wp)) return R9K_ERR_ALIGN;
    const uintptr_t lo = (uintptr_t)wq, hi = lo + (uintptr_t)(N * K), plo = (uintptr_t)wp;
    if (plo < hi && lo < plo + (uintptr_t)(N * K)) return R9K_ERR_ARG;  // in place is not supported
    if (int rc = check_device()) return rc;
    return launch_result(launch_pack_weight(wq, N, K, wp, (hipStream_t)stream));
}

int r9k_gemm_fp8_block_plan(int64_t M, int64_t K, int64_t N, int packed, int *kernel, int *ksplit) {
    if (!kernel || !ksplit) return R9K_ERR_NULLPTR;
    if (int rc = check_gemm_shape(M, K, N)) return rc;
    if (packed != 0 && packed != 1) return R9K_ERR_ARG;
    if (M == 0) {
        *kernel = R9K_KERNEL_NONE;
        *ksplit = 0;
        return R9K_OK;
    }
    const GemmRoute r = route_gemm(M, K, N, packed != 0);
    *kernel = r.kernel;
    *ksplit = r.kernel == R9K_KERNEL_DECODE ? r.dc.ksplit
              : r.kernel == R9K_KERNEL_TILED ? r.tp.ksplit
              : r.kernel == R9K_KERNEL_MID   ? r.mc.ksplit
                                              : skinny_config(M, K, N).ksplit;
    return R9K_OK;
}

int r9k_set_dispatch(int skinny_max_m, int engine) {
    read_env();
    if (skinny_max_m < 0) return R9K_ERR_SHAPE;
    if (engine != R9K_ENGINE_AUTO && engine != R9K_ENGINE_SKINNY && engine != R9K_ENGINE_TILED &&
        engine != R9K_ENGINE_SPLITK)
        return R9K_ERR_ARG;
    g_skinny_max_m = skinny_max_m;
    g_engine = engine;
    return R9K_OK;
}

int r9k_set_tiled_plan(int shape, int ksplit) {
    static constexpr int to_internal[] = {-1, TILE_C, TILE_B, TILE_M1, TILE_M2};
    if (shape < R9K_TILE_AUTO || shape > R9K_TILE_256X64 || ksplit < 0) return R9K_ERR_ARG;
    set_tiled_override(to_internal[shape], ksplit);
    return R9K_OK;
}

int r9k_get_tiled_plan(int *shape, int *ksplit) {
    if (!shape || !ksplit) return R9K_ERR_NULLPTR;
    int sh = -1, ks = 0;
    get_tiled_override(&sh, &ks);
    switch (sh) {
        case TILE_C: *shape = R9K_TILE_256X256; break;
        case TILE_B: *shape = R9K_TILE_256X128; break;
        case TILE_M1: *shape = R9K_TILE_128X64; break;
        case TILE_M2: *shape = R9K_TILE_256X64; break;
        default: *shape = R9K_TILE_AUTO; break;
    }
    *ksplit = ks;
    return R9K_OK;
}

int r9k_get_dispatch(int *skinny_max_m, int *engine) {
    if (!skinny_max_m || !engine) return R9K_ERR_NULLPTR;
    read_env();
    *skinny_max_m = g_skinny_max_m.load();
    *engine = g_engine.load();
    return R9K_OK;
}

static int check_moe_shape(int64_t T, int64_t H, int64_t E, int64_t I, int64_t topk) {
    if (T < 0 || T > 256 || H <= 0 || I <= 0 || H % 128 || I % 128 || E <= 0 || topk < 1 || topk > E)
        return R9K_ERR_SHAPE;
    if (T * topk > 4096 || H > MAX_DIM || I > MAX_DIM || E > 65536) return R9K_ERR_SHAPE;
    return R9K_OK;
}

int r9k_moe_fp8_decode_workspace(int64_t T, int64_t H, int64_t E, int64_t I, int64_t topk, size_t *bytes) {
    if (!bytes) return R9K_ERR_NULLPTR;
    if (int rc = check_moe_shape(T, H, E, I, topk)) return rc;
    *bytes = moe_layout(T, H, E, I, topk).total;
    return R9K_OK;
}

int r9k_moe_ws_offset(int64_t T, int64_t H, int64_t E, int64_t I, int64_t topk, int which, size_t *offset) {
    if (!offset) return R9K_ERR_NULLPTR;
    if (int rc = check_moe_shape(T, H, E, I, topk)) return rc;
    const MoeLayout L = moe_layout(T, H, E, I, topk);
    switch (which) {
        case 0: *offset = L.gu; return R9K_OK;
        case 1: *offset = L.h; return R9K_OK;
        case 2: *offset = L.y; return R9K_OK;
        case 3: *offset = L.hq; return R9K_OK;
        case 4: *offset = L.hs; return R9K_OK;
    }
    return R9K_ERR_ARG;
}

static int run_moe(const uint16_t *x, int64_t T, int64_t H, const int32_t *topk_ids, const float *topk_w,
                   int64_t topk, const uint8_t *w13, const float *w13_s, const uint8_t *w2, const float *w2_s,
                   int64_t E, int64_t I, uint16_t *out, void *workspace, size_t ws_bytes, int fused, void *stream,
                   bool packed, const uint16_t *shared, const float *shared_w) {
    if (!x || !topk_ids || !topk_w || !w13 || !w13_s || !w2 || !w2_s || !out || !workspace) return R9K_ERR_NULLPTR;
    if (int rc = check_moe_shape(T, H, E, I, topk)) return rc;
    if (fused != 0 && fused != 1) return R9K_ERR_ARG;
    if (!aligned16(x) || !aligned16(topk_ids) || !aligned16(topk_w) || !aligned16(w13) || !aligned16(w13_s) ||
        !aligned16(w2) || !aligned16(w2_s) || !aligned16(out) || !aligned16(workspace) ||
        (shared && !aligned16(shared)) || (shared_w && !aligned16(shared_w)))
        return R9K_ERR_ALIGN;
    if (shared_w && !shared) return R9K_ERR_NULLPTR;  // a weight for a term that is not there
    if (T == 0) return R9K_OK;
    const MoeLayout L = moe_layout(T, H, E, I, topk);
    if (ws_bytes < L.total) return R9K_ERR_WORKSPACE;
    if (int rc = check_device()) return rc;
    uint8_t *b = (uint8_t *)workspace;
    MoeArgs a{x, topk_ids, topk_w, w13, w13_s, w2, w2_s, out, (uint16_t *)(b + L.gu), (uint16_t *)(b + L.h),
              b + L.hq, (float *)(b + L.hs), (float *)(b + L.y), T, H, E, I, topk, packed, shared, shared_w};
    return launch_result(launch_moe_decode(a, fused == 1, (hipStream_t)stream));
}

int r9k_moe_fp8_decode(const uint16_t *x, int64_t T, int64_t H, const int32_t *topk_ids, const float *topk_w,
                       int64_t topk, const uint8_t *w13, const float *w13_s, const uint8_t *w2, const float *w2_s,
                       int64_t E, int64_t I, uint16_t *out, void *workspace, size_t ws_bytes, int fused,
                       void *stream) {
    return run_moe(x, T, H, topk_ids, topk_w, topk, w13, w13_s, w2, w2_s, E, I, out, workspace, ws_bytes, fused,
                   stream, false, nullptr, nullptr);
}

int r9k_moe_fp8_decode_packed(const uint16_t *x, int64_t T, int64_t H, const int32_t *topk_ids,
                              const float *topk_w, int64_t topk, const uint8_t *w13p, const float *w13_s,
                              const uint8_t *w2p, const float *w2_s, int64_t E, int64_t I, uint16_t *out,
                              void *workspace, size_t ws_bytes, int fused, void *stream) {
    return run_moe(x, T, H, topk_ids, topk_w, topk, w13p, w13_s, w2p, w2_s, E, I, out, workspace, ws_bytes, fused,
                   stream, true, nullptr, nullptr);
}

int r9k_moe_fp8_decode_ex(const uint16_t *x, int64_t T, int64_t H, const int32_t *topk_ids, const float *topk_w,
                          int64_t topk, const uint8_t *w13, const float *w13_s, const uint8_t *w2,
                          const float *w2_s, int64_t E, int64_t I, uint16_t *out, void *workspace,
                          size_t ws_bytes, const r9k_moe_opts *opts, void *stream) {
    if (!opts) return R9K_ERR_NULLPTR;
    if (opts->packed != 0 && opts->packed != 1) return R9K_ERR_ARG;
    return run_moe(x, T, H, topk_ids, topk_w, topk, w13, w13_s, w2, w2_s, E, I, out, workspace, ws_bytes,
                   opts->fused, stream, opts->packed == 1, opts->shared, opts->shared_w);
}

int r9k_moe_route(const float *logits, int64_t T, int64_t E, int64_t topk, int32_t *topk_ids, float *topk_w,
                  void *stream) {
    if (!logits || !topk_ids || !topk_w) return R9K_ERR_NULLPTR;
    if (T < 0 || T > MAX_DIM || E < 1 || E > 65536 || topk < 1 || topk > E || topk > 64) return R9K_ERR_SHAPE;
    if (!aligned16(logits) || !aligned16(topk_ids) || !aligned16(topk_w)) return R9K_ERR_ALIGN;
    if (T == 0) return R9K_OK;
    if (int rc = check_device()) return rc;
    return launch_result(launch_moe_route(logits, T, E, (int)topk, topk_ids, topk_w, (hipStream_t)stream));
}

}  // extern "C"
