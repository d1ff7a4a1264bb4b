// gemm_api.hip -- the C ABI (include/dense_fp32_tiled.h): argument checks,
// variant dispatch and kernel launches for the gfx950 fp32 GEMM kernels.
#include <hip/hip_runtime.h>

#include <mutex>
#include <stdint.h>
#include <string.h>

#include "dense_fp32_tiled.h"
#include "gemm_kernels.hpp"
#include "pad_choice.hpp"

namespace {

using namespace dft;

// ---- tile configurations ------------------------------------------------------
constexpr MfmaShape kMfmaShape{128, 128, 16, 64, 64, 256, 4};
constexpr int kMfmaPadA = mfma_pad_a(kMfmaShape, kGfx950Lds);
constexpr int kMfmaPadB = mfma_pad_b(kMfmaShape, kGfx950Lds);

template <int STAGES, int PADA, int PADB, int VEC>
using MfmaT = MfmaCfg<128, 128, 16, 64, 64, STAGES, PADA, PADB, VEC>;

constexpr ValuShape kValuShape{128, 128, 16, 16, 256, 4};
constexpr int kValuPadA = valu_pad_a(kValuShape, kGfx950Lds);
constexpr int kValuPadB = valu_pad_b(kValuShape, kGfx950Lds);

template <int VEC>
using ValuT = ValuCfg<128, 128, 16, 8, 8, 2, kValuPadA, kValuPadB, VEC>;

struct Args {
    int64_t M, N, K;
    const float* A;
    int64_t lda;
    const float* B;
    int64_t ldb;
    float* C;
    int64_t ldc;
};

using LaunchFn = hipError_t (*)(const Args&, hipStream_t);

// Launches go through hipLaunchKernel so that the returned status is this
// launch's own (hipGetLastError would also report errors left by earlier,
// unrelated runtime calls on the thread).
template <class Kernel>
hipError_t launch_tiles(Kernel kernel, int bm, int bn, int threads, const Args& a, hipStream_t stream) {
    int64_t M = a.M, N = a.N, K = a.K, lda = a.lda, ldb = a.ldb, ldc = a.ldc;
    const float* A = a.A;
    const float* B = a.B;
    float* C = a.C;
    const int64_t tiles_m = (M + bm - 1) / bm;
    int64_t tiles_n = (N + bn - 1) / bn;
    void* args[] = {&M, &N, &K, &A, &lda, &B, &ldb, &C, &ldc, &tiles_n};
    return hipLaunchKernel(reinterpret_cast<const void*>(kernel), dim3((unsigned)(tiles_m * tiles_n)),
                           dim3(threads), args, 0, stream);
}

template <class Cfg>
hipError_t launch_mfma(const Args& a, hipStream_t stream) {
    return launch_tiles(gemm_mfma_kernel<Cfg>, Cfg::BM, Cfg::BN, Cfg::THREADS, a, stream);
}

template <class Cfg>
hipError_t launch_valu(const Args& a, hipStream_t stream) {
    return launch_tiles(gemm_valu_kernel<Cfg>, Cfg::BM, Cfg::BN, Cfg::THREADS, a, stream);
}

template <class Cfg>
gemm_tile_config mfma_config(int variant, int vec) {
    gemm_tile_config c{};
    c.variant = variant;
    c.bm = Cfg::BM; c.bn = Cfg::BN; c.bk = Cfg::BK;
    c.threads = Cfg::THREADS; c.wave_size = kWave;
    c.tm = Cfg::WM; c.tn = Cfg::WN;
    c.stages = Cfg::STAGES;
    c.barriers_per_tile = Cfg::STAGES == 2 ? 1 : 2;
    c.a_rows = Cfg::TileA::rows; c.a_cols = Cfg::TileA::cols; c.a_pad = Cfg::TileA::pad;
    c.a_row_stride = Cfg::TileA::row_stride; c.a_stage_elems = Cfg::TileA::stage_elems;
    c.b_rows = Cfg::TileB::rows; c.b_cols = Cfg::TileB::cols; c.b_pad = Cfg::TileB::pad;
    c.b_row_stride = Cfg::TileB::row_stride; c.b_stage_elems = Cfg::TileB::stage_elems;
    c.lds_bytes = Cfg::LDS_BYTES;
    c.vec_width = vec;
    c.lds_banks_b32 = kGfx950Lds.banks_b32; c.lds_lanes_b32 = kGfx950Lds.lanes_b32;
    c.lds_banks_b128 = kGfx950Lds.banks_b128; c.lds_lanes_b128 = kGfx950Lds.lanes_b128;
    c.a_transposed = 0;
    return c;
}

template <class Cfg>
gemm_tile_config valu_config(int variant, int vec) {
    gemm_tile_config c{};
    c.variant = variant;
    c.bm = Cfg::BM; c.bn = Cfg::BN; c.bk = Cfg::BK;
    c.threads = Cfg::THREADS; c.wave_size = kWave;
    c.tm = Cfg::TM; c.tn = Cfg::TN;
    c.stages = Cfg::STAGES;
    c.barriers_per_tile = Cfg::STAGES == 2 ? 1 : 2;
    c.a_rows = Cfg::TileA::rows; c.a_cols = Cfg::TileA::cols; c.a_pad = Cfg::TileA::pad;
    c.a_row_stride = Cfg::TileA::row_stride; c.a_stage_elems = Cfg::TileA::stage_elems;
    c.b_rows = Cfg::TileB::rows; c.b_cols = Cfg::TileB::cols; c.b_pad = Cfg::TileB::pad;
    c.b_row_stride = Cfg::TileB::row_stride; c.b_stage_elems = Cfg::TileB::stage_elems;
    c.lds_bytes = Cfg::LDS_BYTES;
    c.vec_width = vec;
    c.lds_banks_b32 = kGfx950Lds.banks_b32; c.lds_lanes_b32 = kGfx950Lds.lanes_b32;
    c.lds_banks_b128 = kGfx950Lds.banks_b128; c.lds_lanes_b128 = kGfx950Lds.lanes_b128;
    c.a_transposed = 1;
    return c;
}

struct Variant {
    LaunchFn vec4;    // 16-byte global loads (needs aligned A/B and ld % 4 == 0)
    LaunchFn scalar;  // 4-byte masked loads, any alignment
    gemm_tile_config (*config)(int variant, int vec);
    int lds_bytes;
};

const Variant kVariants[GEMM_VARIANT_COUNT] = {
    /* AUTO   */ {launch_mfma<MfmaT<2, kMfmaPadA, kMfmaPadB, 4>>, launch_mfma<MfmaT<2, kMfmaPadA, kMfmaPadB, 1>>,
                  mfma_config<MfmaT<2, kMfmaPadA, kMfmaPadB, 4>>, MfmaT<2, kMfmaPadA, kMfmaPadB, 4>::LDS_BYTES},
    /* MFMA   */ {launch_mfma<MfmaT<2, kMfmaPadA, kMfmaPadB, 4>>, launch_mfma<MfmaT<2, kMfmaPadA, kMfmaPadB, 1>>,
                  mfma_config<MfmaT<2, kMfmaPadA, kMfmaPadB, 4>>, MfmaT<2, kMfmaPadA, kMfmaPadB, 4>::LDS_BYTES},
    /* VALU   */ {launch_valu<ValuT<4>>, launch_valu<ValuT<1>>, valu_config<ValuT<4>>, ValuT<4>::LDS_BYTES},
    /* STAGES1*/ {launch_mfma<MfmaT<1, kMfmaPadA, kMfmaPadB, 4>>, launch_mfma<MfmaT<1, kMfmaPadA, kMfmaPadB, 1>>,
                  mfma_config<MfmaT<1, kMfmaPadA, kMfmaPadB, 4>>, MfmaT<1, kMfmaPadA, kMfmaPadB, 4>::LDS_BYTES},
    /* NOPAD  */ {launch_mfma<MfmaT<2, 0, 0, 4>>, launch_mfma<MfmaT<2, 0, 0, 1>>, mfma_config<MfmaT<2, 0, 0, 4>>,
                  MfmaT<2, 0, 0, 4>::LDS_BYTES},
    /* SCALAR */ {launch_mfma<MfmaT<2, kMfmaPadA, kMfmaPadB, 1>>, launch_mfma<MfmaT<2, kMfmaPadA, kMfmaPadB, 1>>,
                  mfma_config<MfmaT<2, kMfmaPadA, kMfmaPadB, 1>>, MfmaT<2, kMfmaPadA, kMfmaPadB, 1>::LDS_BYTES},
};

// ---- per-device properties (cached) ---------------------------------------------
struct DeviceInfo {
    int state;  // 0 unknown, 1 gfx950, -1 unsupported
    int max_lds;
};
constexpr int kMaxDevices = 64;
DeviceInfo g_devices[kMaxDevices];
std::mutex g_devices_mu;

int device_check(int* max_lds) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return GEMM_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return GEMM_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_devices_mu);
    DeviceInfo& d = g_devices[dev];
    if (d.state == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return GEMM_ERR_HIP;
        d.state = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : -1;
        d.max_lds = (int)prop.sharedMemPerBlock;
    }
    if (d.state != 1) return GEMM_ERR_UNSUPPORTED;
    *max_lds = d.max_lds;
    return GEMM_OK;
}

bool overlaps(const void* p, int64_t p_bytes, const void* q, int64_t q_bytes) {
    const uintptr_t a0 = (uintptr_t)p, a1 = a0 + (uintptr_t)p_bytes;
    const uintptr_t b0 = (uintptr_t)q, b1 = b0 + (uintptr_t)q_bytes;
    return a0 < b1 && b0 < a1;
}

// Bytes spanned by a rows x cols row-major matrix with leading dimension ld.
int64_t span_bytes(int64_t rows, int64_t cols, int64_t ld) {
    if (rows == 0 || cols == 0) return 0;
    return ((rows - 1) * ld + cols) * 4;
}

int validate(const Args& a) {
    if (a.M < 0 || a.N < 0 || a.K < 0) return GEMM_ERR_INVALID_DIM;
    const int64_t k1 = a.K > 1 ? a.K : 1, n1 = a.N > 1 ? a.N : 1;
    if (a.lda < k1 || a.ldb < n1 || a.ldc < n1) return GEMM_ERR_INVALID_LD;
    // Offsets up to M*ld must fit in int64 bytes with ample margin.
    const int64_t lim = (int64_t)1 << 60;
    if (a.M > lim / a.lda || a.K > lim / a.ldb || a.M > lim / a.ldc) return GEMM_ERR_TOO_LARGE;
    const bool c_used = a.M > 0 && a.N > 0;
    const bool ab_used = c_used && a.K > 0;
    if (c_used && a.C == nullptr) return GEMM_ERR_NULL;
    if (ab_used && (a.A == nullptr || a.B == nullptr)) return GEMM_ERR_NULL;
    if (ab_used) {
        const int64_t c_bytes = span_bytes(a.M, a.N, a.ldc);
        if (overlaps(a.C, c_bytes, a.A, span_bytes(a.M, a.K, a.lda)) ||
            overlaps(a.C, c_bytes, a.B, span_bytes(a.K, a.N, a.ldb)))
            return GEMM_ERR_ALIAS;
    }
    return GEMM_OK;
}

int run(const Args& a, hipStream_t stream, int variant) {
    if (variant < 0 || variant >= GEMM_VARIANT_COUNT) return GEMM_ERR_UNSUPPORTED;
    int st = validate(a);
    if (st != GEMM_OK) return st;
    if (a.M == 0 || a.N == 0) return GEMM_OK;
    int max_lds = 0;
    st = device_check(&max_lds);
    if (st != GEMM_OK) return st;

    if (a.K == 0) {
        const int64_t total = a.M * a.N;
        int64_t blocks = (total + 255) / 256;
        if (blocks > 65536) blocks = 65536;
        int64_t M = a.M, N = a.N, ldc = a.ldc;
        float* C = a.C;
        void* args[] = {&M, &N, &C, &ldc};
        return hipLaunchKernel(reinterpret_cast<const void*>(zero_fill_kernel), dim3((unsigned)blocks), dim3(256),
                               args, 0, stream) == hipSuccess
                   ? GEMM_OK
                   : GEMM_ERR_HIP;
    }

    const Variant& v = kVariants[variant];
    if (v.lds_bytes > max_lds) return GEMM_ERR_CONFIG;
    const gemm_tile_config cfg = v.config(variant, 4);
    const int64_t tiles = ((a.M + cfg.bm - 1) / cfg.bm) * ((a.N + cfg.bn - 1) / cfg.bn);
    if (tiles > (int64_t)0x7fffffff / cfg.threads) return GEMM_ERR_TOO_LARGE;

    const bool aligned = (a.lda % 4 == 0) && (a.ldb % 4 == 0) && (((uintptr_t)a.A & 15) == 0) &&
                         (((uintptr_t)a.B & 15) == 0);
    const LaunchFn fn = aligned ? v.vec4 : v.scalar;
    return fn(a, stream) == hipSuccess ? GEMM_OK : GEMM_ERR_HIP;
}

}  // namespace

// ---- exported C ABI ---------------------------------------------------------------
extern "C" {

int gemm_f32(int64_t M, int64_t N, int64_t K, const float* A, int64_t lda, const float* B, int64_t ldb,
             float* C, int64_t ldc, void* stream) {
    return run(Args{M, N, K, A, lda, B, ldb, C, ldc}, (hipStream_t)stream, GEMM_VARIANT_AUTO);
}

int gemm_f32_ex(int64_t M, int64_t N, int64_t K, const float* A, int64_t lda, const float* B, int64_t ldb,
                float* C, int64_t ldc, void* stream, int variant) {
    return run(Args{M, N, K, A, lda, B, ldb, C, ldc}, (hipStream_t)stream, variant);
}

int gemm_f32_tile_config(int variant, gemm_tile_config* out) {
    if (out == nullptr) return GEMM_ERR_NULL;
    if (variant < 0 || variant >= GEMM_VARIANT_COUNT) return GEMM_ERR_UNSUPPORTED;
    const int vec = variant == GEMM_VARIANT_MFMA_SCALAR ? 1 : 4;
    *out = kVariants[variant].config(variant, vec);
    return GEMM_OK;
}

const char* gemm_f32_status_string(int status) {
    switch (status) {
        case GEMM_OK: return "success";
        case GEMM_ERR_INVALID_DIM: return "invalid dimension: M, N and K must be >= 0";
        case GEMM_ERR_INVALID_LD: return "invalid leading dimension: need lda >= max(1,K), ldb >= max(1,N), ldc >= max(1,N)";
        case GEMM_ERR_NULL: return "NULL pointer for an operand with non-zero extent";
        case GEMM_ERR_ALIAS: return "C overlaps A or B";
        case GEMM_ERR_UNSUPPORTED: return "unsupported: the current device is not gfx950, or the variant is unknown";
        case GEMM_ERR_CONFIG: return "tile configuration exceeds the device's LDS per workgroup";
        case GEMM_ERR_HIP: return "HIP runtime error or launch failure";
        case GEMM_ERR_TOO_LARGE: return "problem too large for the kernel's index range";
        default: return "unknown status";
    }
}

int gemm_lds_layout(int32_t rows, int32_t cols, int32_t pad, int32_t stages, int32_t* row_stride,
                    int32_t* stage_elems, int32_t* total_elems, int32_t* bytes) {
    const LdsLayout l{rows, cols, pad, stages};
    if (!l.valid()) return GEMM_ERR_INVALID_DIM;
    if ((int64_t)rows * (cols + pad) * stages * 4 > 0x7fffffff) return GEMM_ERR_TOO_LARGE;
    if (row_stride) *row_stride = l.row_stride();
    if (stage_elems) *stage_elems = l.stage_elems();
    if (total_elems) *total_elems = l.total_elems();
    if (bytes) *bytes = l.bytes();
    return GEMM_OK;
}

int64_t gemm_lds_offset(int32_t rows, int32_t cols, int32_t pad, int32_t stages, int32_t stage, int32_t row,
                        int32_t col) {
    const LdsLayout l{rows, cols, pad, stages};
    if (!l.valid()) return -1;
    if (stage < 0 || stage >= stages || row < 0 || row >= rows || col < 0 || col >= cols) return -1;
    if ((int64_t)rows * (cols + pad) * stages > 0x7fffffff) return -1;
    return l.offset(stage, row, col);
}

int32_t gemm_lds_bank(int64_t word_offset, int32_t banks) {
    if (banks < 1 || word_offset < 0) return -1;
    return bank_of(word_offset, banks);
}

int32_t gemm_lds_conflict_degree(const int64_t* lane_words, int32_t lanes, int32_t width, int32_t banks,
                                 int32_t group) {
    if (lane_words == nullptr) return -1;
    return conflict_degree([=](int l) { return lane_words[l]; }, lanes, width, banks, group);
}

int32_t gemm_lds_page_pad(int32_t columns, int32_t simultaneous_rows, int32_t banks) {
    if (columns < 1 || simultaneous_rows < 0 || banks < 1) return -1;
    return page_pad(columns, simultaneous_rows, banks);
}

}  // extern "C"
