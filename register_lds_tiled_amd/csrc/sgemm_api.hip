// sgemm_api.hip -- the C ABI declared in include/sgemm.h: argument
// validation, path selection and launch.  Validation happens before any HIP
// call; nothing is launched when it fails.
#include <atomic>
#include <cstdint>
#include <cstdio>

#include "sgemm.h"
#include "tiles.h"

namespace {

thread_local char g_last_error[256] = "";

int hip_fail(hipError_t e) {
    std::snprintf(g_last_error, sizeof(g_last_error), "%s: %s", hipGetErrorName(e),
                  hipGetErrorString(e));
    return SGEMM_EHIP;
}

// Byte range [lo, hi) spanned by a rows x cols row-major matrix of esize-byte
// elements with leading dimension ld (rows, cols >= 1).  The extent is
// formed in 128 bits; ok is false when the range would pass the end of the
// address space (no such matrix can exist).
struct Range {
    uintptr_t lo, hi;
    bool ok;
};
Range span(const void* p, long long rows, long long cols, long long ld, long long esize = 4) {
    const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
    const unsigned __int128 bytes =
        ((unsigned __int128)(rows - 1) * (unsigned __int128)ld + (unsigned __int128)cols) *
        (unsigned __int128)esize;
    const unsigned __int128 hi = (unsigned __int128)lo + bytes;
    if (hi > (unsigned __int128)UINTPTR_MAX) return {lo, UINTPTR_MAX, false};
    return {lo, (uintptr_t)hi, true};
}
bool overlaps(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }

// Compute units and XCDs of the device a stream's launches run on, queried
// once per device (the first 64 device ids) and then read from the cache.
// The XCD count falls back to one XCD per 32 CUs (gfx950's XCD) where the
// runtime does not report it.
constexpr int kMaxDevices = 64;
std::atomic<int> g_cus[kMaxDevices], g_xcds[kMaxDevices];

hipError_t device_shape(hipStream_t stream, int& cus, int& xcds) {
    int dev = 0;
    hipError_t e = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const bool cached = dev >= 0 && dev < kMaxDevices;
    if (cached && g_cus[dev].load(std::memory_order_acquire) > 0) {
        xcds = g_xcds[dev].load(std::memory_order_relaxed);
        cus = g_cus[dev].load(std::memory_order_relaxed);
        return hipSuccess;
    }
    int c = 0, x = 0;
    e = hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    if (hipDeviceGetAttribute(&x, hipDeviceAttributeNumberOfXccs, dev) != hipSuccess || x < 1) {
        (void)hipGetLastError();   // not reported: clear it, use the fallback
        x = c >= 32 ? c / 32 : 1;
    }
    cus = c > 0 ? c : 1;
    xcds = x;
    if (cached) {
        g_xcds[dev].store(xcds, std::memory_order_relaxed);
        g_cus[dev].store(cus, std::memory_order_release);
    }
    return hipSuccess;
}

// The default path's kernel choice (plain product or fused epilogue): A of
// at most 16 rows streams B once, B of at most 16 columns streams A once,
// everything else takes the tiled matrix-core kernels.
hipError_t launch_auto(const sgemm::GemmArgs& a, hipStream_t s) {
    if (sgemm::skinny_m_fits(a)) return sgemm::launch_skinny_m(a, s);
    if (sgemm::skinny_n_fits(a)) return sgemm::launch_skinny_n(a, s);
    return sgemm::launch_mfma(a, s);
}

// ab_size: bytes per element of A and B (C is always fp32).
int validate(int M, int N, int K, const void* A, int lda, const void* B, int ldb,
             const float* C, int ldc, int ab_size = 4) {
    if (M < 0 || N < 0 || K < 0) return SGEMM_EINVAL_DIM;
    const int kmin = K > 1 ? K : 1, nmin = N > 1 ? N : 1;
    if (lda < kmin || ldb < nmin || ldc < nmin) return SGEMM_EINVAL_LD;
    if (M == 0 || N == 0) return SGEMM_OK;
    if (C == nullptr) return SGEMM_EINVAL_PTR;
    if (K > 0 && (A == nullptr || B == nullptr)) return SGEMM_EINVAL_PTR;
    // One workgroup per 64x64 tile at most; the grid's thread count must fit
    // the 32-bit launch limit.
    const long long tiles = ((long long)M + 63) / 64 * (((long long)N + 63) / 64);
    if (tiles * 256 > 0xFFFFFFFFll) return SGEMM_EINVAL_DIM;
    const Range rc = span(C, M, N, ldc);
    if (!rc.ok) return SGEMM_EINVAL_DIM;
    if (K > 0) {
        const Range ra = span(A, M, K, lda, ab_size), rb = span(B, K, N, ldb, ab_size);
        if (!ra.ok || !rb.ok) return SGEMM_EINVAL_DIM;
        if (overlaps(rc, ra) || overlaps(rc, rb)) return SGEMM_EALIAS;
    }
    return SGEMM_OK;
}

}  // namespace

extern "C" {

int sgemm_abi_version(void) { return 4; }

const char* sgemm_status_string(int status) {
    switch (status) {
        case SGEMM_OK: return "SGEMM_OK: success";
        case SGEMM_EINVAL_DIM: return "SGEMM_EINVAL_DIM: negative or too large dimension";
        case SGEMM_EINVAL_LD: return "SGEMM_EINVAL_LD: leading dimension smaller than the row";
        case SGEMM_EINVAL_PTR: return "SGEMM_EINVAL_PTR: NULL pointer for a non-empty matrix";
        case SGEMM_EALIAS: return "SGEMM_EALIAS: C overlaps A, B or bias";
        case SGEMM_EHIP: return "SGEMM_EHIP: HIP runtime error (see sgemm_last_error)";
        case SGEMM_EINVAL_PATH: return "SGEMM_EINVAL_PATH: unknown path selector";
        case SGEMM_EINVAL_ACT: return "SGEMM_EINVAL_ACT: unknown activation selector";
        default: return "unknown sgemm status";
    }
}

const char* sgemm_last_error(void) { return g_last_error; }

int sgemm_f32_path(int M, int N, int K, const float* A, int lda, const float* B, int ldb,
                   float* C, int ldc, void* stream, int path) {
    if (path < SGEMM_PATH_AUTO || path > SGEMM_PATH_VALU_PAGE) return SGEMM_EINVAL_PATH;
    const int v = validate(M, N, K, A, lda, B, ldb, C, ldc);
    if (v != SGEMM_OK) return v;
    if (M == 0 || N == 0) return SGEMM_OK;
    sgemm::GemmArgs a{M, N, K, A, lda, B, ldb, C, ldc};
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = device_shape(s, a.cus, a.xcds);
    if (e != hipSuccess) return hip_fail(e);
    switch (path) {
        case SGEMM_PATH_VALU: e = sgemm::launch_valu(a, s); break;
        case SGEMM_PATH_VALU_PAGE: e = sgemm::launch_valu_page(a, s); break;
        case SGEMM_PATH_MFMA: e = sgemm::launch_mfma(a, s); break;
        case SGEMM_PATH_AUTO:
        default: e = launch_auto(a, s); break;
    }
    return e == hipSuccess ? SGEMM_OK : hip_fail(e);
}

int sgemm_valu_tile_count(void) { return sgemm::valu_tile_count(); }

const char* sgemm_valu_tile_name(int tile) { return sgemm::valu_tile_name(tile); }

int sgemm_f32_valu_tile(int M, int N, int K, const float* A, int lda, const float* B, int ldb,
                        float* C, int ldc, void* stream, int tile) {
    if (tile < 0 || tile >= sgemm::valu_tile_count()) return SGEMM_EINVAL_PATH;
    const int v = validate(M, N, K, A, lda, B, ldb, C, ldc);
    if (v != SGEMM_OK) return v;
    if (M == 0 || N == 0) return SGEMM_OK;
    sgemm::GemmArgs a{M, N, K, A, lda, B, ldb, C, ldc};
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = device_shape(s, a.cus, a.xcds);
    if (e != hipSuccess) return hip_fail(e);
    e = sgemm::launch_valu_tile(a, tile, s);
    return e == hipSuccess ? SGEMM_OK : hip_fail(e);
}

int sgemm_f32(int M, int N, int K, const float* A, int lda, const float* B, int ldb,
              float* C, int ldc, void* stream) {
    return sgemm_f32_path(M, N, K, A, lda, B, ldb, C, ldc, stream, SGEMM_PATH_AUTO);
}

int sgemm_f32_ex(int M, int N, int K, const float* A, int lda, const float* B, int ldb,
                 float* C, int ldc, float alpha, float beta, const float* bias, int act,
                 void* stream) {
    if (act != SGEMM_ACT_NONE && act != SGEMM_ACT_RELU) return SGEMM_EINVAL_ACT;
    const int v = validate(M, N, K, A, lda, B, ldb, C, ldc);
    if (v != SGEMM_OK) return v;
    if (M == 0 || N == 0) return SGEMM_OK;
    if (bias != nullptr) {
        const Range rb = span(bias, 1, N, N);
        if (!rb.ok) return SGEMM_EINVAL_DIM;
        if (overlaps(span(C, M, N, ldc), rb)) return SGEMM_EALIAS;
    }
    sgemm::GemmArgs a{M, N, K, A, lda, B, ldb, C, ldc};
    a.alpha = alpha;
    a.beta = beta;
    a.bias = bias;
    a.act = act;
    // The kernels sgemm_f32 runs, each with the epilogue in its store; the
    // identity epilogue is the plain product, bit for bit.
    a.epi = !(alpha == 1.f && beta == 0.f && bias == nullptr && act == SGEMM_ACT_NONE);
    const hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = device_shape(s, a.cus, a.xcds);
    if (e != hipSuccess) return hip_fail(e);
    e = launch_auto(a, s);
    return e == hipSuccess ? SGEMM_OK : hip_fail(e);
}

static int gemm_lowp(int M, int N, int K, const void* A, int lda, const void* B, int ldb,
                     float* C, int ldc, void* stream, sgemm::Lowp type) {
    const int v = validate(M, N, K, A, lda, B, ldb, C, ldc, 2);
    if (v != SGEMM_OK) return v;
    if (M == 0 || N == 0) return SGEMM_OK;
    sgemm::LowpArgs a{M, N, K, static_cast<const unsigned short*>(A), lda,
                      static_cast<const unsigned short*>(B), ldb, C, ldc};
    const hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = device_shape(s, a.cus, a.xcds);
    if (e != hipSuccess) return hip_fail(e);
    e = sgemm::launch_lowp(a, type, s);
    return e == hipSuccess ? SGEMM_OK : hip_fail(e);
}

int gemm_bf16_f32(int M, int N, int K, const void* A, int lda, const void* B, int ldb,
                  float* C, int ldc, void* stream) {
    return gemm_lowp(M, N, K, A, lda, B, ldb, C, ldc, stream, sgemm::Lowp::bf16);
}

int gemm_f16_f32(int M, int N, int K, const void* A, int lda, const void* B, int ldb,
                 float* C, int ldc, void* stream) {
    return gemm_lowp(M, N, K, A, lda, B, ldb, C, ldc, stream, sgemm::Lowp::f16);
}

int sgemm_micro4x4_f32(int K, const float* A, const float* B, float* C, void* stream) {
    if (K < 0) return SGEMM_EINVAL_DIM;
    if (C == nullptr) return SGEMM_EINVAL_PTR;
    if (K > 0 && (A == nullptr || B == nullptr)) return SGEMM_EINVAL_PTR;
    const Range rc = span(C, 4, 4, 4);
    if (!rc.ok) return SGEMM_EINVAL_DIM;
    if (K > 0) {
        const Range ra = span(A, 4, K, K), rb = span(B, K, 4, 4);
        if (!ra.ok || !rb.ok) return SGEMM_EINVAL_DIM;
        if (overlaps(rc, ra) || overlaps(rc, rb)) return SGEMM_EALIAS;
    }
    const hipError_t e = sgemm::launch_micro4x4(K, A, B, C, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? SGEMM_OK : hip_fail(e);
}

}  // extern "C"
