// Drives the C ABI of libmx (include/mx.h) through its host-side validation, row chunking and
// error mapping, built with AddressSanitizer and UndefinedBehaviorSanitizer against the
// launcher stand-ins of stubs.cpp (no GPU, no device memory: tensor pointers are fake,
// 16-byte aligned addresses that nothing dereferences).  Every expectation follows the error
// rules and buffer layouts that include/mx.h states.  Prints one line per failed check and
// exits non-zero if any failed.
#include <cmath>
#include <cstdio>
#include <cstring>
#include <limits>

#include "mx.h"
#include "stubs.h"

static int g_checks = 0, g_failed = 0;

#define CHECK(cond)                                                                  \
    do {                                                                             \
        ++g_checks;                                                                  \
        if (!(cond)) {                                                               \
            ++g_failed;                                                              \
            std::printf("FAILED line %d: %s\n", __LINE__, #cond);                    \
        }                                                                            \
    } while (0)

// fake device addresses: 2^44 plus an offset, 256-byte aligned, never dereferenced
static uint8_t* fake(uint64_t off) { return reinterpret_cast<uint8_t*>((uint64_t(1) << 44) + off); }
static const uint8_t* ptr(const void* p) { return static_cast<const uint8_t*>(p); }

static void expect_status(mx_status got, mx_status want, int line)
{
    ++g_checks;
    if (got != want) {
        ++g_failed;
        std::printf("FAILED line %d: status %d (%s), expected %d\n", line, (int)got, mx_status_string(got), (int)want);
    }
}
#define EXPECT(call, want)                 \
    do {                                   \
        g_launches.clear();                \
        expect_status((call), (want), __LINE__); \
    } while (0)
#define EXPECT_NO_LAUNCH(call, want)       \
    do {                                   \
        EXPECT(call, want);                \
        CHECK(g_launches.empty());         \
    } while (0)

static void status_strings()
{
    for (int s = -5; s <= 0; ++s) {
        const char* t = mx_status_string((mx_status)s);
        CHECK(t != nullptr && std::strlen(t) > 0 && std::strcmp(t, "unknown status") != 0);
    }
    CHECK(std::strcmp(mx_status_string((mx_status)7), "unknown status") == 0);
}

static void quantize_rules()
{
    uint8_t *x = fake(0), *c = fake(1u << 30), *s = fake(3u << 30);
    const float nan = std::numeric_limits<float>::quiet_NaN(), inf = std::numeric_limits<float>::infinity();
    // invalid descriptions: no launch
    EXPECT_NO_LAUNCH(mx_quantize(x, MX_BF16, -1, 64, 64, 32, MX_SCALE_E8M0, 1.0f, MX_LAYOUT_ROWMAJOR, c, s, nullptr), MX_ERR_INVALID_ARG);
    EXPECT_NO_LAUNCH(mx_quantize(x, MX_BF16, 4, -2, 64, 32, MX_SCALE_E8M0, 1.0f, MX_LAYOUT_ROWMAJOR, c, s, nullptr), MX_ERR_INVALID_ARG);
    EXPECT_NO_LAUNCH(mx_quantize(x, MX_BF16, 4, 33, 64, 4, MX_SCALE_E8M0, 1.0f, MX_LAYOUT_ROWMAJOR, c, s, nullptr), MX_ERR_INVALID_ARG);
    EXPECT_NO_LAUNCH(mx_quantize(x, MX_BF16, 4, 48, 64, 32, MX_SCALE_E8M0, 1.0f, MX_LAYOUT_ROWMAJOR, c, s, nullptr), MX_ERR_INVALID_ARG);
    for (int b : {0, 3, 12, 512, -32})
        EXPECT_NO_LAUNCH(mx_quantize(x, MX_BF16, 4, 1024, 1024, b, MX_SCALE_E8M0, 1.0f, MX_LAYOUT_ROWMAJOR, c, s, nullptr), MX_ERR_INVALID_ARG);
    EXPECT_NO_LAUNCH(mx_quantize(x, MX_BF16, 4, 64, 64, 32, (mx_scale_fmt)5, 1.0f, MX_LAYOUT_ROWMAJOR, c, s, nullptr), MX_ERR_INVALID_ARG);
    EXPECT_NO_LAUNCH(mx_quantize(x, MX_BF16, 4, 64, 64, 32, MX_SCALE_E8M0, 1.0f, (mx_layout)9, c, s, nullptr), MX_ERR_INVALID_ARG);
    for (float g : {0.0f, -1.0f, nan, inf, 1e-40f})
        EXPECT_NO_LAUNCH(mx_quantize(x, MX_BF16, 4, 64, 64, 32, MX_SCALE_E4M3, g, MX_LAYOUT_ROWMAJOR, c, s, nullptr), MX_ERR_INVALID_ARG);
    EXPECT_NO_LAUNCH(mx_quantize(x, (mx_dtype)7, 4, 64, 64, 32, MX_SCALE_E8M0, 1.0f, MX_LAYOUT_ROWMAJOR, c, s, nullptr), MX_ERR_INVALID_ARG);
    EXPECT_NO_LAUNCH(mx_quantize(x, MX_BF16, 4, 64, 63, 32, MX_SCALE_E8M0, 1.0f, MX_LAYOUT_ROWMAJOR, c, s, nullptr), MX_ERR_INVALID_ARG);
    EXPECT_NO_LAUNCH(mx_quantize(nullptr, MX_BF16, 4, 64, 64, 32, MX_SCALE_E8M0, 1.0f, MX_LAYOUT_ROWMAJOR, c, s, nullptr), MX_ERR_INVALID_ARG);
    EXPECT_NO_LAUNCH(mx_quantize(x, MX_BF16, 4, 64, 64, 32, MX_SCALE_E8M0, 1.0f, MX_LAYOUT_ROWMAJOR, nullptr, s, nullptr), MX_ERR_INVALID_ARG);
    EXPECT_NO_LAUNCH(mx_quantize(x, MX_BF16, 4, 64, 64, 32, MX_SCALE_E8M0, 1.0f, MX_LAYOUT_ROWMAJOR, c, nullptr, nullptr), MX_ERR_INVALID_ARG);
    EXPECT_NO_LAUNCH(mx_quantize(x + 8, MX_BF16, 4, 64, 64, 32, MX_SCALE_E8M0, 1.0f, MX_LAYOUT_ROWMAJOR, c, s, nullptr), MX_ERR_ALIGNMENT);
    EXPECT_NO_LAUNCH(mx_quantize(x, MX_BF16, 4, 64, 64, 32, MX_SCALE_E8M0, 1.0f, MX_LAYOUT_ROWMAJOR, c, s + 4, nullptr), MX_ERR_ALIGNMENT);
    EXPECT_NO_LAUNCH(mx_quantize(x, MX_BF16, 4, 64, 64, 16, MX_SCALE_E8M0, 1.0f, MX_LAYOUT_TILED, c, s, nullptr), MX_ERR_UNSUPPORTED);
    EXPECT_NO_LAUNCH(mx_quantize(x, MX_BF16, 4, (int64_t(1) << 22) + 32, (int64_t(1) << 22) + 32, 32, MX_SCALE_E8M0, 1.0f,
                                 MX_LAYOUT_TILED, c, s, nullptr), MX_ERR_UNSUPPORTED);
    EXPECT_NO_LAUNCH(mx_quantize(x, MX_BF16, 4, 64, 64, 64, MX_SCALE_E8M0, 1.0f, MX_LAYOUT_PRESHUFFLED, c, s, nullptr), MX_ERR_UNSUPPORTED);
    EXPECT_NO_LAUNCH(mx_quantize(x, MX_BF16, 4, (int64_t(1) << 25) + 32, (int64_t(1) << 25) + 32, 32, MX_SCALE_E8M0, 1.0f,
                                 MX_LAYOUT_ROWMAJOR, c, s, nullptr), MX_ERR_UNSUPPORTED);
    // empty tensors: success, nothing launched (null pointers allowed)
    EXPECT_NO_LAUNCH(mx_quantize(nullptr, MX_BF16, 0, 64, 64, 32, MX_SCALE_E8M0, 1.0f, MX_LAYOUT_ROWMAJOR, nullptr, nullptr, nullptr), MX_OK);
    EXPECT_NO_LAUNCH(mx_quantize(nullptr, MX_F32, 5, 0, 0, 32, MX_SCALE_E8M0, 1.0f, MX_LAYOUT_ROWMAJOR, nullptr, nullptr, nullptr), MX_OK);

    // one launch
    EXPECT(mx_quantize(x, MX_BF16, 5, 64, 64, 32, MX_SCALE_E8M0, 1.0f, MX_LAYOUT_ROWMAJOR, c, s, nullptr), MX_OK);
    CHECK(g_launches.size() == 1 && std::strcmp(g_launches[0].what, "quantize") == 0 && g_launches[0].rows == 5);

    // row chunks: k = 2^20 -> 2^29 / 2^19 = 1024 rows per launch; codes k/2 bytes per row,
    // row-major scales k/32 bytes per row
    const int64_t K = int64_t(1) << 20;
    EXPECT(mx_quantize(x, MX_BF16, 2000, K, K, 32, MX_SCALE_UE5M3, 0.37f, MX_LAYOUT_ROWMAJOR, c, s, nullptr), MX_OK);
    CHECK(g_launches.size() == 2);
    if (g_launches.size() == 2) {
        CHECK(g_launches[0].rows == 1024 && g_launches[1].rows == 976);
        CHECK(ptr(g_launches[1].in) == x + 1024 * K * 2);
        CHECK(ptr(g_launches[1].out) == c + 1024 * (K / 2));
        CHECK(ptr(g_launches[1].aux) == s + 1024 * (K / 32));
    }
    // tiled scales: chunks of whole 256-row tiles; a tile's scales take stages(k) 2 KB blocks
    const int64_t K2 = int64_t(1) << 21;
    EXPECT(mx_quantize(x, MX_F32, 1000, K2, K2, 32, MX_SCALE_E8M0, 1.0f, MX_LAYOUT_TILED, c, s, nullptr), MX_OK);
    CHECK(g_launches.size() == 2);
    if (g_launches.size() == 2) {
        CHECK(g_launches[0].rows == 512 && g_launches[1].rows == 488);
        CHECK(ptr(g_launches[1].in) == x + 512 * K2 * 4);
        CHECK(ptr(g_launches[1].aux) == s + (512 / 256) * (K2 / 256) * 2048);
    }
    CHECK(mx_scale_bytes(1000, K2, 32, MX_LAYOUT_TILED) == size_t(4) * (K2 / 256) * 2048);
    CHECK(mx_scale_bytes(20, 4096, 32, MX_LAYOUT_PRESHUFFLED) == size_t(3) * 2 * 512);
    CHECK(mx_scale_bytes(int64_t(1) << 50, 64, 32, MX_LAYOUT_ROWMAJOR) == (size_t(1) << 51));
    CHECK(mx_scale_bytes(4, 64, 16, MX_LAYOUT_TILED) == 0 && mx_scale_bytes(-1, 64, 32, MX_LAYOUT_ROWMAJOR) == 0);

    // a launch error maps to MX_ERR_HIP
    g_fail_next = true;
    EXPECT(mx_quantize(x, MX_BF16, 5, 64, 64, 32, MX_SCALE_E8M0, 1.0f, MX_LAYOUT_ROWMAJOR, c, s, nullptr), MX_ERR_HIP);
    g_fail_next = false;

    // dequantize: the same rules on the output side
    EXPECT_NO_LAUNCH(mx_dequantize(c, s, 4, 64, 32, MX_SCALE_E8M0, 1.0f, MX_LAYOUT_ROWMAJOR, x, MX_BF16, 63, nullptr), MX_ERR_INVALID_ARG);
    EXPECT_NO_LAUNCH(mx_dequantize(c, s, 4, 64, 32, MX_SCALE_E8M0, 1.0f, MX_LAYOUT_ROWMAJOR, x + 4, MX_BF16, 64, nullptr), MX_ERR_ALIGNMENT);
    EXPECT(mx_dequantize(c, s, 2000, K, 32, MX_SCALE_E4M3, 1.0f, MX_LAYOUT_ROWMAJOR, x, MX_F32, K, nullptr), MX_OK);
    CHECK(g_launches.size() == 2);
    if (g_launches.size() == 2) {
        CHECK(ptr(g_launches[1].out) == x + 1024 * K * 4 && ptr(g_launches[1].in) == c + 1024 * (K / 2));
    }
}

static void gemm_rules()
{
    uint8_t *x = fake(0), *wc = fake(1u << 30), *ws = fake(3u << 30), *y = fake(uint64_t(8) << 30),
            *work = fake(uint64_t(64) << 30);
    EXPECT_NO_LAUNCH(mx_gemm(x, -1, 64, 64, 64, wc, ws, 32, MX_SCALE_E8M0, 1.0f, MX_LAYOUT_ROWMAJOR, MX_A16, y, MX_BF16, 64, nullptr, 0, nullptr), MX_ERR_INVALID_ARG);
    EXPECT_NO_LAUNCH(mx_gemm(x, 4, -1, 64, 64, wc, ws, 32, MX_SCALE_E8M0, 1.0f, MX_LAYOUT_ROWMAJOR, MX_A16, y, MX_BF16, 64, nullptr, 0, nullptr), MX_ERR_INVALID_ARG);
    EXPECT_NO_LAUNCH(mx_gemm(x, 4, 64, 64, 64, wc, ws, 32, MX_SCALE_E8M0, 1.0f, MX_LAYOUT_ROWMAJOR, (mx_act_mode)5, y, MX_BF16, 64, nullptr, 0, nullptr), MX_ERR_INVALID_ARG);
    EXPECT_NO_LAUNCH(mx_gemm(x, 4, 64, 64, 64, wc, ws, 32, MX_SCALE_E8M0, 1.0f, MX_LAYOUT_ROWMAJOR, MX_A16, y, (mx_dtype)3, 64, nullptr, 0, nullptr), MX_ERR_INVALID_ARG);
    EXPECT_NO_LAUNCH(mx_gemm(x, 4, 64, 64, 32, wc, ws, 32, MX_SCALE_E8M0, 1.0f, MX_LAYOUT_ROWMAJOR, MX_A16, y, MX_BF16, 64, nullptr, 0, nullptr), MX_ERR_INVALID_ARG);
    EXPECT_NO_LAUNCH(mx_gemm(x, 4, 64, 64, 64, wc, ws, 32, MX_SCALE_E8M0, 1.0f, MX_LAYOUT_ROWMAJOR, MX_A16, y, MX_BF16, 63, nullptr, 0, nullptr), MX_ERR_INVALID_ARG);
    EXPECT_NO_LAUNCH(mx_gemm(x, 4, 64, 256, 256, wc, ws, 32, MX_SCALE_E4M3, 1.0f, MX_LAYOUT_ROWMAJOR, MX_A4, y, MX_BF16, 64, work, 1 << 20, nullptr), MX_ERR_UNSUPPORTED);
    EXPECT_NO_LAUNCH(mx_gemm(x, 4, 64, 256, 256, wc, ws, 16, MX_SCALE_E8M0, 1.0f, MX_LAYOUT_ROWMAJOR, MX_A4, y, MX_BF16, 64, work, 1 << 20, nullptr), MX_ERR_UNSUPPORTED);
    EXPECT_NO_LAUNCH(mx_gemm(x, 4, 64, 64, 64, wc, ws, 32, MX_SCALE_E8M0, 1.0f, MX_LAYOUT_ROWMAJOR, MX_A16, nullptr, MX_BF16, 64, nullptr, 0, nullptr), MX_ERR_INVALID_ARG);
    EXPECT_NO_LAUNCH(mx_gemm(x, 4, 64, 64, 64, wc, ws, 32, MX_SCALE_E8M0, 1.0f, MX_LAYOUT_ROWMAJOR, MX_A16, y + 2, MX_BF16, 64, nullptr, 0, nullptr), MX_ERR_ALIGNMENT);
    EXPECT_NO_LAUNCH(mx_gemm(nullptr, 4, 64, 64, 64, wc, ws, 32, MX_SCALE_E8M0, 1.0f, MX_LAYOUT_ROWMAJOR, MX_A16, y, MX_BF16, 64, nullptr, 0, nullptr), MX_ERR_INVALID_ARG);
    EXPECT_NO_LAUNCH(mx_gemm(x, 4, 64, 64, 64, wc + 1, ws, 32, MX_SCALE_E8M0, 1.0f, MX_LAYOUT_ROWMAJOR, MX_A16, y, MX_BF16, 64, nullptr, 0, nullptr), MX_ERR_ALIGNMENT);
    EXPECT_NO_LAUNCH(mx_gemm(x, 4, 64, (int64_t(1) << 22) + 512, (int64_t(1) << 22) + 512, wc, ws, 32, MX_SCALE_E8M0, 1.0f,
                             MX_LAYOUT_ROWMAJOR, MX_A16, y, MX_BF16, 64, nullptr, 0, nullptr), MX_ERR_UNSUPPORTED);
    // tiled weight scales are for the W4A4 matrix-core product only
    EXPECT_NO_LAUNCH(mx_gemm(x, 4, 64, 256, 256, wc, ws, 32, MX_SCALE_E8M0, 1.0f, MX_LAYOUT_TILED, MX_A16, y, MX_BF16, 64, nullptr, 0, nullptr), MX_ERR_UNSUPPORTED);
    // preshuffled weight scales are for the m = 1 W4A16 product only
    EXPECT_NO_LAUNCH(mx_gemm(x, 2, 64, 256, 256, wc, ws, 32, MX_SCALE_E8M0, 1.0f, MX_LAYOUT_PRESHUFFLED, MX_A16, y, MX_BF16, 64, nullptr, 0, nullptr), MX_ERR_UNSUPPORTED);
    // empty products
    EXPECT_NO_LAUNCH(mx_gemm(nullptr, 0, 64, 64, 64, nullptr, nullptr, 32, MX_SCALE_E8M0, 1.0f, MX_LAYOUT_ROWMAJOR, MX_A16, nullptr, MX_BF16, 64, nullptr, 0, nullptr), MX_OK);
    EXPECT(mx_gemm(nullptr, 3, 5, 0, 0, nullptr, nullptr, 32, MX_SCALE_E8M0, 1.0f, MX_LAYOUT_ROWMAJOR, MX_A16, y, MX_F32, 5, nullptr, 0, nullptr), MX_OK);
    CHECK(g_launches.size() == 1 && std::strcmp(g_launches[0].what, "fill_zero") == 0 && g_launches[0].rows == 3);

    // W4A16 in row chunks: per row max(n, k/2) = 2^20 units -> 512 rows (a multiple of 256) per launch
    const int64_t N = int64_t(1) << 20, K = 1024;
    EXPECT(mx_gemm(x, 1300, N, K, K, wc, ws, 32, MX_SCALE_E8M0, 1.0f, MX_LAYOUT_ROWMAJOR, MX_A16, y, MX_BF16, N, nullptr, 0, nullptr), MX_OK);
    CHECK(g_launches.size() == 3);
    if (g_launches.size() == 3) {
        CHECK(g_launches[0].rows == 512 && g_launches[1].rows == 512 && g_launches[2].rows == 276);
        CHECK(ptr(g_launches[2].in) == x + 1024 * K * 2 && ptr(g_launches[2].out) == y + 1024 * N * 2);
        CHECK(ptr(g_launches[2].aux) == wc && ptr(g_launches[2].aux2) == ws);
    }

    // W4A4: activation pre-pass into the workspace (codes, then tiled scales at a 256-byte
    // boundary), then the product reading them
    const int64_t M4 = 300, N4 = 512, K4 = 256;
    const size_t need = mx_gemm_workspace_size(M4, N4, K4, 32, MX_A4);
    CHECK(need == 38400 + 4096);
    CHECK(mx_gemm_workspace_size(M4, N4, K4, 32, MX_A16) == 0 && mx_gemm_workspace_size(M4, N4, K4, 16, MX_A4) == 0);
    EXPECT_NO_LAUNCH(mx_gemm(x, M4, N4, K4, K4, wc, ws, 32, MX_SCALE_E8M0, 1.0f, MX_LAYOUT_ROWMAJOR, MX_A4, y, MX_BF16, N4, nullptr, need, nullptr), MX_ERR_INVALID_ARG);
    EXPECT_NO_LAUNCH(mx_gemm(x, M4, N4, K4, K4, wc, ws, 32, MX_SCALE_E8M0, 1.0f, MX_LAYOUT_ROWMAJOR, MX_A4, y, MX_BF16, N4, work, need - 1, nullptr), MX_ERR_INVALID_ARG);
    EXPECT_NO_LAUNCH(mx_gemm(x, M4, N4, K4, K4, wc, ws, 32, MX_SCALE_E8M0, 1.0f, MX_LAYOUT_ROWMAJOR, MX_A4, y, MX_BF16, N4, work + 8, need, nullptr), MX_ERR_ALIGNMENT);
    EXPECT(mx_gemm(x, M4, N4, K4, K4, wc, ws, 32, MX_SCALE_E8M0, 1.0f, MX_LAYOUT_ROWMAJOR, MX_A4, y, MX_BF16, N4, work, need, nullptr), MX_OK);
    CHECK(g_launches.size() == 2);
    if (g_launches.size() == 2) {
        CHECK(std::strcmp(g_launches[0].what, "quantize") == 0 && g_launches[0].rows == M4);
        CHECK(ptr(g_launches[0].in) == x && ptr(g_launches[0].out) == work && ptr(g_launches[0].aux) == work + 38400);
        CHECK(std::strcmp(g_launches[1].what, "gemm_a4") == 0 && ptr(g_launches[1].in) == work &&
              ptr(g_launches[1].aux) == work + 38400 && ptr(g_launches[1].out) == y);
    }
    // workspace sizes for very large shapes stay exact in size_t
    CHECK(mx_gemm_workspace_size(int64_t(1) << 40, 64, int64_t(1) << 22, 32, MX_A4) ==
          (size_t(1) << 61) + (size_t(1) << 32) * (size_t(1) << 14) * 2048);
    CHECK(mx_gemm_workspace_size(-1, 64, 64, 32, MX_A4) == 0);
}

static void statistics_and_fp8()
{
    uint8_t *x = fake(0), *out = fake(1u << 30), *work = fake(2u << 30), *c = fake(3u << 30), *s = fake(4u << 30),
            *y = fake(uint64_t(8) << 30);
    double* o = reinterpret_cast<double*>(out);
    const size_t need = mx_quant_error_workspace_size(64, 256, 32);
    CHECK(need == 768);
    EXPECT_NO_LAUNCH(mx_quant_error(x, MX_BF16, 64, 256, 256, 32, MX_SCALE_E8M0, 1.0f, nullptr, 0, o, work, need - 1, nullptr), MX_ERR_INVALID_ARG);
    EXPECT_NO_LAUNCH(mx_quant_error(x, MX_BF16, 64, 256, 256, 32, MX_SCALE_E8M0, 1.0f, nullptr, 0, o, nullptr, need, nullptr), MX_ERR_INVALID_ARG);
    EXPECT_NO_LAUNCH(mx_quant_error(x, MX_BF16, 64, 256, 256, 32, MX_SCALE_E8M0, 1.0f, y, 255, o, work, need, nullptr), MX_ERR_INVALID_ARG);
    EXPECT_NO_LAUNCH(mx_quant_error(x, MX_BF16, 64, 256, 256, 32, MX_SCALE_E8M0, 1.0f, nullptr, 0, nullptr, work, need, nullptr), MX_ERR_INVALID_ARG);
    EXPECT_NO_LAUNCH(mx_quant_error(x, MX_BF16, 64, 256, 256, 32, MX_SCALE_E8M0, 1.0f, y + 2, 256, o, work, need, nullptr), MX_ERR_ALIGNMENT);
    EXPECT(mx_quant_error(x, MX_BF16, 64, 256, 256, 32, MX_SCALE_E8M0, 1.0f, y, 256, o, work, need, nullptr), MX_OK);
    CHECK(g_launches.size() == 1 && std::strcmp(g_launches[0].what, "quant_error") == 0 && ptr(g_launches[0].aux) == work);

    const size_t sneed = mx_tensor_stats_workspace_size(64, 256);
    CHECK(sneed == 256 && mx_tensor_stats_workspace_size(0, 256) == 0);
    EXPECT_NO_LAUNCH(mx_tensor_stats(x, MX_BF16, 64, 256, 255, o, work, sneed, nullptr), MX_ERR_INVALID_ARG);
    EXPECT_NO_LAUNCH(mx_tensor_stats(x, MX_BF16, 64, 256, 256, o, work, sneed - 8, nullptr), MX_ERR_INVALID_ARG);
    EXPECT(mx_tensor_stats(x, MX_BF16, 64, 256, 256, o, work, sneed, nullptr), MX_OK);
    CHECK(g_launches.size() == 1 && std::strcmp(g_launches[0].what, "tensor_stats") == 0);
    // 2^31 load units (8 elements each) and beyond: unsupported
    const int64_t big_rows = int64_t(1) << 31;
    EXPECT_NO_LAUNCH(mx_tensor_stats(x, MX_BF16, big_rows, 8, 8, o, work, mx_tensor_stats_workspace_size(big_rows, 8), nullptr),
                     MX_ERR_UNSUPPORTED);

    EXPECT_NO_LAUNCH(mx_quantize_fp8(x, MX_BF16, 4, 64, 64, 32, MX_SCALE_E8M0, 0.0f, c, s, nullptr), MX_ERR_INVALID_ARG);
    EXPECT(mx_quantize_fp8(x, MX_F32, 4, 64, 64, 32, MX_SCALE_UE5M3, 2.5f, c, s, nullptr), MX_OK);
    CHECK(g_launches.size() == 1 && std::strcmp(g_launches[0].what, "quantize_fp8") == 0);
    EXPECT(mx_dequantize_fp8(c, s, 4, 64, 32, MX_SCALE_E8M0, 1.0f, y, MX_BF16, 64, nullptr), MX_OK);
    CHECK(g_launches.size() == 1 && std::strcmp(g_launches[0].what, "dequantize_fp8") == 0);
    EXPECT(mx_gemm_fp8(x, 16, 96, 256, 256, c, s, 32, MX_SCALE_E8M0, 1.0f, y, MX_F32, 96, nullptr), MX_OK);
    CHECK(g_launches.size() == 1 && std::strcmp(g_launches[0].what, "gemm_w8") == 0 && g_launches[0].rows == 16);

    CHECK(mx_adaptive_block_size(std::nan("")) == 32 && mx_adaptive_block_size(0.005) == 128 &&
          mx_adaptive_block_size(0.05) == 64);
    CHECK(mx_layer_block_size((mx_layer_kind)9) == 0 && mx_layer_block_size(MX_LAYER_QKV) == 64);
    CHECK(mx_use_fp8(1e-5) == 1 && mx_use_fp8(0.02) == 0);
}

int main()
{
    status_strings();
    quantize_rules();
    gemm_rules();
    statistics_and_fp8();
    if (g_failed) {
        std::printf("%d of %d checks failed\n", g_failed, g_checks);
        return 1;
    }
    std::printf("all %d checks passed\n", g_checks);
    return 0;
}
