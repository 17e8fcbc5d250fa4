// Host-only stand-ins for the device launchers of libmx, so that the C-ABI layer
// (csrc/mx_api.cpp) can be built with the host compiler under AddressSanitizer and
// UndefinedBehaviorSanitizer and driven without a GPU.  Each launcher records its call (which
// launcher, the row or m count it was handed, and its principal pointers) and returns
// hipSuccess, or hipErrorInvalidValue when the driver asks the next launch to fail.  The three
// helper functions return values of the right kind: a4_uses_mfma the k condition of the
// matrix-core W4A4 kernel, the group counts a positive number within their caps.
#include <vector>

#include "mx_internal.h"
#include "stubs.h"

std::vector<LaunchRecord> g_launches;
bool g_fail_next = false;

namespace {
hipError_t record(const char* what, int64_t rows, const void* in, const void* out, const void* aux = nullptr,
                  const void* aux2 = nullptr)
{
    g_launches.push_back(LaunchRecord{what, rows, in, out, aux, aux2});
    if (g_fail_next) {
        g_fail_next = false;
        return hipErrorInvalidValue;
    }
    return hipSuccess;
}
}  // namespace

namespace mxk {
bool a4_uses_mfma(const GemmArgs& a) { return a.k % 128 == 0; }
int quant_error_groups(int64_t rows, int64_t k, int) { return rows * k > (1 << 20) ? kErrMaxGroups : 16; }
int stats_groups(int64_t rows, int64_t k) { return rows * k > (1 << 20) ? kStatsMaxGroups : 16; }

hipError_t launch_quantize(const QuantArgs& a, hipStream_t) { return record("quantize", a.rows, a.x, a.codes, a.scales); }
hipError_t launch_dequantize(const DequantArgs& a, hipStream_t) { return record("dequantize", a.rows, a.codes, a.y, a.scales); }
hipError_t launch_quantize_fp8(const QuantArgs& a, hipStream_t) { return record("quantize_fp8", a.rows, a.x, a.codes, a.scales); }
hipError_t launch_dequantize_fp8(const DequantArgs& a, hipStream_t) { return record("dequantize_fp8", a.rows, a.codes, a.y, a.scales); }
hipError_t launch_quant_error(const ErrArgs& a, hipStream_t) { return record("quant_error", a.rows, a.x, a.out, a.partials); }
hipError_t launch_tensor_stats(const StatsArgs& a, hipStream_t) { return record("tensor_stats", a.rows, a.x, a.out, a.partials); }
hipError_t launch_gemm_a16(const GemmArgs& a, hipStream_t) { return record("gemm_a16", a.m, a.x, a.y, a.wc, a.ws); }
hipError_t launch_gemm_a4(const GemmArgs& a, hipStream_t) { return record("gemm_a4", a.m, a.xq_codes, a.y, a.xq_scales, a.x); }
hipError_t launch_gemm_w8(const W8Args& a, hipStream_t) { return record("gemm_w8", a.m, a.x, a.y, a.wc, a.ws); }
hipError_t launch_fill_zero(void* y, int64_t m, int64_t, int64_t, bool, hipStream_t) { return record("fill_zero", m, nullptr, y); }
}  // namespace mxk
