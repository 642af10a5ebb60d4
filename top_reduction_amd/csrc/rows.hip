// rows.hip -- row targets of a packed batch (vllm-metal release v0.4.0,
// Summary): validates cu_seqlens on the device and writes the optional
// gather_indices and logits_cu_seqlens outputs. The head kernels derive each
// row's source themselves (row_source), so this kernel only runs when one of
// those outputs or the error word is requested.
#include "lmh_internal.h"

namespace lmh {
namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void k_rows(RowsArgs a) {
    const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    const int32_t S = a.num_segments;
    int32_t bits = 0;

    if (i < S) {
        const int32_t lo = a.cu[i], hi = a.cu[i + 1];
        const int32_t len = hi - lo;
        if (len < 0) bits |= LMH_DEVERR_LAYOUT;
        if (i < a.num_decode && len != 1) bits |= LMH_DEVERR_LAYOUT;
        if (a.ex == nullptr && len == 0) bits |= LMH_DEVERR_LAYOUT;
        if (i == 0 && lo != 0) bits |= LMH_DEVERR_LAYOUT;
        if (i == S - 1 && (int64_t)hi > a.num_tokens) bits |= LMH_DEVERR_LAYOUT;
    }
    if (i < a.rows) {
        const int32_t t = row_source((int32_t)i, a.cu, a.num_decode, a.num_tokens, a.ex);
        if (t < 0) bits |= (a.ex != nullptr) ? LMH_DEVERR_INDEX : LMH_DEVERR_LAYOUT;
        if (a.gather_out) a.gather_out[i] = t;
    }
    if (a.lcu_out != nullptr && i <= S) {
        if (a.ex == nullptr) {
            a.lcu_out[i] = (int32_t)i;
        } else {
            const int32_t c = a.cu[i];
            int32_t n = 0;
            for (int32_t r = 0; r < a.rows; ++r) n += (a.ex[r] < c) ? 1 : 0;
            a.lcu_out[i] = n;
        }
    }
    if (bits != 0 && a.err != nullptr) atomicOr(a.err, bits);
}

}  // namespace

hipError_t launch_rows(const RowsArgs& a, hipStream_t s) {
    const int64_t n = (a.rows > a.num_segments + 1) ? a.rows : (int64_t)a.num_segments + 1;
    const dim3 grid((unsigned)((n + kThreads - 1) / kThreads));
    hipLaunchKernelGGL(k_rows, grid, dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace lmh
