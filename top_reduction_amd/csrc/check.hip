// check.hip -- bitwise self-check of selective logits rows against the rows
// of a full projection (vllm-metal release, Summary: selective logits are
// only used for a head whose selected rows match the model's own output bit
// for bit; the load-time probe that checks this is replaced here by an entry
// point that compares against logits the caller supplies).
#include <climits>

#include "lmh_internal.h"

namespace lmh {
namespace {

constexpr int kCheckThreads = 256;

__global__ void k_check_init(int64_t* res) {
    if (threadIdx.x == 0) {
        res[0] = 0;
        res[1] = INT64_MAX;
    }
}

// grid (x: column blocks, y: logits rows); each thread compares a strided
// set of columns of one row and adds its counts with one atomic at the end
// (none when everything matches)
__global__ __launch_bounds__(kCheckThreads) void k_selfcheck(const float* sel, int64_t sel_ld,
                                                          const float* full, int64_t full_ld,
                                                          int64_t vocab, const int32_t* cu,
                                                          int32_t num_decode, int64_t num_tokens,
                                                          const int32_t* ex, int64_t* res) {
    const int32_t r = (int32_t)blockIdx.y;
    const int32_t t = row_source(r, cu, num_decode, num_tokens, ex);
    if (t < 0) return;
    const float* a = sel + (int64_t)r * sel_ld;
    const float* b = full + (int64_t)t * full_ld;
    unsigned long long cnt = 0;
    long long first = LLONG_MAX;
    for (int64_t v = (int64_t)blockIdx.x * kCheckThreads + threadIdx.x; v < vocab;
         v += (int64_t)gridDim.x * kCheckThreads) {
        if (__float_as_uint(a[v]) != __float_as_uint(b[v])) {
            ++cnt;
            const long long flat = (long long)r * vocab + v;
            first = flat < first ? flat : first;
        }
    }
    if (cnt != 0) {
        atomicAdd(reinterpret_cast<unsigned long long*>(&res[0]), cnt);
        atomicMin(reinterpret_cast<long long*>(&res[1]), first);
    }
}

}  // namespace

hipError_t launch_selfcheck(const float* sel, int64_t sel_ld, const float* full, int64_t full_ld,
                            int32_t rows, int64_t vocab, const int32_t* cu, int32_t num_decode,
                            int64_t num_tokens, const int32_t* ex, int64_t* res, hipStream_t s) {
    hipLaunchKernelGGL(k_check_init, dim3(1), dim3(64), 0, s, res);
    if (rows <= 0) return hipGetLastError();
    const int64_t cols = (vocab + kCheckThreads - 1) / kCheckThreads;
    const dim3 grid((unsigned)(cols < 64 ? cols : 64), (unsigned)rows);
    hipLaunchKernelGGL(k_selfcheck, grid, dim3(kCheckThreads), 0, s, sel, sel_ld, full, full_ld, vocab,
                       cu, num_decode, num_tokens, ex, res);
    return hipGetLastError();
}

}  // namespace lmh
