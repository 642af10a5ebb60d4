// noalloc.hip -- logprob_reduce without a workspace argument, for callers
// that cannot allocate device memory (code under HIP graph capture, tight
// serving loops, harnesses that forbid hipMalloc).
//
// The reduction's scratch (the two-launch path's per-item partials and block
// keys, or the single-launch path's partials and per-slice top-K lists) and
// the single-launch path's per-row arrival counters live in one file-scope
// device array per GPU, `scratch`, held until the process ends. Host code
// never passes the array's name to a kernel (in host code it stands for a
// host-side shadow, not a device address): the first call on a device, with
// that device current, asks the runtime for the array's device address on
// that device, keeps it, and clears the counters with a small fill kernel on
// the caller's stream; every later call on that device passes the kept
// pointer. No call allocates or frees memory.
//
// Every call on one GPU shares that GPU's array, and the array keeps what the
// last call left in it. The partials and lists need no clearing (each launch
// writes everything it reads); the counters are zero between calls because
// each row's last workgroup puts its counter back to zero. Calls that overlap
// on one GPU (on different streams, or from different host threads without
// ordering) race on the array; callers order them.
#include <mutex>

#include "lmh_internal.h"

namespace {

constexpr size_t kWorkBytes = LMH_NOALLOC_SCRATCH_BYTES;                    // partials, keys, lists
constexpr size_t kCounterBytes = (size_t)LMH_SINGLE_MAX_ROWS * sizeof(uint32_t);
constexpr size_t kScratchBytes = kWorkBytes + kCounterBytes;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];   // device address of `scratch`, per device

__global__ void k_zero_words(uint32_t* p, int n) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0u;
}

// The device address of `scratch` on the current device, looked up once; the
// first lookup on a device also enqueues the clearing of the counters on s.
hipError_t scratch_address(void** out, hipStream_t s) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (p == nullptr) return hipErrorInvalidSymbol;
        constexpr int n = (int)(kCounterBytes / sizeof(uint32_t));
        hipLaunchKernelGGL(k_zero_words, dim3((n + 255) / 256), dim3(256), 0, s,
                           reinterpret_cast<uint32_t*>(static_cast<char*>(p) + kWorkBytes), n);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace

extern "C" {

lmh_status logprob_reduce_noalloc(const void* logits, lmh_dtype logits_dt, int64_t rows, int64_t vocab,
                                  int64_t logits_ld, const int32_t* selected_ids, int32_t k, float* lse,
                                  float* selected_logprob, int32_t* topk_ids, float* topk_logprobs,
                                  int32_t* device_error, void* stream) {
    size_t need = 0;
    const lmh_status st = lmh::reduce_validate(logits, logits_dt, rows, vocab, logits_ld, selected_ids, k,
                                               lse, selected_logprob, topk_ids, topk_logprobs, &need);
    if (st != LMH_OK) return st;
    if (rows == 0) return LMH_OK;   // nothing is read or written
    if (need > kWorkBytes) return LMH_ERR_WORKSPACE;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    void* ws = nullptr;
    if (scratch_address(&ws, s) != hipSuccess) return LMH_ERR_HIP;
    uint32_t* counters = reinterpret_cast<uint32_t*>(static_cast<char*>(ws) + kWorkBytes);
    return lmh::reduce_enqueue(logits, logits_dt, rows, vocab, logits_ld, selected_ids, k, lse,
                               selected_logprob, topk_ids, topk_logprobs, ws, device_error, s, counters);
}

}  // extern "C"
