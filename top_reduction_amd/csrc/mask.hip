// mask.hip -- token bitmask on the compacted logits (vllm-metal release
// v0.4.0, Testing: bitmask application under the compacted layout).
//
//   Segment s owns the logits rows lcu[s] .. lcu[s+1]-1 (the head's
//   logits_cu_seqlens; without them segment s is row s). Token v of those
//   rows keeps its value when bit v % 32 of word v / 32 of mask row s is
//   set, and becomes -inf otherwise.
//
// The logits are written, never read. Each thread owns one 16-byte group of
// a row (8 bf16/f16 or 4 fp32 tokens, inside one mask word), so a wave's
// stores cover consecutive memory: a fully masked group is one 16-byte store
// of -inf, a fully kept one writes nothing, a mixed one writes its masked
// tokens one element at a time. The row pitch's padding past the vocabulary
// is never touched.
#include "lmh_internal.h"

namespace lmh {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kMaskThreads = 256;

// The buffer may hold a window of the compacted rows: buffer row i is
// compacted row win0 + i, for `rows` rows, out of total_rows (the fused
// path masks one chunk of logits at a time); segment bounds are checked
// against total_rows and clipped to the window.
template <int ES>   // element size: 2 (bf16, f16) or 4 (fp32)
__global__ __launch_bounds__(kMaskThreads) void k_apply_bitmask(uint8_t* __restrict__ logits, int64_t ld,
                                                                int64_t rows, int64_t win0, int64_t total_rows,
                                                                int64_t V, const uint32_t* __restrict__ mask,
                                                                int64_t mask_ld, const int32_t* __restrict__ lcu,
                                                                int32_t chunks, uint32_t ninf,
                                                                int32_t* __restrict__ err) {
    constexpr int EPG = 16 / ES;                     // tokens per 16-byte group (divides 32)
    const int32_t s = (int32_t)(blockIdx.x / (uint32_t)chunks);
    const int64_t g = (int64_t)(blockIdx.x - (uint32_t)s * (uint32_t)chunks) * kMaskThreads + threadIdx.x;
    int64_t r0 = s, r1 = (int64_t)s + 1;
    if (lcu != nullptr) {
        r0 = lcu[s];
        r1 = lcu[s + 1];
    }
    if (r0 < 0 || r1 < r0 || r1 > total_rows) {   // malformed bounds: the segment is left alone
        if (err != nullptr && g == 0) atomicOr(err, LMH_DEVERR_LAYOUT);
        return;
    }
    r0 = (r0 > win0 ? r0 : win0) - win0;             // the segment's rows inside the window
    r1 = (r1 < win0 + rows ? r1 : win0 + rows) - win0;
    const int64_t v0 = g * EPG;
    if (v0 >= V || r0 >= r1) return;
    const int nv = V - v0 < EPG ? (int)(V - v0) : EPG;              // tokens of this group in the row
    const uint32_t keep = (mask[(int64_t)s * mask_ld + v0 / 32] >> (v0 % 32)) & ((1u << EPG) - 1u);
    const uint32_t live = (1u << nv) - 1u;
    if ((keep & live) == live) return;                                // nothing masked
    for (int64_t r = r0; r < r1; ++r) {
        uint8_t* row = logits + r * ld * ES;
        if (keep == 0u && nv == EPG) {
            const u32x4 fill = {ninf, ninf, ninf, ninf};
            *reinterpret_cast<u32x4*>(row + v0 * ES) = fill;   // base and pitch 16-byte aligned, v0 * ES too
        } else {
            for (int e = 0; e < nv; ++e) {
                if (((keep >> e) & 1u) == 0u) {
                    if (ES == 2)
                        reinterpret_cast<uint16_t*>(row)[v0 + e] = (uint16_t)ninf;
                    else
                        reinterpret_cast<uint32_t*>(row)[v0 + e] = ninf;
                }
            }
        }
    }
}

}  // namespace

hipError_t launch_apply_bitmask(const MaskArgs& a, hipStream_t s) {
    if (a.segments == 0) return hipSuccess;
    const int64_t groups = (a.vocab + (a.dt == LMH_F32 ? 3 : 7)) / (a.dt == LMH_F32 ? 4 : 8);   // 16-byte groups
    const int64_t chunks = (groups + kMaskThreads - 1) / kMaskThreads;
    const dim3 grid((unsigned)(chunks * a.segments));
    uint8_t* lg = static_cast<uint8_t*>(a.logits);
    const uint32_t* m = reinterpret_cast<const uint32_t*>(a.mask);
    const int64_t total = a.total_rows > 0 ? a.total_rows : a.rows;
    if (a.dt == LMH_F32)
        hipLaunchKernelGGL((k_apply_bitmask<4>), grid, dim3(kMaskThreads), 0, s, lg, a.ld, a.rows, a.win0, total,
                           a.vocab, m, a.mask_ld, a.lcu, (int32_t)chunks, 0xFF800000u, a.err);
    else
        hipLaunchKernelGGL((k_apply_bitmask<2>), grid, dim3(kMaskThreads), 0, s, lg, a.ld, a.rows, a.win0, total,
                           a.vocab, m, a.mask_ld, a.lcu, (int32_t)chunks,
                           a.dt == LMH_BF16 ? 0xFF80FF80u : 0xFC00FC00u, a.err);
    return hipGetLastError();
}

}  // namespace lmh
