// head_common.h -- device helpers and launch parameters shared by the head
// kernels (head.hip, pipe.hip): the bf16 MFMA step, the affine group
// dequantisation, the quantised k order and the head's output scaling.
#pragma once

#include <type_traits>

#include "lmh_internal.h"

namespace lmh {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kNaN = __builtin_nanf("");

__device__ inline f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                    __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Affine group-quantised weights: token v, hidden index k, g = k >> gshift:
//   W[v][k] = bf16( fma(scale[v][g], q(v, k), bias[v][g]) )
// q(v, k) the unsigned BITS-bit code at bit k*BITS of row v of q (32-bit
// words, little-endian), scale and bias bf16. The product of a bf16 and a
// code of at most 8 bits is exact in fp32, so the only roundings are the fma's
// and the final round to nearest even.
struct QuantW {
    const uint32_t* q;        // [V][qld] words
    int64_t qld;
    const uint16_t* scales;   // [V][sld]
    const uint16_t* biases;   // [V][sld]
    int64_t sld;
    int32_t gshift;           // log2(group size)
};

struct HeadParams {
    const uint16_t* hidden;
    int64_t num_tokens, H, hld;
    const uint16_t* W;        // bf16 weights (unused with quantised weights)
    int64_t V, wld;
    QuantW qw;                // quantised weights (unused with bf16 weights)
    const int32_t* cu;
    int32_t num_decode;
    const int32_t* ex;
    int32_t row0, R;
    void* out;
    int64_t old;
    int32_t scale_mode;       // 0 none, 1 multiply by scale, 2 divide by scale
    float scale;
    // reduction partials from the tiled epilogue (nullptr: none): per logits
    // row and 64-logit block, the block's (max, sum of exp(x - max)) at
    // part[row * nb + b] and its key at bkeys[row * kld + b]
    float2* part;
    uint32_t* bkeys;
    int32_t nb, kld;
};

// Head output scaling on the fp32 accumulator, before any output rounding
// (vllm-metal release, Summary: heads that scale their logits outside the
// projection). The division is IEEE fp32 division, correctly rounded.
__device__ inline float scale_logit(float v, int32_t mode, float s) {
    return mode == 1 ? v * s : (mode == 2 ? v / s : v);
}

// ---------------------------------------------------------------------------
// Quantised-weight k order. One 16-byte run of codes (QB = 512/BITS hidden
// elements: 128 for 4-bit, 64 for 8-bit) feeds SPB = QB/32 MFMA k-steps: in
// step s of a run, lane quarter j (lanes 16j..16j+15) takes the 8 elements
// starting at QB/4*j + 8*s, so each lane's codes for the whole run are one
// contiguous 16-byte word group and every lane quarter stays inside one
// quantisation group (group sizes 32..128). Both quantised kernels use this
// order for the hidden operand too, so a row's logits are bitwise the same in
// both; the sum over k is the same as the bf16 kernels' with the hidden
// elements permuted accordingly.
// ---------------------------------------------------------------------------
template <int BITS>
struct QOrder {
    static constexpr int QB = 512 / BITS;   // hidden elements per 16-byte code run
    static constexpr int SPB = QB / 32;     // MFMA k-steps per run
    static constexpr int QQ = QB / 4;       // elements per lane quarter per run
};

// Tile order of the tiled heads. The hardware places workgroup i on XCD
// i % 8, and each XCD gets a contiguous run of the logical tile order. The
// order takes the row tiles in bands of LMH_TILE_MBAND (the vocabulary
// tiles of one band in turn, the band's row tiles fastest), so an XCD's
// concurrent tiles share a few hidden-row tiles, which stay in its L2, and
// each W slab is read by the band's row tiles together.
#ifndef LMH_TILE_MBAND
#define LMH_TILE_MBAND 4
#endif
__device__ inline void tile_of(int32_t logical, int32_t mtiles, int32_t ntiles, int32_t& mt, int32_t& nt) {
    constexpr int32_t MB = LMH_TILE_MBAND;
    const int32_t band_tiles = MB * ntiles;
    const int32_t b = logical / band_tiles;
    const int32_t rem = logical - b * band_tiles;
    const int32_t mb = mtiles - b * MB < MB ? mtiles - b * MB : MB;   // row tiles of this band
    nt = rem / mb;
    mt = b * MB + (rem - nt * mb);
}

__device__ inline uint32_t pack_bf16x2(float lo, float hi) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    // v_cvt_pk_bf16_f32: round to nearest even
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, bf16x2));
}

// 8 consecutive weights of a row from their codes (4-bit: the 8 nibbles of
// w0; 8-bit: the bytes of w0 then w1), as an MFMA operand: dword j holds
// elements 2j (low half) and 2j+1.
template <int BITS>
__device__ inline u32x4 dequant8(uint32_t w0, uint32_t w1, float s, float b) {
    u32x4 r;
    if constexpr (BITS == 4) {
        // opaque masks keep the byte structure visible to the selector, so
        // each code converts with one v_cvt_f32_ubyteN
        uint32_t lo, hi;
        asm("v_and_b32 %0, 0x0f0f0f0f, %1" : "=v"(lo) : "v"(w0));
        asm("v_and_b32 %0, 0x0f0f0f0f, %1" : "=v"(hi) : "v"(w0 >> 4));
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float e0 = (float)((lo >> (8 * j)) & 0xFFu);
            const float e1 = (float)((hi >> (8 * j)) & 0xFFu);
            r[j] = pack_bf16x2(fmaf(e0, s, b), fmaf(e1, s, b));
        }
    } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t w = j < 2 ? w0 : w1;
            const float e0 = (float)((w >> (16 * (j & 1))) & 0xFFu);
            const float e1 = (float)((w >> (16 * (j & 1) + 8)) & 0xFFu);
            r[j] = pack_bf16x2(fmaf(e0, s, b), fmaf(e1, s, b));
        }
    }
    return r;
}

// Buffer resource over `bytes` bytes at `base` (raw, stride 0): stores at
// offsets at or past `bytes` are dropped by the hardware.
__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(base, (short)0, (int)bytes, 0x00020000);
}

HeadParams to_params(const HeadArgs& a) {
    HeadParams p;
    p.hidden = static_cast<const uint16_t*>(a.hidden);
    p.num_tokens = a.num_tokens;
    p.H = a.hidden_dim;
    p.hld = a.hidden_ld;
    p.W = static_cast<const uint16_t*>(a.weight);
    p.V = a.vocab;
    p.wld = a.weight_ld;
    p.cu = a.cu;
    p.num_decode = a.num_decode;
    p.ex = a.ex;
    p.row0 = a.row0;
    p.R = a.rows;
    p.out = a.out;
    p.old = a.out_ld;
    p.scale_mode = a.scale_mode;
    p.scale = a.scale;
    p.qw.q = a.q;
    p.qw.qld = a.q_ld;
    p.qw.scales = a.scales;
    p.qw.biases = a.biases;
    p.qw.sld = a.s_ld;
    p.qw.gshift = a.gshift;
    p.part = a.part;
    p.bkeys = a.bkeys;
    p.nb = a.part_nb;
    p.kld = a.keys_ld;
    return p;
}

}  // namespace
}  // namespace lmh
