// Device helpers shared by the tiled bf16 prefill kernels (dk = 128): MFMA
// wrappers on hi/lo bf16 operands, DPP row primitives, and the LDS tile
// layouts that the state-carrying waves read.  Not a public header.
#pragma once
#include "common.h"

namespace pdn {
namespace tile {

constexpr int DK = 128;

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) uint16_t lds_u16;

// State rows.  The chain keeps S in 8 accumulator blocks; lane (ln, g) holds
// element e of block ib as state row (key channel) srow(ib, g, e) and value
// column ln of its 16.  Pairing blocks 2t and 2t + 1 as one 16x16x32 B operand
// then gives lane g the contiguous channels 32t + 8g .. 32t + 8g + 7, the same
// channels a 16-byte read of a key or query row hands to the A operand.
__device__ __forceinline__ int srow(int ib, int g, int e) { return 32 * (ib >> 1) + 8 * g + 4 * (ib & 1) + e; }

// Key/query tiles: element (token r, channel pc) of a row-major bf16 tile
// with 128 channels per row.
// 16-byte chunks are XORed with f(r) = 4 (r % 4) + (r / 4) % 4, which makes
// both the 16-row MFMA operand reads and the 4x4 transpose reads hit 16
// distinct 16-byte bank groups.
__device__ __forceinline__ int kq_off(int r, int pc) {
    const int f = ((r & 3) << 2) | ((r >> 2) & 3);
    return r * DK + ((((pc >> 3) ^ f) << 3) | (pc & 7));
}

typedef bf16 bf16x2 __attribute__((ext_vector_type(2)));

// hi/lo bf16 split of two values, as packed words: hi = RNE(x), lo = RNE(x - hi).
// One packed conversion gives both hi halves; they are widened back with a
// shift and a mask, so the split costs three operations per value.
__device__ __forceinline__ void split2(float a, float b, uint32_t& hi, uint32_t& lo) {
    hi = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
    const float ah = __builtin_bit_cast(float, hi << 16);
    const float bh = __builtin_bit_cast(float, hi & 0xffff0000u);
    lo = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a - ah, b - bh}, bf16x2));
}

__device__ __forceinline__ f32x4 mfma32(const bf16x8& a, const bf16x8& b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// acc += (hi, lo) * (hi, lo), dropping lo*lo
__device__ __forceinline__ f32x4 mm22(const bf16x8 (&a)[2], const bf16x8 (&b)[2], f32x4 c) {
    c = mfma32(a[1], b[0], c);
    c = mfma32(a[0], b[1], c);
    return mfma32(a[0], b[0], c);
}

// hi/lo split of two accumulator blocks stacked as one 16x16x32 operand
// (elements lo4[0..3], hi4[0..3])
__device__ __forceinline__ void split_pair(const f32x4& lo4, const f32x4& hi4, bf16x8 (&o)[2]) {
    uint4 h, l;
    split2(lo4[0], lo4[1], h.x, l.x);
    split2(lo4[2], lo4[3], h.y, l.y);
    split2(hi4[0], hi4[1], h.z, l.z);
    split2(hi4[2], hi4[3], h.w, l.w);
    o[0] = __builtin_bit_cast(bf16x8, h);
    o[1] = __builtin_bit_cast(bf16x8, l);
}

__device__ __forceinline__ bf16x8 as_bf16x8(const uint4& u) { return __builtin_bit_cast(bf16x8, u); }

// x as held by lane src (0..63) of this wave (a lane permute through the LDS
// crossbar; no LDS memory is read)
__device__ __forceinline__ float lane_get(float x, int src) {
    return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(src << 2, __builtin_bit_cast(int, x)));
}

// Hardware exp2 / sqrt (about 1 ulp).  Decay exponents here are <= 0, so
// exp2 only ever underflows towards 0.
__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float sqrt_hw(float x) { return __builtin_amdgcn_sqrtf(x); }

__device__ __forceinline__ f32x4 mfma16(const bf16x4& a, const bf16x4& b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}
// acc += (hi, lo) * (hi, lo) on 16x16x16 operands, dropping lo*lo
__device__ __forceinline__ f32x4 mm22x16(const bf16x4 (&a)[2], const bf16x4 (&b)[2], f32x4 c) {
    c = mfma16(a[1], b[0], c);
    c = mfma16(a[0], b[1], c);
    return mfma16(a[0], b[0], c);
}
// hi/lo split of an accumulator block used as a 16x16x16 B operand
__device__ __forceinline__ void split_d(const f32x4& v, bf16x4 (&o)[2]) {
    uint2 h, l;
    split2(v[0], v[1], h.x, l.x);
    split2(v[2], v[3], h.y, l.y);
    o[0] = __builtin_bit_cast(bf16x4, h);
    o[1] = __builtin_bit_cast(bf16x4, l);
}
// two 16x16x16 B operands stacked along k into one 16x16x32 B operand
__device__ __forceinline__ bf16x8 cat4(const bf16x4& a, const bf16x4& b) {
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

// DPP move of x from the lane given by `ctrl`; lanes with no source or
// outside `row_mask` read 0.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp0(float x) {
    return __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, ROW_MASK, 0xf, false));
}

// Inclusive prefix sum over the 64 lanes: shifts within 16-lane rows, then
// the row totals carried across rows (row_bcast:15 / row_bcast:31).
__device__ __forceinline__ float wave_incl_scan(float x) {
    x += dpp0<0x111, 0xf>(x);  // row_shr:1
    x += dpp0<0x112, 0xf>(x);  // row_shr:2
    x += dpp0<0x114, 0xf>(x);  // row_shr:4
    x += dpp0<0x118, 0xf>(x);  // row_shr:8
    x += dpp0<0x142, 0xa>(x);  // row_bcast:15 into rows 1 and 3
    x += dpp0<0x143, 0xc>(x);  // row_bcast:31 into rows 2 and 3
    return x;
}

// Inclusive prefix sum inside each 16-lane DPP row.
__device__ __forceinline__ float row_incl_scan(float x) {
    x += dpp0<0x111, 0xf>(x);  // row_shr:1
    x += dpp0<0x112, 0xf>(x);  // row_shr:2
    x += dpp0<0x114, 0xf>(x);  // row_shr:4
    x += dpp0<0x118, 0xf>(x);  // row_shr:8
    return x;
}

// Broadcast of lane J of each 16-lane row to the whole row (DPP row_newbcast).
template <int J>
__device__ __forceinline__ float row_bcast(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x150 + J, 0xf, 0xf, true));
}
// Inverse of a unit lower-triangular 16x16 block I + L, one row per lane of a
// 16-lane DPP row.  Lane r starts with x = e_r and ntr = -(row r of L); step j
// broadcasts the finished row j across the block and every row r takes
// x_r += ntr_j x_j.  Rows r <= j have L_rj = 0 and stay unchanged, and x_j is
// zero beyond column j, so step j touches columns 0..j only.  Steps J .. 14:
template <int J>
__device__ __forceinline__ void block_row_solve(float (&x)[16], const float (&ntr)[16]) {
    if constexpr (J < 15) {
#pragma unroll
        for (int c = 0; c <= J; ++c) x[c] = fmaf(row_bcast<J>(x[c]), ntr[J], x[c]);
        block_row_solve<J + 1>(x, ntr);
    }
}
__device__ __forceinline__ void block_row_solve(float (&x)[16], const float (&ntr)[16]) { block_row_solve<0>(x, ntr); }

}  // namespace tile
}  // namespace pdn
