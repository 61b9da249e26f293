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
// zero beyond column j, so step j touches columns 0..j only (steps 0 .. 14).
//
// Each step is one FMA per column with the broadcast as its DPP source
// (v_fmac_f32 with row_newbcast), written out because the compiler keeps the
// broadcast as a separate move.  One asm block per step: the leading s_nop 1
// gives the two wait states a DPP source needs after a VALU write of it, and
// inside a block every source was written at least two instructions earlier
// (in the previous block).  No memory is accessed.
#define PDN_FMAC_BCAST(J, D) "v_fmac_f32_dpp %" #D ", %" #D ", %[n] row_newbcast:" #J " row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
__device__ __forceinline__ void block_row_solve(float (&x)[16], const float (&ntr)[16]) {
    asm volatile("s_nop 1\n\t" PDN_FMAC_BCAST(0, 0) : "+v"(x[0]) : [n] "v"(ntr[0]));
    asm volatile("s_nop 1\n\t" PDN_FMAC_BCAST(1, 0) PDN_FMAC_BCAST(1, 1) : "+v"(x[0]), "+v"(x[1]) : [n] "v"(ntr[1]));
    asm volatile("s_nop 1\n\t" PDN_FMAC_BCAST(2, 0) PDN_FMAC_BCAST(2, 1) PDN_FMAC_BCAST(2, 2) : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]) : [n] "v"(ntr[2]));
    asm volatile("s_nop 1\n\t" PDN_FMAC_BCAST(3, 0) PDN_FMAC_BCAST(3, 1) PDN_FMAC_BCAST(3, 2) PDN_FMAC_BCAST(3, 3) : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3]) : [n] "v"(ntr[3]));
    asm volatile("s_nop 1\n\t" PDN_FMAC_BCAST(4, 0) PDN_FMAC_BCAST(4, 1) PDN_FMAC_BCAST(4, 2) PDN_FMAC_BCAST(4, 3) PDN_FMAC_BCAST(4, 4) : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3]), "+v"(x[4]) : [n] "v"(ntr[4]));
    asm volatile("s_nop 1\n\t" PDN_FMAC_BCAST(5, 0) PDN_FMAC_BCAST(5, 1) PDN_FMAC_BCAST(5, 2) PDN_FMAC_BCAST(5, 3) PDN_FMAC_BCAST(5, 4) PDN_FMAC_BCAST(5, 5) : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3]), "+v"(x[4]), "+v"(x[5]) : [n] "v"(ntr[5]));
    asm volatile("s_nop 1\n\t" PDN_FMAC_BCAST(6, 0) PDN_FMAC_BCAST(6, 1) PDN_FMAC_BCAST(6, 2) PDN_FMAC_BCAST(6, 3) PDN_FMAC_BCAST(6, 4) PDN_FMAC_BCAST(6, 5) PDN_FMAC_BCAST(6, 6) : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3]), "+v"(x[4]), "+v"(x[5]), "+v"(x[6]) : [n] "v"(ntr[6]));
    asm volatile("s_nop 1\n\t" PDN_FMAC_BCAST(7, 0) PDN_FMAC_BCAST(7, 1) PDN_FMAC_BCAST(7, 2) PDN_FMAC_BCAST(7, 3) PDN_FMAC_BCAST(7, 4) PDN_FMAC_BCAST(7, 5) PDN_FMAC_BCAST(7, 6) PDN_FMAC_BCAST(7, 7) : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3]), "+v"(x[4]), "+v"(x[5]), "+v"(x[6]), "+v"(x[7]) : [n] "v"(ntr[7]));
    asm volatile("s_nop 1\n\t" PDN_FMAC_BCAST(8, 0) PDN_FMAC_BCAST(8, 1) PDN_FMAC_BCAST(8, 2) PDN_FMAC_BCAST(8, 3) PDN_FMAC_BCAST(8, 4) PDN_FMAC_BCAST(8, 5) PDN_FMAC_BCAST(8, 6) PDN_FMAC_BCAST(8, 7) PDN_FMAC_BCAST(8, 8) : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3]), "+v"(x[4]), "+v"(x[5]), "+v"(x[6]), "+v"(x[7]), "+v"(x[8]) : [n] "v"(ntr[8]));
    asm volatile("s_nop 1\n\t" PDN_FMAC_BCAST(9, 0) PDN_FMAC_BCAST(9, 1) PDN_FMAC_BCAST(9, 2) PDN_FMAC_BCAST(9, 3) PDN_FMAC_BCAST(9, 4) PDN_FMAC_BCAST(9, 5) PDN_FMAC_BCAST(9, 6) PDN_FMAC_BCAST(9, 7) PDN_FMAC_BCAST(9, 8) PDN_FMAC_BCAST(9, 9) : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3]), "+v"(x[4]), "+v"(x[5]), "+v"(x[6]), "+v"(x[7]), "+v"(x[8]), "+v"(x[9]) : [n] "v"(ntr[9]));
    asm volatile("s_nop 1\n\t" PDN_FMAC_BCAST(10, 0) PDN_FMAC_BCAST(10, 1) PDN_FMAC_BCAST(10, 2) PDN_FMAC_BCAST(10, 3) PDN_FMAC_BCAST(10, 4) PDN_FMAC_BCAST(10, 5) PDN_FMAC_BCAST(10, 6) PDN_FMAC_BCAST(10, 7) PDN_FMAC_BCAST(10, 8) PDN_FMAC_BCAST(10, 9) PDN_FMAC_BCAST(10, 10) : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3]), "+v"(x[4]), "+v"(x[5]), "+v"(x[6]), "+v"(x[7]), "+v"(x[8]), "+v"(x[9]), "+v"(x[10]) : [n] "v"(ntr[10]));
    asm volatile("s_nop 1\n\t" PDN_FMAC_BCAST(11, 0) PDN_FMAC_BCAST(11, 1) PDN_FMAC_BCAST(11, 2) PDN_FMAC_BCAST(11, 3) PDN_FMAC_BCAST(11, 4) PDN_FMAC_BCAST(11, 5) PDN_FMAC_BCAST(11, 6) PDN_FMAC_BCAST(11, 7) PDN_FMAC_BCAST(11, 8) PDN_FMAC_BCAST(11, 9) PDN_FMAC_BCAST(11, 10) PDN_FMAC_BCAST(11, 11) : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3]), "+v"(x[4]), "+v"(x[5]), "+v"(x[6]), "+v"(x[7]), "+v"(x[8]), "+v"(x[9]), "+v"(x[10]), "+v"(x[11]) : [n] "v"(ntr[11]));
    asm volatile("s_nop 1\n\t" PDN_FMAC_BCAST(12, 0) PDN_FMAC_BCAST(12, 1) PDN_FMAC_BCAST(12, 2) PDN_FMAC_BCAST(12, 3) PDN_FMAC_BCAST(12, 4) PDN_FMAC_BCAST(12, 5) PDN_FMAC_BCAST(12, 6) PDN_FMAC_BCAST(12, 7) PDN_FMAC_BCAST(12, 8) PDN_FMAC_BCAST(12, 9) PDN_FMAC_BCAST(12, 10) PDN_FMAC_BCAST(12, 11) PDN_FMAC_BCAST(12, 12) : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3]), "+v"(x[4]), "+v"(x[5]), "+v"(x[6]), "+v"(x[7]), "+v"(x[8]), "+v"(x[9]), "+v"(x[10]), "+v"(x[11]), "+v"(x[12]) : [n] "v"(ntr[12]));
    asm volatile("s_nop 1\n\t" PDN_FMAC_BCAST(13, 0) PDN_FMAC_BCAST(13, 1) PDN_FMAC_BCAST(13, 2) PDN_FMAC_BCAST(13, 3) PDN_FMAC_BCAST(13, 4) PDN_FMAC_BCAST(13, 5) PDN_FMAC_BCAST(13, 6) PDN_FMAC_BCAST(13, 7) PDN_FMAC_BCAST(13, 8) PDN_FMAC_BCAST(13, 9) PDN_FMAC_BCAST(13, 10) PDN_FMAC_BCAST(13, 11) PDN_FMAC_BCAST(13, 12) PDN_FMAC_BCAST(13, 13) : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3]), "+v"(x[4]), "+v"(x[5]), "+v"(x[6]), "+v"(x[7]), "+v"(x[8]), "+v"(x[9]), "+v"(x[10]), "+v"(x[11]), "+v"(x[12]), "+v"(x[13]) : [n] "v"(ntr[13]));
    asm volatile("s_nop 1\n\t" PDN_FMAC_BCAST(14, 0) PDN_FMAC_BCAST(14, 1) PDN_FMAC_BCAST(14, 2) PDN_FMAC_BCAST(14, 3) PDN_FMAC_BCAST(14, 4) PDN_FMAC_BCAST(14, 5) PDN_FMAC_BCAST(14, 6) PDN_FMAC_BCAST(14, 7) PDN_FMAC_BCAST(14, 8) PDN_FMAC_BCAST(14, 9) PDN_FMAC_BCAST(14, 10) PDN_FMAC_BCAST(14, 11) PDN_FMAC_BCAST(14, 12) PDN_FMAC_BCAST(14, 13) PDN_FMAC_BCAST(14, 14) : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3]), "+v"(x[4]), "+v"(x[5]), "+v"(x[6]), "+v"(x[7]), "+v"(x[8]), "+v"(x[9]), "+v"(x[10]), "+v"(x[11]), "+v"(x[12]), "+v"(x[13]), "+v"(x[14]) : [n] "v"(ntr[14]));
}
#undef PDN_FMAC_BCAST

}  // namespace tile
}  // namespace pdn
