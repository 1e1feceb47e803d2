// Chunk-level MFMA helpers shared by the scan backward and the Mamba2 (SSD)
// scan (gfx950): fp32 16x16x4 products, split-bf16 16x16x32 / 16x16x16
// products, 16-lane reductions and the per-lane gate values of a 16-token
// chunk.
//
// Accumulator layout: lane l = 16 h + i (h = l / 16) holds rows 4h + r,
// column i of a 16x16 tile.  A 16-deep fp32 contraction is four
// v_mfma_f32_16x16x4_f32; in step s lane l supplies contraction index 4h + s,
// so an accumulator tile is the B operand of a product that contracts its
// rows, and the accumulator tile of X^T is the A operand of X times a matrix.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace tg {
namespace chunk {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

constexpr int L = 16;  // chunk length (tokens)
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ f32x4 mfma(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
// c + A B over a 16-deep contraction: a[s] = A[i][4h + s], b[s] = B[4h + s][i].
__device__ __forceinline__ f32x4 mm(const f32x4 a, const f32x4 b, f32x4 c) {
  c = mfma(a[0], b[0], c);
  c = mfma(a[1], b[1], c);
  c = mfma(a[2], b[2], c);
  return mfma(a[3], b[3], c);
}
__device__ __forceinline__ f32x4 z4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }
__device__ __forceinline__ f32x4 ld4(const float* p) { return *reinterpret_cast<const f32x4*>(p); }
__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

// ---- split-bf16 products (bf16 inputs) ------------------------------------------
// An fp32 operand x is carried as hi + lo bf16 (x - hi - lo within 2^-18 |x|);
// q, k and dO are exact in bf16.  A product of an exact operand with a split
// one takes two MFMAs (hi, lo); of two split ones three (lo x lo dropped).
// 16x16x32 operands: lane l supplies contraction indices kmap(h, e) =
// e < 4 ? 4h + e : 16 + 4h + (e - 4), the same permutation on both sides, so
// two accumulator row tiles (rows 4h + r and 16 + 4h + r) form one B operand.

// Two floats -> two bf16 (round to nearest even), `a` in the low half.
__device__ __forceinline__ uint32_t pk2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}
__device__ __forceinline__ float lo_f(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_f(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ uint2 pack4(const f32x4 x) { return make_uint2(pk2(x[0], x[1]), pk2(x[2], x[3])); }
__device__ __forceinline__ void split4(const f32x4 x, uint2& hi, uint2& lo) {
  const uint32_t h0 = pk2(x[0], x[1]), h1 = pk2(x[2], x[3]);
  hi = make_uint2(h0, h1);
  lo = make_uint2(pk2(x[0] - lo_f(h0), x[1] - hi_f(h0)), pk2(x[2] - lo_f(h1), x[3] - hi_f(h1)));
}
__device__ __forceinline__ uint4 cat(const uint2 a, const uint2 b) { return make_uint4(a.x, a.y, b.x, b.y); }
// hi and lo of the 8 values (x0 = kmap entries 0..3, x1 = entries 4..7).
__device__ __forceinline__ void split8(const f32x4 x0, const f32x4 x1, uint4& hi, uint4& lo) {
  uint2 h0, l0, h1, l1;
  split4(x0, h0, l0);
  split4(x1, h1, l1);
  hi = cat(h0, h1);
  lo = cat(l0, l1);
}
__device__ __forceinline__ f32x4 mma32(const uint4 a, const uint4 b, const f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma16b(const uint2 a, const uint2 b, const f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a), __builtin_bit_cast(s16x4, b), c,
                                                   0, 0, 0);
}
// Exact (bf16-valued) A operand of a 32-deep contraction from an fp32 LDS row:
// p points at column 4h of the block.
__device__ __forceinline__ uint4 exact8(const float* p) { return cat(pack4(ld4(p)), pack4(ld4(p + 16))); }

// x = hi + lo as split4, with the exact residual x - float(hi) from a
// 16x16x16 MFMA: -I times the packed hi (exact products) added to x as the
// fp32 accumulator input.  The sum is exactly representable, so lo is bitwise
// split4's, and the vector ALU does only the two conversions.  x is one
// accumulator tile, which is also the B operand layout of hi; negI is the A
// operand of -I (neg_identity()).
__device__ __forceinline__ uint2 neg_identity(int h4, int i16) {
  const int j = i16 - 4 * h4;
  return make_uint2((j == 0 ? 0xBF80u : 0u) | (j == 1 ? 0xBF800000u : 0u),
                    (j == 2 ? 0xBF80u : 0u) | (j == 3 ? 0xBF800000u : 0u));
}
__device__ __forceinline__ void split4m(const f32x4 x, const uint2 negI, uint2& hi, uint2& lo) {
  hi = pack4(x);
  lo = pack4(mma16b(negI, hi, x));
}
__device__ __forceinline__ void split8m(const f32x4 x0, const f32x4 x1, const uint2 negI, uint4& hi, uint4& lo) {
  uint2 h0, l0, h1, l1;
  split4m(x0, negI, h0, l0);
  split4m(x1, negI, h1, l1);
  hi = cat(h0, h1);
  lo = cat(l0, l1);
}

// ---- bf16 tiles of 256-byte rows in LDS (d = 128) --------------------------------
// Rows in 4-row blocks of 1 KB (the 64 lanes x 16 bytes of one LDS DMA) at an
// 1088-byte stride, block b shifted by a further {0, 2, 1, 3}[b % 4] x 16
// bytes, and the 16-byte chunk c of row r at slot c ^ 4(r % 4): MFMA operand
// reads (two 8-byte pieces 32 bytes apart, 16 rows) and transposing reads
// (4 rows x 16 columns) then hit every LDS bank once per half-wave.
constexpr int kTileRow16 = 4352;  // bytes of 16 rows
__device__ __forceinline__ int tile_blk(int b) { return b * 1088 + 16 * ((0x3120 >> (4 * (b & 3))) & 3); }
__device__ __forceinline__ int tile_off(int row, int col) {
  return tile_blk(row >> 2) + (row & 3) * 256 + 16 * ((col >> 3) ^ (4 * (row & 3))) + 2 * (col & 7);
}
// The global 16-byte chunk that lane `ln` of a block DMA loads, so that it
// lands at its swizzled slot (row ln / 16 of the block, slot ln % 16).
__device__ __forceinline__ int tile_dma_chunk(int ln) { return (ln & 15) ^ (4 * (ln >> 4)); }

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) const u32x2 lds_cu2;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) void lds_void;
// 16x16x32 operand (A or B) of row `row` at byte offset o = tile_off(row,
// 32m + 4h): columns 32m + kmap(h, 0..7).  o2 is o + 32, passed as a
// separate register so that the two 8-byte reads are not fused into one
// ds_read2_b64 (several times slower on this part).
__device__ __forceinline__ uint4 tile_a8(const char* t, int o, int o2) {
  const u32x2 x = *(lds_cu2*)(t + o), y = *(lds_cu2*)(t + o2);
  return make_uint4(x[0], x[1], y[0], y[1]);
}
// Transposing read: lane i of 16-lane group h passes the address of (row0 +
// 4h + i / 4, col0 + 4 (i % 4)) and gets rows row0 + 4h + 0..3 of column
// col0 + i (4 bf16), i.e. the accumulator / 16x16x16 operand layout.
__device__ __forceinline__ uint2 tile_tr(const char* t, int o) {
  return __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(t + o)));
}
__device__ __forceinline__ f32x4 bf4(const uint2 w) {
  return f32x4{lo_f(w.x), hi_f(w.x), lo_f(w.y), hi_f(w.y)};
}
// Buffer descriptor over `bytes` bytes from `base` (raw, no stride).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, static_cast<int>(bytes), 0x00020000);
}

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}
// Sum over the 16 lanes of a row (lanes 16h .. 16h+15); every lane gets it.
__device__ __forceinline__ float row_sum16(float v) {
  v += dpp<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp<0x141>(v);  // row_half_mirror
  v += dpp<0x140>(v);  // row_mirror
  return v;
}

// Per-lane gate values of one chunk.
struct Gates {
  f32x4 gam, del, bet;  // gamma, delta, beta at rows 4h + r
  f32x4 Gm, Gmt;        // Gamma at (row, col) and at (col, row), zero where masked
  float gam_c, del_c, bet_c, gam_last;  // at column i, and gamma_last
};

__device__ __forceinline__ Gates make_gates(const float* g, const float* b, int h4, int i16) {
  // G = inclusive prefix sum of g over the chunk: a scan across the 16 lanes
  // of each row (lane i ends with G_i), then the lane's rows 4h + r and the
  // last token read from the lanes that hold them.  Row and column values
  // come from the same G, so Gamma_ii = 1 exactly.
  float G = g[i16];
  G += dpp<0x111>(G);  // row_shr:1
  G += dpp<0x112>(G);  // row_shr:2
  G += dpp<0x114>(G);  // row_shr:4
  G += dpp<0x118>(G);  // row_shr:8
  const int base = 16 * h4;
  const float glast = __shfl(G, base + 15, 64) * kLog2e, gc = G * kLog2e;
  Gates s;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int row = 4 * h4 + r;
    const float gr = __shfl(G, base + row, 64) * kLog2e;
    s.gam[r] = ex2(gr);
    s.del[r] = ex2(glast - gr);
    s.bet[r] = b[row];
    s.Gm[r] = row >= i16 ? ex2(gr - gc) : 0.f;
    s.Gmt[r] = i16 >= row ? ex2(gc - gr) : 0.f;
  }
  s.gam_c = ex2(gc);
  s.del_c = ex2(glast - gc);
  s.bet_c = b[i16];
  s.gam_last = ex2(glast);
  return s;
}

template <bool F32IN>
__device__ __forceinline__ f32x4 load4(const void* base, size_t idx) {
  if (F32IN) return ld4(static_cast<const float*>(base) + idx);
  const uint2 w = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(base) + idx);
  return f32x4{__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xffff0000u), __uint_as_float(w.y << 16),
               __uint_as_float(w.y & 0xffff0000u)};
}
template <bool F32IN>
__device__ __forceinline__ float load1(const void* base, size_t idx) {
  if (F32IN) return static_cast<const float*>(base)[idx];
  return __uint_as_float(uint32_t(static_cast<const uint16_t*>(base)[idx]) << 16);
}

}  // namespace chunk
}  // namespace tg
