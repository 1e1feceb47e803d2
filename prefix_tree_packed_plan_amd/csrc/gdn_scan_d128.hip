// Chunked tree Gated DeltaNet forward for bf16, d_k = d_v = 128, on gfx950.
//
// Method ("Tree Training", arXiv 2511.00413, section 3.2 Eq. 10 and the
// chunked form of appendix A.2), per 64-token chunk of one segment and one
// value head, with G the in-chunk prefix of g, gamma = exp(G), b = beta:
//     A_ij = b_i exp(G_i - G_j) k_i.k_j  (j < i),   T = (I + A)^-1,
//     R = diag(b) V - diag(b gamma) K S0,   U = T R,
//     O = scale (diag(gamma) Q S0 + P U),   P_ij = exp(G_i - G_j) q_i.k_j  (j <= i),
//     S1 = gamma_L S0 + (diag(exp(G_L - G)) K)^T U.
// A segment starts from its parent's final state (zero at a root), which the
// host hands over level by level.
//
// Work-group = one (segment, value head), 8 waves; wave w owns value columns
// [16w, 16w + 16) and keeps that 128 x 16 slice of the fp32 state in MFMA
// accumulator registers for the whole segment.  Per chunk:
//
//   prep (no state needed)   every wave: its own copy of the gate prefix
//                            (DPP scan).  Waves 0 and 1: the three K K^T
//                            tiles of one 32-token half, the two 16 x 16
//                            diagonal inverses (fp32 forward substitution)
//                            and the off-diagonal block -T_bb A_ba T_aa, i.e.
//                            the 32 x 32 inverse of that half.  Waves 2..7:
//                            the K K^T tiles coupling the halves and the
//                            Q K^T tiles.  All land in LDS as ready-made MFMA
//                            operands, split hi + lo where they feed the state.
//   state, part 1            R = diag(b)(V - gamma K S0) and O^T = S0^T Q^T
//                            (overlaps the prep of waves 0 and 1).
//   ---- barrier ----
//   state, part 2            two-level solve: U_top = T_top R_top,
//                            R_bot -= A_bt U_top, U_bot = T_bot R_bot; then
//                            O^T += U^T P^T and S = gamma_L S + K^T W.
//
// Every product runs on v_mfma_f32_16x16x32_bf16 except the two 16 x 16 x 16
// steps of the off-diagonal inverse block.  Products that feed the state carry
// their fp32 operand as hi + lo bf16 (relative 2^-17; lo x lo dropped); the
// output path uses hi only.  The output is produced transposed, so a lane
// holds 4 consecutive value columns of one token and stores 8 bytes.
//
// Data movement: q, k, v, g and beta of chunk n + 1 are DMA'd from HBM into
// LDS (global_load_lds, 16 bytes per lane, no staging registers) at the start
// of chunk n, into the other half of double buffers, so the loads have a
// whole chunk to land.  The output of chunk n is staged in LDS and leaves as
// whole 256-byte token rows during chunk n + 1.  Both go through buffer descriptors, so
// per-lane offsets are loop constants and masked output rows are dropped by
// the descriptor's range check.
//
// Tile layout in LDS (see toff): rows in 4-row blocks of 1 KB (one DMA
// instruction each) at a 1088-byte stride, block b shifted by a further
// {0, 2, 1, 3}[b % 4] x 16 bytes, and the 16-byte chunk c of row r stored at
// slot c ^ 4(r % 4).  With it the two read patterns used here -- MFMA operand
// reads (two 8-byte pieces 32 bytes apart, one ds_read2_b64) of 16 rows and
// the transposing read ds_read_b64_tr_b16 of 4 rows x 16 columns -- hit every
// LDS bank once per half-wave.
#include <hip/hip_runtime.h>

#include "../../include/tree_gdn.h"
#include "launch.hpp"

namespace tg {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) void lds_void;

constexpr int CH = 64;   // chunk length (tokens)
constexpr int D = 128;   // d_k = d_v
constexpr int NW = 8;    // waves per work-group
constexpr int TSZ = 17408;      // LDS bytes of one 64 x 128 bf16 tile (see toff)
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ uint32_t pk2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}
__device__ __forceinline__ float lo_f(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_f(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
// x = hi + lo with hi, lo bf16 (4 values -> 2 packed words each).
__device__ __forceinline__ void split4(const f32x4 x, uint2& hi, uint2& lo) {
  const uint32_t h0 = pk2(x[0], x[1]), h1 = pk2(x[2], x[3]);
  hi = make_uint2(h0, h1);
  lo = make_uint2(pk2(x[0] - lo_f(h0), x[1] - hi_f(h0)), pk2(x[2] - lo_f(h1), x[3] - hi_f(h1)));
}
// Two accumulator tiles (rows 16c.. and 16c+16..) as one K = 32 operand.
__device__ __forceinline__ void split8(const f32x4 x0, const f32x4 x1, uint4& hi, uint4& lo) {
  uint2 h0, l0, h1, l1;
  split4(x0, h0, l0);
  split4(x1, h1, l1);
  hi = make_uint4(h0.x, h0.y, h1.x, h1.y);
  lo = make_uint4(l0.x, l0.y, l1.x, l1.y);
}
__device__ __forceinline__ f32x4 mma32(const uint4 a, const uint4 b, const f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma16(const uint2 a, const uint2 b, const f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a), __builtin_bit_cast(s16x4, b), c,
                                                   0, 0, 0);
}
// hi x hi + hi x lo + lo x hi.
__device__ __forceinline__ f32x4 mma32x3(const uint4 ah, const uint4 al, const uint4 bh, const uint4 bl, f32x4 c) {
  c = mma32(ah, bh, c);
  c = mma32(ah, bl, c);
  return mma32(al, bh, c);
}
__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }
__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float dpp_shr(float x, int n) {
  switch (n) {
    case 1: return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x111, 0xF, 0xF, true));
    case 2: return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x112, 0xF, 0xF, true));
    case 4: return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x114, 0xF, 0xF, true));
    default: return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x118, 0xF, 0xF, true));
  }
}
// Sum over the 4 lanes of a quad (lanes 4k..4k+3), result in all four.
__device__ __forceinline__ float quad_sum(float x) {
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, true));  // [1,0,3,2]
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, true));  // [2,3,0,1]
  return x;
}

// ---- 64 x 128 bf16 tiles in LDS ------------------------------------------------
// Byte offset of the 4-row block b, and of element (row, col).
__device__ __forceinline__ int blk_off(int b) { return b * 1088 + 16 * ((0x3120 >> (4 * (b & 3))) & 3); }
__device__ __forceinline__ int toff(int row, int col) {
  return blk_off(row >> 2) + (row & 3) * 256 + 16 * ((col >> 3) ^ (4 * (row & 3))) + 2 * (col & 7);
}
// Rows 16 apart are 4352 bytes apart (the block shifts repeat every 4 blocks).
constexpr int ROW16 = 4352;
// A operand of a 16x16x32 MFMA (or the B operand, the roles are symmetric)
// at byte offset `o` = toff(row, col0 + 4h): row `row`, columns
// col0 + kmap(h, 0..7), kmap(h, j) = j<4 ? 4h+j : 16+4h+(j-4); the two 8-byte
// pieces are 32 bytes apart in this layout.  The same K order lets two
// accumulator tiles (rows 4h..4h+3 of each) serve as one K = 32 operand
// without moving data.
__device__ __forceinline__ uint4 ld_a8(const char* t, int o) {
  const uint2* p = reinterpret_cast<const uint2*>(t + o);
  const uint2 x = p[0], y = p[4];
  return make_uint4(x.x, x.y, y.x, y.y);
}
// Transposing read at byte offset `o` = toff(row0 + 4h + i/4, col0 + 4(i%4))
// for lane i of 16-lane group h: the lane gets rows row0 + 4h + 0..3 of
// column col0 + i.
__device__ __forceinline__ uint2 ld_tr(const char* t, int o) {
  return __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(t + o)));
}
__device__ __forceinline__ f32x4 bf4(const uint2 x) { return f32x4{lo_f(x.x), hi_f(x.x), lo_f(x.y), hi_f(x.y)}; }

// 16x16 fp32 blocks, row-major, 4-float groups permuted by row / 4.
__device__ __forceinline__ int aoff(int r, int c) { return r * 16 + 4 * ((c >> 2) ^ ((r >> 2) & 3)) + (c & 3); }

struct Smem {
  alignas(16) char kb[2][TSZ];       // K tiles
  alignas(16) char qb[2][TSZ];       // Q tiles
  alignas(16) char vb[2][TSZ];       // V tiles
  // A operands, per lane, hi and lo: 0..3 = row block b of the two 32 x 32
  // inverses (b = 0, 1: T_top; b = 2, 3: T_bot); 4, 5 = -A rows 32..47 and
  // 48..63, columns 0..31.
  alignas(16) uint4 ttab[6][2][64];
  // B operands of O^T += U^T P^T: (j-half p, row block b) = (0,0) (0,1) (0,2) (1,2) (0,3) (1,3).
  alignas(16) uint4 ptab[6][64];
  alignas(16) float abb[2][2][256];  // waves 0, 1: gated diagonal K K^T blocks
  alignas(16) float tbb[2][2][256];  // waves 0, 1: (I + A_bb)^-1
  alignas(16) float gt[NW][4][CH];   // per wave: G log2(e), exp(G), beta, exp(G_L - G)
  alignas(16) float graw[2][CH];
  alignas(16) float braw[2][CH];
  // Output rows of the previous chunk, 256 bytes per token, 16-byte chunk c
  // of row r at slot c ^ (r % 16).
  alignas(16) char ost[CH * D * 2];
};

// Buffer descriptor over `bytes` bytes from `base` (raw, no stride).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, static_cast<int>(bytes), 0x00020000);
}
// DMA of the 4-row blocks first, first + step, ... of a 64 x 128 bf16 tile:
// lane l loads the 16-byte chunk (l % 16) ^ 4(l / 16) of row 4b + l / 16,
// which the layout puts at LDS byte 16 l of the block.  `voff` is that
// lane's byte offset for b = 0; `rstride` the bytes between rows.
__device__ __forceinline__ void dma_tile(__amdgpu_buffer_rsrc_t r, int voff, int rstride, char* tile, int first,
                                         int step) {
  for (int b = first; b < 16; b += step)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)(tile + blk_off(b)), 16, voff, 4 * b * rstride, 0, 0);
}
// Same for a partial chunk of Ln rows: rows past the end repeat row Ln - 1.
__device__ __forceinline__ void dma_tile_tail(__amdgpu_buffer_rsrc_t r, int coff, int rstride, int Ln, char* tile,
                                              int first, int step, int lane) {
  for (int b = first; b < 16; b += step)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)(tile + blk_off(b)), 16,
                                             min(4 * b + (lane >> 4), Ln - 1) * rstride + coff, 0, 0, 0);
}

// Raw 16 x 16 Gram tile D[x][y] = X[16xb + x] . Y[16yb + y] over 128
// features: lane (y = i, h) holds x = 4h + 0..3.  ao[kk] = toff(i, 32kk + 4h).
__device__ __forceinline__ f32x4 gram(const char* X, int xb, const char* Y, int yb, const int* ao) {
  uint4 a[4], b[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    a[kk] = ld_a8(X + ROW16 * xb, ao[kk]);
    b[kk] = ld_a8(Y + ROW16 * yb, ao[kk]);
  }
  f32x4 acc = zero4();
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) acc = mma32(a[kk], b[kk], acc);
  return acc;
}

// Gram tiles of waves 2..7: kind (0: -A block, 1: P^T block), key block jb,
// query/row block ib.  Waves 4 and 5 share SIMDs with waves 0 and 1 and get
// one tile each, the others three.
__device__ __forceinline__ int tile_code(int idx) {
  // (kind << 4) | (jb << 2) | ib
  constexpr int codes[14] = {(0 << 4) | (0 << 2) | 2, (0 << 4) | (1 << 2) | 2, (0 << 4) | (0 << 2) | 3,
                             (0 << 4) | (1 << 2) | 3, (1 << 4) | (0 << 2) | 0, (1 << 4) | (0 << 2) | 1,
                             (1 << 4) | (1 << 2) | 1, (1 << 4) | (0 << 2) | 2, (1 << 4) | (1 << 2) | 2,
                             (1 << 4) | (2 << 2) | 2, (1 << 4) | (0 << 2) | 3, (1 << 4) | (1 << 2) | 3,
                             (1 << 4) | (2 << 2) | 3, (1 << 4) | (3 << 2) | 3};
  return codes[idx];
}

__global__ __launch_bounds__(64 * NW) void gdn_d128_kernel(ScanArgs args) {
  __shared__ Smem sm;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int cw = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h4 = lane >> 4;
  const int i16 = lane & 15;

  // Block -> (item, value head).  When value heads come in pairs per q/k head
  // and h_v is a multiple of 16, the pair lands on blocks b and b + 8, which
  // the dispatcher places on the same XCD, so the second read of their q and
  // k tiles is served by that XCD's L2.
  int item, h;
  {
    const int b = blockIdx.x;
    item = b / args.h_v;
    const int r = b - item * args.h_v;
    if (args.h_v == 2 * args.h_qk && args.h_v % 16 == 0) {
      const int p = r & 15;
      h = 2 * ((r >> 4) * 8 + (p & 7)) + (p >> 3);
    } else {
      h = r;
    }
  }
  const int hq = h / (args.h_v / args.h_qk);
  const int seg = args.items[item];
  const int seg_beg = args.seg_off[seg];
  const int seg_end = args.seg_off[seg + 1];
  const int par = args.parent[seg];
  const uint16_t* qg = static_cast<const uint16_t*>(args.q);
  const uint16_t* kg = static_cast<const uint16_t*>(args.k);
  const uint16_t* vg = static_cast<const uint16_t*>(args.v);
  uint16_t* og = static_cast<uint16_t*>(args.o);
  const int col_w = 16 * cw;
  float* gtw = &sm.gt[cw][0][0];  // this wave's gate tables

  // Loop-constant byte offsets: operand reads of rows i16 (+16 per row
  // block) at columns 32kk + 4h4; transposing reads of K at columns 32m (+16
  // is +32 bytes) and of V at this wave's columns; DMA and output lanes.
  int ao[4], ko[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    ao[kk] = toff(i16, 32 * kk + 4 * h4);
    ko[kk] = toff(4 * h4 + (i16 >> 2), 32 * kk + 4 * (i16 & 3));
  }
  const int vo = toff(4 * h4 + (i16 >> 2), col_w + 4 * (i16 & 3));
  const int rs_qk = args.h_qk * D * 2, rs_v = args.h_v * D * 2;  // bytes between token rows
  const int cofs = 16 * ((lane & 15) ^ (4 * (lane >> 4)));        // this lane's 16-byte chunk of a row
  const int voff_qk = (lane >> 4) * rs_qk + cofs, voff_v = (lane >> 4) * rs_v + cofs;
  // Output staging: this lane writes token 16b + i16, value columns
  // col_w + 4h4..+3 (8 bytes); it later stores 16-byte chunk lane % 16 of
  // token rows 8cw + lane / 16 (+4).
  const int sto_w = i16 * 256 + 16 * ((2 * cw + (h4 >> 1)) ^ i16) + 8 * (h4 & 1);
  int sto_r[2];
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int row = 8 * cw + (lane >> 4) + 4 * k;
    sto_r[k] = row * 256 + 16 * ((lane & 15) ^ (row & 15));
  }
  const int ooff = (8 * cw + (lane >> 4)) * rs_v + 16 * (lane & 15);

  // ---- initial state: S[mt] rows 16mt + 4h4 + 0..3, column col_w + i16 --------
  const size_t head_elems = static_cast<size_t>(D) * D;
  f32x4 S[8];
  {
    const float* src = nullptr;
    if (par >= 0)
      src = args.states ? args.states + (static_cast<size_t>(par) * args.h_v + h) * head_elems
                        : args.slots + (static_cast<size_t>(args.slot[par]) * args.h_v + h) * head_elems;
    if (src) {
#pragma unroll
      for (int mt = 0; mt < 8; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) S[mt][r] = src[(16 * mt + 4 * h4 + r) * D + col_w + i16];
    } else {
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) S[mt] = zero4();
    }
  }

  // Chunk at token tc into buffer buf: 48 tile blocks and two gate rows.
  auto fetch = [&](int tc, int buf) {
    const int Ln = min(CH, seg_end - tc);
    const auto rk = rsrc(kg + (static_cast<size_t>(tc) * args.h_qk + hq) * D, CH * rs_qk);
    const auto rq = rsrc(qg + (static_cast<size_t>(tc) * args.h_qk + hq) * D, CH * rs_qk);
    const auto rv = rsrc(vg + (static_cast<size_t>(tc) * args.h_v + h) * D, CH * rs_v);
    if (Ln == CH) {
      dma_tile(rk, voff_qk, rs_qk, sm.kb[buf], cw, NW);
      dma_tile(rq, voff_qk, rs_qk, sm.qb[buf], cw, NW);
      dma_tile(rv, voff_v, rs_v, sm.vb[buf], cw, NW);
    } else {
      dma_tile_tail(rk, cofs, rs_qk, Ln, sm.kb[buf], cw, NW, lane);
      dma_tile_tail(rq, cofs, rs_qk, Ln, sm.qb[buf], cw, NW, lane);
      dma_tile_tail(rv, cofs, rs_v, Ln, sm.vb[buf], cw, NW, lane);
    }
    if (cw >= NW - 2) {
      const float* src = (cw == NW - 1 ? args.beta : args.g) + static_cast<size_t>(tc) * args.h_v + h;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc(src, CH * args.h_v * 4),
                                               (lds_void*)(cw == NW - 1 ? sm.braw[buf] : sm.graw[buf]), 4,
                                               min(lane, Ln - 1) * args.h_v * 4, 0, 0, 0);
    }
  };

  // Output of the previous chunk (transposed tiles packed to bf16): token
  // 16b + i16, value columns col_w + 4h4 + 0..3.
  // Whole token rows of the staged output; the descriptor ends after row
  // Ln - 1, so rows past it are not written.
  auto store_out = [&](int tc, int Ln) {
    const auto ro = rsrc(og + (static_cast<size_t>(tc) * args.h_v + h) * D, (Ln - 1) * rs_v + D * 2);
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(sm.ost + sto_r[k]);
      __builtin_amdgcn_raw_buffer_store_b128(v, ro, ooff + 4 * k * rs_v, 0, 0);
    }
  };

  fetch(seg_beg, 0);
  int s = 0;
  int prev_t0 = -1, prev_L = 0;

  for (int t0 = seg_beg; t0 < seg_end; t0 += CH, s ^= 1) {
    const int Lc = min(CH, seg_end - t0);
    const char* Ks = sm.kb[s];
    const char* Qs = sm.qb[s];
    const char* Vs = sm.vb[s];

    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's DMA of the chunk has landed
    __syncthreads();                                   // (A) ... and every other wave's
    if (t0 + CH < seg_end) fetch(t0 + CH, s ^ 1);

    // -- gates, per wave: inclusive prefix of g within rows of 16 lanes (DPP),
    //    then across rows
    {
      float x = lane < Lc ? sm.graw[s][lane] : 0.f;
      x += dpp_shr(x, 1);
      x += dpp_shr(x, 2);
      x += dpp_shr(x, 4);
      x += dpp_shr(x, 8);
      const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 15));
      const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 31));
      const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 47));
      const int row = lane >> 4;
      x += (row >= 1 ? r0 : 0.f) + (row >= 2 ? r1 : 0.f) + (row >= 3 ? r2 : 0.f);
      const float g2 = x * kLog2e;
      const float g2L = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(g2), 63));
      gtw[lane] = g2;
      gtw[CH + lane] = ex2(g2);
      gtw[2 * CH + lane] = lane < Lc ? sm.braw[s][lane] : 0.f;
      gtw[3 * CH + lane] = ex2(g2L - g2);
    }
    asm volatile("" ::: "memory");

    // -- prep
    if (cw < 2) {
      // 32 x 32 inverse of rows/columns 32cw .. 32cw + 31.
      const int ba = 2 * cw, bb = 2 * cw + 1;
      const f32x4 daa = gram(Ks, ba, Ks, ba, ao);  // lane i, rows j
      const f32x4 dbb = gram(Ks, bb, Ks, bb, ao);
      const f32x4 dba = gram(Ks, bb, Ks, ba, ao);  // lane j (block a), rows i (block b)
      {
#pragma unroll
        for (int blk = 0; blk < 2; ++blk) {
          const int ib = ba + blk;
          const f32x4 d = blk ? dbb : daa;
          const float gi = gtw[16 * ib + i16];
          const float bi = gtw[2 * CH + 16 * ib + i16];
          const f32x4 gj = *reinterpret_cast<const f32x4*>(&gtw[16 * ib + 4 * h4]);
          f32x4 v;
#pragma unroll
          for (int r = 0; r < 4; ++r) v[r] = 4 * h4 + r < i16 ? bi * d[r] * ex2(gi - gj[r]) : 0.f;
          *reinterpret_cast<f32x4*>(&sm.abb[cw][blk][aoff(i16, 4 * h4)]) = v;
        }
      }
      f32x4 aba;  // A_ba[4h4 + r][i16] (rows in block b, column in block a)
      {
        const float gj = gtw[16 * ba + i16];
        const f32x4 gi = *reinterpret_cast<const f32x4*>(&gtw[16 * bb + 4 * h4]);
        const f32x4 bi = *reinterpret_cast<const f32x4*>(&gtw[2 * CH + 16 * bb + 4 * h4]);
#pragma unroll
        for (int r = 0; r < 4; ++r) aba[r] = bi[r] * dba[r] * ex2(gi[r] - gj);
      }
      asm volatile("" ::: "memory");
      // (I + A_bb)^-1 of both diagonal blocks, fp32 forward substitution with
      // lane (j, p) = (lane/4, lane%4) owning column j and the terms m = 4q + p
      // of every row sum (a step is <= 4 FMAs and a quad sum per block).
      {
        const int jc = lane >> 2, ph = lane & 3;
        float arow[2][16][4];
#pragma unroll
        for (int blk = 0; blk < 2; ++blk)
#pragma unroll
          for (int rr = 1; rr < 16; ++rr)
#pragma unroll
            for (int q = 0; 4 * q < rr; ++q) arow[blk][rr][q] = sm.abb[cw][blk][aoff(rr, 4 * q + ph)];
        float t[2][4];
#pragma unroll
        for (int blk = 0; blk < 2; ++blk)
#pragma unroll
          for (int q = 0; q < 4; ++q) t[blk][q] = 4 * q + ph == jc ? 1.f : 0.f;
#pragma unroll
        for (int rr = 1; rr < 16; ++rr) {
#pragma unroll
          for (int blk = 0; blk < 2; ++blk) {
            // A_bb is strictly lower (zeros from the gated tile), so terms with
            // 4q + ph >= rr read zeros and need no mask.
            float part = 0.f;
#pragma unroll
            for (int q = 0; 4 * q < rr; ++q) part += arow[blk][rr][q] * t[blk][q];
            const float sum = quad_sum(part);
            const float val = rr > jc ? -sum : (rr == jc ? 1.f : 0.f);
            if ((rr & 3) == ph) t[blk][rr >> 2] = val;
          }
        }
#pragma unroll
        for (int blk = 0; blk < 2; ++blk)
#pragma unroll
          for (int q = 0; q < 4; ++q) sm.tbb[cw][blk][aoff(4 * q + ph, jc)] = t[blk][q];
      }
      asm volatile("" ::: "memory");
      // Tiles of the 32 x 32 inverse [[T_aa, 0], [X, T_bb]], X = -T_bb A_ba T_aa.
      {
        const f32x4 ta = *reinterpret_cast<const f32x4*>(&sm.tbb[cw][0][aoff(i16, 4 * h4)]);  // T_aa[i16][4h4..]
        const f32x4 tb = *reinterpret_cast<const f32x4*>(&sm.tbb[cw][1][aoff(i16, 4 * h4)]);  // T_bb[i16][4h4..]
        f32x4 tat;                                                                             // T_aa[4h4..][i16]
#pragma unroll
        for (int r = 0; r < 4; ++r) tat[r] = sm.tbb[cw][0][aoff(4 * h4 + r, i16)];
        uint2 tah, tal, tbh, tbl, tath, tatl, abh, abl;
        split4(ta, tah, tal);
        split4(tb, tbh, tbl);
        split4(tat, tath, tatl);
        split4(aba, abh, abl);
        // Z = A_ba^T T_bb^T, X^T = -T_aa^T Z
        f32x4 z = mma16(abh, tbh, zero4());
        z = mma16(abh, tbl, z);
        z = mma16(abl, tbh, z);
        uint2 zh, zl;
        split4(z, zh, zl);
        f32x4 xt = mma16(tath, zh, zero4());
        xt = mma16(tath, zl, xt);
        xt = mma16(tatl, zh, xt);
        uint2 xh, xl;
        split4(-xt, xh, xl);
        sm.ttab[ba][0][lane] = make_uint4(tah.x, tah.y, 0u, 0u);
        sm.ttab[ba][1][lane] = make_uint4(tal.x, tal.y, 0u, 0u);
        sm.ttab[bb][0][lane] = make_uint4(xh.x, xh.y, tbh.x, tbh.y);
        sm.ttab[bb][1][lane] = make_uint4(xl.x, xl.y, tbl.x, tbl.y);
      }
    } else {
      const int first = cw == 4 ? 12 : cw == 5 ? 13 : (cw < 4 ? cw - 2 : cw - 4);  // 0,1,(12),(13),2,3
#pragma unroll
      for (int it = 0; it < 3; ++it) {
        if (it > 0 && (cw == 4 || cw == 5)) break;
        const int idx = first + 4 * it;  // waves 2,3,6,7: idx, idx + 4, idx + 8
        const int code = tile_code(idx);
        const int kind = code >> 4, jb = (code >> 2) & 3, ib = code & 3;
        const f32x4 d = gram(Ks, jb, kind ? Qs : Ks, ib, ao);  // lane i (block ib), rows j (block jb)
        const float gi = gtw[16 * ib + i16];
        const f32x4 gj = *reinterpret_cast<const f32x4*>(&gtw[16 * jb + 4 * h4]);
        if (kind == 0) {
          const float bi = gtw[2 * CH + 16 * ib + i16];
          f32x4 v;
#pragma unroll
          for (int r = 0; r < 4; ++r) v[r] = -bi * d[r] * ex2(gi - gj[r]);
          uint2 vh, vl;
          split4(v, vh, vl);
          reinterpret_cast<uint2*>(&sm.ttab[4 + ib - 2][0][lane])[jb & 1] = vh;
          reinterpret_cast<uint2*>(&sm.ttab[4 + ib - 2][1][lane])[jb & 1] = vl;
        } else {
          f32x4 v;
#pragma unroll
          for (int r = 0; r < 4; ++r) v[r] = 16 * jb + 4 * h4 + r <= 16 * ib + i16 ? args.scale * d[r] * ex2(gi - gj[r]) : 0.f;
          const int pp = ib < 2 ? ib : 2 * ib - 2 + (jb >> 1);
          reinterpret_cast<uint2*>(&sm.ptab[pp][lane])[jb & 1] = make_uint2(pk2(v[0], v[1]), pk2(v[2], v[3]));
          if (jb == ib && (jb & 1) == 0)  // the other half of this operand is above the diagonal
            reinterpret_cast<uint2*>(&sm.ptab[pp][lane])[1] = make_uint2(0u, 0u);
        }
      }
    }

    // -- state, part 1: R = diag(b)(V - gamma K S0), O^T = scale gamma (S0^T Q^T)
    f32x4 R[4], OT[4];
    {
      uint4 sh[4], sl[4];
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) split8(S[2 * kk], S[2 * kk + 1], sh[kk], sl[kk]);
#pragma unroll
      for (int b = 0; b < 4; ++b) R[b] = OT[b] = zero4();
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const uint4 ak = ld_a8(Ks + ROW16 * b, ao[kk]);
          const uint4 aq = ld_a8(Qs + ROW16 * b, ao[kk]);
          R[b] = mma32(ak, sh[kk], R[b]);
          R[b] = mma32(ak, sl[kk], R[b]);
          OT[b] = mma32(sh[kk], aq, OT[b]);
        }
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const f32x4 gv = *reinterpret_cast<const f32x4*>(&gtw[CH + 16 * b + 4 * h4]);
        const f32x4 bv = *reinterpret_cast<const f32x4*>(&gtw[2 * CH + 16 * b + 4 * h4]);
        const f32x4 vv = bf4(ld_tr(Vs + ROW16 * b, vo));
        R[b] = bv * (vv - gv * R[b]);
        OT[b] *= args.scale * gtw[CH + 16 * b + i16];
      }
    }
    // The previous chunk's output rows leave here, after the next chunk's
    // DMA has been issued, so they do not queue ahead of it.
    if (prev_t0 >= 0) store_out(prev_t0, prev_L);
    __syncthreads();  // (D) the inverse, -A and P^T operands of every wave are in LDS

    // -- state, part 2: two-level solve, output and state update
    {
      uint4 rh, rl, u0h, u0l, u1h, u1l;
      split8(R[0], R[1], rh, rl);
      const f32x4 U0 = mma32x3(sm.ttab[0][0][lane], sm.ttab[0][1][lane], rh, rl, zero4());
      const f32x4 U1 = mma32x3(sm.ttab[1][0][lane], sm.ttab[1][1][lane], rh, rl, zero4());
      split8(U0, U1, u0h, u0l);
      R[2] = mma32x3(sm.ttab[4][0][lane], sm.ttab[4][1][lane], u0h, u0l, R[2]);
      R[3] = mma32x3(sm.ttab[5][0][lane], sm.ttab[5][1][lane], u0h, u0l, R[3]);
      split8(R[2], R[3], rh, rl);
      const f32x4 U2 = mma32x3(sm.ttab[2][0][lane], sm.ttab[2][1][lane], rh, rl, zero4());
      const f32x4 U3 = mma32x3(sm.ttab[3][0][lane], sm.ttab[3][1][lane], rh, rl, zero4());
      split8(U2, U3, u1h, u1l);

      OT[0] = mma32(u0h, sm.ptab[0][lane], OT[0]);
      OT[1] = mma32(u0h, sm.ptab[1][lane], OT[1]);
      OT[2] = mma32(u0h, sm.ptab[2][lane], OT[2]);
      OT[2] = mma32(u1h, sm.ptab[3][lane], OT[2]);
      OT[3] = mma32(u0h, sm.ptab[4][lane], OT[3]);
      OT[3] = mma32(u1h, sm.ptab[5][lane], OT[3]);

      uint4 w0h, w0l, w1h, w1l;
      {
        const f32x4 d0 = *reinterpret_cast<const f32x4*>(&gtw[3 * CH + 0 + 4 * h4]);
        const f32x4 d1 = *reinterpret_cast<const f32x4*>(&gtw[3 * CH + 16 + 4 * h4]);
        const f32x4 d2 = *reinterpret_cast<const f32x4*>(&gtw[3 * CH + 32 + 4 * h4]);
        const f32x4 d3 = *reinterpret_cast<const f32x4*>(&gtw[3 * CH + 48 + 4 * h4]);
        split8(d0 * U0, d1 * U1, w0h, w0l);
        split8(d2 * U2, d3 * U3, w1h, w1l);
      }
      const float gL = gtw[CH + CH - 1];
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) {
        const char* kt = Ks + 32 * (mt & 1);
        const uint2 k0 = ld_tr(kt, ko[mt >> 1]), k1 = ld_tr(kt + ROW16, ko[mt >> 1]);
        const uint2 k2 = ld_tr(kt + 2 * ROW16, ko[mt >> 1]), k3 = ld_tr(kt + 3 * ROW16, ko[mt >> 1]);
        const uint4 a0 = make_uint4(k0.x, k0.y, k1.x, k1.y), a1 = make_uint4(k2.x, k2.y, k3.x, k3.y);
        f32x4 acc = S[mt] * gL;
        acc = mma32(a0, w0h, acc);
        acc = mma32(a0, w0l, acc);
        acc = mma32(a1, w1h, acc);
        S[mt] = mma32(a1, w1l, acc);
      }
#pragma unroll
      for (int b = 0; b < 4; ++b)
        *reinterpret_cast<uint2*>(sm.ost + sto_w + b * 16 * 256) = make_uint2(pk2(OT[b][0], OT[b][1]), pk2(OT[b][2], OT[b][3]));
    }
    prev_t0 = t0;
    prev_L = Lc;
  }
  __syncthreads();  // every wave's staged rows of the last chunk
  store_out(prev_t0, prev_L);

  // ---- segment end: publish the state -------------------------------------------
  float* dst = nullptr;
  if (args.states)
    dst = args.states + (static_cast<size_t>(seg) * args.h_v + h) * head_elems;
  else if (args.slot[seg] >= 0)
    dst = args.slots + (static_cast<size_t>(args.slot[seg]) * args.h_v + h) * head_elems;
  if (dst) {
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) dst[(16 * mt + 4 * h4 + r) * D + col_w + i16] = S[mt][r];
  }
}

}  // namespace

hipError_t launch_scan_d128(const ScanArgs& a, hipStream_t stream) {
  gdn_d128_kernel<<<dim3(static_cast<unsigned>(a.n_items) * a.h_v), 64 * NW, 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace tg
