// Chunked tree Gated DeltaNet forward for bf16, d_k = d_v = 128, on gfx950.
//
// Method ("Tree Training", arXiv 2511.00413, section 3.2 Eq. 10 and the
// chunked form of appendix A.2), per 32-token chunk of one segment and one
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
// accumulator registers for the whole segment.  Registers are held to 128
// per lane and LDS to 72 KB so that two work-groups share a compute unit;
// their phases drift apart, so one's MFMA work fills the other's latency.
// Per chunk:
//
//   gates                    made for the next chunk by one wave (GW) in its
//                            slack before the chunk barrier: the in-chunk
//                            prefix G (DPP scan) and the tables every wave
//                            reads, double-buffered in LDS.
//   prep (no state needed)   Waves 0 and 1: one 16 x 16 diagonal block of
//                            K K^T each and its inverse (I + A_bb)^-1 (fp32
//                            right-looking substitution).  Wave 2: the
//                            off-diagonal block A_10.  Waves 3, 6, 7: the three
//                            Q K^T blocks.  All land in LDS as ready-made MFMA
//                            operands, split hi + lo where they feed the state.
//   state, part 1            R = diag(b)(V - gamma K S0) and O^T = S0^T Q^T.
//   ---- barrier ----
//   state, part 2            U_0 = T_00 R_0, R_1 -= A_10 U_0, U_1 = T_11 R_1;
//                            O^T += U^T P^T;  S = gamma_L S + K^T W.
//
// Products that feed the state carry their fp32 operand as hi + lo bf16
// (relative 2^-17; lo x lo dropped); the output path uses hi only.  Where the
// decay inside a chunk makes the second row block's share of K S0 or Q S0
// (scaled by gamma_i) no larger than the error the other rows already carry,
// those MFMAs are not issued (part 1 has one instantiation per such class).  The
// state's own split, and those of R in the solve, take their exact residual
// x - hi from an MFMA (split4m), which leaves the vector ALU two conversions
// per pair of values.  The
// output is produced transposed, so a lane holds 4 consecutive value columns
// of one token.
//
// Data movement: q, k, v, g and beta of chunk n + 1 are DMA'd from HBM into
// LDS (buffer loads straight to LDS, 16 bytes per lane, no staging registers)
// at the start of chunk n, into the other half of double buffers.  The output
// of chunk n is staged in LDS and leaves as whole 256-byte token rows during
// chunk n + 1.  Loads and stores go through buffer descriptors, so per-lane
// offsets are loop constants and masked output rows are dropped by the
// descriptor's range check.
//
// Tile layout in LDS (see toff): rows in 4-row blocks of 1 KB (one DMA
// instruction each) at a 1088-byte stride, block b shifted by a further
// {0, 2, 1, 3}[b % 4] x 16 bytes, and the 16-byte chunk c of row r stored at
// slot c ^ 4(r % 4).  With it the two read patterns used here -- MFMA operand
// reads (two 8-byte pieces 32 bytes apart, two ds_read_b64) of 16 rows and
// the transposing read ds_read_b64_tr_b16 of 4 rows x 16 columns -- hit every
// LDS bank once per half-wave.
#include <hip/hip_runtime.h>

#include <utility>

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
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) const u32x2 lds_u2;

constexpr int CH = 32;          // chunk length (tokens)
constexpr int D = 128;          // d_k = d_v
constexpr int NW = 8;           // waves per work-group
constexpr int GW = 3;           // the wave that loads g, beta and makes the gate tables
constexpr int DW0 = 4;          // waves DW0, DW0 + 1 DMA the q, k, v tiles and store the output (16 rows each)
constexpr int TSZ = 8704;       // LDS bytes of one 32 x 128 bf16 tile (see toff)
constexpr int ROW16 = 4352;     // bytes between rows 16 apart
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
// hi x hi + hi x lo + lo x hi (K = 16).
__device__ __forceinline__ f32x4 mma16x3(const uint2 ah, const uint2 al, const uint2 bh, const uint2 bl, f32x4 c) {
  c = mma16(ah, bh, c);
  c = mma16(ah, bl, c);
  return mma16(al, bh, c);
}
__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }
// x = hi + lo as split4, with the residual lo = x - float(hi) formed by a
// 16x16x16 MFMA instead of the vector ALU: -I times the packed hi (exact
// products) added to x, which enters as the fp32 accumulator input.  The sum
// is exactly representable, so lo is bitwise the same as split4's; the vector
// ALU only does the two conversions.  x is one accumulator tile (lane (n, h)
// holds rows 4h..4h+3 of column n), which is also the B operand layout of hi;
// negI is the A operand of -I (lane (m, h): -1 at column m of 4h..4h+3).
__device__ __forceinline__ void split4m(const f32x4 x, const uint2 negI, uint2& hi, uint2& lo) {
  hi = make_uint2(pk2(x[0], x[1]), pk2(x[2], x[3]));
  const f32x4 r = mma16(negI, hi, x);
  lo = make_uint2(pk2(r[0], r[1]), pk2(r[2], r[3]));
}
__device__ __forceinline__ void split8m(const f32x4 x0, const f32x4 x1, const uint2 negI, uint4& hi, uint4& lo) {
  uint2 h0, l0, h1, l1;
  split4m(x0, negI, h0, l0);
  split4m(x1, negI, h1, l1);
  hi = make_uint4(h0.x, h0.y, h1.x, h1.y);
  lo = make_uint4(l0.x, l0.y, l1.x, l1.y);
}
__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }
// Lane i gets lane i - n of its row of 16 (0 for the first n lanes of a row).
__device__ __forceinline__ float dpp_shr(float x, int n) {
  switch (n) {
    case 1: return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x111, 0xF, 0xF, true));
    case 2: return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x112, 0xF, 0xF, true));
    case 4: return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x114, 0xF, 0xF, true));
    default: return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x118, 0xF, 0xF, true));
  }
}
// Sum over the 4 lanes of a quad (lanes 4k..4k+3), result in all four.
// f(integral_constant<int, M>) for M in order (compile-time step indices).
template <typename F, int... M>
__device__ __forceinline__ void for_each_index(F&& f, std::integer_sequence<int, M...>) {
  (f(std::integral_constant<int, M>{}), ...);
}
// Lane k of each quad, broadcast to the whole quad (DPP quad_perm [k,k,k,k]).
template <int K>
__device__ __forceinline__ float quad_bcast(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), K * 0x55, 0xF, 0xF, true));
}
__device__ __forceinline__ float quad_sum(float x) {
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, true));  // [1,0,3,2]
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, true));  // [2,3,0,1]
  return x;
}

// ---- 32 x 128 bf16 tiles in LDS ------------------------------------------------
// Byte offset of the 4-row block b, and of element (row, col).
__device__ __forceinline__ int blk_off(int b) { return b * 1088 + 16 * ((0x3120 >> (4 * (b & 3))) & 3); }
__device__ __forceinline__ int toff(int row, int col) {
  return blk_off(row >> 2) + (row & 3) * 256 + 16 * ((col >> 3) ^ (4 * (row & 3))) + 2 * (col & 7);
}
// A operand of a 16x16x32 MFMA (or the B operand, the roles are symmetric)
// at byte offset `o` = toff(row, col0 + 4h): row `row`, columns
// col0 + kmap(h, 0..7), kmap(h, j) = j<4 ? 4h+j : 16+4h+(j-4); the two 8-byte
// pieces are 32 bytes apart in this layout.  The same K order lets two
// accumulator tiles (rows 4h..4h+3 of each) serve as one K = 32 operand
// without moving data.  The second piece is read at `o2`, a loop-constant
// copy of o + 32 that the compiler cannot see through, so the pieces stay
// two ds_read_b64 (fused into one ds_read2_b64 they take several times as
// long on this part) and each address is one register plus an immediate.
__device__ __forceinline__ uint4 ld_a8(const char* t, int o, int o2) {
  const u32x2 x = *(const lds_u2*)(t + o), y = *(const lds_u2*)(t + o2);
  return make_uint4(x[0], x[1], y[0], y[1]);
}
// Transposing read at byte offset `o` = toff(row0 + 4h + i/4, col0 + 4(i%4))
// for lane i of 16-lane group h: the lane gets rows row0 + 4h + 0..3 of
// column col0 + i.
__device__ __forceinline__ uint2 ld_tr(const char* t, int o) {
  return __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(t + o)));
}
__device__ __forceinline__ f32x4 bf4(const uint2 x) { return f32x4{lo_f(x.x), hi_f(x.x), lo_f(x.y), hi_f(x.y)}; }

struct Smem {
  alignas(16) char kb[2][TSZ];       // K tiles
  alignas(16) char qb[2][TSZ];       // Q tiles
  alignas(16) char vb[2][TSZ];       // V tiles
  // 16x16x16 A operands per lane, hi in .xy and lo in .zw: 0 = T_00,
  // 1 = T_11, 2 = -A_10.
  alignas(16) uint4 ttab[3][64];
  // 16x16x32 B operands of O^T += U^T P^T for token blocks 0 and 1.
  alignas(16) uint4 ptab[2][64];
  // Waves 0, 1: their gated diagonal block by columns, -A[4q + p][m] at [m][p][3 - q].
  alignas(16) float abb[2][256];
  // Gate tables of the chunk in buffer s: G log2(e), exp(G), beta, exp(G_L - G).
  alignas(16) float gt[2][4][CH];
  // Largest gamma of the chunk's second 16-row block (rows 16..31).
  alignas(16) float gmax1[2];
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

// Raw 16 x 16 Gram tile D[x][y] = X[x] . Y[y] over 128 features (X, Y point
// at row blocks of tiles): lane (y = i, h) holds x = 4h + 0..3.
// ao[kk] = toff(i, 32kk + 4h), ao2[kk] its opaque copy + 32.
__device__ __forceinline__ f32x4 gram(const char* X, const char* Y, const int* ao, const int* ao2) {
  uint4 a[4], b[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    a[kk] = ld_a8(X, ao[kk], ao2[kk]);
    b[kk] = ld_a8(Y, ao[kk], ao2[kk]);
  }
  f32x4 acc = zero4();
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) acc = mma32(a[kk], b[kk], acc);
  return acc;
}

// PATHS = false: block item = one segment of a level, starting from its
// parent's state.  PATHS = true: block item = one rescan walk, the segments
// of a root-to-leaf path in order with the state carried in registers from
// one to the next; outputs and states are written only for the segments the
// walk owns.
// CK: the checkpoint pass of the scan backward instead of the forward: every
// segment at once from its parent's final state (the forward's `states`,
// read only), storing the start state of every 4th chunk (every 128 tokens)
// at the backward's checkpoint slots, and for each 16-token half of a chunk
// (one backward chunk) its T = (I + A)^-1, K K^T and Q K^T as fp32 16 x 16
// tables; no output, no Q S0 and no state publication.
static_assert(kBwdCkpt * 16 == 4 * CH, "a checkpoint every 128 tokens: every 8th 16-token backward chunk");

template <bool PATHS, bool CK = false>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(4, 4))) void gdn_d128_kernel(ScanArgs args) {
  static_assert(!(PATHS && CK), "checkpoints are taken per segment");
  __shared__ Smem sm;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int cw = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h4 = lane >> 4;
  const int i16 = lane & 15;
  // -I as a 16x16x16 A operand (split4m).
  uint2 negI;
  {
    const int j = i16 - 4 * h4;
    negI = make_uint2((j == 0 ? 0xBF80u : 0u) | (j == 1 ? 0xBF800000u : 0u),
                      (j == 2 ? 0xBF80u : 0u) | (j == 3 ? 0xBF800000u : 0u));
  }

  // Block -> (item, value head), XCD-aware.  The dispatcher deals blocks to
  // the 8 XCDs in turn (block b on XCD b % 8).  Within each run of 4 items,
  // XCDs 2i and 2i + 1 take the two halves of item i's value heads, so each
  // token's g and beta (one 128-byte line holds all heads' values) are
  // fetched into two L2s rather than all eight, and value heads that share a
  // q/k head (adjacent heads) read its tiles through one L2.  Items past the
  // last whole run, and head counts not a multiple of 4, keep the plain
  // order.  (One XCD per item fetched 8% less but was not faster.)
  int item, h;
  {
    const int b = blockIdx.x;
    const int full = (args.n_items / 4) * 4;
    if (args.h_v % 4 == 0 && b < full * args.h_v) {
      const int gi = b / (4 * args.h_v), r = b - gi * 4 * args.h_v;
      const int x = r & 7;
      item = 4 * gi + (x >> 1);
      h = (x & 1) * (args.h_v >> 1) + (r >> 3);
    } else {
      item = b / args.h_v;
      h = b - item * args.h_v;
    }
  }
  const int hq = h / (args.h_v / args.h_qk);
  int wj = 0, wend = 0;  // walk cursor (PATHS)
  int seg;
  bool own = true;  // this block writes the current segment's outputs and state
  if (PATHS) {
    wj = args.walk_off[item];
    wend = args.walk_off[item + 1];
    const int e = args.walk[wj];
    seg = e < 0 ? ~e : e;
    own = e >= 0;
  } else {
    seg = args.items[item];
  }
  const int seg_beg = args.seg_off[seg];
  int seg_end = args.seg_off[seg + 1];
  const int par = args.parent[seg];
  const uint16_t* qg = static_cast<const uint16_t*>(args.q);
  const uint16_t* kg = static_cast<const uint16_t*>(args.k);
  const uint16_t* vg = static_cast<const uint16_t*>(args.v);
  uint16_t* og = static_cast<uint16_t*>(args.o);
  const int col_w = 16 * cw;

  // Loop-constant byte offsets of the hot reads: operand reads of rows i16
  // (+16 per row block) at columns 32kk + 4h4; transposing reads of K at
  // columns 32m (+16 is +32 bytes) and of V at this wave's columns.
  int ao[4], ao2[4], ko[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    ao[kk] = toff(i16, 32 * kk + 4 * h4);
    ao2[kk] = ao[kk] + 32;
    asm volatile("" : "+v"(ao2[kk]));
    ko[kk] = toff(4 * h4 + (i16 >> 2), 32 * kk + 4 * (i16 & 3));
  }
  const int vo = toff(4 * h4 + (i16 >> 2), col_w + 4 * (i16 & 3));
  const int rs_qk = args.h_qk * D * 2, rs_v = args.h_v * D * 2;  // bytes between token rows

  // ---- initial state: S[mt] rows 16mt + 4h4 + 0..3, column col_w + i16 --------
  const size_t head_elems = static_cast<size_t>(D) * D;
  f32x4 S[8];
  {
    const float* src = nullptr;
    if (par >= 0)
      src = args.states ? args.states + (static_cast<size_t>(par) * args.h_v + h) * head_elems
                        : args.slots + (static_cast<size_t>(args.slot[par]) * args.h_v + h) * head_elems;
    else if (args.init)  // a root with a caller-given initial state
      src = args.init + (static_cast<size_t>(args.root_idx[seg]) * args.h_v + h) * head_elems;
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

  // Chunk at token tc into buffer buf: waves DW0 and DW0 + 1, which have the
  // least work before the chunk barrier, load row blocks 0-3 and 4-7 (rows
  // 4b..4b+3) of the K, Q and V tiles; wave GW the g and beta rows.  In a
  // partial chunk, rows past the end repeat row Ln - 1.  V is read by this
  // work-group only, so it goes through L2 as non-temporal (as do the output
  // rows): K and Q, which the other value head of the pair reads on the same
  // XCD, and the parent states stay there longer.
  auto fetch = [&](int tc, int end, int buf) {
    // Offsets of once-per-chunk accesses are recomputed from an opaque copy
    // of the lane number rather than held in registers across the loop.
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int cofs = 16 * ((ln & 15) ^ (4 * (ln >> 4)));  // this lane's 16-byte chunk of a row
    const int Ln = min(CH, end - tc);
    const auto rk = rsrc(kg + (static_cast<size_t>(tc) * args.h_qk + hq) * D, CH * rs_qk);
    const auto rq = rsrc(qg + (static_cast<size_t>(tc) * args.h_qk + hq) * D, CH * rs_qk);
    const auto rv = rsrc(vg + (static_cast<size_t>(tc) * args.h_v + h) * D, CH * rs_v);
    if (cw == DW0 || cw == DW0 + 1) {
#pragma unroll
      for (int bi = 0; bi < 4; ++bi) {
        const int blk = 4 * (cw - DW0) + bi;
        const int row = min(4 * blk + (ln >> 4), Ln - 1);
        const int ok = row * rs_qk + cofs, ov = row * rs_v + cofs;
        const int lo = blk_off(blk);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void*)(sm.kb[buf] + lo), 16, ok, 0, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rq, (lds_void*)(sm.qb[buf] + lo), 16, ok, 0, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void*)(sm.vb[buf] + lo), 16, ov, 0, 0, kCacheNT);
      }
    }
    if (cw == GW && lane < CH) {  // lane l writes LDS word l of the row
      const size_t base = static_cast<size_t>(tc) * args.h_v + h;
      const int go = min(lane, Ln - 1) * args.h_v * 4;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc(args.g + base, CH * args.h_v * 4), (lds_void*)sm.graw[buf], 4, go,
                                               0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc(args.beta + base, CH * args.h_v * 4), (lds_void*)sm.braw[buf], 4,
                                               go, 0, 0, 0);
    }
  };

  // Gate tables of the chunk in buffer buf (L tokens), by wave GW once its
  // own DMA of g and beta has landed: inclusive prefix G of g over rows of
  // 16 lanes (DPP), then row 1 adds row 0's total.
  auto make_gates = [&](int buf, int L) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    float x = lane < L ? sm.graw[buf][lane & (CH - 1)] : 0.f;
    x += dpp_shr(x, 1);
    x += dpp_shr(x, 2);
    x += dpp_shr(x, 4);
    x += dpp_shr(x, 8);
    x += lane >= 16 ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 15)) : 0.f;
    const float g2 = x * kLog2e;
    const float g2L = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(g2), CH - 1));
    const float gam = ex2(g2);
    if (lane < CH) {
      float* gt = &sm.gt[buf][0][0];
      gt[lane] = g2;
      gt[CH + lane] = gam;
      gt[2 * CH + lane] = lane < L ? sm.braw[buf][lane] : 0.f;
      gt[3 * CH + lane] = ex2(g2L - g2);
    }
    // Max of gamma over rows 16..31 (lane row 1): a running max along the row.
    float gm = lane >= 16 && lane < CH ? gam : 0.f;
    gm = fmaxf(gm, dpp_shr(gm, 1));
    gm = fmaxf(gm, dpp_shr(gm, 2));
    gm = fmaxf(gm, dpp_shr(gm, 4));
    gm = fmaxf(gm, dpp_shr(gm, 8));
    gm = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(gm), CH - 1));
    if (lane == 0) sm.gmax1[buf] = gm;
  };

  // Whole token rows of the staged output, by the DMA waves (rows 16(cw -
  // DW0) .. +15); the descriptor ends after row Ln - 1, so rows past it are
  // not written.  A lane stores 16-byte chunk lane % 16 of token rows
  // 4b + lane / 16.
  auto store_out = [&](int tc, int Ln) {
    if (cw != DW0 && cw != DW0 + 1) return;
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const auto ro = rsrc(og + (static_cast<size_t>(tc) * args.h_v + h) * D, (Ln - 1) * rs_v + D * 2);
#pragma unroll
    for (int bi = 0; bi < 4; ++bi) {
      const int orow = 4 * (4 * (cw - DW0) + bi) + (ln >> 4);
      const u32x4 v = *reinterpret_cast<const u32x4*>(sm.ost + orow * 256 + 16 * ((ln & 15) ^ (orow & 15)));
      __builtin_amdgcn_raw_buffer_store_b128(v, ro, orow * rs_v + 16 * (ln & 15), 0, kCacheNT);
    }
  };

  fetch(seg_beg, seg_end, 0);
  if (cw == GW) make_gates(0, min(CH, seg_end - seg_beg));
  int s = 0;
  int prev_t0 = -1, prev_L = 0;
  bool prev_own = true;

  for (int t0 = seg_beg;;) {
    const int Lc = min(CH, seg_end - t0);
    const char* Ks = sm.kb[s];
    const char* Qs = sm.qb[s];
    const char* Vs = sm.vb[s];
    // Next chunk: the rest of this segment, else (walks) the start of the
    // next segment on the path.
    int nt0 = t0 + CH, nend = seg_end, nseg = seg;
    if (PATHS && nt0 >= seg_end && wj + 1 < wend) {
      const int e = args.walk[wj + 1];
      nseg = e < 0 ? ~e : e;
      nt0 = args.seg_off[nseg];
      nend = args.seg_off[nseg + 1];
    }
    const bool more = nt0 < nend;

    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's DMA of the chunk has landed
    __syncthreads();                                   // (A) ... and every other wave's
    if (more) fetch(nt0, nend, s ^ 1);
    // The previous chunk's output rows leave right after the next chunk's
    // DMA is issued (not ahead of it), a whole chunk before the wait above
    // has to count them.
    if constexpr (!CK) {
      if (prev_t0 >= 0 && prev_own) store_out(prev_t0, prev_L);
    } else if ((((t0 - seg_beg) / CH) & 3) == 0) {
      // Checkpoint (t0 - seg_beg) / 128 of the segment: S is this chunk's
      // start state; tile (mt, cw) in the lanes' accumulator order.
      int ln = lane;
      asm volatile("" : "+v"(ln));
      float* const dst =
          args.ckpt + (static_cast<size_t>(args.gck[seg] + (t0 - seg_beg) / (4 * CH)) * args.h_v + h) * head_elems +
          cw * 256 + 4 * ln;
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) __builtin_nontemporal_store(S[mt], reinterpret_cast<f32x4*>(dst + mt * 8 * 256));
    }

    // -- gate tables of this chunk (made by wave GW during the previous one)
    const float* gtw = &sm.gt[s][0][0];

    // CK: the tables of backward chunk 2 (chunk index) + b, rows past the
    // segment end zeroed (there the backward's rows are zero); none for a
    // half past the end.
    const int nb_ck = CK ? min(16, max(0, Lc - 16 * (cw == 7 ? 1 : (cw < 2 ? cw : 0)))) : 0;
    auto table_rsrc = [&](int b) {
      const int c16 = 2 * ((t0 - seg_beg) / CH) + b;
      return rsrc(args.tws + (static_cast<size_t>(args.gchunk[seg] + c16) * args.h_v + h) * (3 * 256), 3 * 256 * 4);
    };

    // -- prep
    if (cw < 2) {
      // Diagonal block cw: A[i][j] = b_i exp(G_i - G_j) k_i.k_j (j < i) and
      // T = (I + A)^-1 by right-looking fp32 substitution: once row m of T
      // is final, every row r > m subtracts A[r][m] T[m][:].  Lane (j, p) =
      // (lane/4, lane%4) holds T[4q + p][j] in t[q]; row m is broadcast
      // from the quad lane that owns it, so a step is one DPP move and up to
      // 4 independent FMAs (no reduction on the dependency chain).
      // -A is stored by columns: abb[m][p][3 - q] = -A[4q + p][m], so step m
      // reads the 4 - m/4 rows it updates as one contiguous piece.
      const f32x4 d = gram(Ks + ROW16 * cw, Ks + ROW16 * cw, ao, ao2);  // lane i, rows j
      if constexpr (CK) {
        if (nb_ck > 0) {  // K K^T[4h + r][i], row-major
          const auto rt = table_rsrc(cw);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float x = 4 * h4 + r < nb_ck && i16 < nb_ck ? d[r] : 0.f;
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(x), rt, 4 * (256 + (4 * h4 + r) * 16 + i16), 0, 0);
          }
        }
      }
      {
        const float gi = gtw[16 * cw + i16];
        const float bi = gtw[2 * CH + 16 * cw + i16];
        const f32x4 gj = *reinterpret_cast<const f32x4*>(&gtw[16 * cw + 4 * h4]);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int m = 4 * h4 + r;
          sm.abb[cw][m * 16 + (i16 & 3) * 4 + 3 - (i16 >> 2)] = m < i16 ? -bi * d[r] * ex2(gi - gj[r]) : 0.f;
        }
      }
      asm volatile("" ::: "memory");
      const int jc = lane >> 2, ph = lane & 3;
      float na[15][4];  // na[m][3 - q] = -A[4q + ph][m], for q >= m / 4
#pragma unroll
      for (int m = 0; m < 15; ++m) {
        const float* pa = &sm.abb[cw][m * 16 + ph * 4];
        if (m < 4) {
          const float4 v = *reinterpret_cast<const float4*>(pa);
          na[m][0] = v.x, na[m][1] = v.y, na[m][2] = v.z, na[m][3] = v.w;
        } else if (m < 8) {
          const float2 v = *reinterpret_cast<const float2*>(pa);
          na[m][0] = v.x, na[m][1] = v.y, na[m][2] = pa[2];
        } else if (m < 12) {
          const float2 v = *reinterpret_cast<const float2*>(pa);
          na[m][0] = v.x, na[m][1] = v.y;
        } else {
          na[m][0] = pa[0];
        }
      }
      float t[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) t[q] = 4 * q + ph == jc ? 1.f : 0.f;
      auto step = [&](auto mc) {
        constexpr int m = decltype(mc)::value;
        const float bc = quad_bcast<m & 3>(t[m >> 2]);  // T[m][jc]
#pragma unroll
        for (int q = m >> 2; q < 4; ++q) t[q] = fmaf(na[m][3 - q], bc, t[q]);
      };
      for_each_index(step, std::make_integer_sequence<int, 15>{});
      // T[4q + ph][jc] -> operand lane (row 4q + ph, group jc / 4), element jc % 4.
      uint16_t* tt = reinterpret_cast<uint16_t*>(&sm.ttab[cw][0]);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int e = (4 * q + ph + 16 * (jc >> 2)) * 8 + (jc & 3);
        const uint32_t w = pk2(t[q], 0.f);
        tt[e] = static_cast<uint16_t>(w);
        tt[e + 4] = static_cast<uint16_t>(pk2(t[q] - lo_f(w), 0.f));
      }
      if constexpr (CK) {
        if (nb_ck > 0) {  // T[4q + ph][jc], row-major
          const auto rt = table_rsrc(cw);
#pragma unroll
          for (int q = 0; q < 4; ++q)
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(t[q]), rt, 4 * ((4 * q + ph) * 16 + jc), 0, 0);
        }
      }
    } else if (cw == 2) {
      // -A_10 as the A operand of R_1 -= A_10 U_0: lane i (token 16 + i),
      // rows j (tokens 0..15).
      const f32x4 d = gram(Ks, Ks + ROW16, ao, ao2);
      const float gi = gtw[16 + i16];
      const float bi = gtw[2 * CH + 16 + i16];
      const f32x4 gj = *reinterpret_cast<const f32x4*>(&gtw[4 * h4]);
      f32x4 v;
#pragma unroll
      for (int r = 0; r < 4; ++r) v[r] = -bi * d[r] * ex2(gi - gj[r]);
      uint2 vh, vl;
      split4(v, vh, vl);
      sm.ttab[2][lane] = make_uint4(vh.x, vh.y, vl.x, vl.y);
    } else if (CK && (cw == 3 || cw == 7)) {
      // Q K^T of half b = 0 (wave 3) or 1 (wave 7): lane i (key), rows j
      // (query), stored at [query][key].
      const int b = cw == 7 ? 1 : 0;
      const f32x4 d = gram(Qs + ROW16 * b, Ks + ROW16 * b, ao, ao2);
      if (nb_ck > 0) {
        const auto rt = table_rsrc(b);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float x = 4 * h4 + r < nb_ck && i16 < nb_ck ? d[r] : 0.f;
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(x), rt, 4 * (512 + (4 * h4 + r) * 16 + i16), 0, 0);
        }
      }
    } else if (!CK && (cw == 3 || cw >= 6)) {
      // P^T block (jb, ib) = (0, 0), (0, 1), (1, 1): lane i (query), rows j (key).
      const int jb = cw == 7 ? 1 : 0, ib = cw == 3 ? 0 : 1;
      const f32x4 d = gram(Ks + ROW16 * jb, Qs + ROW16 * ib, ao, ao2);
      const float gi = gtw[16 * ib + i16];
      const f32x4 gj = *reinterpret_cast<const f32x4*>(&gtw[16 * jb + 4 * h4]);
      f32x4 v;
#pragma unroll
      for (int r = 0; r < 4; ++r)
        v[r] = 16 * jb + 4 * h4 + r <= 16 * ib + i16 ? args.scale * d[r] * ex2(gi - gj[r]) : 0.f;
      reinterpret_cast<uint2*>(&sm.ptab[ib][lane])[jb] = make_uint2(pk2(v[0], v[1]), pk2(v[2], v[3]));
      if (ib == 0)  // the other half of this operand is above the diagonal
        reinterpret_cast<uint2*>(&sm.ptab[0][lane])[1] = make_uint2(0u, 0u);
    }

    // -- state, part 1: R = diag(b)(V - gamma K S0), O^T = scale gamma (S0^T Q^T)
    // S is decayed by gamma_L for the update of part 2 as soon as each pair
    // of tiles has been split, far ahead of the MFMAs that accumulate into it.
    //
    // Rows 16..31 enter both products scaled by their gamma_i <= g1 (the
    // block's largest).  With S0 = hi + lo (|S0 - hi| <= 2^-9 |S0|, the lo
    // pass leaving 2^-18), a term is dropped only where its bound falls to
    // what the other rows already carry: the lo pass of K S0 when g1 <= 2^-10
    // (g1 2^-9 < 2^-18 of sum |K||S0|), Q S0 when g1 <= 2^-12 (below the
    // 2^-9 of the hi-only output product of rows 0..15), and the hi pass of
    // K S0 too when g1 <= 2^-18.  The class is uniform over the work-group.
    const float gL = gtw[CH + CH - 1];
    f32x4 R[2], OT[2];
    R[0] = R[1] = OT[0] = OT[1] = zero4();
    auto part1 = [&](auto cls) {
      constexpr int C = decltype(cls)::value;  // 0: all terms, 1: no lo pass, 2: no Q S0, 3: no K S0 (rows 16..31)
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        uint4 sh, sl;
        split8m(S[2 * kk], S[2 * kk + 1], negI, sh, sl);
        S[2 * kk] *= gL;
        S[2 * kk + 1] *= gL;
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          if (b == 0 || C < 3) {
            const uint4 ak = ld_a8(Ks + ROW16 * b, ao[kk], ao2[kk]);
            R[b] = mma32(ak, sh, R[b]);
            if (b == 0 || C < 1) R[b] = mma32(ak, sl, R[b]);
          }
          if (!CK && (b == 0 || C < 2)) {
            // Kept apart from the K read at the same offsets: fused into one
            // ds_read2st64_b64 they cost several times as much.
            asm volatile("" ::: "memory");
            const uint4 aq = ld_a8(Qs + ROW16 * b, ao[kk], ao2[kk]);
            OT[b] = mma32(sh, aq, OT[b]);
          }
        }
      }
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const f32x4 bv = *reinterpret_cast<const f32x4*>(&gtw[2 * CH + 16 * b + 4 * h4]);
        const f32x4 vv = bf4(ld_tr(Vs + ROW16 * b, vo));
        // R = b (v - gamma K S0), the subtraction fused (one rounding) in every
        // instantiation; without K S0 (rows 16..31 of class 3) R = b v.
        if (b == 0 || C < 3) {
          const f32x4 gv = *reinterpret_cast<const f32x4*>(&gtw[CH + 16 * b + 4 * h4]);
#pragma unroll
          for (int r = 0; r < 4; ++r) R[b][r] = bv[r] * __builtin_fmaf(-gv[r], R[b][r], vv[r]);
        } else {
          R[b] = bv * vv;
        }
        if (!CK && (b == 0 || C < 2)) OT[b] *= args.scale * gtw[CH + 16 * b + i16];
      }
    };
    {
      const float g1 = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(sm.gmax1[s])));
      if (g1 > 0x1p-10f)
        part1(std::integral_constant<int, 0>{});
      else if (g1 > 0x1p-12f)
        part1(std::integral_constant<int, 1>{});
      else if (g1 > 0x1p-18f)
        part1(std::integral_constant<int, 2>{});
      else
        part1(std::integral_constant<int, 3>{});
    }
    __syncthreads();  // (D) the inverse, -A and P^T operands of every wave are in LDS

    // -- state, part 2: block solve, output and state update
    {
      uint2 rh, rl, u0h, u0l, u1h, u1l;
      const uint4 t0 = sm.ttab[0][lane], t1 = sm.ttab[1][lane], na = sm.ttab[2][lane];
      split4m(R[0], negI, rh, rl);
      const f32x4 U0 = mma16x3(make_uint2(t0.x, t0.y), make_uint2(t0.z, t0.w), rh, rl, zero4());
      split4(U0, u0h, u0l);
      R[1] = mma16x3(make_uint2(na.x, na.y), make_uint2(na.z, na.w), u0h, u0l, R[1]);
      split4m(R[1], negI, rh, rl);
      const f32x4 U1 = mma16x3(make_uint2(t1.x, t1.y), make_uint2(t1.z, t1.w), rh, rl, zero4());
      split4(U1, u1h, u1l);

      const uint4 uh = make_uint4(u0h.x, u0h.y, u1h.x, u1h.y);
      if constexpr (!CK) {
        OT[0] = mma32(uh, sm.ptab[0][lane], OT[0]);
        OT[1] = mma32(uh, sm.ptab[1][lane], OT[1]);
      }

      uint4 wh, wl;
      {
        const f32x4 d0 = *reinterpret_cast<const f32x4*>(&gtw[3 * CH + 4 * h4]);
        const f32x4 d1 = *reinterpret_cast<const f32x4*>(&gtw[3 * CH + 16 + 4 * h4]);
        split8(d0 * U0, d1 * U1, wh, wl);
      }
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) {
        const char* kt = Ks + 32 * (mt & 1);
        const uint2 k0 = ld_tr(kt, ko[mt >> 1]), k1 = ld_tr(kt + ROW16, ko[mt >> 1]);
        const uint4 a = make_uint4(k0.x, k0.y, k1.x, k1.y);
        S[mt] = mma32(a, wh, S[mt]);
        S[mt] = mma32(a, wl, S[mt]);
      }
      // Stage this chunk's output: token 16b + i16, value columns col_w + 4h4..+3.
      if constexpr (!CK) {
        int ln = lane;
        asm volatile("" : "+v"(ln));
        const int li = ln & 15, lh = ln >> 4;
        const int sto_w = li * 256 + 16 * ((2 * cw + (lh >> 1)) ^ li) + 8 * (lh & 1);
#pragma unroll
        for (int b = 0; b < 2; ++b)
          *reinterpret_cast<uint2*>(sm.ost + sto_w + b * 16 * 256) =
              make_uint2(pk2(OT[b][0], OT[b][1]), pk2(OT[b][2], OT[b][3]));
      }
    }
    prev_t0 = t0;
    prev_L = Lc;
    prev_own = own;
    if (PATHS && t0 + CH >= seg_end) {  // a walk's segment ends: its owner publishes the state
      if (own && args.states) {
        // Lane offsets from an opaque copy of the lane number, so that no
        // address of this once-per-segment store is held across the loop.
        int ln = lane;
        asm volatile("" : "+v"(ln));
        float* dst = args.states + (static_cast<size_t>(seg) * args.h_v + h) * head_elems +
                     (4 * (ln >> 4)) * D + col_w + (ln & 15);
#pragma unroll
        for (int mt = 0; mt < 8; ++mt)
#pragma unroll
          for (int r = 0; r < 4; ++r) dst[(16 * mt + r) * D] = S[mt][r];
      }
      if (more) own = args.walk[++wj] >= 0;
    }
    if (!more) break;
    // The next chunk's gate tables, in this wave's slack before barrier A.
    if (cw == GW) make_gates(s ^ 1, min(CH, nend - nt0));
    t0 = nt0;
    seg_end = nend;
    seg = nseg;
    s ^= 1;
  }
  __syncthreads();  // every wave's staged rows of the last chunk
  if constexpr (!CK) {
    if (prev_own) store_out(prev_t0, prev_L);
  }

  // ---- segment end: publish the state -------------------------------------------
  if (!PATHS && !CK) {
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
}

}  // namespace

hipError_t launch_scan_d128_checkpoints(const ScanArgs& a, hipStream_t stream) {
  if (a.n_items <= 0) return hipSuccess;
  gdn_d128_kernel<false, true><<<dim3(static_cast<unsigned>(a.n_items) * a.h_v), 64 * NW, 0, stream>>>(a);
  return hipGetLastError();
}

hipError_t launch_scan_d128(const ScanArgs& a, bool paths, hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>(a.n_items) * a.h_v);
  if (paths)
    gdn_d128_kernel<true><<<grid, 64 * NW, 0, stream>>>(a);
  else
    gdn_d128_kernel<false><<<grid, 64 * NW, 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace tg
