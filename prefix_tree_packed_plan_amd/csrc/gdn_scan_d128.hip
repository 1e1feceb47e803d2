// Chunked tree Gated DeltaNet forward for bf16, d_k = d_v = 128, on gfx950.
//
// Same method and chunk algebra as gdn_scan.hip ("Tree Training", arXiv
// 2511.00413, section 3.2 Eq. 10 and appendix A.2):
//     A_ij = b_i exp(G_i - G_j) k_i.k_j  (j < i),  (I + A) U = diag(b) V - diag(b gamma) K S0,
//     O = scale (diag(gamma) Q S0 + ((Q K^T) o Gamma) U),  S1 = gamma_L S0 + (diag(exp(G_L - G)) K)^T U,
// with the same register layout of S, U and O (wave w serves value head
// w / 4 and value columns [32(w%4), +32) as 16x16 MFMA accumulator tiles),
// the same hi/lo split-bf16 state path and the same right-looking block
// solve.  What differs is the movement of data, built for CDNA4:
//
//   * q, k and v go from HBM straight into LDS with the asynchronous
//     global-to-LDS DMA (16 bytes per lane, no staging registers).  The next
//     chunk is fetched while the current one is being solved: k is double
//     buffered (the state update still reads the current chunk's k), q, v,
//     g and beta are single buffered (their last reader is before the
//     mid-chunk barrier).
//   * Tiles stay row-major (token x feature) in LDS.  The transposed
//     operands -- K^T for the state update, V in accumulator layout -- come
//     from the transposing LDS read ds_read_b64_tr_b16, which hands lane i of
//     each 16-lane group element i%4 of the 64-bit words read by lanes
//     4j + i/4, j = 0..3 (four rows of one column).  No transposed copies.
//   * Tiles are laid out in padded 4-row blocks with 16-byte chunks swizzled
//     by row (see toff), which spreads the access patterns here over the LDS
//     banks.  The DMA writes each lane's 16 bytes to consecutive slots of a
//     block, so the lane loads the global chunk that belongs in its slot.
//   * Output rows leave through a per-wave LDS staging block as 16-byte
//     stores that are issued one chunk later, after the next DMA has been
//     waited for, so no wait on loads ever waits on these stores.
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
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) void lds_void;
typedef const __attribute__((address_space(1))) void gbl_void;

constexpr int CH = 64;   // chunk length (tokens)
constexpr int D = 128;   // d_k = d_v
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ uint32_t pk2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}
__device__ __forceinline__ float lo_f(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_f(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ void split4(const f32x4 x, uint2& hi, uint2& lo) {
  const uint32_t h0 = pk2(x[0], x[1]), h1 = pk2(x[2], x[3]);
  hi = make_uint2(h0, h1);
  lo = make_uint2(pk2(x[0] - lo_f(h0), x[1] - hi_f(h0)), pk2(x[2] - lo_f(h1), x[3] - hi_f(h1)));
}
__device__ __forceinline__ uint32_t split1(float x) {
  const uint32_t h = pk2(x, x);
  const uint32_t l = pk2(x - lo_f(h), 0.f);
  return (h & 0xffffu) | (l << 16);
}
__device__ __forceinline__ void unpack4(const uint4 w, uint2& hi, uint2& lo) {
  hi = make_uint2((w.x & 0xffffu) | (w.y << 16), (w.z & 0xffffu) | (w.w << 16));
  lo = make_uint2((w.x >> 16) | (w.y & 0xffff0000u), (w.z >> 16) | (w.w & 0xffff0000u));
}
__device__ __forceinline__ f32x4 mma32(const uint4 a, const uint4 b, const f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma16(const uint2 a, const uint2 b, const f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a), __builtin_bit_cast(s16x4, b), c,
                                                   0, 0, 0);
}
__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }
__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }
// Sum over the 4 lanes of a quad (lanes 4k..4k+3), result in all four (DPP).
__device__ __forceinline__ float quad_sum(float x) {
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, true));  // [1,0,3,2]
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, true));  // [2,3,0,1]
  return x;
}

// LDS tile of 64 x 128 bf16 (token x feature): 16 blocks of 4 rows, each
// block 1 KB of data (one DMA instruction) plus 64 bytes of padding; row r4
// of a block holds its sixteen 16-byte chunks with chunk c in slot c ^ r4.
// The padding moves consecutive blocks 16 banks apart and the slot swizzle
// separates the 4 rows of a block, so 16 consecutive rows read at one
// column spread over all banks.  Every access below is one of a few lane
// base addresses plus a compile-time offset.
constexpr int TBLK = 4 * D + 32;  // block stride in elements (1088 bytes)
constexpr int TILE = 16 * TBLK;

__device__ __forceinline__ int toff(int row, int col) {
  const int r4 = row & 3;
  return (row >> 2) * TBLK + r4 * D + ((((col >> 3) & ~3) | (((col >> 3) & 3) ^ r4)) << 3) + (col & 7);
}
// A operand of a 16x16x32 MFMA (contraction over columns): row `row`,
// columns col0 + kmap(h, 0..7), kmap(h, j) = j<4 ? 4h+j : 16+4h+(j-4).
__device__ __forceinline__ uint4 tile_a8(const short* t, int row, int col0, int h) {
  const uint2 x = *reinterpret_cast<const uint2*>(t + toff(row, col0 + 4 * h));
  const uint2 y = *reinterpret_cast<const uint2*>(t + toff(row, col0 + 16 + 4 * h));
  return make_uint4(x.x, x.y, y.x, y.y);
}
// Transposing read: lane i of 16-lane group h gets rows row0 + 4h + 0..3 of
// column col0 + i of the tile (lane i reads row row0 + 4h + i/4, columns
// col0 + 4(i%4) .. +3).
__device__ __forceinline__ uint2 tile_tr(const short* t, int row0, int col0, int h, int i) {
  const short* p = t + toff(row0 + 4 * h + (i >> 2), col0 + 4 * (i & 3));
  return __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p)));
}

// Compact lower 16x16 blocks: block (rb, cb), cb <= rb, is number rb(rb+1)/2 + cb.
__device__ __forceinline__ int blk(int rb, int cb) { return (rb * (rb + 1)) / 2 + cb; }
// 16x16 fp32/word block, rows of 16 words, 4-word groups swizzled by row/4.
__device__ __forceinline__ int bsw(int r, int c) { return r * 16 + (c ^ (4 * ((r >> 2) & 3))); }

struct SmemD128 {
  alignas(16) short kb[2][TILE];          // K tiles (double buffered)
  alignas(16) short qb[TILE];             // Q tile
  alignas(16) short vb[TILE];             // V tile
  alignas(16) float gb[CH];               // raw g of the chunk
  alignas(16) float bb[CH];               // raw beta of the chunk
  alignas(16) uint32_t a[10][256];        // lower blocks of A: diagonal fp32, off-diagonal -A packed hi|lo
  alignas(16) uint32_t tb[4][256];        // (I + A_bb)^-1 packed hi|lo
  alignas(16) short p[10][16 * 16];       // lower blocks of (Q K^T) o Gamma, bf16
  alignas(16) float g2[CH];               // G * log2(e)
  alignas(16) float gam[CH];              // exp(G)
  alignas(16) float bet[CH];
  alignas(16) uint16_t ost[CH * D];       // output staging, CH x (D / NWV) per wave
};

// DMA of one 64 x 128 bf16 tile (rows tc .. tc+63 of a [N, H, 128] tensor at
// head hh; rows past the segment end repeat its last row) into an LDS tile.
// The tile is 16 blocks of 1 KB (4 rows); this wave issues blocks first,
// first + step, ...
__device__ __forceinline__ void dma_tile(const uint16_t* gsrc, int n_heads, int hh, int tc, int Ln, short* tile,
                                         int first, int step, int lane) {
  for (int b = first; b < 16; b += step) {
    const int row = 4 * b + (lane >> 4);
    const int slot = lane & 15;
    const int chunk = slot ^ (row & 3);
    const int src_row = tc + min(row, Ln - 1);
    const uint16_t* src = gsrc + (static_cast<size_t>(src_row) * n_heads + hh) * D + 8 * chunk;
    __builtin_amdgcn_global_load_lds((gbl_void*)src, (lds_void*)(tile + b * TBLK), 16, 0, 0);
  }
}

// One work-group per (segment, value head), NWV waves; wave cw owns value
// columns [NC cw, NC cw + NC), NC = 128 / NWV, as NC/16 accumulator tiles.
template <int NWV>
__global__ __launch_bounds__(64 * NWV) void gdn_d128_kernel(ScanArgs args) {
  constexpr int NC = D / NWV;    // value columns per wave
  constexpr int NTW = NC / 16;   // 16-column tiles per wave
  constexpr int MT = D / 16;     // d_k row tiles of the state
  constexpr int KK = D / 32;     // 32-wide contraction steps over d_k
  constexpr int TPW = (20 + NWV - 1) / NWV;  // Gram tiles per wave (at most)
  constexpr int CPR = NC / 8;    // 16-byte chunks per output row of a wave
  static_assert(NWV >= 4 && NWV <= 8 && NC % 16 == 0, "wave layout");
  __shared__ SmemD128 sm;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int cw = tid >> 6;
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
  const int col_w = NC * cw;

  // ---- initial state -------------------------------------------------------
  const size_t head_elems = static_cast<size_t>(D) * D;
  f32x4 S[MT][NTW];
  {
    const float* src = nullptr;
    if (par >= 0)
      src = args.states ? args.states + (static_cast<size_t>(par) * args.h_v + h) * head_elems
                        : args.slots + (static_cast<size_t>(args.slot[par]) * args.h_v + h) * head_elems;
    if (src) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
          for (int r = 0; r < 4; ++r) S[mt][nt][r] = src[(16 * mt + 4 * h4 + r) * D + col_w + 16 * nt + i16];
    } else {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt) S[mt][nt] = zero4();
    }
  }

  // Fetch the chunk at token tc (K into buffer kbuf): 48 tile blocks and two
  // gate rows, dealt over the waves.
  auto fetch = [&](int tc, int kbuf) {
    const int Ln = min(CH, seg_end - tc);
    dma_tile(kg, args.h_qk, hq, tc, Ln, sm.kb[kbuf], cw, NWV, lane);
    dma_tile(qg, args.h_qk, hq, tc, Ln, sm.qb, cw, NWV, lane);
    dma_tile(vg, args.h_v, h, tc, Ln, sm.vb, cw, NWV, lane);
    if (cw < 2) {
      const float* src = cw ? args.beta : args.g;
      const size_t gi = static_cast<size_t>(tc + min(lane, Ln - 1)) * args.h_v + h;
      __builtin_amdgcn_global_load_lds((gbl_void*)(src + gi), (lds_void*)(cw ? sm.bb : sm.gb), 4, 0, 0);
    }
  };

  // Store this wave's staged output rows (the chunk at token tc, Ln rows).
  uint16_t* st = sm.ost + cw * CH * NC;
  auto store_out = [&](int tc, int Ln) {
#pragma unroll
    for (int it = 0; it < CPR; ++it) {
      const int ci = lane + 64 * it;
      const int row = ci / CPR, c = ci % CPR;
      const uint4 val = *reinterpret_cast<const uint4*>(st + row * NC + 8 * (c ^ (((row >> 2) & 3) % CPR)));
      if (row < Ln)
        *reinterpret_cast<uint4*>(og + (static_cast<size_t>(tc + row) * args.h_v + h) * D + col_w + 8 * c) = val;
    }
  };

  fetch(seg_beg, 0);
  int kcur = 0;
  int prev_t0 = -1, prev_L = 0;

  for (int t0 = seg_beg; t0 < seg_end; t0 += CH) {
    const int Lc = min(CH, seg_end - t0);
    const short* Ks = sm.kb[kcur];
    const short* Qs = sm.qb;

    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's DMA of the chunk has landed
    __syncthreads();                                   // (A) ... and every other wave's

    // -- gate prefix (wave 0): G, exp(G), beta; zero past Lc
    if (cw == 0) {
      float Gc = lane < Lc ? sm.gb[lane] : 0.f;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const float t = __shfl_up(Gc, off, 64);
        if (lane >= off) Gc += t;
      }
      const float g2 = Gc * kLog2e;
      sm.g2[lane] = g2;
      sm.gam[lane] = ex2(g2);
      sm.bet[lane] = lane < Lc ? sm.bb[lane] : 0.f;
    }
    // -- last chunk's output rows leave now
    if (prev_t0 >= 0) store_out(prev_t0, prev_L);
    __syncthreads();  // (B) gates are in LDS

    // -- Grams: the 20 lower 16x16 tiles dealt over the waves; waves 0..3 take
    //    K K^T diagonal block cw first and invert it below.
    //    Tile order: 0..3 diag K K^T, 4..9 other K K^T, 10..19 Q K^T.
#pragma unroll
    for (int it = 0; it < TPW; ++it) {
      const int tau = cw + NWV * it;
      if (tau < 20) {
        int kk_mat, rb, cb;
        if (tau < 4) {
          kk_mat = 1, rb = tau, cb = tau;
        } else if (tau < 10) {
          const int t = tau - 4;
          kk_mat = 1, rb = t < 1 ? 1 : t < 3 ? 2 : 3, cb = t - ((rb - 1) * rb) / 2;
        } else {
          const int t = tau - 10;
          kk_mat = 0, rb = t < 1 ? 0 : t < 3 ? 1 : t < 6 ? 2 : 3, cb = t - (rb * (rb + 1)) / 2;
        }
        const short* lhs = kk_mat ? Ks : Qs;
        f32x4 acc = zero4();
#pragma unroll
        for (int kk = 0; kk < KK; ++kk)
          acc = mma32(tile_a8(lhs, 16 * rb + i16, 32 * kk, h4), tile_a8(Ks, 16 * cb + i16, 32 * kk, h4), acc);
        const int j = 16 * cb + i16;
        const int i0 = 16 * rb + 4 * h4;
        const float g2j = sm.g2[j];
        const f32x4 g2i = *reinterpret_cast<const f32x4*>(&sm.g2[i0]);
        if (kk_mat) {
          const f32x4 bi = *reinterpret_cast<const f32x4*>(&sm.bet[i0]);
          uint32_t* ab = sm.a[blk(rb, cb)];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int i = i0 + r;
            const float val = j < i ? bi[r] * acc[r] * ex2(g2i[r] - g2j) : 0.f;
            ab[bsw(4 * h4 + r, i16)] = rb == cb ? __float_as_uint(val) : split1(-val);
          }
        } else {
          short* pb = sm.p[blk(rb, cb)];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int i = i0 + r;
            const float val = j <= i ? args.scale * acc[r] * ex2(g2i[r] - g2j) : 0.f;
            pb[(4 * h4 + r) * 16 + i16] = static_cast<short>(pk2(val, 0.f) & 0xffffu);
          }
        }
      }
    }

    // -- inverse of diagonal block cw of (I + A), waves 0..3: fp32 forward
    //    substitution T = (I + A_bb)^-1 with all 64 lanes: lane (j, p) =
    //    (lane/4, lane%4) owns column j and the terms m = 4q + p of every row
    //    sum; a row step is <= 4 FMAs and a quad sum, so the 15-step
    //    dependent chain stays short, and the 36 entries a lane needs are
    //    loaded before the chain starts.
    if (cw < 4) {
      const float* Ab = reinterpret_cast<const float*>(sm.a[blk(cw, cw)]);
      const int jc = lane >> 2, ph = lane & 3;
      float arow[16][4];
#pragma unroll
      for (int rr = 1; rr < 16; ++rr)
#pragma unroll
        for (int q = 0; 4 * q < rr; ++q) arow[rr][q] = Ab[bsw(rr, 4 * q + ph)];
      float t[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) t[q] = 4 * q + ph == jc ? 1.f : 0.f;
#pragma unroll
      for (int rr = 1; rr < 16; ++rr) {
        // A_bb is strictly lower (zeros from the Gram tile), so the terms
        // with 4q + ph >= rr read zeros and need no mask.
        float part = 0.f;
#pragma unroll
        for (int q = 0; 4 * q < rr; ++q) part += arow[rr][q] * t[q];
        const float sum = quad_sum(part);
        const float val = rr > jc ? -sum : (rr == jc ? 1.f : 0.f);
        if ((rr & 3) == ph) t[rr >> 2] = val;
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) sm.tb[cw][bsw(4 * q + ph, jc)] = split1(t[q]);
    }

    // -- K S0 and Q S0
    f32x4 R[4][NTW], O[4][NTW];
#pragma unroll
    for (int mr = 0; mr < 4; ++mr)
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt) R[mr][nt] = O[mr][nt] = zero4();
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      uint4 sh[NTW], sl[NTW];
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt) {
        uint2 h0, l0, h1, l1;
        split4(S[2 * kk][nt], h0, l0);
        split4(S[2 * kk + 1][nt], h1, l1);
        sh[nt] = make_uint4(h0.x, h0.y, h1.x, h1.y);
        sl[nt] = make_uint4(l0.x, l0.y, l1.x, l1.y);
      }
#pragma unroll
      for (int mr = 0; mr < 4; ++mr) {
        const uint4 ak = tile_a8(Ks, 16 * mr + i16, 32 * kk, h4);
        const uint4 aq = tile_a8(Qs, 16 * mr + i16, 32 * kk, h4);
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt) {
          R[mr][nt] = mma32(ak, sh[nt], R[mr][nt]);
          R[mr][nt] = mma32(ak, sl[nt], R[mr][nt]);
          O[mr][nt] = mma32(aq, sh[nt], O[mr][nt]);
        }
      }
    }

    // -- R = diag(b) V - diag(b gamma) K S0; O = scale gamma Q S0
#pragma unroll
    for (int mr = 0; mr < 4; ++mr) {
      const int i0 = 16 * mr + 4 * h4;
      const f32x4 bv = *reinterpret_cast<const f32x4*>(&sm.bet[i0]);
      const f32x4 gv = *reinterpret_cast<const f32x4*>(&sm.gam[i0]);
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt) {
        const uint2 x = tile_tr(sm.vb, 16 * mr, col_w + 16 * nt, h4, i16);
        const f32x4 vv = f32x4{lo_f(x.x), hi_f(x.x), lo_f(x.y), hi_f(x.y)};
        R[mr][nt] = bv * (vv - gv * R[mr][nt]);
        O[mr][nt] = (args.scale * gv) * O[mr][nt];
      }
    }
    __syncthreads();  // (D) A, P and the block inverses of every wave are in LDS

    // -- fetch the next chunk while this one is solved
    if (t0 + CH < seg_end) fetch(t0 + CH, kcur ^ 1);

    // -- right-looking blocked forward substitution (I + A) U = R; each
    //    solved block updates the later right-hand sides, the outputs of its
    //    and later rows, and the state (pre-scaled by gamma_L).
    const float g2L = sm.g2[CH - 1];
    const float gL = sm.gam[CH - 1];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt) S[mt][nt] *= gL;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      uint2 th, tl;
      unpack4(*reinterpret_cast<const uint4*>(&sm.tb[c][bsw(i16, 4 * h4)]), th, tl);
      const f32x4 g2r = *reinterpret_cast<const f32x4*>(&sm.g2[16 * c + 4 * h4]);
      const f32x4 decay = f32x4{ex2(g2L - g2r[0]), ex2(g2L - g2r[1]), ex2(g2L - g2r[2]), ex2(g2L - g2r[3])};
      uint2 uh[NTW], ul[NTW], wh[NTW], wl[NTW];
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt) {
        uint2 xh, xl;
        split4(R[c][nt], xh, xl);
        f32x4 u = zero4();
        u = mma16(th, xh, u);
        u = mma16(th, xl, u);
        u = mma16(tl, xh, u);
        split4(u, uh[nt], ul[nt]);
        split4(decay * u, wh[nt], wl[nt]);
      }
#pragma unroll
      for (int b = c + 1; b < 4; ++b) {
        uint2 ah, al;
        unpack4(*reinterpret_cast<const uint4*>(&sm.a[blk(b, c)][bsw(i16, 4 * h4)]), ah, al);
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt) {
          R[b][nt] = mma16(ah, uh[nt], R[b][nt]);
          R[b][nt] = mma16(ah, ul[nt], R[b][nt]);
          R[b][nt] = mma16(al, uh[nt], R[b][nt]);
        }
      }
#pragma unroll
      for (int mr = c; mr < 4; ++mr) {
        const uint2 ap = *reinterpret_cast<const uint2*>(&sm.p[blk(mr, c)][i16 * 16 + 4 * h4]);
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt) O[mr][nt] = mma16(ap, uh[nt], O[mr][nt]);
      }
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const uint2 ak = tile_tr(Ks, 16 * c, 16 * mt, h4, i16);
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt) {
          S[mt][nt] = mma16(ak, wh[nt], S[mt][nt]);
          S[mt][nt] = mma16(ak, wl[nt], S[mt][nt]);
        }
      }
    }

    // -- stage this chunk's output rows (16-byte chunks swizzled by row
    //    group); they are stored during the next chunk
#pragma unroll
    for (int mr = 0; mr < 4; ++mr)
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = 16 * mr + 4 * h4 + r;
          const int col = 16 * nt + i16;
          st[row * NC + (((col >> 3) ^ (((row >> 2) & 3) % CPR)) << 3) + (col & 7)] =
              static_cast<uint16_t>(pk2(O[mr][nt][r], 0.f) & 0xffffu);
        }
    prev_t0 = t0;
    prev_L = Lc;
    kcur ^= 1;
  }
  store_out(prev_t0, prev_L);

  // ---- segment end: publish the state --------------------------------------
  float* dst = nullptr;
  if (args.states)
    dst = args.states + (static_cast<size_t>(seg) * args.h_v + h) * head_elems;
  else if (args.slot[seg] >= 0)
    dst = args.slots + (static_cast<size_t>(args.slot[seg]) * args.h_v + h) * head_elems;
  if (dst) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
        for (int r = 0; r < 4; ++r) dst[(16 * mt + 4 * h4 + r) * D + col_w + 16 * nt + i16] = S[mt][nt][r];
  }
}

}  // namespace

hipError_t launch_scan_d128(const ScanArgs& a, hipStream_t stream) {
  constexpr int NWV = 8;
  gdn_d128_kernel<NWV><<<dim3(static_cast<unsigned>(a.n_items) * a.h_v), 64 * NWV, 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace tg
