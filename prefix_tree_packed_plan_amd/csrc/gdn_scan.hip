// Chunked tree Gated DeltaNet forward for gfx950 (CDNA4).
//
// Method: "Tree Training" (arXiv 2511.00413) section 3.2 "SSM Layers (GDN)",
// Eq. 10 -- every segment starts from its parent's final state, a root from
// zero -- and appendix A.2, the chunked (WY/UT) form of the gated delta rule.
// Per value head, with a_t = exp(g_t):
//     S_t = a_t S_{t-1} (I - b_t k_t k_t^T) + b_t v_t k_t^T,   o_t = S_t q_t,
// kept as S [d_k, d_v] (the appendix's state orientation).
//
// Chunk algebra (64-token segment-local chunks, start state S0,
// G = within-chunk cumulative sum of g, gamma = exp(G)):
//     A_ij = b_i exp(G_i - G_j) k_i.k_j          (j < i, else 0)
//     (I + A) U = diag(b) V - diag(b gamma) K S0
//     O = scale * ( diag(gamma) Q S0 + ((Q K^T) o Gamma) U ),  Gamma_ij = exp(G_i - G_j), j <= i
//     S1 = gamma_L S0 + (diag(exp(G_L - G)) K)^T U
// Every exponent formed is G_i - G_j with j <= i, i.e. non-positive for g <= 0.
// Exponentials are taken base 2 on G * log2(e), one v_exp_f32 each.
//
// Work item: one segment and a group of G value heads that share a query/key
// head, per work-group; the segment's chunks run in order with every fp32
// state held in MFMA accumulator registers the whole time ("DFS keeps [the
// state] on-chip", "Tree Training" section 3.3).  The state leaves the chip
// only at the segment end, into the state its children read (one launch per
// trie level orders the two).  With G = 2 the group's q and k are read from
// HBM and staged once for both value heads, and two waves share each SIMD.
//
// Layout on the chip (d_v = 32 * NWV, G * NWV wavefronts):
//   wave w serves value head w / NWV and owns value columns [32c, 32c+32),
//   c = w % NWV, of S, U and O as 16x16 MFMA accumulator tiles.  The
//   accumulator layout of a 16x16 tile (lane l holds rows 4(l/16)+r, r=0..3,
//   of column l%16) doubles as the B operand of the next product with the
//   contraction index on the rows, so S, U and the solve never leave
//   registers.  For that, every 16x16x32 MFMA here reads its k index in the
//   order kmap(h, j) = j<4 ? 4h+j : 16+4h+(j-4), h = l/16 -- one fixed
//   permutation applied to both operands, which leaves the product unchanged.
//
// Precision: q, k, v and the Gram matrices are exact in bf16 x bf16 -> fp32.
// Products that feed the state (K S0, the triangular solve, K^T U) carry each
// fp32 operand as hi + lo bf16 (x = hi + lo to 2^-17 |x|; the lo x lo term is
// dropped), which keeps the segment states within ~1e-5 of fp32; for bf16
// inputs the output path (Q S0, P U) uses hi parts only.  fp32 inputs are
// split the same way, and their output path carries Q S0 and P U as hi + lo
// too, so fp32 outputs are accurate to fp32 level as well.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "../../include/tree_gdn.h"
#include "launch.hpp"

namespace tg {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int CH = 64;  // chunk length (tokens)
constexpr float kLog2e = 1.4426950408889634f;

// ---- bf16 packing --------------------------------------------------------------
// Two floats -> two bf16 (round to nearest even) in one word, `a` in the low half.
__device__ __forceinline__ uint32_t pk2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}
__device__ __forceinline__ float lo_f(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_f(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// x = hi + lo for 4 floats; hi and lo as 4 packed bf16 (2 words each).
__device__ __forceinline__ void split4(const f32x4 x, uint2& hi, uint2& lo) {
  const uint32_t h0 = pk2(x[0], x[1]), h1 = pk2(x[2], x[3]);
  hi = make_uint2(h0, h1);
  lo = make_uint2(pk2(x[0] - lo_f(h0), x[1] - hi_f(h0)), pk2(x[2] - lo_f(h1), x[3] - hi_f(h1)));
}

// One float as one word: bf16 hi in the low half, bf16 lo in the high half.
__device__ __forceinline__ uint32_t split1(float x) {
  const uint32_t h = pk2(x, x);
  const uint32_t l = pk2(x - lo_f(h), 0.f);
  return (h & 0xffffu) | (l << 16);
}
// Four such words -> packed hi (2 words) and packed lo (2 words).
__device__ __forceinline__ void unpack4(const uint4 w, uint2& hi, uint2& lo) {
  hi = make_uint2((w.x & 0xffffu) | (w.y << 16), (w.z & 0xffffu) | (w.w << 16));
  lo = make_uint2((w.x >> 16) | (w.y & 0xffff0000u), (w.z >> 16) | (w.w & 0xffff0000u));
}

__device__ __forceinline__ uint4 cat(const uint2 a, const uint2 b) { return make_uint4(a.x, a.y, b.x, b.y); }

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
// Scheduling fence: nothing moves across it, which bounds live ranges (and so
// register pressure) between the phases of a chunk.
__device__ __forceinline__ void fence() { __builtin_amdgcn_sched_barrier(0); }

// A operand (or the B operand of a transposed matrix) of a 16x16x32 MFMA from
// a bf16 row-major LDS table: row `row`, columns col0 + kmap(h, 0..7).
__device__ __forceinline__ uint4 lds_a8(const short* buf, int stride, int row, int col0, int h) {
  const short* p = buf + row * stride + col0 + 4 * h;
  const uint2 x = *reinterpret_cast<const uint2*>(p);
  const uint2 y = *reinterpret_cast<const uint2*>(p + 16);
  return make_uint4(x.x, x.y, y.x, y.y);
}

__device__ __forceinline__ uint32_t word(const uint4& v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

// Column e (0..7) of R consecutive bf16 rows, packed two tokens per word.
template <int R>
__device__ __forceinline__ void pack_column(const uint4 (&rows)[R], int e, uint32_t (&pk)[R / 2]) {
#pragma unroll
  for (int m = 0; m < R / 2; ++m) {
    const uint32_t a = word(rows[2 * m], e / 2), b = word(rows[2 * m + 1], e / 2);
    pk[m] = (e & 1) ? ((a >> 16) | (b & 0xffff0000u)) : ((a & 0xffffu) | (b << 16));
  }
}

// Gram tile tau (0..19) of a chunk: 0..3 the diagonal blocks of K K^T, 4..9
// its other lower blocks, 10..19 the lower blocks of Q K^T.
__device__ __forceinline__ void gram_tile(int tau, int& kk_mat, int& rb, int& cb) {
  if (tau < 4) {
    kk_mat = 1, rb = tau, cb = tau;
  } else if (tau < 10) {
    const int t = tau - 4;
    kk_mat = 1, rb = t < 1 ? 1 : t < 3 ? 2 : 3, cb = t - ((rb - 1) * rb) / 2;
  } else {
    const int t = tau - 10;
    kk_mat = 0, rb = t < 1 ? 0 : t < 3 ? 1 : t < 6 ? 2 : 3, cb = t - (rb * (rb + 1)) / 2;
  }
}

template <int DK, int DV, bool F32IN, int G>
struct Smem {
  static constexpr int P = F32IN ? 2 : 1;  // bf16 parts per q/k element
  static constexpr int KS = DK + 8;        // row stride of Q, K (tokens x d_k)
  static constexpr int TS = CH + 8;        // row stride of K^T, V^T, P (x tokens)
  static constexpr int AS = CH + 4;        // row stride of A
  // Every table is read with 8- or 16-byte LDS loads: keep them 16-aligned.
  alignas(16) short qk[2][P][CH * KS];     // Q, K row-major; output staging after the solve barrier
  alignas(16) short kt[P][DK * TS];        // K^T
  alignas(16) float vt_f[F32IN ? G * DV * TS : 4];
  alignas(16) short vt_h[F32IN ? 8 : G * DV * TS];
  // Lower 16x16 blocks of A: off-diagonal blocks hold -A as packed hi|lo bf16
  // words (the solve's operands), diagonal blocks hold A in fp32 (the
  // inverses' input).
  alignas(16) uint32_t a[G][CH * AS];
  alignas(16) uint32_t tb[G][4][16 * 20];  // (I + A_bb)^-1, packed hi|lo
  alignas(16) short p[G][CH * TS];         // (Q K^T) o Gamma, lower incl. diagonal, bf16 (hi part for fp32 inputs)
  alignas(16) short pl[F32IN ? G : 1][F32IN ? CH * TS : 8];  // its lo part (fp32 inputs)
  alignas(16) float g2[G][CH];             // G * log2(e)
  alignas(16) float gam[G][CH];            // exp(G)
  alignas(16) float bet[G][CH];
};

// PATHS = false: block item = one segment of a level, starting from its
// parent's state.  PATHS = true: block item = one rescan walk, the segments
// of a root-to-leaf path in order with the state carried in registers from
// one to the next; outputs and states are written only for the segments the
// walk owns.
template <int DK, int DV, bool F32IN, int G, bool PATHS>
__global__ __launch_bounds__(64 * G * (DV / 32)) void gdn_level_kernel(ScanArgs args) {
  constexpr int NWV = DV / 32;  // waves per value head
  constexpr int NW = G * NWV;
  constexpr int NT = 64 * NW;
  constexpr int MT = DK / 16;  // d_k row tiles of the state
  constexpr int KK = DK / 32;  // 32-wide contraction steps over d_k
  constexpr int BPW = 4 / NWV;  // diagonal blocks inverted per wave
  using SM = Smem<DK, DV, F32IN, G>;
  constexpr int P = SM::P;
  using TIn = typename std::conditional<F32IN, float, uint16_t>::type;
  __shared__ SM sm;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int vh = w / NWV;  // value head within the group
  const int cw = w % NWV;  // value-column block
  const int h4 = lane >> 4;
  const int i16 = lane & 15;

  const int n_grp = args.h_v / G;
  const int item = blockIdx.x / n_grp;
  const int grp = blockIdx.x - item * n_grp;
  const int h = grp * G + vh;
  const int hq = (grp * G) / (args.h_v / args.h_qk);
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
  const int par = args.parent[seg];

  // ---- initial state (parent's final state, or zero) ------------------------
  const size_t head_elems = static_cast<size_t>(DK) * DV;
  f32x4 S[MT][2];
  {
    const float* src = nullptr;
    if (par >= 0)
      src = args.states ? args.states + (static_cast<size_t>(par) * args.h_v + h) * head_elems
                        : args.slots + (static_cast<size_t>(args.slot[par]) * args.h_v + h) * head_elems;
    else if (args.init)  // a root with a caller-given initial state
      src = args.init + (static_cast<size_t>(args.root_idx[seg]) * args.h_v + h) * head_elems;
    if (src) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
          for (int r = 0; r < 4; ++r) S[mt][nt][r] = src[(16 * mt + 4 * h4 + r) * DV + 32 * cw + 16 * nt + i16];
    } else {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) S[mt][nt] = zero4();
    }
  }

  const TIn* __restrict__ qg = static_cast<const TIn*>(args.q);
  const TIn* __restrict__ kg = static_cast<const TIn*>(args.k);
  const TIn* __restrict__ vg = static_cast<const TIn*>(args.v);
  TIn* __restrict__ og = static_cast<TIn*>(args.o);

  // ---- chunk staging --------------------------------------------------------
  // Thread tid owns RQ consecutive token rows of one 16-byte column slice of
  // q and k, and RV rows of v (rows of the G value heads stacked), so every
  // global load is a full 16-byte vector (16 lanes cover 256 contiguous bytes)
  // and the transposed copies into K^T and V^T are runs of RQ (RV) tokens.
  // All loads of a chunk are issued before the first is consumed.
  constexpr int EPV = 16 / sizeof(TIn);  // elements per 16-byte vector
  constexpr int QV = DK / EPV;            // vectors per q/k row
  constexpr int VV = DV / EPV;
  constexpr int RQ = CH * QV / NT;        // q/k rows per thread
  constexpr int RV = G * CH * VV / NT;    // v rows per thread
  static_assert(CH * QV % NT == 0 && G * CH * VV % NT == 0 && RQ % 2 == 0 && RV % 2 == 0 &&
                    CH % RV == 0,
                "staging shape");
  const int cq = (tid % QV) * EPV, rq0 = (tid / QV) * RQ;
  const int cv = (tid % VV) * EPV, vrow0 = (tid / VV) * RV;
  const int vg0 = vrow0 / CH, rv0 = vrow0 % CH;  // value head and first row of this thread's v rows
  const int hv_load = grp * G + vg0;
  uint4 qr[RQ], kr[RQ], vr[RV];
  float gr = 0.f, br = 0.f;

  // Output staging: each wave's 64 x 32 block of O goes through LDS (inside
  // the Q/K table, free after the solve barrier) to leave as 16-byte stores.
  constexpr int EPO = 16 / sizeof(TIn);
  TIn* ost = reinterpret_cast<TIn*>(&sm.qk[0][0][0]) + w * CH * 32;
  static_assert(sizeof(TIn) * NW * CH * 32 <= sizeof(sm.qk), "output staging fits");

  for (;;) {
  const int seg_beg = args.seg_off[seg];
  const int seg_end = args.seg_off[seg + 1];
  for (int t0 = seg_beg; t0 < seg_end; t0 += CH) {
    const int Lc = min(CH, seg_end - t0);

    // -- issue the chunk's loads
#pragma unroll
    for (int i = 0; i < RQ; ++i) {
      const int r = rq0 + i;
      if (r < Lc) {
        const size_t base = (static_cast<size_t>(t0 + r) * args.h_qk + hq) * DK + cq;
        qr[i] = *reinterpret_cast<const uint4*>(qg + base);
        kr[i] = *reinterpret_cast<const uint4*>(kg + base);
      } else {
        qr[i] = kr[i] = make_uint4(0, 0, 0, 0);
      }
    }
#pragma unroll
    for (int i = 0; i < RV; ++i) {
      const int r = rv0 + i;
      vr[i] = r < Lc ? *reinterpret_cast<const uint4*>(vg + (static_cast<size_t>(t0 + r) * args.h_v + hv_load) * DV + cv)
                     : make_uint4(0, 0, 0, 0);
    }
    if (tid < G * CH) {  // wave w < G: lane r holds token r of value head grp*G + w
      const bool ok = lane < Lc;
      const size_t gi = static_cast<size_t>(t0 + lane) * args.h_v + grp * G + w;
      gr = ok ? args.g[gi] : 0.f;
      br = ok ? args.beta[gi] : 0.f;
    }

    __syncthreads();  // (A) the previous chunk is done with every LDS table

    // -- write the chunk into LDS
    if constexpr (!F32IN) {
#pragma unroll
      for (int i = 0; i < RQ; ++i) {
        *reinterpret_cast<uint4*>(&sm.qk[0][0][(rq0 + i) * SM::KS + cq]) = qr[i];
        *reinterpret_cast<uint4*>(&sm.qk[1][0][(rq0 + i) * SM::KS + cq]) = kr[i];
      }
#pragma unroll
      for (int e = 0; e < EPV; ++e) {
        uint32_t pk[RQ / 2];
        pack_column<RQ>(kr, e, pk);
        short* dst = &sm.kt[0][(cq + e) * SM::TS + rq0];
        if constexpr (RQ == 2) {
          *reinterpret_cast<uint32_t*>(dst) = pk[0];
        } else {
#pragma unroll
          for (int m = 0; m < RQ / 2; m += 2) *reinterpret_cast<uint2*>(dst + 2 * m) = make_uint2(pk[m], pk[m + 1]);
        }
      }
#pragma unroll
      for (int e = 0; e < EPV; ++e) {
        uint32_t pk[RV / 2];
        pack_column<RV>(vr, e, pk);
        short* dst = &sm.vt_h[(vg0 * DV + cv + e) * SM::TS + rv0];
        if constexpr (RV == 2) {
          *reinterpret_cast<uint32_t*>(dst) = pk[0];
        } else {
#pragma unroll
          for (int m = 0; m < RV / 2; m += 2) *reinterpret_cast<uint2*>(dst + 2 * m) = make_uint2(pk[m], pk[m + 1]);
        }
      }
    } else {
      // fp32 inputs: q and k go in as hi + lo bf16 parts, v stays fp32.
#pragma unroll
      for (int i = 0; i < RQ; ++i) {
#pragma unroll
        for (int e = 0; e < EPV; ++e) {
          const float qf = __uint_as_float(word(qr[i], e)), kf = __uint_as_float(word(kr[i], e));
          const uint32_t qs = split1(qf), ks = split1(kf);
          const int r = rq0 + i, c = cq + e;
          sm.qk[0][0][r * SM::KS + c] = static_cast<short>(qs & 0xffffu);
          sm.qk[1][0][r * SM::KS + c] = static_cast<short>(ks & 0xffffu);
          sm.kt[0][c * SM::TS + r] = static_cast<short>(ks & 0xffffu);
          sm.qk[0][P - 1][r * SM::KS + c] = static_cast<short>(qs >> 16);
          sm.qk[1][P - 1][r * SM::KS + c] = static_cast<short>(ks >> 16);
          sm.kt[P - 1][c * SM::TS + r] = static_cast<short>(ks >> 16);
        }
      }
#pragma unroll
      for (int i = 0; i < RV; ++i)
#pragma unroll
        for (int e = 0; e < EPV; ++e)
          sm.vt_f[(vg0 * DV + cv + e) * SM::TS + rv0 + i] = __uint_as_float(word(vr[i], e));
    }
    if (w < G) {  // gate prefix G = inclusive cumsum of g (wave prefix scan)
      float Gc = gr;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const float t = __shfl_up(Gc, off, 64);
        if (lane >= off) Gc += t;
      }
      const float g2 = Gc * kLog2e;
      sm.g2[w][lane] = g2;
      sm.gam[w][lane] = ex2(g2);
      sm.bet[w][lane] = br;
    }
    __syncthreads();  // (B) the chunk is staged

    const short* Qs = sm.qk[0][0];
    const short* Ks = sm.qk[1][0];

    // -- intra-chunk Grams: K K^T -> A, Q K^T -> P; 20 lower 16x16 tiles per
    //    value head, dealt over its NWV waves with each wave's diagonal blocks
    //    first, so the wave inverts them with no barrier.
#pragma unroll
    for (int it = 0; it < 20 / NWV; ++it) {
      int kk_mat, rb, cb;
      gram_tile(cw + NWV * it, kk_mat, rb, cb);
      const short* lhs = kk_mat ? Ks : Qs;
      f32x4 acc = zero4();
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        const uint4 a = lds_a8(lhs, SM::KS, 16 * rb + i16, 32 * kk, h4);
        const uint4 b = lds_a8(Ks, SM::KS, 16 * cb + i16, 32 * kk, h4);
        acc = mma32(a, b, acc);
        if constexpr (F32IN) {
          const uint4 al = lds_a8(kk_mat ? sm.qk[1][P - 1] : sm.qk[0][P - 1], SM::KS, 16 * rb + i16, 32 * kk, h4);
          const uint4 bl = lds_a8(sm.qk[1][P - 1], SM::KS, 16 * cb + i16, 32 * kk, h4);
          acc = mma32(al, b, acc);
          acc = mma32(a, bl, acc);
        }
      }
      const int j = 16 * cb + i16;
      const int i0 = 16 * rb + 4 * h4;
      const float g2j = sm.g2[vh][j];
      const f32x4 g2i = *reinterpret_cast<const f32x4*>(&sm.g2[vh][i0]);
      if (kk_mat) {
        const f32x4 bi = *reinterpret_cast<const f32x4*>(&sm.bet[vh][i0]);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = i0 + r;
          const float val = j < i ? bi[r] * acc[r] * ex2(g2i[r] - g2j) : 0.f;
          sm.a[vh][i * SM::AS + j] = rb == cb ? __float_as_uint(val) : split1(-val);
        }
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = i0 + r;
          const float val = j <= i ? acc[r] * ex2(g2i[r] - g2j) : 0.f;
          const uint32_t hw = pk2(val, 0.f);
          sm.p[vh][i * SM::TS + j] = static_cast<short>(hw & 0xffffu);
          if constexpr (F32IN) sm.pl[vh][i * SM::TS + j] = static_cast<short>(pk2(val - lo_f(hw), 0.f) & 0xffffu);
        }
      }
      if (it == BPW - 1) {
        // Inverse of I + A_bb for this wave's diagonal blocks: fp32 forward
        // substitution, lane = column, rows of A_bb read from LDS.
        const int b = cw + NWV * (h4 % BPW);
        const int jc = i16;
        const float* Ab = reinterpret_cast<const float*>(&sm.a[vh][(16 * b) * SM::AS + 16 * b]);
        float t[16];
#pragma unroll
        for (int m = 0; m < 16; ++m) t[m] = m == jc ? 1.f : 0.f;
#pragma unroll
        for (int rr = 1; rr < 16; ++rr) {
          f32x4 row[4];
#pragma unroll
          for (int q = 0; q < 4; ++q)
            if (4 * q < rr) row[q] = *reinterpret_cast<const f32x4*>(&Ab[rr * SM::AS + 4 * q]);
          float acc2 = 0.f;
#pragma unroll
          for (int m = 0; m < rr; ++m) acc2 += row[m / 4][m % 4] * t[m];
          t[rr] = rr > jc ? -acc2 : t[rr];
        }
        if (h4 < BPW) {
#pragma unroll
          for (int rr = 0; rr < 16; ++rr) sm.tb[vh][b][rr * 20 + jc] = split1(t[rr]);
        }
      }
      fence();
    }

    // -- state-path products that need no solve: K S0 and Q S0
    f32x4 R[4][2], O[4][2];
#pragma unroll
    for (int mr = 0; mr < 4; ++mr)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) R[mr][nt] = O[mr][nt] = zero4();
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      uint4 sh[2], sl[2];
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        uint2 h0, l0, h1, l1;
        split4(S[2 * kk][nt], h0, l0);
        split4(S[2 * kk + 1][nt], h1, l1);
        sh[nt] = cat(h0, h1);
        sl[nt] = cat(l0, l1);
      }
#pragma unroll
      for (int mr = 0; mr < 4; ++mr) {
        const uint4 ak = lds_a8(Ks, SM::KS, 16 * mr + i16, 32 * kk, h4);
        const uint4 aq = lds_a8(Qs, SM::KS, 16 * mr + i16, 32 * kk, h4);
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          R[mr][nt] = mma32(ak, sh[nt], R[mr][nt]);
          R[mr][nt] = mma32(ak, sl[nt], R[mr][nt]);
          O[mr][nt] = mma32(aq, sh[nt], O[mr][nt]);
        }
        if constexpr (F32IN) {
          const uint4 akl = lds_a8(sm.qk[1][P - 1], SM::KS, 16 * mr + i16, 32 * kk, h4);
          const uint4 aql = lds_a8(sm.qk[0][P - 1], SM::KS, 16 * mr + i16, 32 * kk, h4);
#pragma unroll
          for (int nt = 0; nt < 2; ++nt) {
            R[mr][nt] = mma32(akl, sh[nt], R[mr][nt]);
            O[mr][nt] = mma32(aql, sh[nt], O[mr][nt]);
            O[mr][nt] = mma32(aq, sl[nt], O[mr][nt]);
          }
        }
      }
      fence();
    }
    // -- R = diag(b) V - diag(b gamma) K S0 (in place of K S0); O = gamma Q S0
#pragma unroll
    for (int mr = 0; mr < 4; ++mr) {
      const int i0 = 16 * mr + 4 * h4;
      const f32x4 bv = *reinterpret_cast<const f32x4*>(&sm.bet[vh][i0]);
      const f32x4 gv = *reinterpret_cast<const f32x4*>(&sm.gam[vh][i0]);
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const int col = vh * DV + 32 * cw + 16 * nt + i16;
        f32x4 vv;
        if constexpr (F32IN) {
          vv = *reinterpret_cast<const f32x4*>(&sm.vt_f[col * SM::TS + i0]);
        } else {
          const uint2 x = *reinterpret_cast<const uint2*>(&sm.vt_h[col * SM::TS + i0]);
          vv = f32x4{lo_f(x.x), hi_f(x.x), lo_f(x.y), hi_f(x.y)};
        }
        R[mr][nt] = bv * (vv - gv * R[mr][nt]);
        O[mr][nt] = gv * O[mr][nt];
      }
    }
    __syncthreads();  // (D) A, P and the block inverses of every wave are in LDS

    // -- blocked forward substitution (I + A) U = R over 16-row blocks, right-
    //    looking: as soon as U_c = (I + A_cc)^-1 R_c is known it updates the
    //    later right-hand sides (R_b -= A_bc U_c), the outputs of rows at or
    //    after block c (O += P_{., c} U_c) and the state (S += K_c^T W_c with
    //    W_c = diag(exp(G_L - G)) U_c, S pre-scaled by gamma_L), so only the
    //    current block's U and W are ever live.
    const float g2L = sm.g2[vh][CH - 1];
    const float gL = sm.gam[vh][CH - 1];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) S[mt][nt] *= gL;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      uint2 th, tl;
      unpack4(*reinterpret_cast<const uint4*>(&sm.tb[vh][c][i16 * 20 + 4 * h4]), th, tl);
      const f32x4 g2r = *reinterpret_cast<const f32x4*>(&sm.g2[vh][16 * c + 4 * h4]);
      const f32x4 decay = f32x4{ex2(g2L - g2r[0]), ex2(g2L - g2r[1]), ex2(g2L - g2r[2]), ex2(g2L - g2r[3])};
      uint2 uh[2], ul[2], wh[2], wl[2];
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
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
        unpack4(*reinterpret_cast<const uint4*>(&sm.a[vh][(16 * b + i16) * SM::AS + 16 * c + 4 * h4]), ah, al);
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          R[b][nt] = mma16(ah, uh[nt], R[b][nt]);
          R[b][nt] = mma16(ah, ul[nt], R[b][nt]);
          R[b][nt] = mma16(al, uh[nt], R[b][nt]);
        }
      }
#pragma unroll
      for (int mr = c; mr < 4; ++mr) {
        const uint2 ap = *reinterpret_cast<const uint2*>(&sm.p[vh][(16 * mr + i16) * SM::TS + 16 * c + 4 * h4]);
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) O[mr][nt] = mma16(ap, uh[nt], O[mr][nt]);
        if constexpr (F32IN) {  // fp32 outputs: P and U as hi + lo as well
          const uint2 apl = *reinterpret_cast<const uint2*>(&sm.pl[vh][(16 * mr + i16) * SM::TS + 16 * c + 4 * h4]);
#pragma unroll
          for (int nt = 0; nt < 2; ++nt) {
            O[mr][nt] = mma16(ap, ul[nt], O[mr][nt]);
            O[mr][nt] = mma16(apl, uh[nt], O[mr][nt]);
          }
        }
      }
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const uint2 ak = *reinterpret_cast<const uint2*>(&sm.kt[0][(16 * mt + i16) * SM::TS + 16 * c + 4 * h4]);
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          S[mt][nt] = mma16(ak, wh[nt], S[mt][nt]);
          S[mt][nt] = mma16(ak, wl[nt], S[mt][nt]);
        }
        if constexpr (F32IN) {
          const uint2 akl = *reinterpret_cast<const uint2*>(&sm.kt[P - 1][(16 * mt + i16) * SM::TS + 16 * c + 4 * h4]);
#pragma unroll
          for (int nt = 0; nt < 2; ++nt) S[mt][nt] = mma16(akl, wh[nt], S[mt][nt]);
        }
      }
      fence();
    }

    // -- store O: through this wave's LDS staging block (rows of 32 values,
    //    16-byte chunks XOR-swizzled by row group) into 16-byte global stores
#pragma unroll
    for (int mr = 0; mr < 4; ++mr)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = 16 * mr + 4 * h4 + r;
          const int col = (16 * nt + i16) ^ (EPO * ((row >> 2) & 3));
          const float val = args.scale * O[mr][nt][r];
          if constexpr (F32IN)
            ost[row * 32 + col] = val;
          else
            ost[row * 32 + col] = static_cast<uint16_t>(pk2(val, 0.f) & 0xffffu);
        }
    constexpr int CPR = 32 / EPO;  // 16-byte chunks per row
#pragma unroll
    for (int it = 0; it < CPR; ++it) {
      const int ci = lane + 64 * it;
      const int row = ci / CPR, c = ci % CPR;
      const int col = (EPO * c) ^ (EPO * ((row >> 2) & 3));
      const uint4 val = *reinterpret_cast<const uint4*>(&ost[row * 32 + col]);
      if (own && row < Lc)
        *reinterpret_cast<uint4*>(og + (static_cast<size_t>(t0 + row) * args.h_v + h) * DV + 32 * cw + EPO * c) = val;
    }

  }

  // ---- segment end: publish the state for the children / the caller --------
  float* dst = nullptr;
  if (PATHS) {
    if (own) dst = args.states ? args.states + (static_cast<size_t>(seg) * args.h_v + h) * head_elems : nullptr;
  } else if (args.states) {
    dst = args.states + (static_cast<size_t>(seg) * args.h_v + h) * head_elems;
  } else if (args.slot[seg] >= 0) {
    dst = args.slots + (static_cast<size_t>(args.slot[seg]) * args.h_v + h) * head_elems;
  }
  if (dst) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int r = 0; r < 4; ++r) dst[(16 * mt + 4 * h4 + r) * DV + 32 * cw + 16 * nt + i16] = S[mt][nt][r];
  }
  if (!PATHS || ++wj == wend) break;
  const int e = args.walk[wj];  // the next segment of the walk
  seg = e < 0 ? ~e : e;
  own = e >= 0;
  }
}

template <int DK, int DV, bool F32IN, int G>
hipError_t launch_one(const ScanArgs& a, bool paths, hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>(a.n_items) * (a.h_v / G));
  if (paths)
    gdn_level_kernel<DK, DV, F32IN, G, true><<<grid, 64 * G * (DV / 32), 0, stream>>>(a);
  else
    gdn_level_kernel<DK, DV, F32IN, G, false><<<grid, 64 * G * (DV / 32), 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace

bool scan_supported(int d_k, int d_v, int dtype) {
  if (d_k != d_v) return false;
  if (dtype == TREE_DTYPE_F32) return d_k == 32 || d_k == 64;
  return d_k == 32 || d_k == 64 || d_k == 128;
}

hipError_t launch_scan(const ScanArgs& a, int d_k, int d_v, int dtype, bool paths, hipStream_t stream) {
  const bool f32 = dtype == TREE_DTYPE_F32;
  if (d_k == 128 && d_v == 128 && !f32) return launch_scan_d128(a, paths, stream);
  if (d_k == 64 && d_v == 64)
    return f32 ? launch_one<64, 64, true, 1>(a, paths, stream) : launch_one<64, 64, false, 1>(a, paths, stream);
  if (d_k == 32 && d_v == 32) {
    // Value heads 2j and 2j + 1 share a query/key head when the group size
    // h_v / h_qk is even: one work-group then serves both and stages their q
    // and k once.
    if ((a.h_v / a.h_qk) % 2 == 0)
      return f32 ? launch_one<32, 32, true, 2>(a, paths, stream) : launch_one<32, 32, false, 2>(a, paths, stream);
    return f32 ? launch_one<32, 32, true, 1>(a, paths, stream) : launch_one<32, 32, false, 1>(a, paths, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace tg
