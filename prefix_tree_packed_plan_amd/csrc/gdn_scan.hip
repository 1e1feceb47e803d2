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
//
// Work item: one (segment, value head) per work-group; the segment's chunks run
// in order with the fp32 state held in MFMA accumulator registers the whole
// time ("DFS keeps [the state] on-chip", "Tree Training" section 3.3).  The
// state leaves the chip only at the segment end, into the state of a parent
// that its children then read (one launch per trie level orders the two).
//
// Layout on the chip (d_v = 32 * NW, NW wavefronts):
//   wave w owns value columns [32w, 32w+32) of S, U and O, as 16x16 MFMA
//   accumulator tiles.  The accumulator layout of a 16x16 tile (lane l holds
//   rows 4(l/16)+r, r=0..3, of column l%16) doubles as the B operand of the
//   next product with the contraction index on the rows, so S, U and the
//   solve never leave registers.  For that, every MFMA here reads its k index
//   in the order kmap(h, j) = j<4 ? 4h+j : 16+4h+(j-4), h = l/16 -- a fixed
//   permutation applied to both operands, which leaves the product unchanged.
//
// Precision: q, k, v and the Gram matrices are exact in bf16 x bf16 -> fp32.
// Products that feed the state (K S0, the triangular solve, K^T U) carry the
// fp32 operand as hi + lo bf16 pairs (x = hi + lo to 2^-17), which keeps the
// segment states within ~1e-5 of fp32; the output path (Q S0, P U) uses the
// hi part only.  fp32 inputs are split the same way.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "../../include/tree_gdn.h"
#include "launch.hpp"

namespace tg {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int CH = 64;  // chunk length (tokens)

struct Pair4 {
  s16x4 a, b;
};

__device__ __forceinline__ short bf16_bits(float f) {
  return __builtin_bit_cast(short, static_cast<__bf16>(f));
}
__device__ __forceinline__ float bf16_float(short b) {
  return __uint_as_float(static_cast<uint32_t>(static_cast<uint16_t>(b)) << 16);
}

// x = hi + lo with hi = bf16(x), lo = bf16(x - hi).
__device__ __forceinline__ void split4(const f32x4 x, s16x4& hi, s16x4& lo) {
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const short h = bf16_bits(x[r]);
    hi[r] = h;
    lo[r] = bf16_bits(x[r] - bf16_float(h));
  }
}
__device__ __forceinline__ s16x4 hi4(const f32x4 x) {
  s16x4 h;
#pragma unroll
  for (int r = 0; r < 4; ++r) h[r] = bf16_bits(x[r]);
  return h;
}
__device__ __forceinline__ bf16x8 cat8(const s16x4 a, const s16x4 b) {
  return __builtin_bit_cast(bf16x8, Pair4{a, b});
}

__device__ __forceinline__ f32x4 mma32(const bf16x8 a, const bf16x8 b, const f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma16(const s16x4 a, const s16x4 b, const f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

// A-operand (or B-operand of a transposed matrix) of a 16x16x32 MFMA from a
// bf16 row-major LDS buffer: row `row`, columns col0 + kmap(h, 0..7).
__device__ __forceinline__ bf16x8 lds_a8(const short* buf, int stride, int row, int col0, int h) {
  const short* p = buf + row * stride + col0 + 4 * h;
  const uint2 x = *reinterpret_cast<const uint2*>(p);
  const uint2 y = *reinterpret_cast<const uint2*>(p + 16);
  return __builtin_bit_cast(bf16x8, make_uint4(x.x, x.y, y.x, y.y));
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

template <int DK, int DV, bool F32IN>
struct Smem {
  static constexpr int P = F32IN ? 2 : 1;  // bf16 parts per input element
  static constexpr int KS = DK + 8;        // row stride of Q, K (tokens x d_k)
  static constexpr int TS = CH + 8;        // row stride of K^T, V^T, P (x tokens)
  static constexpr int AS = CH + 4;        // row stride of A (fp32)
  // Every table is read with 8- or 16-byte LDS loads: keep them 16-aligned.
  alignas(16) short q[P][CH * KS];
  alignas(16) short k[P][CH * KS];
  alignas(16) short kt[P][DK * TS];
  alignas(16) float vt_f[F32IN ? DV * TS : 4];
  alignas(16) short vt_h[F32IN ? 8 : DV * TS];
  alignas(16) float a[CH * AS];      // strictly lower A (fp32)
  alignas(16) float tb[4][16 * 20];  // inverses of the 16x16 diagonal blocks of I + A
  alignas(16) short p[CH * TS];      // (Q K^T) o Gamma, lower incl. diagonal, bf16
  alignas(16) float gcum[CH];        // G
  alignas(16) float gam[CH];         // exp(G)
  alignas(16) float bet[CH];
  alignas(16) float graw[CH];
};

template <int DK, int DV, bool F32IN>
__global__ __launch_bounds__(64 * (DV / 32)) void gdn_level_kernel(ScanArgs args) {
  constexpr int NW = DV / 32;
  constexpr int NT = 64 * NW;
  constexpr int MT = DK / 16;  // d_k row tiles of the state
  constexpr int KK = DK / 32;  // 32-wide contraction steps over d_k
  using SM = Smem<DK, DV, F32IN>;
  constexpr int P = SM::P;
  __shared__ SM sm;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int h4 = lane >> 4;
  const int i16 = lane & 15;

  const int item = blockIdx.x / args.h_v;
  const int h = blockIdx.x - item * args.h_v;
  const int hq = h / (args.h_v / args.h_qk);
  const int seg = args.items[item];
  const int seg_beg = args.seg_off[seg];
  const int seg_end = args.seg_off[seg + 1];
  const int par = args.parent[seg];

  // The upper blocks of P that the output product reads are never written:
  // clear them once.
  for (int e = tid; e < 16 * 16; e += NT) {
    const int r = e >> 4, c = e & 15;
    sm.p[r * SM::TS + 16 + c] = 0;
    sm.p[(32 + r) * SM::TS + 48 + c] = 0;
  }

  // ---- initial state (parent's final state, or zero) ------------------------
  const size_t head_elems = static_cast<size_t>(DK) * DV;
  f32x4 S[MT][2];
  {
    const float* src = nullptr;
    if (par >= 0) {
      src = args.states ? args.states + (static_cast<size_t>(par) * args.h_v + h) * head_elems
                        : args.slots + (static_cast<size_t>(args.slot[par]) * args.h_v + h) * head_elems;
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          S[mt][nt][r] = src ? src[(16 * mt + 4 * h4 + r) * DV + 32 * w + 16 * nt + i16] : 0.f;
  }

  using TIn = typename std::conditional<F32IN, float, uint16_t>::type;
  const TIn* __restrict__ qg = static_cast<const TIn*>(args.q);
  const TIn* __restrict__ kg = static_cast<const TIn*>(args.k);
  const TIn* __restrict__ vg = static_cast<const TIn*>(args.v);
  TIn* __restrict__ og = static_cast<TIn*>(args.o);

  for (int t0 = seg_beg; t0 < seg_end; t0 += CH) {
    const int Lc = min(CH, seg_end - t0);
    __syncthreads();  // the previous chunk is done with the LDS buffers

    // ---- stage the chunk: Q, K row-major; K^T, V^T token-contiguous -------
    constexpr int EPV = 16 / sizeof(TIn);  // elements per 16-byte vector
    {
      constexpr int QV = DK / EPV;
      for (int e = tid; e < CH * QV; e += NT) {
        const int r = e / QV, cv = (e - r * QV) * EPV;
        float qf[EPV], kf[EPV];
        if (r < Lc) {
          const size_t base = (static_cast<size_t>(t0 + r) * args.h_qk + hq) * DK + cv;
          const uint4 qr = *reinterpret_cast<const uint4*>(qg + base);
          const uint4 kr = *reinterpret_cast<const uint4*>(kg + base);
          const uint32_t qw[4] = {qr.x, qr.y, qr.z, qr.w};
          const uint32_t kw[4] = {kr.x, kr.y, kr.z, kr.w};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            if constexpr (F32IN) {
              qf[i] = __uint_as_float(qw[i]);
              kf[i] = __uint_as_float(kw[i]);
            } else {
              qf[2 * i] = __uint_as_float(qw[i] << 16);
              qf[2 * i + 1] = __uint_as_float(qw[i] & 0xffff0000u);
              kf[2 * i] = __uint_as_float(kw[i] << 16);
              kf[2 * i + 1] = __uint_as_float(kw[i] & 0xffff0000u);
            }
          }
        } else {
#pragma unroll
          for (int i = 0; i < EPV; ++i) qf[i] = kf[i] = 0.f;
        }
#pragma unroll
        for (int i = 0; i < EPV; ++i) {
          const short qh = bf16_bits(qf[i]);
          const short kh = bf16_bits(kf[i]);
          sm.q[0][r * SM::KS + cv + i] = qh;
          sm.k[0][r * SM::KS + cv + i] = kh;
          sm.kt[0][(cv + i) * SM::TS + r] = kh;
          if constexpr (F32IN) {
            const short ql = bf16_bits(qf[i] - bf16_float(qh));
            const short kl = bf16_bits(kf[i] - bf16_float(kh));
            sm.q[P - 1][r * SM::KS + cv + i] = ql;
            sm.k[P - 1][r * SM::KS + cv + i] = kl;
            sm.kt[P - 1][(cv + i) * SM::TS + r] = kl;
          }
        }
      }
      constexpr int VV = DV / EPV;
      for (int e = tid; e < CH * VV; e += NT) {
        const int r = e / VV, cv = (e - r * VV) * EPV;
        uint4 vr = make_uint4(0, 0, 0, 0);
        if (r < Lc) {
          const size_t base = (static_cast<size_t>(t0 + r) * args.h_v + h) * DV + cv;
          vr = *reinterpret_cast<const uint4*>(vg + base);
        }
        const uint32_t vw[4] = {vr.x, vr.y, vr.z, vr.w};
        if constexpr (F32IN) {
#pragma unroll
          for (int i = 0; i < 4; ++i) sm.vt_f[(cv + i) * SM::TS + r] = __uint_as_float(vw[i]);
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            sm.vt_h[(cv + 2 * i) * SM::TS + r] = static_cast<short>(vw[i] & 0xffffu);
            sm.vt_h[(cv + 2 * i + 1) * SM::TS + r] = static_cast<short>(vw[i] >> 16);
          }
        }
      }
      for (int r = tid; r < CH; r += NT) {
        const bool ok = r < Lc;
        const size_t gi = static_cast<size_t>(t0 + r) * args.h_v + h;
        sm.graw[r] = ok ? args.g[gi] : 0.f;
        sm.bet[r] = ok ? args.beta[gi] : 0.f;
      }
    }
    __syncthreads();

    // ---- gate prefix: G = inclusive cumsum of g within the chunk ----------
    float G = sm.graw[lane];
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const float t = __shfl_up(G, off, 64);
      if (lane >= off) G += t;
    }
    if (w == 0) {
      sm.gcum[lane] = G;
      sm.gam[lane] = expf(G);
    }

    // ---- intra-chunk Grams: K K^T -> A (fp32), Q K^T -> P (bf16) ------------
    // 10 lower 16x16 blocks per matrix, dealt round-robin over the waves.
    for (int tau = w; tau < 20; tau += NW) {
      const int mat = tau / 10;  // 0: K K^T, 1: Q K^T
      const int t10 = tau - 10 * mat;
      const int rb = t10 < 1 ? 0 : t10 < 3 ? 1 : t10 < 6 ? 2 : 3;
      const int cb = t10 - (rb * (rb + 1)) / 2;
      const short* lhs = mat == 0 ? sm.k[0] : sm.q[0];
      f32x4 acc = zero4();
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        const bf16x8 a = lds_a8(lhs, SM::KS, 16 * rb + i16, 32 * kk, h4);
        const bf16x8 b = lds_a8(sm.k[0], SM::KS, 16 * cb + i16, 32 * kk, h4);
        acc = mma32(a, b, acc);
        if constexpr (F32IN) {
          const short* lhs_lo = mat == 0 ? sm.k[P - 1] : sm.q[P - 1];
          const bf16x8 al = lds_a8(lhs_lo, SM::KS, 16 * rb + i16, 32 * kk, h4);
          const bf16x8 bl = lds_a8(sm.k[P - 1], SM::KS, 16 * cb + i16, 32 * kk, h4);
          acc = mma32(al, b, acc);
          acc = mma32(a, bl, acc);
        }
      }
      const int j = 16 * cb + i16;
      const float Gj = __shfl(G, j, 64);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 16 * rb + 4 * h4 + r;
        const float Gi = __shfl(G, i, 64);
        if (mat == 0) {
          sm.a[i * SM::AS + j] = j < i ? sm.bet[i] * acc[r] * expf(Gi - Gj) : 0.f;
        } else {
          sm.p[i * SM::TS + j] = bf16_bits(j <= i ? acc[r] * expf(Gi - Gj) : 0.f);
        }
      }
    }
    __syncthreads();

    // ---- state-path products that do not need the solve: K S0, Q S0 --------
    f32x4 KS[4][2], QS[4][2];
#pragma unroll
    for (int mr = 0; mr < 4; ++mr)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) KS[mr][nt] = QS[mr][nt] = zero4();
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      bf16x8 sh[2], sl[2];
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        s16x4 h0, l0, h1, l1;
        split4(S[2 * kk][nt], h0, l0);
        split4(S[2 * kk + 1][nt], h1, l1);
        sh[nt] = cat8(h0, h1);
        sl[nt] = cat8(l0, l1);
      }
#pragma unroll
      for (int mr = 0; mr < 4; ++mr) {
        const bf16x8 ak = lds_a8(sm.k[0], SM::KS, 16 * mr + i16, 32 * kk, h4);
        const bf16x8 aq = lds_a8(sm.q[0], SM::KS, 16 * mr + i16, 32 * kk, h4);
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          KS[mr][nt] = mma32(ak, sh[nt], KS[mr][nt]);
          KS[mr][nt] = mma32(ak, sl[nt], KS[mr][nt]);
          QS[mr][nt] = mma32(aq, sh[nt], QS[mr][nt]);
        }
        if constexpr (F32IN) {
          const bf16x8 akl = lds_a8(sm.k[P - 1], SM::KS, 16 * mr + i16, 32 * kk, h4);
          const bf16x8 aql = lds_a8(sm.q[P - 1], SM::KS, 16 * mr + i16, 32 * kk, h4);
#pragma unroll
          for (int nt = 0; nt < 2; ++nt) {
            KS[mr][nt] = mma32(akl, sh[nt], KS[mr][nt]);
            QS[mr][nt] = mma32(aql, sh[nt], QS[mr][nt]);
            QS[mr][nt] = mma32(aq, sl[nt], QS[mr][nt]);
          }
        }
      }
    }

    // ---- inverses of the diagonal 16x16 blocks of (I + A) -------------------
    // Forward substitution in fp32, one column per lane.
    {
      constexpr int BPW = 4 / NW;  // diagonal blocks per wave
      const int b = w + NW * (h4 % BPW);
      const int jc = i16;
      const float* Ab = sm.a + (16 * b) * SM::AS + 16 * b;
      float t[16];
#pragma unroll
      for (int m = 0; m < 16; ++m) t[m] = m == jc ? 1.f : 0.f;
#pragma unroll
      for (int rr = 1; rr < 16; ++rr) {
        float acc = 0.f;
#pragma unroll
        for (int m = 0; m < rr; ++m) acc += Ab[rr * SM::AS + m] * t[m];
        if (rr > jc) t[rr] = -acc;
      }
      if (h4 < BPW) {
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) sm.tb[b][rr * 20 + jc] = t[rr];
      }
    }
    __syncthreads();

    // ---- right-hand side R = diag(b) V - diag(b gamma) K S0; O = gamma Q S0
    f32x4 R[4][2], O[4][2];
#pragma unroll
    for (int mr = 0; mr < 4; ++mr) {
      const int i0 = 16 * mr + 4 * h4;
      const f32x4 bv = *reinterpret_cast<const f32x4*>(&sm.bet[i0]);
      const f32x4 gv = *reinterpret_cast<const f32x4*>(&sm.gam[i0]);
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const int col = 32 * w + 16 * nt + i16;
        float vv[4];
        if constexpr (F32IN) {
          const f32x4 x = *reinterpret_cast<const f32x4*>(&sm.vt_f[col * SM::TS + i0]);
#pragma unroll
          for (int r = 0; r < 4; ++r) vv[r] = x[r];
        } else {
          const uint2 x = *reinterpret_cast<const uint2*>(&sm.vt_h[col * SM::TS + i0]);
          vv[0] = __uint_as_float(x.x << 16);
          vv[1] = __uint_as_float(x.x & 0xffff0000u);
          vv[2] = __uint_as_float(x.y << 16);
          vv[3] = __uint_as_float(x.y & 0xffff0000u);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          R[mr][nt][r] = bv[r] * (vv[r] - gv[r] * KS[mr][nt][r]);
          O[mr][nt][r] = gv[r] * QS[mr][nt][r];
        }
      }
    }

    // ---- blocked forward substitution (I + A) U = R, 16-row blocks ----------
    f32x4 U[4][2];
    s16x4 Uh[4][2], Ul[4][2];
#pragma unroll
    for (int bb = 0; bb < 4; ++bb) {
      f32x4 X[2] = {R[bb][0], R[bb][1]};
#pragma unroll
      for (int c = 0; c < bb; ++c) {
        const f32x4 av = *reinterpret_cast<const f32x4*>(&sm.a[(16 * bb + i16) * SM::AS + 16 * c + 4 * h4]);
        s16x4 ah, al;
        split4(-av, ah, al);
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          X[nt] = mma16(ah, Uh[c][nt], X[nt]);
          X[nt] = mma16(ah, Ul[c][nt], X[nt]);
          X[nt] = mma16(al, Uh[c][nt], X[nt]);
        }
      }
      const f32x4 tv = *reinterpret_cast<const f32x4*>(&sm.tb[bb][i16 * 20 + 4 * h4]);
      s16x4 th, tl;
      split4(tv, th, tl);
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        s16x4 xh, xl;
        split4(X[nt], xh, xl);
        f32x4 u = zero4();
        u = mma16(th, xh, u);
        u = mma16(th, xl, u);
        u = mma16(tl, xh, u);
        U[bb][nt] = u;
        split4(u, Uh[bb][nt], Ul[bb][nt]);
      }
    }

    // ---- O += P U, then store rows of this chunk ----------------------------
#pragma unroll
    for (int mr = 0; mr < 4; ++mr) {
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        if (kk == 1 && mr < 2) continue;
        const bf16x8 ap = lds_a8(sm.p, SM::TS, 16 * mr + i16, 32 * kk, h4);
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
          O[mr][nt] = mma32(ap, cat8(Uh[2 * kk][nt], Uh[2 * kk + 1][nt]), O[mr][nt]);
      }
    }
#pragma unroll
    for (int mr = 0; mr < 4; ++mr)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 16 * mr + 4 * h4 + r;
        if (i < Lc) {
          const size_t base = (static_cast<size_t>(t0 + i) * args.h_v + h) * DV + 32 * w + i16;
#pragma unroll
          for (int nt = 0; nt < 2; ++nt) {
            const float val = args.scale * O[mr][nt][r];
            if constexpr (F32IN)
              og[base + 16 * nt] = val;
            else
              og[base + 16 * nt] = static_cast<uint16_t>(bf16_bits(val));
          }
        }
      }

    // ---- state update S1 = gamma_L S0 + K^T (diag(exp(G_L - G)) U) ----------
    const float GL = sm.gcum[CH - 1];
    const float gL = sm.gam[CH - 1];
    s16x4 Wh[4][2], Wl[4][2];
#pragma unroll
    for (int bb = 0; bb < 4; ++bb) {
      const f32x4 gc = *reinterpret_cast<const f32x4*>(&sm.gcum[16 * bb + 4 * h4]);
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        f32x4 x;
#pragma unroll
        for (int r = 0; r < 4; ++r) x[r] = expf(GL - gc[r]) * U[bb][nt][r];
        split4(x, Wh[bb][nt], Wl[bb][nt]);
      }
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) S[mt][nt] *= gL;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const bf16x8 a = lds_a8(sm.kt[0], SM::TS, 16 * mt + i16, 32 * kk, h4);
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          S[mt][nt] = mma32(a, cat8(Wh[2 * kk][nt], Wh[2 * kk + 1][nt]), S[mt][nt]);
          S[mt][nt] = mma32(a, cat8(Wl[2 * kk][nt], Wl[2 * kk + 1][nt]), S[mt][nt]);
        }
        if constexpr (F32IN) {
          const bf16x8 al = lds_a8(sm.kt[P - 1], SM::TS, 16 * mt + i16, 32 * kk, h4);
#pragma unroll
          for (int nt = 0; nt < 2; ++nt)
            S[mt][nt] = mma32(al, cat8(Wh[2 * kk][nt], Wh[2 * kk + 1][nt]), S[mt][nt]);
        }
      }
    }
  }

  // ---- segment end: publish the state for the children / the caller --------
  float* dst = nullptr;
  if (args.states)
    dst = args.states + (static_cast<size_t>(seg) * args.h_v + h) * head_elems;
  else if (args.slot[seg] >= 0)
    dst = args.slots + (static_cast<size_t>(args.slot[seg]) * args.h_v + h) * head_elems;
  if (dst) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          dst[(16 * mt + 4 * h4 + r) * DV + 32 * w + 16 * nt + i16] = S[mt][nt][r];
  }
}

template <int DK, int DV, bool F32IN>
hipError_t launch_one(const ScanArgs& a, hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>(a.n_items) * a.h_v);
  gdn_level_kernel<DK, DV, F32IN><<<grid, 64 * (DV / 32), 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace

bool scan_supported(int d_k, int d_v, int dtype) {
  if (d_k != d_v) return false;
  if (dtype == TREE_DTYPE_F32) return d_k == 32;
  return d_k == 32 || d_k == 128;
}

hipError_t launch_scan_level(const ScanArgs& a, int d_k, int d_v, int dtype, hipStream_t stream) {
  const bool f32 = dtype == TREE_DTYPE_F32;
  if (d_k == 128 && d_v == 128 && !f32) return launch_one<128, 128, false>(a, stream);
  if (d_k == 32 && d_v == 32) return f32 ? launch_one<32, 32, true>(a, stream) : launch_one<32, 32, false>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace tg
