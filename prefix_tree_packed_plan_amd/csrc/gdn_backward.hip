// Backward of the chunked tree Gated DeltaNet for gfx950 (CDNA4).
//
// Method: "Tree Training" (arXiv 2511.00413) section 3.1 Eq. 6 (every
// token's output counted once), section 3.2 "SSM Layers (GDN)" Eq. 10 and
// appendix A.2: a segment starts from its parent's final state, so the
// gradient of that state is the sum over all children of the gradients of
// their start states, accumulated in fp32 (appendix B.5).  Segments run
// level by level from the deepest up; within a segment, 16-token chunks run
// from the last to the first.
//
// Chunk algebra (start state S0 [d_k, d_v], G the within-chunk cumulative
// sum of g, gamma = exp(G), delta_i = exp(G_last - G_i),
// Gamma_ij = exp(G_i - G_j) for j <= i):
//   forward   KK = K K^T, A = tril(diag(b) (KK o Gamma), -1), T = (I + A)^-1,
//             W0 = V - diag(gamma) K S0, R = diag(b) W0, U = T R,
//             P = tril(Q K^T o Gamma), O = scale (diag(gamma) Q S0 + P U),
//             S1 = gamma_last S0 + K^T diag(delta) U;
//   backward  (dOs = scale dO, dS1 the gradient of S1)
//             dU  = diag(delta) K dS1 + P^T dOs,  dR = T^T dU,
//             dA  = -tril(dR U^T, -1),            dP = tril(dOs U^T),
//             dV  = diag(b) dR,
//             dQ  = diag(gamma) dOs S0^T + (dP o Gamma) K,
//             dK  = diag(delta) U dS1^T - diag(gamma) dV S0^T + (dP o Gamma)^T Q
//                   + (dKK + dKK^T) K,  dKK = diag(b) (dA o Gamma),
//             db  = rowsum(dR o W0) + rowsum(dA o KK o Gamma),
//             dS0 = gamma_last dS1 + Q^T diag(gamma) dOs - K^T diag(gamma) dV,
//   and the gate gradient through G: with dGam = dP o QK + diag(b) (dA o KK)
//   and M = dGam o Gamma,
//             dG_i = gamma_i rowsum(Q S0 o dOs - dV o K S0)_i
//                    - delta_i rowsum(K dS1 o U)_i + rowsum(M)_i - colsum(M)_i,
//             dG_last += gamma_last sum(S0 o dS1) + sum_i delta_i rowsum(K dS1 o U)_i,
//             dg_t = sum_{i >= t} dG_i within the chunk.
// (dT = dU R^T and dA = -T^T dT T^T reduce to -dR U^T because T R = U.)
// (I + A)^-1 for the nilpotent A is the product
// (I + N)(I + N^2)(I + N^4)(I + N^8), N = -A: six 16x16 MFMA products.
//
// Launches: a prep kernel computes every chunk's T, KK and QK (state-free, all
// chunks at once); a checkpoint pass re-runs every segment forward from its
// parent's final state (the forward's `states`; all segments at once) and
// writes the start state of every kBwdCkpt-th chunk to the workspace (the
// states kernel below; at bf16 d = 128 the forward scan kernel's own
// checkpoint instantiation, which also writes the chunk tables, in place of
// prep); then launches level by level, deepest first, walk each segment's
// chunks backwards, re-running the chunks between two checkpoints forward
// when they reach them.  With two value heads per q/k head, the first head of
// each pair stores its part of dq and dk and the second, one launch later,
// adds to it (see the level loop of tree_gdn_scan_backward).  Work
// item: one segment and one value head per work-group of d/16 waves; wave w
// owns column tile w (16 columns) of every [16, d] chunk tensor and of the
// state gradient dS, which stays in MFMA accumulator registers across the
// segment.
//
// MFMA: for bf16 inputs the dense [16, d] x [d, d] products run on
// v_mfma_f32_16x16x32_bf16 with each fp32 operand carried as hi + lo bf16
// (q, k and dO are exact in bf16); the [16, 16] products, the inverse and
// every product for fp32 inputs run on v_mfma_f32_16x16x4_f32.
// Lane l = 16 h + i (h = l / 16) holds accumulator rows 4h + r, column i.
// A 16-deep contraction is four MFMAs; in step s lane l supplies index
// 4h + s of the contraction, so an accumulator tile is the B operand of a
// product that contracts its rows, and the accumulator tile of X^T is the A
// operand of a product with X on the left.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "../../include/tree_gdn.h"
#include "chunk_mfma.hpp"
#include "launch.hpp"

namespace tg {
namespace {

using namespace chunk;

template <int D>
struct BwdSmem {
  static constexpr int S = D + 4;  // row stride (floats) of the [16, d] and [d, d] tables
  static constexpr int NW = D / 16;
  // Small tables first and dS1 last: every address below stays within the
  // 64 KiB reach of an LDS instruction's offset from one base register.
  alignas(16) float g[L];
  alignas(16) float b[L];
  alignas(16) float gl[NW][4];          // per-wave partial sum(S0 o dS1)
  alignas(16) float rows[NW][3][L];     // per-wave partial row sums
  alignas(16) float m[3][L * 17];       // M, M^T and dA o KK o Gamma
  // Per-wave 16x16 partials (dR U^T, dOs U^T): part in the lanes'
  // accumulator order (lane l's 4 values at 4l), part_t the transpose in the
  // same order, so that either orientation is one 16-byte read per lane.
  alignas(16) float part[NW][2][L * L];
  alignas(16) float part_t[NW][2][L * L];
  alignas(16) float q[L * S];
  alignas(16) float k[L * S];
  alignas(16) float o[L * S];  // scale * dO
  alignas(16) float u[L * S];
  alignas(16) float r[L * S];  // dR
  alignas(16) float ds[D * S];  // dS1
};

// T = (I + A)^-1 and T^T as accumulator tiles from the lane's KK tile.
// A[row][col] = b_row Gamma[row][col] KK[row][col] for row > col.
__device__ __forceinline__ void solve(const f32x4 kk, const Gates& s, int h4, int i16, f32x4& T, f32x4& Tt) {
  f32x4 N, Nt, I;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int row = 4 * h4 + r;
    N[r] = row > i16 ? -s.bet[r] * s.Gm[r] * kk[r] : 0.f;
    Nt[r] = i16 > row ? -s.bet_c * s.Gmt[r] * kk[r] : 0.f;  // N[col][row]; KK is symmetric
    I[r] = row == i16 ? 1.f : 0.f;
  }
  // Every factor is a polynomial in N, so all of them commute; X Y takes
  // X^T's tile as the A operand, (X Y)^T = Y^T X^T takes Y's tile.
  const f32x4 N2 = mm(Nt, N, z4()), N2t = mm(N, Nt, z4());
  const f32x4 N4 = mm(N2t, N2, z4()), N4t = mm(N2, N2t, z4());
  const f32x4 N8 = mm(N4t, N4, z4());
  const f32x4 X1 = I + N, X1t = I + Nt;
  const f32x4 X2 = mm(X1t, N2, X1), X2t = mm(N2, X1t, X1t);
  const f32x4 X3 = mm(X2t, N4, X2), X3t = mm(N4, X2t, X2t);
  T = mm(X3t, N8, X3);
  Tt = mm(N8, X3t, X3t);  // (X3 N8)^T = N8^T X3^T; N8^T's A operand is N8's tile
}

// One chunk of the forward recurrence on a work-group's state: St (this
// wave's 16 columns of S0, as row tiles) becomes S1 = gamma_last S0 +
// K^T diag(delta) T diag(b) (V - diag(gamma) K S0).  sk, sg, sb: the chunk's
// K rows (row stride D + 4), g and beta, staged in LDS; Tt: the lane's tile of
// T^T; vc: the lane's V values (rows 4 h4 + 0..3 of its column), zero past
// the segment end.  The states kernel and the level kernel's re-run of the
// chunks after a checkpoint both step the state here, so where the states
// kernel takes the checkpoints the re-run start states are bitwise its own.
// (At bf16 d = 128 the checkpoints come from the forward scan kernel, whose
// 32-token chunks round differently; the re-run starts from them.)
template <int D, bool F32IN>
__device__ __forceinline__ void fwd_chunk_state(f32x4 (&St)[D / 16], const float* sk, const float* sg, const float* sb,
                                                const f32x4 Tt, const f32x4 vc, const uint2 negI, int h4, int i16) {
  constexpr int NT = D / 16;
  constexpr int S = D + 4;
  const Gates gt = make_gates(sg, sb, h4, i16);
  f32x4 ks = z4();
  if constexpr (F32IN) {
#pragma unroll
    for (int rt = 0; rt < NT; ++rt) ks = mm(ld4(&sk[i16 * S + 16 * rt + 4 * h4]), St[rt], ks);
  } else {
#pragma unroll
    for (int m = 0; m < NT / 2; ++m) {
      const uint4 ak = exact8(&sk[i16 * S + 32 * m + 4 * h4]);
      uint4 bh, bl;
      split8m(St[2 * m], St[2 * m + 1], negI, bh, bl);
      ks = mma32(ak, bl, mma32(ak, bh, ks));
    }
  }
  f32x4 R;
#pragma unroll
  for (int r = 0; r < 4; ++r) R[r] = gt.bet[r] * (vc[r] - gt.gam[r] * ks[r]);
  const f32x4 U = mm(Tt, R, z4());
  const f32x4 dU = gt.del * U;
  uint2 uh, ul;
  if constexpr (!F32IN) split4(dU, uh, ul);
#pragma unroll
  for (int rt = 0; rt < NT; ++rt) {
    f32x4 akt;
#pragma unroll
    for (int s = 0; s < 4; ++s) akt[s] = sk[(4 * h4 + s) * S + 16 * rt + i16];
    if constexpr (F32IN) {
      St[rt] = mm(akt, dU, gt.gam_last * St[rt]);
    } else {
      const uint2 a = pack4(akt);
      St[rt] = mma16b(a, ul, mma16b(a, uh, gt.gam_last * St[rt]));
    }
  }
}

// Forward re-run of the checkpoints: the start state of every kBwdCkpt-th
// chunk, for all segments at once (a segment starts from its parent's final
// state, which the forward already wrote), into the workspace as 16x16 tiles
// (row tile rt, column tile ct at (rt * NT + ct) * 256 floats), each in the
// lanes' accumulator order (lane l's 4 values at 4l): one 16-byte store per
// lane and tile.  Few registers, so two work-groups share a compute unit.
template <int D>
struct StatesSmem {
  static constexpr int S = D + 4;
  alignas(16) float g[L];
  alignas(16) float b[L];
  alignas(16) float k[L * S];
};

template <int D, bool F32IN>
__global__ __launch_bounds__(4 * D, 2) void gdn_bwd_states_kernel(ScanBwdArgs a) {
  constexpr int NT = D / 16;
  constexpr int S = D + 4;
  __shared__ StatesSmem<D> sm;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int h4 = lane >> 4;
  const int i16 = lane & 15;
  const uint2 negI = neg_identity(h4, i16);  // A operand of -I (split8m)
  const int col = 16 * w + i16;
  const int seg = blockIdx.x / a.h_v;
  const int h = blockIdx.x - seg * a.h_v;
  const int hq = h / (a.h_v / a.h_qk);
  const int t_beg = a.seg_off[seg], t_end = a.seg_off[seg + 1];
  const int nc = (t_end - t_beg + L - 1) / L;
  const size_t DD = size_t(D) * D;
  const size_t cstride = size_t(a.h_v) * DD;
  // Checkpoints: the start state of every kBwdCkpt-th chunk of the segment.
  float* hws = a.hws + (size_t(a.gck[seg]) * a.h_v + h) * DD;
  constexpr int TW = 3 * L * L;
  const size_t tstride = size_t(a.h_v) * TW;
  const float* tws = a.tws + (size_t(a.gchunk[seg]) * a.h_v + h) * TW;
  const int st_row = tid / (D / 4);
  const int st_col = 4 * (tid % (D / 4));
  auto load_tile = [&](const float* p, f32x4 (&x)[NT]) {
#pragma unroll
    for (int rt = 0; rt < NT; ++rt)
#pragma unroll
      for (int r = 0; r < 4; ++r) x[rt][r] = p[size_t(16 * rt + 4 * h4 + r) * D + col];
  };
  auto store_ws = [&](float* p, const f32x4 (&x)[NT]) {
#pragma unroll
    for (int rt = 0; rt < NT; ++rt)
      __builtin_nontemporal_store(x[rt], reinterpret_cast<f32x4*>(p + (rt * NT + w) * 256 + 4 * lane));
  };

  {
    f32x4 St[NT];
    const int par = a.parent[seg];
    const float* src = par >= 0 ? a.states + (size_t(par) * a.h_v + h) * DD
                                : (a.init ? a.init + (size_t(a.root_idx[seg]) * a.h_v + h) * DD : nullptr);
    if (src) {
      load_tile(src, St);
    } else {
#pragma unroll
      for (int rt = 0; rt < NT; ++rt) St[rt] = z4();
    }
    // Inputs and T^T of chunk c in registers, fetched one chunk ahead as raw
    // words from rows clamped into the chunk, unconditionally; the conversion
    // and the zeroing of rows past the segment end wait for the use.  (Loads
    // converted where they are issued made the compiler wait for each at once,
    // and with it for the chunk-state stores issued just before.)
    using KRaw = typename std::conditional<F32IN, f32x4, uint2>::type;
    using VRaw = typename std::conditional<F32IN, float, uint16_t>::type;
    KRaw kraw;
    VRaw vraw[4];
    f32x4 Ttn;
    float graw = 0.f, braw = 0.f;
    int nf = 0;  // rows of the fetched chunk
    auto fetch = [&](int c) {
      const int t0 = t_beg + c * L;
      nf = min(L, t_end - t0);
      kraw = *reinterpret_cast<const KRaw*>(static_cast<const VRaw*>(a.k) +
                                            (size_t(t0 + min(st_row, nf - 1)) * a.h_qk + hq) * D + st_col);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 4 * h4 + r;
        vraw[r] = static_cast<const VRaw*>(a.v)[(size_t(t0 + min(row, nf - 1)) * a.h_v + h) * D + col];
        Ttn[r] = tws[c * tstride + i16 * L + row];
      }
      if (tid < L) {
        const size_t gi = size_t(t0 + min(tid, nf - 1)) * a.h_v + h;
        graw = a.g[gi];
        braw = a.beta[gi];
      }
    };
    fetch(0);
    // The chunks after the last checkpoint are re-run by the level kernel.
    const int c_last = ((nc - 1) / kBwdCkpt) * kBwdCkpt;
    for (int c = 0; c <= c_last; ++c) {
      if (c % kBwdCkpt == 0) store_ws(hws + (c / kBwdCkpt) * cstride, St);
      if (c == c_last) break;
      f32x4 kv, vc;
      if constexpr (F32IN) {
        kv = kraw;
#pragma unroll
        for (int r = 0; r < 4; ++r) vc[r] = vraw[r];
      } else {
        kv = f32x4{__uint_as_float(kraw.x << 16), __uint_as_float(kraw.x & 0xffff0000u),
                   __uint_as_float(kraw.y << 16), __uint_as_float(kraw.y & 0xffff0000u)};
#pragma unroll
        for (int r = 0; r < 4; ++r) vc[r] = __uint_as_float(uint32_t(vraw[r]) << 16);
      }
      if (st_row >= nf) kv = z4();
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (4 * h4 + r >= nf) vc[r] = 0.f;
      *reinterpret_cast<f32x4*>(&sm.k[st_row * S + st_col]) = kv;
      if (tid < L) {
        sm.g[tid] = tid < nf ? graw : 0.f;
        sm.b[tid] = tid < nf ? braw : 0.f;
      }
      const f32x4 Tt = Ttn;
      __syncthreads();
      if (c + 1 < nc) fetch(c + 1);
      fwd_chunk_state<D, F32IN>(St, sm.k, sm.g, sm.b, Tt, vc, negI, h4, i16);
      __syncthreads();
    }
  }

}

template <int D, bool F32IN>
__global__ __launch_bounds__(4 * D) void gdn_bwd_kernel(ScanBwdArgs a) {
  constexpr int NT = D / 16;  // row tiles of the state = waves
  constexpr int S = D + 4;
  using SM = BwdSmem<D>;
  __shared__ SM sm;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // Wave-uniform; as a scalar at d = 128 (scalar LDS offsets leave room in
  // the vector registers there).
  const int w = D == 128 && !F32IN ? __builtin_amdgcn_readfirstlane(tid >> 6) : tid >> 6;
  const int h4 = lane >> 4;
  const int i16 = lane & 15;
  const int col = 16 * w + i16;

  // This launch's work items: group 0, then group 1 (see ScanBwdArgs).
  const int hv_n = a.h_v / a.head_step;
  const int g0 = a.n_items * hv_n;
  const bool grp1 = int(blockIdx.x) >= g0;
  const int bl = grp1 ? int(blockIdx.x) - g0 : int(blockIdx.x);
  const int item = bl / hv_n;
  const int h = (bl - item * hv_n) * a.head_step + (grp1 ? a.head_off2 : a.head_off);
  const bool dq_add = grp1 ? a.dq_accum2 : a.dq_accum;
  const int seg = (grp1 ? a.items2 : a.items)[item];
  const int hq = h / (a.h_v / a.h_qk);
  const int t_beg = a.seg_off[seg], t_end = a.seg_off[seg + 1];
  const int nc = (t_end - t_beg + L - 1) / L;
  const size_t DD = size_t(D) * D;
  const size_t cstride = size_t(a.h_v) * DD;  // between consecutive checkpoints in the workspace
  // The start states of chunks 0, kBwdCkpt, 2 kBwdCkpt, ... of the segment
  // (states kernel), and this work-group's scratch for the start states of
  // the chunks after one of them, re-run forward when the walk reaches them.
  const float* hws = a.hws + (size_t(a.gck[seg]) * a.h_v + h) * DD;
  float* const scr = a.scr + size_t(blockIdx.x) * (kBwdCkpt - 1) * DD;
  // T, KK and QK of every chunk (from the prep kernel), [16, 16] fp32 each.
  constexpr int TW = 3 * L * L;
  const size_t tstride = size_t(a.h_v) * TW;
  const float* tws = a.tws + (size_t(a.gchunk[seg]) * a.h_v + h) * TW;
  const int dq_head = a.dq_heads == a.h_v ? h : hq;

  // Staging: thread -> (row, 4 columns) of a [16, d] chunk tensor.
  const int st_row = tid / (D / 4);
  const int st_col = 4 * (tid % (D / 4));

  auto load_tile = [&](const float* p, f32x4 (&x)[NT]) {
#pragma unroll
    for (int rt = 0; rt < NT; ++rt)
#pragma unroll
      for (int r = 0; r < 4; ++r) x[rt][r] = p[size_t(16 * rt + 4 * h4 + r) * D + col];
  };
  auto store_tile = [&](float* p, const f32x4 (&x)[NT]) {
#pragma unroll
    for (int rt = 0; rt < NT; ++rt)
#pragma unroll
      for (int r = 0; r < 4; ++r) p[size_t(16 * rt + 4 * h4 + r) * D + col] = x[rt][r];
  };
  // Chunk start states, as the states kernel stores them.
  auto load_ws = [&](const float* p, f32x4 (&x)[NT]) {
#pragma unroll
    for (int rt = 0; rt < NT; ++rt) x[rt] = ld4(p + (rt * NT + w) * 256 + 4 * lane);
  };

  // ---- pass 2: chunks backwards ---------------------------------------------------
  f32x4 dS[NT];
#pragma unroll
  for (int rt = 0; rt < NT; ++rt) dS[rt] = z4();
  if (a.dstates) load_tile(a.dstates + (size_t(seg) * a.h_v + h) * DD, dS);
  for (int j = a.kid_off[seg]; j < a.kid_off[seg + 1]; ++j) {
    f32x4 x[NT];
    load_tile(a.dsseg + (size_t(a.kid[j]) * a.h_v + h) * DD, x);
#pragma unroll
    for (int rt = 0; rt < NT; ++rt) dS[rt] += x[rt];
  }

  // Chunk c's inputs, fetched one chunk ahead; its start state and its T /
  // T^T / KK / QK tiles are loaded at the chunk top (held a chunk ahead, they
  // push the kernel past its registers, and every spill reload waits for all
  // outstanding loads and stores).
  // The inputs come as raw words from rows clamped into the chunk, loaded
  // unconditionally; their conversion and the zeroing of rows past the
  // segment end wait for the chunk top.  (Loads converted where they are
  // issued made the compiler wait for each at once, and with it for the
  // gradient stores issued just before.)
  using KRaw = typename std::conditional<F32IN, f32x4, uint2>::type;
  using VRaw = typename std::conditional<F32IN, float, uint16_t>::type;
  KRaw qraw, kraw, oraw;
  VRaw vraw[4];
  float graw = 0.f, braw = 0.f;
  auto fetch = [&](int c) {
    // Lane-dependent offsets from an opaque copy of the thread id, recomputed
    // here rather than held (spilled) across the chunk: a spill reload waits
    // for every outstanding load and store.
    int tl = tid;
    asm volatile("" : "+v"(tl));
    const int ln = tl & 63, lh4 = ln >> 4, lcol = 16 * (tl >> 6) + (ln & 15);
    const int lrow = tl / (D / 4), lcol4 = 4 * (tl % (D / 4));
    const int t0 = t_beg + c * L;
    const int n = min(L, t_end - t0);
    const int srow = t0 + min(lrow, n - 1);
    const size_t qi = (size_t(srow) * a.h_qk + hq) * D + lcol4;
    const size_t oi = (size_t(srow) * a.h_v + h) * D + lcol4;
    qraw = *reinterpret_cast<const KRaw*>(static_cast<const VRaw*>(a.q) + qi);
    kraw = *reinterpret_cast<const KRaw*>(static_cast<const VRaw*>(a.k) + qi);
    oraw = *reinterpret_cast<const KRaw*>(static_cast<const VRaw*>(a.dout) + oi);
#pragma unroll
    for (int r = 0; r < 4; ++r)
      vraw[r] = static_cast<const VRaw*>(a.v)[(size_t(t0 + min(4 * lh4 + r, n - 1)) * a.h_v + h) * D + lcol];
    if (tl < L) {
      const size_t gi = size_t(t0 + min(tl, n - 1)) * a.h_v + h;
      graw = a.g[gi];
      braw = a.beta[gi];
    }
  };
  auto unpack = [](const KRaw x) -> f32x4 {
    if constexpr (F32IN)
      return x;
    else
      return f32x4{__uint_as_float(x.x << 16), __uint_as_float(x.x & 0xffff0000u), __uint_as_float(x.y << 16),
                   __uint_as_float(x.y & 0xffff0000u)};
  };
  // Forward re-run of chunks c0 .. c1 - 2 from the checkpoint ckp = S0(c0):
  // S0(c + 1) goes to scratch slot c - c0 (tile layout, as load_ws reads it),
  // stepped by the same code as the states kernel, so bitwise its values.
  auto rerun = [&](int c0, int c1, const float* ckp) {
    f32x4 St[NT];
    load_ws(ckp, St);
    // Inputs of chunk c, fetched one chunk ahead as raw words from rows
    // clamped into the chunk (converted and masked when staged), as in the
    // states kernel.  Every lane-dependent offset is recomputed from an
    // opaque copy of the thread id, so that none is held across the chunk
    // loop below, whose registers are full.
    KRaw kr;
    VRaw vr[4];
    f32x4 Ttn;
    float gr = 0.f, br = 0.f;
    auto load = [&](int c) {
      int tl = tid;
      asm volatile("" : "+v"(tl));
      const int ln = tl & 63, lh4 = ln >> 4, li16 = ln & 15, lcol = 16 * (tl >> 6) + li16;
      const int lrow = tl / (D / 4), lcol4 = 4 * (tl % (D / 4));
      const int t0 = t_beg + c * L;
      const int nf = min(L, t_end - t0);
      kr = *reinterpret_cast<const KRaw*>(static_cast<const VRaw*>(a.k) +
                                          (size_t(t0 + min(lrow, nf - 1)) * a.h_qk + hq) * D + lcol4);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 4 * lh4 + r;
        vr[r] = static_cast<const VRaw*>(a.v)[(size_t(t0 + min(row, nf - 1)) * a.h_v + h) * D + lcol];
        Ttn[r] = tws[c * tstride + li16 * L + row];
      }
      if (tl < L) {
        const size_t gi = size_t(t0 + min(tl, nf - 1)) * a.h_v + h;
        gr = a.g[gi];
        br = a.beta[gi];
      }
    };
    load(c0);
    for (int c = c0; c + 1 < c1; ++c) {
      int tl = tid;
      asm volatile("" : "+v"(tl));
      const int ln = tl & 63, lh4 = ln >> 4, li16 = ln & 15, lw = tl >> 6;
      const int lrow = tl / (D / 4), lcol4 = 4 * (tl % (D / 4));
      const int nf = min(L, t_end - (t_beg + c * L));
      f32x4 kv = unpack(kr), vc;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if constexpr (F32IN)
          vc[r] = vr[r];
        else
          vc[r] = __uint_as_float(uint32_t(vr[r]) << 16);
        if (4 * lh4 + r >= nf) vc[r] = 0.f;
      }
      if (lrow >= nf) kv = z4();
      *reinterpret_cast<f32x4*>(&sm.k[lrow * S + lcol4]) = kv;
      if (tl < L) {
        sm.g[tl] = tl < nf ? gr : 0.f;
        sm.b[tl] = tl < nf ? br : 0.f;
      }
      const f32x4 Tt = Ttn;
      __syncthreads();
      if (c + 2 < c1) load(c + 1);
      fwd_chunk_state<D, F32IN>(St, sm.k, sm.g, sm.b, Tt, vc, neg_identity(lh4, li16), lh4, li16);
      float* const p = scr + size_t(c - c0) * DD;
#pragma unroll
      for (int rt = 0; rt < NT; ++rt) *reinterpret_cast<f32x4*>(p + (rt * NT + lw) * 256 + 4 * ln) = St[rt];
      __syncthreads();  // K, g and beta of the chunk read
    }
  };

  fetch(nc - 1);

  for (int blk = (nc - 1) / kBwdCkpt; blk >= 0; --blk) {
  const int c0 = blk * kBwdCkpt;
  const int c1 = min(nc, c0 + kBwdCkpt);
  const float* const ckp = hws + blk * cstride;
  if (c1 - c0 > 1) rerun(c0, c1, ckp);
  for (int c = c1 - 1; c >= c0; --c) {
    const int t0 = t_beg + c * L;
    const int n = min(L, t_end - t0);
    const float* s0p = c == c0 ? ckp : scr + size_t(c - c0 - 1) * DD;
    f32x4 S0[NT];
    load_ws(s0p, S0);
    f32x4 T, Tt, kk, qk;
    {
      const float* tp = tws + c * tstride;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int e = (4 * h4 + r) * L + i16;
        T[r] = tp[e];
        Tt[r] = tp[i16 * L + 4 * h4 + r];
        kk[r] = tp[L * L + e];
        qk[r] = tp[2 * L * L + e];
      }
    }
    f32x4 vt;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float x;
      if constexpr (F32IN)
        x = vraw[r];
      else
        x = __uint_as_float(uint32_t(vraw[r]) << 16);
      vt[r] = 4 * h4 + r < n ? x : 0.f;
    }
    {
      const bool in = st_row < n;
      const f32x4 qv = in ? unpack(qraw) : z4(), kv = in ? unpack(kraw) : z4(), ov = in ? unpack(oraw) : z4();
      *reinterpret_cast<f32x4*>(&sm.q[st_row * S + st_col]) = qv;
      *reinterpret_cast<f32x4*>(&sm.k[st_row * S + st_col]) = kv;
      *reinterpret_cast<f32x4*>(&sm.o[st_row * S + st_col]) = F32IN ? ov * a.scale : ov;
    }
    if (tid < L) {
      sm.g[tid] = tid < n ? graw : 0.f;
      sm.b[tid] = tid < n ? braw : 0.f;
    }
    {
      float* const dsw = &sm.ds[4 * h4 * S + col];
#pragma unroll
      for (int rt = 0; rt < NT; ++rt)
#pragma unroll
        for (int r = 0; r < 4; ++r) dsw[(16 * rt + r) * S] = dS[rt][r];
    }
    __syncthreads();  // chunk tensors and dS1 staged

    const Gates gt = make_gates(sm.g, sm.b, h4, i16);
    f32x4 ks = z4(), qs = z4(), kd = z4();  // K S0, Q S0, K dS1 at column tile w
    if constexpr (F32IN) {
#pragma unroll
      for (int rt = 0; rt < NT; ++rt) {
        const f32x4 ak = ld4(&sm.k[i16 * S + 16 * rt + 4 * h4]);
        const f32x4 aq = ld4(&sm.q[i16 * S + 16 * rt + 4 * h4]);
        ks = mm(ak, S0[rt], ks);
        qs = mm(aq, S0[rt], qs);
        kd = mm(ak, dS[rt], kd);
      }
    } else {
      // -I for the MFMA split residual, from an opaque lane copy so that it
      // is not held across the chunk.
      int ln = lane;
      asm volatile("" : "+v"(ln));
      const uint2 negI = neg_identity(ln >> 4, ln & 15);
#pragma unroll
      for (int m = 0; m < NT / 2; ++m) {
        const uint4 ak = exact8(&sm.k[i16 * S + 32 * m + 4 * h4]);
        const uint4 aq = exact8(&sm.q[i16 * S + 32 * m + 4 * h4]);
        uint4 sh, sl, dh, dl;
        split8m(S0[2 * m], S0[2 * m + 1], negI, sh, sl);
        split8m(dS[2 * m], dS[2 * m + 1], negI, dh, dl);
        ks = mma32(ak, sl, mma32(ak, sh, ks));
        qs = mma32(aq, sl, mma32(aq, sh, qs));
        kd = mma32(ak, dl, mma32(ak, dh, kd));
      }
    }
    float glp = 0.f;
#pragma unroll
    for (int rt = 0; rt < NT; ++rt)
#pragma unroll
      for (int r = 0; r < 4; ++r) glp += S0[rt][r] * dS[rt][r];

    f32x4 P, W0, R, dOc;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = 4 * h4 + r;
      P[r] = row >= i16 ? qk[r] * gt.Gm[r] : 0.f;
      W0[r] = vt[r] - gt.gam[r] * ks[r];
      R[r] = gt.bet[r] * W0[r];
      dOc[r] = F32IN ? sm.o[row * S + col] : sm.o[row * S + col] * a.scale;
    }
    const f32x4 U = mm(Tt, R, z4());
    const f32x4 dU = mm(P, dOc, gt.del * kd);
    const f32x4 dR = mm(T, dU, z4());
    const f32x4 dV = gt.bet * dR;
    f32x4 pg, pd, pb;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = 4 * h4 + r;
      if (row < n) a.dv[(size_t(t0 + row) * a.h_v + h) * D + col] = dV[r];
      pg[r] = row_sum16(qs[r] * dOc[r] - dV[r] * ks[r]);
      pd[r] = row_sum16(kd[r] * U[r]);
      pb[r] = row_sum16(dR[r] * W0[r]);
      sm.u[row * S + col] = U[r];
      sm.r[row * S + col] = dR[r];
    }
    glp = row_sum16(glp);
    if (i16 == 0) {
      int ln = lane;  // opaque: see fetch
      asm volatile("" : "+v"(ln));
      const int lh4 = ln >> 4;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        sm.rows[w][0][4 * lh4 + r] = pg[r];
        sm.rows[w][1][4 * lh4 + r] = pd[r];
        sm.rows[w][2][4 * lh4 + r] = pb[r];
      }
      sm.gl[w][lh4] = glp;
    }
    // S0 rows 16w .. 16w+15 as the B operand of products with S0^T:
    // S0row[jt][e] = S0[16w + i][16jt + 4h + e], from tile (w, jt); issued
    // before the barrier so that the round trip overlaps it.
    f32x4 S0row[NT];
#pragma unroll
    for (int jt = 0; jt < NT; ++jt) {
      const float* tp = s0p + (w * NT + jt) * 256 + 4 * (16 * (i16 >> 2) + 4 * h4) + (i16 & 3);
#pragma unroll
      for (int e = 0; e < 4; ++e) S0row[jt][e] = tp[4 * e];
    }
    // The partial products below read only this wave's own columns of U and
    // dR, which it has just written: LDS serves one wave's accesses in order,
    // so only the compiler has to be kept from reordering them.
    asm volatile("" ::: "memory");

    {
      const f32x4 au = ld4(&sm.u[i16 * S + 16 * w + 4 * h4]);
      const f32x4 ar = ld4(&sm.r[i16 * S + 16 * w + 4 * h4]);
      const f32x4 ao = ld4(&sm.o[i16 * S + 16 * w + 4 * h4]);
      const f32x4 dap = mm(ar, au, z4());  // dR U^T over this wave's columns
      const f32x4 dpp_ = mm(ao, au, z4()) * (F32IN ? 1.f : a.scale);  // dOs U^T
      *reinterpret_cast<f32x4*>(&sm.part[w][0][4 * lane]) = dap;
      *reinterpret_cast<f32x4*>(&sm.part[w][1][4 * lane]) = dpp_;
      // Element (row 4h + r, column i) of the transpose is read by lane
      // 16 (i / 4) + 4h + r as its value i % 4.
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int e = 4 * (16 * (i16 >> 2) + 4 * h4 + r) + (i16 & 3);
        sm.part_t[w][0][e] = dap[r];
        sm.part_t[w][1][e] = dpp_[r];
      }
    }
    __syncthreads();  // dA, dP partials

    f32x4 dA, dAt, dP, dPt;
    {
      f32x4 x = z4(), xt = z4(), y = z4(), yt = z4();
#pragma unroll
      for (int v = 0; v < NT; ++v) {
        x += ld4(&sm.part[v][0][4 * lane]);
        xt += ld4(&sm.part_t[v][0][4 * lane]);
        y += ld4(&sm.part[v][1][4 * lane]);
        yt += ld4(&sm.part_t[v][1][4 * lane]);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 4 * h4 + r;
        dA[r] = row > i16 ? -x[r] : 0.f;
        dAt[r] = i16 > row ? -xt[r] : 0.f;
        dP[r] = row >= i16 ? y[r] : 0.f;
        dPt[r] = i16 >= row ? yt[r] : 0.f;
      }
    }
    const f32x4 dQKP = dP * gt.Gm, dQKPt = dPt * gt.Gmt;
    const f32x4 dKK = dA * gt.bet * gt.Gm, dKKt = dAt * gt.bet_c * gt.Gmt;
    if (w == 0) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 4 * h4 + r;
        const float mv = (dP[r] * qk[r] + dA[r] * gt.bet[r] * kk[r]) * gt.Gm[r];
        sm.m[0][row * 17 + i16] = mv;
        sm.m[1][i16 * 17 + row] = mv;
        sm.m[2][row * 17 + i16] = dA[r] * kk[r] * gt.Gm[r];
      }
    }
    f32x4 kc, qc;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      kc[r] = sm.k[(4 * h4 + r) * S + col];
      qc[r] = sm.q[(4 * h4 + r) * S + col];
    }
    f32x4 xo = z4(), xv = z4(), xu = z4();  // dOs S0^T, dV S0^T, diag(delta) U dS1^T
    const float* const dsr = &sm.ds[(16 * w + i16) * S + 4 * h4];
    if constexpr (F32IN) {
#pragma unroll
      for (int jt = 0; jt < NT; ++jt) {
        const int o4 = i16 * S + 16 * jt + 4 * h4;
        xo = mm(ld4(&sm.o[o4]), S0row[jt], xo);
        xv = mm(gt.bet_c * ld4(&sm.r[o4]), S0row[jt], xv);
        xu = mm(gt.del_c * ld4(&sm.u[o4]), ld4(dsr + 16 * jt), xu);
      }
    } else {
      int ln = lane;
      asm volatile("" : "+v"(ln));
      const uint2 negI = neg_identity(ln >> 4, ln & 15);
#pragma unroll
      for (int m = 0; m < NT / 2; ++m) {
        const int o4 = i16 * S + 32 * m + 4 * h4;
        uint4 sh, sl, dh, dl, vh, vl, uh, ul;
        split8m(S0row[2 * m], S0row[2 * m + 1], negI, sh, sl);
        split8m(ld4(dsr + 32 * m), ld4(dsr + 32 * m + 16), negI, dh, dl);
        split8(gt.bet_c * ld4(&sm.r[o4]), gt.bet_c * ld4(&sm.r[o4 + 16]), vh, vl);
        split8(gt.del_c * ld4(&sm.u[o4]), gt.del_c * ld4(&sm.u[o4 + 16]), uh, ul);
        const uint4 ao = exact8(&sm.o[o4]);
        xo = mma32(ao, sl, mma32(ao, sh, xo));
        xv = mma32(vl, sh, mma32(vh, sl, mma32(vh, sh, xv)));
        xu = mma32(ul, dh, mma32(uh, dl, mma32(uh, dh, xu)));
      }
      xo = xo * a.scale;
    }
    const f32x4 dQ = gt.gam * xo + mm(dQKPt, kc, z4());
    f32x4 dK = mm(dQKP, qc, z4());
    dK = mm(dKKt, kc, dK);
    dK = mm(dKK, kc, dK);
    dK = dK + xu - gt.gam * xv;
    // With two value heads per q/k head, the first stores its part of dq, dk
    // and the second, in a later launch, adds to it: a + b, deterministic and
    // equal to the ordered head-group sum.
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = 4 * h4 + r;
      if (row < n) {
        const size_t o = (size_t(t0 + row) * a.dq_heads + dq_head) * D + col;
        if (dq_add) {
          unsafeAtomicAdd(a.dq + o, dQ[r]);
          unsafeAtomicAdd(a.dk + o, dK[r]);
        } else {
          a.dq[o] = dQ[r];
          a.dk[o] = dK[r];
        }
      }
    }
    const f32x4 gdo = gt.gam * dOc, gdv = -(gt.gam * dV);
    uint4 gh, gl;  // [diag(gamma) dOs; -diag(gamma) dV] as one 32-deep B operand
    if constexpr (!F32IN) split8(gdo, gdv, gh, gl);
#pragma unroll
    for (int rt = 0; rt < NT; ++rt) {
      f32x4 aqt, akt;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        aqt[s] = sm.q[(4 * h4 + s) * S + 16 * rt + i16];
        akt[s] = sm.k[(4 * h4 + s) * S + 16 * rt + i16];
      }
      if constexpr (F32IN) {
        dS[rt] = mm(aqt, gdo, gt.gam_last * dS[rt]);
        dS[rt] = mm(akt, gdv, dS[rt]);
      } else {
        const uint4 a = cat(pack4(aqt), pack4(akt));  // [Q^T | K^T]
        dS[rt] = mma32(a, gl, mma32(a, gh, gt.gam_last * dS[rt]));
      }
    }
    if (c > 0) fetch(c - 1);
    __syncthreads();  // every read of this chunk's tables done

    if (w == 0 && lane < 3 * L) {  // gate gradients of token i = lane % 16
      // Lanes 16 p + i (p = 0, 1, 2) each gather one of the three per-token
      // partial sums over the waves and one row sum of a 16 x 16 table:
      // (d_gam, row i of M), (d_dl, row i of M^T), (db, row i of
      // dA o KK o Gamma).  Every sum keeps the order of a single lane's loop.
      const int i = lane & 15, p = lane >> 4;
      float s1 = 0.f, s2 = 0.f, gl = 0.f;
#pragma unroll
      for (int v = 0; v < NT; ++v) {
        s1 += sm.rows[v][p][i];
        gl += sm.gl[v][0] + sm.gl[v][1] + sm.gl[v][2] + sm.gl[v][3];
      }
      const float* const mp = &sm.m[p][i * 17];
#pragma unroll
      for (int j = 0; j < L; ++j) s2 += mp[j];
      const float d_dl = __shfl(s1, i + L, 64), db = __shfl(s1, i + 2 * L, 64);
      const float cs = __shfl(s2, i + L, 64), eb = __shfl(s2, i + 2 * L, 64);
      if (lane < L) {
        const float d_gam = s1, rs = s2;
        const float dl = gt.del_c * d_dl;
        const float dl_sum = row_sum16(dl);
        float dG = gt.gam_c * d_gam - dl + rs - cs;
        if (i == L - 1) dG += gt.gam_last * gl + dl_sum;
        // dg_t = sum of dG_i over i >= t within the chunk.
        float dg = 0.f;
#pragma unroll
        for (int j = 0; j < L; ++j) {
          const float x = __shfl(dG, j, 64);
          dg += j >= i ? x : 0.f;
        }
        if (i < n) {
          a.dg[size_t(t0 + i) * a.h_v + h] = dg;
          a.dbeta[size_t(t0 + i) * a.h_v + h] = db + eb;
        }
      }
    }
  }
  }

  // Start-state gradient: to the parent (summed there over its children) or
  // to the root's initial state.
  const int root = a.root_idx[seg];
  if (root < 0) {
    store_tile(a.dsseg + (size_t(seg) * a.h_v + h) * DD, dS);
  } else if (a.dinit) {
    store_tile(a.dinit + (size_t(root) * a.h_v + h) * DD, dS);
  }
}

// T = (I + A)^-1, KK and QK of every chunk and value head: state-free, so
// all chunks of the trie run in parallel before the level launches.  One
// wave per (chunk, value head); tokens past a segment's end are zero rows
// with g = beta = 0, as in the level kernel.
template <int D, bool F32IN>
__global__ __launch_bounds__(256) void gdn_bwd_prep_kernel(ScanBwdArgs a) {
  __shared__ float sg[4][L], sb[4][L];
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int h4 = lane >> 4;
  const int i16 = lane & 15;
  const int64_t item = int64_t(blockIdx.x) * 4 + w;
  const bool live = item < int64_t(a.n_chunks) * a.h_v;
  const int c = live ? int(item / a.h_v) : 0;
  const int h = live ? int(item - int64_t(c) * a.h_v) : 0;
  const int seg = a.chunk_seg[c];
  const int hq = h / (a.h_v / a.h_qk);
  const int t0 = a.seg_off[seg] + (c - a.gchunk[seg]) * L;
  const int n = live ? min(L, a.seg_off[seg + 1] - t0) : 0;
  if (lane < L) {
    const bool tin = lane < n;
    sg[w][lane] = tin ? a.g[size_t(t0 + lane) * a.h_v + h] : 0.f;
    sb[w][lane] = tin ? a.beta[size_t(t0 + lane) * a.h_v + h] : 0.f;
  }
  const bool rin = i16 < n;
  const size_t rbase = (size_t(t0 + (rin ? i16 : 0)) * a.h_qk + hq) * D;
  f32x4 kk = z4(), qk = z4();
  if constexpr (F32IN) {
#pragma unroll
    for (int m = 0; m < D / 16; ++m) {
      const f32x4 ak = rin ? load4<true>(a.k, rbase + 16 * m + 4 * h4) : z4();
      const f32x4 aq = rin ? load4<true>(a.q, rbase + 16 * m + 4 * h4) : z4();
      kk = mm(ak, ak, kk);
      qk = mm(aq, ak, qk);
    }
  } else {
#pragma unroll
    for (int m = 0; m < D / 32; ++m) {
      const size_t i0 = rbase + 32 * m + 4 * h4;
      const uint4 ak = rin ? cat(pack4(load4<false>(a.k, i0)), pack4(load4<false>(a.k, i0 + 16))) : make_uint4(0, 0, 0, 0);
      const uint4 aq = rin ? cat(pack4(load4<false>(a.q, i0)), pack4(load4<false>(a.q, i0 + 16))) : make_uint4(0, 0, 0, 0);
      kk = mma32(ak, ak, kk);  // bf16 x bf16 products are exact in fp32
      qk = mma32(aq, ak, qk);
    }
  }
  __syncthreads();
  const Gates gt = make_gates(sg[w], sb[w], h4, i16);
  f32x4 T, Tt;
  solve(kk, gt, h4, i16, T, Tt);
  if (live) {
    float* tp = a.tws + (size_t(c) * a.h_v + h) * (3 * L * L);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int e = (4 * h4 + r) * L + i16;
      tp[e] = T[r];
      tp[L * L + e] = kk[r];
      tp[2 * L * L + e] = qk[r];
    }
  }
}

// dst[t, j, :] = sum over the G value heads of q/k head j of src[t, j G + m, :],
// in head order.
__global__ void head_group_sum(const float* __restrict__ src, float* __restrict__ dst, int64_t n_out4, int G,
                               int d4) {
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= n_out4) return;
  const int64_t th = i / d4;  // (token, q/k head)
  const int c = int(i - th * d4);
  const f32x4* s = reinterpret_cast<const f32x4*>(src) + (th * G) * d4 + c;
  f32x4 acc = s[0];
  for (int m = 1; m < G; ++m) acc += s[int64_t(m) * d4];
  reinterpret_cast<f32x4*>(dst)[i] = acc;
}

template <int D, bool F32IN>
hipError_t launch_bwd_level(const ScanBwdArgs& a, hipStream_t stream) {
  const int n = (a.n_items + a.n_items2) * (a.h_v / a.head_step);
  if (n <= 0) return hipSuccess;
  gdn_bwd_kernel<D, F32IN><<<dim3(n), dim3(4 * D), 0, stream>>>(a);
  return hipGetLastError();
}

template <int D, bool F32IN>
hipError_t launch_prep(const ScanBwdArgs& a, bool tables, bool states, hipStream_t stream) {
  const int64_t items = int64_t(a.n_chunks) * a.h_v;
  if (items <= 0) return hipSuccess;
  if (tables) gdn_bwd_prep_kernel<D, F32IN><<<dim3(unsigned((items + 3) / 4)), dim3(256), 0, stream>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !states) return e;
  gdn_bwd_states_kernel<D, F32IN><<<dim3(unsigned(a.n_seg * a.h_v)), dim3(4 * D), 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace

bool scan_backward_supported(int d_k, int d_v, int dtype) {
  return d_k == d_v && (d_k == 32 || d_k == 64 || d_k == 128) && (dtype == TREE_DTYPE_BF16 || dtype == TREE_DTYPE_F32);
}

hipError_t launch_scan_backward_prep(const ScanBwdArgs& a, int d, int dtype, bool tables, bool states,
                                     hipStream_t stream) {
  const bool f32 = dtype == TREE_DTYPE_F32;
  switch (d) {
    case 32:
      return f32 ? launch_prep<32, true>(a, tables, states, stream) : launch_prep<32, false>(a, tables, states, stream);
    case 64:
      return f32 ? launch_prep<64, true>(a, tables, states, stream) : launch_prep<64, false>(a, tables, states, stream);
    case 128:
      return f32 ? launch_prep<128, true>(a, tables, states, stream)
                 : launch_prep<128, false>(a, tables, states, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_scan_backward_level(const ScanBwdArgs& a, int d, int dtype, hipStream_t stream) {
  const bool f32 = dtype == TREE_DTYPE_F32;
  switch (d) {
    case 32: return f32 ? launch_bwd_level<32, true>(a, stream) : launch_bwd_level<32, false>(a, stream);
    case 64: return f32 ? launch_bwd_level<64, true>(a, stream) : launch_bwd_level<64, false>(a, stream);
    case 128: return f32 ? launch_bwd_level<128, true>(a, stream) : launch_bwd_level<128, false>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_head_group_sum(const float* src, float* dst, int64_t n_tok, int h_qk, int group, int d,
                                 hipStream_t stream) {
  const int64_t n4 = n_tok * h_qk * (d / 4);
  if (n4 == 0) return hipSuccess;
  const int threads = 256;
  head_group_sum<<<dim3(unsigned((n4 + threads - 1) / threads)), dim3(threads), 0, stream>>>(src, dst, n4, group,
                                                                                              d / 4);
  return hipGetLastError();
}

}  // namespace tg
