// Tree Mamba2 (SSD) forward with a forked state for gfx950 (CDNA4).
//
// Method: the tree-recurrence 0.1.0 project page ("How a tree runs": a fork
// starts each segment from its parent's final state; "Not yet": forking the
// Mamba2 state) and "Tree Training" section 3.1 Eq. 6 (the result equals
// the standalone forward of any path through a segment).  Per head h, with
// scalar decay rate A_h < 0, step dt_t >= 0 (after softplus), x_t [P], and
// B_t, C_t [N] of the head's group:
//     S_t = exp(dt_t A_h) S_{t-1} + dt_t B_t x_t^T,   y_t = S_t^T C_t + D_h x_t,
// S [N, P].  This is the gated delta rule without its erase term, so the
// chunk algebra is that of the GDN scan with T = I (16-token chunks, start
// state S0, G = cumulative sum of g = dt A, gamma = exp(G),
// delta_i = exp(G_last - G_i), Gamma_ij = exp(G_i - G_j) for j <= i):
//     U = diag(dt) X,   P = tril((C B^T) o Gamma),
//     Y = diag(gamma) C S0 + P U + X diag(D),
//     S1 = gamma_last S0 + B^T diag(delta) U.
// Padding rows of a partial chunk carry dt = 0, which leaves the state
// alone, as the pages' masked padding does.
//
// Schedule: one launch per trie level (the fork); a work-group per (segment,
// head), P/16 waves, wave w owning columns 16w..16w+15 of S, which stays in
// MFMA accumulator registers for the whole segment and leaves the chip only
// at the segment end, into the state its children read.
//
// Precision: for bf16 inputs the products with the state (C S0, B^T U) take
// the fp32 operand as hi + lo bf16 (two passes; B and C are exact); C B^T is
// exact; P U is fp32.  fp32 inputs use fp32 MFMA throughout.
#include <hip/hip_runtime.h>

#include "../../include/tree_gdn.h"
#include "chunk_mfma.hpp"
#include "launch.hpp"

namespace tg {
namespace {

using namespace chunk;

template <int N, int P>
struct SsdSmem {
  static constexpr int S = N + 4;  // row stride (floats)
  alignas(16) float g[L];   // dt A
  alignas(16) float b[L];   // dt
  alignas(16) float bm[L * S];  // B rows
  alignas(16) float cm[L * S];  // C rows
  alignas(16) float y[L * P];   // the chunk's outputs, stored as whole rows after the chunk
};

template <int N, int P, bool F32IN>
__global__ __launch_bounds__(4 * P, 2) void ssd_level_kernel(SsdArgs a) {
  constexpr int NT = N / 16;  // row tiles of the state
  constexpr int NTH = 4 * P;  // threads
  constexpr int S = N + 4;
  __shared__ SsdSmem<N, P> sm;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int h4 = lane >> 4;
  const int i16 = lane & 15;
  const int col = 16 * w + i16;

  const int item = blockIdx.x / a.n_heads;
  const int h = blockIdx.x - item * a.n_heads;
  const int seg = a.items[item];
  const int grp = h / (a.n_heads / a.n_groups);
  const int par = a.parent[seg];
  const size_t hs = size_t(N) * P;
  const float Ah = a.A[h];
  const float Dh = a.D ? a.D[h] : 0.f;

  f32x4 St[NT];
  {
    const float* src = nullptr;
    if (par >= 0)
      src = a.states ? a.states + (size_t(par) * a.n_heads + h) * hs
                     : a.slots + (size_t(a.slot[par]) * a.n_heads + h) * hs;
    else if (a.init)
      src = a.init + (size_t(a.root_idx[seg]) * a.n_heads + h) * hs;
#pragma unroll
    for (int rt = 0; rt < NT; ++rt)
#pragma unroll
      for (int r = 0; r < 4; ++r) St[rt][r] = src ? src[size_t(16 * rt + 4 * h4 + r) * P + col] : 0.f;
  }

  const int t_beg = a.seg_off[seg], t_end = a.seg_off[seg + 1];
  for (int t0 = t_beg; t0 < t_end; t0 += L) {
    const int n = min(L, t_end - t0);
    // -- stage B and C rows (4 elements per thread and step), dt and dt A
#pragma unroll
    for (int e = tid; e < 4 * N; e += NTH) {
      const int row = e / (N / 4), c4 = 4 * (e % (N / 4));
      const bool in = row < n;
      const size_t gi = (size_t(t0 + row) * a.n_groups + grp) * N + c4;
      *reinterpret_cast<f32x4*>(&sm.bm[row * S + c4]) = in ? load4<F32IN>(a.B, gi) : z4();
      *reinterpret_cast<f32x4*>(&sm.cm[row * S + c4]) = in ? load4<F32IN>(a.C, gi) : z4();
    }
    if (tid < L) {
      const float dt = tid < n ? a.dt[size_t(t0 + tid) * a.n_heads + h] : 0.f;
      sm.b[tid] = dt;
      sm.g[tid] = dt * Ah;
    }
    f32x4 xv;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = 4 * h4 + r;
      xv[r] = row < n ? load1<F32IN>(a.x, (size_t(t0 + row) * a.n_heads + h) * P + col) : 0.f;
    }
    __syncthreads();

    const Gates gt = make_gates(sm.g, sm.b, h4, i16);
    // C B^T is only needed transposed: Pt[row][col] = P[col][row].
    f32x4 qkt = z4(), cs = z4();
    if constexpr (F32IN) {
#pragma unroll
      for (int m = 0; m < NT; ++m) {
        const f32x4 ac = ld4(&sm.cm[i16 * S + 16 * m + 4 * h4]);
        const f32x4 ab = ld4(&sm.bm[i16 * S + 16 * m + 4 * h4]);
        qkt = mm(ab, ac, qkt);
        cs = mm(ac, St[m], cs);
      }
    } else {
#pragma unroll
      for (int m = 0; m < NT / 2; ++m) {
        const uint4 ac = exact8(&sm.cm[i16 * S + 32 * m + 4 * h4]);
        const uint4 ab = exact8(&sm.bm[i16 * S + 32 * m + 4 * h4]);
        qkt = mma32(ab, ac, qkt);  // bf16 x bf16 products are exact in fp32
        uint4 sh, sl;
        split8(St[2 * m], St[2 * m + 1], sh, sl);
        cs = mma32(ac, sl, mma32(ac, sh, cs));
      }
    }
    f32x4 Pt, U;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      Pt[r] = qkt[r] * gt.Gmt[r];  // Gmt is zero above the mask
      U[r] = gt.bet[r] * xv[r];
    }
    const f32x4 Y = mm(Pt, U, gt.gam * cs) + Dh * xv;
#pragma unroll
    for (int r = 0; r < 4; ++r) sm.y[(4 * h4 + r) * P + col] = Y[r];
    // -- S = gamma_last S + B^T diag(delta) U
    const f32x4 dU = gt.del * U;
    uint2 uh, ul;
    if constexpr (!F32IN) split4(dU, uh, ul);
#pragma unroll
    for (int rt = 0; rt < NT; ++rt) {
      f32x4 abt;
#pragma unroll
      for (int s = 0; s < 4; ++s) abt[s] = sm.bm[(4 * h4 + s) * S + 16 * rt + i16];
      if constexpr (F32IN) {
        St[rt] = mm(abt, dU, gt.gam_last * St[rt]);
      } else {
        const uint2 ab = pack4(abt);
        St[rt] = mma16b(ab, ul, mma16b(ab, uh, gt.gam_last * St[rt]));
      }
    }
    __syncthreads();  // the chunk's tables are read and its outputs staged
    // -- store the chunk's rows of y: a (token, head) row is P contiguous
    //    values, written by consecutive threads with 16-byte stores
    {
      constexpr int EPS = F32IN ? 4 : 8;  // elements per 16-byte store
      constexpr int PER_ROW = P / EPS;
      for (int e = tid; e < L * PER_ROW; e += NTH) {
        const int row = e / PER_ROW, c0 = EPS * (e % PER_ROW);
        if (row >= n) continue;
        const float* src = &sm.y[row * P + c0];
        const size_t oi = (size_t(t0 + row) * a.n_heads + h) * P + c0;
        if constexpr (F32IN) {
          *reinterpret_cast<f32x4*>(static_cast<float*>(a.y) + oi) = ld4(src);
        } else {
          const uint4 v = cat(pack4(ld4(src)), pack4(ld4(src + 4)));
          *reinterpret_cast<uint4*>(static_cast<uint16_t*>(a.y) + oi) = v;
        }
      }
    }
  }

  float* dst = a.states ? a.states + (size_t(seg) * a.n_heads + h) * hs
                        : (a.slot[seg] >= 0 ? a.slots + (size_t(a.slot[seg]) * a.n_heads + h) * hs : nullptr);
  if (dst) {
#pragma unroll
    for (int rt = 0; rt < NT; ++rt)
#pragma unroll
      for (int r = 0; r < 4; ++r) dst[size_t(16 * rt + 4 * h4 + r) * P + col] = St[rt][r];
  }
}

template <int N, int P, bool F32IN>
hipError_t launch_ssd(const SsdArgs& a, hipStream_t stream) {
  if (a.n_items <= 0) return hipSuccess;
  ssd_level_kernel<N, P, F32IN><<<dim3(unsigned(a.n_items * a.n_heads)), dim3(4 * P), 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace

bool ssd_supported(int d_state, int head_dim, int dtype) {
  if (dtype != TREE_DTYPE_BF16 && dtype != TREE_DTYPE_F32) return false;
  return (d_state == 64 || d_state == 128) && (head_dim == 32 || head_dim == 64);
}

hipError_t launch_ssd_scan(const SsdArgs& a, int d_state, int head_dim, int dtype, hipStream_t stream) {
  const bool f32 = dtype == TREE_DTYPE_F32;
  if (d_state == 128 && head_dim == 64) return f32 ? launch_ssd<128, 64, true>(a, stream) : launch_ssd<128, 64, false>(a, stream);
  if (d_state == 128 && head_dim == 32) return f32 ? launch_ssd<128, 32, true>(a, stream) : launch_ssd<128, 32, false>(a, stream);
  if (d_state == 64 && head_dim == 64) return f32 ? launch_ssd<64, 64, true>(a, stream) : launch_ssd<64, 64, false>(a, stream);
  if (d_state == 64 && head_dim == 32) return f32 ? launch_ssd<64, 32, true>(a, stream) : launch_ssd<64, 32, false>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace tg
