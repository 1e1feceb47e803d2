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

// Block -> (item, head), XCD-aware.  Work-groups are dealt to the 8 XCDs in
// turn (block b runs on XCD b % 8), and every head of a segment reads the
// same B and C rows (one group, or a few, for all heads).  Within each run of
// 8 items the blocks are ordered so that XCD x gets every head of item
// 8 j + x, and the B/C rows of a segment are fetched into one XCD's L2 instead
// of all eight.  Items past the last whole run of 8 keep the plain order.
__device__ __forceinline__ void ssd_block_item(int b, int n_items, int n_heads, int& item, int& h) {
  const int full = (n_items / 8) * 8;
  if (b < full * n_heads) {
    const int gi = b / (8 * n_heads), r = b - gi * 8 * n_heads;
    item = 8 * gi + (r & 7);
    h = r >> 3;
  } else {
    const int r = b - full * n_heads;
    item = full + r / n_heads;
    h = r - (r / n_heads) * n_heads;
  }
}

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

  int item, h;
  ssd_block_item(blockIdx.x, a.n_items, a.n_heads, item, h);
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

// ---- bf16, d_state = 128 -----------------------------------------------------------
// The same algebra with the chunk's inputs moved by DMA: B and C rows (256
// bytes each) land in swizzled bf16 tiles, x rows in a row-major tile and dt
// in a row of floats, all written to LDS by buffer loads straight from HBM,
// one chunk ahead into the other half of double buffers.  MFMA operands are
// read from the tiles as they are (C and B rows for C S0 and C B^T; B^T and x
// by transposing reads), the state's hi/lo split takes its residual from an
// MFMA, and the outputs are staged as bf16 and stored as whole rows during the
// next chunk.
// The chunk's gate tables, made once per work-group by one wave during the
// previous chunk: Gamma^T in the lanes' accumulator order, gamma, delta and dt
// by token, gamma_last (double-buffered), and the making wave's prefix G.
// Empty where each wave makes its own gates: the extra LDS would cost the
// two-wave instantiation a work-group per CU.
template <bool SHARED>
struct SsdGateTables {
  alignas(16) float gmt[2][4 * 64];
  alignas(16) float grow[2][3][L];
  alignas(16) float glast[2][4];
  alignas(16) float gp[L];
};
template <>
struct SsdGateTables<false> {};

template <int P>
struct SsdTileSmem {
  alignas(16) char bt[2][kTileRow16];  // B rows of the chunk
  alignas(16) char ct[2][kTileRow16];  // C rows
  alignas(16) char xt[2][L * P * 2];   // x rows (row-major, 2P bytes each)
  alignas(16) float dt[2][L];
  alignas(16) uint16_t ys[2][L * P];   // staged outputs (bf16, row-major)
  SsdGateTables<(P / 16 >= 4)> gt;
};

template <int P>
__global__ __launch_bounds__(4 * P) __attribute__((amdgpu_waves_per_eu(4, 4))) void ssd_bf16_n128_kernel(SsdArgs a) {
  constexpr int N = 128;
  constexpr int NT = N / 16;  // row tiles of the state
  constexpr int NW = P / 16;  // waves
  constexpr int XB = L * P * 2 / 1024;  // 1 KB DMA blocks of the x tile
  // With four waves or more, one wave per chunk (in turn) makes the chunk's
  // gate tables for all of them, a chunk ahead; with two, each wave makes its
  // own (the shared form costs that instantiation occupancy).
  constexpr bool SHARED_GATES = NW >= 4;
  __shared__ SsdTileSmem<P> sm;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h4 = lane >> 4;
  const int i16 = lane & 15;
  const int col = 16 * w + i16;
  const uint2 negI = neg_identity(h4, i16);

  int item, h;
  ssd_block_item(blockIdx.x, a.n_items, a.n_heads, item, h);
  const int seg = a.items[item];
  const int grp = h / (a.n_heads / a.n_groups);
  const int par = a.parent[seg];
  const size_t hs = size_t(N) * P;
  const float Ah = a.A[h];
  const float Dh = a.D ? a.D[h] : 0.f;
  const uint16_t* Bg = static_cast<const uint16_t*>(a.B);
  const uint16_t* Cg = static_cast<const uint16_t*>(a.C);
  const uint16_t* xg = static_cast<const uint16_t*>(a.x);
  uint16_t* yg = static_cast<uint16_t*>(a.y);
  const int rs_bc = a.n_groups * N * 2, rs_x = a.n_heads * P * 2;  // bytes between token rows

  // Loop-constant LDS offsets: operand reads of row i16 at columns 32m + 4h4
  // (o2 = o + 32, opaque); transposing reads of B at columns 16rt and of x at
  // this wave's columns.
  // With shared gates tile_off(i16, 32m + 4h4) = aoff + (64 m ^ 64 (i16 & 3))
  // is recomputed at each chunk from an opaque copy rather than held in
  // eight registers; the two-wave form holds them.
  const int ak64 = 64 * (i16 & 3), aoff = tile_off(i16, 4 * h4) - ak64;
  int ao[NT / 2], ao2[NT / 2];
  if constexpr (!SHARED_GATES) {
#pragma unroll
    for (int m = 0; m < NT / 2; ++m) {
      ao[m] = tile_off(i16, 32 * m + 4 * h4);
      ao2[m] = ao[m] + 32;
      asm volatile("" : "+v"(ao2[m]));
    }
  }
  // B^T rows 16rt.. at bo[rt / 2] + 32 (rt % 2): the swizzle keeps a 16-column
  // step inside a 32-column block a plain 32-byte step, but not across blocks.
  int bo[NT / 2];
#pragma unroll
  for (int m = 0; m < NT / 2; ++m) bo[m] = tile_off(4 * h4 + (i16 >> 2), 32 * m + 4 * (i16 & 3));
  const int xo = (4 * h4 + (i16 >> 2)) * (2 * P) + 2 * (16 * w + 4 * (i16 & 3));

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

  // Chunk at token tc (rows past the segment end repeat its last row; their
  // dt is taken as zero below) into buffer buf.  Wave w loads B and C row
  // blocks w, w + NW, ...; the first waves the x blocks; dt is loaded by wave
  // gw, the one that makes the chunk's gate tables (with shared gates), else
  // by the last wave.
  auto fetch = [&](int tc, int end, int buf, int gw) {
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int Ln = min(L, end - tc);
    const auto rb = rsrc(Bg + (size_t(tc) * a.n_groups + grp) * N, L * rs_bc);
    const auto rc = rsrc(Cg + (size_t(tc) * a.n_groups + grp) * N, L * rs_bc);
    const int cofs = 16 * tile_dma_chunk(ln);
#pragma unroll
    for (int blk = w; blk < 4; blk += NW) {
      const int ob = min(4 * blk + (ln >> 4), Ln - 1) * rs_bc + cofs;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_void*)(sm.bt[buf] + tile_blk(blk)), 16, ob, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rc, (lds_void*)(sm.ct[buf] + tile_blk(blk)), 16, ob, 0, 0, 0);
    }
    if (w < XB) {  // rows of 2P bytes, 1024 / (2P) rows per block
      // x is read by this work-group alone: non-temporal (kCacheNT), so that
      // it does not push out of L2 the B/C rows, dt and parent states that
      // other heads of the segment read later.
      constexpr int RPB = 1024 / (2 * P), CPR = 2 * P / 16;
      const auto rx = rsrc(xg + (size_t(tc) * a.n_heads + h) * P, L * rs_x);
      const int ox = min(RPB * w + ln / CPR, Ln - 1) * rs_x + 16 * (ln % CPR);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lds_void*)(sm.xt[buf] + 1024 * w), 16, ox, 0, 0, kCacheNT);
    }
    if (w == (SHARED_GATES ? gw : NW - 1) && lane < L) {
      const auto rd = rsrc(a.dt + size_t(tc) * a.n_heads + h, L * a.n_heads * 4);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rd, (lds_void*)sm.dt[buf], 4, min(lane, Ln - 1) * a.n_heads * 4, 0,
                                               0, 0);
    }
  };
  // Whole rows of the staged outputs of the chunk at tc (n rows), through a
  // buffer descriptor whose range ends after row n - 1, so padding rows are
  // dropped.  (Plain stores through the generic output pointer made the
  // compiler wait for every outstanding load, the next chunk's DMA included,
  // before the following LDS reads.)
  // Gate tables of the chunk in buffer buf (n tokens), by the wave that
  // loaded its dt: G = prefix of g = dt A over the chunk (DPP scan over each
  // row of 16 lanes); padding rows have dt = 0.
  auto make_gate_tables = [&](int n, int buf) {
    if constexpr (SHARED_GATES) {
      const float dti = i16 < n ? sm.dt[buf][i16] : 0.f;
      float G = dti * Ah;
      G += dpp<0x111>(G);
      G += dpp<0x112>(G);
      G += dpp<0x114>(G);
      G += dpp<0x118>(G);
      // G of every token through LDS: written and read by this wave alone,
      // whose LDS accesses are served in order.
      if (h4 == 0) sm.gt.gp[i16] = G;
      asm volatile("" ::: "memory");
      const f32x4 Gr = ld4(&sm.gt.gp[4 * h4]);
      const float glast = sm.gt.gp[L - 1] * kLog2e, gc = G * kLog2e;
      f32x4 gm;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 4 * h4 + r;
        gm[r] = i16 >= row ? ex2(gc - Gr[r] * kLog2e) : 0.f;
      }
      *reinterpret_cast<f32x4*>(&sm.gt.gmt[buf][4 * lane]) = gm;
      if (h4 == 0) {
        sm.gt.grow[buf][0][i16] = ex2(gc);
        sm.gt.grow[buf][1][i16] = ex2(glast - gc);
        sm.gt.grow[buf][2][i16] = dti;
        if (i16 == 0) sm.gt.glast[buf][0] = ex2(glast);
      }
    }
  };
  auto store_y = [&](int tc, int n, int buf) {
    constexpr int CPR = 2 * P / 16;  // 16-byte chunks per row
    const auto ry = rsrc(yg + (size_t(tc) * a.n_heads + h) * P, (n - 1) * rs_x + 2 * P);
    for (int e = tid; e < L * CPR; e += 4 * P) {
      const int row = e / CPR, c = e % CPR;
      const u32x4 v = *reinterpret_cast<const u32x4*>(&sm.ys[buf][row * P + 8 * c]);
      __builtin_amdgcn_raw_buffer_store_b128(v, ry, row * rs_x + 16 * c, 0, kCacheNT);  // not read again here
    }
  };

  const int t_beg = a.seg_off[seg], t_end = a.seg_off[seg + 1];
  fetch(t_beg, t_end, 0, 0);
  if (SHARED_GATES && w == 0) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's dt of the first chunk has landed
    make_gate_tables(min(L, t_end - t_beg), 0);
  }
  int s = 0, prev_t0 = -1, prev_n = 0;
  for (int t0 = t_beg;;) {
    const int n = min(L, t_end - t0);
    const int nt0 = t0 + L;
    const bool more = nt0 < t_end;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's DMA of the chunk has landed
    __syncthreads();                                   // ... and every other wave's
    const char* Bs = sm.bt[s];
    const char* Cs = sm.ct[s];
    // The chunk's transposing reads (x, and B^T for the state update) come
    // before the next chunk's DMA is issued: after it, the compiler makes them
    // wait for that DMA to land, which would serialise the prefetch.
    const uint2 xr = tile_tr(sm.xt[s], xo);
    uint2 bT[NT];
#pragma unroll
    for (int rt = 0; rt < NT; ++rt) bT[rt] = tile_tr(Bs, bo[rt >> 1] + 32 * (rt & 1));
    // The next chunk's gate tables: made by wave (chunk index + 1) % NW, which
    // also loads that chunk's dt, at the end of this chunk.
    const int gw = ((t0 - t_beg) / L + 1) % NW;
    if (more) fetch(nt0, t_end, s ^ 1, gw);
    if (prev_t0 >= 0) store_y(prev_t0, prev_n, s ^ 1);

    // -- C B^T (exact), C S0 (S0 as hi + lo)
    f32x4 qkt = z4(), cs = z4();
    int ab0 = aoff, ak = ak64;
    if constexpr (SHARED_GATES) asm volatile("" : "+v"(ab0), "+v"(ak));
#pragma unroll
    for (int m = 0; m < NT / 2; ++m) {
      int aom, ao2m;
      if constexpr (SHARED_GATES) {
        aom = ab0 + ((64 * m) ^ ak);
        ao2m = aom + 32;
        asm volatile("" : "+v"(ao2m));
      } else {
        aom = ao[m];
        ao2m = ao2[m];
      }
      const uint4 ac = tile_a8(Cs, aom, ao2m);
      // Kept apart from the C read at the same offsets: fused into one
      // ds_read2st64_b64 they cost several times as much.
      asm volatile("" ::: "memory");
      const uint4 ab = tile_a8(Bs, aom, ao2m);
      qkt = mma32(ab, ac, qkt);
      uint4 sh, sl;
      split8m(St[2 * m], St[2 * m + 1], negI, sh, sl);
      cs = mma32(ac, sl, mma32(ac, sh, cs));
    }

    // -- gates: G = prefix of g = dt A over the chunk (DPP scan over each row
    //    of 16 lanes); padding rows have dt = 0
    Gates gt;
    if constexpr (SHARED_GATES) {
      gt.Gmt = ld4(&sm.gt.gmt[s][4 * lane]);
      gt.gam = ld4(&sm.gt.grow[s][0][4 * h4]);
      gt.del = ld4(&sm.gt.grow[s][1][4 * h4]);
      gt.bet = ld4(&sm.gt.grow[s][2][4 * h4]);
      gt.gam_last = sm.gt.glast[s][0];
    } else {  // G = prefix of g = dt A over the chunk; padding rows have dt = 0
      const float dti = i16 < n ? sm.dt[s][i16] : 0.f;
      float G = dti * Ah;
      G += dpp<0x111>(G);
      G += dpp<0x112>(G);
      G += dpp<0x114>(G);
      G += dpp<0x118>(G);
      const int base = 16 * h4;
      const float glast = __shfl(G, base + 15, 64) * kLog2e, gc = G * kLog2e;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 4 * h4 + r;
        const float gr = __shfl(G, base + row, 64) * kLog2e;
        gt.gam[r] = ex2(gr);
        gt.del[r] = ex2(glast - gr);
        gt.bet[r] = __shfl(dti, base + row, 64);
        gt.Gmt[r] = i16 >= row ? ex2(gc - gr) : 0.f;
      }
      gt.gam_last = ex2(glast);
    }
    const f32x4 xv = bf4(xr);
    f32x4 Pt, U;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      Pt[r] = qkt[r] * gt.Gmt[r];
      U[r] = gt.bet[r] * xv[r];
    }
    f32x4 Y;
    {  // P U on split-bf16 MFMA (hi x hi + hi x lo + lo x hi)
      uint2 ph, pl, uh2, ul2;
      split4m(Pt, negI, ph, pl);
      split4m(U, negI, uh2, ul2);
      Y = mma16b(pl, uh2, mma16b(ph, ul2, mma16b(ph, uh2, gt.gam * cs))) + Dh * xv;
    }
    {
      const uint2 yp = pack4(Y);
      uint16_t* yr = &sm.ys[s][(4 * h4) * P + col];
      yr[0] = static_cast<uint16_t>(yp.x);
      yr[P] = static_cast<uint16_t>(yp.x >> 16);
      yr[2 * P] = static_cast<uint16_t>(yp.y);
      yr[3 * P] = static_cast<uint16_t>(yp.y >> 16);
    }
    // -- S = gamma_last S + B^T diag(delta) U
    uint2 uh, ul;
    split4m(gt.del * U, negI, uh, ul);
#pragma unroll
    for (int rt = 0; rt < NT; ++rt) {
      St[rt] = mma16b(bT[rt], ul, mma16b(bT[rt], uh, gt.gam_last * St[rt]));
    }
    if (SHARED_GATES && more && w == gw) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's loads of the next chunk have landed
      make_gate_tables(min(L, t_end - nt0), s ^ 1);
    }
    prev_t0 = t0;
    prev_n = n;
    if (!more) break;
    t0 = nt0;
    s ^= 1;
  }
  __syncthreads();  // the last chunk's staged rows
  store_y(prev_t0, prev_n, s);

  float* dst = a.states ? a.states + (size_t(seg) * a.n_heads + h) * hs
                        : (a.slot[seg] >= 0 ? a.slots + (size_t(a.slot[seg]) * a.n_heads + h) * hs : nullptr);
  if (dst) {
    // Offsets from an opaque copy of the lane number: shared with the
    // parent-state load at the top, they were held (spilled) across the
    // whole segment.
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int o = (4 * (ln >> 4)) * P + 16 * w + (ln & 15);
#pragma unroll
    for (int rt = 0; rt < NT; ++rt)
#pragma unroll
      for (int r = 0; r < 4; ++r) dst[size_t(16 * rt + r) * P + o] = St[rt][r];
  }
}

template <int N, int P, bool F32IN>
hipError_t launch_ssd(const SsdArgs& a, hipStream_t stream) {
  if (a.n_items <= 0) return hipSuccess;
  const dim3 grid(unsigned(a.n_items * a.n_heads)), block(4 * P);
  if constexpr (N == 128 && !F32IN)
    ssd_bf16_n128_kernel<P><<<grid, block, 0, stream>>>(a);
  else
    ssd_level_kernel<N, P, F32IN><<<grid, block, 0, stream>>>(a);
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
